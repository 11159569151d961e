"""Builds libvsa.so (HIP C++ for gfx950) in-tree.

    python -m block_sparse_attention_vsa_amd.build      # or build() from Python

Each source under csrc/ is compiled with hipcc to an object in _build/, in
parallel, then linked into block_sparse_attention_vsa_amd/libvsa.so. Every call
recompiles: the build is the check that the sources compile for gfx950.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libvsa.so")

SOURCES = ["status.hip", "pattern.hip", "permute.hip", "attn_fwd.hip", "attn_bwd.hip", "scores.hip", "select.hip",
           "profile.hip", "semantic.hip", "attn_varlen.hip", "attn_fp8.hip"]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms stay off; plain float code is scheduled as scalar-per-lane ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# Host-side AddressSanitizer and UndefinedBehaviorSanitizer (device code is
# compiled as usual): every -fsanitize= is scoped to the host pass.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_BUILD = os.path.join(BUILD, "sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libvsa_sanitized.so")


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    out_dir = SAN_BUILD if sanitize else BUILD
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l and "is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every source and link libvsa.so; with sanitize, a separate
    _build/sanitize/libvsa_sanitized.so whose host code carries ASan and UBSan
    (load it with the sanitizer runtime preloaded, see sanitizer_runtime())."""
    os.makedirs(SAN_BUILD if sanitize else BUILD, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize), srcs))
    lib = SAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    extra = ["-fsanitize=address", "-fsanitize=undefined", "-shared-libasan"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *extra, "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(lib)} failed:\n{' '.join(cmd)}\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def sanitizer_runtime() -> str:
    """Path of the compiler's shared ASan runtime (to LD_PRELOAD into an
    uninstrumented Python that loads the sanitized library)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the clang ASan runtime was not found")
    return path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
