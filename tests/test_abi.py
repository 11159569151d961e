"""C-ABI checks that need no GPU: libvsa.so loads, exports every function that
include/vsa.h declares, and rejects bad arguments on the host before any HIP
call (null pointers with valid sizes never reach a launch)."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_vsa_amd as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(V.LIB_PATH), reason="libvsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = declared_functions()
    assert len(names) >= 16
    lib = V.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in V._SIGNATURES, f"binding lacks {n}"
    # the binding exposes a Python function of the same name for each entry point
    for n in names:
        assert callable(getattr(V, n)), n


def test_status_strings_and_version():
    assert V.vsa_status_string(0) == "ok"
    assert V.vsa_status_string(1) == "invalid argument"
    assert V.vsa_status_string(99) == "unknown status"
    assert V.vsa_version() >= 100


def test_host_selftest_of_index_helpers():
    assert V.lib().vsa_selftest_host() == V.VSA_OK


def test_cube_dims_on_video_grids():
    assert V.vsa_cube_dims((21, 30, 52)) == (624, 39936)
    assert V.vsa_cube_dims((4, 8, 8)) == (4, 256)
    with pytest.raises(V.VsaError):
        V.vsa_cube_dims((0, 8, 8))


def g(T=4, Hh=8, W=8):
    return V.vsa_grid(T, Hh, W)


def test_attention_validation_before_any_hip_call():
    L = V.lib()
    fake = ctypes.c_void_p(0x1000)          # aligned, never dereferenced: validation fails first
    blk = V.vsa_blocks()
    blk.mask = 0x1000
    call = lambda **kw: L.vsa_block_sparse_attn_fwd(
        kw.get("q", fake), fake, fake, fake, None, kw.get("B", 1), 2, 256, kw.get("D", 128), kw.get("dtype", 0),
        kw.get("bs", 128), None, ctypes.byref(kw.get("blocks", blk)), kw.get("scale", 0.1), None, 0, None)
    assert call(q=None) == V.VSA_ERR_INVALID
    assert "null" in V.vsa_last_error()
    assert call(q=ctypes.c_void_p(0x1004)) == V.VSA_ERR_INVALID
    assert call(B=0) == V.VSA_ERR_INVALID
    assert call(D=96) == V.VSA_ERR_UNSUPPORTED
    assert call(bs=32) == V.VSA_ERR_UNSUPPORTED
    assert call(dtype=1, bs=128) == V.VSA_ERR_UNSUPPORTED
    assert call(dtype=7) == V.VSA_ERR_UNSUPPORTED
    assert call(scale=0.0) == V.VSA_ERR_INVALID
    assert call(scale=float("inf")) == V.VSA_ERR_INVALID
    both = V.vsa_blocks(0x1000, 0x1000, 0x1000, 4)
    assert call(blocks=both) == V.VSA_ERR_INVALID
    neither = V.vsa_blocks()
    assert call(blocks=neither) == V.VSA_ERR_INVALID
    half = V.vsa_blocks(None, 0x1000, None, 4)
    assert call(blocks=half) == V.VSA_ERR_INVALID
    assert "exactly one" in V.vsa_last_error() or "list form" in V.vsa_last_error()


def test_permuted_attention_validation():
    L = V.lib()
    fake = ctypes.c_void_p(0x1000)
    blk = V.vsa_blocks()
    blk.mask = 0x1000
    hf = (ctypes.c_uint8 * 2)(1, 0)
    call = lambda **kw: L.vsa_block_sparse_attn_fwd_permuted(
        kw.get("q", fake), fake, fake, fake, None, 1, kw.get("H", 2), kw.get("grid", g()), kw.get("D", 128),
        kw.get("dtype", 0), kw.get("bs", 128), ctypes.cast(hf, ctypes.c_void_p), None, ctypes.byref(blk),
        kw.get("scale", 0.1), None)
    assert call(q=None) == V.VSA_ERR_INVALID
    assert call(grid=g(0)) == V.VSA_ERR_INVALID
    assert call(D=64) == V.VSA_ERR_UNSUPPORTED            # frame-major heads: D = 128 only
    assert "D = 128" in V.vsa_last_error()
    assert call(dtype=1, bs=64) == V.VSA_ERR_UNSUPPORTED   # and bf16 only
    assert call(H=2000) == V.VSA_ERR_UNSUPPORTED
    assert call(bs=32) == V.VSA_ERR_UNSUPPORTED
    assert call(scale=-1.0) == V.VSA_ERR_INVALID


def test_chosen_attention_validation():
    L = V.lib()
    fake = ctypes.c_void_p(0x1000)
    lay = (ctypes.c_int32 * 2)(0, 1)
    bad = (ctypes.c_int32 * 2)(0, 3)
    call = lambda **kw: L.vsa_block_sparse_attn_fwd_chosen(
        fake, fake, fake, fake, None, 1, 2, kw.get("grid", g()), kw.get("D", 128), 0, 128,
        kw.get("cand", fake), ctypes.cast(kw.get("lay", lay), ctypes.c_void_p), kw.get("P", 2),
        kw.get("choice", fake), None, 0.1, None)
    assert call(cand=None) == V.VSA_ERR_INVALID
    assert call(choice=None) == V.VSA_ERR_INVALID
    assert call(P=0) == V.VSA_ERR_INVALID
    assert call(P=5) == V.VSA_ERR_INVALID
    assert call(lay=bad) == V.VSA_ERR_INVALID
    assert call(grid=g(0)) == V.VSA_ERR_INVALID
    assert call(D=64) == V.VSA_ERR_UNSUPPORTED


def test_permute_validation():
    L = V.lib()
    p = ctypes.c_void_p(0x1000)
    assert L.vsa_permute(None, p, 1, 2, g(), 128, 0, 0, 0, None, None) == V.VSA_ERR_INVALID
    assert L.vsa_permute(p, p, 1, 2, g(), 80, 0, 0, 0, None, None) == V.VSA_ERR_UNSUPPORTED
    assert L.vsa_permute(p, p, 1, 2, g(), 128, 3, 0, 0, None, None) == V.VSA_ERR_UNSUPPORTED
    assert L.vsa_permute(p, p, 1, 2, g(), 128, 0, 5, 0, None, None) == V.VSA_ERR_INVALID
    assert L.vsa_permute(p, p, 1, 2, g(0), 128, 0, 0, 0, None, None) == V.VSA_ERR_INVALID
    sel = (ctypes.c_uint8 * 2)(1, 0)
    assert L.vsa_permute(p, p, 1, 2, g(), 128, 0, 1, 0, ctypes.cast(sel, ctypes.c_void_p), None) == V.VSA_ERR_INVALID


def test_scores_select_mask_validation():
    L = V.lib()
    p = ctypes.c_void_p(0x1000)
    assert L.vsa_block_scores(p, p, 1, 2, 256, 128, 0, 96, None, 0.1, p, p, p, None) == V.VSA_ERR_UNSUPPORTED
    assert L.vsa_block_scores(p, p, 1, 2, 256, 128, 1, 64, None, 0.1, p, p, p, None) == V.VSA_ERR_UNSUPPORTED
    assert L.vsa_block_scores(p, p, 1, 2, 256, 128, 0, 64, None, 0.1, p, None, p, None) == V.VSA_ERR_INVALID
    odd = ctypes.c_void_p(0x1004)                    # pooled vectors are read 16 bytes at a time
    assert L.vsa_block_scores(p, p, 1, 2, 256, 128, 0, 64, None, 0.1, p, odd, p, None) == V.VSA_ERR_INVALID
    assert L.vsa_block_scores(p, p, 1, 2, 256, 128, 0, 64, None, 0.1, p, p, odd, None) == V.VSA_ERR_INVALID
    assert L.vsa_select_topk(p, 1, 2, 4, 4, None, 0, 1.0, p, p, None) == V.VSA_ERR_INVALID     # k_max < 1
    assert L.vsa_select_topk(p, 1, 2, 4, 4, None, 5, 1.0, p, p, None) == V.VSA_ERR_INVALID     # k_max > nkb
    assert L.vsa_select_topk(p, 1, 2, 4, 4, None, 2, 0.0, p, p, None) == V.VSA_ERR_INVALID     # top_p <= 0
    assert L.vsa_select_topk(p, 1, 2, 4, 4, None, 2, 1.5, p, p, None) == V.VSA_ERR_INVALID     # top_p > 1
    assert L.vsa_select_topk(p, 1, 2, 4, 5000, None, 2, 1.0, p, p, None) == V.VSA_ERR_UNSUPPORTED
    assert L.vsa_mask_to_list(p, 1, 2, 4, 4, None, 0, 0, p, p, None) == V.VSA_ERR_INVALID
    bad = (ctypes.c_int32 * 2)(0, 3)
    assert L.vsa_mask_to_list(p, 1, 2, 4, 4, ctypes.cast(bad, ctypes.c_void_p), 2, 4, p, p, None) == V.VSA_ERR_INVALID
    assert L.vsa_pattern_mask(g(), 0, 0, 1, p, None) == V.VSA_ERR_INVALID
    assert L.vsa_pattern_mask(g(), 64, 2, 1, p, None) == V.VSA_ERR_INVALID
    assert L.vsa_pattern_mask(g(), 64, 0, -1, p, None) == V.VSA_ERR_INVALID


def test_profile_validation_and_workspace_size():
    L = V.lib()
    p = ctypes.c_void_p(0x1000)
    lay = (ctypes.c_int32 * 2)(0, 1)
    layp = ctypes.cast(lay, ctypes.c_void_p)
    ws = V.vsa_profile_workspace_bytes(1, 12, (21, 30, 52), 128, 328, 2)
    assert ws > 0
    assert V.vsa_profile_workspace_bytes(1, 12, (21, 30, 52), 96, 328, 2) == 0
    assert L.vsa_profile_heads(p, p, p, 1, 12, V.vsa_grid(21, 30, 52), 128, 0, 128, p, 328, p, layp, 2, 0.1,
                               p, p, p, 16, None) == V.VSA_ERR_WORKSPACE
    assert L.vsa_profile_heads(p, p, p, 1, 12, V.vsa_grid(21, 30, 52), 128, 0, 128, p, 328, p, layp, 5, 0.1,
                               p, p, p, ws, None) == V.VSA_ERR_INVALID
    bad = (ctypes.c_int32 * 2)(0, 2)
    assert L.vsa_profile_heads(p, p, p, 1, 12, V.vsa_grid(21, 30, 52), 128, 0, 128, p, 328, p,
                               ctypes.cast(bad, ctypes.c_void_p), 2, 0.1, p, p, p, ws, None) == V.VSA_ERR_INVALID
    # a head of 2^23 tokens x 128 channels is 2 GiB: beyond the 32-bit descriptor size, rejected before any launch
    big = V.vsa_grid(128, 256, 256)
    assert L.vsa_profile_heads(p, p, p, 1, 1, big, 128, 0, 128, p, 328, p, layp, 2, 0.1,
                               p, p, p, 1 << 40, None) == V.VSA_ERR_INVALID
    assert L.vsa_profile_heads_noalloc(p, p, p, 1, 1, big, 128, 0, 128, p, 328, p, layp, 2, 0.1,
                                       p, p, None) == V.VSA_ERR_INVALID


def test_check_block_list_host():
    idx = np.array([[0, 2, 5, -1], [1, 1, 0, 0], [3, -1, -1, -1]], np.int32)
    V.vsa_check_block_list_host(idx[[0, 2]], np.array([3, 1], np.int32), 6)
    with pytest.raises(V.VsaError, match="ascending"):
        V.vsa_check_block_list_host(idx, np.array([3, 2, 1], np.int32), 6)
    with pytest.raises(V.VsaError, match="outside"):
        V.vsa_check_block_list_host(idx[[0]], np.array([3], np.int32), 5)
    with pytest.raises(V.VsaError, match="kv_cnt"):
        V.vsa_check_block_list_host(idx[[0]], np.array([5], np.int32), 6)


def test_attn_workspace_is_not_needed():
    assert V.vsa_attn_workspace_bytes(1, 12, 32760, 128, 256) == 0


def test_backward_validation_and_workspace_size():
    L = V.lib()
    fake = ctypes.c_void_p(0x1000)
    blk = V.vsa_blocks()
    blk.mask = 0x1000
    # B=1, H=2, N=256, bs=128: 512 padded rows -> lse2 and delta 2048 bytes each,
    # 2 x 2 x 2 transposed list entries and 4 counts, each rounded to 256 bytes
    ws_mask = V.vsa_attn_bwd_workspace_bytes(1, 2, 256, 128, 0)
    ws_list = V.vsa_attn_bwd_workspace_bytes(1, 2, 256, 128, 1)
    assert ws_mask == 2048 + 2048 + 256 + 256
    assert ws_list == ws_mask + 256                       # the mask built from the lists
    assert V.vsa_attn_bwd_workspace_bytes(1, 2, 256, 32, 0) == 0
    call = lambda **kw: L.vsa_block_sparse_attn_bwd(
        kw.get("q", fake), fake, fake, fake, fake, kw.get("lse", fake), kw.get("dq", fake), fake, fake,
        kw.get("B", 1), 2, 256, kw.get("D", 128), kw.get("dtype", 0), kw.get("bs", 128), None,
        ctypes.byref(kw.get("blocks", blk)), kw.get("scale", 0.1), kw.get("ws", fake), kw.get("ws_bytes", ws_mask),
        None)
    assert call(q=None) == V.VSA_ERR_INVALID
    assert call(lse=None) == V.VSA_ERR_INVALID
    assert call(dq=ctypes.c_void_p(0x1008)) == V.VSA_ERR_INVALID
    assert call(B=0) == V.VSA_ERR_INVALID
    assert call(D=64) == V.VSA_ERR_UNSUPPORTED
    assert call(dtype=1) == V.VSA_ERR_UNSUPPORTED
    assert call(bs=32) == V.VSA_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == V.VSA_ERR_INVALID
    assert call(blocks=V.vsa_blocks()) == V.VSA_ERR_INVALID
    assert call(blocks=V.vsa_blocks(None, 0x1000, 0x1000, 0)) == V.VSA_ERR_INVALID
    assert call(ws=None) == V.VSA_ERR_WORKSPACE
    assert call(ws_bytes=ws_mask - 1) == V.VSA_ERR_WORKSPACE
    assert str(ws_mask) in V.vsa_last_error()
    # the list form needs the larger workspace
    assert call(blocks=V.vsa_blocks(None, 0x1000, 0x1000, 2)) == V.VSA_ERR_WORKSPACE


def test_semantic_validation_and_workspace_sizes():
    L = V.lib()
    fake = ctypes.c_void_p(0x1000)
    # k-means: bf16 centroids 51200, norms 800 -> 1024, order 8000 -> 8192,
    # offsets 808 -> 1024, chunk table 2 x 4 x 100 x 4 = 3200 -> 3328
    assert V.vsa_kmeans_workspace_bytes(1, 2, 1000, 100, 128) == 51200 + 1024 + 8192 + 1024 + 3328
    assert V.vsa_kmeans_workspace_bytes(1, 2, 1000, 100, 64) == 0
    km = lambda **kw: L.vsa_kmeans(kw.get("x", fake), 1, 2, kw.get("N", 1000), kw.get("D", 128), kw.get("dtype", 0),
                                   kw.get("C", 100), kw.get("iters", 3), fake, fake, fake, fake,
                                   kw.get("ws", 1 << 20), None)
    assert km(x=None) == V.VSA_ERR_INVALID
    assert km(C=0) == V.VSA_ERR_INVALID
    assert km(C=1001) == V.VSA_ERR_INVALID                  # more clusters than tokens
    assert km(N=10000, C=2000) == V.VSA_ERR_UNSUPPORTED
    assert km(iters=0) == V.VSA_ERR_INVALID
    assert km(D=64) == V.VSA_ERR_UNSUPPORTED
    assert km(dtype=1) == V.VSA_ERR_UNSUPPORTED
    assert km(ws=100) == V.VSA_ERR_WORKSPACE
    # cluster order: chunk table of 4 chunks x 8 clusters per head
    assert V.vsa_cluster_order_workspace_bytes(1, 2, 1000, 8) == 2 * 4 * 8 * 4
    co = lambda **kw: L.vsa_cluster_order(fake, 1, 2, 1000, kw.get("C", 8), fake, fake, fake,
                                          kw.get("ws", 1 << 20), None)
    assert co(C=2000) == V.VSA_ERR_UNSUPPORTED
    assert co(ws=255) == V.VSA_ERR_WORKSPACE
    gr = lambda **kw: L.vsa_gather_rows(kw.get("src", fake), kw.get("dst", ctypes.c_void_p(0x2000)), 1, 2, 100,
                                        kw.get("D", 128), kw.get("dtype", 0), fake, 0, None)
    assert gr(src=None) == V.VSA_ERR_INVALID
    assert gr(dst=fake) == V.VSA_ERR_INVALID                 # in place is refused
    assert gr(D=96) == V.VSA_ERR_UNSUPPORTED
    sc = lambda **kw: L.vsa_cluster_scores(fake, kw.get("ck", fake), fake, 1, 2, 8, 16, kw.get("D", 128),
                                           kw.get("scale", 0.1), fake, None)
    assert sc(ck=ctypes.c_void_p(0x1004)) == V.VSA_ERR_INVALID
    assert sc(D=32) == V.VSA_ERR_UNSUPPORTED
    assert sc(scale=0.0) == V.VSA_ERR_INVALID
    # varlen attention
    # chunk table 2 x 8, kept keys 2 x 7, order 2 x (1000 // 128 + 7), count: each rounded to 256 bytes
    assert V.vsa_varlen_attn_workspace_bytes(1, 2, 1000, 7) == 256 * 4
    blk = V.vsa_blocks()
    blk.mask = 0x1000
    va = lambda **kw: L.vsa_varlen_sparse_attn_fwd(
        fake, fake, fake, fake, None, 1, 2, 1000, kw.get("D", 128), 0, fake, 7, fake, kw.get("Ck", 9),
        ctypes.byref(kw.get("blocks", blk)), 0.1, kw.get("ws", fake), kw.get("ws_bytes", 1024), None)
    assert va(D=64) == V.VSA_ERR_UNSUPPORTED
    assert va(blocks=V.vsa_blocks()) == V.VSA_ERR_INVALID
    assert va(Ck=5000) == V.VSA_ERR_UNSUPPORTED               # mask row longer than a workgroup holds
    assert va(ws=None) == V.VSA_ERR_WORKSPACE
    assert va(ws_bytes=1023) == V.VSA_ERR_WORKSPACE


def test_fp8_validation():
    L = V.lib()
    fake = ctypes.c_void_p(0x1000)
    qz = lambda **kw: L.vsa_fp8_quantize(kw.get("x", fake), 1, 2, 100, kw.get("D", 128), kw.get("dtype", 0),
                                         kw.get("kind", 0), fake, fake, None)
    assert qz(x=None) == V.VSA_ERR_INVALID
    assert qz(D=64) == V.VSA_ERR_UNSUPPORTED
    assert qz(dtype=1) == V.VSA_ERR_UNSUPPORTED
    assert qz(kind=5) == V.VSA_ERR_INVALID
    blk = V.vsa_blocks()
    blk.mask = 0x1000
    at = lambda **kw: L.vsa_block_sparse_attn_fwd_fp8(
        fake, fake, fake, fake, fake, kw.get("vs", fake), fake, None, 1, 2, 1000, kw.get("D", 128), kw.get("bs", 128),
        None, ctypes.byref(kw.get("blocks", blk)), kw.get("scale", 0.1), None)
    assert at(vs=None) == V.VSA_ERR_INVALID
    assert at(D=64) == V.VSA_ERR_UNSUPPORTED
    assert at(bs=64) == V.VSA_ERR_UNSUPPORTED
    assert at(scale=-1.0) == V.VSA_ERR_INVALID
    assert at(blocks=V.vsa_blocks()) == V.VSA_ERR_INVALID


def test_trace_log_names_rejected_calls():
    """VSA_TRACE=1 logs every rejected call (and every launch) to stderr; unset,
    the library prints nothing."""
    import subprocess
    import sys
    code = ("import ctypes, block_sparse_attention_vsa_amd as V; "
            "print(V.lib().vsa_pattern_mask(V.vsa_grid(4, 8, 8), 0, 0, 1, ctypes.c_void_p(0x1000), None))")
    on = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, VSA_TRACE="1"), cwd=ROOT,
                        capture_output=True, text=True, timeout=120)
    assert on.stdout.strip() == "1"
    assert "[vsa] rejected (status 1): vsa_pattern_mask: bs must be in [1, 1024]" in on.stderr
    off = subprocess.run([sys.executable, "-c", code], env=dict(os.environ, VSA_TRACE="0"), cwd=ROOT,
                         capture_output=True, text=True, timeout=120)
    assert off.stdout.strip() == "1" and "[vsa]" not in off.stderr
