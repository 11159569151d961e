"""vsa_profile_heads_noalloc (the profiler with the library's static scratch
instead of a caller workspace) against vsa_profile_heads: bit-identical errors
and choices on two calls in a row, the second on a smaller problem (the scratch
then still holds the first call's data), and a problem too large for the static
scratch rejected on the host before any HIP call."""
import ctypes
import os

import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from oracle import masks as OM
from workloads import WAN480, make_qkv, profile_rows

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(not os.path.exists(V.LIB_PATH), reason="libvsa.so not built")
def test_noalloc_rejects_a_problem_beyond_the_static_scratch():
    """On the host, before any HIP call: the long-horizon profile (128 MiB of
    scratch) exceeds the 96 MiB array; the Wan and HunyuanVideo profiles fit."""
    L = V.lib()
    cap = V.vsa_profile_scratch_capacity()
    assert cap == 96 << 20
    assert V.vsa_profile_workspace_bytes(1, 12, (21, 30, 52), 128, 328, 2) <= cap
    assert V.vsa_profile_workspace_bytes(1, 24, (33, 45, 80), 128, 1188, 2) <= cap
    assert V.vsa_profile_workspace_bytes(1, 12, (126, 30, 52), 128, 1966, 2) > cap
    p = ctypes.c_void_p(0x1000)
    lay = (ctypes.c_int32 * 2)(0, 1)
    st = L.vsa_profile_heads_noalloc(p, p, p, 1, 12, V.vsa_grid(126, 30, 52), 128, 0, 128, p, 1966, p,
                                     ctypes.cast(lay, ctypes.c_void_p), 2, 0.1, p, p, None)
    assert st == V.VSA_ERR_WORKSPACE
    assert "static scratch" in V.vsa_last_error()
    st = L.vsa_profile_heads_noalloc(p, p, p, 1, 12, V.vsa_grid(21, 30, 52), 128, 0, 128, p, 328, p,
                                     ctypes.cast(lay, ctypes.c_void_p), 5, 0.1, p, p, None)
    assert st == V.VSA_ERR_INVALID


def _profile_case(w, rows, cands, layout):
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).cuda() for x in make_qkv(w))
    rd = torch.from_numpy(np.ascontiguousarray(rows, np.int32)).cuda()
    cd = torch.from_numpy(np.ascontiguousarray(cands, np.uint8)).cuda()
    ref = V.vsa_profile_heads(q, k, v, w.grid, w.bs, rd, cd, layout)
    B, H, P = w.B, w.H, len(layout)
    out = (torch.full((B, H, P), float("nan"), dtype=torch.float32, device="cuda"),
           torch.full((B, H), -1, dtype=torch.int32, device="cuda"))
    got = V.vsa_profile_heads_noalloc(q, k, v, w.grid, w.bs, rd, cd, layout, out=out)
    torch.cuda.synchronize()
    assert got[0] is out[0] and got[1] is out[1]
    return ref, got


@pytest.mark.gpu
def test_noalloc_matches_workspace_form_on_two_calls():
    # call 1: the Wan 480p profile at amplitude 4.0 (12 heads, 328 rows, a mixed choice)
    w = WAN480.scaled(name="wan480_amp4", amplitude=4.0)
    print(f"[gpu-case] noalloc wan480 H={w.H}", flush=True)
    cands = np.stack([OM.pattern_mask(w.grid, w.bs, "spatial", 1), OM.pattern_mask(w.grid, w.bs, "temporal", 0)])
    ref, got = _profile_case(w, profile_rows(w), cands, [0, 1])
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    ch = ref[1].cpu().numpy()
    assert 0 < ch.sum() < ch.size
    # call 2, right after: a smaller problem (3 heads, 3 candidates, bs 64); the
    # scratch still holds call 1's bit table and partial records
    grid = (8, 12, 16)
    w2 = WAN480.scaled(name="noalloc_small", T=grid[0], Hh=grid[1], W=grid[2], H=3, bs=64, seed=9)
    print(f"[gpu-case] noalloc small grid={grid}", flush=True)
    rows = np.sort(np.random.default_rng([9, 3]).choice(w2.N, size=40, replace=False))
    cands2 = np.stack([OM.pattern_mask(grid, 64, "spatial", 0), OM.pattern_mask(grid, 64, "temporal", 8),
                       OM.pattern_mask(grid, 64, "spatial", 1)])
    ref2, got2 = _profile_case(w2, rows, cands2, [0, 1, 0])
    assert torch.equal(ref2[0], got2[0]) and torch.equal(ref2[1], got2[1])
    assert torch.isfinite(got2[0]).all()
