"""GPU parity of the structural entry points against the oracle, bit for bit:
pattern masks, cube lengths, mask -> list, and the permutations."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from oracle import layout as OL
from oracle import masks as OM
from tests.gpu_util import announce, dev, dev_u8, host
from workloads import WAN480, HUNYUAN720, LONG126

pytestmark = pytest.mark.gpu

SMALL = [(4, 8, 8), (5, 6, 7), (7, 9, 11), (1, 1, 1), (3, 1, 5)]
LARGE = [WAN480.grid, HUNYUAN720.grid, LONG126.grid]
MASK_CASES = [(g, bs) for g in SMALL for bs in (16, 64, 128)] + [(g, bs) for g in LARGE for bs in (64, 128)]


@pytest.mark.parametrize("grid,bs", MASK_CASES)
def test_pattern_masks_bit_exact(grid, bs):
    announce(f"pattern mask grid={grid} bs={bs}")
    for kind, code in (("spatial", V.VSA_PATTERN_SPATIAL), ("temporal", V.VSA_PATTERN_TEMPORAL)):
        for w in (0, 1, 2, 276):
            got = host(V.vsa_pattern_mask(grid, bs, code, w))
            assert np.array_equal(got, OM.pattern_mask(grid, bs, kind, w)), (kind, w)


@pytest.mark.parametrize("grid", [(4, 8, 8), (5, 6, 7), (1, 1, 1), (21, 30, 52), (126, 30, 52)])
def test_cube_block_len(grid):
    announce(f"cube len grid={grid}")
    _, counts, _ = OL.cube_map(*grid, 4)
    assert np.array_equal(host(V.vsa_cube_block_len(grid)), counts)


@pytest.mark.parametrize("shape,density", [((1, 2, 7, 9), 0.4), ((2, 3, 33, 300), 0.1), ((1, 1, 5, 1536), 0.05),
                                           ((1, 2, 256, 256), 0.0), ((1, 1, 3, 70), 1.0)])
def test_mask_to_list(shape, density):
    announce(f"mask_to_list {shape}")
    m = (np.random.default_rng(sum(shape)).random(shape) < density).astype(np.uint8)
    idx, cnt = V.vsa_mask_to_list(dev_u8(m))
    ri, rc = OM.mask_to_list(m)
    gi, gc = host(idx), host(cnt)
    assert np.array_equal(gc, rc)
    for a, b, c in zip(gi.reshape(-1, gi.shape[-1]), ri.reshape(-1, ri.shape[-1]), rc.reshape(-1)):
        assert np.array_equal(a[:c], b[:c])


def test_mask_to_list_per_head_selection_and_cap():
    announce("mask_to_list head selection")
    P, nqb, nkb = 2, 40, 50
    m = (np.random.default_rng(1).random((P, nqb, nkb)) < 0.3).astype(np.uint8)
    sel = [1, 0, 0, 1, 1]
    idx, cnt = V.vsa_mask_to_list(dev_u8(m), head_mask_idx=sel, B=2)
    gi, gc = host(idx), host(cnt)
    for b in range(2):
        for h, p in enumerate(sel):
            ri, rc = OM.mask_to_list(m[p])
            assert np.array_equal(gc[b, h], rc)
            for qb in range(nqb):
                assert np.array_equal(gi[b, h, qb, :rc[qb]], ri[qb, :rc[qb]])
    # capacity below the kept count keeps the first max_kv blocks
    idx, cnt = V.vsa_mask_to_list(dev_u8(m[None]), max_kv=5)
    gi, gc = host(idx), host(cnt)
    ri, rc = OM.mask_to_list(m)
    assert np.array_equal(gc[0], np.minimum(rc, 5))
    for p in range(P):
        for qb in range(nqb):
            c = min(rc[p, qb], 5)
            assert np.array_equal(gi[0, p, qb, :c], ri[p, qb, :c])


@pytest.mark.parametrize("grid", [(4, 8, 8), (5, 6, 7), (3, 1, 5), (21, 30, 52)])
@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (64, torch.bfloat16), (128, torch.float32),
                                     (64, torch.float32)])
def test_frame_major_permute_bit_exact(grid, D, dtype):
    announce(f"permute frame-major grid={grid} D={D} {dtype}")
    N = int(np.prod(grid))
    H = 3
    x = np.random.default_rng(N + D).standard_normal((2, H, N, D)).astype(np.float32)
    xd = dev(x, dtype)
    xv = host(xd)
    sel = [1, 0, 1]
    y = V.vsa_permute(xd, grid, V.VSA_PERM_FRAME_MAJOR, False, sel)
    assert np.array_equal(host(y), OL.permute(xv, grid, "frame_major", False, sel))
    z = V.vsa_permute(y, grid, V.VSA_PERM_FRAME_MAJOR, True, sel)
    assert torch.equal(z, xd)
    yall = V.vsa_permute(xd, grid, V.VSA_PERM_FRAME_MAJOR)
    assert np.array_equal(host(yall), OL.permute(xv, grid, "frame_major"))


@pytest.mark.parametrize("grid", [(4, 8, 8), (5, 6, 7), (1, 1, 1), (9, 3, 13), (21, 30, 52)])
@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (64, torch.float32)])
def test_cube_permute_bit_exact(grid, D, dtype):
    announce(f"permute cube grid={grid} D={D} {dtype}")
    N = int(np.prod(grid))
    x = np.random.default_rng(N).standard_normal((1, 2, N, D)).astype(np.float32)
    xd = dev(x, dtype)
    xv = host(xd)
    y = V.vsa_permute(xd, grid, V.VSA_PERM_CUBE4)
    assert np.array_equal(host(y), OL.permute(xv, grid, "cube4"))
    z = V.vsa_permute(y, grid, V.VSA_PERM_CUBE4, inverse=True)
    assert torch.equal(z, xd)


def test_permute_full_hunyuan_shape_all_heads():
    """The permutation's benchmarked shape: HunyuanVideo 720p, all 24 heads."""
    w = HUNYUAN720
    announce("permute frame-major hunyuan 24 heads")
    N = w.N
    xd = torch.randn((1, 24, N, 128), dtype=torch.bfloat16, device="cuda", generator=torch.Generator("cuda").manual_seed(0))
    y = V.vsa_permute(xd, w.grid, V.VSA_PERM_FRAME_MAJOR)
    pi = torch.from_numpy(OL.frame_major_map(*w.grid)).cuda()
    ref = torch.empty_like(xd)
    ref[:, :, pi] = xd
    assert torch.equal(y, ref)
    assert torch.equal(V.vsa_permute(y, w.grid, V.VSA_PERM_FRAME_MAJOR, inverse=True), xd)
