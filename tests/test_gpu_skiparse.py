"""GPU parity of the Skiparse-2D path (OSP-Next page, "Method"; reading in
oracle/skiparse.py) against the oracle: the padded subset-major permutation,
block lengths and block-diagonal mask bit-exact; the whole layer (permute ->
block-sparse attention -> inverse permute) element by element on small ragged
grids and on sampled rows at the Wan 480p shape."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from block_sparse_attention_vsa_amd import pipelines as PL
from oracle import skiparse as SK
from tests.gpu_util import announce, assert_close_bf16, assert_lse_close, dev, dev_i32, host
from workloads import WAN480, make_qkv, sample_rows

pytestmark = pytest.mark.gpu

MODES = {"token": V.VSA_SKIPARSE_TOKEN, "group": V.VSA_SKIPARSE_GROUP}


@pytest.mark.parametrize("grid,k,bs", [((2, 9, 7), 3, 64), ((3, 6, 10), 2, 128), ((2, 17, 23), 4, 64),
                                       ((1, 4, 4), 1, 64)])
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (64, torch.float32)])
def test_layout_bit_exact(grid, k, bs, mode, D, dtype):
    announce(f"skiparse layout grid={grid} k={k} bs={bs} {mode} D={D}")
    N = int(np.prod(grid))
    x = torch.from_numpy(np.random.default_rng(N + k).standard_normal((1, 3, N, D)).astype(np.float32)).to(dtype).cuda()
    m = MODES[mode]
    fwd = V.vsa_skiparse_permute(x, grid, m, k, bs)
    ref = SK.permute(x.float().cpu().numpy(), grid, k, mode, bs)
    assert torch.equal(fwd.float().cpu(), torch.from_numpy(ref).float())
    assert torch.equal(V.vsa_skiparse_permute(fwd, grid, m, k, bs, inverse=True), x)
    _, blk, _ = SK.layout(grid, k, mode, bs)
    assert (host(V.vsa_skiparse_block_len(grid, m, k, bs)) == blk).all()
    assert (host(V.vsa_skiparse_mask(grid, m, k, bs)) == SK.block_mask(grid, k, mode, bs)).all()


@pytest.mark.parametrize("grid,k,bs", [((2, 9, 7), 3, 64), ((3, 6, 10), 2, 128), ((2, 8, 12), 2, 64),
                                       ((1, 3, 3), 3, 64)])
@pytest.mark.parametrize("mode", list(MODES))
def test_layer_full_oracle_small(grid, k, bs, mode):
    announce(f"skiparse layer grid={grid} k={k} bs={bs} {mode}")
    N = int(np.prod(grid))
    g = np.random.default_rng(N * 3 + k)
    qd, kd, vd = (dev(g.standard_normal((1, 2, N, 128)).astype(np.float32)) for _ in range(3))
    q, kk, v = host(qd), host(kd), host(vd)
    stats = {}
    o = PL.skiparse_layer(qd, kd, vd, grid, MODES[mode], k, bs, stats=stats)
    ro, _ = SK.attention(q, kk, v, grid, k, mode)
    assert_close_bf16(host(o), ro, f"skiparse {mode} grid={grid} k={k}")
    # the attention in the padded layout, with its LSE, against the oracle's own layout
    blk = stats["blk_len"]
    _, lse = V.vsa_block_sparse_attn_fwd(*stats["permuted"], bs, kv_idx=stats["kv_idx"], kv_cnt=stats["kv_cnt"],
                                         blk_len=blk, return_lse=True)
    slot, _, _ = SK.layout(grid, k, mode, bs)
    _, rl = SK.attention(q, kk, v, grid, k, mode)
    assert_lse_close(host(lse)[:, :, slot], rl, f"skiparse lse {mode}")


@pytest.mark.parametrize("mode", list(MODES))
def test_layer_wan_full_shape_sampled(mode):
    """Wan 480p (12 heads, 21 x 30 x 52 tokens), k = 2, bs 128: the permuted Q
    equals the oracle's move bit for bit, and O on every block's first and last
    row plus seeded rows equals the oracle's Skiparse-2D attention."""
    w = WAN480
    announce(f"skiparse wan full shape {mode}")
    q, k, v = make_qkv(w)
    stats = {}
    o = PL.skiparse_layer(dev(q), dev(k), dev(v), w.grid, MODES[mode], 2, 128, stats=stats)
    qs = stats["permuted"][0]
    ref_qs = SK.permute(host(dev(q[:, :2])), w.grid, 2, mode, 128)
    assert np.array_equal(host(qs[:, :2]), ref_qs)
    rows = sample_rows(w.N, w.bs, 768, 23)
    ro, _ = SK.attention(q, k, v, w.grid, 2, mode, rows=rows)
    assert_close_bf16(host(o)[:, :, rows], ro, f"skiparse wan {mode}")
