"""The Sparse VideoGen step (pattern masks -> head profiler -> attention that
reads each head's choice on the device) has no host round trip, so it can be
captured once in a HIP graph and replayed. Every replay is checked bit for bit
against the eager run, with eager work and synchronisations between replays,
and with the inputs refilled in place (so a replay must recompute)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from block_sparse_attention_vsa_amd import pipelines as PL
from tests.gpu_util import announce
from workloads import WAN480, make_qkv, profile_rows

pytestmark = pytest.mark.gpu


def test_svg_step_replays_in_a_hip_graph():
    w = WAN480.scaled(name="graph", T=6, H=4)
    announce("svg step in a HIP graph")
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in make_qkv(w))
    g = np.random.default_rng(3)
    alt = [torch.from_numpy(g.standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16).to(dev)
           for _ in range(3)]
    rows = torch.from_numpy(profile_rows(w)).to(dev)
    ws = torch.empty((V.vsa_profile_workspace_bytes(1, w.H, w.grid, 128, rows.numel(), 2),), dtype=torch.uint8,
                     device=dev)

    def step():
        cand = PL.svg_masks(w.grid, w.bs, 1, 0, dev)
        _, ch = V.vsa_profile_heads(q, k, v, w.grid, w.bs, rows, cand, [0, 1], workspace=ws)
        o = V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], ch)
        return o, ch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                           # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g, ch_g = step()
    torch.cuda.synchronize()
    for rep in range(4):
        src = alt[rep % 3] if rep else None
        if src is not None:                              # new inputs, same buffers
            q.copy_(src)
            k.copy_(src.flip(2).contiguous())
        o_ref, ch_ref = step()                           # eager on the same inputs
        torch.cuda.synchronize()
        o_ref, ch_ref = o_ref.clone(), ch_ref.clone()
        torch.randn(1 << 20, device=dev).sum().item()    # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ch_g, ch_ref), f"replay {rep}: choice"
        assert torch.equal(o_g, o_ref), f"replay {rep}: output"


LAYERS = {
    "cube": ((8, 12, 16), lambda q, k, v, grid: PL.cube_layer(q, k, v, grid, 0.15, 0.9)),
    "long": ((12, 8, 16), lambda q, k, v, grid: PL.long_layer(q, k, v, grid, 128, 1, 4)),
    "skiparse": ((3, 10, 12), lambda q, k, v, grid: PL.skiparse_layer(q, k, v, grid, V.VSA_SKIPARSE_GROUP, 2, 64)),
    "semantic": ((4, 12, 20), lambda q, k, v, grid: PL.semantic_layer(q, k, v, 16, 32, 2, 0.9)),
}


@pytest.mark.parametrize("name", list(LAYERS))
def test_layers_replay_in_a_hip_graph(name):
    """The other four flows have no host round trip either: each is captured
    once, replayed on refilled inputs with eager work between replays, and every
    replay equals the eager run bit for bit."""
    grid, layer = LAYERS[name]
    announce(f"{name} layer in a HIP graph")
    w = WAN480.scaled(name="graph_" + name, T=grid[0], Hh=grid[1], W=grid[2], H=2)
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in make_qkv(w))
    g = np.random.default_rng(7)
    alt = [torch.from_numpy(g.standard_normal(q.shape).astype(np.float32)).to(torch.bfloat16).to(dev)
           for _ in range(3)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer(q, k, v, grid)                             # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        o_g = layer(q, k, v, grid)
    torch.cuda.synchronize()
    for rep in range(4):
        if rep:                                          # new inputs, same buffers
            q.copy_(alt[rep % 3])
            k.copy_(alt[(rep + 1) % 3])
            v.copy_(alt[(rep + 2) % 3])
        o_ref = layer(q, k, v, grid).clone()             # eager on the same inputs
        torch.cuda.synchronize()
        torch.randn(1 << 20, device=dev).sum().item()    # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_ref), f"{name} replay {rep}: output differs from eager"
