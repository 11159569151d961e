"""Batch independence of the layers: a call on two batch entries gives, bit for
bit, the outputs of the two single-entry calls (every kernel of these layers
works per (batch entry, head); the split-K head profiler is the exception, its
key splits depend on B x H, and is compared with the oracle at B = 2 instead in
its own tests)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from block_sparse_attention_vsa_amd import pipelines as PL
from tests.gpu_util import announce, dev
from workloads import WAN480, make_qkv

pytestmark = pytest.mark.gpu


def two_entries(grid, H, seed, generator="sinusoid", **extra):
    w = WAN480.scaled(name="batch", T=grid[0], Hh=grid[1], W=grid[2], H=H, seed=seed, generator=generator,
                      extra=dict(WAN480.extra, **extra))
    a = make_qkv(w)
    b = make_qkv(w.scaled(seed=seed + 1))
    return [dev(x) for x in a], [dev(x) for x in b]


def check(layer, a, b, what):
    oa = layer(*a)
    ob = layer(*b)
    oab = layer(*(torch.cat((x, y), dim=0) for x, y in zip(a, b)))
    assert torch.equal(oab[0:1], oa) and torch.equal(oab[1:2], ob), f"{what}: batch entries differ from single calls"


def test_cube_layer_batch():
    announce("batch: cube layer")
    grid = (8, 12, 16)
    a, b = two_entries(grid, 3, 51)
    check(lambda q, k, v: PL.cube_layer(q, k, v, grid, 0.15, 0.9), a, b, "cube layer")


def test_long_layer_batch():
    announce("batch: long layer")
    grid = (12, 8, 16)
    a, b = two_entries(grid, 2, 53)
    check(lambda q, k, v: PL.long_layer(q, k, v, grid, 128, 1, 4), a, b, "long layer")


@pytest.mark.parametrize("mode", [V.VSA_SKIPARSE_TOKEN, V.VSA_SKIPARSE_GROUP])
def test_skiparse_layer_batch(mode):
    announce(f"batch: skiparse mode {mode}")
    grid = (3, 10, 12)
    a, b = two_entries(grid, 2, 55)
    check(lambda q, k, v: PL.skiparse_layer(q, k, v, grid, mode, 2, 64), a, b, "skiparse layer")


def test_semantic_layer_batch():
    announce("batch: semantic layer")
    grid = (4, 12, 20)
    a, b = two_entries(grid, 2, 57, generator="mixture", n_components=8, mean_scale=0.75)
    check(lambda q, k, v: PL.semantic_layer(q, k, v, 16, 32, 2, 0.9), a, b, "semantic layer")
