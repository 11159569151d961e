"""Seeded synthetic inputs for block-sparse attention over a 3D video token grid.

This module only draws random numbers and fixes workload shapes. It holds no step
of the method itself (no mask rule, no layout map, no pooling, no selection, no
attention): both the HIP path and the CPU oracle consume what it returns, so it
must stay free of the arithmetic they are compared on.

Every tensor is drawn in fp32 by ``numpy.random.default_rng([seed, stream])``
with stream ids Q=0, K=1, V=2, profiler rows=3, generator parameters=4 and
per-head random masks 100+h, then rounded to bf16 (round-to-nearest-even, via
torch's CPU cast) unless the workload is fp32.

The shapes stand in for the video diffusion transformers the pages measure on
(Wan 2.1 1.3B at 480p, HunyuanVideo at 720p, a 6x-longer Wan horizon); no
trained weights or benchmark items are used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

STREAM_Q, STREAM_K, STREAM_V, STREAM_ROWS, STREAM_PARAMS = 0, 1, 2, 3, 4
STREAM_MASK_BASE = 100


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    D: int
    T: int
    Hh: int
    W: int
    bs: int
    dtype: str            # "bf16" or "f32"
    seed: int
    generator: str        # "gaussian", "sinusoid", "mixture", "sinusoid_outliers"
    amplitude: float = 0.5
    extra: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        return self.T * self.Hh * self.W

    @property
    def nb(self) -> int:
        return -(-self.N // self.bs)

    @property
    def grid(self):
        return (self.T, self.Hh, self.W)

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workloads. Sizes follow the latent grids of the video models the pages
# name; masks and budgets are arguments of the path, listed in ``extra``.
TINY = Workload("tiny_4x8x8", B=1, H=2, D=64, T=4, Hh=8, W=8, bs=64, dtype="f32",
                seed=0, generator="gaussian", extra=dict(mask_density=0.5))
WAN480 = Workload("wan2.1_480p_21x30x52", B=1, H=12, D=128, T=21, Hh=30, W=52, bs=128,
                  dtype="bf16", seed=1, generator="sinusoid",
                  extra=dict(w_spatial=1, w_temporal=0, profile_frac=0.01))
HUNYUAN720 = Workload("hunyuan_720p_33x45x80", B=1, H=24, D=128, T=33, Hh=45, W=80, bs=128,
                      dtype="bf16", seed=2, generator="sinusoid",
                      extra=dict(w_spatial=2, w_temporal=276))
WAN480_CUBE = Workload("wan2.1_480p_cube4_topp", B=1, H=12, D=128, T=21, Hh=30, W=52, bs=64,
                       dtype="bf16", seed=3, generator="mixture",
                       extra=dict(cube=4, n_components=32, mean_scale=0.5,
                                  k_frac=0.15, top_p=0.9))
LONG126 = Workload("long_horizon_126x30x52", B=1, H=12, D=128, T=126, Hh=30, W=52, bs=128,
                   dtype="bf16", seed=4, generator="sinusoid_outliers",
                   extra=dict(w_local=1, density=0.10, outlier_frac=0.03, outlier_logit=3.0))

# Sparse VideoGen2-style layer on the Wan shape: 64 spatially coherent semantic
# components, k-means with 128 query and 256 key clusters, size-weighted top-p 0.9.
WAN480_SEMANTIC = Workload("wan2.1_480p_semantic", B=1, H=12, D=128, T=21, Hh=30, W=52, bs=128,
                           dtype="bf16", seed=5, generator="mixture",
                           extra=dict(n_components=64, mean_scale=0.75, Cq=128, Ck=256, iters=3, top_p=0.9))

ALL = [TINY, WAN480, HUNYUAN720, WAN480_CUBE, LONG126, WAN480_SEMANTIC]
BY_NAME = {w.name: w for w in ALL}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, stream])


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) and return them as fp32 (exactly representable)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def sinusoid_features(T: int, Hh: int, W: int, D: int = 128) -> np.ndarray:
    """Per-token positional features f(t, y, x) in natural token order, shape [N, D].

    The D channels are split over the three axes (t gets the remainder), each axis
    filled with interleaved [sin(p w_j), cos(p w_j)] pairs, w_j = 10000^(-2j/d_axis).
    """
    d_y = d_x = (D // 3) // 2 * 2
    d_t = D - d_y - d_x
    tt, yy, xx = np.meshgrid(np.arange(T), np.arange(Hh), np.arange(W), indexing="ij")
    out = np.empty((T * Hh * W, D), np.float64)
    col = 0
    for p, d_axis in ((tt.ravel(), d_t), (yy.ravel(), d_y), (xx.ravel(), d_x)):
        for j in range(d_axis // 2):
            w = 10000.0 ** (-2.0 * j / d_axis)
            out[:, col + 2 * j] = np.sin(p * w)
            out[:, col + 2 * j + 1] = np.cos(p * w)
        col += d_axis
    return out.astype(np.float32)


def axis_gate(H: int, D: int = 128) -> np.ndarray:
    """0/1 gate [H, D]: even heads see the t channels (a same-frame, spatial-type
    head), odd heads see the y,x channels (a same-position, temporal-type head)."""
    d_y = d_x = (D // 3) // 2 * 2
    d_t = D - d_y - d_x
    g = np.zeros((H, D), np.float32)
    g[0::2, :d_t] = 1.0
    g[1::2, d_t:] = 1.0
    return g


def planted_head_type(H: int) -> np.ndarray:
    """0 = spatial-type (even heads), 1 = temporal-type (odd heads)."""
    return (np.arange(H) % 2).astype(np.int32)


def _normal(seed, stream, shape):
    return rng(seed, stream).standard_normal(shape, dtype=np.float32)


def make_qkv(w: Workload, B: int | None = None, H: int | None = None):
    """Draw Q, K, V of shape [B, H, N, D] as fp32 arrays holding the exact input
    values (bf16-representable for bf16 workloads)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    N, D = w.N, w.D
    shape = (B, H, N, D)
    q = _normal(w.seed, STREAM_Q, shape)
    k = _normal(w.seed, STREAM_K, shape)
    v = _normal(w.seed, STREAM_V, shape)
    if w.generator in ("sinusoid", "sinusoid_outliers"):
        f = sinusoid_features(w.T, w.Hh, w.W, D)            # [N, D]
        g = axis_gate(H, D)                                 # [H, D]
        add = w.amplitude * g[:, None, :] * f[None, :, :]   # [H, N, D]
        q += add[None]
        k += add[None]
        del add
        if w.generator == "sinusoid_outliers":
            pr = rng(w.seed, STREAM_PARAMS)
            nb = w.nb
            n_out = int(round(w.extra["outlier_frac"] * nb))
            blocks = np.sort(pr.choice(nb, size=n_out, replace=False))
            u = pr.standard_normal(D)
            u = (u / np.linalg.norm(u)).astype(np.float32)
            q += u
            amp = np.float32(w.extra["outlier_logit"] * math.sqrt(D))
            for b in blocks:
                k[:, :, b * w.bs:min((b + 1) * w.bs, N), :] += amp * u
    elif w.generator == "mixture":
        pr = rng(w.seed, STREAM_PARAMS)
        C = w.extra["n_components"]
        s = w.extra["mean_scale"]
        centres = pr.uniform(0.0, 1.0, size=(C, 3)) * np.array([w.T, w.Hh, w.W])
        means = (s * pr.standard_normal((H, C, D))).astype(np.float32)
        tt, yy, xx = np.meshgrid(np.arange(w.T), np.arange(w.Hh), np.arange(w.W), indexing="ij")
        pos = np.stack([tt.ravel(), yy.ravel(), xx.ravel()], 1).astype(np.float64)
        d2 = ((pos[:, None, :] - centres[None, :, :]) ** 2).sum(-1)
        z = np.argmin(d2, axis=1)                            # nearest centre per token
        mu = means[:, z, :]                                  # [H, N, D]
        q += mu[None]
        k += mu[None]
    elif w.generator != "gaussian":
        raise ValueError(w.generator)
    if w.dtype == "bf16":
        q, k, v = to_bf16_values(q), to_bf16_values(k), to_bf16_values(v)
    return q, k, v


def outlier_blocks(w: Workload) -> np.ndarray:
    """The key blocks (natural layout) that received a planted outlier."""
    pr = rng(w.seed, STREAM_PARAMS)
    n_out = int(round(w.extra["outlier_frac"] * w.nb))
    return np.sort(pr.choice(w.nb, size=n_out, replace=False))


def random_block_mask(w: Workload, H: int | None = None) -> np.ndarray:
    """Per-head random block mask [H, nb, nb] (uint8) with the diagonal always kept
    and an exact count of round(density * nb^2) kept blocks per head."""
    H = w.H if H is None else H
    nb = w.nb
    total = int(round(w.extra["mask_density"] * nb * nb))
    out = np.zeros((H, nb, nb), np.uint8)
    off = [(i, j) for i in range(nb) for j in range(nb) if i != j]
    for h in range(H):
        r = rng(w.seed, STREAM_MASK_BASE + h)
        pick = r.choice(len(off), size=total - nb, replace=False)
        out[h, np.arange(nb), np.arange(nb)] = 1
        for p in pick:
            out[h, off[p][0], off[p][1]] = 1
    return out


def profile_rows(w: Workload, frac: float = 0.01) -> np.ndarray:
    """ceil(frac * N) distinct query rows (natural order), sorted, shared by all heads."""
    R = int(math.ceil(frac * w.N))
    return np.sort(rng(w.seed, STREAM_ROWS).choice(w.N, size=R, replace=False)).astype(np.int32)


def sample_rows(N: int, bs: int, n_random: int, seed: int, stream: int = 7) -> np.ndarray:
    """Rows for sampled parity at large N: the first and last row of every block
    plus ``n_random`` seeded rows, sorted and unique."""
    nb = -(-N // bs)
    first = np.arange(nb) * bs
    last = np.minimum(first + bs, N) - 1
    rnd = rng(seed, stream).choice(N, size=min(n_random, N), replace=False)
    return np.unique(np.concatenate([first, last, rnd])).astype(np.int64)
