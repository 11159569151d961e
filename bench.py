"""Benchmark of block-sparse video attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

One step = one pass of the Sparse VideoGen layer over a Wan-2.1-1.3B-shaped 480p
layer (B=1, H=12, D=128, 21x30x52 latent tokens, bf16): pattern masks, the 1 %-row
per-head profiler, frame-major permutation of Q, K, V for temporal heads,
mask -> block lists, block-sparse attention, inverse permutation of O. Inputs sit
in HBM before the timed region. Prints one JSON line.

`value` is the step's effective throughput: kept attention flops (4 D per valid
query-key pair of every kept block) divided by the step time. `roofline`
describes the attention kernel alone, timed with HIP events on its own stream.
`extra_layers` times the other layers of the pages at their shapes (the 6/6
spatial/temporal split, the backward, FP8, Skiparse-2D, HunyuanVideo, the cube
top-p/top-k layer, the long horizon, the semantic layer), each step as device
work queued behind a lead spin so that no host latency sits inside an event
pair, with dense attention at the same shape for the speedups. `cpu_baseline`
is the fp64 CPU oracle on a sample of query blocks of the same workload, on this
host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import (WAN480, WAN480_CUBE, WAN480_SEMANTIC, LONG126, HUNYUAN720, make_qkv,  # noqa: E402
                       profile_rows, rng)

PEAK_BF16_TFLOPS = 2516.6       # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5033.2        # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the cube and long-horizon sub-step timings")
    ap.add_argument("--cpu-sample-blocks", type=int, default=256, help="query blocks per head for the CPU oracle")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB three times (HBM counter calibration)")
    ap.add_argument("--cpu-leg", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--choice", type=str, default="", help=argparse.SUPPRESS)
    return ap.parse_args()


# ----------------------------------------------------------------- CPU leg ---
def _cpu_worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


_CPU = {}


def _cpu_unit(args):
    from oracle.attention import masked_attention
    h, qb = args
    q, k, v, blk_by_head, mask_by_head, bs = (_CPU[x] for x in ("q", "k", "v", "blk", "mask", "bs"))
    blk = blk_by_head[h]
    rows = np.nonzero(blk == qb)[0]
    t0 = time.perf_counter()
    masked_attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], mask_by_head[h], blk, blk, rows=rows)
    return time.perf_counter() - t0


def cpu_leg(args):
    """Child program (never touches the GPU): regenerates the step's inputs, builds
    the two candidate masks with the oracle and times the oracle's attention, then
    the oracle's other steps on small samples (one JSON line each)."""
    from oracle.masks import pattern_mask
    w = WAN480
    q, k, v = make_qkv(w)
    choice = [int(c) for c in args.choice.split(",")]
    m_s = pattern_mask(w.grid, w.bs, "spatial", w.extra["w_spatial"])
    m_t = pattern_mask(w.grid, w.bs, "temporal", w.extra["w_temporal"])
    print(json.dumps(cpu_baseline(q, k, v, choice, m_s, m_t, args.cpu_sample_blocks)), flush=True)
    print(json.dumps(cpu_rows(q, k, v, m_s, m_t)), flush=True)


def cpu_rows(q, k, v, m_s, m_t):
    """The oracle's other steps of the layer, each on a bounded sample, in this one
    process: wall time of the call as it stands (fp64 numpy)."""
    from oracle.layout import permute
    from oracle.masks import pattern_mask
    from oracle.profile import profile_heads
    from oracle.scores import block_scores
    from oracle.select import select
    w = WAN480
    N, D = w.N, w.D

    def wall(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    out = {}
    t = wall(lambda: (pattern_mask(w.grid, w.bs, "spatial", w.extra["w_spatial"]),
                      pattern_mask(w.grid, w.bs, "temporal", w.extra["w_temporal"])))
    out["a1_pattern_masks"] = {"ms": round(t * 1e3, 3), "sample": "both candidate masks of the Wan grid (all of a1)"}
    t = wall(lambda: permute(q[:, :1], w.grid, "frame_major"))
    out["a3_permute"] = {"ms": round(t * 1e3, 3), "GBps": round(2 * N * D * 2 / t / 1e9, 3),
                         "sample": "frame-major move of one head of Q (32,760 x 128), bytes counted as bf16 read + write"}
    t = wall(lambda: block_scores(q[:, :1], k[:, :1], w.bs))
    out["a4_block_scores"] = {"ms": round(t * 1e3, 3), "sample": "pooling and pooled scores of one head, bs 128"}
    nc = WAN480_CUBE.extra.get("cube", 4)
    ncube = -(-w.T // nc) * -(-w.Hh // nc) * -(-w.W // nc)
    sc = rng(0, 99).standard_normal((1, 1, ncube, ncube))
    k_max = int(WAN480_CUBE.extra["k_frac"] * ncube)
    t = wall(lambda: select(sc, None, k_max, WAN480_CUBE.extra["top_p"]))
    out["a5_select"] = {"ms": round(t * 1e3, 3),
                        "sample": f"top-p {WAN480_CUBE.extra['top_p']} / k_max {k_max} over one head's {ncube} x {ncube} "
                                  "cube scores (seeded normal scores)"}
    rows = profile_rows(w, w.extra["profile_frac"])
    sub = rows[:: max(1, rows.size // 32)][:32]
    t = wall(lambda: profile_heads(q[:, :1], k[:, :1], v[:, :1], w.grid, w.bs, sub, [m_s, m_t], [0, 1]))
    out["a2_profile"] = {"ms": round(t * 1e3, 3), "ms_per_row": round(t * 1e3 / sub.size, 3),
                         "sample": f"one head, {sub.size} of the step's {rows.size} sampled rows (the step profiles "
                                   f"{w.H} x {rows.size} rows), dense output and both candidates"}
    out["what"] = ("the oracle's other steps timed beside this run's GPU figures (components_ms, permute_standalone, "
                   "extra_layers.cube_topp_wan480); one process, fp64")
    return out


def run_cpu_leg(choice, blocks_per_head):
    """(cpu_baseline, oracle row timings) from the child program, or (None, None)."""
    import subprocess
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-leg", "--choice", ",".join(str(int(c)) for c in choice),
           "--cpu-sample-blocks", str(blocks_per_head)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    if res.returncode != 0:
        print(f"bench.py: CPU baseline leg failed:\n{res.stderr[-2000:]}", file=sys.stderr)
        return None, None
    lines = [ln for ln in res.stdout.strip().splitlines() if ln.startswith("{")]
    return json.loads(lines[0]), (json.loads(lines[1]) if len(lines) > 1 else None)


def cpu_baseline(q, k, v, choice, m_s, m_t, blocks_per_head):
    """Times the oracle's masked attention on a sample of query blocks (all heads,
    evenly spaced blocks), in a fork pool of one single-threaded worker per core."""
    import multiprocessing as mp
    from oracle.layout import frame_major_map
    w = WAN480
    bs = w.bs
    N = w.N
    blk_nat = np.arange(N) // bs
    blk_fm = frame_major_map(*w.grid) // bs
    H = q.shape[1]
    _CPU.update(q=q.astype(np.float64), k=k.astype(np.float64), v=v.astype(np.float64), bs=bs,
                blk=[blk_fm if choice[h] else blk_nat for h in range(H)],
                mask=[m_t if choice[h] else m_s for h in range(H)])
    nb = w.nb
    picks = np.unique(np.linspace(0, nb - 1, blocks_per_head).round().astype(int))
    units = [(h, int(qb)) for h in range(H) for qb in picks]
    # kept flops of the sample: 4 D per valid (query, key) pair
    nblk = np.full(nb, bs, np.int64)
    nblk[-1] = N - (nb - 1) * bs
    flops = 0.0
    for h, qb in units:
        m = m_t if choice[h] else m_s
        flops += 4.0 * w.D * nblk[qb] * float((m[qb].astype(np.int64) * nblk).sum())
    cores = min(os.cpu_count() or 1, 16)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(cores, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_unit, units, chunksize=1)
    wall = time.perf_counter() - t0
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / wall / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 numpy oracle masked attention on {len(units)} query blocks "
                       f"({len(picks)} evenly spaced per head x {H} heads) of the Wan 480p layer with the "
                       f"step's per-head masks; {flops:.3e} kept flops in {wall:.2f} s wall; "
                       f"one single-threaded worker per core; host CPU {model}")}


# ------------------------------------------------------------------ helpers --
def kept_flops_from_lists(kv_idx, kv_cnt, N, bs, D, blk_len=None):
    """4 D * sum over kept (query block, key block) of valid_q * valid_k."""
    idx = kv_idx.cpu().numpy()
    cnt = kv_cnt.cpu().numpy()
    nb = -(-N // bs)
    if blk_len is None:
        n = np.full(nb, bs, np.int64)
        n[-1] = N - (nb - 1) * bs
    else:
        n = blk_len.cpu().numpy().astype(np.int64)
    total = 0.0
    mv = idx.shape[-1]
    fi = idx.reshape(-1, nb, mv)
    fc = cnt.reshape(-1, nb)
    for u in range(fi.shape[0]):
        ar = np.arange(mv)[None, :] < fc[u][:, None]
        kn = np.where(ar, n[np.clip(fi[u], 0, nb - 1)], 0).sum(1)
        total += float((n * kn).sum())
    return 4.0 * D * total


def source_digest(*names):
    h = hashlib.sha256()
    for nme in names:
        with open(os.path.join(ROOT, "block_sparse_attention_vsa_amd", "csrc", nme), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_key, digest):
    """HBM bytes per launch measured with rocprofv3 counters for this exact source
    (profiles/traffic.json), or None when the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_digest") != digest:
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.acc = {}

    def ev(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def lead(self, ms=3.0):
        """A device spin of about `ms` milliseconds (at most; the counter runs at
        the shader clock) queued before timed work: the host queues the timed
        calls while the GPU is still busy, so the event pairs that follow bracket
        device work only, never the host's launch latency."""
        self.torch.cuda._sleep(int(ms * 2.4e6))

    def per_call_ms(self, fn, reps, warm=1):
        """Device time of fn per call: `reps` calls queued back to back behind a
        lead spin long enough for the host to queue all of them."""
        for _ in range(warm):
            fn()
        self.torch.cuda.synchronize()
        self.lead(max(3.0, 0.3 * reps))
        e0 = self.ev()
        for _ in range(reps):
            fn()
        e1 = self.ev()
        self.torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def add(self, key, e0, e1):
        self.acc.setdefault(key, []).append((e0, e1))

    def mean_ms(self, key):
        self.torch.cuda.synchronize()
        pairs = self.acc.get(key, [])
        return sum(a.elapsed_time(b) for a, b in pairs) / max(1, len(pairs))


# --------------------------------------------------------------------- main --
def main():
    args = parse()
    if args.cpu_leg:
        cpu_leg(args)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); the per-head work "
              f"shards across GPUs with no exchange, which is not exercised here.", file=sys.stderr)
        sys.exit(2)

    w = WAN480
    q_np, k_np, v_np = make_qkv(w)
    rows_np = profile_rows(w, w.extra["profile_frac"])

    import torch
    import block_sparse_attention_vsa_amd as V
    from block_sparse_attention_vsa_amd import pipelines as PL

    dev = torch.device("cuda:0")
    q = torch.from_numpy(q_np).to(torch.bfloat16).to(dev)
    k = torch.from_numpy(k_np).to(torch.bfloat16).to(dev)
    v = torch.from_numpy(v_np).to(torch.bfloat16).to(dev)
    rows = torch.from_numpy(rows_np).to(dev)
    B, H, N, D = q.shape
    bs = w.bs
    grid = w.grid
    ws = torch.empty((V.vsa_profile_workspace_bytes(B, H, grid, D, rows.numel(), 2),), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    T = Timer(torch)
    ws_s, ws_t = w.extra["w_spatial"], w.extra["w_temporal"]

    def step(timed):
        e0 = T.ev()
        cand = PL.svg_masks(grid, bs, ws_s, ws_t, dev)
        e1 = T.ev()
        _, ch = V.vsa_profile_heads(q, k, v, grid, bs, rows, cand, [0, 1], workspace=ws)
        e2 = T.ev()
        # a6 + a3 + a7 + a8 in one launch: the kernel reads each head's choice,
        # compacts the chosen mask row and applies the frame-major order of
        # temporal heads in its loads and stores; no host round trip in the step
        o = V.vsa_block_sparse_attn_fwd_chosen(q, k, v, grid, bs, cand, [0, 1], ch)
        e3 = T.ev()
        if timed:
            for key, a, b in (("a1_pattern_masks", e0, e1), ("a2_profile", e1, e2),
                              ("a3_a6_a7_a8_attention", e2, e3)):
                T.add(key, a, b)
        return o, ch, cand

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        o, ch, cand = step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # kept blocks of the last step's choice (outside the timed region)
    sel = [int(c) for c in ch[0].cpu().tolist()]
    idx, cnt = V.vsa_mask_to_list(cand, head_mask_idx=sel, B=B)
    flops = kept_flops_from_lists(idx, cnt, N, bs, D)
    attn_ms = T.mean_ms("a3_a6_a7_a8_attention")
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    comp = {key: round(T.mean_ms(key), 4) for key in T.acc}

    # dense baselines at the same [B, H, N, D]
    dense = dense_baselines(torch, V, T, q, k, v, bs)
    dense_ours, dense_sdpa, dense_ms = dense["ours_all_blocks"], dense["torch_sdpa"], dense["best"]

    n_moved = sum(sel)
    # the standalone permutation kernel (a3 / a8 as separate calls), every head
    # moved: read + write of one [B, H, N, D] tensor per call
    all_heads = [1] * H
    pdst = torch.empty_like(q)
    perm_ms = T.per_call_ms(lambda: V.vsa_permute(q, grid, V.VSA_PERM_FRAME_MAJOR, False, all_heads, out=pdst), 10)
    perm_gbs = 2 * q.numel() * q.element_size() / (perm_ms * 1e-3) / 1e9
    del pdst

    # the step's attention launch alone, warm and cold, and what this GPU reaches on plain work
    kstats = launch_stats(torch, T, lambda: V.vsa_block_sparse_attn_fwd_chosen(q, k, v, grid, bs, cand, [0, 1], ch),
                          flops)
    achievable = achievable_peaks(torch, T)

    extra = {}
    if not args.no_extra:
        extra = extra_layers(torch, V, PL, T, dense, attn_tflops, kstats["warm"]["tflops_at_median"])

    digest = source_digest("attn_fwd.hip", "mfma_tile.h", "vsa_internal.h")
    # the chosen-candidate launch carries the frame-major loop whenever a
    # candidate is frame-major (decided on the device per head)
    kname = "attn_fwd_bf16_d128_kernel<128, true>"
    traffic = stored_traffic(f"{kname}/wan480_svg", digest)
    roofline = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "kernel": kname, "per_launch_flops": flops,
                "avg_launch_ms": round(attn_ms, 4),
                "frac_of_achievable": round(attn_tflops / achievable["bf16_gemm_tflops"], 4)}

    cpu, cpu_steps = None, None
    if not args.no_cpu_baseline:
        cpu, cpu_steps = run_cpu_leg(sel, args.cpu_sample_blocks)

    if args.copy_calibration_mib:
        src = torch.empty((args.copy_calibration_mib << 20,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    value = flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "effective TFLOP/s on kept blocks (bf16), % MFMA peak, speedup vs dense attn",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "wan2.1-1.3B 480p layer, Sparse VideoGen step (profile 1% rows, spatial w=1 / "
                               "temporal w=0 per head; the attention kernel reads the choice, the chosen mask and the frame-major order of temporal heads itself)",
                   "B": B, "H": H, "N": N, "D": D, "grid": list(grid), "block": bs,
                   "heads_temporal": int(n_moved), "kept_block_density": round(float(cnt.sum().item()) / (B * H * w.nb * w.nb), 4)},
        "pct_mfma_peak_step": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "pct_mfma_peak_kernel": round(100 * attn_tflops / PEAK_BF16_TFLOPS, 2),
        "speedup_vs_dense_kernel": round(dense_ms / attn_ms, 2),
        "speedup_vs_dense_step": round(dense_ms / ms_step, 2),
        "dense_ms": {"ours_all_blocks": round(dense_ours, 3), "torch_sdpa": None if dense_sdpa is None else round(dense_sdpa, 3)},
        "components_ms": comp,
        "attention_launch_stats": kstats,
        "achievable_peaks": achievable,
        "environment": environment(torch),
        "permute_standalone": {"ms": round(perm_ms, 4), "GBps": round(perm_gbs, 1),
                               "frac_of_hbm_peak": round(perm_gbs / 8000.0, 3),
                               "frac_of_copy": round(perm_gbs / achievable["copy_GBps"], 3),
                               "what": "vsa_permute frame-major, all 12 heads of one [1,12,32760,128] bf16 tensor"},
        "extra_layers": extra,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_oracle_steps": cpu_steps,
    }
    print(json.dumps(out), flush=True)


def dense_baselines(torch, V, T, q, k, v, bs, reps=3):
    """Dense attention at the shape of q: this library with every tile kept (the
    all-ones block mask) and torch's scaled_dot_product_attention; `best` is the
    faster, the denominator of a speedup. A backend torch lacks at this size is
    reported as None."""
    B, H, N, D = q.shape
    nb = -(-N // bs)
    ones = torch.ones((B, H, nb, nb), dtype=torch.uint8, device=q.device)
    ours = T.per_call_ms(lambda: V.vsa_block_sparse_attn_fwd(q, k, v, bs, mask=ones), reps)
    del ones
    sdpa = None
    try:
        import torch.nn.functional as F
        sdpa = T.per_call_ms(lambda: F.scaled_dot_product_attention(q, k, v), reps)
    except Exception as ex:   # report, do not hide
        print(f"bench.py: torch SDPA baseline failed at N={N}: {str(ex)[:200]}", file=sys.stderr)
    torch.cuda.empty_cache()
    best = min(x for x in (ours, sdpa) if x is not None)
    return {"ours_all_blocks": round(ours, 3), "torch_sdpa": None if sdpa is None else round(sdpa, 3),
            "best": best, "dense_flops": 4.0 * B * H * N * N * D}


def launch_stats(torch, T, fn, flops, runs=50, warm=5, flush_bytes=1 << 30):
    """One kernel launch timed alone: `runs` launches after `warm`, each bracketed
    by HIP events on the current stream behind a lead spin (so the bracket holds
    no host latency); warm (inputs left in the caches by the previous launch) and
    cold (a 1 GiB buffer written before each launch, which evicts L2 and the
    256 MB MALL). Median, p10, p90 in ms and TFLOP/s at the median."""
    dev = torch.device("cuda:0")
    buf = torch.empty((flush_bytes,), dtype=torch.uint8, device=dev)
    out = {}
    for mode in ("warm", "cold"):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ts = []
        for i in range(runs):
            T.lead(1.0)                      # the launch below is queued before the GPU gets to it
            if mode == "cold":
                buf.fill_(i & 255)
            e0 = T.ev()
            fn()
            e1 = T.ev()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ts = np.array(ts)
        med = float(np.median(ts))
        out[mode] = {"median_ms": round(med, 4), "p10_ms": round(float(np.percentile(ts, 10)), 4),
                     "p90_ms": round(float(np.percentile(ts, 90)), 4),
                     "tflops_at_median": round(flops / (med * 1e-3) / 1e12, 2)}
    del buf
    return out


def achievable_peaks(torch, T):
    """What this GPU reaches on plain work: a bf16 GEMM (torch / hipBLASLt,
    8192^3) and a 1 GiB device-to-device copy."""
    dev = torch.device("cuda:0")
    n = 8192
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    e0 = T.ev()
    for _ in range(10):
        torch.matmul(a, b)
    e1 = T.ev()
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e12
    del a, b
    src = torch.empty((1 << 30,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = T.ev()
    for _ in range(10):
        dst.copy_(src)
    e1 = T.ev()
    torch.cuda.synchronize()
    copy = 2.0 * (1 << 30) / (e0.elapsed_time(e1) / 10 * 1e-3) / 1e9
    del src, dst
    return {"bf16_gemm_tflops": round(gemm, 1), "copy_GBps": round(copy, 1),
            "what": "torch.matmul bf16 8192x8192x8192; 1 GiB device copy (read + write counted)"}


def environment(torch):
    env = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
           "device": torch.cuda.get_device_name(0)}
    try:
        import shutil
        import subprocess
        # run the tool's script with this interpreter: its "#!/usr/bin/env" line
        # would otherwise have env replace itself with python inside the child
        smi = os.path.realpath(shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi")
        r = subprocess.run([sys.executable, smi, "--showclocks"], capture_output=True, text=True, timeout=30)
        env["clocks"] = [ln.strip() for ln in r.stdout.splitlines() if "clk" in ln.lower()][:6]
    except Exception as ex:   # report, do not hide
        env["clocks"] = f"rocm-smi unavailable: {ex}"
    return env


def time_backward(torch, V, T, q, k, v, bs, fwd_flops, reps=4, **blocks):
    """Forward (with LSE) once, then the backward under the same block set: device
    time per call over reps - 1 calls queued back to back after one untimed
    call; dO is seeded unit normal."""
    g = torch.Generator(device=q.device).manual_seed(7)
    do = torch.randn(q.shape, generator=g, device=q.device, dtype=torch.float32).to(q.dtype)
    o, lse = V.vsa_block_sparse_attn_fwd(q, k, v, bs, return_lse=True, **blocks)
    B, H, N, _ = q.shape
    ws = torch.empty((V.vsa_attn_bwd_workspace_bytes(B, H, N, bs, "kv_idx" in blocks),), dtype=torch.uint8,
                     device=q.device)
    grads = [torch.empty_like(q) for _ in range(3)]
    t = T.per_call_ms(lambda: V.vsa_block_sparse_attn_bwd(q, k, v, o, lse, do, bs, dq=grads[0], dk=grads[1],
                                                            dv=grads[2], workspace=ws, **blocks), reps - 1)
    ms = [t]
    t = float(np.mean(ms))
    fl = 2.5 * fwd_flops          # 10 D per kept pair (S, dP, dV, dQ, dK) against the forward's 4 D
    del do, o, lse, ws, grads
    return {"ms": round(t, 4), "flops": fl, "tflops": round(fl / (t * 1e-3) / 1e12, 2),
            "pct_mfma_peak": round(100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}


def queued(torch, T, steps, reps):
    """Device time of each labelled call of a sequence: the sequence is queued
    `reps` times back to back behind a lead spin, with an event between calls,
    and timed on repetitions 1 .. reps-1 (repetition 0 is a warm-up). `steps` is
    a list of (label, fn); returns ({label: mean ms}, the last outputs)."""
    torch.cuda.synchronize()
    T.lead(max(3.0, 0.4 * reps * len(steps)))
    marks, outs = [], {}
    for rep in range(reps):
        e = [T.ev()]
        for label, fn in steps:
            outs[label] = fn()
            e.append(T.ev())
        if rep:
            marks.append(e)
    torch.cuda.synchronize()
    ms = {}
    for e in marks:
        for n, (label, _) in enumerate(steps):
            ms.setdefault(label, []).append(e[n].elapsed_time(e[n + 1]))
    return {label: round(float(np.mean(v_)), 4) for label, v_ in ms.items()}, outs


def speedups(dense, attn_ms, layer_ms):
    return {"dense_ms": {"ours_all_blocks": dense["ours_all_blocks"], "torch_sdpa": dense["torch_sdpa"]},
            "speedup_vs_dense_kernel": round(dense["best"] / attn_ms, 2),
            "speedup_vs_dense_pipeline": round(dense["best"] / layer_ms, 2)}


def extra_layers(torch, V, PL, T, wan_dense, wan_attn_tflops, wan_alone_tflops):
    """The other layers of the pages at their shapes, each step timed as device
    work (queued behind a lead spin, so no host latency is inside a bracket),
    with the dense baselines at the same shape for the speedups."""
    res = {}
    dev = torch.device("cuda:0")

    # Wan 480p with a 6/6 head split (even heads spatial w=1, odd heads temporal
    # w=0 in frame-major order): the step's kernel with the choice read on the
    # device, the same kernel with host lists, and the separate sequence
    # permute x3 -> attention -> inverse permute
    w = WAN480
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in make_qkv(w))
    sel = [h % 2 for h in range(w.H)]
    ch = torch.tensor([sel], dtype=torch.int32, device=dev)
    cand = PL.svg_masks(w.grid, w.bs, w.extra["w_spatial"], w.extra["w_temporal"], dev)
    idx, cnt = V.vsa_mask_to_list(cand, head_mask_idx=sel, B=1)
    FMK = V.VSA_PERM_FRAME_MAJOR
    qm, km, vm, om, o_s = (torch.empty_like(q) for _ in range(5))
    o_c = V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], ch)
    o_f = V.vsa_block_sparse_attn_fwd_permuted(q, k, v, w.grid, w.bs, head_fm=sel, kv_idx=idx, kv_cnt=cnt)
    ms = {"chosen_attention": T.per_call_ms(
              lambda: V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], ch, out=o_c), 5),
          "fused_attention": T.per_call_ms(
              lambda: V.vsa_block_sparse_attn_fwd_permuted(q, k, v, w.grid, w.bs, head_fm=sel, kv_idx=idx,
                                                           kv_cnt=cnt, out=o_f), 5),
          "separate_permute_qkv": T.per_call_ms(
              lambda: [V.vsa_permute(x, w.grid, FMK, False, sel, out=y) for x, y in ((q, qm), (k, km), (v, vm))], 5),
          "separate_attention": T.per_call_ms(
              lambda: V.vsa_block_sparse_attn_fwd(qm, km, vm, w.bs, kv_idx=idx, kv_cnt=cnt, out=om), 5),
          "separate_permute_o": T.per_call_ms(lambda: V.vsa_permute(om, w.grid, FMK, True, sel, out=o_s), 5)}
    ms = {k_: round(v_, 4) for k_, v_ in ms.items()}
    fl = kept_flops_from_lists(idx, cnt, w.N, w.bs, 128)
    split_tflops = fl / (ms["chosen_attention"] * 1e-3) / 1e12
    # the split's launch alone, timed as the all-spatial launch is in attention_launch_stats
    # (one launch per lead spin, median): both then run at the clock a lone launch gets
    alone = launch_stats(torch, T, lambda: V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], ch,
                                                                             out=o_c), fl, runs=20, warm=3)
    res["svg_6_6_split_wan480"] = {
        "ms": ms, "kept_flops": fl, "chosen_attn_tflops": round(split_tflops, 2),
        "fused_attn_tflops": round(fl / (ms["fused_attention"] * 1e-3) / 1e12, 2),
        "rate_vs_all_spatial_step_kernel": round(split_tflops / wan_attn_tflops, 3),
        "chosen_alone": alone,
        "rate_vs_all_spatial_alone": round(alone["warm"]["tflops_at_median"] / wan_alone_tflops, 3),
        "separate_total_ms": round(ms["separate_permute_qkv"] + ms["separate_attention"] + ms["separate_permute_o"], 4),
        "bit_identical": bool(torch.equal(o_c, o_f) and torch.equal(o_f, o_s)),
        **speedups(wan_dense, ms["chosen_attention"], ms["chosen_attention"])}
    del qm, km, vm, om, o_f, o_s, o_c, cand, ch
    torch.cuda.empty_cache()

    # backward (dQ, dK, dV) at the same shape with the spatial w=1 block mask on
    # every head, natural order (trainable sparse attention)
    m = V.vsa_pattern_mask(w.grid, w.bs, V.VSA_PATTERN_SPATIAL, w.extra["w_spatial"])
    mask = m.reshape(1, 1, w.nb, w.nb).expand(1, w.H, w.nb, w.nb).contiguous()
    bi, bc = V.vsa_mask_to_list(mask)
    res["attn_bwd_spatial_wan480"] = time_backward(torch, V, T, q, k, v, w.bs,
                                                   kept_flops_from_lists(bi, bc, w.N, w.bs, 128), mask=mask)
    res["attn_bwd_spatial_wan480"]["what"] = ("vsa_block_sparse_attn_bwd, [1,12,32760,128] bf16, bs 128, spatial "
                                              "w=1 block mask on all heads")

    # FP8 (e4m3) attention under the same mask: quantisation of Q, K, V, then the
    # fp8 kernel, against the bf16 kernel on the same inputs
    fl_sp = kept_flops_from_lists(bi, bc, w.N, w.bs, 128)
    q8, qsc = V.vsa_fp8_quantize(q, V.VSA_FP8_ROWS)
    k8, ksc = V.vsa_fp8_quantize(k, V.VSA_FP8_ROWS)
    vt8, vsc = V.vsa_fp8_quantize(v, V.VSA_FP8_VT)
    o8, ob = torch.empty_like(q), torch.empty_like(q)
    ms, _ = queued(torch, T, [
        ("quantise_qkv", lambda: (V.vsa_fp8_quantize(q, V.VSA_FP8_ROWS, out=q8, scales=qsc),
                                  V.vsa_fp8_quantize(k, V.VSA_FP8_ROWS, out=k8, scales=ksc),
                                  V.vsa_fp8_quantize(v, V.VSA_FP8_VT, out=vt8, scales=vsc))),
        ("fp8_attention", lambda: V.vsa_block_sparse_attn_fwd_fp8(q8, k8, vt8, qsc, ksc, vsc, w.bs, mask=mask, out=o8)),
        ("bf16_attention", lambda: V.vsa_block_sparse_attn_fwd(q, k, v, w.bs, mask=mask, out=ob))], 4)
    rel = float(((o8.float() - ob.float()).abs().mean() / ob.float().abs().mean()).item())
    res["fp8_spatial_wan480"] = {"ms": ms, "kept_flops": fl_sp,
                                 "fp8_attn_tflops": round(fl_sp / (ms["fp8_attention"] * 1e-3) / 1e12, 2),
                                 "bf16_attn_tflops": round(fl_sp / (ms["bf16_attention"] * 1e-3) / 1e12, 2),
                                 "pct_fp8_mfma_peak": round(100 * fl_sp / (ms["fp8_attention"] * 1e-3) / 1e12
                                                            / PEAK_FP8_TFLOPS, 2),
                                 "speedup_vs_bf16": round(ms["bf16_attention"] / ms["fp8_attention"], 3),
                                 "mean_rel_diff_vs_bf16": round(rel, 4)}
    del q8, k8, vt8, o8, ob, m, mask, bi, bc

    # Skiparse-2D (OSP-Next page, "Method"), k = 2, both patterns, at the Wan shape
    for mode_name, mode in (("token", V.VSA_SKIPARSE_TOKEN), ("group", V.VSA_SKIPARSE_GROUP)):
        kf, sbs = 2, 128
        ns, nbk = V.vsa_skiparse_dims(w.grid, mode, kf, sbs)
        qs_, ks_, vs_, os_ = (torch.empty((1, w.H, ns, w.D), dtype=q.dtype, device=dev) for _ in range(4))
        o = torch.empty_like(q)
        blk = V.vsa_skiparse_block_len(w.grid, mode, kf, sbs)
        sm = V.vsa_skiparse_mask(w.grid, mode, kf, sbs)
        smask = sm.expand(1, w.H, -1, -1).contiguous()
        si, sc = V.vsa_mask_to_list(smask)
        ms, _ = queued(torch, T, [
            ("permute_qkv", lambda: [V.vsa_skiparse_permute(x, w.grid, mode, kf, sbs, out=y)
                                     for x, y in ((q, qs_), (k, ks_), (v, vs_))]),
            ("mask_and_lists", lambda: (V.vsa_skiparse_block_len(w.grid, mode, kf, sbs, out=blk),
                                        V.vsa_skiparse_mask(w.grid, mode, kf, sbs, out=sm),
                                        V.vsa_mask_to_list(smask, out=(si, sc)))),
            ("attention", lambda: V.vsa_block_sparse_attn_fwd(qs_, ks_, vs_, sbs, kv_idx=si, kv_cnt=sc, blk_len=blk,
                                                              out=os_)),
            ("permute_o", lambda: V.vsa_skiparse_permute(os_, w.grid, mode, kf, sbs, inverse=True, out=o))], 4)
        fl = kept_flops_from_lists(si, sc, ns, sbs, 128, blk)
        layer = sum(ms.values())
        res[f"skiparse_{mode_name}_k2_wan480"] = {
            "ms": ms, "layer_ms": round(layer, 4), "kept_flops": fl,
            "kept_pair_density": round(fl / (4.0 * w.D * w.H * w.N * w.N), 4),
            "attn_tflops": round(fl / (ms["attention"] * 1e-3) / 1e12, 2),
            "pct_mfma_peak": round(100 * fl / (ms["attention"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "permute_GBps": round(3 * (q.numel() + qs_.numel()) * 2 / (ms["permute_qkv"] * 1e-3) / 1e9, 1),
            **speedups(wan_dense, ms["attention"], layer)}
        del qs_, ks_, vs_, os_, o, blk, sm, smask, si, sc
    del q, k, v
    torch.cuda.empty_cache()

    # HunyuanVideo 720p layer (24 heads, 118,800 tokens): planted 12/12 split, even
    # heads spatial w=2, odd heads temporal w=276 in frame-major order (folded into
    # the attention's loads and stores); and the a3 permutation of one tensor with
    # all 24 heads moved
    w = HUNYUAN720
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in make_qkv(w))
    sel = [h % 2 for h in range(w.H)]
    ch = torch.tensor([sel], dtype=torch.int32, device=dev)
    cand = PL.svg_masks(w.grid, w.bs, w.extra["w_spatial"], w.extra["w_temporal"], dev)
    idx, cnt = V.vsa_mask_to_list(cand, head_mask_idx=sel, B=1)
    fl = kept_flops_from_lists(idx, cnt, w.N, w.bs, 128)
    o = torch.empty_like(q)
    ms, _ = queued(torch, T, [
        ("masks", lambda: PL.svg_masks(w.grid, w.bs, w.extra["w_spatial"], w.extra["w_temporal"], dev)),
        ("chosen_attention", lambda: V.vsa_block_sparse_attn_fwd_chosen(q, k, v, w.grid, w.bs, cand, [0, 1], ch,
                                                                         out=o))], 3)
    t_att = ms["chosen_attention"]
    pdst = torch.empty_like(q)
    p_ms = T.per_call_ms(lambda: V.vsa_permute(q, w.grid, V.VSA_PERM_FRAME_MAJOR, False, [1] * w.H, out=pdst), 10)
    p_gbs = 2 * q.numel() * q.element_size() / (p_ms * 1e-3) / 1e9
    del pdst
    dense = dense_baselines(torch, V, T, q, k, v, w.bs, reps=2)
    res["svg_hunyuan720"] = {"ms": ms, "attention_ms": round(t_att, 3), "kept_flops": fl,
                             "attn_tflops": round(fl / (t_att * 1e-3) / 1e12, 2),
                             "pct_mfma_peak": round(100 * fl / (t_att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                             "permute_all_heads": {"ms": round(p_ms, 4), "GBps": round(p_gbs, 1),
                                                   "frac_of_hbm_peak": round(p_gbs / PEAK_HBM_GBS, 3),
                                                   "bytes": 2 * q.numel() * q.element_size()},
                             **speedups(dense, t_att, sum(ms.values())),
                             "what": "vsa_block_sparse_attn_fwd_chosen, [1,24,118800,128] bf16, bs 128, planted split"}
    del q, k, v, o, cand, idx, cnt, ch
    torch.cuda.empty_cache()

    w = WAN480_CUBE
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in make_qkv(w))
    n_cubes, k_max = PL.cube_budget(w.grid, w.extra["k_frac"])
    blk = V.vsa_cube_block_len(w.grid)
    # every step writes into buffers allocated once, as a layer run step after step would
    st = {}
    cube_buf = [V.vsa_permute(x, w.grid, V.VSA_PERM_CUBE4) for x in (q, k, v)]
    s_buf = V.vsa_block_scores(cube_buf[0], cube_buf[1], 64, blk_len=blk)
    sel_buf = V.vsa_select_topk(s_buf[0], k_max, w.extra["top_p"])
    oc_buf, o_buf = torch.empty_like(cube_buf[0]), torch.empty_like(q)

    def cube_permute_qk():
        st["qc"], st["kc"] = (V.vsa_permute(x, w.grid, V.VSA_PERM_CUBE4, out=b) for x, b in zip((q, k), cube_buf))

    def cube_permute_v():
        st["vc"] = V.vsa_permute(v, w.grid, V.VSA_PERM_CUBE4, out=cube_buf[2])

    def cube_scores():
        st["S"] = V.vsa_block_scores(st["qc"], st["kc"], 64, blk_len=blk, out=s_buf)[0]

    def cube_select():
        st["idx"], st["cnt"] = V.vsa_select_topk(st["S"], k_max, w.extra["top_p"], out=sel_buf)

    def cube_attn():
        st["oc"] = V.vsa_block_sparse_attn_fwd(st["qc"], st["kc"], st["vc"], 64, kv_idx=st["idx"], kv_cnt=st["cnt"],
                                               blk_len=blk, out=oc_buf)

    def cube_back():
        st["o"] = V.vsa_permute(st["oc"], w.grid, V.VSA_PERM_CUBE4, inverse=True, out=o_buf)

    # V is moved to the cube layout after the selection, right before the attention that
    # reads it: K (just pooled) and V (just written) are then what the last-level cache holds
    ms, _ = queued(torch, T, [("a3_cube_permute_qk", cube_permute_qk), ("a4_block_scores", cube_scores),
                              ("a5_select_topk", cube_select), ("a3_cube_permute_v", cube_permute_v),
                              ("a7_attention", cube_attn), ("a8_cube_permute_o", cube_back)], 4)
    qc, kc, vc, S, idx, cnt, oc = (st[x] for x in ("qc", "kc", "vc", "S", "idx", "cnt", "oc"))
    fl = kept_flops_from_lists(idx, cnt, oc.shape[2], 64, 128, blk)
    t_att = ms["a7_attention"]
    # the same attention launch alone, back to back on the layer's last lists
    oc_alone = torch.empty_like(oc)
    t_alone = T.per_call_ms(lambda: V.vsa_block_sparse_attn_fwd(qc, kc, vc, 64, kv_idx=idx, kv_cnt=cnt, blk_len=blk,
                                                                out=oc_alone), 10)
    del oc_alone
    nat_b = q.numel() * q.element_size()                         # one natural-order tensor
    cube_b = qc.numel() * qc.element_size()                      # one cube-major tensor, pad slots included
    gbs = {"a3_cube_permute_qkv": 3 * (nat_b + cube_b),          # read every token, write every slot
           "a4_block_scores": 2 * nat_b + S.numel() * 4,         # the valid rows of Q and K read, S written
           "a8_cube_permute_o": cube_b + nat_b}
    t_of = dict(ms, a3_cube_permute_qkv=ms["a3_cube_permute_qk"] + ms["a3_cube_permute_v"])
    hbm = {key: {"GBps": round(b / (t_of[key] * 1e-3) / 1e9, 1),
                 "frac_of_hbm_peak": round(b / (t_of[key] * 1e-3) / 1e9 / PEAK_HBM_GBS, 3)}
           for key, b in gbs.items()}
    res["cube_topp_wan480"] = {"ms": ms, "layer_ms": round(sum(ms.values()), 4), "hbm": hbm,
                               "k_max": k_max, "mean_kept": round(float(cnt.float().mean().item()), 2),
                               "kept_flops": fl, "attn_tflops": round(fl / (t_att * 1e-3) / 1e12, 2),
                               "pct_mfma_peak": round(100 * fl / (t_att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                               "a7_alone": {"ms": round(t_alone, 4), "tflops": round(fl / (t_alone * 1e-3) / 1e12, 2),
                                            "what": "the layer's attention launch alone, 10 back to back"},
                               **speedups(wan_dense, t_att, sum(ms.values())),
                               "backward": time_backward(torch, V, T, qc, kc, vc, 64, fl, kv_idx=idx, kv_cnt=cnt,
                                                         blk_len=blk)}
    del q, k, v, qc, kc, vc, oc, S, st, cube_buf, s_buf, sel_buf, oc_buf, o_buf
    torch.cuda.empty_cache()

    w = LONG126
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in make_qkv(w))
    k_total = int(round(w.extra["density"] * w.nb))
    st = {}

    def long_mask():
        st["forced"] = V.vsa_pattern_mask(w.grid, w.bs, V.VSA_PATTERN_SPATIAL, w.extra["w_local"])

    def long_scores():
        st["S"] = V.vsa_block_scores(q, k, w.bs)[0]

    def long_select():
        st["idx"], st["cnt"] = V.vsa_select_topk(st["S"], k_total, 1.0, forced=st["forced"])

    def long_attn():
        st["o"] = V.vsa_block_sparse_attn_fwd(q, k, v, w.bs, kv_idx=st["idx"], kv_cnt=st["cnt"])

    ms, _ = queued(torch, T, [("a1_local_mask", long_mask), ("a4_block_scores", long_scores),
                              ("a5_select_topk", long_select), ("a7_attention", long_attn)], 3)
    S, idx, cnt = st["S"], st["idx"], st["cnt"]
    fl = kept_flops_from_lists(idx, cnt, w.N, w.bs, 128)
    t_att = ms["a7_attention"]
    a4_b = 2 * q.numel() * q.element_size() + S.numel() * 4      # Q and K read once, S written
    a4_gbs = a4_b / (ms["a4_block_scores"] * 1e-3) / 1e9
    del st, S
    dense = dense_baselines(torch, V, T, q, k, v, w.bs, reps=2)
    res["long_horizon_126x30x52"] = {"ms": ms, "layer_ms": round(sum(ms.values()), 4),
                                     "hbm": {"a4_block_scores": {"GBps": round(a4_gbs, 1),
                                                                 "frac_of_hbm_peak": round(a4_gbs / PEAK_HBM_GBS, 3)}},
                                     "k_total": k_total, "kept_flops": fl,
                                     "attn_tflops": round(fl / (t_att * 1e-3) / 1e12, 2),
                                     "pct_mfma_peak": round(100 * fl / (t_att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                                     **speedups(dense, t_att, sum(ms.values()))}
    del q, k, v
    torch.cuda.empty_cache()

    # Sparse VideoGen2-style layer: k-means of Q and K, cluster-major storage,
    # size-weighted top-p, attention over the kept clusters, O moved back
    w = WAN480_SEMANTIC
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in make_qkv(w))
    Cq, Ck, iters, top_p = w.extra["Cq"], w.extra["Ck"], w.extra["iters"], w.extra["top_p"]
    st = {}

    def km_q():
        st["cq"], st["lq"], st["nq"] = V.vsa_kmeans(q, Cq, iters)

    def km_k():
        st["ck"], st["lk"], st["nk"] = V.vsa_kmeans(k, Ck, iters)

    def order():
        st["pq"], st["oq"] = V.vsa_cluster_order(st["lq"], Cq)
        st["pk"], st["ok"] = V.vsa_cluster_order(st["lk"], Ck)

    def gather():
        st["qs"] = V.vsa_gather_rows(q, st["pq"])
        st["ks"] = V.vsa_gather_rows(k, st["pk"])
        st["vs"] = V.vsa_gather_rows(v, st["pk"])

    def scores_select():
        st["S"] = V.vsa_cluster_scores(st["cq"], st["ck"], st["nk"])
        st["idx"], st["cnt"] = V.vsa_select_topk(st["S"], Ck, top_p)

    def attn():
        st["os"] = V.vsa_varlen_sparse_attn_fwd(st["qs"], st["ks"], st["vs"], st["oq"], st["ok"], kv_idx=st["idx"],
                                                kv_cnt=st["cnt"])

    def back():
        st["o"] = V.vsa_gather_rows(st["os"], st["pq"], inverse=True)

    ms, _ = queued(torch, T, [("kmeans_q", km_q), ("kmeans_k", km_k), ("cluster_order_qk", order),
                              ("gather_qkv", gather), ("scores_select", scores_select), ("varlen_attention", attn),
                              ("gather_o", back)], 4)
    nqh, nkh, ih, chh = (st[x].cpu().numpy().astype(np.int64) for x in ("nq", "nk", "idx", "cnt"))
    kept = 0.0
    for h in range(w.H):
        for a in range(Cq):
            kept += float(nqh[0, h, a]) * float(nkh[0, h, ih[0, h, a, :chh[0, h, a]]].sum())
    fl = 4.0 * w.D * kept
    t_att = ms["varlen_attention"]
    res["semantic_wan480"] = {"ms": ms, "total_ms": round(sum(ms.values()), 4), "Cq": Cq, "Ck": Ck, "iters": iters,
                              "top_p": top_p, "kept_pair_density": round(kept / (w.H * w.N * w.N), 4),
                              "kept_flops": fl, "attn_tflops": round(fl / (t_att * 1e-3) / 1e12, 2),
                              "pct_mfma_peak": round(100 * fl / (t_att * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                              **speedups(wan_dense, t_att, sum(ms.values()))}
    del q, k, v, st
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
