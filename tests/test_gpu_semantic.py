"""GPU parity of the semantic-aware permutation path against the oracle:
k-means (equal to the oracle's fp64 assignment wherever bf16 rounding of the
centroids cannot change a token's nearest centroid, at every iteration, plus the
properties that hold at any size), the stable cluster-major order and row
gathers (bit-exact), size-weighted cluster scores, attention over
variable-size clusters (element by element on ragged clusters; sampled rows at
the full video shape), and the whole layer on separable data and at the full
video shape."""
import numpy as np
import pytest
import torch

import block_sparse_attention_vsa_amd as V
from block_sparse_attention_vsa_amd import pipelines as PL
from oracle import attention as OA
from oracle import masks as OM
from oracle import semantic as OS
from tests.gpu_util import announce, assert_close_bf16, assert_lse_close, dev, dev_i32, dev_u8, host
from workloads import WAN480_SEMANTIC, make_qkv, sample_rows, to_bf16_values

pytestmark = pytest.mark.gpu


def bf16(x):
    """Values rounded to bf16, held in fp64."""
    return to_bf16_values(x).astype(np.float64)


def rand_bf16(shape, seed, scale=1.0):
    return bf16(scale * np.random.default_rng(seed).standard_normal(shape))


def decided_assignment(x, cent, mode):
    """Reference labels of x for centroids `cent` and the tokens whose label a
    correct kernel cannot get wrong. The kernel ranks centroids by
    ||m~||^2 - 2 <x, m~>, m~ = bf16(m) (round to nearest even), with fp32 sums;
    the fp32 accumulation moves a score by at most 2^-16 (sum m~^2 + 2 sum |x m~|).

    mode "seed":   the centroids are bf16 values already (the seeds); reference =
                   the oracle's fp64 assignment; only the fp32 term applies.
    mode "worst":  reference = the oracle's fp64 assignment to the exact centroids;
                   |m~_i - m_i| <= 2^-8 |m_i| (8 significant bits), so rounding can
                   move a score by at most 2^-8 (2 + 2^-8) sum m_i^2 + 2^-7 sum |x_i| |m_i|,
                   added to the fp32 term.
    mode "kernel": the decision taken in the kernel's precision: reference = the
                   fp64 argmin with the centroids rounded to bf16 as the kernel
                   rounds them; only the fp32 term applies.
    Returns (reference labels, mask of tokens whose reference centroid beats every
    other by more than the bounds of both)."""
    x = np.asarray(x, np.float64)
    m = np.asarray(cent, np.float64)
    if mode == "kernel":
        m = bf16(m)
    ref = OS.assign(x, m)
    n2 = (m * m).sum(1)
    xm = np.abs(x) @ np.abs(m).T
    bound = 2.0 ** -16 * (n2[None, :] + 2.0 * xm)
    if mode == "worst":
        bound = bound + 2.0 ** -8 * (2.0 + 2.0 ** -8) * n2[None, :] + 2.0 ** -7 * xm
    d = n2[None, :] - 2.0 * (x @ m.T)
    r = np.arange(len(x))
    slack = d - d[r, ref][:, None] - bound - bound[r, ref][:, None]
    slack[r, ref] = np.inf
    return ref, slack.min(1) > 0


def check_iteration(lab, x, start, t, what):
    """Labels of iteration t, started from centroids `start`: equal to the
    plain oracle wherever no bf16 rounding of the centroids can flip them, and
    equal to the decision in the kernel's precision wherever fp32 sums cannot."""
    modes = (("seed", 0.99),) if t == 1 else (("worst", 0.7), ("kernel", 0.995))
    for mode, least in modes:
        ref, ok = decided_assignment(x, start, mode)
        frac = ok.mean()
        print(f"{what} t={t} {mode}: decided {frac:.4f}, agree {(lab == ref).mean():.4f}")
        assert frac > least, f"{what} t={t} {mode}: decided {frac:.4f}"
        assert (lab[ok] == ref[ok]).all(), f"{what} t={t} {mode}"


def check_kmeans_properties(x, cent, lab, cnt, C, what):
    """Centroids are the member means of the returned labels (empty clusters
    excepted), counts match the labels, labels lie in [0, C)."""
    B, H, N, D = x.shape
    assert ((lab >= 0) & (lab < C)).all(), what
    for b in range(B):
        for h in range(H):
            bc = np.bincount(lab[b, h], minlength=C)
            assert (bc == cnt[b, h]).all(), what
            sums = np.zeros((C, D))
            np.add.at(sums, lab[b, h], x[b, h])
            nz = bc > 0
            np.testing.assert_allclose(cent[b, h][nz], sums[nz] / bc[nz, None], rtol=1e-5, atol=1e-5,
                                       err_msg=what)


@pytest.mark.parametrize("N,C", [(1000, 37), (300, 64), (129, 129), (2048, 1)])
def test_kmeans_first_iteration(N, C):
    """One iteration from the seeds (tokens, so exact bf16 values): every label
    that fp32 accumulation cannot flip matches the oracle, and the centroids are
    the member means."""
    announce(f"kmeans 1 iter N={N} C={C}")
    x = rand_bf16((1, 2, N, 128), N + C)
    cent, lab, cnt = (host(t) for t in V.vsa_kmeans(dev(x), C, 1))
    check_kmeans_properties(x, cent, lab, cnt, C, f"N={N} C={C}")
    for h in range(2):
        check_iteration(lab[0, h], x[0, h], x[0, h][(np.arange(C) * N) // C], 1, f"N={N} C={C} h={h}")


@pytest.mark.parametrize("C,iters", [(37, 3), (200, 2)])
def test_kmeans_each_iteration_against_the_oracle_step(C, iters):
    """Iteration t of the GPU k-means starts from the centroids a (t - 1)-iteration
    run returns (the seeds for t = 1); its labels equal the oracle's fp64
    assignment to those centroids wherever no bf16 rounding of the centroids can
    change the nearest one, and the decision taken in the kernel's precision
    wherever fp32 sums cannot."""
    announce(f"kmeans per-iteration C={C} iters={iters}")
    N = 3000
    x = rand_bf16((1, 2, N, 128), 77 + C)
    xd = dev(x)
    prev = np.stack([x[0, h][(np.arange(C) * N) // C] for h in range(2)])[None]
    for t in range(1, iters + 1):
        cent, lab, cnt = (host(tt) for tt in V.vsa_kmeans(xd, C, t))
        check_kmeans_properties(x, cent, lab, cnt, C, f"t={t}")
        for h in range(2):
            check_iteration(lab[0, h], x[0, h], prev[0, h], t, f"C={C} h={h}")
        prev = cent


def test_kmeans_iterations_on_separable_blobs():
    """Blobs stored one after another, one seed in each, several iterations:
    labels and centroids equal the oracle's."""
    announce("kmeans blobs 4 iters")
    C, per, D = 24, 50, 128
    g = np.random.default_rng(7)
    xs = []
    for h in range(2):
        centers = 2.0 * g.standard_normal((C, D))
        xs.append(bf16(np.repeat(centers, per, axis=0) + 0.3 * g.standard_normal((C * per, D))))
    x = np.stack(xs)[None]
    cent, lab, cnt = (host(t) for t in V.vsa_kmeans(dev(x), C, 4))
    for h in range(2):
        rc, rl, rn = OS.kmeans(x[0, h], C, 4)
        assert (lab[0, h] == rl).all() and (cnt[0, h] == rn).all()
        np.testing.assert_allclose(cent[0, h], rc, rtol=1e-5, atol=1e-5)


def test_kmeans_empty_cluster_keeps_its_centroid():
    """Duplicate seeds: ties go to the lower index, the higher cluster stays empty
    and keeps its seed."""
    announce("kmeans empty cluster")
    x = rand_bf16((1, 1, 256, 128), 8)
    x[0, 0, 128] = x[0, 0, 0]                          # seeds 0 and 1 (positions 0 and 128) coincide
    cent, lab, cnt = (host(t) for t in V.vsa_kmeans(dev(x), 2, 1))
    assert cnt[0, 0].tolist() == [256, 0] and (lab == 0).all()
    np.testing.assert_array_equal(cent[0, 0, 1], x[0, 0, 0])
    np.testing.assert_allclose(cent[0, 0, 0], x[0, 0].mean(0), rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("N,C", [(1000, 37), (256, 1), (777, 1024), (5000, 300)])
def test_cluster_order_bit_exact(N, C):
    announce(f"cluster order N={N} C={C}")
    g = np.random.default_rng(N + C)
    lab = g.integers(0, C, (2, 3, N)).astype(np.int32)
    if C > 4:
        lab[lab == 3] = 2                              # an empty cluster
    perm, off = (host(t) for t in V.vsa_cluster_order(dev_i32(lab), C))
    for b in range(2):
        for h in range(3):
            rp, ro = OS.cluster_order(lab[b, h], C)
            assert (perm[b, h] == rp).all() and (off[b, h] == ro).all()


@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (64, torch.float32)])
def test_gather_rows_bit_exact(D, dtype):
    announce(f"gather rows D={D} {dtype}")
    g = np.random.default_rng(D)
    x = torch.from_numpy(g.standard_normal((2, 3, 517, D)).astype(np.float32)).to(dtype).cuda()
    perm = np.stack([[g.permutation(517) for _ in range(3)] for _ in range(2)]).astype(np.int32)
    pd = dev_i32(perm)
    fwd = V.vsa_gather_rows(x, pd)
    back = V.vsa_gather_rows(fwd, pd, inverse=True)
    xh = x.cpu()
    ref = torch.stack([torch.stack([xh[b, h][torch.from_numpy(perm[b, h]).long()] for h in range(3)]) for b in range(2)])
    assert torch.equal(fwd.cpu(), ref)
    assert torch.equal(back, x)


def test_cluster_scores():
    announce("cluster scores")
    g = np.random.default_rng(11)
    cq = g.standard_normal((1, 2, 37, 128)).astype(np.float32)
    ck = g.standard_normal((1, 2, 300, 128)).astype(np.float32)
    kn = g.integers(0, 50, (1, 2, 300)).astype(np.int32)
    kn[0, 0, :5] = 0
    S = host(V.vsa_cluster_scores(torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), dev_i32(kn), scale=0.1))
    for h in range(2):
        ref = OS.cluster_scores(cq[0, h], ck[0, h], kn[0, h], 0.1)
        fin = np.isfinite(ref)
        assert (np.isfinite(S[0, h]) == fin).all()
        np.testing.assert_allclose(S[0, h][fin], ref[fin], rtol=1e-5, atol=1e-5)


def offsets_of(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)


def varlen_case(H, sizes_q, sizes_k, density, seed):
    g = np.random.default_rng(seed)
    N = int(sum(sizes_q))
    assert N == int(sum(sizes_k))
    q, k, v = (rand_bf16((1, H, N, 128), seed + i) for i in range(3))
    Cq, Ck = len(sizes_q), len(sizes_k)
    mask = (g.random((1, H, Cq, Ck)) < density).astype(np.uint8)
    qo = np.broadcast_to(offsets_of(sizes_q), (1, H, Cq + 1)).copy()
    ko = np.broadcast_to(offsets_of(sizes_k), (1, H, Ck + 1)).copy()
    qblk = np.repeat(np.arange(Cq), sizes_q)
    kblk = np.repeat(np.arange(Ck), sizes_k)
    return q, k, v, mask, qo, ko, qblk, kblk


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_varlen_attention_ragged_clusters_full_oracle(seed):
    """Clusters of sizes 0, 1, under and over one 64-key tile and one 128-row
    chunk; a query cluster with nothing kept; mask and list forms bit-identical."""
    announce(f"varlen attn seed={seed}")
    g = np.random.default_rng(100 + seed)
    sizes_q = np.array([0, 1, 5, 64, 127, 128, 129, 300, 31, 0, 200, 17])
    sizes_k = g.multinomial(sizes_q.sum(), np.r_[0.0, g.dirichlet(np.ones(13))])    # key cluster 0 empty
    q, k, v, mask, qo, ko, qblk, kblk = varlen_case(2, sizes_q, sizes_k, 0.35, seed)
    mask[0, 0, 6, :] = 0                                    # query cluster 6 keeps nothing
    qd, kd, vd = dev(q), dev(k), dev(v)
    o, lse = V.vsa_varlen_sparse_attn_fwd(qd, kd, vd, dev_i32(qo), dev_i32(ko), mask=dev_u8(mask), return_lse=True)
    ro, rl, p = OA.masked_attention(q, k, v, mask, qblk, kblk, return_probs=True)
    go, gl = host(o), host(lse)
    assert_close_bf16(go, ro, f"varlen seed={seed}")
    assert_lse_close(gl, rl, f"varlen seed={seed}")
    # every element within the bound of its two bf16 roundings (P before P V, O
    # once; 2^-8 each) plus 2e-4 for the fp32 arithmetic
    bound = (2.0 ** -8 + 2e-4) * (np.einsum("bhij,bhjd->bhid", p, np.abs(v)) + np.abs(ro))
    assert (np.abs(go - ro) <= bound).all(), f"varlen seed={seed}: past the rounding bound"
    rows6 = slice(qo[0, 0, 6], qo[0, 0, 7])
    assert (go[0, 0, rows6] == 0).all() and np.isneginf(gl[0, 0, rows6]).all()
    idx, cnt = OM.mask_to_list(mask)
    o2 = V.vsa_varlen_sparse_attn_fwd(qd, kd, vd, dev_i32(qo), dev_i32(ko), kv_idx=dev_i32(idx), kv_cnt=dev_i32(cnt))
    assert torch.equal(o, o2)
    o3 = V.vsa_varlen_sparse_attn_fwd(qd, kd, vd, dev_i32(qo), dev_i32(ko), mask=dev_u8(mask))
    assert torch.equal(o, o3)



@pytest.mark.parametrize("slope", [10.0, 3.0, -6.0])
def test_varlen_offset_paths_with_scores_rising_or_falling(slope):
    """As for the block kernel: scores moving by `slope` log2 units per 64 keys
    along the kept key clusters drive the running offset through every path."""
    announce(f"varlen offset paths slope={slope}")
    rng = np.random.default_rng(32)
    sizes_q, sizes_k = np.array([260, 240]), np.array([100, 150, 250])
    N, D = 500, 128
    scale = 1.0 / np.sqrt(D)
    per_key = slope / 64 / (scale * np.log2(np.e))
    q = bf16(0.05 * rng.standard_normal((1, 1, N, D)))
    k = 0.05 * rng.standard_normal((1, 1, N, D))
    q[..., 0] = 1.0
    k[..., 0] = per_key * (np.arange(N) - (N - 1 if slope > 0 else 0))
    k = bf16(k)
    v = rand_bf16((1, 1, N, D), 33)
    mask = np.ones((1, 1, 2, 3), np.uint8)
    qo, ko = offsets_of(sizes_q)[None, None], offsets_of(sizes_k)[None, None]
    o, lse = V.vsa_varlen_sparse_attn_fwd(dev(q), dev(k), dev(v), dev_i32(qo), dev_i32(ko), mask=dev_u8(mask),
                                          return_lse=True)
    qblk, kblk = np.repeat(np.arange(2), sizes_q), np.repeat(np.arange(3), sizes_k)
    ro, rl, p = OA.masked_attention(q, k, v, mask, qblk, kblk, return_probs=True)
    bound = (2.0 ** -8 + 2e-4) * (np.einsum("bhij,bhjd->bhid", p, np.abs(v)) + np.abs(ro))
    assert (np.abs(host(o) - ro) <= bound).all(), f"varlen slope={slope}: past the rounding bound"
    assert_lse_close(host(lse), rl, f"varlen offset paths slope={slope}")

def test_varlen_attention_unsorted_lists_and_all_kept():
    announce("varlen attn unsorted / dense")
    sizes = np.array([70, 130, 1, 250, 60, 9])
    q, k, v, mask, qo, ko, qblk, kblk = varlen_case(1, sizes, sizes[::-1].copy(), 0.5, 21)
    mask[...] = 1
    idx = np.stack([np.random.default_rng(a).permutation(6) for a in range(6)])[None, None].astype(np.int32)
    cnt = np.full((1, 1, 6), 6, np.int32)
    o = V.vsa_varlen_sparse_attn_fwd(dev(q), dev(k), dev(v), dev_i32(qo), dev_i32(ko), kv_idx=dev_i32(idx),
                                     kv_cnt=dev_i32(cnt))
    ref = OA.dense_attention(q, k, v)[0]
    assert_close_bf16(host(o), ref, "varlen all kept")


def test_semantic_layer_on_separable_data_matches_oracle():
    """Well-separated components stored one after another (one seed per component
    for both Q and K): the GPU layer reproduces the oracle's clusters, selection
    and output."""
    announce("semantic layer separable")
    C, per, D, H = 8, 96, 128, 2
    g = np.random.default_rng(31)
    qs, ks = [], []
    for h in range(H):
        mu = 1.5 * g.standard_normal((C, D))
        qs.append(np.repeat(mu, per, 0) + 0.5 * g.standard_normal((C * per, D)))
        ks.append(np.repeat(mu, per, 0) + 0.5 * g.standard_normal((C * per, D)))
    q = bf16(np.stack(qs)[None])
    k = bf16(np.stack(ks)[None])
    v = rand_bf16(q.shape, 32)
    ro, _, P = OS.semantic_pipeline(q, k, v, C, C, 3, 0.9)
    stats = {}
    o = PL.semantic_layer(dev(q), dev(k), dev(v), C, C, 3, 0.9, stats=stats)
    assert (host(stats["q_labels"]) == P["q_labels"]).all()
    assert (host(stats["k_labels"]) == P["k_labels"]).all()
    gi, gc = host(stats["kv_idx"]), host(stats["kv_cnt"])
    assert (gc == P["kv_cnt"]).all()
    for b in range(1):
        for h in range(H):
            for a in range(C):
                assert (gi[b, h, a, :gc[b, h, a]] == P["kv_idx"][b, h, a, :P["kv_cnt"][b, h, a]]).all()
    assert_close_bf16(host(o), ro, "semantic layer")


def test_varlen_attention_full_semantic_shape_sampled():
    """The Wan 480p semantic layer's shape and cluster structure (oracle k-means
    with 128 query / 256 key clusters, size-weighted top-p 0.9 on 2 heads), the
    cluster-major tensors built on the host: sampled rows against the oracle."""
    w = WAN480_SEMANTIC
    announce("varlen attn full semantic shape")
    H = 2
    q, k, v = make_qkv(w, H=H)
    Cq, Ck = w.extra["Cq"], w.extra["Ck"]
    rows = sample_rows(w.N, 128, 256, 17)
    ro, rl, P = OS.semantic_pipeline(q, k, v, Cq, Ck, w.extra["iters"], w.extra["top_p"], rows=rows)
    qsto, ksto, vsto = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    qo = np.zeros((1, H, Cq + 1), np.int32)
    ko = np.zeros((1, H, Ck + 1), np.int32)
    pos_of = np.zeros((H, w.N), np.int64)
    for h in range(H):
        pq, oq = OS.cluster_order(P["q_labels"][0, h], Cq)
        pk, ok = OS.cluster_order(P["k_labels"][0, h], Ck)
        qsto[0, h], ksto[0, h], vsto[0, h] = q[0, h, pq], k[0, h, pk], v[0, h, pk]
        qo[0, h], ko[0, h] = oq, ok
        pos_of[h, pq] = np.arange(w.N)
    o, lse = V.vsa_varlen_sparse_attn_fwd(dev(qsto), dev(ksto), dev(vsto), dev_i32(qo), dev_i32(ko),
                                          kv_idx=dev_i32(P["kv_idx"]), kv_cnt=dev_i32(P["kv_cnt"]),
                                          return_lse=True)
    go, gl = host(o), host(lse)
    for h in range(H):
        assert_close_bf16(go[0, h, pos_of[h, rows]], ro[0, h], f"semantic shape head {h}")
        assert_lse_close(gl[0, h, pos_of[h, rows]], rl[0, h], f"semantic shape head {h}")


@pytest.mark.parametrize("which", ["q", "k"])
def test_kmeans_full_semantic_shape(which):
    """k-means at the full shape (12 heads, 32760 tokens; 128 query or 256 key
    clusters, 3 iterations): the properties on every head, and on two heads each
    iteration against the oracle's fp64 assignment to the centroids the GPU
    started that iteration from (equal wherever no bf16 rounding of the
    centroids can change the nearest one) and against the same decision taken in
    the kernel's precision (equal wherever fp32 sums cannot change it)."""
    w = WAN480_SEMANTIC
    announce(f"kmeans full semantic shape {which}")
    q, k, v = make_qkv(w)
    x = q if which == "q" else k
    C = w.extra["Cq"] if which == "q" else w.extra["Ck"]
    it = w.extra["iters"]
    xd = dev(x)
    cent, lab, cnt = (host(t) for t in V.vsa_kmeans(xd, C, it))
    check_kmeans_properties(x, cent, lab, cnt, C, "kmeans full")
    assert (cnt.sum(-1) == w.N).all()
    heads = (0, 11)
    prev = {h: x[0, h][(np.arange(C) * w.N) // C] for h in heads}
    for t in range(1, it + 1):
        c_t, l_t, _ = (host(tt) for tt in V.vsa_kmeans(xd, C, t))
        if t == it:
            assert (l_t == lab).all() and (c_t == cent).all()      # deterministic
        for h in heads:
            check_iteration(l_t[0, h], x[0, h], prev[h], t, f"{which} head {h}")
            prev[h] = c_t[0, h]


def test_semantic_layer_full_shape_end_to_end():
    """The semantic layer as the benchmark runs it (Wan 480p shape, 12 heads,
    128 query / 256 key clusters, 3 iterations, top-p 0.9), through
    pipelines.semantic_layer: the k-means outputs are the member means of their
    labels; the cluster scores equal the oracle's size-weighted scores of the
    GPU's own centroids and counts; the kept clusters equal the oracle's top-p
    selection on those scores (gap rule); and O on sampled rows equals oracle
    attention over the kept clusters of the layer's own labels."""
    from tests.selection_rules import check_selection
    w = WAN480_SEMANTIC
    announce("semantic layer full shape")
    q, k, v = make_qkv(w)
    Cq, Ck, top_p = w.extra["Cq"], w.extra["Ck"], w.extra["top_p"]
    stats = {}
    o = PL.semantic_layer(dev(q), dev(k), dev(v), Cq, Ck, w.extra["iters"], top_p, stats=stats)
    go = host(o)
    lq, lk = host(stats["q_labels"]), host(stats["k_labels"])
    cq, ck = host(stats["q_centroids"]), host(stats["k_centroids"])
    nq, nk = host(stats["q_counts"]), host(stats["k_counts"])
    S, idx, cnt = host(stats["scores"]), host(stats["kv_idx"]), host(stats["kv_cnt"])
    heads = (0, 5, 11)
    check_kmeans_properties(q[:, heads], cq[:, heads], lq[:, heads], nq[:, heads], Cq, "q")
    check_kmeans_properties(k[:, heads], ck[:, heads], lk[:, heads], nk[:, heads], Ck, "k")
    scale = 1.0 / np.sqrt(w.D)
    S_ref = np.stack([OS.cluster_scores(cq[0, h], ck[0, h], nk[0, h], scale) for h in range(w.H)])[None]
    fin = np.isfinite(S_ref)
    assert (np.isfinite(S) == fin).all()
    np.testing.assert_allclose(S[fin], S_ref[fin], rtol=1e-5, atol=1e-5)
    n, exact, bad = check_selection(S_ref, None, Ck, top_p, idx, cnt)
    print(f"semantic full shape: {exact}/{n} rows exact, {len(bad)} bad")
    assert not bad, f"rows outside the gap rule: {bad[:5]}"
    rows = sample_rows(w.N, 128, 512, 29)
    for h in heads:
        mask = np.zeros((Cq, Ck), np.uint8)
        for a in range(Cq):
            mask[a, idx[0, h, a, :cnt[0, h, a]]] = 1
        ro, _ = OA.masked_attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], mask, lq[0, h], lk[0, h],
                                    scale, rows=rows)
        assert_close_bf16(go[0, h, rows], ro[0, 0], f"semantic layer head {h}")
