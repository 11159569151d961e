"""Pins of the semantic-aware permutation oracle against results fixed
independently of it: a hand-worked k-means, scikit-learn's Lloyd k-means, the
exact attention mass of a cluster when keys equal their centroid, torch SDPA when
every cluster is kept, and the same attention computed in cluster-major storage."""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import semantic as OS
from workloads import to_bf16_values


def bf16(x):
    """Values rounded to bf16, held in fp64."""
    return to_bf16_values(x).astype(np.float64)


def blobs(N, C, D, seed, spread=0.05):
    g = np.random.default_rng(seed)
    centers = 3.0 * g.standard_normal((C, D))
    lab = g.integers(0, C, N)
    return centers[lab] + spread * g.standard_normal((N, D)), lab


def test_kmeans_hand_worked_1d():
    """Points 0, 1, 10, 11 (D = 1, exact in bf16), C = 2: seeds at positions 0 and
    2 (values 0 and 10); one iteration gives clusters {0, 1} and {10, 11} with
    means 0.5 and 10.5, and a second iteration changes nothing."""
    x = np.array([[0.0], [1.0], [10.0], [11.0]])
    cent, lab, cnt = OS.kmeans(x, 2, 1)
    assert lab.tolist() == [0, 0, 1, 1]
    assert cent[:, 0].tolist() == [0.5, 10.5] and cnt.tolist() == [2, 2]
    cent2, lab2, _ = OS.kmeans(x, 2, 2)
    assert lab2.tolist() == [0, 0, 1, 1] and cent2[:, 0].tolist() == [0.5, 10.5]


def test_kmeans_empty_cluster_keeps_centroid_and_ties_go_low():
    """N = 4, C = 2: seeds at positions 0 and 2, both the value 0, so every point is
    equally near both; all go to cluster 0 (mean 3) and cluster 1 stays empty with
    its seed."""
    x = np.array([[0.0], [5.0], [0.0], [7.0]])
    cent, lab, cnt = OS.kmeans(x, 2, 1)
    assert lab.tolist() == [0, 0, 0, 0]
    assert cnt.tolist() == [4, 0]
    assert cent[0, 0] == 3.0 and cent[1, 0] == 0.0


@pytest.mark.parametrize("iters", [1, 2, 4])
def test_kmeans_matches_scikit_learn_on_generic_data(iters):
    """Generic data, the same seeds: after `iters` Lloyd iterations the centroids
    equal scikit-learn's, and its final labels (one more assignment, in fp64)
    equal this oracle's assignment to those centroids outright, for every token."""
    from sklearn.cluster import KMeans
    g = np.random.default_rng(1)
    x = bf16(g.standard_normal((500, 16)))
    C = 12
    seeds = x[(np.arange(C) * len(x)) // C]
    cent, lab, cnt = OS.kmeans(x, C, iters)
    assert (cnt > 0).all()                                   # (scikit-learn relocates empty clusters)
    km = KMeans(n_clusters=C, init=seeds, n_init=1, max_iter=iters, tol=0.0, algorithm="lloyd").fit(x)
    np.testing.assert_allclose(km.cluster_centers_, cent, atol=1e-12)
    np.testing.assert_array_equal(km.labels_, OS.assign(x, cent))


def test_assign_is_nearest_centroid_by_brute_force():
    """The assignment equals a scalar loop over every (token, centroid) pair of
    squared Euclidean distances, the first minimum winning; duplicated centroids
    send their tokens to the lower index."""
    g = np.random.default_rng(9)
    x = g.standard_normal((60, 5))
    m = g.standard_normal((7, 5))
    m[5] = m[2]                                              # a duplicate: index 2 must win
    got = OS.assign(x, m)
    for i in range(len(x)):
        best, bd = 0, None
        for c in range(len(m)):
            d = sum((x[i, j] - m[c, j]) ** 2 for j in range(5))
            if bd is None or d < bd:
                best, bd = c, d
        assert got[i] == best
    assert 5 not in got.tolist()


def test_kmeans_converges_like_scikit_learn_on_sorted_blobs():
    """Blobs stored one after another, one seed in each: both converge to the
    planted partition with the blob means as centroids."""
    from sklearn.cluster import KMeans
    C, per, D = 6, 90, 24
    g = np.random.default_rng(2)
    centers = 3.0 * g.standard_normal((C, D))
    x = bf16(np.repeat(centers, per, axis=0) + 0.3 * g.standard_normal((C * per, D)))
    seeds = x[(np.arange(C) * len(x)) // C]
    cent, lab, _ = OS.kmeans(x, C, 5)
    km = KMeans(n_clusters=C, init=seeds, n_init=1, max_iter=5, tol=0.0, algorithm="lloyd").fit(x)
    np.testing.assert_array_equal(lab, np.repeat(np.arange(C), per))
    np.testing.assert_array_equal(km.labels_, lab)
    np.testing.assert_allclose(km.cluster_centers_, cent, atol=1e-12)
    np.testing.assert_allclose(cent, x.reshape(C, per, D).mean(1), atol=1e-12)


def test_kmeans_recovers_planted_blobs():
    x, truth = blobs(800, 6, 32, 2, spread=0.02)
    _, lab, _ = OS.kmeans(bf16(x), 12, 8)
    # every found cluster lies inside one planted blob
    for c in np.unique(lab):
        assert np.unique(truth[lab == c]).size == 1


def test_cluster_order_is_stable_cluster_major():
    lab = np.random.default_rng(3).integers(0, 7, 500)
    lab[lab == 4] = 5                                        # an empty cluster
    perm, off = OS.cluster_order(lab, 7)
    assert sorted(perm.tolist()) == list(range(500))
    assert (np.diff(lab[perm]) >= 0).all()
    for c in range(7):
        seg = perm[off[c]:off[c + 1]]
        assert (lab[seg] == c).all() and (np.diff(seg) > 0).all()
    assert off[4] == off[5] and off[-1] == 500


def test_size_weighted_scores_are_exact_attention_mass():
    """Keys equal to their cluster's centroid, a query equal to its centroid: the
    softmax over S_a. is exactly the share of the query's attention that each key
    cluster receives (computed by plain attention over all keys)."""
    g = np.random.default_rng(4)
    D, Ck = 16, 5
    ck = g.standard_normal((Ck, D))
    sizes = np.array([3, 1, 7, 0, 4])
    kl = np.repeat(np.arange(Ck), sizes)
    k = ck[kl]
    cq = g.standard_normal((2, D))
    scale = 0.3
    S = OS.cluster_scores(cq, ck, sizes, scale)
    assert np.isneginf(S[:, 3]).all()
    for a in range(2):
        q = cq[a][None, None, None, :]
        _, _, p = OA.masked_attention(q, k[None, None], k[None, None], np.ones((1, 1), np.uint8), [0],
                                      np.zeros(len(k), np.int64), scale, return_probs=True)
        mass = np.bincount(kl, weights=p[0, 0, 0], minlength=Ck)
        e = np.exp(S[a] - S[a][np.isfinite(S[a])].max())
        np.testing.assert_allclose(e / e.sum(), mass, atol=1e-12)


def test_pipeline_keeping_every_cluster_is_dense_attention():
    g = np.random.default_rng(5)
    q, k, v = (g.standard_normal((1, 2, 96, 16)) for _ in range(3))
    o, lse, parts = OS.semantic_pipeline(q, k, v, 4, 6, 3, top_p=1.0)
    assert (parts["kv_cnt"] == 6).all()
    ref = torch.nn.functional.scaled_dot_product_attention(*(torch.tensor(x) for x in (q, k, v))).numpy()
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_pipeline_in_cluster_major_storage():
    """Storing Q by query cluster and K, V by key cluster, attending over the kept
    clusters' contiguous key ranges and moving O back gives the same result."""
    g = np.random.default_rng(6)
    q, k, v = (g.standard_normal((1, 1, 120, 8)) for _ in range(3))
    o, _, P = OS.semantic_pipeline(q, k, v, 5, 7, 4, top_p=0.8)
    pq, oq = OS.cluster_order(P["q_labels"][0, 0], 5)
    pk, ok = OS.cluster_order(P["k_labels"][0, 0], 7)
    qs, ks, vs = q[0, 0, pq], k[0, 0, pk], v[0, 0, pk]
    out = np.zeros_like(qs)
    for a in range(5):
        keys = np.concatenate([np.arange(ok[b], ok[b + 1]) for b in P["kv_idx"][0, 0, a, :P["kv_cnt"][0, 0, a]]])
        s = (qs[oq[a]:oq[a + 1]] @ ks[keys].T) / np.sqrt(8)
        p = np.exp(s - s.max(1, keepdims=True))
        out[oq[a]:oq[a + 1]] = (p / p.sum(1, keepdims=True)) @ vs[keys]
    back = np.zeros_like(out)
    back[pq] = out
    np.testing.assert_allclose(back, o[0, 0], atol=1e-12)
    # budget: top-p 0.8 keeps fewer than all clusters somewhere
    assert P["kv_cnt"].min() < 7


def test_kept_flops_counts_pairs():
    qc = np.array([[[2, 3]]])
    kc = np.array([[[4, 0, 5]]])
    idx = np.array([[[[0, 2, -1], [1, -1, -1]]]])
    cnt = np.array([[[2, 1]]])
    assert OS.kept_flops_semantic(qc, kc, idx, cnt, 8) == 4 * 8 * (2 * 9 + 3 * 0)
