"""Pins for the oracle's SVG2 path (CPU only).

* Lloyd k-means: a hand-worked 1-D example with a tie; an empty cluster keeps
  its centroid; scikit-learn's Lloyd from the same initial centroids at
  convergence (a library routine); recovery of the generating mixture
  components; the inertia never increases.
* Cluster permutation: a pure-Python counting sort.
* Top-p: hand cases; p = 1 keeps every non-empty cluster; p near 0 keeps
  the argmax alone.
* Varlen attention: all pairs equal dense attention; K = 0 gives the mean of
  V over the selected clusters.
"""

import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import svg2, numerics
from oracle.attention import dense_attention
from synth import SVG2_COG
from synth.generators import mixture_qkv


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_kmeans_hand_example():
    g = load("kmeans_small.json")
    x = np.array(g["x"])[:, None]
    for iters, key in ((1, "after_1_iteration"), (3, "after_3_iterations")):
        a, c, s, _ = svg2.kmeans(x, g["init_idx"], iters)
        np.testing.assert_array_equal(a, g[key]["assign"])
        np.testing.assert_allclose(c[:, 0], g[key]["centroids"], rtol=1e-15)
        np.testing.assert_array_equal(s, g[key]["sizes"])
    _, _, _, margin = svg2.kmeans(x, g["init_idx"], 1)
    assert margin == 0.0                        # the tie is recorded as a zero margin


def test_kmeans_empty_cluster_keeps_centroid():
    """Worked by hand.  Centroids start at (0,0), (0,0), (0,1).  Iteration 1:
    the ties go to cluster 0, so assign = [0, 0, 2] and cluster 1 is empty.
    It keeps (0,0) while cluster 0 moves to (0.5, 0).  Iteration 2: point
    (0,0) is now nearest to the kept centroid 1, so assign = [1, 0, 2]."""
    x = np.array([[0.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    a, c, s, _ = svg2.kmeans(x, [0, 0, 2], 1)
    np.testing.assert_array_equal(a, [0, 0, 2])
    np.testing.assert_array_equal(s, [2, 0, 1])
    np.testing.assert_array_equal(c, [[0.5, 0.0], [0.0, 0.0], [0.0, 1.0]])
    a, c, s, _ = svg2.kmeans(x, [0, 0, 2], 2)
    np.testing.assert_array_equal(a, [1, 0, 2])
    np.testing.assert_array_equal(c, [[1.0, 0.0], [0.0, 0.0], [0.0, 1.0]])


def test_kmeans_matches_sklearn_lloyd_at_convergence():
    sklearn_cluster = pytest.importorskip("sklearn.cluster")
    rng = np.random.default_rng(21)
    means = rng.standard_normal((6, 5)) * 4
    comp = rng.integers(0, 6, size=400)
    x = means[comp] + 0.5 * rng.standard_normal((400, 5))
    init = np.array([np.flatnonzero(comp == j)[0] for j in range(6)])
    a, c, s, _ = svg2.kmeans(x, init, 20)
    km = sklearn_cluster.KMeans(n_clusters=6, init=x[init], n_init=1, max_iter=20, tol=0.0,
                                algorithm="lloyd").fit(x)
    np.testing.assert_array_equal(a, km.labels_)
    np.testing.assert_allclose(c, km.cluster_centers_, rtol=1e-12, atol=1e-12)


def test_kmeans_inertia_non_increasing_and_fixed_point():
    rng = np.random.default_rng(22)
    x = rng.standard_normal((300, 4))
    init = rng.choice(300, size=7, replace=False)
    prev = np.inf
    for it in range(1, 9):
        a, c, s, _ = svg2.kmeans(x, init, it)
        inertia = ((x - c[a]) ** 2).sum()
        assert inertia <= prev + 1e-9
        prev = inertia
    a30, c30, _, _ = svg2.kmeans(x, init, 30)
    # fixed point: each point's nearest centroid is its own, and each centroid is its cluster mean
    d2 = ((x[:, None, :] - c30[None]) ** 2).sum(-1)
    np.testing.assert_array_equal(d2.argmin(axis=1), a30)
    for j in range(7):
        if (a30 == j).any():
            np.testing.assert_allclose(c30[j], x[a30 == j].mean(axis=0), rtol=1e-12)


def test_kmeans_recovers_mixture_components():
    w = SVG2_COG
    g = mixture_qkv(w)
    for h in (0, w.H - 1):
        for side, kk in (("q", w.kq), ("k", w.kk)):
            x = numerics.as_f64(g[side][h], "bf16")
            a, c, s, margin = svg2.kmeans(x, g["init_" + side][h], w.iters)
            np.testing.assert_array_equal(a, g["comp_" + side][h])
            assert margin > 1e-3


def test_cluster_permute_counting_sort():
    rng = np.random.default_rng(23)
    k = 9
    a = rng.integers(0, k, size=200)
    a[a == 4] = 5                               # an empty cluster
    perm, offs = svg2.cluster_permute(a, k)
    buckets = [[] for _ in range(k)]
    for i, c in enumerate(a):
        buckets[c].append(i)
    np.testing.assert_array_equal(perm, [i for b in buckets for i in b])
    np.testing.assert_array_equal(offs, np.cumsum([0] + [len(b) for b in buckets]))


def test_select_pairs_hand_cases():
    g = load("topp_small.json")
    for case in g["cases"]:
        sizes = np.array(case["sizes"])
        kk = sizes.size
        rng = np.random.default_rng(kk)
        ck = rng.standard_normal((kk, 4))
        ptr, idx, _ = svg2.select_pairs(np.zeros((1, 4)), ck, sizes, case["p"])
        np.testing.assert_array_equal(idx[ptr[0]:ptr[1]], case["expect"])


def test_select_pairs_extremes():
    rng = np.random.default_rng(24)
    cq, ck = rng.standard_normal((5, 8)), rng.standard_normal((12, 8))
    sizes = rng.integers(1, 50, size=12)
    sizes[3] = 0
    ptr, idx, _ = svg2.select_pairs(cq, ck, sizes, 1.0)
    live = np.flatnonzero(sizes > 0)
    for i in range(5):
        np.testing.assert_array_equal(idx[ptr[i]:ptr[i + 1]], live)
    ptr, idx, _ = svg2.select_pairs(cq, ck, sizes, 1e-9)
    for i in range(5):
        logits = ck[live] @ cq[i] / np.sqrt(8) + np.log(sizes[live])
        np.testing.assert_array_equal(idx[ptr[i]:ptr[i + 1]], [live[logits.argmax()]])


def test_varlen_all_pairs_is_dense_and_k_zero_mean():
    rng = np.random.default_rng(25)
    N, d = 90, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    aq, ak = rng.integers(0, 4, size=N), rng.integers(0, 6, size=N)
    ptr = np.arange(0, 25, 6, dtype=np.int32)
    idx = np.tile(np.arange(6, dtype=np.int32), 4)
    np.testing.assert_allclose(svg2.varlen_attention(q, k, v, aq, ak, ptr, idx), dense_attention(q, k, v),
                               rtol=1e-12, atol=1e-13)
    ptr = np.array([0, 2, 3, 3, 6], dtype=np.int32)
    idx = np.array([1, 4, 0, 2, 3, 5], dtype=np.int32)
    o = svg2.varlen_attention(q, np.zeros((N, d)), v, aq, ak, ptr, idx)
    for i in range(N):
        sel = idx[ptr[aq[i]]:ptr[aq[i] + 1]]
        keys = np.isin(ak, sel)
        expect = v[keys].mean(axis=0) if keys.any() else np.zeros(d)
        np.testing.assert_allclose(o[i], expect, rtol=1e-12, atol=1e-13)


def test_svg2_workload_margin_audit():
    """The SVG2 workload's seed gives decisions that do not hinge on rounding:
    every k-means assignment beats the runner-up by >= 0.1% of its squared
    distance; every top-p crossing clears p by > 1e-8 on both sides, and the
    last kept cluster's probability beats the first dropped one by > 1e-8.
    (The GPU path scores pairs in float64 from float64 centroids.)  Every
    assignment also clears the worst-case float32 rounding of the squared
    distances (ratio > 1.01), so a float32 argmin in any summation order
    takes the same decisions as the float64 one."""
    w = SVG2_COG
    g = mixture_qkv(w)
    for h in range(w.H):
        q = numerics.as_f64(g["q"][h], "bf16")
        k = numerics.as_f64(g["k"][h], "bf16")
        aq, cq, sq, mq, rq = svg2.kmeans(q, g["init_q"][h], w.iters, f32_audit=True)
        ak, ck, sk, mk, rk = svg2.kmeans(k, g["init_k"][h], w.iters, f32_audit=True)
        assert mq > 1e-3 and mk > 1e-3
        assert rq > 1.01 and rk > 1.01, (h, rq, rk)
        ptr, idx, marg = svg2.select_pairs(cq, ck, sk, w.top_p)
        assert marg.min() > 1e-8, (h, marg.min(axis=0))


def test_kmeans_f32_audit_closed_forms():
    """The float32 decision audit on 1-D cases worked by hand (d = 1, so the
    error bound is B = 5u (x^2 + m^2 + 2|x m|), u = 2^-24).  Points 1, 0, 3
    against centroids 0 and 3 give gaps 3, 9, 9 over bounds 85u, 45u, 225u;
    the smallest ratio is 3 / (85u).  A point 2^-30 off the midpoint of 0
    and 1 gives gap 2^-29 over 12.5u: ratio 2^-5 / 12.5 = 0.0025, a decision
    that float32 rounding could flip."""
    x = np.array([[1.0], [0.0], [3.0]])
    r = svg2.kmeans(x, [1, 2], 1, f32_audit=True)[4]
    assert r == pytest.approx(3 * 2 ** 24 / 85, rel=1e-12)
    x = np.array([[0.0], [1.0], [0.5 + 2.0 ** -30]])
    r = svg2.kmeans(x, [0, 1], 1, f32_audit=True)[4]
    assert r == pytest.approx(0.0025, rel=1e-6)
    # A centroid equal to the winner bit for bit is no decision.  Centroids
    # 0, 0, 4: point 0 vs 4 gives 16 / 80u, point 4 vs 0 gives 16 / 400u,
    # point 1 vs 4 gives 8 / 130u; without the skip point 0 would give 0.
    x = np.array([[0.0], [4.0], [1.0]])
    r = svg2.kmeans(x, [0, 0, 1], 1, f32_audit=True)[4]
    assert r == pytest.approx(16 / 400 * 2 ** 24, rel=1e-12)
