"""Pins of the HVA-style clustering oracle (CPU only).

* Brute force: candidate windows found by decoding every cluster id (not by
  the oracle's neighbour offsets), and a tiny local k-means written out with
  scalar float32 operations, one token and one dim at a time.
* Reduction to a library routine: with at most two windows along every axis
  every token sees every centroid, so local k-means is Lloyd's algorithm;
  scikit-learn's Lloyd from the same seeds must agree at convergence.
* Hand-worked cases: a 1-D grid with a tie (the lower id wins), the Lowe
  flags of two middle tokens, refresh with no and with every flag.
* Invariants: the objective never rises over iterations; every token's
  cluster is one of its candidates; centroids are their members' means.
* On well-separated data the float32 decisions equal float64 ones.
"""

import numpy as np
import pytest

from oracle import hva


def ids_decode(cid, n):
    nF, nY, nX = n
    return cid // (nY * nX), (cid // nX) % nY, cid % nX


def test_candidates_by_decoding_every_cluster():
    F, rows, cols, win = 5, 4, 7, (2, 3, 2)
    nF, nY, nX = -(-F // 2), -(-rows // 3), -(-cols // 2)
    cand = hva.candidates(F, rows, cols, win)
    for t in range(F * rows * cols):
        f, r = divmod(t, rows * cols)
        y, x = divmod(r, cols)
        a, b, c = f // 2, y // 3, x // 2
        want = [j for j in range(nF * nY * nX)
                if all(abs(u - v) <= 1 for u, v in zip(ids_decode(j, (nF, nY, nX)), (a, b, c)))]
        got = [j for j in cand[t] if j >= 0]
        assert got == want, t


def brute_local_kmeans(x, F, rows, cols, T, win, iters, r2=np.float32(0.64)):
    """Scalar-loop local k-means with float32 distances (dims in order)."""
    wf, wy, wx = win
    n = (-(-F // wf), -(-rows // wy), -(-cols // wx))
    C = n[0] * n[1] * n[2]
    k = C + (1 if T else 0)
    N, d = x.shape
    Nv = F * rows * cols

    def cell(t):
        f, r = divmod(t, rows * cols)
        y, xx = divmod(r, cols)
        return f // wf, y // wy, xx // wx

    assign = [((a * n[1] + b) * n[2] + c) for a, b, c in (cell(t) for t in range(Nv))] + [C] * T
    cent = [[0.0] * d for _ in range(k)]

    def update():
        for j in range(k):
            members = [t for t in range(N) if assign[t] == j]
            if members:
                cent[j] = [sum(float(x[t, c]) for t in members) / len(members) for c in range(d)]

    update()
    flags = [0] * N
    for _ in range(iters):
        new = list(assign)
        for t in range(Nv):
            a, b, c = cell(t)
            best, d1, d2 = None, np.float32(np.inf), np.float32(np.inf)
            for j in range(C):
                if not all(abs(u - v) <= 1 for u, v in zip(ids_decode(j, n), (a, b, c))):
                    continue
                acc = np.float32(0.0)
                for dim in range(d):
                    diff = np.float32(x[t, dim]) - np.float32(cent[j][dim])
                    acc = np.float32(acc + np.float32(diff * diff))
                if acc < d1:
                    best, d2, d1 = j, d1, acc
                elif acc < d2:
                    d2 = acc
            new[t] = best
            flags[t] = int(bool(np.isfinite(d2)) and bool(d1 >= np.float32(r2 * d2)))
        assign[:] = new
        update()
    return np.array(assign), np.array(cent), np.array(flags)


def test_tiny_against_scalar_brute_force():
    F, rows, cols, T, d, win = 3, 4, 5, 3, 3, (2, 2, 2)
    rng = np.random.default_rng(3)
    x = np.round(rng.standard_normal((F * rows * cols + T, d)) * 8) / 8   # exact in bf16
    for iters in (1, 3):
        a, c, s, r = hva.local_kmeans(x, F, rows, cols, T, win, iters)
        ba, bc, bf = brute_local_kmeans(x, F, rows, cols, T, win, iters)
        np.testing.assert_array_equal(a, ba)
        np.testing.assert_array_equal(c, bc)
        np.testing.assert_array_equal(r, bf)
        np.testing.assert_array_equal(s, np.bincount(a, minlength=c.shape[0]))


def test_one_dimensional_hand_worked_with_tie():
    """Six tokens in one row, windows of two: values 0 9 10 11 17 30.
    Seeds 4.5, 10.5, 23.5.  Token 17 is 6.5 from both 10.5 and 23.5: the tie
    goes to window 1.  After the update the means are 0, 11.75, 30, and the
    second assignment keeps every token where it is."""
    x = np.array([0, 9, 10, 11, 17, 30], dtype=np.float64)[:, None]
    a, c, s, r = hva.local_kmeans(x, 1, 1, 6, 0, (1, 1, 2), iters=1)
    np.testing.assert_array_equal(a, [0, 1, 1, 1, 1, 2])
    np.testing.assert_array_equal(c[:, 0], [0.0, 11.75, 30.0])
    np.testing.assert_array_equal(s, [1, 4, 1])
    a2, c2, _, _ = hva.local_kmeans(x, 1, 1, 6, 0, (1, 1, 2), iters=2)
    np.testing.assert_array_equal(a2, a)
    np.testing.assert_array_equal(c2, c)


def test_lowe_flags_hand_worked():
    """Values 0, 4.875, 5.125, 10 in windows of two: means 2.4375 and 7.5625.
    The middle tokens are 2.4375 from their own mean and 2.6875 from the
    other: 5.94140625 >= 0.64 * 7.22265625, flagged.  The end tokens have
    5.94140625 against 57.19140625: not flagged."""
    x = np.array([0, 4.875, 5.125, 10], dtype=np.float64)[:, None]
    a, c, _, r = hva.local_kmeans(x, 1, 1, 4, 0, (1, 1, 2), iters=1)
    np.testing.assert_array_equal(a, [0, 0, 1, 1])
    np.testing.assert_array_equal(c[:, 0], [2.4375, 7.5625])
    np.testing.assert_array_equal(r, [0, 1, 1, 0])
    # with r2 = 0.9: 5.94140625 < 0.9 * 7.22265625 = 6.50: nothing flagged
    _, _, _, r = hva.local_kmeans(x, 1, 1, 4, 0, (1, 1, 2), iters=1, r2=np.float32(0.9))
    assert not r.any()
    # with r2 = 0.36 every token is flagged except the ends (5.94 < 0.36 * 57.19 = 20.6)
    _, _, _, r = hva.local_kmeans(x, 1, 1, 4, 0, (1, 1, 2), iters=1, r2=np.float32(0.36))
    np.testing.assert_array_equal(r, [0, 1, 1, 0])


def test_few_windows_is_lloyd_from_the_window_seeds():
    """Two windows along every axis: each token's candidates are all eight
    windows, so local k-means is Lloyd's; scikit-learn (float64, same seeds)
    agrees at convergence on well-separated data."""
    sklearn = pytest.importorskip("sklearn.cluster")
    F, rows, cols, win, d = 4, 6, 6, (2, 3, 3), 8
    rng = np.random.default_rng(5)
    _, _, _, cid, _ = hva.grid_windows(F, rows, cols, win)
    means = rng.standard_normal((8, d)) * 6
    # 80% of a window's tokens from its own component, 20% from any: the seeds
    # are mixtures, and Lloyd moves the strays to their components
    lab = np.where(rng.random(cid.size) < 0.8, cid, rng.integers(0, 8, size=cid.size))
    x = np.round((means[lab] + 0.3 * rng.standard_normal((cid.size, d))) * 64) / 64
    seeds, _ = hva.means(x, cid, 8, np.zeros((8, d)))
    a, c, s, _ = hva.local_kmeans(x, F, rows, cols, 0, win, iters=40)
    assert np.any(a != cid)                                    # tokens did move
    km = sklearn.KMeans(n_clusters=8, init=seeds, n_init=1, max_iter=300, tol=0.0, algorithm="lloyd").fit(x)
    np.testing.assert_array_equal(a, km.labels_)
    np.testing.assert_allclose(c, km.cluster_centers_, rtol=0, atol=1e-12)


def blob_like(F, rows, cols, T, d, m, seed):
    rng = np.random.default_rng(seed)
    f, y, xx = np.meshgrid(np.arange(F), np.arange(rows), np.arange(cols), indexing="ij")
    pos = np.stack([f.ravel() * 3.0, y.ravel(), xx.ravel()], axis=1)
    cen = rng.random((m, 3)) * np.array([3.0 * F, rows, cols])
    comp = ((pos[:, None] - cen[None]) ** 2).sum(axis=2).argmin(axis=1)
    mu = rng.standard_normal((m + 1, d)) * 2
    comp = np.concatenate([comp, np.full(T, m)])
    return np.round((mu[comp] + 0.5 * rng.standard_normal((comp.size, d))) * 32) / 32


def test_objective_never_rises_and_invariants():
    F, rows, cols, T, d, win = 6, 8, 10, 5, 16, (2, 3, 4)
    x = blob_like(F, rows, cols, T, d, 12, seed=8)
    cand = hva.candidates(F, rows, cols, win)
    prev = np.inf
    for iters in range(0, 7):
        a, c, s, r = hva.local_kmeans(x, F, rows, cols, T, win, iters)
        e = hva.sse(x, a, c)
        assert e <= prev * (1 + 1e-9)
        prev = e
        Nv = F * rows * cols
        assert all(a[t] in cand[t] for t in range(Nv))
        assert np.all(a[Nv:] == c.shape[0] - 1)
        for j in range(c.shape[0]):
            if s[j]:
                np.testing.assert_allclose(c[j], x[a == j].mean(axis=0), rtol=1e-15, atol=1e-15)


def test_float32_decisions_equal_float64_when_separated():
    F, rows, cols, d, win = 4, 6, 8, 16, (2, 3, 4)
    rng = np.random.default_rng(11)
    _, _, _, cid, _ = hva.grid_windows(F, rows, cols, win)
    mu = rng.standard_normal((cid.max() + 1, d)) * 10
    x = np.round((mu[cid] + 0.2 * rng.standard_normal((cid.size, d))) * 16) / 16
    cent, _ = hva.means(x, cid, cid.max() + 1, np.zeros((cid.max() + 1, d)))
    cand = hva.candidates(F, rows, cols, win)
    best, _, _, _ = hva.assign_local(x, cent, cand)
    d64 = np.where(cand >= 0, ((x[:, None, :] - cent[np.maximum(cand, 0)]) ** 2).sum(axis=2), np.inf)
    np.testing.assert_array_equal(best, cand[np.arange(cid.size), d64.argmin(axis=1)])


def test_refresh_with_every_flag_is_one_more_iteration():
    F, rows, cols, T, d, win = 5, 6, 9, 4, 8, (2, 3, 3)
    x = blob_like(F, rows, cols, T, d, 10, seed=12)
    a, c, _, _ = hva.local_kmeans(x, F, rows, cols, T, win, iters=2)
    a3, c3, s3, _ = hva.local_kmeans(x, F, rows, cols, T, win, iters=3)
    ones = np.ones(x.shape[0], dtype=np.uint8)
    ra, rc, rs = hva.refresh_step(x, a, c, ones, F, rows, cols, T, win)
    np.testing.assert_array_equal(ra, a3)
    np.testing.assert_array_equal(rc, c3)
    np.testing.assert_array_equal(rs, s3)


def test_refresh_with_no_flag_keeps_clusters_and_takes_new_means():
    F, rows, cols, T, d, win = 5, 6, 9, 4, 8, (2, 3, 3)
    x = blob_like(F, rows, cols, T, d, 10, seed=13)
    a, c, _, _ = hva.local_kmeans(x, F, rows, cols, T, win, iters=3)
    x2 = x + np.round(np.random.default_rng(1).standard_normal(x.shape) * 4) / 32
    ra, rc, rs = hva.refresh_step(x2, a, c, np.zeros(x.shape[0], np.uint8), F, rows, cols, T, win)
    np.testing.assert_array_equal(ra, a)
    for j in range(c.shape[0]):
        if rs[j]:
            np.testing.assert_allclose(rc[j], x2[a == j].mean(axis=0), rtol=1e-15, atol=1e-15)
        else:
            np.testing.assert_array_equal(rc[j], c[j])
