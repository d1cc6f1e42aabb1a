"""Pins of the SVG-EAR oracle (CPU only).

* Closed forms: a skipped block whose keys are all equal is compensated
  exactly, so with such keys the compensated attention equals dense
  attention whatever the exact sets; with every block exact it is dense
  attention.
* Brute force: a tiny case written out with Python floats from the formula
  (exact keys plus n_b-weighted centroid keys).
* Hand-worked block statistics, routing order and exact sets.
* The routing score bounds the centroid's actual error in a block's
  attention mass for the mean query (the inequality it is built on).
"""

import math

import numpy as np

from oracle import ear
from oracle.attention import dense_attention


def rng_qkv(N, d, seed, scale=1.0):
    r = np.random.default_rng(seed)
    return (r.standard_normal((N, d)) * scale, r.standard_normal((N, d)) * scale, r.standard_normal((N, d)))


def full(parts, n):
    return np.concatenate([parts[i] for i in range(n)], axis=0)


def test_identical_keys_in_each_block_make_compensation_exact():
    N, d, bq, bk = 64 * 6 + 20, 32, 64, 64
    q, k, v = rng_qkv(N, d, 1, 1.5)
    for b in range(-(-N // bk)):                 # every block's keys equal to its first one
        k[b * bk:(b + 1) * bk] = k[b * bk]
    nqb, nkb = -(-N // bq), -(-N // bk)
    rng = np.random.default_rng(2)
    exact = (rng.random((nqb, nkb)) < 0.3).astype(np.uint8)
    exact[:, -1] = 1                             # the ragged last block is always exact
    got = full(ear.ear_attention(q, k, v, exact, bq, bk), nqb)
    np.testing.assert_allclose(got, dense_attention(q, k, v), rtol=0, atol=1e-12)


def test_every_block_exact_is_dense_attention():
    N, d, bq, bk = 300, 16, 64, 64
    q, k, v = rng_qkv(N, d, 3, 2.0)
    nqb, nkb = -(-N // bq), -(-N // bk)
    got = full(ear.ear_attention(q, k, v, np.ones((nqb, nkb), np.uint8), bq, bk), nqb)
    np.testing.assert_allclose(got, dense_attention(q, k, v), rtol=0, atol=1e-12)
    # routing with route_k >= nKB makes every block exact, from any mask
    n, kbar, vbar, rad = ear.block_stats(k, v, bk)
    sc = ear.route_scores(q, n, kbar, rad, bq)
    x = ear.exact_sets(np.zeros((nqb, nkb), np.uint8), sc, N, bk, route_k=nkb)
    assert x.all()


def brute(q, k, v, exact, bq, bk):
    """O row by row in Python floats: exact keys of the exact blocks, one
    centroid key per other block with weight n_b."""
    N, d = q.shape
    tau = 1.0 / math.sqrt(d)
    nkb = -(-N // bk)
    out = np.zeros((N, v.shape[1]))
    for i in range(N):
        Q = i // bq
        terms = []                                # (logit, weight, value row)
        for b in range(nkb):
            rows = list(range(b * bk, min(N, (b + 1) * bk)))
            if exact[Q][b]:
                for j in rows:
                    terms.append((tau * sum(float(q[i, c]) * float(k[j, c]) for c in range(d)), 1.0,
                                  [float(x) for x in v[j]]))
            else:
                kb = [sum(float(k[j, c]) for j in rows) / len(rows) for c in range(d)]
                vb = [sum(float(v[j, c]) for j in rows) / len(rows) for c in range(v.shape[1])]
                terms.append((tau * sum(float(q[i, c]) * kb[c] for c in range(d)), float(len(rows)), vb))
        mx = max(t for t, _, _ in terms)
        w = [(wt * math.exp(t - mx), val) for t, wt, val in terms]
        z = sum(a for a, _ in w)
        out[i] = [sum(a * val[c] for a, val in w) / z for c in range(v.shape[1])]
    return out


def test_against_brute_force_tiny():
    N, d, bq, bk = 37, 4, 8, 8
    q, k, v = rng_qkv(N, d, 5, 1.2)
    nqb, nkb = -(-N // bq), -(-N // bk)
    exact = (np.random.default_rng(6).random((nqb, nkb)) < 0.4).astype(np.uint8)
    exact[:, -1] = 1
    exact[2, :] = 0                              # a q-block with only compensated blocks
    got = full(ear.ear_attention(q, k, v, exact, bq, bk), nqb)
    np.testing.assert_allclose(got, brute(q, k, v, exact, bq, bk), rtol=1e-12, atol=1e-12)


def test_block_stats_hand_worked():
    k = np.array([[0, 0], [2, 0], [0, 2], [2, 2], [5, 5]], dtype=np.float64)
    v = np.array([[1, 0], [3, 0], [1, 0], [3, 4], [7, 7]], dtype=np.float64)
    n, kbar, vbar, rad = ear.block_stats(k, v, bk=4)
    np.testing.assert_array_equal(n, [4, 1])
    np.testing.assert_array_equal(kbar, [[1, 1], [5, 5]])
    np.testing.assert_array_equal(vbar, [[2, 1], [7, 7]])
    np.testing.assert_allclose(rad, [math.sqrt(2), 0.0])


def test_route_order_and_exact_sets():
    """Two q-blocks over four kv-blocks of 2 keys: block 1 has radius 0 (its
    compensation is exact: score -inf), blocks 2 and 3 are the same block
    twice (a tie: the lower index goes first)."""
    d, bk = 2, 2
    k = np.array([[1, 0], [-1, 0],     # block 0: centroid 0, radius 1
                  [3, 3], [3, 3],      # block 1: radius 0
                  [2, 0], [0, 2],      # block 2: centroid (1, 1), radius sqrt(2)
                  [2, 0], [0, 2]],     # block 3: the same
                 dtype=np.float64)
    v = np.zeros_like(k)
    q = np.array([[1, 1], [1, 1], [0, 0], [0, 0]], dtype=np.float64)   # two q-blocks of 2 rows
    n, kbar, vbar, rad = ear.block_stats(k, v, bk)
    sc = ear.route_scores(q, n, kbar, rad, bq=2)
    tau = 1 / math.sqrt(2)
    qn = math.sqrt(2)
    want0 = [math.log(2) + 0 + math.log(math.expm1(tau * qn * 1)), -math.inf,
             math.log(2) + tau * 2 + math.log(math.expm1(tau * qn * math.sqrt(2)))]
    np.testing.assert_allclose(sc[0, :3], want0)
    assert sc[0, 2] == sc[0, 3] and sc[1, 0] == -math.inf       # qbar = 0: nothing to route by
    x = ear.exact_sets(np.zeros((2, 4), np.uint8), sc, N=8, bk=bk, route_k=1)
    np.testing.assert_array_equal(x[0], [0, 0, 1, 0])            # the tie goes to block 2
    x = ear.exact_sets(np.array([[0, 0, 1, 0], [0, 0, 0, 0]], np.uint8), sc, N=8, bk=bk, route_k=1)
    np.testing.assert_array_equal(x[0], [0, 0, 1, 1])            # kept block 2, routes block 3
    x = ear.exact_sets(np.zeros((2, 4), np.uint8), sc, N=7, bk=bk, route_k=0)
    np.testing.assert_array_equal(x[:, 3], [1, 1])               # the ragged last block is exact


def test_route_score_bounds_the_centroid_mass_error():
    """For the mean query of each q-block, | sum_j e^{s_j} - n_b e^{t_b} | <=
    E_Qb for every block: the score is the bound the routing ranks by."""
    N, d, bq, bk = 64 * 5, 16, 64, 64
    q, k, v = rng_qkv(N, d, 9, 1.0)
    n, kbar, vbar, rad = ear.block_stats(k, v, bk)
    sc = ear.route_scores(q, n, kbar, rad, bq)
    tau = 1 / math.sqrt(d)
    for Q in range(N // bq):
        qbar = q[Q * bq:(Q + 1) * bq].mean(axis=0)
        for b in range(N // bk):
            mass = np.exp(tau * (k[b * bk:(b + 1) * bk] @ qbar)).sum()
            comp = n[b] * math.exp(tau * kbar[b] @ qbar)
            assert abs(mass - comp) <= math.exp(sc[Q, b]) * (1 + 1e-12)
