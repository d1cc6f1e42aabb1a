"""Pins for the oracle's attention (CPU only).

Each check comes from outside the oracle's own code:
* a per-element brute force in Python floats;
* PyTorch's scaled_dot_product_attention in float64 on the CPU (a library
  routine);
* closed forms: K = 0 gives the mean of V over the kept keys; a constant V
  gives that constant;
* permutation equivariance.
"""

import math

import numpy as np
import pytest
import torch

from oracle.attention import (softmax_attention, dense_attention, block_sparse_attention,
                              block_sparse_attention_full)


def brute_force(q, k, v, scale, keep=None):
    m, n, dv = q.shape[0], k.shape[0], v.shape[1]
    out = [[0.0] * dv for _ in range(m)]
    for i in range(m):
        logits = []
        for j in range(n):
            if keep is not None and not keep[i][j]:
                continue
            s = 0.0
            for c in range(q.shape[1]):
                s += float(q[i, c]) * float(k[j, c])
            logits.append((j, s * scale))
        if not logits:
            continue
        mx = max(s for _, s in logits)
        w = [(j, math.exp(s - mx)) for j, s in logits]
        z = sum(x for _, x in w)
        for c in range(dv):
            out[i][c] = sum(x * float(v[j, c]) for j, x in w) / z
    return np.array(out)


def test_brute_force_dense_and_masked():
    rng = np.random.default_rng(0)
    q, k, v = rng.standard_normal((5, 3)), rng.standard_normal((7, 3)), rng.standard_normal((7, 2))
    np.testing.assert_allclose(softmax_attention(q, k, v, 0.7), brute_force(q, k, v, 0.7), rtol=1e-12, atol=1e-13)
    keep = rng.random((5, 7)) < 0.5
    keep[0] = False                      # empty row -> 0
    np.testing.assert_allclose(softmax_attention(q, k, v, 0.7, keep), brute_force(q, k, v, 0.7, keep),
                               rtol=1e-12, atol=1e-13)
    assert np.all(softmax_attention(q, k, v, 0.7, keep)[0] == 0.0)


@pytest.mark.parametrize("d", [64, 128])
def test_matches_torch_sdpa_float64(d):
    rng = np.random.default_rng(d)
    N = 200
    q, k, v = (rng.standard_normal((N, d)) * 2 for _ in range(3))
    ours = dense_attention(q, k, v, chunk=64)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None])[0].numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-10, atol=1e-12)
    keep = rng.random((N, N)) < 0.3
    keep[:, 0] = True
    ours_m = softmax_attention(q, k, v, 1 / math.sqrt(d), keep)
    ref_m = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=torch.from_numpy(keep)[None])[0].numpy()
    np.testing.assert_allclose(ours_m, ref_m, rtol=1e-10, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((9, 4)) * 5
    v = rng.standard_normal((11, 3))
    keep = rng.random((9, 11)) < 0.4
    keep[:, 3] = True
    o = softmax_attention(q, np.zeros((11, 4)), v, 0.5, keep)
    for i in range(9):
        np.testing.assert_allclose(o[i], v[keep[i]].mean(axis=0), rtol=1e-13, atol=1e-14)
    const = np.tile(np.array([[1.5, -2.0, 0.25]]), (11, 1))
    o = softmax_attention(q, rng.standard_normal((11, 4)), const, 0.5, keep)
    np.testing.assert_allclose(o, np.tile(const[:1], (9, 1)), rtol=1e-13)
    one = np.zeros((9, 11), dtype=bool)
    one[np.arange(9), np.arange(9)] = True
    o = softmax_attention(q, rng.standard_normal((11, 4)), v, 0.5, one)
    np.testing.assert_allclose(o, v[:9], rtol=1e-15)


def test_large_logits_are_stable():
    rng = np.random.default_rng(2)
    q, k, v = rng.standard_normal((4, 8)) * 100, rng.standard_normal((6, 8)) * 100, rng.standard_normal((6, 2))
    o = softmax_attention(q, k, v, 1.0)
    assert np.all(np.isfinite(o))
    s = q @ k.T
    np.testing.assert_allclose(o, v[s.argmax(axis=1)], rtol=1e-9, atol=1e-9)


def test_permutation_equivariance():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((13, 5)), rng.standard_normal((17, 5)), rng.standard_normal((17, 4))
    pk = rng.permutation(17)
    pq = rng.permutation(13)
    o = softmax_attention(q, k, v, 0.3)
    np.testing.assert_allclose(softmax_attention(q, k[pk], v[pk], 0.3), o, rtol=1e-12)
    np.testing.assert_allclose(softmax_attention(q[pq], k, v, 0.3), o[pq], rtol=1e-12)


def test_block_sparse_all_ones_is_dense_with_ragged_tail():
    rng = np.random.default_rng(4)
    N, d, bq, bk = 75, 16, 16, 8          # 5 q-blocks (tail 11), 10 k-blocks (tail 3)
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    bm = np.ones((5, 10), dtype=np.uint8)
    np.testing.assert_allclose(block_sparse_attention_full(q, k, v, bm, bq, bk), dense_attention(q, k, v),
                               rtol=1e-12, atol=1e-13)


def test_block_sparse_kept_set_through_k_zero():
    """K = 0 makes each row's output the mean of V over exactly the keys of its
    q-block's kept tiles, so the output pins the kept set (tail keys >= N
    excluded, kept tiles taken whole)."""
    rng = np.random.default_rng(5)
    N, d, bq, bk = 45, 8, 8, 16
    nqb, nkb = 6, 3
    q, v = rng.standard_normal((N, d)), rng.standard_normal((N, 5))
    bm = (rng.random((nqb, nkb)) < 0.5).astype(np.uint8)
    bm[:, 2] = 1
    bm[1] = 0
    out = block_sparse_attention(q, np.zeros((N, d)), v, bm, bq, bk)
    for qb in range(nqb):
        keys = [j for j in range(N) if bm[qb, j // bk]]
        expect = v[keys].mean(axis=0) if keys else np.zeros(5)
        np.testing.assert_allclose(out[qb], np.tile(expect, (out[qb].shape[0], 1)), rtol=1e-13, atol=1e-14)
    assert out[5].shape[0] == N - 5 * bq
