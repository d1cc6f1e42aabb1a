"""Pins of the oracle's layout functions against brute-force definitions.

The frame-major -> position-major permutation (the SVG1 abstract's layout
transformation) and the key-tiled transposed storage of V are checked element
by element with plain loops on small ragged shapes, where an index mix-up
(f and p swapped, a transposed tile, a shifted pad) changes some element.
"""

import numpy as np

from oracle import layout


def test_permute_matches_loop_definition():
    F, S, T, d = 3, 5, 2, 4
    N = F * S + T
    x = np.arange(2 * N * d).reshape(2, N, d)
    y = layout.permute(x, F, S, T, [0, 1])
    np.testing.assert_array_equal(y[0], x[0])          # spatial head copied
    for f in range(F):
        for p in range(S):
            np.testing.assert_array_equal(y[1, p * F + f], x[1, f * S + p])
    np.testing.assert_array_equal(y[1, F * S:], x[1, F * S:])   # text rows in place
    np.testing.assert_array_equal(layout.unpermute(y, F, S, T, [0, 1]), x)


def test_key_tiled_transpose_matches_loop_definition():
    H, N, d, bk = 2, 75, 3, 16
    x = np.arange(1, H * N * d + 1, dtype=np.int64).reshape(H, N, d)
    t = layout.key_tiled_transpose(x, bk)
    nkb = -(-N // bk)
    assert t.shape == (H, nkb, d, bk)
    for h in range(H):
        for kb in range(nkb):
            for c in range(d):
                for j in range(bk):
                    key = kb * bk + j
                    expect = x[h, key, c] if key < N else 0
                    assert t[h, kb, c, j] == expect
    # every input element appears exactly once, and the pad is zero
    assert np.count_nonzero(t) == x.size
    assert t.sum() == x.sum()


def test_key_tiled_transpose_exact_multiple_has_no_pad():
    x = np.random.default_rng(0).standard_normal((1, 128, 8))
    t = layout.key_tiled_transpose(x, 64)
    np.testing.assert_array_equal(t.transpose(0, 1, 3, 2).reshape(1, 128, 8), x)
