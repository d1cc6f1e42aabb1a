"""Pins of the FP8 (E4M3) oracle (CPU only).

Each check comes from outside the code it checks:
* hand-worked code values from the format's definition;
* brute force: the nearest of all 253 finite E4M3 values, found by
  enumeration, ties to the even code;
* round trips on every code, and inputs built to be exactly representable
  (then FP8 attention must equal the plain attention oracle);
* the half-ulp error bound of round-to-nearest.
"""

import numpy as np
import pytest

from oracle import fp8
from oracle.attention import block_sparse_attention, dense_attention


FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_known_codes():
    known = {0x00: 0.0, 0x38: 1.0, 0xB8: -1.0, 0x40: 2.0, 0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0,
             0x08: 2.0 ** -6, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x0F: 1.875 * 2.0 ** -6,
             0x77: 1.875 * 2.0 ** 7, 0x30: 0.5}
    for c, v in known.items():
        assert fp8.e4m3_decode(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(fp8.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert np.signbit(fp8.e4m3_decode(np.array([0x80], np.uint8))[0])


def test_round_hand_cases_and_ties():
    cases = [
        (1.0, 0x38), (-1.0, 0xB8), (448.0, 0x7E), (-448.0, 0xFE), (0.0, 0x00),
        (1.0625, 0x38),             # tie between 1.0 (m=0) and 1.125 (m=1): even m=0
        (1.1875, 0x3A),             # tie between 1.125 (m=1) and 1.25 (m=2): even m=2
        (1.0625 + 2 ** -20, 0x39),  # just above the tie
        (432.0, 0x7E),              # tie between 416 (m=5) and 448 (m=6): even m=6
        (2.0 ** -10, 0x00),         # half the subnormal step: tie between 0 and 2^-9, even 0
        (3 * 2.0 ** -10, 0x02),     # tie between k=1 and k=2: even k=2
        (5 * 2.0 ** -10, 0x02),     # tie between k=2 and k=3: even k=2
        (15 * 2.0 ** -10, 0x08),    # tie between k=7 (odd) and the smallest normal (k=8): 0x08
        (0.96875, 0x38),            # tie between 0.9375 (0x37, odd) and 1.0 (0x38): 1.0
    ]
    for y, want in cases:
        got = int(fp8.e4m3_round(np.array([y], np.float32))[0])
        assert got == want, (y, hex(got), hex(want))


def brute_nearest(y):
    vals = fp8.e4m3_decode(FINITE)
    out = []
    for x in np.asarray(y, dtype=np.float32).astype(np.float64):
        dist = np.abs(vals - x)
        best = dist.min()
        cands = [int(c) for c, dd in zip(FINITE, dist) if dd == best]
        # equal distance: the even code; +0 / -0 follow the input's sign
        cands = [c for c in cands if (c & 0x80) == (0x80 if np.signbit(x) else 0)] or cands
        even = [c for c in cands if c % 2 == 0]
        out.append((even or cands)[0])
    return np.array(out, dtype=np.uint8)


def test_round_is_the_nearest_value_by_enumeration():
    rng = np.random.default_rng(8)
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), size=4000))
    y = (mags * rng.choice([-1.0, 1.0], size=mags.size)).astype(np.float32)
    vals = np.sort(np.unique(np.abs(fp8.e4m3_decode(FINITE))))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)           # every tie point
    eps = np.nextafter(mids, np.float32(np.inf)) - mids
    y = np.concatenate([y, mids, -mids, mids + eps, mids - eps])
    y = y[np.abs(y) <= 448.0]
    np.testing.assert_array_equal(fp8.e4m3_round(y), brute_nearest(y))


def test_round_trip_every_code():
    vals = fp8.e4m3_decode(FINITE).astype(np.float32)
    np.testing.assert_array_equal(fp8.e4m3_round(vals), FINITE)


def test_quantize_exact_inputs_and_scales():
    """x = decode(c) / 64 with a group maximum of exactly 7: inv = 448 / 7 =
    64 and every x * 64 is a code value, so the codes come back unchanged
    and the scale is 7 / 448 = 1/64."""
    rng = np.random.default_rng(3)
    c = rng.choice(FINITE[np.abs(fp8.e4m3_decode(FINITE)) < 448], size=(10, 64))
    x = (fp8.e4m3_decode(c) / 64).astype(np.float32)
    x[:, 5] = 7.0                                     # each row's maximum
    codes, scales = fp8.quantize_rows(x)
    assert np.all(scales == np.float32(1 / 64))
    np.testing.assert_array_equal(fp8.dequantize(codes, scales, 1), x.astype(np.float64))
    kc, ks = fp8.quantize_key_blocks(x, 4)            # blocks of 4 rows: same maximum 7
    np.testing.assert_array_equal(fp8.dequantize(kc, ks, 4), x.astype(np.float64))
    zc, zs = fp8.quantize_rows(np.zeros((3, 8), np.float32))
    assert np.all(zc == 0) and np.all(zs == 0)


def test_quantize_error_within_half_ulp():
    """|x - decode(code) * scale| is at most half a unit in the last place of
    the code's binade (times the scale), plus the fp32 roundings of the
    product and of the scale."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((257, 128)) * np.exp2(rng.uniform(-6, 6, size=(257, 1)))).astype(np.float32)
    for codes, scales, g in (fp8.quantize_rows(x) + (1,), fp8.quantize_key_blocks(x, 64) + (64,)):
        dq = fp8.dequantize(codes, scales, g)
        s = np.repeat(scales.astype(np.float64), g)[:x.shape[0]][:, None]
        y = np.abs(x.astype(np.float64)) / s
        ulp = np.where(y < 2.0 ** -6, 2.0 ** -9, np.exp2(np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
        bound = s * (ulp / 2 + y * 2.0 ** -22)
        assert np.all(np.abs(dq - x) <= bound + 1e-30)


def test_fp8_attention_equals_plain_attention_on_exact_inputs():
    """Exactly representable Q and K: FP8 attention is the plain block-sparse
    attention, and with every tile kept it is dense attention."""
    rng = np.random.default_rng(11)
    N, d, bq, bk = 200, 64, 64, 64
    finite = FINITE[np.abs(fp8.e4m3_decode(FINITE)) <= 64]
    q = (fp8.e4m3_decode(rng.choice(finite, size=(N, d))) / 64).astype(np.float32)
    k = (fp8.e4m3_decode(rng.choice(finite, size=(N, d))) / 64).astype(np.float32)
    q[:, 0] = 7.0
    k[:, 1] = -7.0                                   # every row / block has maximum magnitude 7
    v = rng.standard_normal((N, d)).astype(np.float32)
    nqb = nkb = -(-N // 64)
    bm = (rng.random((nqb, nkb)) < 0.5).astype(np.uint8)
    bm[:, 0] = 1
    got = fp8.fp8_block_sparse_attention(q, k, v, bm, bq, bk)
    want = block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), bm, bq, bk)
    for qb in want:
        np.testing.assert_array_equal(got[qb], want[qb])
    full = fp8.fp8_block_sparse_attention(q, k, v, np.ones((nqb, nkb), np.uint8), bq, bk)
    dense = dense_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64))
    np.testing.assert_allclose(np.concatenate([full[i] for i in range(nqb)]), dense, rtol=0, atol=1e-13)


def test_round_top_of_the_range():
    """464 is the tie between 448 (m = 6, even) and the code above it, so it
    rounds to 448; anything above it is out of range."""
    assert int(fp8.e4m3_round(np.array([464.0], np.float32))[0]) == 0x7E
    with pytest.raises(ValueError):
        fp8.e4m3_round(np.array([470.0], np.float32))


# ---------------------------------------------------------------------------
# The FP8 P.V mode: per-channel V codes, probabilities coded after the lazy
# reference.

def test_quantize_channels_known_values():
    """Column maxima 448 (scale 1: the codes are the values), 7 (values
    decode(c) / 64: inv = 64 exactly) and 0 (codes 0, scale 0)."""
    rng = np.random.default_rng(21)
    finite = FINITE[np.abs(fp8.e4m3_decode(FINITE)) < 448]
    x = np.zeros((50, 3), np.float32)
    x[:, 0] = fp8.e4m3_decode(rng.choice(finite, size=50))
    x[7, 0] = -448.0
    x[:, 1] = fp8.e4m3_decode(rng.choice(finite, size=50)) / 64
    x[3, 1] = 7.0
    codes, scales = fp8.quantize_channels(x)
    assert codes.shape == x.shape
    np.testing.assert_array_equal(scales, np.array([1.0, 7.0 / 448.0, 0.0], np.float32))
    np.testing.assert_array_equal(fp8.e4m3_decode(codes[:, 0]), x[:, 0])
    np.testing.assert_array_equal(fp8.e4m3_decode(codes[:, 1]) * np.float64(scales[1]), x[:, 1])
    assert np.all(codes[:, 2] == 0)


def _exact_v(rng, N, d):
    """V whose every column has maximum magnitude 448 and only code values
    (channel scale 1: the codes stand for V exactly)."""
    finite = FINITE[np.abs(fp8.e4m3_decode(FINITE)) <= 64]
    v = fp8.e4m3_decode(rng.choice(finite, size=(N, d))).astype(np.float32)
    v[rng.integers(0, N), :] = 448.0
    return v


def test_fp8_pv_equal_logits_is_the_kept_keys_mean():
    """q = 0: every logit is 0, every p is 1 (a code value), so each row's
    output is the mean of V over its q-block's kept keys."""
    rng = np.random.default_rng(22)
    N, d, bq, bk = 150, 64, 64, 64
    q = np.zeros((N, d), np.float32)
    k = rng.standard_normal((N, d)).astype(np.float32)
    v = _exact_v(rng, N, d)
    bm = (rng.random((3, 3)) < 0.6).astype(np.uint8)
    bm[0] = 0
    bm[1, 2] = 1                                     # the short last block
    got = fp8.fp8_pv_block_sparse_attention(q, k, v, bm, bq, bk)
    for qb in range(3):
        O, bound, near = got[qb]
        kept = np.flatnonzero(bm[qb])
        if kept.size == 0:
            assert np.all(O == 0)
            continue
        cols = np.concatenate([np.arange(kb * bk, min(N, (kb + 1) * bk)) for kb in kept])
        want = v[cols].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(O, np.broadcast_to(want, O.shape), rtol=0, atol=1e-12)
        assert np.all(bound == 0) and not near.any()


def _integer_logit_inputs(rng, N, d, bk, lift_block):
    """Q and K exactly representable (row / block maxima 448 in dims that
    the dot products never use), with integer dot products in [-3, 3], plus
    +12 on every key of block lift_block (dim 2: q = 4, k = 3)."""
    q = np.zeros((N, d), np.float32)
    k = np.zeros((N, d), np.float32)
    q[:, 0] = 448.0                                  # q . k never meets dim 0 (k = 0 there)
    k[::bk, 1] = 448.0                               # each 64-row block's maximum; q = 0 in dim 1
    for x in (q, k):
        for r in range(N):
            dims = rng.choice(np.arange(3, d), size=3, replace=False)
            x[r, dims] = rng.choice([-1.0, 1.0], size=3)
    q[:, 2] = 4.0
    k[lift_block * bk:(lift_block + 1) * bk, 2] = 3.0
    return q, k


def test_fp8_pv_exact_powers_equal_plain_attention_with_a_move():
    """Logits that are integers in exp2 units (scale ln 2): every p is a
    power of two, a code value, so the FP8 P.V output is plain attention
    with the same V.  Rows whose q-block keeps block 3 see its logits 12
    above the others: the reference moves there (by more than 8) and the
    earlier sums, coded against the old reference, are rescaled exactly
    (those q-blocks keep no later block, whose p would fall below the
    smallest code)."""
    rng = np.random.default_rng(23)
    N, d, bq, bk = 5 * 64 + 17, 64, 64, 64
    q, k = _integer_logit_inputs(rng, N, d, bk, lift_block=3)
    v = _exact_v(rng, N, d)
    nb = -(-N // 64)
    bm = (rng.random((nb, nb)) < 0.6).astype(np.uint8)
    bm[:, 0] = 1
    bm[:3, 3] = 1
    bm[:3, 4:] = 0                                   # nothing after the lift (its p would leave the code range)
    bm[3:, 3] = 0
    bm[4, 5] = 1
    ln2 = float(np.log(2.0))
    got = fp8.fp8_pv_block_sparse_attention(q, k, v, bm, bq, bk, scale=ln2)
    want = block_sparse_attention(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64), bm, bq, bk,
                                  scale=ln2)
    for qb in range(nb):
        O, bound, near = got[qb]
        assert not near.any()
        np.testing.assert_allclose(O, want[qb], rtol=0, atol=1e-12)


def test_fp8_pv_probability_rounding_hand_case():
    """Two keys with logits 0 and 1/2 (exp2 units): p = 2^-1/2 = 0.7071 is
    coded as 0.6875 (1.375 * 2^-1; the neighbours are 0.6875 and 0.75), the
    largest as 1.  V = [[448, 1], [1, 448]] is coded exactly, so
    O = (0.6875 * v0 + v1) / 1.6875."""
    q = np.array([[448.0, 1.0], [448.0, 1.0]], np.float32)
    k = np.array([[0.0, 0.0], [0.0, 1.0]], np.float32)
    v = np.array([[448.0, 1.0], [1.0, 448.0]], np.float32)
    scale = 0.5 / float(np.log2(np.e))
    O, bound, near = fp8.fp8_pv_block_sparse_attention(q, k, v, np.ones((1, 1), np.uint8), 64, 64, scale=scale)[0]
    want = (0.6875 * np.array([448.0, 1.0]) + np.array([1.0, 448.0])) / 1.6875
    np.testing.assert_allclose(O, np.stack([want, want]), rtol=1e-14, atol=0)
    assert np.all(bound == 0) and not near.any()


def test_fp8_pv_bound_covers_logit_perturbations():
    """Logits moved by a relative 1e-6 (a scale change) can only move
    undecided codes, and the output changes within the returned bound."""
    rng = np.random.default_rng(24)
    N, d, bq, bk = 3 * 64 + 9, 64, 64, 64
    q = (rng.standard_normal((N, d)) * 1.5).astype(np.float32)
    k = (rng.standard_normal((N, d)) * 1.5).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    nb = -(-N // 64)
    bm = np.ones((nb, nb), np.uint8)
    base = fp8.fp8_pv_block_sparse_attention(q, k, v, bm, bq, bk)
    assert sum(float(b.sum()) for _, b, _ in base.values()) > 0      # some codes are undecided
    for delta in (1e-6, -1e-6, 3e-7):
        s = (1 + delta) / np.sqrt(d)
        moved = fp8.fp8_pv_block_sparse_attention(q, k, v, bm, bq, bk, scale=s)
        for qb in range(nb):
            O0, bound, _ = base[qb]
            O1 = moved[qb][0]
            # the logits' own change moves every p by a relative ~|y| * delta * ln 2
            assert np.all(np.abs(O1 - O0).max(axis=1) <= bound * 1.01 + 1e-4 * np.abs(O0).max(axis=1))
