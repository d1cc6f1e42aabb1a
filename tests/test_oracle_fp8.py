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
