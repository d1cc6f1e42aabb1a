"""FP8 attention (oracle; TEST INFRASTRUCTURE, float64 apart from the fp32
quantization arithmetic it defines).

Source: the Sparse-VideoGen write-up, section "Publication record and the
road ahead": FP8 attention is an unchecked item of the project's plan.  The
pages give no FP8 method, so its quantization is this library's own
definition, stated here and checked against itself nowhere else:

* Format: OCP FP8 E4M3 ("e4m3fn"): sign, 4 exponent bits (bias 7), 3
  fraction bits; normals (1 + m/8) * 2^(e-7) for e = 1..15 except the code
  0x7F / 0xFF (NaN), so the largest finite value is 448 = 1.75 * 2^8;
  subnormals (m/8) * 2^-6.  No infinities.
* Rounding: to the nearest representable value, ties to the even code
  (fraction LSB 0).  Inputs never exceed 448 * (1 + 2^-23) in magnitude, so
  overflow does not arise.
* Scales: Q gets one scale per token (row), K one per block of 64 keys of
  the executing layout (the attention's key tile).  For a group of values x
  (bf16, exact in fp32) with largest magnitude a (fp32):
      inv   = 448 / a          (fp32, correctly rounded)
      code  = round_e4m3(fp32(x * inv))
      scale = a / 448          (fp32, correctly rounded)
  The value a code stands for is decode(code) * scale.  A group of zeros
  (a = 0) gets code 0 and scale 0.
* Attention: the block-sparse attention of the bf16 path (same masks, same
  lists, same softmax), with Q and K replaced by their dequantized values
  Q~ = decode(Qcode) * scale_q[row], K~ = decode(Kcode) * scale_k[block],
  and V, P.V and O as in the bf16 path.

Everything after the quantization runs in float64, so this oracle says what
the FP8 path should return up to the rounding of its fp32 accumulation and
of the bf16 probabilities and output.

The FP8 P.V mode (also this library's definition) quantizes the other
product as well:
* V gets one scale per channel (column d) over all N tokens of the head,
  coded as above: v_code = round_e4m3(fp32(v * (448 / a_d))), scale
  a_d / 448.
* P: a query row walks its q-block's kept tiles in ascending order with a
  lazy reference m.  Logits are taken in exp2 units, y = log2(e) * scale *
  (q~ . k~).  A tile whose largest y exceeds m by more than 8 (or the first
  kept tile) moves m to that maximum, and the sums so far are multiplied by
  2^(m_old - m_new).  Each key's probability p = 2^(y - m) (at most 2^8) is
  coded as round_e4m3(fp32(p)) with no scale; the sums take the decoded
  codes p8.
* O = (sum_j p8_j * decode(v_code_j)) / (sum_j p8_j), times the channel
  scales.
Because each p8 is a rounding of an exponential, a logit error of a few
fp32 units can move a p that sits next to a rounding boundary to the
neighbouring code.  fp8_pv_block_sparse_attention therefore also returns,
for each row, a bound on what such moves can change: the codes whose p lies
within a relative eps of a boundary are "undecided" and each may take
either neighbour.
"""

import numpy as np

from .attention import block_sparse_attention, default_scale

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9


def _e4m3_values() -> np.ndarray:
    """The value of each of the 256 codes (NaN for 0x7F / 0xFF)."""
    c = np.arange(256, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * E4M3_SUBNORMAL_STEP, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


_E4M3_VALUES = _e4m3_values()


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF), from the table
    of all 256 codes."""
    return _E4M3_VALUES[np.asarray(codes).astype(np.uint8)]


def e4m3_round(y) -> np.ndarray:
    """Nearest E4M3 code of each fp32 value, ties to the even code.

    Written from the format: for |y| >= 2^-6 take e = floor(log2|y|), the
    fraction f = |y| / 2^e - 1 in [0, 1), and m = round-half-even(8 f); m = 8
    carries into the exponent.  Below 2^-6 the value is k * 2^-9 with
    k = round-half-even(|y| * 2^9) (k = 8 is the smallest normal).  Every
    step is exact in float64 for fp32 inputs (power-of-two scalings), so
    numpy's rint decides the ties exactly.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    a = np.abs(y)
    sign = (np.signbit(y)).astype(np.int64) << 7
    out = np.zeros(a.shape, dtype=np.int64)
    sub = a < E4M3_MIN_NORMAL
    k = np.rint(a[sub] / E4M3_SUBNORMAL_STEP).astype(np.int64)       # 0..8
    out[sub] = k                     # k = 8 is code 0x08, the smallest normal
    nrm = ~sub
    an = a[nrm]
    _, ex = np.frexp(an)             # an = f * 2^ex with f in [0.5, 1)
    e = ex - 1                       # an in [2^e, 2^(e+1))
    m = np.rint((an / np.ldexp(1.0, e) - 1.0) * 8.0).astype(np.int64)
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    if np.any(e > 8) or np.any((e == 8) & (m > 6)):
        raise ValueError("value above the E4M3 range (448)")
    out[nrm] = ((e + 7) << 3) | m
    return (out | sign).astype(np.uint8)


def quantize_groups(x, group_rows: int):
    """Quantize x [N][d] (values exact in fp32) in groups of group_rows
    consecutive rows (the last group may be short): returns the codes uint8
    [N][d] and the fp32 scale of each group."""
    x32 = np.asarray(x, dtype=np.float32)
    N = x32.shape[0]
    ng = -(-N // group_rows)
    if N == 0 or x32.size == 0:
        return np.zeros(x32.shape, dtype=np.uint8), np.zeros(ng, dtype=np.float32)
    # every group at once: rows padded with zeros to whole groups (a zero
    # never raises a group's maximum and is not returned)
    blk = np.zeros((ng * group_rows,) + x32.shape[1:], dtype=np.float32)
    blk[:N] = x32
    blk = blk.reshape(ng, group_rows, -1)
    a = np.abs(blk).max(axis=(1, 2))                      # fp32 group maxima
    live = a > 0
    inv = np.zeros(ng, dtype=np.float32)
    inv[live] = np.float32(E4M3_MAX) / a[live]            # fp32 division, rounded once
    y = (blk * inv[:, None, None]).astype(np.float32)     # fp32 products, rounded once
    codes = e4m3_round(y).reshape(ng * group_rows, -1)[:N].reshape(x32.shape)
    scales = np.zeros(ng, dtype=np.float32)
    scales[live] = a[live] / np.float32(E4M3_MAX)
    return codes, scales


def quantize_rows(x):
    """Per-token (row) scales: the Q side."""
    return quantize_groups(x, 1)


def quantize_key_blocks(x, bk: int = 64):
    """Per-block scales over blocks of bk rows: the K side, in the executing
    layout."""
    return quantize_groups(x, bk)


def dequantize(codes, scales, group_rows: int):
    """decode(code) * scale of its group, float64 [N][d]."""
    s = np.repeat(np.asarray(scales, dtype=np.float64), group_rows)[:codes.shape[0]]
    return e4m3_decode(codes) * s[:, None]


def fp8_block_sparse_attention(q, k, v, bitmap, bq, bk, scale=None, qblocks=None):
    """Block-sparse attention of one head with FP8 Q and K (definition
    above).  q, k, v: [N][d] values exact in fp32 (bf16 inputs), all in the
    executing layout.  Returns {qb: O rows} as block_sparse_attention."""
    qc, qs = quantize_rows(q)
    kc, ks = quantize_key_blocks(k, bk)
    qd = dequantize(qc, qs, 1)
    kd = dequantize(kc, ks, bk)
    scale = default_scale(q.shape[1]) if scale is None else scale
    return block_sparse_attention(qd, kd, np.asarray(v, dtype=np.float64), bitmap, bq, bk, scale, qblocks)


LAZY_LOG2 = 8.0          # the reference moves when a tile's maximum exceeds it by more than this (exp2 units)


def quantize_channels(x):
    """Per-channel scales: one per column of x [N][d] over all N rows (the V
    side of the FP8 P.V mode).  Returns the codes [N][d] and the fp32 scale
    of each column."""
    codes_t, scales = quantize_groups(np.asarray(x, dtype=np.float32).T, 1)
    return np.ascontiguousarray(codes_t.T), scales


def _lazy_references(tile_max):
    """The lazy reference of each (row, kept tile), walking the tiles in
    order: [R][T] float64 (tile_max: [R][T], the tiles' largest logits in
    exp2 units).  Also returns, per row, whether some move decision lies
    within 1e-3 of the threshold (then fp32 rounding could decide it the
    other way)."""
    R, T = tile_max.shape
    ref = np.empty((R, T))
    m = np.full(R, -np.inf)
    near = np.zeros(R, dtype=bool)
    for t in range(T):
        mt = tile_max[:, t]
        first = np.isneginf(m)
        with np.errstate(invalid="ignore"):
            gap = mt - m
        near |= ~first & (np.abs(gap - LAZY_LOG2) < 1e-3)
        m = np.where(first | (gap > LAZY_LOG2), mt, m)
        ref[:, t] = m
    return ref, near


def fp8_pv_block_sparse_attention(q, k, v, bitmap, bq, bk, scale=None, qblocks=None, eps=1e-4):
    """Block-sparse attention of one head in the FP8 P.V mode (definition
    above): FP8 Q and K as in fp8_block_sparse_attention, V coded per
    channel, P coded after the lazy reference.  q, k, v: [N][d] values
    exact in fp32, in the executing layout.

    Returns {qb: (O rows, bound rows, ambiguous rows)}: O in float64; bound
    [R], the largest change of any O value that moving the undecided codes
    (p within a relative eps of a rounding boundary) could make, to first
    order; ambiguous [R] bool, rows with a reference move within 1e-3 of the
    threshold."""
    q = np.asarray(q, dtype=np.float32)
    N, d = q.shape
    kc, ks = quantize_key_blocks(k, bk)
    kd = dequantize(kc, ks, bk)
    vc, vs = quantize_channels(v)
    v8 = e4m3_decode(vc)                                  # unscaled code values
    vmax = np.abs(v8 * vs.astype(np.float64)[None, :]).max(axis=1) if N else np.zeros(0)
    scale = default_scale(d) if scale is None else scale
    c = scale * np.log2(np.e)
    nqb = bitmap.shape[0]
    qblocks = range(nqb) if qblocks is None else qblocks
    out = {}
    for qb in qblocks:
        r0, r1 = qb * bq, min(N, (qb + 1) * bq)
        R = r1 - r0
        kept = np.flatnonzero(bitmap[qb])
        if kept.size == 0:
            out[qb] = (np.zeros((R, d)), np.zeros(R), np.zeros(R, dtype=bool))
            continue
        cols = [np.arange(kb * bk, min(N, (kb + 1) * bk)) for kb in kept]
        tile_of = np.concatenate([np.full(cc.size, t) for t, cc in enumerate(cols)])
        cols = np.concatenate(cols)
        qc, qs = quantize_rows(q[r0:r1])                  # per-row scales: the block's rows alone
        y = (dequantize(qc, qs, 1) @ kd[cols].T) * c      # [R][keys], exp2 units
        starts = np.concatenate([[0], np.flatnonzero(np.diff(tile_of)) + 1])   # each tile's first column
        tmax = np.maximum.reduceat(y, starts, axis=1)                          # [R][T] tile maxima
        ref, near = _lazy_references(tmax)
        mfin = ref[:, -1]
        p = np.exp2(y - ref[:, tile_of])                  # each key against its tile's reference
        code = e4m3_round(p.astype(np.float32)).astype(np.int64)     # 0 .. 0x78 (p <= 2^8)
        p8 = e4m3_decode(code)
        # undecided: p within a relative eps of the midpoint to a neighbouring
        # code (positive codes are ordered like their values)
        nxt = e4m3_decode(np.minimum(code + 1, 0x7E))
        prv = e4m3_decode(np.maximum(code - 1, 0))
        und_up = p * (1 + eps) >= (p8 + nxt) / 2
        und_lo = (code > 0) & (p * (1 - eps) <= (p8 + prv) / 2)
        step = np.maximum(np.where(und_up, nxt - p8, 0.0), np.where(und_lo, p8 - prv, 0.0))
        w = np.exp2(ref[:, tile_of] - mfin[:, None])      # the rescales by later moves
        pw = p8 * w
        l = pw.sum(axis=1)
        o = (pw @ v8[cols]) * vs.astype(np.float64)[None, :]
        with np.errstate(invalid="ignore", divide="ignore"):
            O = np.where(l[:, None] > 0, o / l[:, None], 0.0)
            sw = step * w
            bound = np.where(l > 0, (sw @ vmax[cols] + sw.sum(axis=1) * np.abs(O).max(axis=1)) / l, 0.0)
        out[qb] = (O, bound, near)
    return out
