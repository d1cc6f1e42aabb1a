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
"""

import numpy as np

from .attention import block_sparse_attention, default_scale

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * E4M3_SUBNORMAL_STEP, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


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
    codes = np.zeros(x32.shape, dtype=np.uint8)
    scales = np.zeros(ng, dtype=np.float32)
    for g in range(ng):
        blk = x32[g * group_rows:(g + 1) * group_rows]
        a = np.float32(np.abs(blk).max()) if blk.size else np.float32(0)
        if a == 0:
            continue
        inv = np.float32(E4M3_MAX) / a                    # fp32 division, rounded once
        y = (blk * inv).astype(np.float32)                # fp32 product, rounded once
        codes[g * group_rows:(g + 1) * group_rows] = e4m3_round(y)
        scales[g] = a / np.float32(E4M3_MAX)
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
