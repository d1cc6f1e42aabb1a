"""Softmax attention, dense, masked and block-sparse (oracle; float64).

The SVG1 abstract says the cost is in 3D full attention.  That attention is
plain scaled dot-product softmax attention over every token pair of the video
and text sequence.  Reading: scale 1/sqrt(d), no causal mask, no bias, no
dropout.  Each row is an independent softmax.  So the functions below may
evaluate a subset of rows, or split rows into groups, without changing any
value.
"""

import math
import numpy as np


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def softmax_attention(q, k, v, scale, keep=None):
    """O[i] = sum_j softmax_j(scale * q_i . k_j) v_j, over the kept j only.

    q: [m, d], k and v: [n, d] (float64).
    keep: None (all keys) or a bool [m, n] token mask.

    The softmax of a masked row is taken over the kept keys alone, with that
    row's own maximum subtracted.  A row with no kept key gives 0.  That is
    the convention for an empty softmax.
    """
    s = (q @ k.T) * scale
    if keep is not None:
        s = np.where(keep, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    has = np.isfinite(m)
    m = np.where(has, m, 0.0)
    p = np.exp(s - m)                    # exp(-inf) = 0 for masked keys
    l = p.sum(axis=1, keepdims=True)
    o = (p @ v) / np.where(l > 0.0, l, 1.0)
    return np.where(has, o, 0.0)


def dense_attention(q, k, v, scale=None, rows=None, chunk=256):
    """Full attention for one head: q, k, v [N, d] float64 -> O [len(rows), d].

    This is the layer the sparse path replaces, and the baseline its speedup
    is measured against.
    """
    scale = default_scale(q.shape[1]) if scale is None else scale
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    out = np.empty((rows.size, v.shape[1]))
    for a in range(0, rows.size, chunk):
        r = rows[a:a + chunk]
        out[a:a + chunk] = softmax_attention(q[r], k, v, scale)
    return out


def block_sparse_attention(q, k, v, bitmap, bq, bk, scale=None, qblocks=None):
    """Attention over the kept tiles of a block bitmap, for one head.

    Computed in the layout where the pattern is banded (the executing
    layout).  This is the block-sparse attention with per-block keep flags
    that the project write-up's install section names.

    q, k, v: [N, d] float64 in the executing layout.
    bitmap: uint8 [nQB, nKB].  Tile (qb, kb) is kept when nonzero.

    Query row i of block qb attends exactly the keys j < N of every kept
    tile (qb, kb).  A kept tile is computed whole: no mask inside a tile.
    Rows >= N and keys >= N do not exist.

    Returns {qb: O rows of that block}.  The keys kept for one q-block are
    the same for all its rows, so a q-block is one softmax_attention call on
    those columns.
    """
    N = q.shape[0]
    scale = default_scale(q.shape[1]) if scale is None else scale
    nqb = bitmap.shape[0]
    qblocks = range(nqb) if qblocks is None else qblocks
    out = {}
    for qb in qblocks:
        r0, r1 = qb * bq, min(N, (qb + 1) * bq)
        kept = np.flatnonzero(bitmap[qb])
        cols = [np.arange(kb * bk, min(N, (kb + 1) * bk)) for kb in kept]
        cols = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
        if cols.size == 0:
            out[qb] = np.zeros((r1 - r0, v.shape[1]))
        else:
            out[qb] = softmax_attention(q[r0:r1], k[cols], v[cols], scale)
    return out


def block_sparse_attention_full(q, k, v, bitmap, bq, bk, scale=None):
    """block_sparse_attention for every q-block, assembled into [N, d]."""
    parts = block_sparse_attention(q, k, v, bitmap, bq, bk, scale)
    return np.concatenate([parts[qb] for qb in range(bitmap.shape[0])], axis=0)
