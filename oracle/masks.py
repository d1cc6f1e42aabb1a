"""Spatial and temporal token masks, block bitmaps and kept-block lists (oracle).

Sources: the SVG1 abstract (spatial heads: tokens of the query's own frame
dominate; temporal heads: tokens at the same place across frames dominate)
and the project write-up's install section (block-sparse attention over
per-block keep flags).

Token coordinates (readings): video tokens come first in frame-major order,
token (f, p) at t = f*S + p.  The T text tokens follow.  A text token belongs
to no frame and no position, so a text query keeps every key and every query
keeps every text key.

Spatial mask, window ks frames:
    a video query in frame f keeps the video keys of frames f-ks .. f+ks.
Temporal mask, widening wt tokens:
    position-major index r(f, p) = p*F + f lists the F frames of one position
    together.  A video query at position p keeps the video keys whose r lies
    in the own-position run [p*F, p*F + F - 1], widened by wt on each side.

Executing layout: spatial heads run in frame-major order (the identity).
Temporal heads run in position-major order, video row r(f, p), text rows
unchanged.  In that order each head's kept keys form a band.  This is the
reading of the abstract's hardware-efficient layout transformation.
"""

import numpy as np

SPATIAL, TEMPORAL = 0, 1


# ----------------------------------------------------------------------------
# token masks (original, frame-major coordinates)

def spatial_keep(i, j, F, S, ks):
    """Bool mask M_s[i, j] for broadcastable int arrays i (queries), j (keys)."""
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    video = F * S
    text_i = i >= video
    text_j = j >= video
    fi = i // S
    fj = j // S
    return text_i | text_j | (np.abs(fj - fi) <= ks)


def temporal_keep(i, j, F, S, wt):
    """Bool mask M_t[i, j] for broadcastable int arrays i (queries), j (keys)."""
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    video = F * S
    text_i = i >= video
    text_j = j >= video
    pi = i % S
    rj = (j % S) * F + j // S
    lo = pi * F - wt
    hi = pi * F + F - 1 + wt
    return text_i | text_j | ((rj >= lo) & (rj <= hi))


def token_keep(label, i, j, F, S, ks, wt):
    if label == SPATIAL:
        return spatial_keep(i, j, F, S, ks)
    return temporal_keep(i, j, F, S, wt)


# ----------------------------------------------------------------------------
# executing layout

def position_major_index(F, S, T):
    """e[t] = executing (position-major) index of original token t."""
    t = np.arange(F * S + T, dtype=np.int64)
    e = t.copy()
    v = t[:F * S]
    e[:F * S] = (v % S) * F + v // S
    return e


def executing_to_original(label, F, S, T):
    """inv[x] = original token at executing index x for a head of this label."""
    N = F * S + T
    if label == SPATIAL:
        return np.arange(N, dtype=np.int64)
    e = position_major_index(F, S, T)
    inv = np.empty(N, dtype=np.int64)
    inv[e] = np.arange(N, dtype=np.int64)
    return inv


# ----------------------------------------------------------------------------
# block bitmaps

def block_bitmap(label, F, S, T, ks, wt, bq, bk, qblocks=None):
    """uint8 bitmap B[qb, kb]: 1 iff some token pair (i, j) in the tile is kept.

    The tile's rows are queries qb*bq .. qb*bq+bq-1 and its columns keys
    kb*bk .. kb*bk+bk-1, in the executing layout of this label, clipped to N.
    This is the any-overlap cover of the token mask.  It is evaluated element
    by element over the tile's token pairs.  ``qblocks`` restricts the output
    to those rows of B (in that order).
    """
    N = F * S + T
    nqb, nkb = -(-N // bq), -(-N // bk)
    inv = executing_to_original(label, F, S, T)
    qblocks = range(nqb) if qblocks is None else qblocks
    qblocks = list(qblocks)
    out = np.zeros((len(qblocks), nkb), dtype=np.uint8)
    cols_orig = inv                                  # executing col -> original key
    for r, qb in enumerate(qblocks):
        rows_orig = inv[qb * bq:min(N, (qb + 1) * bq)]
        keep = token_keep(label, rows_orig[:, None], cols_orig[None, :], F, S, ks, wt)
        padded = np.zeros((rows_orig.size, nkb * bk), dtype=bool)
        padded[:, :N] = keep
        out[r] = padded.reshape(rows_orig.size, nkb, bk).any(axis=(0, 2))
    return out


def row_kept_ranges(label, F, S, T, ks, wt):
    """Per executing row x: the kept video keys as one executing range [lo, hi).

    Text keys [F*S, N) are always kept as well.  A text row keeps everything
    (lo = 0, hi = N).

    Spatial: the frames f-ks .. f+ks, clipped, are contiguous in frame-major
    order: [max(0, f-ks)*S, min(F, f+ks+1)*S).
    Temporal: the widened own-position run, clipped to the video tokens, is
    contiguous in position-major order: [max(0, pF-wt), min(FS, pF+F+wt)).
    These are the two masks above restated in the executing layout.
    """
    N, video = F * S + T, F * S
    x = np.arange(N, dtype=np.int64)
    lo = np.zeros(N, dtype=np.int64)
    hi = np.full(N, N, dtype=np.int64)
    v = x < video
    if label == SPATIAL:
        f = x[v] // S
        lo[v] = np.maximum(0, f - ks) * S
        hi[v] = np.minimum(F, f + ks + 1) * S
    else:
        p = x[v] // F
        lo[v] = np.maximum(0, p * F - wt)
        hi[v] = np.minimum(video, p * F + F + wt)
    return lo, hi


def block_bitmap_ranges(label, F, S, T, ks, wt, bq, bk):
    """The same bitmap as block_bitmap, from row_kept_ranges (fast at large N).

    Row x keeps key blocks lo//bk .. (hi-1)//bk, plus every block that holds
    a text key.  A q-block's row of B is the union over its rows.
    """
    N, video = F * S + T, F * S
    nqb, nkb = -(-N // bq), -(-N // bk)
    lo, hi = row_kept_ranges(label, F, S, T, ks, wt)
    kb = np.arange(nkb, dtype=np.int64)
    text_blocks = (kb + 1) * bk > video if T > 0 else np.zeros(nkb, dtype=bool)
    out = np.zeros((nqb, nkb), dtype=np.uint8)
    for qb in range(nqb):
        r0, r1 = qb * bq, min(N, (qb + 1) * bq)
        blo = lo[r0:r1, None] // bk
        bhi = (hi[r0:r1, None] - 1) // bk
        hit = ((kb[None, :] >= blo) & (kb[None, :] <= bhi)).any(axis=0)
        out[qb] = hit | text_blocks
    return out


# ----------------------------------------------------------------------------
# kept-block lists

def compact(bitmap):
    """CSR of a 2-D (or [H][nQB][nKB] flattened to rows) bitmap.

    row_ptr[r+1] - row_ptr[r] = kept blocks of row r.  kv_idx lists each
    row's kept column blocks in ascending order.
    """
    b = np.asarray(bitmap).reshape(-1, np.asarray(bitmap).shape[-1]) != 0
    counts = b.sum(axis=1)
    row_ptr = np.zeros(b.shape[0] + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    kv_idx = np.nonzero(b)[1]          # row-major order: ascending per row
    return row_ptr.astype(np.int32), kv_idx.astype(np.int32)


def valid_pairs(bitmap, N, bq, bk):
    """Number of (query, key) pairs with both < N inside the kept tiles."""
    nqb, nkb = bitmap.shape
    rows = np.minimum(N, (np.arange(nqb) + 1) * bq) - np.arange(nqb) * bq
    cols = np.minimum(N, (np.arange(nkb) + 1) * bk) - np.arange(nkb) * bk
    return int((bitmap.astype(np.int64) * rows[:, None] * cols[None, :]).sum())
