"""Frame-major <-> position-major layout permutation (oracle).

Source: the SVG1 abstract's tensor layout transformation.  A temporal head
attends to the same place across frames.  Those keys sit S tokens apart in
frame-major order.  Listing each position's F frames together makes them
contiguous.

Reading: only temporal heads (label 1) are permuted.  Spatial heads are
already banded in frame-major order and are copied.  Text rows stay in place.
"""

import numpy as np

from .masks import position_major_index, TEMPORAL


def permute(x, F, S, T, labels):
    """Y[h, p*F + f] = X[h, f*S + p] for temporal heads.  All else is copied.

    x: [H][N][d] (any dtype).
    """
    e = position_major_index(F, S, T)
    y = np.array(x, copy=True)
    for h, lab in enumerate(labels):
        if lab == TEMPORAL:
            y[h, e] = x[h]
    return y


def unpermute(y, F, S, T, labels):
    """The inverse of permute: X[h, f*S + p] = Y[h, p*F + f] for temporal heads."""
    e = position_major_index(F, S, T)
    x = np.array(y, copy=True)
    for h, lab in enumerate(labels):
        if lab == TEMPORAL:
            x[h] = y[h, e]
    return x


def key_tiled_transpose(x, bk=64):
    """The library's key-tiled transposed storage of V (a storage format of
    this library, not of the pages): out[h, kb, c, j] = x[h, kb*bk + j, c] for
    kb*bk + j < N, else 0.  Shape [H][ceil(N/bk)][d][bk].

    x: [H][N][d] (any dtype; padding uses that dtype's zero).
    """
    H, N, d = x.shape
    nkb = -(-N // bk)
    out = np.zeros((H, nkb, d, bk), dtype=x.dtype)
    for kb in range(nkb):
        rows = x[:, kb * bk:min(N, (kb + 1) * bk), :]          # [H][<=bk][d]
        out[:, kb, :, :rows.shape[1]] = np.transpose(rows, (0, 2, 1))
    return out
