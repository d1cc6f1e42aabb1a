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
