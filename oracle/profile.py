"""Online profiling of heads (oracle).

Sources:
* the SVG1 abstract: an online profiling strategy predicts whether each head
  is spatial or temporal.
* the project write-up, section "Three generations of the same idea": the
  profiling identifies the pattern dynamically, on every call.

The pages do not give the test itself.  Reading: for a small sample of query
rows, compute three outputs on those rows:
* the full attention output;
* the output with the spatial token mask;
* the output with the temporal token mask.
Each masked softmax is normalised over its own kept keys, with its own
maximum.  Then take the mean squared error of each masked output against the
full one, over the n_s * d values.  The head is spatial if MSE_s <= MSE_t
(ties go to spatial), else temporal.  The masks are the token masks of
``oracle.masks`` in original (frame-major) coordinates, not block-expanded.
"""

import numpy as np

from .attention import softmax_attention, default_scale
from .masks import spatial_keep, temporal_keep


def profile_head(q, k, v, F, S, T, sample_idx, ks, wt, scale=None, chunk=128):
    """One head.  q, k, v [N, d] float64 in original order.

    Returns (label, mse_spatial, mse_temporal).
    """
    N, d = q.shape
    scale = default_scale(d) if scale is None else scale
    sample_idx = np.asarray(sample_idx, dtype=np.int64)
    keys = np.arange(N, dtype=np.int64)
    se_s = 0.0
    se_t = 0.0
    for a in range(0, sample_idx.size, chunk):
        rows = sample_idx[a:a + chunk]
        o_full = softmax_attention(q[rows], k, v, scale)
        keep_s = spatial_keep(rows[:, None], keys[None, :], F, S, ks)
        o_s = softmax_attention(q[rows], k, v, scale, keep_s)
        keep_t = temporal_keep(rows[:, None], keys[None, :], F, S, wt)
        o_t = softmax_attention(q[rows], k, v, scale, keep_t)
        se_s += float(((o_s - o_full) ** 2).sum())
        se_t += float(((o_t - o_full) ** 2).sum())
    n = sample_idx.size * d
    mse_s, mse_t = se_s / n, se_t / n
    label = 0 if mse_s <= mse_t else 1
    return label, mse_s, mse_t


def profile_heads(q, k, v, F, S, T, sample_idx, ks, wt, scale=None, heads=None):
    """All heads.  q, k, v [H][N][d] float64.  Returns labels int32[H], mse [H][2]."""
    H = q.shape[0]
    heads = range(H) if heads is None else heads
    labels, mse = [], []
    for h in heads:
        lab, ms, mt = profile_head(q[h], k[h], v[h], F, S, T, sample_idx, ks, wt, scale)
        labels.append(lab)
        mse.append((ms, mt))
    return np.array(labels, dtype=np.int32), np.array(mse, dtype=np.float64)
