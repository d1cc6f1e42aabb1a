"""SVG2-style semantic permutation path (oracle).

Sources:
* the project write-up, section "Three generations of the same idea".  SVG2
  targets inaccurate token identification and wasted compute.  It adds
  semantic-aware sparse attention with an efficient token permutation, a
  dynamic attention kernel and a flash k-means kernel.
* its install section: block-sparse attention with varied block sizes; a
  bundled batched k-means is used by default.
* HyperVAttention ("Efficient Sparse Attention with Spatio-Temporal
  Clustering for Video Diffusion"), sections Problem and Surprising findings.
  Clusters give irregular blocks, and the tiled kernel's CTA density
  differs from the pattern's own density.

The pages do not spell out the selection rule.  Readings:
* Q and K are clustered per head (Lloyd k-means, ``kmeans``).
* Tokens are sorted by cluster, stably.
* Cluster pairs are chosen by top-p over centroid scores.  For query cluster
  i, the score of key cluster j is c_q,i . c_k,j / sqrt(d) + ln|K_j|.  The
  log-size term makes each score stand for the cluster's total attention
  mass.  The scores are softmaxed over the non-empty key clusters and sorted
  by decreasing probability, lower index first on ties.  The shortest
  prefix whose cumulative sum reaches p is kept.
* A query attends exactly the keys of its selected key clusters, token by
  token, with no rounding to tiles.
"""

import ctypes
import os

import numpy as np

from .attention import softmax_attention, default_scale
from . import build_c

_lib = None


def _kmeans_lib():
    global _lib
    if _lib is None:
        path = build_c.build(force=False)
        lib = ctypes.CDLL(path)
        lib.oracle_lloyd_kmeans.restype = ctypes.c_int
        lib.oracle_lloyd_kmeans.argtypes = [
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def kmeans(x, init_idx, iters, f32_audit=False):
    """Lloyd k-means of the rows of x (float64 [n, d]) from centroids x[init_idx].

    Returns (assign int32[n], centroids float64[k, d], sizes int64[k],
    min_rel_margin).  The margin is the smallest (second-best - best) / best
    squared distance over all points and iterations.  It is used to audit
    that the assignments do not hinge on rounding.

    With f32_audit, a fifth value follows: the smallest ratio of a distance
    gap (any other centroid minus the winner) to the sum of the two
    distances' worst-case float32 rounding error.  Above 1, every assignment
    is the same under any float32 evaluation of the squared distances.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    init_idx = np.ascontiguousarray(init_idx, dtype=np.int32)
    n, d = x.shape
    k = init_idx.size
    assign = np.empty(n, dtype=np.int32)
    cent = np.empty((k, d), dtype=np.float64)
    sizes = np.empty(k, dtype=np.int64)
    margin = ctypes.c_double(0.0)
    ratio = ctypes.c_double(0.0)
    rc = _kmeans_lib().oracle_lloyd_kmeans(
        x.ctypes.data, n, d, k, init_idx.ctypes.data, iters, assign.ctypes.data,
        cent.ctypes.data, sizes.ctypes.data, ctypes.byref(margin),
        ctypes.byref(ratio) if f32_audit else None)
    if rc != 0:
        raise ValueError(f"oracle k-means failed with code {rc}")
    if f32_audit:
        return assign, cent, sizes, margin.value, ratio.value
    return assign, cent, sizes, margin.value


def cluster_permute(assign, k):
    """Stable sort of tokens by cluster id.

    perm[n] = original index of the token at sorted position n; ties keep
    the original order.  offs = exclusive prefix sum of the cluster sizes
    (length k + 1).
    """
    assign = np.asarray(assign)
    perm = np.argsort(assign, kind="stable").astype(np.int32)
    offs = np.zeros(k + 1, dtype=np.int32)
    offs[1:] = np.cumsum(np.bincount(assign, minlength=k))
    return perm, offs


def select_pairs(cq, ck, size_k, top_p, scale=None):
    """Top-p key clusters for every query cluster.

    cq [kq, d], ck [kk, d] float64 centroids; size_k [kk] cluster sizes.
    Returns (pair_ptr int32[kq+1], pair_idx int32[...]).  Each row's key
    clusters are listed in ascending order.  Also returns the per-row
    margins (distance of the cumulative sum from p on either side of the
    crossing, and the probability gap between the last kept and the first
    dropped cluster).
    """
    kq, d = cq.shape
    scale = default_scale(d) if scale is None else scale
    size_k = np.asarray(size_k)
    live = np.flatnonzero(size_k > 0)
    ptr = [0]
    idx = []
    margins = []
    for i in range(kq):
        logits = (ck[live] @ cq[i]) * scale + np.log(size_k[live].astype(np.float64))
        p = np.exp(logits - logits.max())
        p = p / p.sum()
        order = np.lexsort((live, -p))          # by decreasing p, then lower index
        c = np.cumsum(p[order])
        hit = np.flatnonzero(c >= top_p)
        n = int(hit[0]) + 1 if hit.size else live.size
        chosen = np.sort(live[order[:n]])
        idx.extend(chosen.tolist())
        ptr.append(len(idx))
        below = top_p - (c[n - 2] if n >= 2 else 0.0)
        above = c[n - 1] - top_p
        gap = p[order[n - 1]] - p[order[n]] if n < live.size else np.inf
        margins.append((below, above, gap))
    return (np.array(ptr, dtype=np.int32), np.array(idx, dtype=np.int32),
            np.array(margins, dtype=np.float64))


def varlen_attention(q, k, v, assign_q, assign_k, pair_ptr, pair_idx, scale=None,
                     qclusters=None):
    """Attention where a query in cluster i attends the keys of its selected
    key clusters, token-exact.  Original token order, one head.

    q, k, v [N, d] float64.  Returns O [N, d].  With ``qclusters``, only
    those query clusters' rows are filled; the other rows are NaN.
    """
    N, d = q.shape
    scale = default_scale(d) if scale is None else scale
    kq = pair_ptr.size - 1
    out = np.full((N, v.shape[1]), np.nan)
    qclusters = range(kq) if qclusters is None else qclusters
    for i in qclusters:
        rows = np.flatnonzero(assign_q == i)
        if rows.size == 0:
            continue
        sel = pair_idx[pair_ptr[i]:pair_ptr[i + 1]]
        cols = np.flatnonzero(np.isin(assign_k, sel))
        if cols.size == 0:
            out[rows] = 0.0
        else:
            out[rows] = softmax_attention(q[rows], k[cols], v[cols], scale)
    return out
