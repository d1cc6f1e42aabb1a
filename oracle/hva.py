"""HVA-style clustering (oracle): 3D local-window k-means and anchor-step
reuse of the clusters.  Test infrastructure: only the tests, the smoke check
and the CPU baseline of the benchmark use this module.

Source: "HyperVAttention: Efficient Sparse Attention with Spatio-Temporal
Clustering for Video Diffusion", sections Approach and Key results.  Centroid
search is restricted to local 3D spatio-temporal windows; assignments are
reused across denoising steps, with full clustering only at anchor steps and,
otherwise, a refresh of a subset of tokens chosen by Lowe's ratio.  The page
gives no formulas.  Readings (each stated again where it is used):

* Geometry.  Video token (f, y, x) of the F x rows x cols latent grid is token
  f*S + y*cols + x (S = rows*cols); the T text tokens follow.  The grid is cut
  into windows of wf x wy x wx tokens (the last ones along an axis may be
  smaller); window (a, b, c) has cluster id (a*nY + b)*nX + c.  The text
  tokens form one more cluster, id C = nF*nY*nX, that never changes members.
* Seeds.  Each window's centroid starts as the mean of its own tokens; the
  text centroid is the mean of the text tokens.
* Local search.  A video token in window (a, b, c) is assigned among the
  centroids of the windows (a', b', c') with |a'-a|, |b'-b|, |c'-c| <= 1 (at
  most 27), by squared L2 distance, ties to the lowest cluster id.
* Precision of the decision.  The distances decide integers, and in this
  method neighbouring windows that split one region have near-equal
  centroids, so ties within rounding are common.  The decision is therefore
  defined in float32, in a fixed order: dist = sum over dims c = 0..d-1, in
  order, of fl(fl(x_c - m_c)^2), each added by a float32 add, where x_c is
  the (bf16-exact) value and m_c the float64 centroid rounded to float32.
  numpy's float32 arithmetic is IEEE single precision with round to nearest
  even, as is the GPU's.
* Update.  Each centroid becomes the float64 mean of its members; a cluster
  with no member keeps its centroid.  Member sums of bf16 values are exact in
  float64 (within the exponent-span bound of the k-means update), so their
  order does not matter.
* Lowe's ratio.  In the last assignment of an anchor step, a video token is
  flagged for refresh when its best distance d1 and the second best d2 among
  its candidates satisfy d1 >= fl(r2 * d2) in float32 (r2 = 0.64: Lowe's ratio
  0.8 on distances, squared), i.e. its match is not distinctive.  A token
  with a single candidate is never flagged.
* Refresh (a non-anchor step, new values X): flagged tokens are re-assigned
  among their candidates against the carried centroids (other tokens keep
  their cluster); then one update from X under the new assignment.
"""

import numpy as np


def grid_windows(F, rows, cols, win):
    """Per video token its window cell (a, b, c) and cluster id; the window
    counts (nF, nY, nX)."""
    wf, wy, wx = win
    nF, nY, nX = -(-F // wf), -(-rows // wy), -(-cols // wx)
    f, y, x = np.meshgrid(np.arange(F), np.arange(rows), np.arange(cols), indexing="ij")
    a, b, c = (f // wf).ravel(), (y // wy).ravel(), (x // wx).ravel()
    cid = (a * nY + b) * nX + c
    return a, b, c, cid.astype(np.int64), (nF, nY, nX)


def candidates(F, rows, cols, win):
    """int64 [F*rows*cols, 27] candidate cluster ids of every video token, in
    increasing id order, padded with -1."""
    a, b, c, _, (nF, nY, nX) = grid_windows(F, rows, cols, win)
    out = np.full((a.size, 27), -1, dtype=np.int64)
    n = np.zeros(a.size, dtype=np.int64)
    for da in (-1, 0, 1):                      # (da, db, dc) in lexicographic order = increasing id
        for db in (-1, 0, 1):
            for dc in (-1, 0, 1):
                aa, bb, cc = a + da, b + db, c + dc
                ok = (aa >= 0) & (aa < nF) & (bb >= 0) & (bb < nY) & (cc >= 0) & (cc < nX)
                ids = (aa * nY + bb) * nX + cc
                rows_ = np.flatnonzero(ok)
                out[rows_, n[rows_]] = ids[rows_]
                n[rows_] += 1
    return out


def n_clusters(F, rows, cols, T, win):
    nF, nY, nX = grid_windows(F, rows, cols, win)[4]
    return nF * nY * nX + (1 if T > 0 else 0)


def means(x, assign, k, prev):
    """float64 means of the members of each cluster (prev where empty), and
    the sizes."""
    d = x.shape[1]
    sizes = np.bincount(assign, minlength=k)
    sums = np.zeros((k, d))
    for c in range(d):
        sums[:, c] = np.bincount(assign, weights=x[:, c], minlength=k)
    cent = prev.copy()
    live = sizes > 0
    cent[live] = sums[live] / sizes[live][:, None]
    return cent, sizes


def f32_dists(x, cent, cand):
    """float32 squared distances [n, 27] of video tokens to their candidate
    centroids (inf for padding), summed over dims in order as stated above."""
    x32 = x.astype(np.float32)
    m32 = cent.astype(np.float32)
    out = np.full(cand.shape, np.float32(np.inf), dtype=np.float32)
    for s in range(cand.shape[1]):
        valid = cand[:, s] >= 0
        m = m32[np.where(valid, cand[:, s], 0)]     # [n, d]
        acc = np.zeros(x.shape[0], dtype=np.float32)
        for c in range(x.shape[1]):
            t = x32[:, c] - m[:, c]
            acc = acc + t * t
        out[valid, s] = acc[valid]
    return out


def assign_local(x, cent, cand, r2=np.float32(0.64)):
    """Best candidate per video token (ties to the lower id: candidates are in
    increasing id order and the first minimum wins) and the Lowe flags."""
    dist = f32_dists(x, cent, cand)
    j = np.argmin(dist, axis=1)                 # first minimum
    rows = np.arange(cand.shape[0])
    best = cand[rows, j]
    d1 = dist[rows, j]
    rest = dist.copy()
    rest[rows, j] = np.float32(np.inf)
    d2 = rest.min(axis=1)
    flag = np.isfinite(d2) & (d1 >= np.float32(r2) * d2)
    return best, flag, d1, d2


def local_kmeans(x, F, rows, cols, T, win, iters, r2=np.float32(0.64)):
    """Full clustering of an anchor step.

    x float64 [N, d] (bf16 values), N = F*rows*cols + T.  Returns
    (assign int32[N], centroids float64[k, d], sizes int64[k],
    refresh uint8[N]) after `iters` assignment + update rounds from the
    window seeds; refresh holds the Lowe flags of the last assignment (text
    tokens 0)."""
    Nv = F * rows * cols
    k = n_clusters(F, rows, cols, T, win)
    _, _, _, cid, _ = grid_windows(F, rows, cols, win)
    assign = np.empty(x.shape[0], dtype=np.int64)
    assign[:Nv] = cid
    assign[Nv:] = k - 1
    cent, sizes = means(x, assign, k, np.zeros((k, x.shape[1])))
    cand = candidates(F, rows, cols, win)
    flag = np.zeros(Nv, dtype=bool)
    for _ in range(iters):
        assign[:Nv], flag, _, _ = assign_local(x[:Nv], cent, cand, r2)
        cent, sizes = means(x, assign, k, cent)
    refresh = np.zeros(x.shape[0], dtype=np.uint8)
    refresh[:Nv] = flag
    return assign.astype(np.int32), cent, sizes, refresh


def refresh_step(x, assign, cent, refresh, F, rows, cols, T, win, r2=np.float32(0.64)):
    """A non-anchor step: flagged tokens re-assigned against the carried
    centroids, then one update from x.  Returns (assign, centroids, sizes)."""
    Nv = F * rows * cols
    k = cent.shape[0]
    cand = candidates(F, rows, cols, win)
    new = np.asarray(assign, dtype=np.int64).copy()
    sel = np.flatnonzero(np.asarray(refresh[:Nv]) != 0)
    if sel.size:
        best, _, _, _ = assign_local(x[sel], cent, cand[sel], r2)
        new[sel] = best
    cent2, sizes = means(x, new, k, cent)
    return new.astype(np.int32), cent2, sizes


def sse(x, assign, cent):
    """Sum of squared distances of the tokens to their centroids (float64)."""
    return float(((x - cent[assign]) ** 2).sum())
