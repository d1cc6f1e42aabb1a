/*
 * svg2.h -- C ABI of the SVG2-style semantic path (gfx950).
 *
 * Sources:
 *   [SVG-W] "Sparse-VideoGen and the sparsity hiding inside video diffusion
 *           attention" (project write-up), section "Three generations of the
 *           same idea": SVG2 adds semantic-aware permutation, a dynamic
 *           attention kernel and a flash k-means kernel.  Its install
 *           section covers block-sparse attention with varied block sizes.
 *   [HVA]   "HyperVAttention: Efficient Sparse Attention with Spatio-Temporal
 *           Clustering for Video Diffusion", sections Problem and Surprising
 *           findings: clusters give irregular blocks.
 * Conventions (device pointers, caller-owned workspaces, host validation,
 * status codes, svg_last_error) are those of svg.h.
 */
#ifndef SVG2_H_
#define SVG2_H_

#include "svg.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVG2_OP_KMEANS = 0,          /* a = k                 */
  SVG2_OP_CLUSTER_PERMUTE = 1, /* a = k                 */
  SVG2_OP_VARLEN = 2,          /* a = kq, b = kk        */
  SVG2_OP_HVA = 3              /* a = k (svg_hva_clusters) */
} svg2_op;

/* Bytes of workspace an SVG2 op needs (host-only, no HIP call). */
size_t svg2_workspace_bytes(svg2_op op, const svg_dims *dims, int32_t a, int32_t b);

/* ---------------------------------------------------------------------------
 * Only N = F*S + T, H and d are read from dims.
 *
 * svg_kmeans: per head, Lloyd k-means of the N rows of X ([H][N][d], `dtype`).
 *   Starts from centroids X[h][init_idx[h][j]] (init_idx in [0, N)).  Runs
 *   `iters` rounds of:
 *     - assign: nearest centroid by squared L2 distance, ties to the lowest
 *       index;
 *     - update: mean of the members; an empty cluster keeps its centroid.
 *   Outputs the last assignment (int32 [H][N]), its centroids (double
 *   [H][k][d]) and the sizes (int32 [H][k]).  A round whose assignment
 *   equals the previous round's is a fixed point of these two steps: every
 *   later round would repeat it.  The kernels of a head's remaining rounds
 *   then return at once; the outputs are those of all `iters` rounds, bit
 *   for bit.  For bf16 X the member sums
 *   are exact in double, so equal to the index-order sums, while the
 *   exponent span of a dimension's nonzero member values is at most
 *   45 - log2(cluster size) bits.
 *   ws: svg2_workspace_bytes(SVG2_OP_KMEANS, dims, k, 0).
 *   1 <= k <= 256, iters >= 1.
 * ------------------------------------------------------------------------- */
svg_status svg_kmeans(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t k,
                      int32_t iters, const int32_t *init_idx, int32_t *assign,
                      double *centroids, int32_t *sizes, void *ws, size_t ws_bytes,
                      void *stream);

/* ---------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 *
 * svg_kmeans_noalloc: svg_kmeans with no workspace argument.  Its scratch
 *   (cluster order, offsets, centroid tables, sort counts, the per-head
 *   fixed-point flags) lives in a device
 *   array the library holds, SVG_KMEANS_NOALLOC_SCRATCH_BYTES per GPU,
 *   allocated when the library's code is loaded on that GPU and kept until
 *   the process ends.  The call allocates nothing.  Outputs and errors are
 *   those of svg_kmeans, bit for bit; a problem whose
 *   svg2_workspace_bytes(SVG2_OP_KMEANS, dims, k, 0) exceeds the array is
 *   SVG_ERR_WORKSPACE with nothing enqueued.  The current device's array is
 *   used, so `stream` must belong to the current device.  All calls on one
 *   GPU share its array: calls that overlap in time there (two streams, two
 *   host threads) race and give wrong results.  A call overwrites every
 *   scratch word before reading it, so one call's leftovers never reach the
 *   next.
 * ------------------------------------------------------------------------- */
#define SVG_KMEANS_NOALLOC_SCRATCH_BYTES (32u << 20)
svg_status svg_kmeans_noalloc(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t k,
                              int32_t iters, const int32_t *init_idx, int32_t *assign,
                              double *centroids, int32_t *sizes, void *stream);

/* Stable counting sort of tokens by cluster.
 *   perm[h][n] = original index of the n-th token in cluster order; ties
 *                keep the original order.
 *   offs[h][c] = first sorted position of cluster c (int32 [H][k+1]).
 * assign[h][n] must lie in [0, k).  A token whose id does not is skipped
 * (no cluster counts it, offs[h][k] counts only the others, and perm[h]
 * from offs[h][k] on is left unwritten), so a bad id never indexes outside
 * a buffer; the call does not report it.
 * ws: svg2_workspace_bytes(SVG2_OP_CLUSTER_PERMUTE, dims, k, 0). */
svg_status svg_cluster_permute(const svg_dims *dims, const int32_t *assign, int32_t k,
                               int32_t *perm, int32_t *offs, void *ws, size_t ws_bytes,
                               void *stream);

/* Row gather / scatter by a per-head permutation (int32 [H][N]):
 *   inverse = 0: Y[h][n] = X[h][perm[h][n]]
 *   inverse = 1: Y[h][perm[h][n]] = X[h][n]
 * X and Y must not overlap. */
svg_status svg_permute_rows(const svg_dims *dims, svg_dtype dtype, const void *X,
                            const int32_t *perm, void *Y, int32_t inverse, void *stream);

/* Top-p cluster pairs (reading of SVG2's selection).  For query cluster i of
 * head h:
 *   l_ij = scale * cq[h][i] . ck[h][j] + ln(size_k[h][j]),
 *   taken over the key clusters with size_k > 0.
 * The l_ij are softmaxed and sorted by decreasing probability (lower j on
 * ties).  The shortest prefix whose cumulative sum reaches top_p is kept,
 * or all clusters if the sum never reaches it.  Computed in double.
 *   pair_ptr: int32 [H][kq+1], offsets into that head's segment
 *             pair_idx + h*kq*kk.
 *   pair_idx: int32 [H][kq*kk], each row's key clusters ascending.
 * cq: double [H][kq][d], ck: double [H][kk][d], size_k: int32 [H][kk].
 * 0 < top_p <= 1, kk <= 256. */
svg_status svg_select_pairs(const svg_dims *dims, const double *cq, const double *ck,
                            const int32_t *size_k, int32_t kq, int32_t kk, double top_p,
                            float softmax_scale, int32_t *pair_ptr, int32_t *pair_idx,
                            void *stream);

/* Variable-size block-sparse attention over cluster pairs ([SVG-W] install
 * section: block-sparse attention with varied block sizes).  Inputs are in
 * cluster order:
 *   - query cluster i is rows q_offs[h][i] .. q_offs[h][i+1] of Qp;
 *   - key cluster j is rows k_offs[h][j] .. k_offs[h][j+1] of Kp and Vp.
 * A query of cluster i attends exactly the keys of its selected clusters,
 * pair_idx[h*kq*kk + pair_ptr[h][i] ...].  The result is token-exact, with
 * no rounding to tiles.
 * Row n of the result is written to O[h][q_perm[h][n]] when q_perm is
 * non-NULL (back to original order), else to O[h][n].
 * One work-group takes 128 rows of one query cluster and walks the
 * concatenation of its selected key ranges in 64-key
 * tiles; the tile DMA gathers the K and V rows of each tile from a table of
 * source rows in LDS.  d = 64 or 128; q_offs, k_offs, pair_ptr and
 * pair_idx in range by contract (as svg_select_pairs and
 * svg_cluster_permute write them).
 * ws: svg2_workspace_bytes(SVG2_OP_VARLEN, dims, kq, kk), which is 0: ws
 * may be NULL. */
svg_status svg_varlen_attn(const svg_dims *dims, svg_dtype dtype,
                           const void *Qp, const void *Kp, const void *Vp,
                           const int32_t *q_offs, const int32_t *k_offs, int32_t kq, int32_t kk,
                           const int32_t *pair_ptr, const int32_t *pair_idx,
                           const int32_t *q_perm, float softmax_scale, void *O,
                           void *ws, size_t ws_bytes, void *stream);

/* Rows of V gathered into the key-tiled V^T layout that svg_varlen_attn_vt
 * reads (the value side of the cluster permutation, in one pass):
 *   Vt[h][kb][c][j] = V[h][perm[h][64*kb + j]][c],  zero where 64*kb + j >= N.
 * V: bf16 [H][N][d]; perm: int32 [H][N], each entry in [0, N) (not
 * checked: an index out of range reads out of bounds); Vt: bf16
 * [H][ceil(N/64)][d][64] (svg_vt_elems elements).  V and Vt must not
 * overlap. */
svg_status svg_permute_rows_vt(const svg_dims *dims, svg_dtype dtype, const void *V,
                               const int32_t *perm, void *Vt, void *stream);

/* svg_varlen_attn on the key-tiled V^T of Vp (as svg_permute_rows_vt writes
 * it): the same result, token-exact.  One work-group takes 128 rows of one
 * query cluster and walks the 64-key windows of Kp / Vt that its selected
 * key ranges touch; each window carries a 64-bit mask of its selected keys
 * and the others score -inf.  d = 64 or 128, N <= 131072 (2048 windows a
 * head); q_offs, k_offs, pair_ptr and pair_idx as for svg_varlen_attn (in
 * range by contract).  No workspace. */
svg_status svg_varlen_attn_vt(const svg_dims *dims, svg_dtype dtype,
                              const void *Qp, const void *Kp, const void *Vt,
                              const int32_t *q_offs, const int32_t *k_offs, int32_t kq, int32_t kk,
                              const int32_t *pair_ptr, const int32_t *pair_idx,
                              const int32_t *q_perm, float softmax_scale, void *O, void *stream);

/* ---------------------------------------------------------------------------
 * HVA-style clustering (HyperVAttention, sections Approach and Key results:
 * centroid search restricted to local 3D spatio-temporal windows; cluster
 * assignments reused across denoising steps, with full clustering only at
 * anchor steps and a Lowe's-ratio-selected subset refreshed otherwise).  The
 * page gives no formulas; this library's reading, per head:
 *   - video token (f, y, x) of the F x rows x cols grid (rows * cols = S) is
 *     row f*S + y*cols + x; the T text rows follow;
 *   - the grid is cut into windows of win[0] x win[1] x win[2] tokens (the
 *     last ones along an axis may be smaller); window (a, b, c) is cluster
 *     (a*nY + b)*nX + c, nF = ceil(F/win[0]), nY = ceil(rows/win[1]),
 *     nX = ceil(cols/win[2]); the text rows form one more cluster,
 *     C = nF*nY*nX, whose members never change;
 *   - seeds: each window's mean, and the text rows' mean;
 *   - a video token chooses among the centroids of its own and the adjacent
 *     windows (|da|, |db|, |dc| <= 1), by the float32 distance
 *     sum over dims in order of fl(fl(x - m)^2) with float32 adds (m: the
 *     double centroid rounded to float32), ties to the lower cluster id;
 *   - update: double means of the members (exact sums of bf16 values); an
 *     empty cluster keeps its centroid;
 *   - Lowe flags (last assignment of svg_hva_cluster): a video token whose
 *     best and second-best distances satisfy d1 >= fl(lowe_r2 * d2) in
 *     float32 (not distinctive) is flagged for refresh; text rows never.
 *
 * svg_hva_clusters: the number of clusters k = C + (T > 0), or 0 for
 *   invalid arguments.
 * svg_hva_cluster (anchor step): seeds, then iters >= 1 rounds of local
 *   assignment and update.  Outputs assign int32 [H][N], centroids double
 *   [H][k][d], sizes int32 [H][k], refresh uint8 [H][N] (the Lowe flags).
 * svg_hva_refresh (non-anchor step, new values X): tokens with refresh != 0
 *   are re-assigned among their candidates against the carried centroids
 *   (as is any token whose cluster is not among its candidates), the others
 *   keep assign; then one update from X.  assign and centroids are read and
 *   written in place, sizes written.
 * X bf16 [H][N][d], d = 64 or 128, F >= 1, rows * cols = S, windows >= 1.
 * ws: svg2_workspace_bytes(SVG2_OP_HVA, dims, k, 0).  Outputs must not
 * overlap X or ws (SVG_ERR_RANGE).
 * ------------------------------------------------------------------------- */
int32_t svg_hva_clusters(const svg_dims *dims, int32_t rows, int32_t cols, const int32_t win[3]);
svg_status svg_hva_cluster(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t rows,
                           int32_t cols, const int32_t win[3], int32_t iters, float lowe_r2,
                           int32_t *assign, double *centroids, int32_t *sizes, uint8_t *refresh,
                           void *ws, size_t ws_bytes, void *stream);
svg_status svg_hva_refresh(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t rows,
                           int32_t cols, const int32_t win[3], const uint8_t *refresh,
                           int32_t *assign, double *centroids, int32_t *sizes, void *ws,
                           size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SVG2_H_ */
