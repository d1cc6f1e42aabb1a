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
  SVG2_OP_VARLEN = 2           /* a = kq, b = kk        */
} svg2_op;

/* Bytes of workspace an SVG2 op needs (host-only, no HIP call). */
size_t svg2_workspace_bytes(svg2_op op, const svg_dims *dims, int32_t a, int32_t b);

/* ---------------------------------------------------------------------------
 * Only N = F*S + T, H and d are read from dims.
 *
 * svg_kmeans: per head, Lloyd k-means of the N rows of X ([H][N][d], `dtype`).
 *   Starts from centroids X[h][init_idx[h][j]].  Runs `iters` rounds of:
 *     - assign: nearest centroid by squared L2 distance, ties to the lowest
 *       index;
 *     - update: mean of the members; an empty cluster keeps its centroid.
 *   Outputs the last assignment (int32 [H][N]), its centroids (double
 *   [H][k][d]; member sums are exact in double) and the sizes (int32 [H][k]).
 *   ws: svg2_workspace_bytes(SVG2_OP_KMEANS, dims, k, 0).
 *   1 <= k <= 256, iters >= 1.
 * ------------------------------------------------------------------------- */
svg_status svg_kmeans(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t k,
                      int32_t iters, const int32_t *init_idx, int32_t *assign,
                      double *centroids, int32_t *sizes, void *ws, size_t ws_bytes,
                      void *stream);

/* Stable counting sort of tokens by cluster.
 *   perm[h][n] = original index of the n-th token in cluster order; ties
 *                keep the original order.
 *   offs[h][c] = first sorted position of cluster c (int32 [H][k+1]).
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
 * ws: svg2_workspace_bytes(SVG2_OP_VARLEN, dims, kq, kk). */
svg_status svg_varlen_attn(const svg_dims *dims, svg_dtype dtype,
                           const void *Qp, const void *Kp, const void *Vp,
                           const int32_t *q_offs, const int32_t *k_offs, int32_t kq, int32_t kk,
                           const int32_t *pair_ptr, const int32_t *pair_idx,
                           const int32_t *q_perm, float softmax_scale, void *O,
                           void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SVG2_H_ */
