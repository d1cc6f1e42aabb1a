/*
 * svg.h -- C ABI of the MI355X (gfx950) sparse video attention library.
 *
 * The library implements the training-free sparse 3D attention of Sparse
 * VideoGen for one GPU:
 *   - online head profiling (spatial vs temporal);
 *   - a frame-major <-> position-major layout permutation;
 *   - block-sparse flash attention over kept tiles.
 * The SVG2-style semantic path is declared in svg2.h.
 * Sources are cited per entry point:
 *   [SVG1]  "Sparse VideoGen: Accelerating Video Diffusion Transformers with
 *           Spatial-Temporal Sparsity", English abstract (arxivdaily listing).
 *   [SVG-W] "Sparse-VideoGen and the sparsity hiding inside video diffusion
 *           attention" (project write-up), sections "Three generations of the
 *           same idea" and the install section.
 *   [HVA]   "HyperVAttention: Efficient Sparse Attention with Spatio-Temporal
 *           Clustering for Video Diffusion", sections Problem and Surprising
 *           findings.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are [H][N][d] contiguous, batch 1, with N = F*S + T.  Video
 *   tokens come first in frame-major order: token (f, p) sits at f*S + p,
 *   for frame f < F and position p < S.  The T text tokens follow.
 * - Every tensor or index pointer is a DEVICE pointer owned by the caller.
 *   The library never allocates, frees or synchronises device memory.  It
 *   enqueues all work on `stream` (a hipStream_t; NULL = the null stream)
 *   and never blocks on it.  Workspace buffers are caller-owned device
 *   memory of at least svg_workspace_bytes(...) bytes.
 * - Each call validates its arguments on the host before it enqueues
 *   anything.  On a bad argument it returns a non-zero svg_status and
 *   enqueues nothing.  svg_last_error() then gives a message (per host
 *   thread).
 * - A HIP launch failure returns SVG_ERR_HIP, with the HIP error name in
 *   svg_last_error().  Faults inside a kernel surface on the caller's next
 *   synchronisation, as with any HIP kernel.
 * - Device-resident index inputs (sample_idx, labels, init_idx, CSR lists,
 *   offsets, permutations) are the caller's contract.  Kernels clamp
 *   nothing: out-of-range indices are undefined behaviour.
 * - softmax_scale < 0 selects 1/sqrt(d).
 * - Block shapes (bq x bk): (16,16), (64,64), (128,64).  Head dim d: 64 or
 *   128.  bf16 inputs use MFMA kernels for (64,64) and (128,64).
 *   fp32 inputs, and bf16 at (16,16), use the plain vector kernels.
 */
#ifndef SVG_H_
#define SVG_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SVG_OK = 0,
  SVG_ERR_NULL = 1,         /* a required pointer is NULL                    */
  SVG_ERR_SHAPE = 2,        /* sizes out of range or inconsistent            */
  SVG_ERR_DTYPE = 3,        /* unknown dtype                                 */
  SVG_ERR_UNSUPPORTED = 4,  /* head dim / block shape without a kernel       */
  SVG_ERR_RANGE = 5,        /* bad parameter value, or input aliases output  */
  SVG_ERR_WORKSPACE = 6,    /* workspace missing or smaller than required    */
  SVG_ERR_HIP = 7           /* HIP runtime error                             */
} svg_status;

typedef enum { SVG_F32 = 0, SVG_BF16 = 1 } svg_dtype;

enum { SVG_SPATIAL = 0, SVG_TEMPORAL = 1 };

/* Problem statement of [SVG1]: F frames of S tokens, T text tokens, H heads,
 * head dim d.  N = F*S + T < 2^31 / d. */
typedef struct { int32_t F, S, T, H, d; } svg_dims;

/* Token masks (readings of [SVG1]):
 *   spatial:  a video query of frame f keeps the video keys of frames
 *             f-ks_frames .. f+ks_frames.
 *   temporal: a video query at position p keeps the video keys whose
 *             position-major index r = p'*F + f' lies in
 *             [p*F - wt_tokens, p*F + F - 1 + wt_tokens].
 *   Both:     every query keeps the text keys; a text query keeps all keys.
 */
typedef struct { int32_t ks_frames, wt_tokens; } svg_mask_params;

/* Workspace queries.  `a`, `b` are per-op extra sizes (see each op). */
typedef enum {
  SVG_OP_PROFILE = 0,        /* a = n_samples                                  */
  SVG_OP_BLOCK_SPARSE = 1,   /* a = bq, b = bk  (bitmap -> CSR inside ws)      */
  SVG_OP_COMPACT = 2,        /* a = rows, b = nKB                              */
  SVG_OP_ATTN_VT = 3,        /* a = bq, b = bk  (split text groups, may be 0)  */
  SVG_OP_ATTN_CSR = 4        /* a = bq, b = bk  (Vt + split partials, may be 0) */
} svg_op;

/* Bytes of workspace an op needs for these sizes (host-only, no HIP call). */
size_t svg_workspace_bytes(svg_op op, const svg_dims *dims, int32_t a, int32_t b);

/* Message of the last non-OK status returned on this host thread. */
const char *svg_last_error(void);

/* Library version string. */
const char *svg_version(void);

/* ---------------------------------------------------------------------------
 * Online profiling ([SVG1]: an online profiling strategy predicts each head's
 * type; [SVG-W] "Three generations": it identifies the pattern dynamically).
 *
 * For the sampled query rows sample_idx[0..n_samples) (original frame-major
 * indices, shared by all heads), computes per head:
 *   - the full attention output;
 *   - the spatial-masked output;
 *   - the temporal-masked output.
 * Each softmax is normalised over its own kept keys with its own maximum.
 * Then
 *   mse[h][0] = mean over samples and d of (O_spatial - O_full)^2,
 *   mse[h][1] = the same for O_temporal,
 *   labels[h] = SVG_SPATIAL if mse[h][0] <= mse[h][1], else SVG_TEMPORAL.
 * Q, K, V: [H][N][d] of `dtype`.  labels: int32[H].  mse: float[H][2] or
 * NULL.  ws: svg_workspace_bytes(SVG_OP_PROFILE, dims, n_samples, 0).
 * 1 <= n_samples <= N; sample_idx in [0, N).
 * ------------------------------------------------------------------------- */
svg_status svg_profile_heads(const svg_dims *dims, svg_dtype dtype,
                             const void *Q, const void *K, const void *V,
                             const int32_t *sample_idx, int32_t n_samples,
                             const svg_mask_params *mask, float softmax_scale,
                             int32_t *labels, float *mse,
                             void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Layout transformation ([SVG1]: the hardware-efficient tensor layout
 * transformation).
 *
 * svg_layout_permute:   Y[h][p*F + f] = X[h][f*S + p] for heads with
 *                       labels[h] == SVG_TEMPORAL (position-major order).
 *                       Text rows and other heads are copied unchanged.
 * svg_layout_unpermute: the inverse, X[h][f*S + p] = Y[h][p*F + f].
 * labels == NULL permutes every head.  X and Y are [H][N][d] of `dtype` and
 * must not overlap (SVG_ERR_RANGE if X == Y).
 * ------------------------------------------------------------------------- */
svg_status svg_layout_permute(const svg_dims *dims, svg_dtype dtype, const void *X, void *Y,
                              const int32_t *labels, void *stream);
svg_status svg_layout_unpermute(const svg_dims *dims, svg_dtype dtype, const void *X, void *Y,
                                const int32_t *labels, void *stream);

/* ---------------------------------------------------------------------------
 * Block mask ([SVG-W] install section: block-sparse attention over per-block
 * keep flags).
 *
 * For each head h, takes the token mask of labels[h] in that head's
 * executing layout:
 *   spatial:  frame-major order (the identity);
 *   temporal: position-major order, as produced by svg_layout_permute.
 * block_mask[h][qb][kb] = 1 iff some query row of block qb and some key of
 * block kb (both < N) are kept by the mask.  This is the any-overlap cover.
 * block_mask: uint8 [H][nQB][nKB], nQB = ceil(N/bq), nKB = ceil(N/bk).
 * ------------------------------------------------------------------------- */
svg_status svg_build_block_mask(const svg_dims *dims, const svg_mask_params *mask,
                                const int32_t *labels, int32_t bq, int32_t bk,
                                uint8_t *block_mask, void *stream);

/* Compacts a bitmap uint8[rows][nKB] into CSR lists.  Each row's kept
 * column blocks are written in ascending order.
 *   row_ptr: int32[rows + 1].  row_ptr[rows] = total kept blocks.
 *   kv_idx:  int32 with capacity rows * nKB.
 * ws: svg_workspace_bytes(SVG_OP_COMPACT, NULL, rows, nKB). */
svg_status svg_compact_block_mask(int32_t rows, int32_t nkb, const uint8_t *block_mask,
                                  int32_t *row_ptr, int32_t *kv_idx,
                                  void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * Block-sparse flash attention ([SVG1]: custom kernels on the transformed
 * layout; [SVG-W] install section: block-sparse attention).
 *
 * For query row i of q-block qb:
 *   O[h][i] = sum_j softmax_j(scale * Q[h][i] . K[h][j]) V[h][j]
 * over exactly the keys j < N of the kept tiles (qb, kb).  Kept tiles are
 * computed whole, and skipped tiles cost no memory traffic.  A row with no
 * kept tile gets O = 0.  Accumulation is fp32.  O has the input dtype.
 * Q, K, V, O: [H][N][d] in the executing layout; O must not alias the
 * inputs.
 *
 * svg_block_sparse_attn:     takes the bitmap, compacts it into ws, then
 *                            runs the attention.  ws:
 *                            svg_workspace_bytes(SVG_OP_BLOCK_SPARSE,
 *                            dims, bq, bk) bytes (the bf16 size; fp32 needs
 *                            only the lists' part).
 * svg_block_sparse_attn_csr: takes prebuilt CSR lists over the H*nQB rows
 *                            (row h*nQB + qb), ascending kv-block ids.  ws:
 *                            NULL, or svg_workspace_bytes(SVG_OP_ATTN_CSR,
 *                            dims, bq, bk) bytes.
 * svg_dense_attn:            every tile kept (the dense baseline), with no
 *                            list memory.
 * Kernels: bf16 with bk = 64, bq = 64 or 128, nKB <= 8192 and N*d*2 < 2^31
 * runs on the key-tiled V^T kernel below: V is first transposed into the
 * workspace (svg_block_sparse_attn always; svg_block_sparse_attn_csr when ws
 * is not NULL), and the text rows' groups may be split by keys as described
 * for svg_block_sparse_attn_csr_vt.  Other bf16 shapes, and
 * svg_block_sparse_attn_csr with ws == NULL, run on the row-major MFMA
 * kernel; fp32 and bf16 (16, 16) run on the vector kernel.  Every kernel
 * computes the same softmax; results differ only by fp32 summation order
 * and the bf16 rounding of the row sum (the V^T kernel sums the bf16
 * probabilities that enter P.V).  A ws that shares a byte with Q, K, V or O
 * is SVG_ERR_RANGE; a smaller one SVG_ERR_WORKSPACE.  Calls that share one
 * ws must not overlap in time.
 * ------------------------------------------------------------------------- */
svg_status svg_block_sparse_attn(const svg_dims *dims, svg_dtype dtype,
                                 const void *Q, const void *K, const void *V,
                                 const uint8_t *block_mask, int32_t bq, int32_t bk,
                                 float softmax_scale, void *O,
                                 void *ws, size_t ws_bytes, void *stream);
svg_status svg_block_sparse_attn_csr(const svg_dims *dims, svg_dtype dtype,
                                     const void *Q, const void *K, const void *V,
                                     const int32_t *row_ptr, const int32_t *kv_idx,
                                     int32_t bq, int32_t bk, float softmax_scale,
                                     void *O, void *ws, size_t ws_bytes, void *stream);
svg_status svg_dense_attn(const svg_dims *dims, svg_dtype dtype,
                          const void *Q, const void *K, const void *V,
                          int32_t bq, int32_t bk, float softmax_scale,
                          void *O, void *stream);

/* ---------------------------------------------------------------------------
 * The same attention with V in the key-tiled transposed layout "Vt" ([SVG1]:
 * custom kernels on the transformed layout).  The layout is this library's
 * choice for the gfx950 matrix cores: the pages fix only the token order,
 * not how a kernel stores V.
 *
 * Vt of a [H][N][d] bf16 tensor V (executing layout), nKB = ceil(N/64):
 *   Vt[((h*nKB + kb)*d + c)*64 + j] = V[h][kb*64 + j][c]   if kb*64 + j < N
 *                                   = 0                    otherwise
 * i.e. per 64-key block, the 64 keys of each dim are contiguous.  Size
 * svg_vt_elems(dims) = H*nKB*64*d bf16 values; the caller owns it.
 *
 * svg_layout_permute_vt: Vt of svg_layout_permute(V) in one pass (each
 *   head's executing layout per labels; labels == NULL permutes every head).
 *   bf16 only.  V and Vt must not overlap.
 * svg_block_sparse_attn_csr_vt, svg_dense_attn_vt: as
 *   svg_block_sparse_attn_csr and svg_dense_attn, with V given as Vt.  Each
 *   output row equals theirs up to fp32 summation order.  bf16 only,
 *   (bq, bk) = (64, 64) or (128, 64), nKB <= 8192, N*d*2 < 2^31; otherwise
 *   SVG_ERR_UNSUPPORTED and nothing is enqueued.
 * svg_block_sparse_attn_csr_vt_layout: the SVG1 layer's permute -> attention
 *   -> inverse permute around one launch ([SVG1]: layout transformation,
 *   custom kernels).  Q and O are in the original token order; K, Vt and the
 *   kept-tile lists in each head's executing layout (per labels; NULL =
 *   every head temporal, as svg_layout_permute).  O equals
 *   svg_layout_unpermute(svg_block_sparse_attn_csr_vt(svg_layout_permute(Q),
 *   K, Vt, ...), labels) bit for bit: the kernel reads Q row p*F + f of a
 *   temporal head from frame-major row f*S + p and writes O back there.
 *   Same limits and errors as svg_block_sparse_attn_csr_vt; labels is a
 *   device pointer, int32[H], read on the device.
 * svg_block_sparse_attn_csr_vt_fused: the same with K in the original token
 *   order too (only Vt and the lists are in the executing layout): the
 *   layout transformation of [SVG1] fused into the kernel's loads and
 *   stores.  The tile DMA gathers each K tile's rows (row p*F + f of a
 *   temporal head's video from frame-major row f*S + p) through a table of
 *   source rows in LDS.  O equals svg_block_sparse_attn_csr_vt_layout's
 *   with K = svg_layout_permute(K) bit for bit.  Same limits and errors.
 * ws, ws_bytes (the three sparse entries): the groups of 256 query rows that
 *   hold a head's last 512 rows (its text rows, which keep every kv-block)
 *   are split by keys over several work-groups when nKB > 48: each part
 *   stores an unnormalised partial (O, maximum, row sum) in ws and a merge
 *   combines them (the flash-decoding split of the same softmax).  ws is
 *   caller-owned device memory of svg_workspace_bytes(SVG_OP_ATTN_VT, dims,
 *   bq, bk) bytes (0 when no split applies), or NULL: then no group is split
 *   and only the fp32 summation order differs.  A non-NULL ws smaller than
 *   that is SVG_ERR_WORKSPACE; ws must not overlap the other buffers.  Calls
 *   that share one ws must not overlap in time.
 * ------------------------------------------------------------------------- */
size_t svg_vt_elems(const svg_dims *dims);
svg_status svg_layout_permute_vt(const svg_dims *dims, svg_dtype dtype, const void *V, void *Vt,
                                 const int32_t *labels, void *stream);
svg_status svg_block_sparse_attn_csr_vt(const svg_dims *dims, svg_dtype dtype,
                                        const void *Q, const void *K, const void *Vt,
                                        const int32_t *row_ptr, const int32_t *kv_idx,
                                        int32_t bq, int32_t bk, float softmax_scale,
                                        void *O, void *ws, size_t ws_bytes, void *stream);
svg_status svg_block_sparse_attn_csr_vt_layout(const svg_dims *dims, svg_dtype dtype,
                                               const void *Q, const void *K, const void *Vt,
                                               const int32_t *row_ptr, const int32_t *kv_idx,
                                               const int32_t *labels, int32_t bq, int32_t bk,
                                               float softmax_scale, void *O, void *ws,
                                               size_t ws_bytes, void *stream);
svg_status svg_block_sparse_attn_csr_vt_fused(const svg_dims *dims, svg_dtype dtype,
                                              const void *Q, const void *K, const void *Vt,
                                              const int32_t *row_ptr, const int32_t *kv_idx,
                                              const int32_t *labels, int32_t bq, int32_t bk,
                                              float softmax_scale, void *O, void *ws,
                                              size_t ws_bytes, void *stream);
svg_status svg_dense_attn_vt(const svg_dims *dims, svg_dtype dtype,
                             const void *Q, const void *K, const void *Vt,
                             int32_t bq, int32_t bk, float softmax_scale,
                             void *O, void *stream);

/* ---------------------------------------------------------------------------
 * SVG-EAR ([SVG-W] "Three generations of the same idea": skipped attention
 * blocks are recovered by parameter-free centroid compensation, and
 * error-aware routing computes high-error blocks exactly).  The pages give
 * no formulas; this library's reading, per head in the executing layout,
 * kv-block b = its n_b <= 64 keys:
 *   - compensation: a block outside a q-block's exact set contributes one
 *     centroid key kbar_b (mean key) with weight n_b and value vbar_b (mean
 *     value): O = (sum_exact e^s v + sum_comp n_b e^t vbar) /
 *     (sum_exact e^s + sum_comp n_b e^t), t = scale * q . kbar_b;
 *   - routing: for q-block Q with mean query qbar, a skipped block's score is
 *     ln n_b + scale qbar.kbar_b + ln(expm1(scale |qbar| r_b)), r_b the
 *     block's key radius (the log of a bound on the centroid's error in the
 *     block's attention mass); the route_k best (ties to the lower block)
 *     join the exact set, as does the ragged last block (fewer than 64
 *     keys), so every compensated block has n_b = 64.
 *
 * svg_ear_centroid_elems: elements of each centroid table,
 *   H * ceil(nKB/64) * 64 * d (slots past the last block are zero).
 * svg_ear_block_stats: from K [H][N][d] and Vt (svg_layout_permute_vt), both
 *   in the executing layout: Kc (bf16 centroid keys, [H][tiles*64][d]), Vct
 *   (bf16 value sums n_b * vbar_b in the key-tiled V^T layout,
 *   [H][tiles][d][64]), kbar (double, dim-major [H][d][nKB]) and radius
 *   (double [H][nKB]).
 * svg_ear_route: from Q (original token order, mapped to the executing
 *   layout per labels as the layout permute does), kbar, radius and the
 *   block mask (uint8 [H][nQB][nKB]): exact_mask (same shape) = the mask,
 *   the ragged last block and the routed blocks.  Decided in double.
 *   route_k >= 0; bk = 64, bq = 64 or 128.
 * svg_block_sparse_attn_ear_vt_layout: svg_block_sparse_attn_csr_vt_layout
 *   over the CSR lists of exact_mask, plus the compensation of every other
 *   block from Kc / Vct.  The lists must hold the ragged last block (as
 *   exact_mask does).  nKB <= 8064; no split of the text rows' groups.
 * Inputs bf16; outputs must not overlap inputs (SVG_ERR_RANGE).
 * ------------------------------------------------------------------------- */
size_t svg_ear_centroid_elems(const svg_dims *dims);
svg_status svg_ear_block_stats(const svg_dims *dims, svg_dtype dtype, const void *K, const void *Vt,
                               void *Kc, void *Vct, double *kbar, double *radius, void *stream);
svg_status svg_ear_route(const svg_dims *dims, svg_dtype dtype, const void *Q, const int32_t *labels,
                         const double *kbar, const double *radius, const uint8_t *block_mask, int32_t bq,
                         int32_t bk, int32_t route_k, float softmax_scale, uint8_t *exact_mask,
                         void *stream);
svg_status svg_block_sparse_attn_ear_vt_layout(const svg_dims *dims, svg_dtype dtype, const void *Q,
                                               const void *K, const void *Vt, const void *Kc,
                                               const void *Vct, const int32_t *row_ptr,
                                               const int32_t *kv_idx, const int32_t *labels, int32_t bq,
                                               int32_t bk, float softmax_scale, void *O, void *stream);

/* ---------------------------------------------------------------------------
 * FP8 attention ([SVG-W] "Publication record and the road ahead": FP8
 * attention is an open item of the plan; the pages give no method, so the
 * quantization below is this library's definition).
 *
 * Format: OCP E4M3 codes (bias 7, largest finite 448, subnormals, no
 * infinities), one byte per value, round to nearest with ties to even.
 * Scales: for a group of values x (bf16) with largest magnitude a,
 *   code = round_e4m3(fp32(x * (448 / a))),  scale = a / 448  (fp32);
 * a group of zeros gets codes 0 and scale 0.  A code stands for
 * decode(code) * scale.
 *
 * svg_quantize_fp8_rows: one scale per row (token) of X [H][N][d] bf16:
 *   X8 uint8 [H][N][d], scale float [H][N].  Row order is kept (use it on Q
 *   in the original token order).
 * svg_layout_permute_fp8: K into each head's executing layout (per labels,
 *   NULL = every head position-major, as svg_layout_permute), then one scale
 *   per block of 64 rows of that layout: X8 uint8 [H][N][d], scale float
 *   [H][ceil(N/64)].
 * svg_block_sparse_attn_fp8_vt_layout: svg_block_sparse_attn_csr_vt_layout
 *   with Q and K given as codes and scales: the logit of query i and key j
 *   is (sum_c Q8_ic K8_jc) * qscale_i * kscale_block(j) * softmax_scale,
 *   accumulated in fp32 on the FP8 matrix cores; softmax, the bf16 P.V with
 *   Vt and the bf16 output O (original token order) are those of the bf16
 *   entry.  Q8 / qscale in the original token order; K8 / kscale, Vt and the
 *   lists in the executing layout.  No split of the text rows' groups.
 * svg_dense_attn_fp8_vt: every tile kept, Q8 / K8 / Vt in one common order.
 *
 * The FP8 P.V mode (also this library's definition) codes V and the
 * probabilities as well:
 * svg_layout_permute_vt_fp8: V [H][N][d] bf16 -> vamax float [H][d], each
 *   channel's largest magnitude over the head's N tokens (channel scale
 *   vamax / 448), and Vt8 uint8 [H][ceil(N/64)][d][64]: V in the executing
 *   layout (per labels, as svg_layout_permute_vt), key-tiled and transposed,
 *   code round_e4m3(fp32(v * (448 / vamax_d))).  Within a tile row, byte
 *   j = 32 h + b holds key 32 (b >> 4) + 16 ((b >> 3) & 1) + 8 h + (b & 7)
 *   (the order the attention holds its probabilities in); keys past N are
 *   code 0.  Runs three kernels on the stream; Vt8 and vamax are written
 *   whole.
 * svg_block_sparse_attn_fp8pv_vt_layout: svg_block_sparse_attn_fp8_vt_layout
 *   with V given as Vt8 / vamax, and P coded too: a query row walks its
 *   q-block's kept tiles in ascending order with a lazy reference m of its
 *   logits y (exp2 units), moved to a tile's maximum when that exceeds m by
 *   more than 8 (the sums so far rescaled by 2^(m_old - m_new)); each
 *   p = 2^(y - m) <= 2^8 becomes round_e4m3(fp32(p)) with no scale; P.V and
 *   the row sum take those codes on the FP8 matrix cores (fp32
 *   accumulation), and O = (P8 . V8) / sum(P8) times the channel scales
 *   (bf16, original token order).
 * Limits: bf16 inputs to the quantizers; d = 128, (bq, bk) = (64, 64) or
 * (128, 64), nKB <= 8192 for the attention (else SVG_ERR_UNSUPPORTED).
 * Buffers must not overlap their inputs (SVG_ERR_RANGE).
 * ------------------------------------------------------------------------- */
svg_status svg_quantize_fp8_rows(const svg_dims *dims, svg_dtype dtype, const void *X, uint8_t *X8,
                                 float *scale, void *stream);
svg_status svg_layout_permute_fp8(const svg_dims *dims, svg_dtype dtype, const void *X, uint8_t *X8,
                                  float *scale, const int32_t *labels, void *stream);
svg_status svg_block_sparse_attn_fp8_vt_layout(const svg_dims *dims, const uint8_t *Q8, const float *qscale,
                                               const uint8_t *K8, const float *kscale, const void *Vt,
                                               const int32_t *row_ptr, const int32_t *kv_idx,
                                               const int32_t *labels, int32_t bq, int32_t bk,
                                               float softmax_scale, void *O, void *stream);
svg_status svg_dense_attn_fp8_vt(const svg_dims *dims, const uint8_t *Q8, const float *qscale,
                                 const uint8_t *K8, const float *kscale, const void *Vt, int32_t bq,
                                 int32_t bk, float softmax_scale, void *O, void *stream);
svg_status svg_layout_permute_vt_fp8(const svg_dims *dims, svg_dtype dtype, const void *V, uint8_t *Vt8,
                                     float *vamax, const int32_t *labels, void *stream);
svg_status svg_block_sparse_attn_fp8pv_vt_layout(const svg_dims *dims, const uint8_t *Q8, const float *qscale,
                                                 const uint8_t *K8, const float *kscale, const uint8_t *Vt8,
                                                 const float *vamax, const int32_t *row_ptr,
                                                 const int32_t *kv_idx, const int32_t *labels, int32_t bq,
                                                 int32_t bk, float softmax_scale, void *O, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* SVG_H_ */
