// C ABI: host-side validation, workspace sizing and kernel dispatch.
//
// Every entry point checks its arguments before it touches the HIP runtime.
// A bad call therefore returns a status and enqueues nothing.  The library
// owns no device memory and never synchronises the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/svg2.h"
#include "svg_common.h"

using svgk::Dims;

namespace {

thread_local char g_err[512] = "";

svg_status fail(svg_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
svg_status fail(svg_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

svg_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return SVG_OK;
  return fail(SVG_ERR_HIP, "%s: HIP error %s", what, hipGetErrorName(e));
}

constexpr int64_t kMaxTokens = (int64_t)1 << 28;

svg_status check_dims(const svg_dims *dm, Dims *out, bool need_video = true) {
  if (dm == nullptr) return fail(SVG_ERR_NULL, "dims is NULL");
  if (dm->F < 0 || dm->S < 0 || dm->T < 0 || dm->H < 1)
    return fail(SVG_ERR_SHAPE, "dims out of range (F=%d S=%d T=%d H=%d)", dm->F, dm->S, dm->T, dm->H);
  if (need_video && (dm->F < 1 || dm->S < 1))
    return fail(SVG_ERR_SHAPE, "F and S must be >= 1 (F=%d S=%d)", dm->F, dm->S);
  const int64_t N = (int64_t)dm->F * dm->S + dm->T;
  if (N < 1 || N > kMaxTokens) return fail(SVG_ERR_SHAPE, "N = F*S + T = %lld out of range", (long long)N);
  if (dm->d != 64 && dm->d != 128)
    return fail(SVG_ERR_UNSUPPORTED, "head dim d=%d unsupported (64 or 128)", dm->d);
  if ((int64_t)dm->H * N * dm->d > ((int64_t)1 << 40))
    return fail(SVG_ERR_SHAPE, "H*N*d too large");
  *out = Dims{dm->F, dm->S, dm->T, dm->H, dm->d, (int)N};
  return SVG_OK;
}

svg_status check_dtype(svg_dtype dt) {
  if (dt != SVG_F32 && dt != SVG_BF16) return fail(SVG_ERR_DTYPE, "unknown dtype %d", (int)dt);
  return SVG_OK;
}

int elem_bytes(svg_dtype dt) { return dt == SVG_BF16 ? 2 : 4; }

svg_status check_blocks(int bq, int bk) {
  if ((bq == 16 && bk == 16) || (bq == 64 && bk == 64) || (bq == 128 && bk == 64)) return SVG_OK;
  return fail(SVG_ERR_UNSUPPORTED, "block shape %dx%d unsupported ((16,16), (64,64), (128,64))", bq, bk);
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool overlaps(const void *a, const void *b, size_t bytes) {
  const char *x = (const char *)a, *y = (const char *)b;
  return x < y + bytes && y < x + bytes;
}

// [a, a + la) and [b, b + lb) share a byte
bool overlaps2(const void *a, size_t la, const void *b, size_t lb) {
  const char *x = (const char *)a, *y = (const char *)b;
  return x < y + lb && y < x + la;
}

size_t block_sparse_ws(const Dims &dm, int bq, int bk) {
  const size_t nqb = (dm.N + bq - 1) / bq, nkb = (dm.N + bk - 1) / bk;
  const size_t rows = (size_t)dm.H * nqb;
  return svgk::compact_ws_bytes((int)rows) + align256((rows + 1) * 4) + align256(rows * nkb * 4);
}

hipError_t run_attention(const Dims &dm, svg_dtype dtype, const void *Q, const void *K,
                         const void *V, void *O, const int32_t *row_ptr, const int32_t *kv_idx,
                         int bq, int bk, float scale, hipStream_t st) {
  // the MFMA kernel addresses a head with 32-bit byte offsets
  if (dtype == SVG_BF16 && bk == 64 && (int64_t)dm.N * dm.d * 2 < ((int64_t)1 << 31))
    return svgk::launch_attn_mfma(dm, Q, K, V, O, row_ptr, kv_idx, bq, bk, scale, st);
  return svgk::launch_attn_simt(dm, dtype == SVG_BF16, Q, K, V, O, row_ptr, kv_idx, bq, bk, scale, st);
}

float resolve_scale(float s, int d) { return s < 0.f ? 1.f / sqrtf((float)d) : s; }

}  // namespace

extern "C" {

const char *svg_last_error(void) { return g_err; }

const char *svg_version(void) { return "svg-mi355x 0.1.0 (gfx950)"; }

size_t svg_workspace_bytes(svg_op op, const svg_dims *dims, int32_t a, int32_t b) {
  Dims dm{};
  switch (op) {
    case SVG_OP_COMPACT:
      return a < 0 ? 0 : svgk::compact_ws_bytes(a);
    case SVG_OP_PROFILE:
      if (check_dims(dims, &dm) != SVG_OK || a < 1) return 0;
      return svgk::profile_ws_bytes(dm, a);
    case SVG_OP_BLOCK_SPARSE:
      if (check_dims(dims, &dm) != SVG_OK || check_blocks(a, b) != SVG_OK) return 0;
      return block_sparse_ws(dm, a, b);
    case SVG_OP_ATTN_VT:
      if (check_dims(dims, &dm) != SVG_OK) return 0;
      return svgk::attn_vt_ws_bytes(dm, a, b);
  }
  return 0;
}

svg_status svg_profile_heads(const svg_dims *dims, svg_dtype dtype, const void *Q, const void *K,
                             const void *V, const int32_t *sample_idx, int32_t n_samples,
                             const svg_mask_params *mask, float softmax_scale, int32_t *labels,
                             float *mse, void *ws, size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (!Q || !K || !V || !sample_idx || !mask || !labels) return fail(SVG_ERR_NULL, "profile: NULL pointer");
  if (n_samples < 1 || n_samples > dm.N) return fail(SVG_ERR_RANGE, "n_samples=%d out of [1, N]", n_samples);
  if (mask->ks_frames < 0 || mask->wt_tokens < 0) return fail(SVG_ERR_RANGE, "mask widths must be >= 0");
  const size_t need = svgk::profile_ws_bytes(dm, n_samples);
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "profile: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(svgk::launch_profile(dm, dtype == SVG_BF16, Q, K, V, sample_idx, n_samples,
                                         mask->ks_frames, mask->wt_tokens,
                                         resolve_scale(softmax_scale, dm.d), labels, mse, ws,
                                         (hipStream_t)stream),
                    "svg_profile_heads");
}

static svg_status layout_common(const svg_dims *dims, svg_dtype dtype, const void *X, void *Y,
                                const int32_t *labels, void *stream, bool inverse) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (!X || !Y) return fail(SVG_ERR_NULL, "layout: NULL tensor");
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * elem_bytes(dtype);
  if (overlaps(X, Y, bytes)) return fail(SVG_ERR_RANGE, "layout: X and Y overlap");
  return hip_status(svgk::launch_layout(dm, elem_bytes(dtype), X, Y, labels, inverse, (hipStream_t)stream),
                    inverse ? "svg_layout_unpermute" : "svg_layout_permute");
}

svg_status svg_layout_permute(const svg_dims *dims, svg_dtype dtype, const void *X, void *Y,
                              const int32_t *labels, void *stream) {
  return layout_common(dims, dtype, X, Y, labels, stream, false);
}

svg_status svg_layout_unpermute(const svg_dims *dims, svg_dtype dtype, const void *X, void *Y,
                                const int32_t *labels, void *stream) {
  return layout_common(dims, dtype, X, Y, labels, stream, true);
}

svg_status svg_build_block_mask(const svg_dims *dims, const svg_mask_params *mask,
                                const int32_t *labels, int32_t bq, int32_t bk, uint8_t *block_mask,
                                void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm)) != SVG_OK) return s;
  if ((s = check_blocks(bq, bk)) != SVG_OK) return s;
  if (!mask || !labels || !block_mask) return fail(SVG_ERR_NULL, "build_block_mask: NULL pointer");
  if (mask->ks_frames < 0 || mask->wt_tokens < 0) return fail(SVG_ERR_RANGE, "mask widths must be >= 0");
  return hip_status(svgk::launch_block_mask(dm, mask->ks_frames, mask->wt_tokens, labels, bq, bk,
                                            block_mask, (hipStream_t)stream),
                    "svg_build_block_mask");
}

svg_status svg_compact_block_mask(int32_t rows, int32_t nkb, const uint8_t *block_mask,
                                  int32_t *row_ptr, int32_t *kv_idx, void *ws, size_t ws_bytes,
                                  void *stream) {
  if (rows < 0 || nkb < 1) return fail(SVG_ERR_SHAPE, "compact: rows=%d nkb=%d", rows, nkb);
  if ((int64_t)rows * nkb >= ((int64_t)1 << 31)) return fail(SVG_ERR_SHAPE, "compact: rows*nkb >= 2^31");
  if (!row_ptr || (rows > 0 && (!block_mask || !kv_idx))) return fail(SVG_ERR_NULL, "compact: NULL pointer");
  const size_t need = svgk::compact_ws_bytes(rows);
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "compact: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(svgk::launch_compact(rows, nkb, block_mask, row_ptr, kv_idx, ws, (hipStream_t)stream),
                    "svg_compact_block_mask");
}

static svg_status attn_checks(const svg_dims *dims, svg_dtype dtype, const void *Q, const void *K,
                              const void *V, const void *O, int bq, int bk, Dims *dm) {
  svg_status s;
  if ((s = check_dims(dims, dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if ((s = check_blocks(bq, bk)) != SVG_OK) return s;
  if (!Q || !K || !V || !O) return fail(SVG_ERR_NULL, "attention: NULL tensor");
  const size_t bytes = (size_t)dm->H * dm->N * dm->d * elem_bytes(dtype);
  if (overlaps(O, Q, bytes) || overlaps(O, K, bytes) || overlaps(O, V, bytes))
    return fail(SVG_ERR_RANGE, "attention: O overlaps an input");
  return SVG_OK;
}

svg_status svg_block_sparse_attn(const svg_dims *dims, svg_dtype dtype, const void *Q, const void *K,
                                 const void *V, const uint8_t *block_mask, int32_t bq, int32_t bk,
                                 float softmax_scale, void *O, void *ws, size_t ws_bytes,
                                 void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = attn_checks(dims, dtype, Q, K, V, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!block_mask) return fail(SVG_ERR_NULL, "block_sparse_attn: block_mask is NULL");
  const int nqb = (dm.N + bq - 1) / bq, nkb = (dm.N + bk - 1) / bk;
  const int64_t rows = (int64_t)dm.H * nqb;
  if (rows * nkb >= ((int64_t)1 << 31)) return fail(SVG_ERR_SHAPE, "block_sparse_attn: H*nQB*nKB >= 2^31");
  const size_t need = block_sparse_ws(dm, bq, bk);
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "block_sparse_attn: workspace %zu < %zu bytes", ws_bytes, need);
  char *w = (char *)ws;
  const size_t c0 = svgk::compact_ws_bytes((int)rows);
  int32_t *row_ptr = (int32_t *)(w + c0);
  int32_t *kv_idx = (int32_t *)(w + c0 + align256((rows + 1) * 4));
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = svgk::launch_compact((int)rows, nkb, block_mask, row_ptr, kv_idx, w, st);
  if (e != hipSuccess) return hip_status(e, "svg_block_sparse_attn (compact)");
  return hip_status(run_attention(dm, dtype, Q, K, V, O, row_ptr, kv_idx, bq, bk,
                                  resolve_scale(softmax_scale, dm.d), st),
                    "svg_block_sparse_attn");
}

svg_status svg_block_sparse_attn_csr(const svg_dims *dims, svg_dtype dtype, const void *Q,
                                     const void *K, const void *V, const int32_t *row_ptr,
                                     const int32_t *kv_idx, int32_t bq, int32_t bk,
                                     float softmax_scale, void *O, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = attn_checks(dims, dtype, Q, K, V, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!row_ptr || !kv_idx) return fail(SVG_ERR_NULL, "block_sparse_attn_csr: NULL list");
  return hip_status(run_attention(dm, dtype, Q, K, V, O, row_ptr, kv_idx, bq, bk,
                                  resolve_scale(softmax_scale, dm.d), (hipStream_t)stream),
                    "svg_block_sparse_attn_csr");
}

svg_status svg_dense_attn(const svg_dims *dims, svg_dtype dtype, const void *Q, const void *K,
                          const void *V, int32_t bq, int32_t bk, float softmax_scale, void *O,
                          void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = attn_checks(dims, dtype, Q, K, V, O, bq, bk, &dm)) != SVG_OK) return s;
  return hip_status(run_attention(dm, dtype, Q, K, V, O, nullptr, nullptr, bq, bk,
                                  resolve_scale(softmax_scale, dm.d), (hipStream_t)stream),
                    "svg_dense_attn");
}

// Key-tiled transposed V (Vt) and the attention entry points that take it.

size_t svg_vt_elems(const svg_dims *dims) {
  if (dims == nullptr || dims->H < 1 || dims->d < 1) return 0;
  const int64_t N = (int64_t)dims->F * dims->S + dims->T;
  if (N < 1) return 0;
  return (size_t)dims->H * (size_t)((N + 63) / 64) * 64 * (size_t)dims->d;
}

svg_status svg_layout_permute_vt(const svg_dims *dims, svg_dtype dtype, const void *V, void *Vt,
                                 const int32_t *labels, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "layout_permute_vt: bf16 only");
  if (!V || !Vt) return fail(SVG_ERR_NULL, "layout_permute_vt: NULL tensor");
  const size_t vbytes = (size_t)dm.H * dm.N * dm.d * 2, tbytes = svg_vt_elems(dims) * 2;
  if (overlaps2(V, vbytes, Vt, tbytes))
    return fail(SVG_ERR_RANGE, "layout_permute_vt: V and Vt overlap");
  return hip_status(svgk::launch_layout_vt(dm, V, Vt, labels, (hipStream_t)stream), "svg_layout_permute_vt");
}

static svg_status vt_checks(const svg_dims *dims, svg_dtype dtype, const void *Q, const void *K,
                            const void *Vt, const void *O, int bq, int bk, Dims *dm) {
  svg_status s;
  if ((s = check_dims(dims, dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "attention on Vt: bf16 only");
  if (bk != 64 || (bq != 64 && bq != 128))
    return fail(SVG_ERR_UNSUPPORTED, "attention on Vt: block shape %dx%d unsupported ((64,64), (128,64))", bq, bk);
  const int64_t nkb = (dm->N + 63) / 64;
  if (nkb > svgk::attn_vt_max_kv_blocks())
    return fail(SVG_ERR_UNSUPPORTED, "attention on Vt: %lld kv-blocks > %d", (long long)nkb,
                svgk::attn_vt_max_kv_blocks());
  if ((int64_t)dm->N * dm->d * 2 >= ((int64_t)1 << 31))
    return fail(SVG_ERR_UNSUPPORTED, "attention on Vt: one head is >= 2 GiB");
  if (!Q || !K || !Vt || !O) return fail(SVG_ERR_NULL, "attention on Vt: NULL tensor");
  const size_t bytes = (size_t)dm->H * dm->N * dm->d * 2, tbytes = svg_vt_elems(dims) * 2;
  if (overlaps(O, Q, bytes) || overlaps(O, K, bytes) || overlaps2(O, bytes, Vt, tbytes))
    return fail(SVG_ERR_RANGE, "attention on Vt: O overlaps an input");
  return SVG_OK;
}

// The split-partials workspace of the sparse V^T entries: NULL (no split),
// or at least attn_vt_ws_bytes and clear of the tensors.
static svg_status attn_ws_check(const Dims &dm, int bq, int bk, const void *Q, const void *K, const void *Vt,
                                const void *O, const void *ws, size_t ws_bytes) {
  if (ws == nullptr) return SVG_OK;
  const size_t need = svgk::attn_vt_ws_bytes(dm, bq, bk);
  if (ws_bytes < need) return fail(SVG_ERR_WORKSPACE, "attention: workspace %zu < %zu bytes", ws_bytes, need);
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * 2;
  const size_t tbytes = (size_t)dm.H * ((dm.N + 63) / 64) * 64 * dm.d * 2;
  if (need > 0 && (overlaps2(ws, need, Q, bytes) || overlaps2(ws, need, K, bytes) ||
                   overlaps2(ws, need, O, bytes) || overlaps2(ws, need, Vt, tbytes)))
    return fail(SVG_ERR_RANGE, "attention: workspace overlaps a tensor");
  return SVG_OK;
}

svg_status svg_block_sparse_attn_csr_vt(const svg_dims *dims, svg_dtype dtype, const void *Q,
                                        const void *K, const void *Vt, const int32_t *row_ptr,
                                        const int32_t *kv_idx, int32_t bq, int32_t bk,
                                        float softmax_scale, void *O, void *ws, size_t ws_bytes,
                                        void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = vt_checks(dims, dtype, Q, K, Vt, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!row_ptr || !kv_idx) return fail(SVG_ERR_NULL, "block_sparse_attn_csr_vt: NULL list");
  if ((s = attn_ws_check(dm, bq, bk, Q, K, Vt, O, ws, ws_bytes)) != SVG_OK) return s;
  return hip_status(svgk::launch_attn_vt(dm, Q, K, Vt, O, row_ptr, kv_idx, bq, bk,
                                         resolve_scale(softmax_scale, dm.d), (hipStream_t)stream, false,
                                         nullptr, ws),
                    "svg_block_sparse_attn_csr_vt");
}

svg_status svg_block_sparse_attn_csr_vt_layout(const svg_dims *dims, svg_dtype dtype, const void *Q,
                                               const void *K, const void *Vt, const int32_t *row_ptr,
                                               const int32_t *kv_idx, const int32_t *labels, int32_t bq,
                                               int32_t bk, float softmax_scale, void *O, void *ws,
                                               size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = vt_checks(dims, dtype, Q, K, Vt, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!row_ptr || !kv_idx) return fail(SVG_ERR_NULL, "block_sparse_attn_csr_vt_layout: NULL list");
  if ((s = attn_ws_check(dm, bq, bk, Q, K, Vt, O, ws, ws_bytes)) != SVG_OK) return s;
  return hip_status(svgk::launch_attn_vt(dm, Q, K, Vt, O, row_ptr, kv_idx, bq, bk,
                                         resolve_scale(softmax_scale, dm.d), (hipStream_t)stream, true, labels,
                                         ws),
                    "svg_block_sparse_attn_csr_vt_layout");
}

svg_status svg_dense_attn_vt(const svg_dims *dims, svg_dtype dtype, const void *Q, const void *K,
                             const void *Vt, int32_t bq, int32_t bk, float softmax_scale, void *O,
                             void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = vt_checks(dims, dtype, Q, K, Vt, O, bq, bk, &dm)) != SVG_OK) return s;
  return hip_status(svgk::launch_attn_vt(dm, Q, K, Vt, O, nullptr, nullptr, bq, bk,
                                         resolve_scale(softmax_scale, dm.d), (hipStream_t)stream),
                    "svg_dense_attn_vt");
}

// ---------------------------------------------------------------------------
// SVG2 path

size_t svg2_workspace_bytes(svg2_op op, const svg_dims *dims, int32_t a, int32_t b) {
  Dims dm{};
  switch (op) {
    case SVG2_OP_KMEANS:
      if (check_dims(dims, &dm, false) != SVG_OK || a < 1) return 0;
      return svgk::kmeans_ws_bytes(dm, a);
    case SVG2_OP_CLUSTER_PERMUTE:
      if (check_dims(dims, &dm, false) != SVG_OK || a < 1) return 0;
      return svgk::cluster_permute_ws_bytes(dm, a);
    case SVG2_OP_VARLEN:
      if (check_dims(dims, &dm, false) != SVG_OK || a < 1 || b < 1) return 0;
      return svgk::varlen_ws_bytes(dm, a, b);
  }
  return 0;
}

svg_status svg_kmeans(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t k, int32_t iters,
                      const int32_t *init_idx, int32_t *assign, double *centroids, int32_t *sizes,
                      void *ws, size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (!X || !init_idx || !assign || !centroids || !sizes) return fail(SVG_ERR_NULL, "kmeans: NULL pointer");
  if (k < 1 || k > 256 || k > dm.N) return fail(SVG_ERR_RANGE, "kmeans: k=%d out of [1, min(256, N)]", k);
  if (iters < 1) return fail(SVG_ERR_RANGE, "kmeans: iters=%d < 1", iters);
  const size_t need = svgk::kmeans_ws_bytes(dm, k);
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "kmeans: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(svgk::launch_kmeans(dm, dtype == SVG_BF16, X, k, iters, init_idx, assign, centroids,
                                        sizes, ws, (hipStream_t)stream),
                    "svg_kmeans");
}

svg_status svg_cluster_permute(const svg_dims *dims, const int32_t *assign, int32_t k, int32_t *perm,
                               int32_t *offs, void *ws, size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if (!assign || !perm || !offs) return fail(SVG_ERR_NULL, "cluster_permute: NULL pointer");
  if (k < 1 || k > 256) return fail(SVG_ERR_RANGE, "cluster_permute: k=%d out of [1, 256]", k);
  const size_t need = svgk::cluster_permute_ws_bytes(dm, k);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(SVG_ERR_WORKSPACE, "cluster_permute: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(svgk::launch_cluster_permute(dm, assign, k, perm, offs, ws, (hipStream_t)stream),
                    "svg_cluster_permute");
}

svg_status svg_permute_rows(const svg_dims *dims, svg_dtype dtype, const void *X, const int32_t *perm,
                            void *Y, int32_t inverse, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (!X || !Y || !perm) return fail(SVG_ERR_NULL, "permute_rows: NULL pointer");
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * elem_bytes(dtype);
  if (overlaps(X, Y, bytes)) return fail(SVG_ERR_RANGE, "permute_rows: X and Y overlap");
  return hip_status(svgk::launch_permute_rows(dm, elem_bytes(dtype), X, perm, Y, inverse != 0,
                                              (hipStream_t)stream),
                    "svg_permute_rows");
}

svg_status svg_select_pairs(const svg_dims *dims, const double *cq, const double *ck,
                            const int32_t *size_k, int32_t kq, int32_t kk, double top_p,
                            float softmax_scale, int32_t *pair_ptr, int32_t *pair_idx, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if (!cq || !ck || !size_k || !pair_ptr || !pair_idx) return fail(SVG_ERR_NULL, "select_pairs: NULL pointer");
  if (kq < 1 || kk < 1 || kk > 256) return fail(SVG_ERR_RANGE, "select_pairs: kq=%d kk=%d (kk <= 256)", kq, kk);
  if (!(top_p > 0.0 && top_p <= 1.0)) return fail(SVG_ERR_RANGE, "select_pairs: top_p=%g not in (0, 1]", top_p);
  return hip_status(svgk::launch_select_pairs(dm, cq, ck, size_k, kq, kk, top_p,
                                              (double)resolve_scale(softmax_scale, dm.d), pair_ptr,
                                              pair_idx, (hipStream_t)stream),
                    "svg_select_pairs");
}

svg_status svg_varlen_attn(const svg_dims *dims, svg_dtype dtype, const void *Qp, const void *Kp,
                           const void *Vp, const int32_t *q_offs, const int32_t *k_offs, int32_t kq,
                           int32_t kk, const int32_t *pair_ptr, const int32_t *pair_idx,
                           const int32_t *q_perm, float softmax_scale, void *O, void *ws,
                           size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (!Qp || !Kp || !Vp || !q_offs || !k_offs || !pair_ptr || !pair_idx || !O)
    return fail(SVG_ERR_NULL, "varlen_attn: NULL pointer");
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "varlen_attn: bf16 inputs only");
  if (kq < 1 || kk < 1 || kk > 256) return fail(SVG_ERR_RANGE, "varlen_attn: kq=%d kk=%d (kk <= 256)", kq, kk);
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * elem_bytes(dtype);
  if (overlaps(O, Qp, bytes) || overlaps(O, Kp, bytes) || overlaps(O, Vp, bytes))
    return fail(SVG_ERR_RANGE, "varlen_attn: O overlaps an input");
  const size_t need = svgk::varlen_ws_bytes(dm, kq, kk);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(SVG_ERR_WORKSPACE, "varlen_attn: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(svgk::launch_varlen(dm, dtype == SVG_BF16, Qp, Kp, Vp, q_offs, k_offs, kq, kk, pair_ptr,
                                        pair_idx, q_perm, resolve_scale(softmax_scale, dm.d), O, ws,
                                        (hipStream_t)stream),
                    "svg_varlen_attn");
}

}  // extern "C"
