// C ABI: host-side validation, workspace sizing and kernel dispatch.
//
// Every entry point checks its arguments before it touches the HIP runtime.
// A bad call therefore returns a status and enqueues nothing.  The library
// owns no device memory and never synchronises the caller's stream.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

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

// The bf16 block-sparse entries that take row-major V run on the key-tiled
// V^T kernel wherever it covers the shape: V is first transposed into the
// caller's workspace (then the split partials of the text groups follow).
bool vt_covers(const Dims &dm, int bq, int bk) {
  return bk == 64 && (bq == 64 || bq == 128) && (dm.N + 63) / 64 <= svgk::attn_vt_max_kv_blocks() &&
         (int64_t)dm.N * dm.d * 2 < ((int64_t)1 << 31);
}

size_t vt_bytes(const Dims &dm) { return (size_t)dm.H * ((dm.N + 63) / 64) * 64 * dm.d * 2; }

// Vt, then the split partials (0 when the V^T kernel does not cover the shape)
size_t rowmajor_v_ws(const Dims &dm, int bq, int bk) {
  if (!vt_covers(dm, bq, bk)) return 0;
  return align256(vt_bytes(dm)) + align256(svgk::attn_vt_ws_bytes(dm, bq, bk));
}

size_t block_sparse_lists_ws(const Dims &dm, int bq, int bk) {
  const size_t nqb = (dm.N + bq - 1) / bq, nkb = (dm.N + bk - 1) / bk;
  const size_t rows = (size_t)dm.H * nqb;
  return svgk::compact_ws_bytes((int)rows) + align256((rows + 1) * 4) + align256(rows * nkb * 4);
}

// bf16 = false: the fp32 path needs the lists only
size_t block_sparse_ws(const Dims &dm, int bq, int bk, bool bf16 = true) {
  return block_sparse_lists_ws(dm, bq, bk) + (bf16 ? rowmajor_v_ws(dm, bq, bk) : 0);
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

// Scratch of svg_kmeans_noalloc: one copy of this array per GPU, held for
// the life of the process.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address): it looks up
// each device's address once, with that device current, and uses only that.
constexpr size_t kNoallocScratchBytes = (size_t)SVG_KMEANS_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch copy.
hipError_t scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// Row-major V through the V^T kernel: V -> Vt (rows as given) at the start of
// vws, the split partials after it, then the attention.
hipError_t run_attention_vt(const Dims &dm, const void *Q, const void *K, const void *V, void *O,
                            const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk, float scale,
                            void *vws, hipStream_t st) {
  void *vt = vws;
  void *part = svgk::attn_vt_ws_bytes(dm, bq, bk) > 0 ? (char *)vws + align256(vt_bytes(dm)) : nullptr;
  hipError_t e = svgk::launch_layout_vt(dm, V, vt, nullptr, st, svgk::kVtIdentity);
  if (e != hipSuccess) return e;
  return svgk::launch_attn_vt(dm, Q, K, vt, O, row_ptr, kv_idx, bq, bk, scale, st, false, nullptr, part);
}

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
      if (check_dims(dims, &dm, false) != SVG_OK || check_blocks(a, b) != SVG_OK) return 0;
      return block_sparse_ws(dm, a, b);
    case SVG_OP_ATTN_VT:
      if (check_dims(dims, &dm) != SVG_OK) return 0;
      return svgk::attn_vt_ws_bytes(dm, a, b);
    case SVG_OP_ATTN_CSR:
      if (check_dims(dims, &dm, false) != SVG_OK || check_blocks(a, b) != SVG_OK) return 0;
      return rowmajor_v_ws(dm, a, b);
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

// A workspace the library writes must not share a byte with the tensors.
static svg_status ws_clear(const Dims &dm, svg_dtype dtype, size_t need, const void *Q, const void *K,
                           const void *V, const void *O, const void *ws, const char *what) {
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * elem_bytes(dtype);
  if (need > 0 && (overlaps2(ws, need, Q, bytes) || overlaps2(ws, need, K, bytes) ||
                   overlaps2(ws, need, V, bytes) || overlaps2(ws, need, O, bytes)))
    return fail(SVG_ERR_RANGE, "%s: workspace overlaps a tensor", what);
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
  const bool bf16 = dtype == SVG_BF16;
  const size_t need = block_sparse_ws(dm, bq, bk, bf16);
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "block_sparse_attn: workspace %zu < %zu bytes", ws_bytes, need);
  if ((s = ws_clear(dm, dtype, need, Q, K, V, O, ws, "block_sparse_attn")) != SVG_OK) return s;
  char *w = (char *)ws;
  const size_t c0 = svgk::compact_ws_bytes((int)rows);
  int32_t *row_ptr = (int32_t *)(w + c0);
  int32_t *kv_idx = (int32_t *)(w + c0 + align256((rows + 1) * 4));
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = svgk::launch_compact((int)rows, nkb, block_mask, row_ptr, kv_idx, w, st);
  if (e != hipSuccess) return hip_status(e, "svg_block_sparse_attn (compact)");
  const float scale = resolve_scale(softmax_scale, dm.d);
  if (bf16 && vt_covers(dm, bq, bk))
    return hip_status(run_attention_vt(dm, Q, K, V, O, row_ptr, kv_idx, bq, bk, scale,
                                       w + block_sparse_lists_ws(dm, bq, bk), st),
                      "svg_block_sparse_attn");
  return hip_status(run_attention(dm, dtype, Q, K, V, O, row_ptr, kv_idx, bq, bk, scale, st),
                    "svg_block_sparse_attn");
}

svg_status svg_block_sparse_attn_csr(const svg_dims *dims, svg_dtype dtype, const void *Q,
                                     const void *K, const void *V, const int32_t *row_ptr,
                                     const int32_t *kv_idx, int32_t bq, int32_t bk,
                                     float softmax_scale, void *O, void *ws, size_t ws_bytes,
                                     void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = attn_checks(dims, dtype, Q, K, V, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!row_ptr || !kv_idx) return fail(SVG_ERR_NULL, "block_sparse_attn_csr: NULL list");
  const float scale = resolve_scale(softmax_scale, dm.d);
  hipStream_t st = (hipStream_t)stream;
  if (ws != nullptr && dtype == SVG_BF16 && vt_covers(dm, bq, bk)) {
    const size_t need = rowmajor_v_ws(dm, bq, bk);
    if (ws_bytes < need)
      return fail(SVG_ERR_WORKSPACE, "block_sparse_attn_csr: workspace %zu < %zu bytes", ws_bytes, need);
    if ((s = ws_clear(dm, dtype, need, Q, K, V, O, ws, "block_sparse_attn_csr")) != SVG_OK) return s;
    return hip_status(run_attention_vt(dm, Q, K, V, O, row_ptr, kv_idx, bq, bk, scale, ws, st),
                      "svg_block_sparse_attn_csr");
  }
  return hip_status(run_attention(dm, dtype, Q, K, V, O, row_ptr, kv_idx, bq, bk, scale, st),
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

svg_status svg_block_sparse_attn_csr_vt_fused(const svg_dims *dims, svg_dtype dtype, const void *Q,
                                              const void *K, const void *Vt, const int32_t *row_ptr,
                                              const int32_t *kv_idx, const int32_t *labels, int32_t bq,
                                              int32_t bk, float softmax_scale, void *O, void *ws,
                                              size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = vt_checks(dims, dtype, Q, K, Vt, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!row_ptr || !kv_idx) return fail(SVG_ERR_NULL, "block_sparse_attn_csr_vt_fused: NULL list");
  if ((s = attn_ws_check(dm, bq, bk, Q, K, Vt, O, ws, ws_bytes)) != SVG_OK) return s;
  return hip_status(svgk::launch_attn_vt_korig(dm, Q, K, Vt, O, row_ptr, kv_idx, bq, bk,
                                               resolve_scale(softmax_scale, dm.d), labels, ws,
                                               (hipStream_t)stream),
                    "svg_block_sparse_attn_csr_vt_fused");
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
// SVG-EAR

size_t svg_ear_centroid_elems(const svg_dims *dims) {
  Dims dm{};
  if (check_dims(dims, &dm, false) != SVG_OK) return 0;
  return (size_t)dm.H * svgk::ear_centroid_tiles(dm) * 64 * dm.d;
}

svg_status svg_ear_block_stats(const svg_dims *dims, svg_dtype dtype, const void *K, const void *Vt, void *Kc,
                               void *Vct, double *kbar, double *radius, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "ear_block_stats: bf16 only");
  if (!K || !Vt || !Kc || !Vct || !kbar || !radius) return fail(SVG_ERR_NULL, "ear_block_stats: NULL pointer");
  const size_t kb = (size_t)dm.H * dm.N * dm.d * 2, cb = svg_ear_centroid_elems(dims) * 2;
  if (overlaps2(Kc, cb, K, kb) || overlaps2(Kc, cb, Vt, vt_bytes(dm)) || overlaps2(Vct, cb, K, kb) ||
      overlaps2(Vct, cb, Vt, vt_bytes(dm)) || overlaps2(Kc, cb, Vct, cb))
    return fail(SVG_ERR_RANGE, "ear_block_stats: outputs overlap the inputs or each other");
  return hip_status(svgk::launch_ear_stats(dm, K, Vt, Kc, Vct, kbar, radius, (hipStream_t)stream),
                    "svg_ear_block_stats");
}

svg_status svg_ear_route(const svg_dims *dims, svg_dtype dtype, const void *Q, const int32_t *labels,
                         const double *kbar, const double *radius, const uint8_t *block_mask, int32_t bq, int32_t bk,
                         int32_t route_k, float softmax_scale, uint8_t *exact_mask, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "ear_route: bf16 only");
  if (bk != 64 || (bq != 64 && bq != 128))
    return fail(SVG_ERR_UNSUPPORTED, "ear_route: block shape %dx%d unsupported ((64,64), (128,64))", bq, bk);
  if (!Q || !kbar || !radius || !block_mask || !exact_mask) return fail(SVG_ERR_NULL, "ear_route: NULL pointer");
  if (route_k < 0) return fail(SVG_ERR_RANGE, "ear_route: route_k=%d < 0", route_k);
  if (svgk::ear_route_qpw(dm) < 1) return fail(SVG_ERR_UNSUPPORTED, "ear_route: too many kv-blocks");
  const size_t mb = (size_t)dm.H * ((dm.N + bq - 1) / bq) * ((dm.N + 63) / 64);
  if (overlaps2(exact_mask, mb, block_mask, mb)) return fail(SVG_ERR_RANGE, "ear_route: exact_mask overlaps block_mask");
  return hip_status(svgk::launch_ear_route(dm, Q, labels, kbar, radius, block_mask, bq, route_k,
                                           (double)resolve_scale(softmax_scale, dm.d), exact_mask,
                                           (hipStream_t)stream),
                    "svg_ear_route");
}

svg_status svg_block_sparse_attn_ear_vt_layout(const svg_dims *dims, svg_dtype dtype, const void *Q, const void *K,
                                               const void *Vt, const void *Kc, const void *Vct,
                                               const int32_t *row_ptr, const int32_t *kv_idx,
                                               const int32_t *labels, int32_t bq, int32_t bk,
                                               float softmax_scale, void *O, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = vt_checks(dims, dtype, Q, K, Vt, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!Kc || !Vct) return fail(SVG_ERR_NULL, "block_sparse_attn_ear: NULL centroid table");
  if (!row_ptr || !kv_idx) return fail(SVG_ERR_NULL, "block_sparse_attn_ear: NULL list");
  if ((dm.N + 63) / 64 > svgk::attn_ear_max_kv_blocks())
    return fail(SVG_ERR_UNSUPPORTED, "block_sparse_attn_ear: more than %d kv-blocks", svgk::attn_ear_max_kv_blocks());
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * 2, cb = svg_ear_centroid_elems(dims) * 2;
  if (overlaps2(O, bytes, Kc, cb) || overlaps2(O, bytes, Vct, cb))
    return fail(SVG_ERR_RANGE, "block_sparse_attn_ear: O overlaps a centroid table");
  return hip_status(svgk::launch_attn_vt_ear(dm, Q, K, Vt, Kc, Vct, O, row_ptr, kv_idx, bq,
                                             resolve_scale(softmax_scale, dm.d), labels, (hipStream_t)stream),
                    "svg_block_sparse_attn_ear_vt_layout");
}

// ---------------------------------------------------------------------------
// FP8 attention

svg_status svg_quantize_fp8_rows(const svg_dims *dims, svg_dtype dtype, const void *X, uint8_t *X8, float *scale,
                                 void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "quantize_fp8_rows: bf16 inputs only");
  if (!X || !X8 || !scale) return fail(SVG_ERR_NULL, "quantize_fp8_rows: NULL pointer");
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * 2;
  if (overlaps2(X, bytes, X8, bytes / 2) || overlaps2(X, bytes, scale, (size_t)dm.H * dm.N * 4))
    return fail(SVG_ERR_RANGE, "quantize_fp8_rows: outputs overlap X");
  return hip_status(svgk::launch_quant_rows_fp8(dm, X, X8, scale, (hipStream_t)stream), "svg_quantize_fp8_rows");
}

svg_status svg_layout_permute_fp8(const svg_dims *dims, svg_dtype dtype, const void *X, uint8_t *X8, float *scale,
                                  const int32_t *labels, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "layout_permute_fp8: bf16 inputs only");
  if (!X || !X8 || !scale) return fail(SVG_ERR_NULL, "layout_permute_fp8: NULL pointer");
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * 2;
  if (overlaps2(X, bytes, X8, bytes / 2) || overlaps2(X, bytes, scale, (size_t)dm.H * ((dm.N + 63) / 64) * 4))
    return fail(SVG_ERR_RANGE, "layout_permute_fp8: outputs overlap X");
  return hip_status(svgk::launch_layout_fp8(dm, X, X8, scale, labels, (hipStream_t)stream), "svg_layout_permute_fp8");
}

// vt_div: 1 for bf16 V^T tiles, 2 for the V^T code tiles of the P.V mode
static svg_status fp8_attn_checks(const svg_dims *dims, const void *Q8, const float *qscale, const void *K8,
                                  const float *kscale, const void *Vt, const void *O, int bq, int bk, Dims *dm,
                                  int vt_div = 1) {
  svg_status s;
  if ((s = check_dims(dims, dm, false)) != SVG_OK) return s;
  if (dm->d != 128) return fail(SVG_ERR_UNSUPPORTED, "fp8 attention: head dim %d unsupported (128)", dm->d);
  if (bk != 64 || (bq != 64 && bq != 128))
    return fail(SVG_ERR_UNSUPPORTED, "fp8 attention: block shape %dx%d unsupported ((64,64), (128,64))", bq, bk);
  if ((dm->N + 63) / 64 > svgk::attn_vt_max_kv_blocks())
    return fail(SVG_ERR_UNSUPPORTED, "fp8 attention: more than %d kv-blocks", svgk::attn_vt_max_kv_blocks());
  if ((int64_t)dm->N * dm->d * 2 >= ((int64_t)1 << 31))
    return fail(SVG_ERR_UNSUPPORTED, "fp8 attention: one head is >= 2 GiB");
  if (!Q8 || !qscale || !K8 || !kscale || !Vt || !O) return fail(SVG_ERR_NULL, "fp8 attention: NULL pointer");
  const size_t obytes = (size_t)dm->H * dm->N * dm->d * 2;
  if (overlaps2(O, obytes, Q8, obytes / 2) || overlaps2(O, obytes, K8, obytes / 2) ||
      overlaps2(O, obytes, Vt, vt_bytes(*dm) / vt_div))
    return fail(SVG_ERR_RANGE, "fp8 attention: O overlaps an input");
  return SVG_OK;
}

svg_status svg_block_sparse_attn_fp8_vt_layout(const svg_dims *dims, const uint8_t *Q8, const float *qscale,
                                               const uint8_t *K8, const float *kscale, const void *Vt,
                                               const int32_t *row_ptr, const int32_t *kv_idx,
                                               const int32_t *labels, int32_t bq, int32_t bk,
                                               float softmax_scale, void *O, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = fp8_attn_checks(dims, Q8, qscale, K8, kscale, Vt, O, bq, bk, &dm)) != SVG_OK) return s;
  if (!row_ptr || !kv_idx) return fail(SVG_ERR_NULL, "block_sparse_attn_fp8_vt_layout: NULL list");
  return hip_status(svgk::launch_attn_fp8(dm, Q8, qscale, K8, kscale, Vt, nullptr, O, row_ptr, kv_idx, bq,
                                          resolve_scale(softmax_scale, dm.d), labels, true, (hipStream_t)stream),
                    "svg_block_sparse_attn_fp8_vt_layout");
}

svg_status svg_dense_attn_fp8_vt(const svg_dims *dims, const uint8_t *Q8, const float *qscale, const uint8_t *K8,
                                 const float *kscale, const void *Vt, int32_t bq, int32_t bk, float softmax_scale,
                                 void *O, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = fp8_attn_checks(dims, Q8, qscale, K8, kscale, Vt, O, bq, bk, &dm)) != SVG_OK) return s;
  return hip_status(svgk::launch_attn_fp8(dm, Q8, qscale, K8, kscale, Vt, nullptr, O, nullptr, nullptr, bq,
                                          resolve_scale(softmax_scale, dm.d), nullptr, false, (hipStream_t)stream),
                    "svg_dense_attn_fp8_vt");
}

svg_status svg_layout_permute_vt_fp8(const svg_dims *dims, svg_dtype dtype, const void *V, uint8_t *Vt8,
                                     float *vamax, const int32_t *labels, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "layout_permute_vt_fp8: bf16 inputs only");
  if (dm.d != 128) return fail(SVG_ERR_UNSUPPORTED, "layout_permute_vt_fp8: head dim %d unsupported (128)", dm.d);
  if (!V || !Vt8 || !vamax) return fail(SVG_ERR_NULL, "layout_permute_vt_fp8: NULL pointer");
  const size_t vbytes = (size_t)dm.H * dm.N * dm.d * 2, tbytes = vt_bytes(dm) / 2;
  if (overlaps2(Vt8, tbytes, V, vbytes) || overlaps2(vamax, (size_t)dm.H * dm.d * 4, V, vbytes) ||
      overlaps2(vamax, (size_t)dm.H * dm.d * 4, Vt8, tbytes))
    return fail(SVG_ERR_RANGE, "layout_permute_vt_fp8: buffers overlap");
  return hip_status(svgk::launch_layout_vt_fp8(dm, V, Vt8, vamax, labels, (hipStream_t)stream),
                    "svg_layout_permute_vt_fp8");
}

svg_status svg_block_sparse_attn_fp8pv_vt_layout(const svg_dims *dims, const uint8_t *Q8, const float *qscale,
                                                 const uint8_t *K8, const float *kscale, const uint8_t *Vt8,
                                                 const float *vamax, const int32_t *row_ptr,
                                                 const int32_t *kv_idx, const int32_t *labels, int32_t bq,
                                                 int32_t bk, float softmax_scale, void *O, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = fp8_attn_checks(dims, Q8, qscale, K8, kscale, Vt8, O, bq, bk, &dm, 2)) != SVG_OK) return s;
  if (!row_ptr || !kv_idx || !vamax) return fail(SVG_ERR_NULL, "block_sparse_attn_fp8pv_vt_layout: NULL pointer");
  if (overlaps2(O, (size_t)dm.H * dm.N * dm.d * 2, vamax, (size_t)dm.H * dm.d * 4))
    return fail(SVG_ERR_RANGE, "block_sparse_attn_fp8pv_vt_layout: O overlaps vamax");
  return hip_status(svgk::launch_attn_fp8(dm, Q8, qscale, K8, kscale, Vt8, vamax, O, row_ptr, kv_idx, bq,
                                          resolve_scale(softmax_scale, dm.d), labels, true, (hipStream_t)stream),
                    "svg_block_sparse_attn_fp8pv_vt_layout");
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
    case SVG2_OP_HVA:
      if (check_dims(dims, &dm, false) != SVG_OK || a < 1) return 0;
      return svgk::hva_ws_bytes(dm, a);
  }
  return 0;
}

static svg_status kmeans_checks(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t k, int32_t iters,
                                const int32_t *init_idx, int32_t *assign, double *centroids, int32_t *sizes,
                                Dims *dm) {
  svg_status s;
  if ((s = check_dims(dims, dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (!X || !init_idx || !assign || !centroids || !sizes) return fail(SVG_ERR_NULL, "kmeans: NULL pointer");
  if (k < 1 || k > 256 || k > dm->N) return fail(SVG_ERR_RANGE, "kmeans: k=%d out of [1, min(256, N)]", k);
  if (iters < 1) return fail(SVG_ERR_RANGE, "kmeans: iters=%d < 1", iters);
  return SVG_OK;
}

svg_status svg_kmeans(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t k, int32_t iters,
                      const int32_t *init_idx, int32_t *assign, double *centroids, int32_t *sizes,
                      void *ws, size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = kmeans_checks(dims, dtype, X, k, iters, init_idx, assign, centroids, sizes, &dm)) != SVG_OK) return s;
  const size_t need = svgk::kmeans_ws_bytes(dm, k);
  if (ws == nullptr || ws_bytes < need)
    return fail(SVG_ERR_WORKSPACE, "kmeans: workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(svgk::launch_kmeans(dm, dtype == SVG_BF16, X, k, iters, init_idx, assign, centroids,
                                        sizes, ws, (hipStream_t)stream),
                    "svg_kmeans");
}

svg_status svg_kmeans_noalloc(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t k, int32_t iters,
                              const int32_t *init_idx, int32_t *assign, double *centroids, int32_t *sizes,
                              void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = kmeans_checks(dims, dtype, X, k, iters, init_idx, assign, centroids, sizes, &dm)) != SVG_OK) return s;
  const size_t need = svgk::kmeans_ws_bytes(dm, k);
  if (need > kNoallocScratchBytes)
    return fail(SVG_ERR_WORKSPACE, "kmeans_noalloc: needs %zu bytes of scratch, the library holds %zu", need,
                kNoallocScratchBytes);
  void *ws = nullptr;
  hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return hip_status(e, "svg_kmeans_noalloc (scratch address)");
  // Every scratch word the kernels read is written earlier in the same call
  // (the sort counts are zeroed by the first table kernel or fully written
  // by the counting pass), so a previous call's contents do not matter.
  return hip_status(svgk::launch_kmeans(dm, dtype == SVG_BF16, X, k, iters, init_idx, assign, centroids,
                                        sizes, ws, (hipStream_t)stream),
                    "svg_kmeans_noalloc");
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

static svg_status hva_geometry(const svg_dims *dims, int32_t rows, int32_t cols, const int32_t *win, Dims *dm) {
  svg_status s;
  if ((s = check_dims(dims, dm)) != SVG_OK) return s;
  if (!win) return fail(SVG_ERR_NULL, "hva: NULL window");
  if (rows < 1 || cols < 1 || (int64_t)rows * cols != dm->S)
    return fail(SVG_ERR_SHAPE, "hva: rows=%d cols=%d do not tile S=%d", rows, cols, dm->S);
  if (win[0] < 1 || win[1] < 1 || win[2] < 1)
    return fail(SVG_ERR_RANGE, "hva: window %dx%dx%d", win[0], win[1], win[2]);
  return SVG_OK;
}

static svg_status hva_checks(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t rows, int32_t cols,
                             const int32_t *win, Dims *dm) {
  svg_status s;
  if ((s = hva_geometry(dims, rows, cols, win, dm)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "hva: bf16 inputs only");
  if (!X) return fail(SVG_ERR_NULL, "hva: NULL X");
  return SVG_OK;
}

int32_t svg_hva_clusters(const svg_dims *dims, int32_t rows, int32_t cols, const int32_t win[3]) {
  Dims dm{};
  if (hva_geometry(dims, rows, cols, win, &dm) != SVG_OK) return 0;
  const int64_t k = svgk::hva_clusters(dm, rows, cols, win);
  return k > (int64_t)INT32_MAX ? 0 : (int32_t)k;
}

svg_status svg_hva_cluster(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t rows, int32_t cols,
                           const int32_t win[3], int32_t iters, float lowe_r2, int32_t *assign, double *centroids,
                           int32_t *sizes, uint8_t *refresh, void *ws, size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = hva_checks(dims, dtype, X, rows, cols, win, &dm)) != SVG_OK) return s;
  if (!assign || !centroids || !sizes || !refresh) return fail(SVG_ERR_NULL, "hva_cluster: NULL pointer");
  if (iters < 1) return fail(SVG_ERR_RANGE, "hva_cluster: iters=%d < 1", iters);
  if (!(lowe_r2 >= 0.f && lowe_r2 <= 1.f)) return fail(SVG_ERR_RANGE, "hva_cluster: lowe_r2=%g not in [0, 1]", lowe_r2);
  const int k = svgk::hva_clusters(dm, rows, cols, win);
  const size_t need = svgk::hva_ws_bytes(dm, k);
  if (ws_bytes < need || ws == nullptr)
    return fail(SVG_ERR_WORKSPACE, "hva_cluster: workspace %zu < %zu bytes", ws_bytes, need);
  const size_t xb = (size_t)dm.H * dm.N * dm.d * 2, ab = (size_t)dm.H * dm.N * 4, rb = (size_t)dm.H * dm.N;
  const size_t cb = (size_t)dm.H * k * dm.d * 8, sb = (size_t)dm.H * k * 4;
  const void *outs[4] = {assign, centroids, sizes, refresh};
  const size_t ob[4] = {ab, cb, sb, rb};
  for (int i = 0; i < 4; ++i) {
    if (overlaps2(outs[i], ob[i], X, xb) || overlaps2(outs[i], ob[i], ws, need))
      return fail(SVG_ERR_RANGE, "hva_cluster: an output overlaps X or ws");
    for (int j = i + 1; j < 4; ++j)
      if (overlaps2(outs[i], ob[i], outs[j], ob[j])) return fail(SVG_ERR_RANGE, "hva_cluster: outputs overlap");
  }
  return hip_status(svgk::launch_hva_cluster(dm, X, rows, cols, win, iters, lowe_r2, assign, centroids, sizes,
                                             refresh, ws, (hipStream_t)stream),
                    "svg_hva_cluster");
}

svg_status svg_hva_refresh(const svg_dims *dims, svg_dtype dtype, const void *X, int32_t rows, int32_t cols,
                           const int32_t win[3], const uint8_t *refresh, int32_t *assign, double *centroids,
                           int32_t *sizes, void *ws, size_t ws_bytes, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = hva_checks(dims, dtype, X, rows, cols, win, &dm)) != SVG_OK) return s;
  if (!assign || !centroids || !sizes || !refresh) return fail(SVG_ERR_NULL, "hva_refresh: NULL pointer");
  const int k = svgk::hva_clusters(dm, rows, cols, win);
  const size_t need = svgk::hva_ws_bytes(dm, k);
  if (ws_bytes < need || ws == nullptr)
    return fail(SVG_ERR_WORKSPACE, "hva_refresh: workspace %zu < %zu bytes", ws_bytes, need);
  const size_t xb = (size_t)dm.H * dm.N * dm.d * 2, ab = (size_t)dm.H * dm.N * 4, rb = (size_t)dm.H * dm.N;
  const size_t cb = (size_t)dm.H * k * dm.d * 8, sb = (size_t)dm.H * k * 4;
  const void *outs[3] = {assign, centroids, sizes};
  const size_t ob[3] = {ab, cb, sb};
  for (int i = 0; i < 3; ++i) {
    if (overlaps2(outs[i], ob[i], X, xb) || overlaps2(outs[i], ob[i], ws, need) ||
        overlaps2(outs[i], ob[i], refresh, rb))
      return fail(SVG_ERR_RANGE, "hva_refresh: an output overlaps X, refresh or ws");
    for (int j = i + 1; j < 3; ++j)
      if (overlaps2(outs[i], ob[i], outs[j], ob[j])) return fail(SVG_ERR_RANGE, "hva_refresh: outputs overlap");
  }
  return hip_status(svgk::launch_hva_refresh(dm, X, rows, cols, win, refresh, assign, centroids, sizes, ws,
                                             (hipStream_t)stream),
                    "svg_hva_refresh");
}

svg_status svg_permute_rows_vt(const svg_dims *dims, svg_dtype dtype, const void *V, const int32_t *perm,
                               void *Vt, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "permute_rows_vt: bf16 only");
  if (!V || !perm || !Vt) return fail(SVG_ERR_NULL, "permute_rows_vt: NULL pointer");
  if (overlaps2(V, (size_t)dm.H * dm.N * dm.d * 2, Vt, vt_bytes(dm)))
    return fail(SVG_ERR_RANGE, "permute_rows_vt: V and Vt overlap");
  return hip_status(svgk::launch_layout_vt(dm, V, Vt, perm, (hipStream_t)stream, svgk::kVtGather),
                    "svg_permute_rows_vt");
}

svg_status svg_varlen_attn_vt(const svg_dims *dims, svg_dtype dtype, const void *Qp, const void *Kp,
                              const void *Vt, const int32_t *q_offs, const int32_t *k_offs, int32_t kq,
                              int32_t kk, const int32_t *pair_ptr, const int32_t *pair_idx,
                              const int32_t *q_perm, float softmax_scale, void *O, void *stream) {
  Dims dm{};
  svg_status s;
  if ((s = check_dims(dims, &dm, false)) != SVG_OK) return s;
  if ((s = check_dtype(dtype)) != SVG_OK) return s;
  if (!Qp || !Kp || !Vt || !q_offs || !k_offs || !pair_ptr || !pair_idx || !O)
    return fail(SVG_ERR_NULL, "varlen_attn_vt: NULL pointer");
  if (dtype != SVG_BF16) return fail(SVG_ERR_UNSUPPORTED, "varlen_attn_vt: bf16 inputs only");
  if (kq < 1 || kk < 1 || kk > 256) return fail(SVG_ERR_RANGE, "varlen_attn_vt: kq=%d kk=%d (kk <= 256)", kq, kk);
  if (!svgk::varlen_vt_covers(dm))
    return fail(SVG_ERR_UNSUPPORTED, "varlen_attn_vt: d=%d N=%d (d = 64 or 128, N <= %d)", dm.d, dm.N,
                64 * svgk::varlen_vt_max_windows());
  const size_t bytes = (size_t)dm.H * dm.N * dm.d * 2;
  if (overlaps(O, Qp, bytes) || overlaps(O, Kp, bytes) || overlaps2(O, bytes, Vt, vt_bytes(dm)))
    return fail(SVG_ERR_RANGE, "varlen_attn_vt: O overlaps an input");
  return hip_status(svgk::launch_varlen_vt(dm, Qp, Kp, Vt, q_offs, k_offs, kq, kk, pair_ptr, pair_idx, q_perm,
                                           resolve_scale(softmax_scale, dm.d), O, (hipStream_t)stream),
                    "svg_varlen_attn_vt");
}

}  // extern "C"
