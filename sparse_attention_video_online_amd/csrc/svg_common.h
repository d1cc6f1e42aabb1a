// Internal declarations shared by the gfx950 kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace svgk {

typedef uint16_t bf16_t;  // storage type of bf16 tensors (raw bits)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, one L2 each

// Work-group ids are handed to the XCDs round-robin.  Remap so that
// consecutive logical work items land on the same XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblk) {
  const int q = nblk / kNumXcd, r = nblk % kNumXcd;
  const int xcd = bid % kNumXcd, local = bid / kNumXcd;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// exp2 on the hardware transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Launchers (host side).  Each returns the hipError_t of its launches.
struct Dims { int F, S, T, H, d, N; };

hipError_t launch_attn_mfma(const Dims &dm, const void *Q, const void *K, const void *V, void *O,
                            const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk,
                            float scale, hipStream_t st);
hipError_t launch_attn_simt(const Dims &dm, bool bf16, const void *Q, const void *K, const void *V,
                            void *O, const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk,
                            float scale, hipStream_t st);
// qo_orig: Q is read and O written in the original token order, rows
// permuted per labels (NULL: every head) as the layout permute does; K and
// Vt are in the executing layout either way.
hipError_t launch_attn_vt(const Dims &dm, const void *Q, const void *K, const void *Vt, void *O,
                          const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk, float scale,
                          hipStream_t st, bool qo_orig = false, const int32_t *labels = nullptr,
                          void *ws = nullptr);
// The sparse launch with Q, K and O in the original token order (K rows
// gathered by the tile DMA; Vt and the lists in the executing layout).
hipError_t launch_attn_vt_korig(const Dims &dm, const void *Q, const void *K, const void *Vt, void *O,
                                const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk, float scale,
                                const int32_t *labels, void *ws, hipStream_t st);
// Bytes of ws the sparse launch splits its text groups into (0: no split).
size_t attn_vt_ws_bytes(const Dims &dm, int bq, int bk);
int attn_vt_max_kv_blocks();
// Row order of the key-tiled V^T copy:
//   kVtLabels:   each head's executing layout per labels (NULL: every head
//                position-major), as svg_layout_permute;
//   kVtFrames:   every head's token order, each frame and the text starting
//                a new 64-key tile (vt_frame_tiles(dm) tiles a head, zero
//                past each end);
//   kVtIdentity: every head's rows as given;
//   kVtGather:   row r of head h is V row labels[h*N + r] of that head
//                (labels: int32 [H][N] gather index).
enum { kVtLabels = 0, kVtFrames = 1, kVtIdentity = 2, kVtGather = 3 };
hipError_t launch_layout_vt(const Dims &dm, const void *V, void *Vt, const int32_t *labels, hipStream_t st,
                            int mode = kVtLabels);
inline int vt_frame_tiles(const Dims &dm) {
  return dm.F * ((dm.S + 63) / 64) + (dm.T + 63) / 64;
}
// SVG-EAR: block centroids, routing, and the attention with compensation.
int ear_centroid_tiles(const Dims &dm);
int ear_route_qpw(const Dims &dm);
int attn_ear_max_kv_blocks();
hipError_t launch_ear_stats(const Dims &dm, const void *K, const void *Vt, void *Kc, void *Vct, double *kbar,
                            double *rad, hipStream_t st);
hipError_t launch_ear_route(const Dims &dm, const void *Q, const int32_t *labels, const double *kbar,
                            const double *rad, const uint8_t *mask, int bq, int route_k, double tau, uint8_t *exact,
                            hipStream_t st);
hipError_t launch_attn_vt_ear(const Dims &dm, const void *Q, const void *K, const void *Vt, const void *Kc,
                              const void *Vct, void *O, const int32_t *row_ptr, const int32_t *kv_idx, int bq,
                              float scale, const int32_t *labels, hipStream_t st);
// FP8 (E4M3) quantization and attention (d = 128 for the attention).
hipError_t launch_quant_rows_fp8(const Dims &dm, const void *X, void *X8, float *scale, hipStream_t st);
hipError_t launch_layout_fp8(const Dims &dm, const void *X, void *X8, float *scale, const int32_t *labels,
                             hipStream_t st);
// vamax non-null: the FP8 P.V mode (Vt = V^T code tiles of launch_layout_vt_fp8)
hipError_t launch_attn_fp8(const Dims &dm, const void *Q8, const float *qscale, const void *K8, const float *kscale,
                           const void *Vt, const float *vamax, void *O, const int32_t *row_ptr,
                           const int32_t *kv_idx, int bq, float scale, const int32_t *labels, bool qo_orig,
                           hipStream_t st);
// V (d = 128) -> per-channel largest magnitudes vamax [H][128] and the V^T
// code tiles [H][ceil(N/64)][128][64] of the executing layout (per labels)
hipError_t launch_layout_vt_fp8(const Dims &dm, const void *V, void *Vt8, float *vamax, const int32_t *labels,
                                hipStream_t st);
hipError_t launch_layout(const Dims &dm, int elem_bytes, const void *X, void *Y,
                         const int32_t *labels, bool inverse, hipStream_t st);
hipError_t launch_permute_rows(const Dims &dm, int elem_bytes, const void *X, const int32_t *perm,
                               void *Y, bool inverse, hipStream_t st);
hipError_t launch_block_mask(const Dims &dm, int ks, int wt, const int32_t *labels, int bq, int bk,
                             uint8_t *mask, hipStream_t st);
size_t compact_ws_bytes(int rows);
hipError_t launch_compact(int rows, int nkb, const uint8_t *mask, int32_t *row_ptr, int32_t *kv_idx,
                          void *ws, hipStream_t st);
size_t profile_ws_bytes(const Dims &dm, int n_samples);
hipError_t launch_profile(const Dims &dm, bool bf16, const void *Q, const void *K, const void *V,
                          const int32_t *sample_idx, int n_samples, int ks, int wt, float scale,
                          int32_t *labels, float *mse, void *ws, hipStream_t st);
size_t kmeans_ws_bytes(const Dims &dm, int k);
hipError_t launch_kmeans(const Dims &dm, bool bf16, const void *X, int k, int iters,
                         const int32_t *init_idx, int32_t *assign, double *centroids,
                         int32_t *sizes, void *ws, hipStream_t st);
size_t cluster_permute_ws_bytes(const Dims &dm, int k);
hipError_t launch_cluster_permute(const Dims &dm, const int32_t *assign, int k, int32_t *perm,
                                  int32_t *offs, void *ws, hipStream_t st);
hipError_t launch_select_pairs(const Dims &dm, const double *cq, const double *ck,
                               const int32_t *size_k, int kq, int kk, double top_p, double scale,
                               int32_t *pair_ptr, int32_t *pair_idx, hipStream_t st);
size_t varlen_ws_bytes(const Dims &dm, int kq, int kk);
hipError_t launch_varlen(const Dims &dm, bool bf16, const void *Qp, const void *Kp, const void *Vp,
                         const int32_t *q_offs, const int32_t *k_offs, int kq, int kk,
                         const int32_t *pair_ptr, const int32_t *pair_idx, const int32_t *q_perm,
                         float scale, void *O, void *ws, hipStream_t st);
// The same attention on the key-tiled V^T of Vp (d = 64 or 128, at most
// varlen_vt_max_windows() 64-key windows a head); no workspace.
int varlen_vt_max_windows();
bool varlen_vt_covers(const Dims &dm);
hipError_t launch_varlen_vt(const Dims &dm, const void *Qp, const void *Kp, const void *Vt, const int32_t *q_offs,
                            const int32_t *k_offs, int kq, int kk, const int32_t *pair_ptr, const int32_t *pair_idx,
                            const int32_t *q_perm, float scale, void *O, hipStream_t st);

// HVA-style local-window clustering (bf16 inputs, d = 64 or 128).
int hva_clusters(const Dims &dm, int rows, int cols, const int win[3]);
size_t hva_ws_bytes(const Dims &dm, int k);
hipError_t launch_hva_cluster(const Dims &dm, const void *X, int rows, int cols, const int win[3], int iters,
                              float r2, int32_t *assign, double *cent, int32_t *sizes, uint8_t *flags, void *ws,
                              hipStream_t st);
hipError_t launch_hva_refresh(const Dims &dm, const void *X, int rows, int cols, const int win[3],
                              const uint8_t *flags, int32_t *assign, double *cent, int32_t *sizes, void *ws,
                              hipStream_t st);

}  // namespace svgk
