// Block-sparse attention on the vector ALUs, fp32 accumulate.  It serves
// fp32 inputs, and small block shapes for which the MFMA tiling does not
// apply.
//
// One work-group per (head, q-block), one thread per query row.  Each kept
// kv-block is staged in LDS as fp32.  Every thread then walks the tile's
// keys with a per-key online softmax (running max, running sum, rescaled
// accumulator), all in fp32.
#include "svg_common.h"

namespace svgk {
namespace {

constexpr int kMaxBk = 64;

template <typename T, int D>
__global__ __launch_bounds__(128)
void attn_fwd_simt(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                   T *__restrict__ O, const int32_t *__restrict__ row_ptr,
                   const int32_t *__restrict__ kv_idx, int N, int nqb, int nkb, int bq, int bk,
                   float c) {
  __shared__ float Ks[kMaxBk][D];
  __shared__ float Vs[kMaxBk][D];
  const int h = blockIdx.y, qb = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t hoff = (size_t)h * N * D;
  const int row = qb * bq + tid;
  const bool active = tid < bq && row < N;

  float q[D];
  float o[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    q[i] = active ? to_f32<T>(Q[hoff + (size_t)row * D + i]) : 0.f;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int t0 = 0, t1 = nkb;
  if (row_ptr != nullptr) {
    t0 = row_ptr[h * nqb + qb];
    t1 = row_ptr[h * nqb + qb + 1];
  }
  for (int t = t0; t < t1; ++t) {
    const int kb = (row_ptr != nullptr) ? kv_idx[t] : t;
    const int k0 = kb * bk;
    const int nk = min(bk, N - k0);
    __syncthreads();
    for (int e = tid; e < nk * D; e += blockDim.x) {
      const int j = e / D, i = e - j * D;
      Ks[j][i] = to_f32<T>(K[hoff + (size_t)(k0 + j) * D + i]);
      Vs[j][i] = to_f32<T>(V[hoff + (size_t)(k0 + j) * D + i]);
    }
    __syncthreads();
    if (active) {
      for (int j = 0; j < nk; ++j) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < D; ++i) s = __builtin_fmaf(q[i], Ks[j][i], s);
        const float mn = fmaxf(m, s);
        const float corr = fast_exp2((m - mn) * c);
        const float p = fast_exp2((s - mn) * c);
        l = l * corr + p;
#pragma unroll
        for (int i = 0; i < D; ++i) o[i] = __builtin_fmaf(o[i], corr, p * Vs[j][i]);
        m = mn;
      }
    }
  }
  if (active) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) O[hoff + (size_t)row * D + i] = from_f32<T>(o[i] * inv);
  }
}

template <typename T, int D>
hipError_t launch_t(const Dims &dm, const void *Q, const void *K, const void *V, void *O,
                    const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk, float c,
                    hipStream_t st) {
  const int nqb = (dm.N + bq - 1) / bq, nkb = (dm.N + bk - 1) / bk;
  if (nqb == 0 || dm.H == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_simt<T, D>), dim3(nqb, dm.H), dim3(bq), 0, st, (const T *)Q,
                     (const T *)K, (const T *)V, (T *)O, row_ptr, kv_idx, dm.N, nqb, nkb, bq, bk, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_simt(const Dims &dm, bool bf16, const void *Q, const void *K, const void *V,
                            void *O, const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk,
                            float scale, hipStream_t st) {
  const float c = scale * kLog2e;
  if (bk > kMaxBk || bq > 128) return hipErrorInvalidValue;
  if (bf16) {
    if (dm.d == 64) return launch_t<bf16_t, 64>(dm, Q, K, V, O, row_ptr, kv_idx, bq, bk, c, st);
    if (dm.d == 128) return launch_t<bf16_t, 128>(dm, Q, K, V, O, row_ptr, kv_idx, bq, bk, c, st);
  } else {
    if (dm.d == 64) return launch_t<float, 64>(dm, Q, K, V, O, row_ptr, kv_idx, bq, bk, c, st);
    if (dm.d == 128) return launch_t<float, 128>(dm, Q, K, V, O, row_ptr, kv_idx, bq, bk, c, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace svgk
