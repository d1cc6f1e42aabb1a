// Online head profiling on sampled query rows (vector-ALU version, used for
// fp32 inputs; bf16 inputs go to the MFMA profiler in profile_mfma.hip).
//
// The SVG1 abstract: an online profiling strategy predicts whether each head
// is spatial or temporal.  The project write-up ("Three generations"):
// patterns are identified dynamically, at run time.  The test, as read here:
//   - for each sampled row, compute the full attention output and the
//     spatial- and temporal-masked outputs.  Each masked softmax runs over its
//     own kept keys with its own running maximum.
//   - take the per-head mean squared error of each masked output against the
//     full one;
//   - the smaller error names the head (ties -> spatial).
//
// Pass kernel: one thread per (head, sampled row, output kind).  The thread
// walks all N keys with a per-key online softmax in fp32, skipping keys
// outside its mask.  All threads of a wave read the same key row at once
// (a broadcast load).
// Reduction kernel: one work-group per head.  It sums the squared errors
// in fp64 in a fixed order, so repeated runs give identical bits.
#include "svg_common.h"

namespace svgk {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(64)
void profile_pass(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
                  const int32_t *__restrict__ sample_idx, int n_s, int F, int S, int N, int ks,
                  int wt, float c, float *__restrict__ out /* [3][H][n_s][D] */, int H) {
  const int h = blockIdx.y, kind = blockIdx.z;
  const int sidx = blockIdx.x * 64 + threadIdx.x;
  if (sidx >= n_s) return;
  const int FS = F * S;
  const int i = sample_idx[sidx];
  const size_t hoff = (size_t)h * N * D;
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = to_f32<T>(Q[hoff + (size_t)i * D + e]);
    o[e] = 0.f;
  }
  const bool text_i = i >= FS;
  const int fi = text_i ? 0 : i / S;
  const int pi = text_i ? 0 : i - fi * S;
  const int64_t tlo = (int64_t)pi * F - wt, thi = (int64_t)pi * F + F - 1 + wt;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j < N; ++j) {
    bool keep = true;
    if (kind != 0 && !text_i && j < FS) {
      const int fj = j / S;
      if (kind == 1) {
        keep = abs(fj - fi) <= ks;
      } else {
        const int64_t rj = (int64_t)(j - fj * S) * F + fj;
        keep = rj >= tlo && rj <= thi;
      }
    }
    if (!keep) continue;
    const T *kr = K + hoff + (size_t)j * D;
    const T *vr = V + hoff + (size_t)j * D;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) s = __builtin_fmaf(q[e], to_f32<T>(kr[e]), s);
    const float mn = fmaxf(m, s);
    const float corr = fast_exp2((m - mn) * c);
    const float p = fast_exp2((s - mn) * c);
    l = l * corr + p;
#pragma unroll
    for (int e = 0; e < D; ++e) o[e] = __builtin_fmaf(o[e], corr, p * to_f32<T>(vr[e]));
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float *dst = out + (((size_t)kind * H + h) * n_s + sidx) * D;
#pragma unroll
  for (int e = 0; e < D; ++e) dst[e] = o[e] * inv;
}

__global__ __launch_bounds__(256)
void profile_reduce(const float *__restrict__ outs, int H, int n_s, int D,
                    int32_t *__restrict__ labels, float *__restrict__ mse) {
  __shared__ double red[2][256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const size_t per = (size_t)n_s * D;
  const float *of = outs + ((size_t)0 * H + h) * per;
  const float *os = outs + ((size_t)1 * H + h) * per;
  const float *ot = outs + ((size_t)2 * H + h) * per;
  double a = 0.0, b = 0.0;
  for (size_t e = tid; e < per; e += 256) {
    const double f = of[e];
    const double ds = (double)os[e] - f, dt = (double)ot[e] - f;
    a += ds * ds;
    b += dt * dt;
  }
  red[0][tid] = a;
  red[1][tid] = b;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double ms = red[0][0] / (double)per, mt = red[1][0] / (double)per;
    labels[h] = ms <= mt ? 0 : 1;
    if (mse != nullptr) {
      mse[2 * h] = (float)ms;
      mse[2 * h + 1] = (float)mt;
    }
  }
}

template <typename T, int D>
hipError_t launch_t(const Dims &dm, const void *Q, const void *K, const void *V,
                    const int32_t *sample_idx, int n_s, int ks, int wt, float c, int32_t *labels,
                    float *mse, void *ws, hipStream_t st) {
  float *outs = (float *)ws;
  hipLaunchKernelGGL((profile_pass<T, D>), dim3((n_s + 63) / 64, dm.H, 3), dim3(64), 0, st,
                     (const T *)Q, (const T *)K, (const T *)V, sample_idx, n_s, dm.F, dm.S, dm.N,
                     ks, wt, c, outs, dm.H);
  hipLaunchKernelGGL(profile_reduce, dim3(dm.H), dim3(256), 0, st, outs, dm.H, n_s, D, labels, mse);
  return hipGetLastError();
}

}  // namespace

size_t profile_mfma_ws_bytes(const Dims &dm, int n_samples);
hipError_t launch_profile_mfma(const Dims &dm, const void *Q, const void *K, const void *V,
                               const int32_t *sample_idx, int n_s, int ks, int wt, float scale, int32_t *labels,
                               float *mse, void *ws, hipStream_t st);

size_t profile_ws_bytes(const Dims &dm, int n_samples) {
  const size_t simt = ((size_t)3 * dm.H * n_samples * dm.d * sizeof(float) + 255) / 256 * 256;
  const size_t mfma = profile_mfma_ws_bytes(dm, n_samples);
  return simt > mfma ? simt : mfma;
}

hipError_t launch_profile(const Dims &dm, bool bf16, const void *Q, const void *K, const void *V,
                          const int32_t *sample_idx, int n_samples, int ks, int wt, float scale,
                          int32_t *labels, float *mse, void *ws, hipStream_t st) {
  const float c = scale * kLog2e;
  if (dm.H == 0) return hipSuccess;
  if (bf16) {  // bf16 runs on the MFMA profiler
    return launch_profile_mfma(dm, Q, K, V, sample_idx, n_samples, ks, wt, scale, labels, mse, ws, st);
  } else {
    if (dm.d == 64)
      return launch_t<float, 64>(dm, Q, K, V, sample_idx, n_samples, ks, wt, c, labels, mse, ws, st);
    if (dm.d == 128)
      return launch_t<float, 128>(dm, Q, K, V, sample_idx, n_samples, ks, wt, c, labels, mse, ws, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace svgk
