// SVG-EAR: block centroids for the compensation of skipped blocks, and the
// error-aware routing that picks which skipped blocks to compute exactly.
//
// The Sparse-VideoGen write-up ("Three generations of the same idea") says
// SVG-EAR recovers skipped attention blocks with parameter-free centroid
// compensation and routes high-error blocks to exact computation.  Reading
// (no formulas on the pages), per head in the executing layout, for kv-block
// b (its n_b <= 64 keys):
//   centroid kbar_b = mean key, value sum = sum of the values (n_b * mean),
//   radius r_b = max_j ||k_j - kbar_b||;
//   a skipped block contributes as one centroid key of weight n_b;
//   for q-block Q with mean query qbar, the centroid's error in the block's
//   attention mass is at most n_b e^{tau qbar.kbar_b} (e^{tau |qbar| r_b} - 1):
//   the route_k skipped blocks with the largest bound (ties to the lower
//   index) become exact, and the ragged last block is always exact (so every
//   compensated block has n_b = 64).
//
// ear_stats   one work-group per (centroid slot, head): fp64 centroid
//             (dim-major, [H][d][nKB]) and radius for the routing; the bf16 centroid row of the
//             attention's centroid K table and its value sums in the
//             key-tiled V^T table (zero rows past the last block).
// ear_route   one work-group per (group of q-blocks, head): fp64 mean
//             queries, the scores of every candidate block (a thread per
//             block reads its fp64 centroid once for the whole group, dim by
//             dim: the centroids are stored dim-major), then one wave per
//             q-block takes the route_k best by repeated wave-wide argmax.
#include "svg_common.h"

namespace svgk {
namespace {

template <int D>
__global__ __launch_bounds__(256)
void ear_stats(const bf16_t *__restrict__ K, const bf16_t *__restrict__ Vt, int N, int nkb, int ntc,
               bf16_t *__restrict__ Kc, bf16_t *__restrict__ Vct, double *__restrict__ kbar,
               double *__restrict__ rad) {
  constexpr int RG = 256 / D;              // row groups of the column sums
  __shared__ double cs[D];
  __shared__ double part[256];
  __shared__ double red[4];
  const int b = blockIdx.x, h = blockIdx.y, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int tc = b >> 6, jj = b & 63;      // centroid tile and slot in it
  bf16_t *kc_row = Kc + ((size_t)h * ntc * 64 + b) * D;
  if (b >= nkb) {                          // padding slot: zero centroid and value sum
    if (t < D) {
      kc_row[t] = 0;
      Vct[(((size_t)h * ntc + tc) * D + t) * 64 + jj] = 0;
    }
    return;
  }
  const int n = min(64, N - 64 * b);
  const bf16_t *Kb = K + ((size_t)h * N + 64 * (size_t)b) * D;
  {
    const int c = t % D, g = t / D;
    double acc = 0.0;
    for (int j = g; j < n; j += RG) acc += (double)bf16_to_f32(Kb[(size_t)j * D + c]);
    part[t] = acc;
  }
  __syncthreads();
  if (t < D) {
    double sum = 0.0;
    for (int g = 0; g < RG; ++g) sum += part[g * D + t];
    const double m = sum / (double)n;
    cs[t] = m;
    kbar[((size_t)h * D + t) * nkb + b] = m;   // dim-major: the routing reads a dim across blocks
    kc_row[t] = f32_to_bf16((float)m);
  }
  __syncthreads();
  {  // radius: four threads per key row
    const int j = t >> 2, q = t & 3;
    double dd = 0.0;
    if (j < n) {
      for (int e = q * (D / 4); e < (q + 1) * (D / 4); ++e) {
        const double x = (double)bf16_to_f32(Kb[(size_t)j * D + e]) - cs[e];
        dd += x * x;
      }
    }
    dd += __shfl_xor(dd, 1);
    dd += __shfl_xor(dd, 2);
    double m = dd;
    for (int s = 4; s < 64; s <<= 1) m = fmax(m, __shfl_xor(m, s));
    if (lane == 0) red[wave] = m;
  }
  __syncthreads();
  if (t == 0) rad[(size_t)h * nkb + b] = sqrt(fmax(fmax(red[0], red[1]), fmax(red[2], red[3])));
  {  // value sums from the V^T tile: row c holds the block's 64 keys of dim c
    const bf16_t *Vtile = Vt + ((size_t)h * nkb + b) * D * 64;
    const int c = t % D, g = t / D;
    constexpr int KPG = 64 / RG;           // keys per group
    double acc = 0.0;
    for (int j = g * KPG; j < (g + 1) * KPG; ++j) acc += (double)bf16_to_f32(Vtile[(size_t)c * 64 + j]);
    part[t] = acc;
  }
  __syncthreads();
  if (t < D) {
    double sum = 0.0;
    for (int g = 0; g < RG; ++g) sum += part[g * D + t];
    Vct[(((size_t)h * ntc + tc) * D + t) * 64 + jj] = f32_to_bf16((float)sum);
  }
}

constexpr int kRouteWaves = 8;             // q-blocks per work-group (at most)
constexpr int kRouteBlocks = 4;            // kv-blocks a thread scores at once

// Dynamic LDS: qbar [qpw][D] doubles, scores [qpw][nkb] doubles, chosen
// flags [qpw][nkb] bytes.  A score is NaN for a block that is not a
// candidate (kept already, or the ragged last block).
template <int D>
__global__ __launch_bounds__(64 * kRouteWaves)
void ear_route(const bf16_t *__restrict__ Q, const int32_t *__restrict__ labels, const double *__restrict__ kbar,
               const double *__restrict__ rad, const uint8_t *__restrict__ mask, int N, int F, int S, int nqb,
               int nkb, int bq, int qpw, int route_k, double tau, uint8_t *__restrict__ exact) {
  extern __shared__ __attribute__((aligned(16))) double lds[];
  double *qbar = lds;
  double *sc = lds + (size_t)qpw * D;
  uint8_t *chosen = reinterpret_cast<uint8_t *>(sc + (size_t)qpw * nkb);
  __shared__ double qnorm[kRouteWaves];
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q0 = blockIdx.x * qpw;
  const bool perm = labels == nullptr || labels[h] == 1;
  const bool ragged = (N % 64) != 0;
  const int Qw = q0 + wave;
  // 1. mean query of q-block Qw (executing-layout rows, read from the
  //    original order as the layout permute maps them).  Lane l reads 16
  //    bytes (8 dims) of row r0 + 4 j + l / (D / 8) for j = 0, 1, ..: all its
  //    rows' loads go out in batches of 8, the sums are float64 (exact for
  //    bf16 values, so the grouping of the rows changes no bit), and the
  //    64 / (D / 8) row groups are added by a butterfly at the end.
  if (wave < qpw && Qw < nqb) {
    constexpr int LPR = D / 8;                // lanes per row
    constexpr int RPI = 64 / LPR;             // rows per load instruction
    const int r0 = Qw * bq, r1 = min(N, r0 + bq);
    const int sub = lane / LPR, part = lane % LPR;
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int rb = r0; rb < r1; rb += 8 * RPI) {
      u32x4 w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = rb + RPI * j + sub;
        int src = r < r1 ? r : r0;
        if (perm && src < F * S) {
          const int p = src / F, f = src - p * F;
          src = f * S + p;
        }
        w[j] = reinterpret_cast<const u32x4 *>(Q + ((size_t)h * N + src) * D)[part];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (rb + RPI * j + sub < r1)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] += (double)__uint_as_float(w[j][q] << 16);
            acc[2 * q + 1] += (double)__uint_as_float(w[j][q] & 0xFFFF0000u);
          }
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
    double n2 = 0.0;
    if (sub == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double m = acc[e] / (double)(r1 - r0);
        qbar[wave * D + 8 * part + e] = m;
        n2 += m * m;
      }
    }
    for (int s2 = 1; s2 < 64; s2 <<= 1) n2 += __shfl_xor(n2, s2);
    if (lane == 0) qnorm[wave] = sqrt(n2);
  }
  __syncthreads();
  // 2. scores: one thread per kv-block, the dot products in dim order; the
  //    centroids are dim-major, so each dim's read is coalesced over the
  //    threads, and the mean queries are LDS broadcasts
  //    Each thread takes up to kRouteBlocks blocks at once (stride 512), so
  //    that many centroid loads are in flight per dim step.
  const int nq = min(qpw, nqb - q0);
  const double ln64 = log(64.0);
  const double *kh = kbar + (size_t)h * D * nkb;
  constexpr int NT = 64 * kRouteWaves;
  for (int b0 = tid; b0 < nkb; b0 += NT * kRouteBlocks) {
    double dot[kRouteBlocks][kRouteWaves];
#pragma unroll
    for (int i = 0; i < kRouteBlocks; ++i)
#pragma unroll
      for (int w = 0; w < kRouteWaves; ++w) dot[i][w] = 0.0;
#pragma unroll 8
    for (int c = 0; c < D; ++c) {
      double x[kRouteBlocks];
#pragma unroll
      for (int i = 0; i < kRouteBlocks; ++i) {
        const int b = b0 + i * NT;
        x[i] = b < nkb ? kh[(size_t)c * nkb + b] : 0.0;
      }
#pragma unroll
      for (int w = 0; w < kRouteWaves; ++w) {
        if (w >= nq) break;
        const double qv = qbar[w * D + c];
#pragma unroll
        for (int i = 0; i < kRouteBlocks; ++i) dot[i][w] = fma(qv, x[i], dot[i][w]);
      }
    }
#pragma unroll
    for (int i = 0; i < kRouteBlocks; ++i) {
      const int b = b0 + i * NT;
      if (b >= nkb) break;
      const double rb = rad[(size_t)h * nkb + b];
      const bool last = ragged && b == nkb - 1;
#pragma unroll
      for (int w = 0; w < kRouteWaves; ++w) {
        if (w >= nq) break;
        const bool cand = !last && mask[((size_t)h * nqb + q0 + w) * nkb + b] == 0;
        sc[(size_t)w * nkb + b] = cand ? ln64 + tau * dot[i][w] + log(expm1(tau * qnorm[w] * rb)) : NAN;
        chosen[(size_t)w * nkb + b] = 0;
      }
    }
  }
  __syncthreads();
  // 3. wave w picks route_k candidates of q-block q0 + w: the largest score,
  //    the lower index on ties (-inf scores are candidates too).  A lane
  //    holds the scores of blocks lane, lane + 64, ... (at most kRouteRegs)
  //    in registers with a bit per taken one; each pick is a lane-local
  //    maximum and a butterfly over the lanes.  Longer rows (more than
  //    64 * kRouteRegs blocks) read their scores from LDS instead.
  if (wave < nq) {
    double *s = sc + (size_t)wave * nkb;
    uint8_t *ch = chosen + (size_t)wave * nkb;
    constexpr int kRouteRegs = 32;
    if (nkb <= 64 * kRouteRegs) {
      double v[kRouteRegs];
      uint32_t live = 0;                     // bit i: block lane + 64 i is a candidate not yet taken
#pragma unroll
      for (int i = 0; i < kRouteRegs; ++i) {
        const int b = lane + 64 * i;
        v[i] = b < nkb ? s[b] : NAN;
        if (v[i] == v[i]) live |= 1u << i;
      }
      for (int it = 0; it < route_k; ++it) {
        double best = NAN;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < kRouteRegs; ++i)
          if (((live >> i) & 1) && (bi < 0 || v[i] > best)) {   // ascending block per lane: equal keeps the lower
            best = v[i];
            bi = lane + 64 * i;
          }
        for (int off = 1; off < 64; off <<= 1) {
          const double ob = __shfl_xor(best, off);
          const int oi = __shfl_xor(bi, off);
          if (oi >= 0 && (bi < 0 || ob > best || (ob == best && oi < bi))) {
            best = ob;
            bi = oi;
          }
        }
        if (bi < 0) break;                   // no candidate left (wave-uniform)
        if ((bi & 63) == lane) live &= ~(1u << (bi >> 6));
      }
      // the taken blocks: candidates no longer live
#pragma unroll
      for (int i = 0; i < kRouteRegs; ++i) {
        const int b = lane + 64 * i;
        if (b < nkb && v[i] == v[i] && !((live >> i) & 1)) ch[b] = 1;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
    } else {
      for (int it = 0; it < route_k; ++it) {
        double best = NAN;
        int bi = -1;
        for (int b = lane; b < nkb; b += 64) {
          const double v = s[b];
          if (v != v || ch[b]) continue;
          if (bi < 0 || v > best) {   // ascending b per lane: equal keeps the lower
            best = v;
            bi = b;
          }
        }
        for (int off = 1; off < 64; off <<= 1) {
          const double ob = __shfl_xor(best, off);
          const int oi = __shfl_xor(bi, off);
          if (oi >= 0 && (bi < 0 || ob > best || (ob == best && oi < bi))) {
            best = ob;
            bi = oi;
          }
        }
        if (bi < 0) break;                // no candidate left (wave-uniform)
        if (lane == 0) ch[bi] = 1;
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_wave_barrier();
      }
    }
    uint8_t *out = exact + ((size_t)h * nqb + q0 + wave) * nkb;
    const uint8_t *in = mask + ((size_t)h * nqb + q0 + wave) * nkb;
    for (int b = lane; b < nkb; b += 64)
      out[b] = (in[b] != 0 || (ragged && b == nkb - 1) || ch[b]) ? 1 : 0;
  }
}

}  // namespace

int ear_centroid_tiles(const Dims &dm) { return (((dm.N + 63) / 64) + 63) / 64; }

hipError_t launch_ear_stats(const Dims &dm, const void *K, const void *Vt, void *Kc, void *Vct, double *kbar,
                            double *rad, hipStream_t st) {
  const int nkb = (dm.N + 63) / 64, ntc = ear_centroid_tiles(dm);
  if (dm.H == 0 || nkb == 0) return hipSuccess;
  if (dm.d == 128)
    hipLaunchKernelGGL(ear_stats<128>, dim3(ntc * 64, dm.H), dim3(256), 0, st, (const bf16_t *)K, (const bf16_t *)Vt,
                       dm.N, nkb, ntc, (bf16_t *)Kc, (bf16_t *)Vct, kbar, rad);
  else
    hipLaunchKernelGGL(ear_stats<64>, dim3(ntc * 64, dm.H), dim3(256), 0, st, (const bf16_t *)K, (const bf16_t *)Vt,
                       dm.N, nkb, ntc, (bf16_t *)Kc, (bf16_t *)Vct, kbar, rad);
  return hipGetLastError();
}

// q-blocks per route work-group: at most 8, and their scores within 128 KB
int ear_route_qpw(const Dims &dm) {
  const int nkb = (dm.N + 63) / 64;
  const size_t per = (size_t)nkb * 9 + (size_t)dm.d * 8;   // score + flag per block, plus qbar
  int q = (int)((128 * 1024) / per);
  return q < 1 ? 0 : (q > kRouteWaves ? kRouteWaves : q);
}

hipError_t launch_ear_route(const Dims &dm, const void *Q, const int32_t *labels, const double *kbar,
                            const double *rad, const uint8_t *mask, int bq, int route_k, double tau, uint8_t *exact,
                            hipStream_t st) {
  const int nkb = (dm.N + 63) / 64, nqb = (dm.N + bq - 1) / bq;
  const int qpw = ear_route_qpw(dm);
  if (qpw < 1) return hipErrorInvalidValue;
  const size_t lds = (size_t)qpw * dm.d * 8 + (size_t)qpw * nkb * 8 + (size_t)qpw * nkb;
  const dim3 grid((nqb + qpw - 1) / qpw, dm.H);
  const void *fn = dm.d == 128 ? (const void *)ear_route<128> : (const void *)ear_route<64>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (dm.d == 128)
    hipLaunchKernelGGL(ear_route<128>, grid, dim3(64 * kRouteWaves), lds, st, (const bf16_t *)Q, labels, kbar, rad,
                       mask, dm.N, dm.F, dm.S, nqb, nkb, bq, qpw, route_k, tau, exact);
  else
    hipLaunchKernelGGL(ear_route<64>, grid, dim3(64 * kRouteWaves), lds, st, (const bf16_t *)Q, labels, kbar, rad,
                       mask, dm.N, dm.F, dm.S, nqb, nkb, bq, qpw, route_k, tau, exact);
  return hipGetLastError();
}

}  // namespace svgk
