// SVG2-style semantic path: k-means of Q and K per head, stable cluster
// permutation, top-p cluster-pair selection, and variable-size block-sparse
// attention over the selected pairs.
//
// Sources: the Sparse-VideoGen write-up, section "Three generations of the
// same idea".  SVG2 permutes tokens by semantic cluster, uses a flash
// k-means kernel, and runs a dynamic attention kernel.  Its install section:
// block-sparse attention with varied block sizes.  HyperVAttention, sections
// Problem and Surprising findings: cluster blocks are irregular, so tiled
// kernels waste work.  The varlen attention (varlen_gather.hip) therefore
// tiles the concatenation of a query cluster's selected key ranges.  It
// does not tile each cluster on its own.
#include <algorithm>

#include "attn_core.h"

namespace svgk {
namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Fixed point of Lloyd's map: an assignment equal to the previous one gives
// back, through the (deterministic) update, the centroids it was computed
// from, so every later iteration repeats that assignment and those
// centroids bit for bit.  chg[2][H] records per head whether the assignment
// of iteration it changed any point (slot it & 1); once one did not, the
// head's kernels of the remaining iterations return at once.  The outputs
// are those of all iterations.  chg == nullptr: every iteration runs (the
// cluster sort outside k-means).
struct KmFix {
  int32_t *chg;
  int it;
  // this iteration's assignment is the previous one's: nothing left to do
  __device__ bool skip_assign(int h) const { return chg && it > 0 && chg[((it - 1) & 1) * gridDim.y + h] == 0; }
  // this iteration's assignment changed nothing: its sort and update repeat the previous ones
  __device__ bool skip_rest(int h) const { return chg && chg[(it & 1) * gridDim.y + h] == 0; }
  // whether the assigning kernel compares against the previous assignment
  __device__ bool track() const { return chg && it > 0; }
  // an assigning wave reports its points: moved (it > 0), or the first iteration
  __device__ void report(int h, bool moved, int lane) const {
    if (!chg) return;
    if (it == 0) {
      if (blockIdx.x == 0 && threadIdx.x == 0) chg[h] = 1;
    } else if (__ballot(moved) != 0ull && lane == 0) {
      chg[(it & 1) * gridDim.y + h] = 1;
    }
  }
};

// ---------------------------------------------------------------------------
// k-means (Lloyd).  Assign: distances in fp32 from fp32 copies of the
// centroids, strict "<" so ties keep the lower index.  Update: the members of
// each cluster are put in index order by the stable counting sort below.
// Then one work-group per cluster sums them in fp64, dimension by dimension,
// in that order (the oracle's order), and divides.  No atomics.  The sums are
// deterministic, and exact for bf16 inputs.

template <typename T>
__global__ __launch_bounds__(128)
void km_init(const T *__restrict__ X, const int32_t *__restrict__ init_idx, int N, int D, int k,
             double *__restrict__ cent, int32_t *__restrict__ chg) {
  const int h = blockIdx.y, j = blockIdx.x;
  if (chg != nullptr && j == 0 && threadIdx.x < 2) chg[threadIdx.x * gridDim.y + h] = 0;
  const int src = init_idx[h * k + j];
  for (int e = threadIdx.x; e < D; e += blockDim.x)
    cent[((size_t)h * k + j) * D + e] = (double)to_f32<T>(X[((size_t)h * N + src) * D + e]);
}

template <typename T, int D>
__global__ __launch_bounds__(256)
void km_assign(const T *__restrict__ X, const double *__restrict__ cent, int N, int k,
               int32_t *__restrict__ assign, KmFix fx) {
  extern __shared__ float cs[];  // [k][D]
  const int h = blockIdx.y;
  if (fx.skip_assign(h)) return;
  const double *ch = cent + (size_t)h * k * D;
  for (int e = threadIdx.x; e < k * D; e += blockDim.x) cs[e] = (float)ch[e];
  __syncthreads();
  const int n0 = blockIdx.x * blockDim.x + threadIdx.x;
  const bool in = n0 < N;
  const int n = in ? n0 : N - 1;   // lanes past N compute a real point and store nothing
  const T *xr = X + ((size_t)h * N + n) * D;
  float x[D];
#pragma unroll
  for (int e = 0; e < D; ++e) x[e] = to_f32<T>(xr[e]);
  float best = INFINITY;
  int arg = 0;
  for (int j = 0; j < k; ++j) {
    const float *c = cs + j * D;
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) {
      const float df = x[e] - c[e];
      s = __builtin_fmaf(df, df, s);
    }
    if (s < best) {  // strict: ties keep the lower index
      best = s;
      arg = j;
    }
  }
  bool moved = false;
  if (in) {
    if (fx.track()) moved = assign[(size_t)h * N + n] != arg;
    assign[(size_t)h * N + n] = arg;
  }
  fx.report(h, moved, threadIdx.x & 63);
}

// Assignment on the matrix cores (bf16 inputs).  ||x - c||^2 = ||x||^2 +
// (||c||^2 - 2 x.c), and ||x||^2 is the same for every centroid, so the
// argmin is that of ||c||^2 - 2 x.c.  x.c runs on v_mfma_f32_32x32x2_f32: x is
// exact in fp32 (a bf16 value), c is the fp64 centroid rounded to fp32, and
// the 64..128-term dot product accumulates in fp32.  That is the precision of
// the vector kernel above, in another summation order; both decide as the
// fp64 oracle wherever the runner-up is farther by more than ~1e-5 of the
// distances.  Ties (identical centroids) keep the lower index: every lane
// scans its centroid rows in increasing order with a strict "<", and the
// two lanes of a point merge with the lower index on equality.
//
// km_prep writes, per head, the fp32 centroids as the MFMA's A operand wants
// them: for each centroid, its even dims then its odd dims, as two rows of
// D/2 floats padded to D/2 + 4 (so the 16 lanes of a ds_read_b128 fall in
// distinct banks), and ||c||^2 (fp64, rounded; +inf for the padding rows up
// to a multiple of 32, so they never win).
constexpr int kKmPad = 4;

template <int D>
struct KmTab {
  static constexpr int ROW = D / 2 + kKmPad;   // floats per half-row
  __host__ __device__ static size_t floats(int kpad) { return (size_t)kpad * (2 * ROW + 1); }
};

template <int D>
__global__ __launch_bounds__(256)
void km_prep(const double *__restrict__ cent, int k, int kpad, float *__restrict__ tab) {
  using TB = KmTab<D>;
  const int h = blockIdx.y;
  float *t = tab + (size_t)h * TB::floats(kpad);
  float *cn = t + (size_t)kpad * 2 * TB::ROW;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= kpad) return;
  if (c >= k) {
    cn[c] = INFINITY;
    for (int e = 0; e < 2 * TB::ROW; ++e) t[(size_t)c * 2 * TB::ROW + e] = 0.f;
    return;
  }
  const double *cr = cent + ((size_t)h * k + c) * D;
  double n2 = 0.0;
  for (int e = 0; e < D; ++e) {
    const double v = cr[e];
    n2 += v * v;
    t[((size_t)c * 2 + (e & 1)) * TB::ROW + (e >> 1)] = (float)v;
  }
  for (int e = D / 2; e < TB::ROW; ++e) {
    t[((size_t)c * 2) * TB::ROW + e] = 0.f;
    t[((size_t)c * 2 + 1) * TB::ROW + e] = 0.f;
  }
  cn[c] = (float)n2;
}

// Tokens per chunk of the stable counting sort by cluster (below).
constexpr int kSortChunk = 1024;

// One wave = 64 points (two 32-point blocks), 4 waves per work-group.
template <int D>
__global__ __launch_bounds__(256)
void km_assign_mfma(const bf16_t *__restrict__ X, const float *__restrict__ tab, int N, int k, int kpad,
                    int32_t *__restrict__ assign, KmFix fx) {
  using TB = KmTab<D>;
  extern __shared__ __attribute__((aligned(16))) float kt[];   // the head's table
  const int h = blockIdx.y;
  if (fx.skip_assign(h)) return;
  const size_t nf = TB::floats(kpad);
  const float *th = tab + (size_t)h * nf;
  for (size_t i = threadIdx.x * 4; i < nf; i += 256 * 4) {
    if (i + 4 <= nf) *reinterpret_cast<f32x4 *>(kt + i) = *reinterpret_cast<const f32x4 *>(th + i);
    else for (size_t j = i; j < nf; ++j) kt[j] = th[j];
  }
  __syncthreads();
  const float *cn = kt + (size_t)kpad * 2 * TB::ROW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int p0 = blockIdx.x * 256 + wave * 64 + l32, p1 = p0 + 32;
  // B operands: x[point][2s + hi] for s = 0..D/2-1, fp32
  float xb0[D / 2], xb1[D / 2];
  auto load_x = [&](int p, float (&xb)[D / 2]) {
    if (p < N) {
      const bf16_t *xr = X + ((size_t)h * N + p) * D;
#pragma unroll
      for (int v = 0; v < D / 8; ++v) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(xr + 8 * v);
#pragma unroll
        for (int q = 0; q < 4; ++q)   // word q holds dims 8v + 2q (low half) and 8v + 2q + 1 (high half)
          xb[4 * v + q] = __uint_as_float(hi ? (w[q] & 0xFFFF0000u) : (w[q] << 16));
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 2; ++s) xb[s] = 0.f;
    }
  };
  load_x(p0, xb0);
  load_x(p1, xb1);
  float best0 = INFINITY, best1 = INFINITY;
  int arg0 = 0, arg1 = 0;
  for (int cb = 0; cb < kpad / 32; ++cb) {
    f32x16 a0 = f32x16{}, a1 = f32x16{};
    const float *ar = kt + ((size_t)(cb * 32 + l32) * 2 + hi) * TB::ROW;
#pragma unroll
    for (int s4 = 0; s4 < D / 8; ++s4) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(ar + 4 * s4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], xb0[4 * s4 + i], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], xb1[4 * s4 + i], a1, 0, 0, 0);
      }
    }
    // lane rows: centroid cb*32 + 8*(r/4) + 4*hi + r%4, increasing in r
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int cbase = cb * 32 + 8 * g + 4 * hi;
      const f32x4 nn = *reinterpret_cast<const f32x4 *>(cn + cbase);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float d0 = __builtin_fmaf(-2.f, a0[4 * g + q], nn[q]);
        const float d1 = __builtin_fmaf(-2.f, a1[4 * g + q], nn[q]);
        if (d0 < best0) {
          best0 = d0;
          arg0 = cbase + q;
        }
        if (d1 < best1) {
          best1 = d1;
          arg1 = cbase + q;
        }
      }
    }
  }
  // merge the two lanes of each point (lower index on equal distance)
  auto merge = [&](float &b, int &a) {
    const float ob = __shfl_xor(b, 32);
    const int oa = __shfl_xor(a, 32);
    if (ob < b || (ob == b && oa < a)) {
      b = ob;
      a = oa;
    }
  };
  merge(best0, arg0);
  merge(best1, arg1);
  bool moved = false;
  if (hi == 0) {
    int32_t *a = assign + (size_t)h * N;
    if (p0 < N) {
      if (fx.track()) moved |= a[p0] != arg0;
      a[p0] = arg0;
    }
    if (p1 < N) {
      if (fx.track()) moved |= a[p1] != arg1;
      a[p1] = arg1;
    }
  }
  fx.report(h, moved, lane);
}

// The assignment for d = 64 on the bf16 matrix cores.  Each fp64 centroid
// value is split into three bf16 terms c = c1 + c2 + c3, each the bf16
// rounding of what the earlier terms leave (24 significant bits in all), so
// x.c = x.c1 + x.c2 + x.c3 with every product exact in fp32 (bf16 x bf16)
// and the sum accumulated in fp32 on v_mfma_f32_32x32x16_bf16: the precision
// of the fp32 kernel above, in another summation order, at 16 dims per
// instruction instead of 2.  Table per head: for each centroid its three
// terms as rows of D bf16, padded to 3 D + 8 (so the 32 lanes of a 16-byte
// read spread over the banks), then ||c||^2 per centroid as in km_prep.
template <int D>
struct KmTab3 {
  static constexpr int ROWH = 3 * D + 8;   // bf16 per centroid
  __host__ __device__ static size_t floats(int kpad) { return (size_t)kpad * (ROWH / 2 + 1); }
};

__device__ __forceinline__ void split3(double c, bf16_t &c1, bf16_t &c2, bf16_t &c3) {
  c1 = f32_to_bf16((float)c);
  double r = c - (double)bf16_to_f32(c1);
  c2 = f32_to_bf16((float)r);
  r -= (double)bf16_to_f32(c2);
  c3 = f32_to_bf16((float)r);
}

// Row j of the three-term table from the centroid's D fp64 values (one
// thread per dim e < D; threads e < 8 also zero the padding; thread 0 takes
// ||c||^2 in dim order, as km_prep).
template <int D>
__device__ __forceinline__ void km_tab3_row(const double *cv, int e, int j, int kpad, float *t) {
  using TB = KmTab3<D>;
  bf16_t *row = reinterpret_cast<bf16_t *>(t) + (size_t)j * TB::ROWH;
  if (e < D) {
    bf16_t c1, c2, c3;
    split3(cv[e], c1, c2, c3);
    row[e] = c1;
    row[D + e] = c2;
    row[2 * D + e] = c3;
  }
  if (e < 8) row[3 * D + e] = 0;
  if (e == 0) {
    double n2 = 0.0;
    for (int i = 0; i < D; ++i) {
      const double v = cv[i];
      n2 += v * v;
    }
    t[(size_t)kpad * (TB::ROWH / 2) + j] = (float)n2;
  }
}

// Initial three-term table: one block per centroid (padding rows: zero
// terms, ||c||^2 = +inf so they never win); also zeroes the sort counts that
// the first assignment fills.
template <int D>
__global__ __launch_bounds__(128)
void km_prep3(const double *__restrict__ cent, int N, int k, int kpad, float *__restrict__ tab,
              int32_t *__restrict__ cnt) {
  using TB = KmTab3<D>;
  __shared__ double cv[D];
  const int h = blockIdx.y, j = blockIdx.x, e = threadIdx.x;
  if (j < k) {   // column j of the sort's per-chunk counts starts at zero
    const int nch = (N + kSortChunk - 1) / kSortChunk;
    for (int b = e; b < nch; b += 128) cnt[((size_t)h * nch + b) * k + j] = 0;
  }
  float *t = tab + (size_t)h * TB::floats(kpad);
  if (j >= k) {
    bf16_t *row = reinterpret_cast<bf16_t *>(t) + (size_t)j * TB::ROWH;
    for (int i = e; i < TB::ROWH; i += 128) row[i] = 0;
    if (e == 0) t[(size_t)kpad * (TB::ROWH / 2) + j] = INFINITY;
    return;
  }
  if (e < D) cv[e] = cent[((size_t)h * k + j) * D + e];
  __syncthreads();
  km_tab3_row<D>(cv, e, j, kpad, t);
}

// kKmWaves waves per work-group (12: with the read-ahead below, 16 would
// spill), grid (G, H) with G work-groups per head.
// The head's table is copied to LDS once, then each wave takes 64-point
// groups (two 32-point blocks) wave-major, group = pass * kKmWaves * G +
// wave * G + blockIdx.x, so groups beyond the first pass spread over the
// work-groups' first waves.  Each point also counts itself into its chunk's
// histogram of the cluster sort.
constexpr int kKmWaves = 12;

template <int D>
__global__ __launch_bounds__(64 * kKmWaves)
void km_assign_bf3(const bf16_t *__restrict__ X, const float *__restrict__ tab, int N, int k, int kpad,
                   int32_t *__restrict__ assign, int32_t *__restrict__ cnt, KmFix fx) {
  using TB = KmTab3<D>;
  constexpr int NT = 64 * kKmWaves;
  extern __shared__ __attribute__((aligned(16))) float kt[];   // the head's table
  const int h = blockIdx.y;
  if (fx.skip_assign(h)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  // B operands: dims 16 s + 8 hi .. + 7 of the lane's point
  bf16x8 xb0[D / 16], xb1[D / 16];
  auto load_x = [&](int p, bf16x8 (&xb)[D / 16]) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      u32x4 w = u32x4{0, 0, 0, 0};
      if (p < N) w = *reinterpret_cast<const u32x4 *>(X + ((size_t)h * N + p) * D + 16 * st + 8 * hi);
      xb[st] = __builtin_bit_cast(bf16x8, w);
    }
  };
  const int ngrp = (N + 63) / 64, gstep = (int)gridDim.x * kKmWaves;
  int grp = wave * (int)gridDim.x + (int)blockIdx.x;
  // the first group's points load while the table streams in
  load_x(grp * 64 + l32, xb0);
  load_x(grp * 64 + 32 + l32, xb1);
  {
    // kpad is a multiple of 32, so the table is whole 16-byte words
    const int nf4 = (int)(TB::floats(kpad) / 4);
    const f32x4 *th = reinterpret_cast<const f32x4 *>(tab + (size_t)h * TB::floats(kpad));
    f32x4 *kt4 = reinterpret_cast<f32x4 *>(kt);
    constexpr int U = 8;   // loads in flight per thread
    for (int i0 = threadIdx.x; i0 < nf4; i0 += NT * U) {
      f32x4 r[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + NT * u < nf4) r[u] = th[i0 + NT * u];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + NT * u < nf4) kt4[i0 + NT * u] = r[u];
    }
  }
  __syncthreads();
  const bf16_t *ct = reinterpret_cast<const bf16_t *>(kt);
  const float *cn = kt + (size_t)kpad * (TB::ROWH / 2);
  bool moved = false;
  for (; grp < ngrp; grp += gstep) {
  const int p0 = grp * 64 + l32, p1 = p0 + 32;
  if (grp != wave * (int)gridDim.x + (int)blockIdx.x) {
    load_x(p0, xb0);
    load_x(p1, xb1);
  }
  float best0 = INFINITY, best1 = INFINITY;
  int arg0 = 0, arg1 = 0;
  for (int cb = 0; cb < kpad / 32; ++cb) {
    // the block's 12 table operands read together, then its 24 MFMAs (one
    // LDS latency exposed per block, not one per MFMA pair): x.c as the
    // three terms in order, 16 dims a step
    const bf16_t *ar = ct + (size_t)(cb * 32 + l32) * TB::ROWH + 8 * hi;
    bf16x8 av[3 * (D / 16)];
#pragma unroll
    for (int i = 0; i < 3 * (D / 16); ++i)
      av[i] = *reinterpret_cast<const bf16x8 *>(ar + (i / (D / 16)) * D + 16 * (i % (D / 16)));
    __builtin_amdgcn_sched_barrier(0);
    f32x16 a0 = f32x16{}, a1 = f32x16{};
#pragma unroll
    for (int i = 0; i < 3 * (D / 16); ++i) {
      a0 = core::mfma32(av[i], xb0[i % (D / 16)], a0);
      a1 = core::mfma32(av[i], xb1[i % (D / 16)], a1);
    }
    // lane rows: centroid cb*32 + 8*(r/4) + 4*hi + r%4, increasing in r
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int cbase = cb * 32 + 8 * g + 4 * hi;
      const f32x4 nn = *reinterpret_cast<const f32x4 *>(cn + cbase);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float d0 = __builtin_fmaf(-2.f, a0[4 * g + q], nn[q]);
        const float d1 = __builtin_fmaf(-2.f, a1[4 * g + q], nn[q]);
        if (d0 < best0) {
          best0 = d0;
          arg0 = cbase + q;
        }
        if (d1 < best1) {
          best1 = d1;
          arg1 = cbase + q;
        }
      }
    }
  }
  // merge the two lanes of each point (lower index on equal distance)
  auto merge = [&](float &b, int &a) {
    const float ob = __shfl_xor(b, 32);
    const int oa = __shfl_xor(a, 32);
    if (ob < b || (ob == b && oa < a)) {
      b = ob;
      a = oa;
    }
  };
  merge(best0, arg0);
  merge(best1, arg1);
  if (hi == 0) {
    // the sort's per-chunk histograms (zeroed beforehand), counted here
    int32_t *ch = cnt + (size_t)h * ((N + kSortChunk - 1) / kSortChunk) * k;
    int32_t *a = assign + (size_t)h * N;
    if (p0 < N) {
      if (fx.track()) moved |= a[p0] != arg0;
      a[p0] = arg0;
      atomicAdd(ch + (size_t)(p0 / kSortChunk) * k + arg0, 1);
    }
    if (p1 < N) {
      if (fx.track()) moved |= a[p1] != arg1;
      a[p1] = arg1;
      atomicAdd(ch + (size_t)(p1 / kSortChunk) * k + arg1, 1);
    }
  }
  }
  fx.report(h, moved, lane);
}

// Centroid of cluster j = mean of its members.  Each thread loads 16 bytes
// of a member row (VE values); the 256 threads form 256 / (D / VE) member
// slots, slot s taking members s, s + slots, ... of the cluster (sorted, so
// in index order), each summing its members in order in fp64; the slot sums
// are then added in slot order.  For bf16 values (8-bit significands) every
// partial sum of n members is a multiple of the smallest member's last bit
// and below n times the largest member, so it is exact in fp64 (53 bits), in
// any order, while the exponent span of a dimension's nonzero member values
// is at most 45 - log2(n): 31 bits for a cluster of 17,774 tokens, 17 at
// 2^28.  Within that bound the centroid is the index-order sum's (the
// oracle's) bit for bit; beyond it the two orders may differ in the last
// bit.  fp32 values agree to rounding.  An empty cluster keeps its
// centroid.  With tab (the MFMA assignment), the
// block also writes centroid j's row of the next iteration's table, as the
// prep kernels do (same values, same summation order of ||c||^2), which
// saves a launch per iteration.  With cnt, it zeroes column j of the sort's
// per-chunk counts for the next assignment to fill.  A head whose assignment
// of this iteration changed no point skips its update (KmFix): the result
// would be the centroids it already holds.
template <typename T>
__global__ __launch_bounds__(256)
void km_update(const T *__restrict__ X, const int32_t *__restrict__ perm, const int32_t *__restrict__ offs, int N,
               int k, int D, double *__restrict__ cent, int32_t *__restrict__ sizes, float *__restrict__ tab,
               int kpad, int tab3, int32_t *__restrict__ cnt, KmFix fx) {
  constexpr int VE = 16 / sizeof(T);
  __shared__ double cv[128];
  __shared__ double part[256 * VE];
  const int h = blockIdx.y, j = blockIdx.x, t = threadIdx.x;
  if (fx.chg != nullptr) {
    // the next assignment's flag starts clear, whether or not this update runs
    if (j == 0 && t == 0) fx.chg[((fx.it + 1) & 1) * gridDim.y + h] = 0;
    if (fx.skip_rest(h)) return;
  }
  const int tpr = D / VE, slots = 256 / tpr, slot = t / tpr, q = t % tpr;
  const int o0 = offs[(size_t)h * (k + 1) + j], o1 = offs[(size_t)h * (k + 1) + j + 1];
  const int len = o1 - o0;
  const int32_t *p = perm + (size_t)h * N;
  const T *Xh = X + (size_t)h * N * D + q * VE;
  double *cj = cent + ((size_t)h * k + j) * D;
  if (cnt != nullptr) {
    const int nch = (N + kSortChunk - 1) / kSortChunk;
    for (int b = t; b < nch; b += 256) cnt[((size_t)h * nch + b) * k + j] = 0;
  }
  {
    double acc[VE];
#pragma unroll
    for (int i = 0; i < VE; ++i) acc[i] = 0.0;
    auto add_row = [&](const u32x4 &w) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[2 * i] += (double)__uint_as_float(w[i] << 16);
          acc[2 * i + 1] += (double)__uint_as_float(w[i] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += (double)__uint_as_float(w[i]);
      }
    };
    // up to four members a slot in flight (a short cluster's last members
    // too): indices, then rows, then the adds in order
    for (int n = o0 + slot; n < o1; n += 4 * slots) {
      int idx[4];
      u32x4 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) idx[u] = n + u * slots < o1 ? p[n + u * slots] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (idx[u] >= 0) w[u] = *reinterpret_cast<const u32x4 *>(Xh + (size_t)idx[u] * D);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (idx[u] >= 0) add_row(w[u]);
    }
#pragma unroll
    for (int i = 0; i < VE; ++i) part[slot * D + q * VE + i] = acc[i];
  }
  __syncthreads();
  if (t < D && len > 0) {
    double c = part[t];
    for (int sl = 1; sl < slots; ++sl) c += part[sl * D + t];
    cj[t] = c / (double)len;
  }
  if (t == 0) sizes[h * k + j] = len;
  if (tab == nullptr) return;
  if (t < D) cv[t] = cj[t];   // each thread reads back its own dim
  __syncthreads();
  if (tab3) {   // the three-term bf16 table (d = 64)
    km_tab3_row<64>(cv, t, j, kpad, tab + (size_t)h * KmTab3<64>::floats(kpad));
    return;
  }
  const int row = D / 2 + kKmPad;
  float *tr = tab + (size_t)h * kpad * (2 * row + 1);
  if (t < D) tr[((size_t)j * 2 + (t & 1)) * row + (t >> 1)] = (float)cv[t];
  if (t < 2 * kKmPad) tr[((size_t)j * 2 + (t & 1)) * row + D / 2 + (t >> 1)] = 0.f;
  if (t == 0) {
    double n2 = 0.0;
    for (int i = 0; i < D; ++i) {
      const double v = cv[i];
      n2 += v * v;
    }
    tr[(size_t)kpad * 2 * row + j] = (float)n2;
  }
}

// ---------------------------------------------------------------------------
// Stable counting sort of each head's tokens by cluster id (k <= 256; ids
// outside [0, k) are skipped by both kernels, so no index leaves its
// buffer), in two launches over chunks of kSortChunk tokens: per-chunk histograms (the
// bf16 k-means assignment counts them itself); then each chunk takes from
// all histograms its first slot per cluster (cluster offsets by a scan of
// the totals, plus the counts of earlier chunks) and places its tokens in
// index order.  Within a chunk, equal ids inside a wave are found with 8
// ballots (one per id bit) and a token's rank is a popcount; per-wave counts
// order the chunk's 16 waves.  cnt is scratch of H * nchunks * k ints.

__global__ __launch_bounds__(256)
void sort_count(const int32_t *__restrict__ assign, int N, int k, int nch, int32_t *__restrict__ cnt, KmFix fx) {
  __shared__ int32_t hist[256];
  const int h = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x;
  if (fx.skip_rest(h)) return;
  hist[tid] = 0;
  __syncthreads();
  const int32_t *a = assign + (size_t)h * N;
  const int n0 = ch * kSortChunk, n1 = min(N, n0 + kSortChunk);
  for (int n = n0 + tid; n < n1; n += 256) {
    const int c = a[n];
    if ((unsigned)c < (unsigned)k) atomicAdd(&hist[c], 1);   // ids outside [0, k) join no cluster
  }
  __syncthreads();
  if (tid < k) cnt[((size_t)h * nch + ch) * k + tid] = hist[tid];
}

// One thread per token of the chunk (kSortChunk threads, 16 waves).
__global__ __launch_bounds__(kSortChunk)
void sort_place(const int32_t *__restrict__ assign, int N, int k, int nch, const int32_t *__restrict__ cnt,
                int32_t *__restrict__ perm, int32_t *__restrict__ offs, KmFix fx) {
  constexpr int NW = kSortChunk / 64;
  __shared__ int32_t start[256];
  __shared__ int32_t wcnt[NW][256];
  __shared__ int32_t wtot[4];
  const int h = blockIdx.y, ch = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (fx.skip_rest(h)) return;
  const int32_t *a = assign + (size_t)h * N;
  const int n = ch * kSortChunk + tid;
  // a token whose id is outside [0, k) is skipped: no cluster counts it (as
  // in sort_count), and it is not placed
  const int craw = n < N ? a[n] : -1;
  const bool valid = (unsigned)craw < (unsigned)k;
  const int c = valid ? craw : 0;
  // cluster t's total and its count in earlier chunks (threads t < k), then
  // an exclusive scan of the totals over the (at most 256) clusters by the
  // first 4 waves: per wave, then across their totals.  Chunk 0 writes the
  // offsets.
  int tot = 0, before = 0, incl = 0;
  if (tid < k) {
    const int32_t *cc = cnt + (size_t)h * nch * k;
#pragma unroll 4
    for (int b = 0; b < nch; ++b) {
      const int v = cc[(size_t)b * k + tid];
      tot += v;
      before += b < ch ? v : 0;
    }
  }
  if (wave < 4) {
    incl = tot;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wtot[wave] = incl;
  }
  for (int e = tid; e < NW * 256; e += kSortChunk) (&wcnt[0][0])[e] = 0;
  __syncthreads();
  if (tid < 256) {
    int wbefore = 0;
    for (int w = 0; w < wave; ++w) wbefore += wtot[w];
    const int excl = wbefore + incl - tot;
    if (tid < k) start[tid] = excl + before;
    if (ch == 0) {
      if (tid < k) offs[(size_t)h * (k + 1) + tid] = excl;
      if (tid == 255) offs[(size_t)h * (k + 1) + k] = wbefore + incl;
    }
  }
  // equal ids within the wave: 8 ballots, one per id bit; rank = earlier lanes
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t bal = __ballot(valid && ((c >> b) & 1));
    same &= ((c >> b) & 1) ? bal : ~bal;
  }
  const int rank = __popcll(same & below);
  if (valid && rank == 0) wcnt[wave][c] = __popcll(same);
  __syncthreads();
  if (tid < k) {  // exclusive prefix over the waves
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int t = wcnt[w][tid];
      wcnt[w][tid] = run;
      run += t;
    }
  }
  __syncthreads();
  if (valid) perm[(size_t)h * N + start[c] + wcnt[wave][c] + rank] = n;
}

size_t sort_scratch_bytes(const Dims &dm, int k) {
  const size_t nch = (dm.N + kSortChunk - 1) / kSortChunk;
  return align256((size_t)dm.H * nch * k * sizeof(int32_t));
}

// counted: cnt already holds the per-chunk histograms of assign
void launch_sort(const Dims &dm, const int32_t *assign, int k, int32_t *perm, int32_t *offs, int32_t *cnt,
                 hipStream_t st, bool counted = false, KmFix fx = KmFix{nullptr, 0}) {
  const int nch = (dm.N + kSortChunk - 1) / kSortChunk;
  if (!counted) hipLaunchKernelGGL(sort_count, dim3(nch, dm.H), dim3(256), 0, st, assign, dm.N, k, nch, cnt, fx);
  hipLaunchKernelGGL(sort_place, dim3(nch, dm.H), dim3(kSortChunk), 0, st, assign, dm.N, k, nch, cnt, perm, offs,
                     fx);
}

// ---------------------------------------------------------------------------
// Top-p pair selection, in fp64.  Kernel 1: one work-group per (head, query
// cluster), one thread per key cluster.  It writes the row's count to
// pair_ptr[h][i+1] and its ascending list to the row's full-width slot
// pair_idx[h][i*kk ...].  Kernel 2: one work-group per head.  It scans the
// counts and moves each row left to its final offset (row by row: a row's
// target never overlaps a later row's slot).

template <int D>
__global__ __launch_bounds__(256)
void select_rows(const double *__restrict__ cq, const double *__restrict__ ck, const int32_t *__restrict__ size_k,
                 int kq, int kk, double top_p, double scale, int32_t *__restrict__ pair_ptr,
                 int32_t *__restrict__ pair_idx) {
  __shared__ double prob[256];
  __shared__ double red[256];
  __shared__ double sp[256];   // probabilities in rank order
  __shared__ double dotv[256];
  __shared__ int32_t order[256];
  __shared__ int32_t keep[256];
  __shared__ int32_t wc[4];
  __shared__ int32_t nsel;
  const int h = blockIdx.y, i = blockIdx.x, j = threadIdx.x;
  const int lane = j & 63, wave = j >> 6;
  // c_q,i . c_k,j: thread j takes key cluster j (kk <= 256) and sums the
  // products over the dims in order, the query centroid broadcast from LDS
  // and its own row's loads issued 32 dims at a time.  This summation order
  // is the library's own (a float64 dot product has no one order); the cut
  // below depends on it only where the probabilities tie within rounding,
  // which the tests audit against.
  if (j < D) red[j] = cq[((size_t)h * kq + i) * D + j];
  __syncthreads();
  if (j < kk) {
    const double2 *kr = reinterpret_cast<const double2 *>(ck + ((size_t)h * kk + j) * D);
    double t = 0.0;
#pragma unroll
    for (int c0 = 0; c0 < D / 2; c0 += 16) {
      double2 w[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) w[u] = kr[c0 + u];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        t = fma(red[2 * (c0 + u)], w[u].x, t);
        t = fma(red[2 * (c0 + u) + 1], w[u].y, t);
      }
    }
    dotv[j] = t;
  }
  __syncthreads();
  const bool live = j < kk && size_k[h * kk + j] > 0;
  double l = -INFINITY;
  if (live) l = dotv[j] * scale + log((double)size_k[h * kk + j]);
  red[j] = l;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (j < off) red[j] = fmax(red[j], red[j + off]);
    __syncthreads();
  }
  const double mx = red[0];
  __syncthreads();
  const double e = live ? exp(l - mx) : 0.0;
  red[j] = e;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (j < off) red[j] += red[j + off];
    __syncthreads();
  }
  const double pj = e / red[0];
  prob[j] = live ? pj : -1.0;
  keep[j] = 0;
  const int nlive = __syncthreads_count(live);
  if (live) {  // rank by (probability desc, index asc)
    int rank = 0;
    for (int t = 0; t < kk; ++t) {
      const double pt = prob[t];
      rank += (pt > pj) || (pt == pj && t < j);
    }
    order[rank] = j;
    sp[rank] = pj;
  }
  __syncthreads();
  if (j == 0) {
    // the running sum in rank order, one add at a time; the first rank at
    // which it reaches top_p closes the set (all live clusters if none).
    // The next eight terms load while eight are added.
    double run = 0.0;
    int n = nlive;
    double cur[8], nxt[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) cur[u] = u < nlive ? sp[u] : 0.0;
    for (int r = 0; r < nlive; r += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) nxt[u] = r + 8 + u < nlive ? sp[r + 8 + u] : 0.0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (r + u < nlive) {
          run += cur[u];
          if (n == nlive && run >= top_p) n = r + u + 1;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) cur[u] = nxt[u];
    }
    nsel = n;
  }
  __syncthreads();
  if (j < nsel) keep[order[j]] = 1;
  __syncthreads();
  // the kept clusters in ascending order: ballot ranks within each wave,
  // plus the counts of earlier waves
  const bool kept = j < kk && keep[j];
  const uint64_t m = __ballot(kept);
  if (lane == 0) wc[wave] = __popcll(m);
  __syncthreads();
  int pos = __popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
  for (int w = 0; w < wave; ++w) pos += wc[w];
  if (kept) pair_idx[(size_t)h * kq * kk + (size_t)i * kk + pos] = j;
  if (j == 0) pair_ptr[(size_t)h * (kq + 1) + i + 1] = wc[0] + wc[1] + wc[2] + wc[3];
}

__global__ __launch_bounds__(256)
void select_compact(int kq, int kk, int32_t *__restrict__ pair_ptr, int32_t *__restrict__ pair_idx) {
  // Rows in batches of 8: every source of a batch is read before any of its
  // targets is written.  Row i's target ends at the start of row i + 1's
  // (the kept counts of rows < i + 1 sum to at most (i + 1) kk), so no write
  // reaches the source of a later batch.
  constexpr int B = 8;
  const int h = blockIdx.x, tid = threadIdx.x;
  int32_t *ptr = pair_ptr + (size_t)h * (kq + 1);
  int32_t *idx = pair_idx + (size_t)h * kq * kk;
  int run = 0;
  for (int i = 0; i < kq; i += B) {
    int n[B], v[B];
#pragma unroll
    for (int b = 0; b < B; ++b) n[b] = i + b < kq ? ptr[i + b + 1] : 0;
#pragma unroll
    for (int b = 0; b < B; ++b) v[b] = tid < n[b] ? idx[(size_t)(i + b) * kk + tid] : 0;
    __syncthreads();
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (i + b < kq) {
        if (tid < n[b]) idx[run + tid] = v[b];
        if (tid == 0) ptr[i + b] = run;
        run += n[b];
      }
    }
    __syncthreads();
  }
  if (tid == 0) ptr[kq] = run;
}



}  // namespace

size_t kmeans_ws_bytes(const Dims &dm, int k) {
  const int kpad = (k + 31) / 32 * 32;
  const size_t tab = dm.d == 64 ? KmTab3<64>::floats(kpad) : KmTab<128>::floats(kpad);
  return align256((size_t)dm.H * dm.N * sizeof(int32_t)) + align256((size_t)dm.H * (k + 1) * sizeof(int32_t)) +
         align256((size_t)dm.H * tab * sizeof(float)) + sort_scratch_bytes(dm, k) +
         align256((size_t)2 * dm.H * sizeof(int32_t));
}

hipError_t launch_kmeans(const Dims &dm, bool bf16, const void *X, int k, int iters, const int32_t *init_idx,
                         int32_t *assign, double *centroids, int32_t *sizes, void *ws, hipStream_t st) {
  int32_t *perm = (int32_t *)ws;
  int32_t *offs = (int32_t *)((char *)ws + align256((size_t)dm.H * dm.N * sizeof(int32_t)));
  float *tab = (float *)((char *)offs + align256((size_t)dm.H * (k + 1) * sizeof(int32_t)));
  const int kpad = (k + 31) / 32 * 32;
  const size_t tab_floats = dm.d == 64 ? KmTab3<64>::floats(kpad) : KmTab<128>::floats(kpad);
  int32_t *scnt = (int32_t *)((char *)tab + align256((size_t)dm.H * tab_floats * sizeof(float)));
  int32_t *chg = (int32_t *)((char *)scnt + sort_scratch_bytes(dm, k));   // [2][H], see KmFix
  if (bf16)
    hipLaunchKernelGGL(km_init<bf16_t>, dim3(k, dm.H), dim3(128), 0, st, (const bf16_t *)X, init_idx, dm.N, dm.d, k,
                       centroids, chg);
  else
    hipLaunchKernelGGL(km_init<float>, dim3(k, dm.H), dim3(128), 0, st, (const float *)X, init_idx, dm.N, dm.d, k,
                       centroids, chg);
  // Assignment: bf16, d = 64 on the bf16 matrix cores (three-term table);
  // bf16, d = 128 on the fp32 matrix cores (fp32 table); fp32 points on the
  // vector ALUs.  With k <= 256 the tables fit in LDS (at most 101 and 137
  // floats per centroid: 103 KB and 140 KB).
  const bool bf3 = bf16 && dm.d == 64, mfma = bf16 && dm.d == 128;
  const size_t lds = bf3 ? KmTab3<64>::floats(kpad) * sizeof(float)
                   : mfma ? KmTab<128>::floats(kpad) * sizeof(float)
                          : (size_t)k * dm.d * sizeof(float);
  const void *fn = bf3 ? (const void *)km_assign_bf3<64>
                 : mfma ? (const void *)km_assign_mfma<128>
                        : (dm.d == 64 ? (const void *)km_assign<float, 64> : (const void *)km_assign<float, 128>);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  if (lds > 65536) {  // table above 64 KiB: raise the dynamic LDS limit
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  const dim3 grid((dm.N + 255) / 256, dm.H), pgrid((kpad + 255) / 256, dm.H);
  // bf16, d = 64: work-groups per head so that all heads fit on the CUs at
  // once (two per CU while two tables fit in LDS), none without a group
  const int ngrp64 = (dm.N + 63) / 64;
  const int per_cu = lds <= 80 * 1024 ? 2 : 1;
  const int g3 = std::max(1, std::min((ngrp64 + kKmWaves - 1) / kKmWaves, 256 * per_cu / std::max(1, dm.H)));
  // the table of the initial centroids; each update then writes the next one
  if (bf3)
    hipLaunchKernelGGL(km_prep3<64>, dim3(kpad, dm.H), dim3(128), 0, st, centroids, dm.N, k, kpad, tab, scnt);
  else if (mfma)
    hipLaunchKernelGGL(km_prep<128>, pgrid, dim3(256), 0, st, centroids, k, kpad, tab);
  for (int it = 0; it < iters; ++it) {
    const KmFix fx{chg, it};
    if (bf3)
      hipLaunchKernelGGL(km_assign_bf3<64>, dim3(g3, dm.H), dim3(64 * kKmWaves), lds, st, (const bf16_t *)X, tab,
                         dm.N, k, kpad, assign, scnt, fx);
    else if (mfma)
      hipLaunchKernelGGL(km_assign_mfma<128>, grid, dim3(256), lds, st, (const bf16_t *)X, tab, dm.N, k, kpad,
                         assign, fx);
    else if (dm.d == 64)
      hipLaunchKernelGGL((km_assign<float, 64>), grid, dim3(256), lds, st, (const float *)X, centroids, dm.N, k,
                         assign, fx);
    else
      hipLaunchKernelGGL((km_assign<float, 128>), grid, dim3(256), lds, st, (const float *)X, centroids, dm.N, k,
                         assign, fx);
    launch_sort(dm, assign, k, perm, offs, scnt, st, bf3, fx);
    float *const next_tab = ((mfma || bf3) && it + 1 < iters) ? tab : nullptr;
    if (bf16)
      hipLaunchKernelGGL(km_update<bf16_t>, dim3(k, dm.H), dim3(256), 0, st, (const bf16_t *)X, perm, offs, dm.N, k,
                         dm.d, centroids, sizes, next_tab, kpad, bf3 ? 1 : 0, bf3 ? scnt : nullptr, fx);
    else
      hipLaunchKernelGGL(km_update<float>, dim3(k, dm.H), dim3(256), 0, st, (const float *)X, perm, offs, dm.N, k,
                         dm.d, centroids, sizes, next_tab, kpad, 0, nullptr, fx);
  }
  return hipGetLastError();
}

size_t cluster_permute_ws_bytes(const Dims &dm, int k) { return sort_scratch_bytes(dm, k); }

hipError_t launch_cluster_permute(const Dims &dm, const int32_t *assign, int k, int32_t *perm, int32_t *offs,
                                  void *ws, hipStream_t st) {
  launch_sort(dm, assign, k, perm, offs, (int32_t *)ws, st);
  return hipGetLastError();
}

hipError_t launch_select_pairs(const Dims &dm, const double *cq, const double *ck, const int32_t *size_k, int kq,
                               int kk, double top_p, double scale, int32_t *pair_ptr, int32_t *pair_idx,
                               hipStream_t st) {
  if (dm.d == 128)
    hipLaunchKernelGGL(select_rows<128>, dim3(kq, dm.H), dim3(256), 0, st, cq, ck, size_k, kq, kk, top_p, scale,
                       pair_ptr, pair_idx);
  else
    hipLaunchKernelGGL(select_rows<64>, dim3(kq, dm.H), dim3(256), 0, st, cq, ck, size_k, kq, kk, top_p, scale,
                       pair_ptr, pair_idx);
  hipLaunchKernelGGL(select_compact, dim3(dm.H), dim3(256), 0, st, kq, kk, pair_ptr, pair_idx);
  return hipGetLastError();
}

size_t varlen_ws_bytes(const Dims &, int, int) { return 0; }

// varlen_gather.hip: the attention with the selected keys gathered by the
// tile DMA (d = 64 or 128; no workspace)
hipError_t launch_varlen_gather(const Dims &dm, const void *Qp, const void *Kp, const void *Vp,
                                const int32_t *q_offs, const int32_t *k_offs, int kq, int kk,
                                const int32_t *pair_ptr, const int32_t *pair_idx, const int32_t *q_perm,
                                float scale, void *O, hipStream_t st);

hipError_t launch_varlen(const Dims &dm, bool bf16, const void *Qp, const void *Kp, const void *Vp,
                         const int32_t *q_offs, const int32_t *k_offs, int kq, int kk, const int32_t *pair_ptr,
                         const int32_t *pair_idx, const int32_t *q_perm, float scale, void *O, void *,
                         hipStream_t st) {
  if (!bf16) return hipErrorInvalidValue;
  return launch_varlen_gather(dm, Qp, Kp, Vp, q_offs, k_offs, kq, kk, pair_ptr, pair_idx, q_perm, scale, O, st);
}

}  // namespace svgk
