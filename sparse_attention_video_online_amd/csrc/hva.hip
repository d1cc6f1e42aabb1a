// HVA-style clustering: k-means restricted to local 3D windows of the latent
// grid, and the refresh of a subset of tokens at a non-anchor step
// (HyperVAttention, sections Approach and Key results: centroid search
// restricted to local spatio-temporal windows; assignments reused across
// denoising steps, fully clustered only at anchor steps, a Lowe's-ratio
// subset refreshed otherwise).
//
// Geometry: video token (f, y, x) of the F x rows x cols grid is row
// f*S + y*cols + x; the text rows follow.  Windows of wf x wy x wx tokens;
// window (a, b, c) is cluster (a*nY + b)*nX + c; the text rows are one more
// cluster (id C) whose members never change.  A video token chooses among
// the centroids of its own and the adjacent windows (at most 27), by
//   dist = sum over dims in order of fl(fl(x - m)^2), float32 adds,
// m the float64 centroid rounded to float32 (fp contraction off, so the
// arithmetic is exactly that), the first minimum winning: the candidates
// are listed in increasing cluster id, so ties go to the lower id.
//
// One work-group per (128 tokens of a window, head) assigns its tokens, sums
// their bf16 values per chosen candidate in LDS (float64) and adds the
// partial sums to the head's float64 cluster sums with global atomics.  Sums of
// bf16 values are exact in float64 (within the exponent-span bound of the
// k-means update), so the order of the atomics changes no bit.  A second
// kernel turns the sums into means (an empty cluster keeps its centroid),
// writes the float32 copy the next assignment reads, and clears the sums.
#include "svg_common.h"

namespace svgk {
namespace {

constexpr int kHvaCand = 27;
constexpr size_t align256(size_t x) { return (x + 255) / 256 * 256; }
constexpr int kHvaThreads = 128;
enum { kHvaInit = 0, kHvaIter = 1, kHvaRefresh = 2 };

struct HvaGrid {
  int F, rows, cols, T;
  int wf, wy, wx;
  int nF, nY, nX;
  int C;      // window clusters; the text cluster (if T > 0) is C
  int k;      // C + (T > 0)
};

// Clears the sums and counts; with cent, writes the float32 copy of the
// centroids (the carried ones of a refresh step).  Grid (k, H), D threads.
template <int D>
__global__ __launch_bounds__(D)
void hva_prep(int k, const double *__restrict__ cent, float *__restrict__ c32, double *__restrict__ sums,
              int32_t *__restrict__ counts) {
  const size_t r = (size_t)blockIdx.y * k + blockIdx.x;
  const int c = threadIdx.x;
  sums[r * D + c] = 0.0;
  if (cent) c32[r * D + c] = (float)cent[r * D + c];
  if (c == 0) counts[r] = 0;
}

// Grid (C * chunks + ceil(T / 128), H): work-group x < C * chunks takes
// chunk x % chunks (128 tokens) of window x / chunks, the others 128 text
// rows each; one token per thread.  mode: kHvaInit (a token joins its own
// window), kHvaIter (local search; with flag_out, the Lowe flags too),
// kHvaRefresh (flag_in tokens search, the others keep assign; a token whose
// cluster is not among its candidates searches as well).
//
// The search keeps two candidates' sums in flight (independent chains, each
// still summed over the dims in order).  For the member sums each token's
// row is also staged in LDS and the tokens are ordered by their chosen
// candidate (a counting sort in LDS); the work-group's two waves each walk
// half of that order, one dim (d = 64) or two per lane, adding runs of one
// candidate in registers and each run to the head's float64 sums with one
// global atomic per dim.
template <int D>
__global__ __launch_bounds__(kHvaThreads)
void hva_assign(const bf16_t *__restrict__ X, HvaGrid g, int chunks, int N, int mode, const float *__restrict__ c32,
                const uint8_t *__restrict__ flag_in, int32_t *__restrict__ assign, uint8_t *__restrict__ flag_out,
                float r2, double *__restrict__ sums, int32_t *__restrict__ counts) {
#pragma clang fp contract(off)
  __shared__ float cm[kHvaCand * D];        // candidate centroids, float32
  __shared__ __attribute__((aligned(16))) bf16_t xs[kHvaThreads * D];   // the tokens' rows
  __shared__ int cnt[kHvaCand], cur[kHvaCand];
  __shared__ int cid[kHvaCand];
  __shared__ int tslot[kHvaThreads], ord[kHvaThreads];
  __shared__ int s_ncand, s_own;
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = g.rows * g.cols;
  const int nwin = g.C * chunks;
  const bool text = (int)blockIdx.x >= nwin;
  const int cell = text ? 0 : (int)blockIdx.x / chunks, part = text ? 0 : (int)blockIdx.x % chunks;
  int a = 0, b = 0, c = 0;
  if (!text) {
    a = cell / (g.nY * g.nX);
    b = (cell / g.nX) % g.nY;
    c = cell % g.nX;
  }
  // the work-group's tokens
  int nt, f0 = 0, y0 = 0, x0 = 0, ny = 1, nx = 1, t0;
  if (text) {
    t0 = ((int)blockIdx.x - nwin) * kHvaThreads;
    nt = min(kHvaThreads, g.T - t0);
  } else {
    f0 = a * g.wf;
    y0 = b * g.wy;
    x0 = c * g.wx;
    const int nf = min(g.wf, g.F - f0);
    ny = min(g.wy, g.rows - y0);
    nx = min(g.wx, g.cols - x0);
    t0 = part * kHvaThreads;
    nt = min(kHvaThreads, nf * ny * nx - t0);
  }
  if (nt <= 0) return;                       // a chunk past a small window's end (uniform)
  if (tid == 0) {
    int n = 0, own = 0;
    if (text) {
      cid[n++] = g.C;
    } else {
      for (int da = -1; da <= 1; ++da)          // lexicographic offsets: increasing id
        for (int db = -1; db <= 1; ++db)
          for (int dc = -1; dc <= 1; ++dc) {
            const int aa = a + da, bb = b + db, cc = c + dc;
            if (aa < 0 || aa >= g.nF || bb < 0 || bb >= g.nY || cc < 0 || cc >= g.nX) continue;
            if (da == 0 && db == 0 && dc == 0) own = n;
            cid[n++] = (aa * g.nY + bb) * g.nX + cc;
          }
    }
    s_ncand = n;
    s_own = own;
  }
  if (tid < kHvaCand) cnt[tid] = 0;
  __syncthreads();
  const int ncand = s_ncand, own = s_own;
  const size_t cbase = (size_t)h * g.k;
  const bool search = !text && mode != kHvaInit;
  if (search)
    for (int i = tid; i < ncand * D; i += kHvaThreads)
      cm[i] = c32[(cbase + cid[i / D]) * D + (i % D)];
  __syncthreads();

  const bf16_t *Xh = X + (size_t)h * N * D;
  if (tid < nt) {
    const int t = t0 + tid;
    int row;
    if (text) {
      row = g.F * S + t;
    } else {
      const int f = f0 + t / (ny * nx), y = y0 + (t / nx) % ny, x = x0 + t % nx;
      row = f * S + y * g.cols + x;
    }
    const u32x4 *src = reinterpret_cast<const u32x4 *>(Xh + (size_t)row * D);
    u32x4 xv[D / 8];
#pragma unroll
    for (int v = 0; v < D / 8; ++v) xv[v] = src[v];
#pragma unroll
    for (int v = 0; v < D / 8; ++v) reinterpret_cast<u32x4 *>(xs + tid * D)[v] = xv[v];
    int slot = text ? 0 : own;
    bool look = search;
    if (search && mode == kHvaRefresh) {
      const int cur = assign[(size_t)h * N + row];
      int found = -1;
      for (int s = 0; s < ncand; ++s) found = (found < 0 && cid[s] == cur) ? s : found;
      look = flag_in[(size_t)h * N + row] != 0 || found < 0;
      if (!look) slot = found;
    }
    if (look) {
      float xf[D];
#pragma unroll
      for (int v = 0; v < D / 8; ++v) {
        const u32x4 u = xv[v];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xf[8 * v + 2 * e] = __uint_as_float(u[e] << 16);
          xf[8 * v + 2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
      }
      float d1 = INFINITY, d2 = INFINITY;
      int best = 0;
      auto take = [&](float dist, int s) {
        if (dist < d1) {
          d2 = d1;
          d1 = dist;
          best = s;
        } else if (dist < d2) {
          d2 = dist;
        }
      };
      int s = 0;
      for (; s + 2 <= ncand; s += 2) {        // two candidates' chains at once
        const float *m0 = cm + s * D;
        float e0 = 0.f, e1 = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          const float t0_ = xf[e] - m0[e], t1_ = xf[e] - m0[D + e];
          const float q0 = t0_ * t0_, q1 = t1_ * t1_;
          e0 = e0 + q0;
          e1 = e1 + q1;
        }
        take(e0, s);                           // in candidate order: ties keep the lower id
        take(e1, s + 1);
      }
      for (; s < ncand; ++s) {
        const float *m = cm + s * D;
        float dist = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) {
          const float df = xf[e] - m[e];
          const float sq = df * df;
          dist = dist + sq;
        }
        take(dist, s);
      }
      slot = best;
      if (flag_out) {
        const float lim = r2 * d2;
        flag_out[(size_t)h * N + row] = d1 >= lim ? 1 : 0;
      }
    } else if (flag_out) {
      flag_out[(size_t)h * N + row] = 0;
    }
    assign[(size_t)h * N + row] = cid[slot];
    tslot[tid] = slot;
    __hip_atomic_fetch_add(&cnt[slot], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
  __syncthreads();
  // the tokens in order of their candidate (any order within one)
  if (tid == 0) {
    int run = 0;
    for (int sl = 0; sl < ncand; ++sl) {
      cur[sl] = run;
      run += cnt[sl];
    }
  }
  __syncthreads();
  if (tid < nt)
    ord[__hip_atomic_fetch_add(&cur[tslot[tid]], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)] = tid;
  __syncthreads();
  // member sums: each wave walks half of that order, lanes over the dims;
  // a run of one candidate adds up in registers (float64) and goes to the
  // head's sums when the candidate changes
  constexpr int PL = D / 64;                  // dims per lane
  const int half = (nt + 1) / 2, p0 = wave * half, p1 = min(nt, p0 + half);
  double racc[PL];
#pragma unroll
  for (int u = 0; u < PL; ++u) racc[u] = 0.0;
  int rs = -1;                               // the run's candidate (wave-uniform)
  auto flush = [&]() {
    if (rs >= 0) {
#pragma unroll
      for (int u = 0; u < PL; ++u) unsafeAtomicAdd(&sums[(cbase + cid[rs]) * D + PL * lane + u], racc[u]);
    }
#pragma unroll
    for (int u = 0; u < PL; ++u) racc[u] = 0.0;
  };
  // lane q holds the wave's q-th token and its candidate (half <= 64); the
  // loop reads them back with readlane and loads eight rows' values at a time
  const int np = p1 - p0;
  const int my_tk = lane < np ? ord[p0 + lane] : 0;
  const int my_sl = lane < np ? tslot[my_tk] : -1;
  for (int q0 = 0; q0 < np; q0 += 8) {
    float val[8][PL];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tk = __builtin_amdgcn_readlane(my_tk, q0 + u < np ? q0 + u : 0);
      const bf16_t *xr = xs + tk * D + PL * lane;
      if constexpr (PL == 1) {
        val[u][0] = __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t *>(xr)) << 16);
      } else {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(xr);
        val[u][0] = __uint_as_float(w << 16);
        val[u][1] = __uint_as_float(w & 0xFFFF0000u);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (q0 + u >= np) break;
      const int sl = __builtin_amdgcn_readlane(my_sl, q0 + u);
      if (sl != rs) {
        flush();
        rs = sl;
      }
#pragma unroll
      for (int t = 0; t < PL; ++t) racc[t] += (double)val[u][t];
    }
  }
  flush();
  if (tid < ncand && cnt[tid] > 0) atomicAdd(&counts[cbase + cid[tid]], cnt[tid]);
}

// Means from the sums (an empty cluster keeps its centroid), the float32
// copy, the sizes; then clears the sums and counts.  Grid (k, H), D threads.
template <int D>
__global__ __launch_bounds__(D)
void hva_finalize(int k, double *__restrict__ sums, int32_t *__restrict__ counts, double *__restrict__ cent,
                  float *__restrict__ c32, int32_t *__restrict__ sizes) {
  const size_t r = (size_t)blockIdx.y * k + blockIdx.x;
  const int c = threadIdx.x;
  const int n = counts[r];
  double m = cent[r * D + c];
  if (n > 0) m = sums[r * D + c] / (double)n;
  cent[r * D + c] = m;
  c32[r * D + c] = (float)m;
  sums[r * D + c] = 0.0;
  __syncthreads();                           // every thread has read counts[r]
  if (c == 0) {
    sizes[r] = n;
    counts[r] = 0;
  }
}

HvaGrid make_grid(const Dims &dm, int rows, int cols, const int win[3]) {
  HvaGrid g{};
  g.F = dm.F;
  g.rows = rows;
  g.cols = cols;
  g.T = dm.T;
  g.wf = win[0];
  g.wy = win[1];
  g.wx = win[2];
  g.nF = (dm.F + win[0] - 1) / win[0];
  g.nY = (rows + win[1] - 1) / win[1];
  g.nX = (cols + win[2] - 1) / win[2];
  g.C = g.nF * g.nY * g.nX;
  g.k = g.C + (dm.T > 0 ? 1 : 0);
  return g;
}

struct HvaWs {
  float *c32;
  double *sums;
  int32_t *counts;
};

HvaWs carve(const Dims &dm, int k, void *ws) {
  HvaWs w;
  w.c32 = (float *)ws;
  w.sums = (double *)((char *)ws + align256((size_t)dm.H * k * dm.d * sizeof(float)));
  w.counts = (int32_t *)((char *)w.sums + align256((size_t)dm.H * k * dm.d * sizeof(double)));
  return w;
}

// Work-groups per window: its largest size over 128 tokens.
int hva_chunks(const HvaGrid &g) { return (g.wf * g.wy * g.wx + kHvaThreads - 1) / kHvaThreads; }

template <int D>
hipError_t run_cluster(const Dims &dm, const HvaGrid &g, const void *X, int iters, float r2, int32_t *assign,
                       double *cent, int32_t *sizes, uint8_t *flags, const HvaWs &w, hipStream_t st) {
  const int ch = hva_chunks(g);
  const dim3 kgrid(g.k, dm.H), agrid(g.C * ch + (g.T + kHvaThreads - 1) / kHvaThreads, dm.H);
  hipLaunchKernelGGL(hva_prep<D>, kgrid, dim3(D), 0, st, g.k, (const double *)nullptr, w.c32, w.sums, w.counts);
  hipLaunchKernelGGL(hva_assign<D>, agrid, dim3(kHvaThreads), 0, st, (const bf16_t *)X, g, ch, dm.N, (int)kHvaInit,
                     (const float *)w.c32, (const uint8_t *)nullptr, assign, (uint8_t *)nullptr, r2, w.sums,
                     w.counts);
  hipLaunchKernelGGL(hva_finalize<D>, kgrid, dim3(D), 0, st, g.k, w.sums, w.counts, cent, w.c32, sizes);
  for (int it = 0; it < iters; ++it) {
    uint8_t *fo = it + 1 == iters ? flags : nullptr;
    hipLaunchKernelGGL(hva_assign<D>, agrid, dim3(kHvaThreads), 0, st, (const bf16_t *)X, g, ch, dm.N, (int)kHvaIter,
                       (const float *)w.c32, (const uint8_t *)nullptr, assign, fo, r2, w.sums, w.counts);
    hipLaunchKernelGGL(hva_finalize<D>, kgrid, dim3(D), 0, st, g.k, w.sums, w.counts, cent, w.c32, sizes);
  }
  return hipGetLastError();
}

template <int D>
hipError_t run_refresh(const Dims &dm, const HvaGrid &g, const void *X, const uint8_t *flags, int32_t *assign,
                       double *cent, int32_t *sizes, const HvaWs &w, hipStream_t st) {
  const int ch = hva_chunks(g);
  const dim3 kgrid(g.k, dm.H), agrid(g.C * ch + (g.T + kHvaThreads - 1) / kHvaThreads, dm.H);
  hipLaunchKernelGGL(hva_prep<D>, kgrid, dim3(D), 0, st, g.k, (const double *)cent, w.c32, w.sums, w.counts);
  hipLaunchKernelGGL(hva_assign<D>, agrid, dim3(kHvaThreads), 0, st, (const bf16_t *)X, g, ch, dm.N,
                     (int)kHvaRefresh, (const float *)w.c32, flags, assign, (uint8_t *)nullptr, 0.f, w.sums,
                     w.counts);
  hipLaunchKernelGGL(hva_finalize<D>, kgrid, dim3(D), 0, st, g.k, w.sums, w.counts, cent, w.c32, sizes);
  return hipGetLastError();
}

}  // namespace

int hva_clusters(const Dims &dm, int rows, int cols, const int win[3]) { return make_grid(dm, rows, cols, win).k; }

size_t hva_ws_bytes(const Dims &dm, int k) {
  return align256((size_t)dm.H * k * dm.d * sizeof(float)) + align256((size_t)dm.H * k * dm.d * sizeof(double)) +
         align256((size_t)dm.H * k * sizeof(int32_t));
}

hipError_t launch_hva_cluster(const Dims &dm, const void *X, int rows, int cols, const int win[3], int iters,
                              float r2, int32_t *assign, double *cent, int32_t *sizes, uint8_t *flags, void *ws,
                              hipStream_t st) {
  const HvaGrid g = make_grid(dm, rows, cols, win);
  const HvaWs w = carve(dm, g.k, ws);
  if (dm.d == 128) return run_cluster<128>(dm, g, X, iters, r2, assign, cent, sizes, flags, w, st);
  return run_cluster<64>(dm, g, X, iters, r2, assign, cent, sizes, flags, w, st);
}

hipError_t launch_hva_refresh(const Dims &dm, const void *X, int rows, int cols, const int win[3],
                              const uint8_t *flags, int32_t *assign, double *cent, int32_t *sizes, void *ws,
                              hipStream_t st) {
  const HvaGrid g = make_grid(dm, rows, cols, win);
  const HvaWs w = carve(dm, g.k, ws);
  if (dm.d == 128) return run_refresh<128>(dm, g, X, flags, assign, cent, sizes, w, st);
  return run_refresh<64>(dm, g, X, flags, assign, cent, sizes, w, st);
}

}  // namespace svgk
