// Variable-size block-sparse attention over cluster pairs (the SVG2 dynamic
// attention kernel: the Sparse-VideoGen write-up's "Three generations" and
// install sections; HyperVAttention's Problem section on irregular cluster
// blocks) on the V^T tile pipeline of the SVG1 attention.
//
// Inputs are in cluster order: query cluster i is rows q_offs[i] ..
// q_offs[i+1] of Qp, key cluster j rows k_offs[j] .. k_offs[j+1] of Kp and
// of Vt (the key-tiled V^T of Vp).  A query of cluster i attends exactly the
// keys of its selected clusters.  One work-group (4 waves, 128 rows) takes
// 128 rows of one query cluster.  It walks the 64-key windows of Kp / Vt
// that its selected key ranges touch: each selected cluster ORs its keys
// into a 64-bit mask per window, and the windows with any selected key are
// listed in ascending order.  The pipeline then runs as for the
// block-sparse attention; a key outside the mask scores -inf, so the result
// is token-exact.  Output rows go back to the original order through q_perm.
#include "attn_vt_core.h"

namespace svgk {
namespace {

using namespace core;

constexpr int kVlWaves = 4;
constexpr int kVlRows = 32 * kVlWaves;
constexpr int kVlMaxWin = 2048;      // windows (64-key blocks) a head may have

// Inclusive sum over the work-group's threads (NT = 64 * waves); tmp holds
// one int per wave.  All threads call it together.
template <int NW>
__device__ __forceinline__ int group_inclusive_sum(int x, int lane, int wave, int *tmp) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) before += v < wave ? tmp[v] : 0;
  int total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) total += tmp[v];
  __syncthreads();
  tmp[NW] = total;   // read by the caller after its next barrier
  return x + before;
}

template <int D>
__global__ __launch_bounds__(64 * kVlWaves, D == 64 ? 2 : 1)
void varlen_vt(const bf16_t *__restrict__ Qp, const bf16_t *__restrict__ Kp, const bf16_t *__restrict__ Vt,
               const int32_t *__restrict__ q_offs, const int32_t *__restrict__ k_offs, int kq, int kk,
               const int32_t *__restrict__ pair_ptr, const int32_t *__restrict__ pair_idx,
               const int32_t *__restrict__ q_perm, int N, int nkb, float c, bf16_t *__restrict__ O) {
  constexpr int NT = 64 * kVlWaves;
  using TT = DTile<D>;
  constexpr int TB = TT::TBYTES;
  __shared__ __attribute__((aligned(1024))) char k0[TB], k1[TB], k2[TB], V0[TB], V1[TB], V2[TB];
  __shared__ int wlist[kVlMaxWin];           // windows in ascending order
  __shared__ uint32_t wmask[2 * kVlMaxWin];  // per window index: selected keys 0-31, 32-63
  __shared__ int tmp[kVlWaves + 1];
  __shared__ int s_cl, s_r0, s_r1;
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int32_t *qo = q_offs + (size_t)h * (kq + 1);
  // 1. this work-group's (query cluster, 128-row chunk): the chunks of the
  //    head's clusters in order, counted by a running sum over NT clusters
  //    at a time
  if (tid == 0) s_cl = -1;
  for (int i = tid; i < 2 * nkb; i += NT) wmask[i] = 0u;
  const int t = blockIdx.x;
  int done = 0;
  for (int i0 = 0; i0 < kq; i0 += NT) {
    const int i = i0 + tid;
    int a = 0, b = 0;
    if (i < kq) {
      a = qo[i];
      b = qo[i + 1];
    }
    const int nch = (b - a + kVlRows - 1) / kVlRows;
    const int incl = done + group_inclusive_sum<kVlWaves>(nch, lane, wave, tmp);
    if (t >= incl - nch && t < incl) {       // at most one thread
      s_cl = i;
      s_r0 = a + (t - (incl - nch)) * kVlRows;
      s_r1 = min(b, s_r0 + kVlRows);
    }
    __syncthreads();
    done += tmp[kVlWaves];
    if (done > t) break;                     // uniform: every thread reads the same total
  }
  __syncthreads();
  const int cl = s_cl;
  if (cl < 0) return;                        // past this head's last chunk (uniform)
  const int r0 = s_r0, r1 = s_r1;
  // 2. windows of the selected key ranges: thread m ORs selected cluster m's
  //    keys into the masks of the windows it touches; the windows with any
  //    selected key are then listed in ascending order (ballot per wave,
  //    wave totals across the group)
  const int32_t *ptr = pair_ptr + (size_t)h * (kq + 1);
  const int32_t *sel = pair_idx + (size_t)h * kq * kk + ptr[cl];
  const int nsel = ptr[cl + 1] - ptr[cl];
  const int32_t *ko = k_offs + (size_t)h * (kk + 1);
  for (int m = tid; m < nsel; m += NT) {
    const int j = sel[m];
    const int ks = ko[j], ke = ko[j + 1];
    for (int w = ks >> 6; 64 * w < ke; ++w) {
      const int lo = max(ks, 64 * w) - 64 * w, hx = min(ke, 64 * w + 64) - 64 * w;   // keys lo .. hx-1
      const uint64_t msk = (hx - lo == 64 ? ~0ull : ((1ull << (hx - lo)) - 1ull)) << lo;
      atomicOr(&wmask[2 * w], (uint32_t)msk);
      atomicOr(&wmask[2 * w + 1], (uint32_t)(msk >> 32));
    }
  }
  __syncthreads();
  int base = 0;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int w0 = 0; w0 < nkb; w0 += NT) {
    const int w = w0 + tid;
    const bool on = w < nkb && (wmask[2 * w] | wmask[2 * w + 1]) != 0u;
    const uint64_t bal = __ballot(on);
    if (lane == 0) tmp[wave] = __popcll(bal);
    __syncthreads();
    int pos = base;
    for (int v = 0; v < wave; ++v) pos += tmp[v];
    if (on) wlist[pos + __popcll(bal & below)] = w;
    for (int v = 0; v < kVlWaves; ++v) base += tmp[v];
    __syncthreads();
  }
  const int nwin = base;
  // 3. the wave's 32 query rows
  const size_t hoff = (size_t)h * N * D;
  const int qrow = r0 + wave * 32 + l32;
  const bool qvalid = qrow < r1;
  bf16x8 qf[D / 16];
  load_q<D>(Qp + hoff, qvalid ? qrow : -1, hi, qf);
  f32x16 o[D / 32];
  float m_run, l_run;
  if (nwin == 0) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    l_run = 0.f;
  } else {
    auto ent_raw = [&](int j) -> int { return wlist[j < nwin ? j : nwin - 1]; };
    // keys of the window outside the selected ranges score -inf (the mask
    // is wave-uniform; a fully selected window skips this in a scalar branch)
    auto prep = [&](f32x16 &s0, f32x16 &s1, int e) -> bool {
      const uint32_t w0 = __builtin_amdgcn_readfirstlane(wmask[2 * e]);
      const uint32_t w1 = __builtin_amdgcn_readfirstlane(wmask[2 * e + 1]);
      if ((w0 & w1) != ~0u) {
        const uint32_t sh = 8u * (uint32_t)hi;
        drop_scores(s0, s1, ~(w0 >> sh), ~(w1 >> sh));
      }
      return true;
    };
    vt_attend<D, kVlWaves>(nwin, ent_raw, prep, Kp + hoff, Vt + (size_t)h * nkb * (BK * D), N, k0, k1, k2, V0, V1,
                           V2, qf, wave, lane, c, o, m_run, l_run);
    __builtin_amdgcn_s_waitcnt(0);   // no DMA may land after the work-group ends
  }
  bf16_t *orow = nullptr;
  if (qvalid) {
    const int dst = q_perm ? q_perm[(size_t)h * N + qrow] : qrow;
    orow = O + hoff + (size_t)dst * D;
  }
  store_o<D>(orow, o, l_run, hi);
}

}  // namespace

int varlen_vt_max_windows() { return kVlMaxWin; }

bool varlen_vt_covers(const Dims &dm) { return (dm.d == 64 || dm.d == 128) && (dm.N + 63) / 64 <= kVlMaxWin; }

hipError_t launch_varlen_vt(const Dims &dm, const void *Qp, const void *Kp, const void *Vt, const int32_t *q_offs,
                            const int32_t *k_offs, int kq, int kk, const int32_t *pair_ptr, const int32_t *pair_idx,
                            const int32_t *q_perm, float scale, void *O, hipStream_t st) {
  if (!varlen_vt_covers(dm)) return hipErrorInvalidValue;
  if (dm.N == 0 || dm.H == 0) return hipSuccess;
  const int nkb = (dm.N + 63) / 64;
  const float c = scale * kLog2e;
  // a grid row per head: at most ceil(N / 128) + kq chunks (each cluster's
  // last chunk may be partial); surplus work-groups exit at once
  const dim3 grid((dm.N + kVlRows - 1) / kVlRows + kq, dm.H), block(64 * kVlWaves);
  if (dm.d == 128)
    hipLaunchKernelGGL(varlen_vt<128>, grid, block, 0, st, (const bf16_t *)Qp, (const bf16_t *)Kp,
                       (const bf16_t *)Vt, q_offs, k_offs, kq, kk, pair_ptr, pair_idx, q_perm, dm.N, nkb, c,
                       (bf16_t *)O);
  else
    hipLaunchKernelGGL(varlen_vt<64>, grid, block, 0, st, (const bf16_t *)Qp, (const bf16_t *)Kp,
                       (const bf16_t *)Vt, q_offs, k_offs, kq, kk, pair_ptr, pair_idx, q_perm, dm.N, nkb, c,
                       (bf16_t *)O);
  return hipGetLastError();
}

}  // namespace svgk
