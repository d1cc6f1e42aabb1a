// Block-sparse flash attention on the key-tiled V^T layout, bf16 in / fp32
// accumulate, gfx950 MFMA, 256 query rows per work-group.
//
// Same operation as attn_mfma.hip: for every q-block of every head, softmax
// attention over the keys of its kept kv-blocks only (the custom sparse
// kernel of the SVG1 abstract, on the block-sparse attention with per-block
// keep flags named in the Sparse-VideoGen write-up's install section).  Two
// things differ.
//
// 1. V arrives as Vt, key-tiled and transposed: for kv-block kb and dim c,
//    the 64 keys kb*64 .. kb*64+63 are contiguous (zero past N).  The V^T
//    MFMA operand (8 consecutive keys of one dim per lane) is then one
//    ds_read_b128.  Plain LDS reads also let the tile DMA stay in flight:
//    the compiler makes no wait of its own between a DMA and a later plain
//    LDS read, so the pipeline below decides every wait itself.
// 2. One work-group = 8 waves = 256 query rows, i.e. 256/bq q-blocks that
//    share one stream of K/V tiles: the union of their kept lists, built in
//    LDS from bitmaps at the start.  A wave whose own q-block does not keep
//    a tile of the union treats it as fully masked.  K/V traffic per query
//    halves against one q-block per work-group.
//
// Pipeline per wave, tile t of the union (3 LDS stages each for K and V^T):
//   (A) mask S(t) (tail / not kept), row maximum, lazy reference update;
//   (B) DMA V(t+2) and K(t+3) into the stages PV(t-1) and QK(t) released;
//       then S(t+1) = K(t+1) Q^T on the matrix cores interleaved with the
//       exponentials of S(t) and O^T += V^T(t) P^T(t);
//   (C) wait until only this step's DMAs are in flight, one barrier.
// S^T's rows (keys) are read from K in the order pi = swap of key groups
// 4-7 and 8-11 in every 16, so the accumulator lane layout of S^T is the
// MFMA B-operand layout of P^T with keys in natural order.
//
// The last 512 query rows of a head (the text rows, which keep every
// kv-block, so their groups carry the longest lists) can be split by keys:
// nsplit work-groups per such group each take a contiguous part of its union
// list and store an unnormalised partial (O, reference maximum, row sum) in
// the caller's workspace; attn_vt_merge then combines the parts
// flash-decoding style.  Otherwise a small head count leaves the whole
// launch waiting on these groups.
#include <type_traits>

#include "attn_vt_core.h"

namespace svgk {
namespace {

using namespace core;

constexpr int kWgRows = 256;     // query rows per work-group
constexpr int kNW = 8;           // waves per work-group

// Row stride (floats) of a partial: O, then the maximum and the sum, padded
// so every row starts 16-byte aligned.
template <int D> constexpr int kPartStride = D + 4;

// COMP (SVG-EAR): after the exact tiles, each work-group walks the centroid
// tiles (64 centroids of skipped blocks each, from Kc / Vct: the centroid
// keys and the key-tiled value sums) that hold a centroid some q-block of the
// group compensates; a q-block masks the centroids of its exact blocks and
// the padding slots past the last block.
template <int D, int BQ, bool DENSE, bool COMP = false, bool KGATHER = false>
__global__ __launch_bounds__(kWgRows * 2, 1)
void attn_fwd_vt(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ Vt,
                 bf16_t *__restrict__ O, const int32_t *__restrict__ row_ptr,
                 const int32_t *__restrict__ kv_idx, int N, int nqb, int nkb, int ngrp,
                 float c /* scale * log2(e) */, const int32_t *__restrict__ labels, int qo_orig, int F, int S,
                 int nsplit, float *__restrict__ part, const bf16_t *__restrict__ Kc,
                 const bf16_t *__restrict__ Vct, uint32_t fm = 0, int fk = 0) {
  constexpr int G = kWgRows / BQ;          // q-blocks per work-group
  using T = DTile<D>;
  constexpr int TB = T::TBYTES;            // K tile bytes == V^T tile bytes
  constexpr int OWN_ALL = (1 << G) - 1;
  // Three LDS stages each for K and V^T.  Separate arrays: the compiler
  // then sees that a DMA into one stage cannot alias reads of another and
  // adds no waits of its own beyond the true dependencies.  Equal arrays are
  // laid out in the order of their mangled names, so the V^T stages (V0..V2)
  // come first, below 64 KB: each V^T read is then a lane register plus an
  // immediate offset, with no address VALU (the K reads above 64 KB need one
  // add per 16-dim step, shared by the tile's two key blocks).
  __shared__ __attribute__((aligned(1024))) char k0[TB], k1[TB], k2[TB], V0[TB], V1[TB], V2[TB];
  __shared__ int ulist[DENSE ? 1 : kMaxKb];
  __shared__ uint32_t bits[DENSE ? 1 : G * kWords];
  __shared__ int wsum[DENSE ? 1 : kWords + 1];

  // Each XCD runs a contiguous slice of the work list (a few heads) in
  // order; within a head the groups go in ascending order, so neighbours
  // that share kv-blocks run together and hit in L2 (reversing the whole
  // order instead doubles the HBM fetch).  A head's last 512 query rows
  // hold its text rows, which keep every kv-block.  Unsplit (nsplit = 1),
  // their groups are about 3x an average one and go first within the head,
  // so that no XCD ends on one.  Split, each is nsplit short work items that
  // go last.
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int nlead = min(ngrp, 512 / kWgRows);
  const int per_head = ngrp + nlead * (nsplit - 1);
  const int h = work / per_head, local = work - h * per_head;
  const int jl = nsplit > 1 ? local - (ngrp - nlead) : local;   // index among the leading items
  const bool lead = jl >= 0 && jl < nlead * nsplit;
  const int lg = lead ? jl / nsplit : 0;             // leading group, 0 = the last group
  const int split = lead ? jl - lg * nsplit : 0;
  const int grp = lead ? ngrp - 1 - lg : (nsplit > 1 ? local : local - nlead);
  const bool parted = lead && nsplit > 1;           // stores a partial for attn_vt_merge
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int gw = wave * 32 / BQ;           // this wave's q-block within the group
  const size_t hoff = (size_t)h * N * D;
  const bf16_t *Qh = Q + hoff, *Kh = K + hoff;
  const bf16_t *Vth = Vt + (size_t)h * nkb * (BK * D);
  bf16_t *Oh = O + hoff;
  const int qrow = grp * kWgRows + wave * 32 + l32;
  // Q and O rows: the executing layout's row qrow, or (qo_orig) the original
  // row it holds: for a temporal head (labels[h] == 1, or every head when
  // labels is NULL) row p*F + f of the video holds frame-major row f*S + p.
  int qsrc = qrow;
  if (qo_orig && (labels == nullptr || labels[h] == 1) && qrow < F * S) {
    const int p = qrow / F, f = qrow - p * F;
    qsrc = f * S + p;
  }

  int nt = nkb;
  if constexpr (!DENSE)
    nt = build_union_list<G, kWgRows * 2>(row_ptr, kv_idx, h, grp, nqb, nkb, tid, lane, wave, ulist, bits, wsum);
  const int ntc = (nkb + 63) >> 6;   // centroid tiles (COMP)
  const int nt_exact = nt;
  if constexpr (COMP) {
    // append the centroid tiles holding a centroid some q-block of the group
    // compensates (flag g: q-block g has one in the tile)
    __shared__ int ntot;
    if (wave == 0) {
      int base = nt;
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      for (int t0 = 0; t0 < ntc; t0 += 64) {
        const int t = t0 + lane;
        int fl = 0;
        if (t < ntc) {
          const int nv = min(64, nkb - 64 * t);
          const uint64_t vm = nv >= 64 ? ~0ull : ((1ull << nv) - 1ull);
#pragma unroll
          for (int g = 0; g < G; ++g) {
            if (grp * G + g < nqb) {
              const uint64_t ex = (uint64_t)bits[g * kWords + 2 * t] | ((uint64_t)bits[g * kWords + 2 * t + 1] << 32);
              if (~ex & vm) fl |= 1 << g;
            }
          }
        }
        const uint64_t bal = __ballot(fl != 0);
        if (fl) ulist[base + __popcll(bal & below)] = t | kCentFlag | (fl << 24);
        base += __popcll(bal);
      }
      if (lane == 0) ntot = base;
    }
    __syncthreads();
    nt = ntot;
  }

  // this work item's part of the union list: entries j0 .. j0 + ntile - 1
  const int j0 = parted ? split * nt / nsplit : 0;
  const int ntile = parted ? (split + 1) * nt / nsplit - j0 : nt;
  // partial slot of this row: O (D floats), then the maximum and the sum
  float *const prow = parted ? part + ((((size_t)h * nlead + lg) * nsplit + split) * kWgRows + wave * 32 + l32) *
                                          kPartStride<D>
                             : nullptr;

  if (ntile == 0) {  // no kept tile in the whole group (or this part): O = 0
    if (parted) {
      for (int dd = hi * 8; dd < D; dd += 16)
#pragma unroll
        for (int u = 0; u < 8; ++u) prow[dd + u] = 0.f;
      if (hi == 0) {
        prow[D] = -INFINITY;
        prow[D + 1] = 0.f;
      }
      return;
    }
    if (qrow < N) {
#pragma unroll
      for (int dd = hi * 8; dd < D; dd += 16)
        *reinterpret_cast<u32x4 *>(Oh + (size_t)qsrc * D + dd) = u32x4{0, 0, 0, 0};
    }
    return;
  }

  // entry j of the union: kv-block | flags << 24; past the end it repeats the
  // last entry (those DMAs land in free stages and are never read).  The LDS
  // read and the move to a scalar register are separate so a step can issue
  // the read early and take the value late.
  auto ent_raw = [&](int j) -> int {
    const int i = j0 + (j < ntile ? j : ntile - 1);
    if constexpr (DENSE) return i | (OWN_ALL << 24);
    else return ulist[i];
  };
  const int own_bit = 1 << (24 + gw);

  bf16x8 qf[D / 16];
  load_q<D>(Qh, qrow < N ? qsrc : -1, hi, qf);
  f32x16 o[D / 32];
  float m_run, l_run;
  auto prep = [&](f32x16 &s0, f32x16 &s1, int e) -> bool {
    bool own = true;
    if constexpr (!DENSE) own = (e & own_bit) != 0;
    if (own && ((e & 0xFFFFFF) + 1) * BK > N) {  // keys past N: only in the last kv-block
      // key offset acc_key_pi(b, r, hi) = acc_key_pi(b, r, 0) + 8 hi: compare
      // the constants against nvalid - 8 hi (no per-key offsets kept live)
      const int nvh = N - (e & 0xFFFFFF) * BK - 8 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (acc_key_pi(0, r, 0) >= nvh) s0[r] = -INFINITY;
        if (acc_key_pi(1, r, 0) >= nvh) s1[r] = -INFINITY;
      }
    }
    return own;
  };
  // centroid tiles (COMP): mask this q-block's exact blocks and the padding
  // slots past the last block
  auto prep_c = [&](f32x16 &s0, f32x16 &s1, int e) -> bool {
    const bool own = (e & own_bit) != 0;
    if (own) {
      // the q-block's exact flags over the tile's 64 centroids and the number
      // that exist are wave-uniform; each lane shifts them to its own keys
      // (k0 + 8 hi, k0 + 32 + 8 hi) and drops flagged or missing centroids
      const int t = e & kCentTileMask;
      const uint32_t w0 = __builtin_amdgcn_readfirstlane(bits[gw * kWords + 2 * t]);
      const uint32_t w1 = __builtin_amdgcn_readfirstlane(bits[gw * kWords + 2 * t + 1]);
      const int nv = nkb - 64 * t;               // centroids that exist in the tile
      auto below = [](int n) -> uint32_t { return n >= 32 ? ~0u : n <= 0 ? 0u : (1u << n) - 1u; };
      const int sh = 8 * hi;
      drop_scores(s0, s1, (w0 >> sh) | ~below(nv - sh), (w1 >> sh) | ~below(nv - 32 - sh));
    }
    return own;
  };
  if constexpr (COMP) {
    // two pipeline passes: the exact tiles with the plain pipeline, then the
    // centroid tiles continuing the same softmax state
    const int nc = nt - nt_exact;
    auto ent_x = [&](int j) -> int { return ulist[j < nt_exact ? j : nt_exact - 1]; };
    auto ent_c = [&](int j) -> int { return ulist[nt_exact + (j < nc ? j : nc - 1)]; };
    if (nt_exact > 0) {
      vt_attend<D, kNW>(nt_exact, ent_x, prep, Kh, Vth, N, k0, k1, k2, V0, V1, V2, qf, wave, lane, c, o, m_run,
                        l_run);
    } else {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
      m_run = -INFINITY;
      l_run = 0.f;
    }
    if (nc > 0) {
      __builtin_amdgcn_s_waitcnt(0);   // the first pass's trailing DMAs land before the stages are reused
      __syncthreads();
      vt_attend<D, kNW>(nc, ent_c, prep_c, Kh, Vth, N, k0, k1, k2, V0, V1, V2, qf, wave, lane, c, o, m_run, l_run,
                        KvBlockRow{}, Centroids{Kc + (size_t)h * ntc * BK * D, Vct + (size_t)h * ntc * D * BK});
    }
  } else if constexpr (KGATHER) {
    // K in the original token order: a permuted head's rows gathered by the
    // tile DMA; any other head's K is already in its executing layout
    __shared__ int kring[4 * BK];
    if (F > 1 && (labels == nullptr || labels[h] == 1)) {
      const int jq = lane / F;
      vt_attend<D, kNW>(ntile, ent_raw, prep, Kh, Vth, N, k0, k1, k2, V0, V1, V2, qf, wave, lane, c, o, m_run,
                        l_run, GatherRows{kring, F, S, N, fm, fk, jq, lane - jq * F});
    } else {
      vt_attend<D, kNW>(ntile, ent_raw, prep, Kh, Vth, N, k0, k1, k2, V0, V1, V2, qf, wave, lane, c, o, m_run,
                        l_run);
    }
  } else {
    vt_attend<D, kNW>(ntile, ent_raw, prep, Kh, Vth, N, k0, k1, k2, V0, V1, V2, qf, wave, lane, c, o, m_run,
                      l_run);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may land after the work-group ends
  if (parted) {
    const float lt = l_run + __shfl_xor(l_run, 32);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4 *>(prow + 32 * db + 8 * g + 4 * hi) =
            f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
    if (hi == 0) {
      prow[D] = m_run;
      prow[D + 1] = lt;
    }
    return;
  }
  store_o<D>(qrow < N ? Oh + (size_t)qsrc * D : nullptr, o, l_run, hi);
}

// Combine the nsplit partials of each row of the leading groups:
// O = sum_s w_s O_s / sum_s w_s l_s with w_s = exp2((m_s - M) c), M the
// largest m_s; rows with no kept key get O = 0.  One work-group per row.
template <int D>
__global__ __launch_bounds__(D)
void attn_vt_merge(const float *__restrict__ part, bf16_t *__restrict__ O, int N, int ngrp, int nlead, int nsplit,
                   float c, const int32_t *__restrict__ labels, int qo_orig, int F, int S) {
  const int r = blockIdx.x, lg = blockIdx.y, h = blockIdx.z, e = threadIdx.x;
  const int qrow = (ngrp - 1 - lg) * kWgRows + r;
  if (qrow >= N) return;
  int qsrc = qrow;
  if (qo_orig && (labels == nullptr || labels[h] == 1) && qrow < F * S) {
    const int p = qrow / F, f = qrow - p * F;
    qsrc = f * S + p;
  }
  const float *base = part + (((size_t)h * nlead + lg) * nsplit * kWgRows + r) * kPartStride<D>;
  const size_t stride = (size_t)kWgRows * kPartStride<D>;   // between the parts of one row
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, base[s * stride + D]);
  float acc = 0.f, L = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float *ps = base + s * stride;
      const float w = fast_exp2((ps[D] - M) * c);
      L += w * ps[D + 1];
      acc += w * ps[e];
    }
  }
  O[((size_t)h * N + qsrc) * D + e] = f32_to_bf16(L > 0.f ? acc / L : 0.f);
}

// Parts per leading group of a sparse launch: about 48 tiles each (near a
// typical group's list), at most 16.  None for a dense launch (every group
// has the same list), at 48 kv-blocks or fewer, or when the launch is more
// than kSplitRounds rounds of work-groups deep: the leading groups, started
// first, then end long before the rest, and splitting them only costs L2
// hits (at the HunyuanVideo layer shape, 44 rounds: 1.5x the HBM fetch of
// the whole launch for a 0.3% shorter run).
constexpr int kNumCu = 256;
constexpr int kSplitRounds = 8;
int attn_vt_nsplit(const Dims &dm, int ngrp, bool dense) {
  const int nkb = (dm.N + BK - 1) / BK;
  if (dense || (long long)dm.H * ngrp > (long long)kSplitRounds * kNumCu) return 1;
  return max(1, min(16, (nkb + 47) / 48));
}

template <int D, int BQ>
hipError_t launch_vt(const Dims &dm, const void *Q, const void *K, const void *Vt, void *O,
                     const int32_t *row_ptr, const int32_t *kv_idx, float c, const int32_t *labels, int qo_orig,
                     float *part, hipStream_t st, bool k_orig = false) {
  constexpr int G = kWgRows / BQ;
  const int nqb = (dm.N + BQ - 1) / BQ, nkb = (dm.N + BK - 1) / BK;
  const int ngrp = (nqb + G - 1) / G;
  if (dm.H * ngrp == 0) return hipSuccess;
  const int nlead = min(ngrp, 512 / kWgRows);
  // The leading (text) groups keep every kv-block: split them by keys when
  // the caller gives the partials' workspace.
  const int nsplit = part == nullptr ? 1 : attn_vt_nsplit(dm, ngrp, row_ptr == nullptr);
  const int grid = dm.H * (ngrp + nlead * (nsplit - 1));
  if (k_orig) {
    // r / F by a multiply: fk = floor(log2 F), fm = ceil(2^(32+fk) / F); a
    // power of two takes fm = 2^31 and fk - 1 (exact: a shift); F = 1 is
    // the identity and never divides
    const int F = dm.F > 1 ? dm.F : 2;
    int fk = 0;
    while ((2 << fk) <= F) ++fk;
    uint32_t fm;
    if ((F & (F - 1)) == 0) {
      fm = 0x80000000u;
      fk -= 1;
    } else {
      const uint64_t one = 1;
      fm = (uint32_t)(((one << (32 + fk)) + F - 1) / F);
    }
    hipLaunchKernelGGL((attn_fwd_vt<D, BQ, false, false, true>), dim3(grid), dim3(kWgRows * 2), 0, st,
                       (const bf16_t *)Q, (const bf16_t *)K, (const bf16_t *)Vt, (bf16_t *)O, row_ptr, kv_idx, dm.N,
                       nqb, nkb, ngrp, c, labels, qo_orig, dm.F, dm.S, nsplit, part, nullptr, nullptr, fm, fk);
  } else if (row_ptr == nullptr)
    hipLaunchKernelGGL((attn_fwd_vt<D, BQ, true>), dim3(grid), dim3(kWgRows * 2), 0, st, (const bf16_t *)Q,
                       (const bf16_t *)K, (const bf16_t *)Vt, (bf16_t *)O, row_ptr, kv_idx, dm.N, nqb, nkb, ngrp,
                       c, labels, qo_orig, dm.F, dm.S, nsplit, part, nullptr, nullptr);
  else
    hipLaunchKernelGGL((attn_fwd_vt<D, BQ, false>), dim3(grid), dim3(kWgRows * 2), 0, st, (const bf16_t *)Q,
                       (const bf16_t *)K, (const bf16_t *)Vt, (bf16_t *)O, row_ptr, kv_idx, dm.N, nqb, nkb, ngrp,
                       c, labels, qo_orig, dm.F, dm.S, nsplit, part, nullptr, nullptr);
  if (nsplit > 1)
    hipLaunchKernelGGL((attn_vt_merge<D>), dim3(kWgRows, nlead, dm.H), dim3(D), 0, st, part, (bf16_t *)O, dm.N,
                       ngrp, nlead, nsplit, c, labels, qo_orig, dm.F, dm.S);
  return hipGetLastError();
}

template <int D, int BQ>
hipError_t launch_vt_ear(const Dims &dm, const void *Q, const void *K, const void *Vt, const void *Kc, const void *Vct,
                         void *O, const int32_t *row_ptr, const int32_t *kv_idx, float c, const int32_t *labels,
                         hipStream_t st) {
  constexpr int G = kWgRows / BQ;
  const int nqb = (dm.N + BQ - 1) / BQ, nkb = (dm.N + BK - 1) / BK;
  const int ngrp = (nqb + G - 1) / G;
  if (dm.H * ngrp == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_fwd_vt<D, BQ, false, true>), dim3(dm.H * ngrp), dim3(kWgRows * 2), 0, st,
                     (const bf16_t *)Q, (const bf16_t *)K, (const bf16_t *)Vt, (bf16_t *)O, row_ptr, kv_idx, dm.N,
                     nqb, nkb, ngrp, c, labels, 1, dm.F, dm.S, 1, nullptr, (const bf16_t *)Kc, (const bf16_t *)Vct);
  return hipGetLastError();
}

}  // namespace

int attn_vt_max_kv_blocks() { return kMaxKb; }

// The exact tiles and the centroid tiles share one union list.
int attn_ear_max_kv_blocks() { return kMaxKb - kMaxKb / 64; }

hipError_t launch_attn_vt_ear(const Dims &dm, const void *Q, const void *K, const void *Vt, const void *Kc,
                              const void *Vct, void *O, const int32_t *row_ptr, const int32_t *kv_idx, int bq,
                              float scale, const int32_t *labels, hipStream_t st) {
  const float c = scale * kLog2e;
  if (dm.d == 128 && bq == 128) return launch_vt_ear<128, 128>(dm, Q, K, Vt, Kc, Vct, O, row_ptr, kv_idx, c, labels, st);
  if (dm.d == 128 && bq == 64) return launch_vt_ear<128, 64>(dm, Q, K, Vt, Kc, Vct, O, row_ptr, kv_idx, c, labels, st);
  if (dm.d == 64 && bq == 128) return launch_vt_ear<64, 128>(dm, Q, K, Vt, Kc, Vct, O, row_ptr, kv_idx, c, labels, st);
  if (dm.d == 64 && bq == 64) return launch_vt_ear<64, 64>(dm, Q, K, Vt, Kc, Vct, O, row_ptr, kv_idx, c, labels, st);
  return hipErrorInvalidValue;
}

size_t attn_vt_ws_bytes(const Dims &dm, int bq, int bk) {
  if (bk != BK || (bq != 64 && bq != 128) || dm.N < 1 || dm.H < 1 || (dm.d != 64 && dm.d != 128)) return 0;
  const int ngrp = ((dm.N + bq - 1) / bq + kWgRows / bq - 1) / (kWgRows / bq);
  const int nsplit = attn_vt_nsplit(dm, ngrp, false);
  if (nsplit == 1) return 0;
  const int nlead = min(ngrp, 512 / kWgRows);
  return (size_t)dm.H * nlead * nsplit * kWgRows * (dm.d + 4) * sizeof(float);
}

hipError_t launch_attn_vt(const Dims &dm, const void *Q, const void *K, const void *Vt, void *O,
                          const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk, float scale,
                          hipStream_t st, bool qo_orig, const int32_t *labels, void *ws) {
  const float c = scale * kLog2e;
  const int qo = qo_orig ? 1 : 0;
  float *const part = static_cast<float *>(ws);
  if (bk != BK) return hipErrorInvalidValue;
  if (dm.d == 128 && bq == 128)
    return launch_vt<128, 128>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, qo, part, st);
  if (dm.d == 128 && bq == 64)
    return launch_vt<128, 64>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, qo, part, st);
  if (dm.d == 64 && bq == 128)
    return launch_vt<64, 128>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, qo, part, st);
  if (dm.d == 64 && bq == 64)
    return launch_vt<64, 64>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, qo, part, st);
  return hipErrorInvalidValue;
}

// The block-sparse launch with Q, K and O in the original token order (K
// rows gathered by the tile DMA).
hipError_t launch_attn_vt_korig(const Dims &dm, const void *Q, const void *K, const void *Vt, void *O,
                                const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk, float scale,
                                const int32_t *labels, void *ws, hipStream_t st) {
  const float c = scale * kLog2e;
  float *const part = static_cast<float *>(ws);
  if (bk != BK || row_ptr == nullptr) return hipErrorInvalidValue;
  if (dm.d == 128 && bq == 128)
    return launch_vt<128, 128>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, 1, part, st, true);
  if (dm.d == 128 && bq == 64)
    return launch_vt<128, 64>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, 1, part, st, true);
  if (dm.d == 64 && bq == 128)
    return launch_vt<64, 128>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, 1, part, st, true);
  if (dm.d == 64 && bq == 64)
    return launch_vt<64, 64>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, labels, 1, part, st, true);
  return hipErrorInvalidValue;
}

}  // namespace svgk
