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
#include <type_traits>

#include "attn_core.h"

namespace svgk {
namespace {

using namespace core;

constexpr int kWgRows = 256;     // query rows per work-group
constexpr int kNW = 8;           // waves per work-group
constexpr int kMaxKb = 8192;     // union-list capacity (kv-blocks per head)
constexpr int kWords = kMaxKb / 32;

// (1, 1) in bf16, the second operand of the row-sum dot products
constexpr bf16x2_t kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// s_waitcnt with vmcnt = n and no wait on the other counters (gfx9 encoding).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// Key (0..63) of accumulator value r of block b (0: keys 0-31, 1: 32-63)
// under the K row order pi.
__device__ __forceinline__ int acc_key_pi(int b, int r, int hi) {
  return 32 * b + 16 * (r >> 3) + 8 * hi + (r & 7);
}

// pi(i): row i of a 32-key block of S^T holds key pi(i) (an involution).
__device__ __forceinline__ int key_pi(int i) {
  const int g = (i >> 2) & 3;
  const int gp = (g == 1) ? 2 : (g == 2) ? 1 : g;
  return (i & 16) | (gp << 2) | (i & 3);
}

// K operand offsets for S^T with rows in the pi order.
template <int D>
__device__ __forceinline__ void k_offsets_pi(int l32, int hi, int (&off)[D / 16]) {
  const int row = key_pi(l32);
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    off[ks] = row * DTile<D>::ROWB + (((2 * ks + hi) ^ swz_k<D>(row)) << 4);
}

// V^T tile in LDS: D rows (dims) of 128 bytes (64 keys), 16-byte chunk c of
// row d stored at position c ^ (d & 7).  Operand read of 16-key chunk j for
// this lane: row d = 32*db + l32, chunk 2j + hi; offsets per j, db added as
// an immediate (32 rows = 4 KB).
__device__ __forceinline__ void vt_offsets(int l32, int hi, int (&off)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) off[j] = l32 * 128 + (((2 * j + hi) ^ (l32 & 7)) << 4);
}

// DMA of one tile whose first byte is `src`; units at or past `bytes` read
// as zero (buffer range check on the per-lane offset).
template <int D, int NW>
__device__ __forceinline__ void dma_tile_buf(const char *src, int bytes, char *tile, int wave, const int *off) {
  constexpr int PER_WAVE = DTile<D>::BLOCKS / NW;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(src), (short)0, bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(tile + (wave * PER_WAVE + i) * 1024), 16, off[i],
                                             0, 0, 0);
}

// DMA offsets of the V^T tile: lane's 16-byte unit p = blk*64 + lane lands at
// LDS position p, which holds row p/8, logical chunk (p%8) ^ (row & 7).
template <int D>
__device__ __forceinline__ void vt_dma_offsets(int wave, int lane, int (&off)[DTile<D>::BLOCKS / kNW]) {
  constexpr int PER = DTile<D>::BLOCKS / kNW;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p = (wave * PER + i) * 64 + lane;
    const int row = p >> 3;
    off[i] = row * 128 + (((p & 7) ^ (row & 7)) << 4);
  }
}

template <int D, int BQ, bool DENSE>
__global__ __launch_bounds__(kWgRows * 2, 1)
void attn_fwd_vt(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ Vt,
                 bf16_t *__restrict__ O, const int32_t *__restrict__ row_ptr,
                 const int32_t *__restrict__ kv_idx, int N, int nqb, int nkb, int ngrp,
                 float c /* scale * log2(e) */) {
  constexpr int G = kWgRows / BQ;          // q-blocks per work-group
  using T = DTile<D>;
  constexpr int TB = T::TBYTES;            // K tile bytes == V^T tile bytes
  constexpr int PK = T::BLOCKS / kNW;      // DMA instructions per wave per tile
  constexpr int OWN_ALL = (1 << G) - 1;
  static_assert(T::BLOCKS % kNW == 0, "tile DMA blocks must split over the waves");
  // Three LDS stages each for K and V^T.  Separate arrays: the compiler
  // then sees that a DMA into one stage cannot alias reads of another and
  // adds no waits of its own beyond the true dependencies.
  __shared__ __attribute__((aligned(1024))) char k0[TB], k1[TB], k2[TB], v0[TB], v1[TB], v2[TB];
  auto kst = [&](auto i_c) -> char * {
    constexpr int I = decltype(i_c)::value % 3;
    if constexpr (I == 0) return k0;
    else if constexpr (I == 1) return k1;
    else return k2;
  };
  auto vst = [&](auto i_c) -> char * {
    constexpr int I = decltype(i_c)::value % 3;
    if constexpr (I == 0) return v0;
    else if constexpr (I == 1) return v1;
    else return v2;
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  __shared__ int ulist[DENSE ? 1 : kMaxKb];
  __shared__ uint32_t bits[DENSE ? 1 : G * kWords];
  __shared__ int wsum[DENSE ? 1 : kWords + 1];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int h = work / ngrp, grp = work - h * ngrp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int gw = wave * 32 / BQ;           // this wave's q-block within the group
  const size_t hoff = (size_t)h * N * D;
  const bf16_t *Qh = Q + hoff, *Kh = K + hoff;
  const bf16_t *Vth = Vt + (size_t)h * nkb * (BK * D);
  bf16_t *Oh = O + hoff;
  const int qrow = grp * kWgRows + wave * 32 + l32;

  // ---- the union of the group's kept lists, ascending, with per-q-block flags
  int nt = nkb;
  if constexpr (!DENSE) {
    const int nw = (nkb + 31) >> 5;
    for (int i = tid; i < G * kWords; i += kWgRows * 2) bits[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int qb = grp * G + g;
      if (qb < nqb) {
        const int b = row_ptr[h * nqb + qb], e = row_ptr[h * nqb + qb + 1];
        for (int i = b + tid; i < e; i += kWgRows * 2) {
          const int kb = kv_idx[i];
          atomicOr(&bits[g * kWords + (kb >> 5)], 1u << (kb & 31));
        }
      }
    }
    __syncthreads();
    // per-word counts, exclusive scan by wave 0 (4 words per lane)
    if (wave == 0) {
      int cnt[4], tot = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int w = 4 * lane + k;
        uint32_t u = 0u;
        if (w < nw) {
#pragma unroll
          for (int g = 0; g < G; ++g) u |= bits[g * kWords + w];
        }
        cnt[k] = __builtin_popcount(u);
        tot += cnt[k];
      }
      int incl = tot;
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const int y = __shfl_up(incl, s);
        if (lane >= s) incl += y;
      }
      int run = incl - tot;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        wsum[4 * lane + k] = run;
        run += cnt[k];
      }
      if (lane == 63) wsum[kWords] = incl;
    }
    __syncthreads();
    for (int w = tid; w < nw; w += kWgRows * 2) {
      uint32_t fl[G], u = 0u;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        fl[g] = bits[g * kWords + w];
        u |= fl[g];
      }
      int pos = wsum[w];
      while (u) {
        const int b = __builtin_ctz(u);
        u &= u - 1u;
        int f = 0;
#pragma unroll
        for (int g = 0; g < G; ++g) f |= (int)((fl[g] >> b) & 1u) << g;
        ulist[pos++] = (32 * w + b) | (f << 24);
      }
    }
    nt = wsum[kWords];
    __syncthreads();
  }

  if (nt == 0) {  // no kept tile in the whole group: O = 0
    if (qrow < N) {
#pragma unroll
      for (int dd = hi * 8; dd < D; dd += 16)
        *reinterpret_cast<u32x4 *>(Oh + (size_t)qrow * D + dd) = u32x4{0, 0, 0, 0};
    }
    return;
  }

  // entry j of the union: kv-block | flags << 24; past the end it repeats the
  // last entry (those DMAs land in free stages and are never read).  The LDS
  // read and the move to a scalar register are separate so a step can issue
  // the read early and take the value late.
  auto ent_raw = [&](int j) -> int {
    const int i = j < nt ? j : nt - 1;
    if constexpr (DENSE) return i | (OWN_ALL << 24);
    else return ulist[i];
  };
  auto ent = [&](int j) -> int { return __builtin_amdgcn_readfirstlane(ent_raw(j)); };
  const int own_bit = 1 << (24 + gw);

  bf16x8 qf[D / 16];
  load_q<D>(Qh, qrow < N ? qrow : -1, hi, qf);
  int koff[D / 16], voff[4], kdma[PK], vdma[PK];
  k_offsets_pi<D>(l32, hi, koff);
  vt_offsets(l32, hi, voff);
  dma_offsets<D, kNW, false>(wave, lane, kdma);
  vt_dma_offsets<D>(wave, lane, vdma);
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Tile DMAs through a buffer resource based at the tile: rows past N fall
  // outside the resource's range and read as zero (their scores are masked).
  auto dma_k = [&](int e, char *tile) {
    const int kb = e & 0xFFFFFF;
    const int left = (N - kb * BK) * T::ROWB;
    dma_tile_buf<D, kNW>(reinterpret_cast<const char *>(Kh) + (size_t)kb * TB, left < TB ? left : TB, tile, wave,
                         kdma);
  };
  auto dma_v = [&](int e, char *tile) {
    const int kb = e & 0xFFFFFF;
    dma_tile_buf<D, kNW>(reinterpret_cast<const char *>(Vth) + (size_t)kb * TB, TB, tile, wave, vdma);
  };

  // prologue: K(0..2), V(0..1) in flight; S(0) = K(0) Q^T
  int e0 = ent(0), e1 = ent(1), e2 = ent(2), e3 = ent(3);
  dma_k(e0, k0);
  dma_k(e1, k1);
  dma_k(e2, k2);
  dma_v(e0, v0);
  dma_v(e1, v1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 s0, s1;
  qk_tile_dma<D>(k0, qf, koff, s0, s1);
  float mx = row_max3(s0, s1);
  __syncthreads();  // every wave is done with K(0) before K(3) overwrites it

  int it = 0;
  // One tile; ST = it % 3 is a compile-time constant (the loop is unrolled
  // by three), so every LDS address is a register plus an immediate.
  auto step = [&](auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    char *const Kdst = kst(std::integral_constant<int, ST>{});            // K(it+3)
    const char *const Kn = kst(std::integral_constant<int, ST + 1>{});    // K(it+1)
    const char *const Vc = vst(std::integral_constant<int, ST>{});        // V(it)
    char *const Vdst = vst(std::integral_constant<int, ST + 2>{});        // V(it+2)
    // (A) tile it: not kept by this wave's q-block -> contributes nothing
    // (its exponentials are taken as exp2(x*0 - inf) = 0 below); keys past N
    // exist only in the last kv-block
    bool own = true;
    if constexpr (!DENSE) own = (e0 & own_bit) != 0;
    if (!own) {
      mx = -INFINITY;
    } else if (((e0 & 0xFFFFFF) + 1) * BK > N) {
      const int nvalid = N - (e0 & 0xFFFFFF) * BK;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (acc_key_pi(0, r, hi) >= nvalid) s0[r] = -INFINITY;
        if (acc_key_pi(1, r, hi) >= nvalid) s1[r] = -INFINITY;
      }
      mx = row_max3(s0, s1);
    }
    const float alpha = update_ref(mx, c, m_run, l_run);
    rescale<D>(o, alpha);

    // (B) DMAs, then D/16 hand-ordered steps (sched_barrier fences): step ks
    // issues the two MFMAs of S(it+1) for dims 16ks..16ks+15 (K operands
    // read one step ahead), the exponentials of 32/(D/16) scores of S(it),
    // and, once a 16-key chunk of P(it) is complete, its O^T += V^T P^T MFMAs.
    dma_v(e2, Vdst);
    dma_k(e3, Kdst);
    const int e4_raw = ent_raw(it + 4);
    constexpr int NKS = D / 16;
    constexpr int PER = 32 / NKS;
    const float cc = own ? c : 0.f;
    const float mc = !own ? INFINITY : (m_run == -INFINITY) ? 0.f : m_run * c;
    f32x16 n0 = f32x16{}, n1 = f32x16{};
    uint32_t pw[16];
    float rs = 0.f;
    bf16x8 ka0 = *reinterpret_cast<const bf16x8 *>(Kn + koff[0]);
    bf16x8 ka1 = *reinterpret_cast<const bf16x8 *>(Kn + koff[0] + 32 * T::ROWB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 kn0 = ka0, kn1 = ka1;
      if (ks + 1 < NKS) {
        kn0 = *reinterpret_cast<const bf16x8 *>(Kn + koff[ks + 1]);
        kn1 = *reinterpret_cast<const bf16x8 *>(Kn + koff[ks + 1] + 32 * T::ROWB);
      }
      n0 = mfma32(ka0, qf[ks], n0);
      n1 = mfma32(ka1, qf[ks], n1);
#pragma unroll
      for (int e = 0; e < PER; e += 2) {
        const int idx = ks * PER + e;      // 0..31: s0 then s1
        const float x0 = idx < 16 ? s0[idx] : s1[idx - 16];
        const float x1 = idx < 16 ? s0[idx + 1] : s1[idx - 15];
        const float p0 = fast_exp2(__builtin_fmaf(x0, cc, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(x1, cc, -mc));
        pw[idx >> 1] = pack_bf16x2(p0, p1);
        // row sum of the probabilities as they enter the MFMA (bf16)
        rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[idx >> 1]), kOnesBf16x2, rs, false);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // chunks of P completed by this step
        if (8 * (j + 1) > (ks + 1) * PER || 8 * (j + 1) <= ks * PER) continue;
        const bf16x8 pj = __builtin_bit_cast(bf16x8, u32x4{pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
        bf16x8 va[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          va[db] = *reinterpret_cast<const bf16x8 *>(Vc + voff[j] + db * 32 * 128);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = mfma32(va[db], pj, o[db]);
      }
      ka0 = kn0;
      ka1 = kn1;
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += rs;
    mx = row_max3(n0, n1);

    // (C) K(it+2) and V(it+1), issued one step ago, have landed once at most
    // this step's 2*PK DMAs are outstanding; then every wave's share is in
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * PK));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    s0 = n0;
    s1 = n1;
    e0 = e1;
    e1 = e2;
    e2 = e3;
    e3 = __builtin_amdgcn_readfirstlane(e4_raw);
    ++it;
  };

  while (it + 3 <= nt) {
    step(C0{});
    step(C1{});
    step(C2{});
  }
  if (it < nt) step(C0{});
  if (it < nt) step(C1{});
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may land after the work-group ends
  store_o<D>(qrow < N ? Oh + (size_t)qrow * D : nullptr, o, l_run, hi);
}

template <int D, int BQ>
hipError_t launch_vt(const Dims &dm, const void *Q, const void *K, const void *Vt, void *O,
                     const int32_t *row_ptr, const int32_t *kv_idx, float c, hipStream_t st) {
  constexpr int G = kWgRows / BQ;
  const int nqb = (dm.N + BQ - 1) / BQ, nkb = (dm.N + BK - 1) / BK;
  const int ngrp = (nqb + G - 1) / G;
  const int grid = dm.H * ngrp;
  if (grid == 0) return hipSuccess;
  if (row_ptr == nullptr)
    hipLaunchKernelGGL((attn_fwd_vt<D, BQ, true>), dim3(grid), dim3(kWgRows * 2), 0, st, (const bf16_t *)Q,
                       (const bf16_t *)K, (const bf16_t *)Vt, (bf16_t *)O, row_ptr, kv_idx, dm.N, nqb, nkb, ngrp,
                       c);
  else
    hipLaunchKernelGGL((attn_fwd_vt<D, BQ, false>), dim3(grid), dim3(kWgRows * 2), 0, st, (const bf16_t *)Q,
                       (const bf16_t *)K, (const bf16_t *)Vt, (bf16_t *)O, row_ptr, kv_idx, dm.N, nqb, nkb, ngrp,
                       c);
  return hipGetLastError();
}

}  // namespace

int attn_vt_max_kv_blocks() { return kMaxKb; }

hipError_t launch_attn_vt(const Dims &dm, const void *Q, const void *K, const void *Vt, void *O,
                          const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk, float scale,
                          hipStream_t st) {
  const float c = scale * kLog2e;
  if (bk != BK) return hipErrorInvalidValue;
  if (dm.d == 128 && bq == 128) return launch_vt<128, 128>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, st);
  if (dm.d == 128 && bq == 64) return launch_vt<128, 64>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, st);
  if (dm.d == 64 && bq == 128) return launch_vt<64, 128>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, st);
  if (dm.d == 64 && bq == 64) return launch_vt<64, 64>(dm, Q, K, Vt, O, row_ptr, kv_idx, c, st);
  return hipErrorInvalidValue;
}

}  // namespace svgk
