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

#include "attn_vt_core.h"

namespace svgk {
namespace {

using namespace core;

constexpr int kWgRows = 256;     // query rows per work-group
constexpr int kNW = 8;           // waves per work-group

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

  int nt = nkb;
  if constexpr (!DENSE)
    nt = build_union_list<G, kWgRows * 2>(row_ptr, kv_idx, h, grp, nqb, nkb, tid, lane, wave, ulist, bits, wsum);

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
  vt_dma_offsets<D, kNW>(wave, lane, vdma);
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
    constexpr int NKS = D / 16;            // QK steps of a tile
    constexpr int PER = 32 / NKS;          // scores of S(it) per loop step
    constexpr int LEAD = 2;                // QK steps issued before the statistics
    // DMAs of V(it+2) and K(it+3) into the stages PV(it-1) and QK(it)
    // released.  Their 2*PK instructions are spread over the loop steps
    // below: issued back to back by every wave right after the barrier, they
    // queue up in the load unit and hold the waves at issue.
    const int kb_k = e3 & 0xFFFFFF, kb_v = e2 & 0xFFFFFF;
    const int kleft = (N - kb_k * BK) * T::ROWB;
    const __amdgpu_buffer_rsrc_t rk =
        tile_rsrc(reinterpret_cast<const char *>(Kh) + (size_t)kb_k * TB, kleft < TB ? kleft : TB);
    const __amdgpu_buffer_rsrc_t rv = tile_rsrc(reinterpret_cast<const char *>(Vth) + (size_t)kb_v * TB, TB);
    auto dma_slot = [&](int ks) {
#pragma unroll
      for (int i = 0; i < 2 * PK; ++i) {
        if (ks != i * (D / 16) / (2 * PK)) continue;
        if (i & 1) dma_block(rv, Vdst, wave * PK + (i >> 1), vdma[i >> 1]);
        else dma_block(rk, Kdst, wave * PK + (i >> 1), kdma[i >> 1]);
      }
    };
    const int e4_raw = ent_raw(it + 4);
    f32x16 n0 = f32x16{}, n1 = f32x16{};
    auto kread = [&](int q, bf16x8 &a0, bf16x8 &a1) {
      a0 = *reinterpret_cast<const bf16x8 *>(Kn + koff[q]);
      a1 = *reinterpret_cast<const bf16x8 *>(Kn + koff[q] + 32 * T::ROWB);
    };
    bf16x8 kl0[LEAD], kl1[LEAD];
#pragma unroll
    for (int q = 0; q < LEAD; ++q) kread(q, kl0[q], kl1[q]);
    __builtin_amdgcn_sched_barrier(0);

    // (A) statistics of S(it), overlapped with the first QK MFMAs of S(it+1).
    // A tile this wave's q-block does not keep contributes nothing: its
    // exponentials are taken as exp2(x*0 - inf) = 0.  Keys past N exist only
    // in the last kv-block.
    n0 = mfma32(kl0[0], qf[0], n0);
    n1 = mfma32(kl1[0], qf[0], n1);
    bool own = true;
    if constexpr (!DENSE) own = (e0 & own_bit) != 0;
    // (scores of a tile this wave does not keep stay finite: exp2(x*0 - inf))
    if (own && ((e0 & 0xFFFFFF) + 1) * BK > N) {
      const int nvalid = N - (e0 & 0xFFFFFF) * BK;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (acc_key_pi(0, r, hi) >= nvalid) s0[r] = -INFINITY;
        if (acc_key_pi(1, r, hi) >= nvalid) s1[r] = -INFINITY;
      }
    }
    float mx = lane_max_tree(s0, s1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 1; q < LEAD; ++q) {
      n0 = mfma32(kl0[q], qf[q], n0);
      n1 = mfma32(kl1[q], qf[q], n1);
    }
    mx = half_swap_max(mx);
    if (!own) mx = -INFINITY;
    const float alpha = update_ref(mx, c, m_run, l_run);
    const float cc = own ? c : 0.f;
    const float mc = !own ? INFINITY : (m_run == -INFINITY) ? 0.f : m_run * c;
    bf16x8 ka0, ka1;
    kread(LEAD, ka0, ka1);
    __builtin_amdgcn_sched_barrier(0);
    rescale<D>(o, alpha);

    // (B) NKS hand-ordered steps (sched_barrier fences): step ks issues the
    // two MFMAs of S(it+1) for QK step ks + LEAD (K operands read one step
    // ahead), the exponentials of PER scores of S(it), and, once a 16-key
    // chunk of P(it) is complete, its O^T += V^T P^T MFMAs.
    uint32_t pw[16];
    float rs = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int q = ks + LEAD;
      dma_slot(ks);
      bf16x8 kn0 = ka0, kn1 = ka1;
      if (q + 1 < NKS) kread(q + 1, kn0, kn1);
      if (q < NKS) {
        n0 = mfma32(ka0, qf[q], n0);
        n1 = mfma32(ka1, qf[q], n1);
      }
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
