// Block-sparse flash attention, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// Computes, for every q-block of every head, softmax attention over the keys
// of its kept kv-blocks only.  This is the custom sparse kernel of the SVG1
// abstract, on the block-sparse attention with per-block keep flags named in
// the Sparse-VideoGen write-up's install section.  Skipped tiles are never
// loaded.
//
// One work-group = one (head, q-block) of BQ rows, BQ/32 waves of 32 query
// rows.  The work-group walks its list of kept kv-blocks in 64-key tiles:
//   - K and V tiles go from global memory straight into LDS
//     (global_load_lds_dwordx4), double-buffered;
//   - S(t+1) = K(t+1) Q^T is issued on the matrix cores while the vector
//     ALUs run the online softmax of S(t), then O^T += V^T(t) P^T(t);
//   - V^T operands come from row-major V through transposing LDS reads
//     (ds_read_b64_tr_b16);
//   - one barrier per tile, after the DMAs of the next tiles have landed.
// The tile math lives in attn_core.h.  Work-group ids are remapped so that
// consecutive q-blocks of one head run on one XCD and share its L2.
#include <type_traits>

#include "attn_core.h"

namespace svgk {
namespace {

using namespace core;

template <int D, int BQ, bool DENSE>
__global__ __launch_bounds__(BQ / 32 * 64, 2)
void attn_fwd_mfma(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K,
                   const bf16_t *__restrict__ V, bf16_t *__restrict__ O,
                   const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ kv_idx,
                   int N, int nqb, int nkb, float c /* scale * log2(e) */) {
  constexpr int NW = BQ / 32;
  using T = DTile<D>;
  constexpr int TB = T::TBYTES;
  constexpr int PER_WAVE = T::BLOCKS / NW;
  // LDS stages: K0 K1 V0 V1 (64 rows each)
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB];

  // A head's last 512 query rows hold its text rows, which keep every
  // kv-block: their q-blocks go first within the head (each XCD runs a
  // contiguous slice of the work list in order), so that no XCD ends on one
  // of them; the rest follow in ascending order for L2 reuse.
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int h = work / nqb, local = work - h * nqb;
  const int nlead = min(nqb, 512 / BQ);
  const int qb = local < nlead ? nqb - 1 - local : local - nlead;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)h * N * D;
  const bf16_t *Qh = Q + hoff, *Kh = K + hoff, *Vh = V + hoff;
  bf16_t *Oh = O + hoff;

  int t0 = 0, t1 = nkb;
  if (!DENSE) {
    t0 = row_ptr[h * nqb + qb];
    t1 = row_ptr[h * nqb + qb + 1];
  }
  const int qrow = qb * BQ + wave * 32 + l32;

  if (t1 <= t0) {  // no kept tile: O = 0 (uniform over the work-group)
    if (qrow < N) {
#pragma unroll
      for (int dd = hi * 8; dd < D; dd += 16)
        *reinterpret_cast<u32x4 *>(Oh + (size_t)qrow * D + dd) = u32x4{0, 0, 0, 0};
    }
    return;
  }

  bf16x8 qf[D / 16];
  load_q<D>(Qh, qrow < N ? qrow : -1, hi, qf);
  int koff[D / 16], voff[D / 32], kdma[PER_WAVE], vdma[PER_WAVE];
  k_offsets<D>(l32, hi, koff);
  v_offsets<D>(lane, voff);
  dma_offsets<D, NW, false>(wave, lane, kdma);
  dma_offsets<D, NW, true>(wave, lane, vdma);
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int nt = t1 - t0;
  // past the end of the list, tile indices are clamped to the last tile: the
  // extra copies land in buffers nobody reads again and keep the loop body
  // free of branches, so the scheduler can interleave MFMA and VALU work
  auto kb_at = [&](int it) {
    const int i = it < nt ? it : nt - 1;
    return DENSE ? t0 + i : kv_idx[t0 + i];
  };
  // DMA of tile kb of X into LDS stage `tile`; the tile holding key N-1 (the
  // only one that can reach past N) clamps its rows to N-1, whose scores are
  // masked later
  auto dma = [&](const bf16_t *Xh, int kb, char *tile, const int (&off)[PER_WAVE], auto isv) {
    if ((kb + 1) * BK <= N) {
      dma_full_buf<D, NW>(Xh, N * T::ROWB, kb * BK * T::ROWB, tile, wave, off);
    } else {
      dma_tile<D, NW, decltype(isv)::value>(Xh, tile, wave, lane, [=](int j) {
        const int key = kb * BK + j;
        return key < N ? key : N - 1;
      });
    }
  };
  using IsK = std::integral_constant<bool, false>;
  using IsV = std::integral_constant<bool, true>;

  // prologue: K(0), V(0), K(1) in flight; S(0) = K(0) Q^T
  int kb_cur = kb_at(0), kb_nxt = kb_at(1);
  dma(Kh, kb_cur, smem, kdma, IsK{});
  dma(Vh, kb_cur, smem + 2 * TB, vdma, IsV{});
  dma(Kh, kb_nxt, smem + TB, kdma, IsK{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 s0, s1;
  qk_tile_dma<D>(smem, qf, koff, s0, s1);
  float mx = row_max3(s0, s1);
  __syncthreads();  // every wave is done with K(0) before K(2) overwrites it

  // One tile; CUR = it & 1 is a compile-time constant (the loop is unrolled
  // by two), so every LDS address is a register plus an immediate.
  auto step = [&](auto cur_c, int it) {
    constexpr int CUR = decltype(cur_c)::value, NXT = CUR ^ 1;
    char *const Kc = smem + CUR * TB;
    const char *const Kn = smem + NXT * TB;
    const char *const Vc = smem + (2 + CUR) * TB;
    char *const Vn = smem + (2 + NXT) * TB;
    // (A) keys past N exist only in the last kv-block; then the reference
    // maximum, and the rescale of O when it moved
    if ((kb_cur + 1) * BK > N) {
      mask_tail(s0, s1, N - kb_cur * BK, hi);
      mx = row_max3(s0, s1);
    }
    const float alpha = update_ref(mx, c, m_run, l_run);
    rescale<D>(o, alpha);

    // (B) DMAs of V(it+1) and K(it+2) into the stages PV(it-1) and QK(it)
    // released; then, ordered by hand (sched_barrier fences), D/16 steps:
    // step ks issues the two MFMAs of S(it+1) for dims 16ks..16ks+15 (K
    // operands read one step ahead), the exponentials of 32/(D/16) scores of
    // S(it), and, once a 16-key chunk of P(it) is complete, that chunk's
    // O^T += V^T P^T MFMAs.
    const int kb_after = kb_at(it + 2);
    dma(Vh, kb_nxt, Vn, vdma, IsV{});
    dma(Kh, kb_after, Kc, kdma, IsK{});
    constexpr int NKS = D / 16;            // QK steps
    constexpr int PER = 32 / NKS;          // scores of S(it) per step
    const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
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
        const float p0 = fast_exp2(__builtin_fmaf(x0, c, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(x1, c, -mc));
        rs += p0 + p1;
        pw[idx >> 1] = pack_bf16x2(p0, p1);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // chunks of P completed by this step
        if (8 * (j + 1) > (ks + 1) * PER || 8 * (j + 1) <= ks * PER) continue;
        const bf16x8 pj = __builtin_bit_cast(bf16x8, u32x4{pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
        bf16x8 va[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const v4s16 lo = ds_read_tr16(Vc + voff[db] + (16 * j) * T::ROWB);
          const v4s16 hi8 = ds_read_tr16(Vc + voff[db] + (16 * j + 8) * T::ROWB);
          va[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi8, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = mfma32(va[db], pj, o[db]);
      }
      ka0 = kn0;
      ka1 = kn1;
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += rs;
    mx = row_max3(n0, n1);

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    s0 = n0;
    s1 = n1;
    kb_cur = kb_nxt;
    kb_nxt = kb_after;
  };

  int it = 0;
  for (; it + 2 <= nt; it += 2) {
    step(std::integral_constant<int, 0>{}, it);
    step(std::integral_constant<int, 1>{}, it + 1);
  }
  if (it < nt) step(std::integral_constant<int, 0>{}, it);
  store_o<D>(qrow < N ? Oh + (size_t)qrow * D : nullptr, o, l_run, hi);
}

template <int D, int BQ>
hipError_t launch_one(const Dims &dm, const void *Q, const void *K, const void *V, void *O,
                      const int32_t *row_ptr, const int32_t *kv_idx, float c, hipStream_t st) {
  constexpr int NT = BQ / 32 * 64;
  static_assert(DTile<D>::BLOCKS % (BQ / 32) == 0, "tile DMA blocks must split over the waves");
  const int nqb = (dm.N + BQ - 1) / BQ, nkb = (dm.N + BK - 1) / BK;
  const int grid = dm.H * nqb;
  if (grid == 0) return hipSuccess;
  if (row_ptr == nullptr)
    hipLaunchKernelGGL((attn_fwd_mfma<D, BQ, true>), dim3(grid), dim3(NT), 0, st, (const bf16_t *)Q,
                       (const bf16_t *)K, (const bf16_t *)V, (bf16_t *)O, row_ptr, kv_idx, dm.N, nqb, nkb, c);
  else
    hipLaunchKernelGGL((attn_fwd_mfma<D, BQ, false>), dim3(grid), dim3(NT), 0, st, (const bf16_t *)Q,
                       (const bf16_t *)K, (const bf16_t *)V, (bf16_t *)O, row_ptr, kv_idx, dm.N, nqb, nkb, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const Dims &dm, const void *Q, const void *K, const void *V, void *O,
                            const int32_t *row_ptr, const int32_t *kv_idx, int bq, int bk,
                            float scale, hipStream_t st) {
  const float c = scale * kLog2e;
  if (bk != BK) return hipErrorInvalidValue;
  if (dm.d == 128 && bq == 128) return launch_one<128, 128>(dm, Q, K, V, O, row_ptr, kv_idx, c, st);
  if (dm.d == 128 && bq == 64) return launch_one<128, 64>(dm, Q, K, V, O, row_ptr, kv_idx, c, st);
  if (dm.d == 64 && bq == 64) return launch_one<64, 64>(dm, Q, K, V, O, row_ptr, kv_idx, c, st);
  if (dm.d == 64 && bq == 128) return launch_one<64, 128>(dm, Q, K, V, O, row_ptr, kv_idx, c, st);
  return hipErrorInvalidValue;
}

}  // namespace svgk
