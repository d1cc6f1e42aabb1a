// Variable-size attention over cluster pairs with the selected keys gathered
// exactly (the SVG2 dynamic attention kernel: the Sparse-VideoGen write-up's
// "Three generations" and install sections; HyperVAttention's Problem
// section: irregular cluster blocks waste tile capacity in tiled kernels).
//
// Inputs in cluster order: query cluster i is rows q_offs[i] .. q_offs[i+1]
// of Qp, key cluster j rows k_offs[j] .. k_offs[j+1] of Kp and Vp (both
// row-major).  A query of cluster i attends exactly the keys of its
// selected clusters.  One work-group takes BQ rows of one query cluster and
// walks the concatenation of its selected key ranges in 64-key tiles, so a
// tile holds selected keys only (the last one is ragged).  The source row of
// every key of the concatenation sits in an LDS table; the tile DMA (global
// to LDS, one 16-byte unit per lane) takes each lane's row from it, so K and
// V rows are gathered on the way in with no search and no register staging.
// V^T operands come from the row-major V tile through transposing LDS reads.
// A concatenation longer than the table is walked in chunks that continue
// the same softmax state.  Output rows go back to the original order through
// q_perm.
#include "attn_core.h"

namespace svgk {
namespace {

using namespace core;

template <int D>
constexpr int vg_cap() { return D == 64 ? 4096 : 2048; }   // keys of the concatenation per row table

// Inclusive sum over the work-group's NT threads; tmp holds NW + 1 ints.  All
// threads call it together; tmp[NW] holds the total after the caller's next
// barrier.
template <int NW>
__device__ __forceinline__ int vg_inclusive_sum(int x, int lane, int wave, int *tmp) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    before += v < wave ? tmp[v] : 0;
    total += tmp[v];
  }
  __syncthreads();
  tmp[NW] = total;
  return x + before;
}

// Buffer resource over n bytes at p (units past n read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t vg_rsrc(const bf16_t *p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t *>(p), (short)0, n, 0x00020000);
}

// One 64-row tile of gathered rows into LDS: lane's unit i is row
// rows[base + urow[i]] at byte col[i] of the row.
template <int D, int NW, int PW>
__device__ __forceinline__ void vg_dma(const bf16_t *head, int N, const int *rows, int base, const int (&urow)[PW],
                                       const int (&col)[PW], char *dst, int wave) {
  const __amdgpu_buffer_rsrc_t rs = vg_rsrc(head, N * DTile<D>::ROWB);
#pragma unroll
  for (int i = 0; i < PW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t *)(dst + (wave * PW + i) * 1024), 16,
                                             rows[base + urow[i]] * DTile<D>::ROWB + col[i], 0, 0, 0);
}

template <int D, int BQ>
__global__ __launch_bounds__(BQ / 32 * 64, 2)
void varlen_gather(const bf16_t *__restrict__ Qp, const bf16_t *__restrict__ Kp, const bf16_t *__restrict__ Vp,
                   const int32_t *__restrict__ q_offs, const int32_t *__restrict__ k_offs, int kq, int kk,
                   const int32_t *__restrict__ pair_ptr, const int32_t *__restrict__ pair_idx,
                   const int32_t *__restrict__ q_perm, int N, float c, bf16_t *__restrict__ O) {
  constexpr int NW = BQ / 32, NT = 64 * NW;
  using T = DTile<D>;
  constexpr int TB = T::TBYTES;
  constexpr int PW = T::BLOCKS / NW;          // DMA instructions per wave per tile
  constexpr int CAP = vg_cap<D>();
  static_assert(T::BLOCKS % NW == 0, "tile DMA blocks must split over the waves");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TB];   // K0 K1 V0 V1
  __shared__ int rows[CAP + BK];              // source row of each key of the chunk (padded to a tile)
  __shared__ int segv[257];                   // start of each selected range in the concatenation
  __shared__ int segr[256];                   // its first row in Kp / Vp
  __shared__ int tmp[NW + 1];
  __shared__ int s_cl, s_r0, s_r1, s_p0, s_p1;
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // 1. this work-group's (query cluster, BQ-row chunk); each thread also
  // loads its cluster's pair-list bounds, so the finder hands them on
  const int32_t *qo = q_offs + (size_t)h * (kq + 1);
  const int32_t *ptr = pair_ptr + (size_t)h * (kq + 1);
  if (tid == 0) s_cl = -1;
  {
    const int t = blockIdx.x;
    int done = 0;
    for (int i0 = 0; i0 < kq; i0 += NT) {
      const int i = i0 + tid;
      int a = 0, b = 0, pa = 0, pb = 0;
      if (i < kq) {
        a = qo[i];
        b = qo[i + 1];
        pa = ptr[i];
        pb = ptr[i + 1];
      }
      const int nch = (b - a + BQ - 1) / BQ;
      const int incl = done + vg_inclusive_sum<NW>(nch, lane, wave, tmp);
      if (t >= incl - nch && t < incl) {     // at most one thread
        s_cl = i;
        s_r0 = a + (t - (incl - nch)) * BQ;
        s_r1 = min(b, s_r0 + BQ);
        s_p0 = pa;
        s_p1 = pb;
      }
      __syncthreads();
      done += tmp[NW];
      if (done > t) break;                   // uniform
    }
  }
  __syncthreads();
  const int cl = s_cl;
  if (cl < 0) return;                        // past the head's last chunk (uniform)
  const int r0 = s_r0, r1 = s_r1;
  // the wave's 32 query rows and their output rows, loaded now so that the
  // loads overlap the dependent loads of step 2
  const size_t hoff = (size_t)h * N * D;
  const int qrow = r0 + wave * 32 + l32;
  const bool qvalid = qrow < r1;
  bf16x8 qf[D / 16];
  load_q<D>(Qp + hoff, qvalid ? qrow : -1, hi, qf);
  const int dst = !qvalid ? -1 : q_perm ? q_perm[(size_t)h * N + qrow] : qrow;

  // 2. the selected ranges, laid end to end
  const int32_t *sel = pair_idx + (size_t)h * kq * kk + s_p0;
  const int nsel = s_p1 - s_p0;
  const int32_t *ko = k_offs + (size_t)h * (kk + 1);
  {
    int run = 0;
    for (int m0 = 0; m0 < nsel; m0 += NT) {
      const int m = m0 + tid;
      int len = 0, first = 0;
      if (m < nsel) {
        const int j = sel[m];
        first = ko[j];
        len = ko[j + 1] - first;
      }
      const int incl = run + vg_inclusive_sum<NW>(len, lane, wave, tmp);
      if (m < nsel) {
        segv[m] = incl - len;
        segr[m] = first;
      }
      __syncthreads();
      run += tmp[NW];
    }
    if (tid == 0) segv[nsel] = run;
  }
  __syncthreads();
  const int nkeys = segv[nsel];

  // 3. the output accumulators
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Tile DMA through buffer resources over the head's rows (every gathered
  // row is < N, so no unit leaves the range); lane's unit i of a tile is row
  // urow[i] of the tile at byte kcol / vcol[i] of the row (the swizzles of
  // the row-major K and V tiles).
  const bf16_t *Kh = Kp + hoff, *Vh = Vp + hoff;
  int urow[PW], kcol[PW], vcol[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int p = (wave * PW + i) * 64 + lane;
    const int row = p / T::CPR, pc = p % T::CPR;
    urow[i] = row;
    kcol[i] = (pc ^ swz_k<D>(row)) * 16;
    vcol[i] = (pc ^ swz_v<D>(row)) * 16;
  }
  int koff[D / 16], voff[D / 32];
  k_offsets<D>(l32, hi, koff);
  v_offsets<D>(lane, voff);

  // 4. the concatenation in chunks of at most CAP keys
  for (int c0 = 0; c0 < nkeys; c0 += CAP) {
    const int cn = min(CAP, nkeys - c0);
    const int ntile = (cn + BK - 1) / BK;
    // row table: thread t takes keys [t*per, (t+1)*per) of the chunk (one
    // search for its first segment, then a walk); the padding up to a whole
    // tile repeats the last key's row (its scores are masked)
    {
      const int per = (cn + NT - 1) / NT;
      const int k0 = tid * per, k1 = min(cn, k0 + per);
      if (k0 < k1) {
        int lo = 0, hi_ = nsel - 1;          // last segment with segv <= c0 + k0
        const int v0 = c0 + k0;
        while (lo < hi_) {
          const int mid = (lo + hi_ + 1) >> 1;
          if (segv[mid] <= v0) lo = mid; else hi_ = mid - 1;
        }
        int m = lo;
        for (int k = k0; k < k1; ++k) {
          const int v = c0 + k;
          while (segv[m + 1] <= v) ++m;      // empty ranges are skipped
          rows[k] = segr[m] + (v - segv[m]);
        }
      }
      __syncthreads();
      if (tid < ntile * BK - cn) rows[cn + tid] = rows[cn - 1];
      __syncthreads();
    }

    auto dma = [&](const bf16_t *head, const int (&col)[PW], int tile, char *dst) {
      vg_dma<D, NW, PW>(head, N, rows, tile * BK, urow, col, dst, wave);
    };
    auto tile_at = [&](int it) { return it < ntile ? it : ntile - 1; };

    // prologue: K(0), V(0), K(1); S(0)
    dma(Kh, kcol, 0, smem);
    dma(Vh, vcol, 0, smem + 2 * TB);
    dma(Kh, kcol, tile_at(1), smem + TB);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16 s0, s1;
    qk_tile_dma<D>(smem, qf, koff, s0, s1);
    float mx = row_max3(s0, s1);
    __syncthreads();                          // every wave is done with K(0) before K(2) lands there

    auto step = [&](auto cur_c, int it) {
      constexpr int CUR = decltype(cur_c)::value, NXT = CUR ^ 1;
      char *const Kc = smem + CUR * TB;
      const char *const Kn = smem + NXT * TB;
      const char *const Vc = smem + (2 + CUR) * TB;
      char *const Vn = smem + (2 + NXT) * TB;
      // (A) the ragged last tile; the reference maximum and the rescale
      if ((it + 1) * BK > cn) {
        mask_tail(s0, s1, cn - it * BK, hi);
        mx = row_max3(s0, s1);
      }
      const float alpha = update_ref(mx, c, m_run, l_run);
      rescale<D>(o, alpha);
      // (B) DMAs of V(it+1) and K(it+2) into the stages PV(it-1) and QK(it)
      // released; D/16 steps: the two MFMAs of S(it+1) for 16 dims, the
      // exponentials of 32/(D/16) scores of S(it), and each completed
      // 16-key chunk's O^T += V^T P^T
      dma(Vh, vcol, tile_at(it + 1), Vn);
      dma(Kh, kcol, tile_at(it + 2), Kc);
      constexpr int NKS = D / 16;
      constexpr int PER = 32 / NKS;
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
          const int idx = ks * PER + e;
          const float x0 = idx < 16 ? s0[idx] : s1[idx - 16];
          const float x1 = idx < 16 ? s0[idx + 1] : s1[idx - 15];
          const float p0 = fast_exp2(__builtin_fmaf(x0, c, -mc));
          const float p1 = fast_exp2(__builtin_fmaf(x1, c, -mc));
          rs += p0 + p1;
          pw[idx >> 1] = pack_bf16x2(p0, p1);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (8 * (j + 1) > (ks + 1) * PER || 8 * (j + 1) <= ks * PER) continue;
          const bf16x8 pj =
              __builtin_bit_cast(bf16x8, u32x4{pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
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
    };
    int it = 0;
    for (; it + 2 <= ntile; it += 2) {
      step(std::integral_constant<int, 0>{}, it);
      step(std::integral_constant<int, 1>{}, it + 1);
    }
    if (it < ntile) step(std::integral_constant<int, 0>{}, it);
    __syncthreads();                          // the row table is rebuilt for the next chunk
  }

  store_o<D>(qvalid ? O + hoff + (size_t)dst * D : nullptr, o, l_run, hi);
}

template <int D, int BQ>
hipError_t launch_vg(const Dims &dm, const void *Qp, const void *Kp, const void *Vp, const int32_t *q_offs,
                     const int32_t *k_offs, int kq, int kk, const int32_t *pair_ptr, const int32_t *pair_idx,
                     const int32_t *q_perm, float c, void *O, hipStream_t st) {
  // a grid row per head: at most ceil(N / BQ) + kq chunks (each cluster's
  // last chunk may be partial); surplus work-groups exit at once.  128 rows
  // (four waves) a work-group at both head dims: at d = 64 each K / V tile
  // then serves twice the rows of 64-row chunks, 17% faster on the SVG2
  // mixture lists despite the more ragged last chunk of a cluster.
  const dim3 grid((dm.N + BQ - 1) / BQ + kq, dm.H), block(BQ / 32 * 64);
  hipLaunchKernelGGL((varlen_gather<D, BQ>), grid, block, 0, st, (const bf16_t *)Qp, (const bf16_t *)Kp,
                     (const bf16_t *)Vp, q_offs, k_offs, kq, kk, pair_ptr, pair_idx, q_perm, dm.N, c, (bf16_t *)O);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_varlen_gather(const Dims &dm, const void *Qp, const void *Kp, const void *Vp,
                                const int32_t *q_offs, const int32_t *k_offs, int kq, int kk,
                                const int32_t *pair_ptr, const int32_t *pair_idx, const int32_t *q_perm,
                                float scale, void *O, hipStream_t st) {
  if (dm.N == 0 || dm.H == 0) return hipSuccess;
  const float c = scale * kLog2e;
  if (dm.d == 128)
    return launch_vg<128, 128>(dm, Qp, Kp, Vp, q_offs, k_offs, kq, kk, pair_ptr, pair_idx, q_perm, c, O, st);
  if (dm.d == 64)
    return launch_vg<64, 128>(dm, Qp, Kp, Vp, q_offs, k_offs, kq, kk, pair_ptr, pair_idx, q_perm, c, O, st);
  return hipErrorInvalidValue;
}

}  // namespace svgk
