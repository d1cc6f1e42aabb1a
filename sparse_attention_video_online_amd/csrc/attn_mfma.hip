// Block-sparse flash attention, bf16 in / fp32 accumulate, on gfx950 MFMA.
//
// Computes, for every q-block of every head, softmax attention over the keys
// of its kept kv-blocks only.  This is the custom sparse kernel of the SVG1
// abstract, on the block-sparse attention with per-block keep flags named in
// the Sparse-VideoGen write-up's install section.  Skipped tiles are never
// loaded.
//
// One work-group = one (head, q-block) of BQ rows, BQ/32 waves of 32 query
// rows.  The work-group walks its list of kept kv-blocks.  Each 64-key tile
// is double-buffered through LDS; the next tile's global loads are issued
// before the current tile's math.  The per-tile math (S^T = K Q^T, online
// softmax, O^T += V^T P^T) lives in attn_core.h.  Work-group ids are
// remapped so that consecutive q-blocks of one head run on one XCD and share
// its L2.
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
  constexpr int NT = BQ / 32 * 64;
  using C = Tile<D, NT>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int h = work / nqb, qb = work - h * nqb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  Regs<D, NT> R;
  int kb = DENSE ? t0 : kv_idx[t0];
  auto rows_of = [&](int kb_) {
    return [=](int j) { const int key = kb_ * BK + j; return key < N ? key : -1; };
  };
  load_tile<D, NT>(Kh, Vh, tid, rows_of(kb), R);
  store_tile<D, NT>(smem, tid, R);
  __syncthreads();

  const int nt = t1 - t0;
  for (int it = 0; it < nt; ++it) {
    const int kbc = kb;
    const bool more = it + 1 < nt;
    if (more) {
      kb = DENSE ? (t0 + it + 1) : kv_idx[t0 + it + 1];
      load_tile<D, NT>(Kh, Vh, tid, rows_of(kb), R);
    }
    const char *Ks = smem + (it & 1) * C::STAGE;
    const char *Vs = Ks + C::KBYTES;

    f32x16 s0, s1;
    qk_tile<D, NT>(Ks, qf, l32, hi, s0, s1);
    if ((kbc + 1) * BK > N) mask_tail(s0, s1, N - kbc * BK, hi);
    bf16x8 pb[4];
    const float alpha = softmax_step(s0, s1, c, m_run, l_run, pb);
    rescale<D>(o, alpha);
    pv_tile<D, NT>(Vs, pb, l32, hi, o);

    if (more) store_tile<D, NT>(smem + ((it + 1) & 1) * C::STAGE, tid, R);
    __syncthreads();
  }
  store_o<D>(qrow < N ? Oh + (size_t)qrow * D : nullptr, o, l_run, hi);
}

template <int D, int BQ>
hipError_t launch_one(const Dims &dm, const void *Q, const void *K, const void *V, void *O,
                      const int32_t *row_ptr, const int32_t *kv_idx, float c, hipStream_t st) {
  constexpr int NT = BQ / 32 * 64;
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
