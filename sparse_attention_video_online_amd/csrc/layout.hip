// Frame-major <-> position-major layout permutation, and per-head row
// gathers / scatters by an index list.
//
// The SVG1 abstract's layout transformation lists the F frames of each grid
// position together, row (f, p) -> p*F + f.  A temporal head's keys then
// form a contiguous band.  A row is d elements (128-256 bytes), so the
// transpose of the [F][S] row grid is a row gather.  Each output row reads
// one whole input row.  Both sides are full 16-byte vector accesses
// (coalesced), and no LDS staging is needed.  The copy is HBM-bound.
#include "svg_common.h"

namespace svgk {
namespace {

// One thread moves 16 bytes.  `vpr` = 16-byte vectors per row.
__global__ __launch_bounds__(256)
void layout_kernel(const u32x4 *__restrict__ X, u32x4 *__restrict__ Y,
                   const int32_t *__restrict__ labels, int F, int S, int N, int vpr,
                   int inverse) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)N * vpr;
  if (i >= total) return;
  const int out_row = (int)(i / vpr);
  const int v = (int)(i - (int64_t)out_row * vpr);
  int in_row = out_row;
  const bool perm = labels == nullptr || labels[h] == 1;
  if (perm && out_row < F * S) {
    if (!inverse) {
      // output row r = p*F + f reads frame-major row f*S + p
      const int p = out_row / F, f = out_row - p * F;
      in_row = f * S + p;
    } else {
      // output row t = f*S + p reads position-major row p*F + f
      const int f = out_row / S, p = out_row - f * S;
      in_row = p * F + f;
    }
  }
  const int64_t hoff = (int64_t)h * total;
  Y[hoff + (int64_t)out_row * vpr + v] = X[hoff + (int64_t)in_row * vpr + v];
}

__global__ __launch_bounds__(256)
void permute_rows_kernel(const u32x4 *__restrict__ X, const int32_t *__restrict__ perm,
                         u32x4 *__restrict__ Y, int N, int vpr, int inverse) {
  const int h = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)N * vpr;
  if (i >= total) return;
  const int n = (int)(i / vpr);
  const int v = (int)(i - (int64_t)n * vpr);
  const int src = perm[(int64_t)h * N + n];
  const int64_t hoff = (int64_t)h * total;
  if (!inverse)
    Y[hoff + (int64_t)n * vpr + v] = X[hoff + (int64_t)src * vpr + v];
  else
    Y[hoff + (int64_t)src * vpr + v] = X[hoff + (int64_t)n * vpr + v];
}

// Vt tile (h, kb): the 64 executing-layout rows kb*64.. of head h, transposed
// to [d][64 keys], zero past N.  Mode kVtLabels: executing row r of a
// permuted head reads frame-major row f*S + p (r = p*F + f, video rows
// only).  Mode kVtIdentity: every head keeps its row order.  Mode kVtGather:
// row r of head h is row labels[h*N + r] of that head (labels is then a
// per-head gather index, in range by contract).  Mode kVtFrames:
// every head keeps its token order and each frame (then the text) starts a
// new tile: tile kb < F*nbf (nbf = ceil(S/64) tiles a frame) holds rows
// f*S + 64j .. of frame f = kb / nbf, j = kb % nbf, zero past the frame's
// end; the text tiles follow.  The tile is staged in LDS row-major with a
// padded stride; every global access is a 16-byte vector and consecutive
// threads touch consecutive 16-byte units.
template <int D>
__global__ __launch_bounds__(256)
void vt_kernel(const u32x4 *__restrict__ X, u32x4 *__restrict__ Y, const int32_t *__restrict__ labels,
               int F, int S, int N, int nkb, int mode) {
  constexpr int STR = D + 8;                 // padded row stride (halfwords)
  constexpr int CPR = D / 8;                 // 16-byte units per row
  __shared__ __attribute__((aligned(16))) uint16_t t[64 * STR];
  const int kb = blockIdx.x, h = blockIdx.y;
  const bool frames = mode == kVtFrames;
  const bool perm = mode == kVtLabels && (labels == nullptr || labels[h] == 1);
  const int32_t *gather = mode == kVtGather ? labels + (size_t)h * N : nullptr;
  const int nbf = (S + 63) / 64;
  const u32x4 *Xh = X + (size_t)h * N * CPR;
  for (int u = threadIdx.x; u < 64 * CPR; u += 256) {
    const int row = u / CPR, ch = u - row * CPR;
    int r = kb * 64 + row;
    bool in = r < N;
    if (frames) {
      if (kb < F * nbf) {
        const int f = kb / nbf, rl = (kb - f * nbf) * 64 + row;
        in = rl < S;
        r = f * S + rl;
      } else {
        r = F * S + (kb - F * nbf) * 64 + row;
        in = r < N;
      }
    }
    u32x4 v = u32x4{0, 0, 0, 0};
    if (in) {
      int src = r;
      if (perm && r < F * S) {
        const int p = r / F, f = r - p * F;
        src = f * S + p;
      }
      if (gather) src = gather[r];
      v = Xh[(size_t)src * CPR + ch];
    }
    *reinterpret_cast<u32x4 *>(t + row * STR + ch * 8) = v;
  }
  __syncthreads();
  u32x4 *Yt = Y + ((size_t)h * nkb + kb) * (D * 8);
  for (int u = threadIdx.x; u < D * 8; u += 256) {
    const int d = u >> 3, kc = u & 7;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)t[(8 * kc + 2 * i) * STR + d] | ((uint32_t)t[(8 * kc + 2 * i + 1) * STR + d] << 16);
    Yt[u] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace

hipError_t launch_layout_vt(const Dims &dm, const void *V, void *Vt, const int32_t *labels, hipStream_t st,
                            int mode) {
  const int nkb = mode == kVtFrames ? vt_frame_tiles(dm) : (dm.N + 63) / 64;
  if (dm.N == 0 || dm.H == 0) return hipSuccess;
  if (dm.d == 128)
    hipLaunchKernelGGL(vt_kernel<128>, dim3(nkb, dm.H), dim3(256), 0, st, (const u32x4 *)V, (u32x4 *)Vt, labels,
                       dm.F, dm.S, dm.N, nkb, mode);
  else
    hipLaunchKernelGGL(vt_kernel<64>, dim3(nkb, dm.H), dim3(256), 0, st, (const u32x4 *)V, (u32x4 *)Vt, labels,
                       dm.F, dm.S, dm.N, nkb, mode);
  return hipGetLastError();
}

hipError_t launch_layout(const Dims &dm, int elem_bytes, const void *X, void *Y,
                         const int32_t *labels, bool inverse, hipStream_t st) {
  const int vpr = dm.d * elem_bytes / 16;
  const int64_t total = (int64_t)dm.N * vpr;
  if (total == 0 || dm.H == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(layout_kernel, dim3(blocks, dm.H), dim3(256), 0, st, (const u32x4 *)X,
                     (u32x4 *)Y, labels, dm.F, dm.S, dm.N, vpr, inverse ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_permute_rows(const Dims &dm, int elem_bytes, const void *X, const int32_t *perm,
                               void *Y, bool inverse, hipStream_t st) {
  const int vpr = dm.d * elem_bytes / 16;
  const int64_t total = (int64_t)dm.N * vpr;
  if (total == 0 || dm.H == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(permute_rows_kernel, dim3(blocks, dm.H), dim3(256), 0, st, (const u32x4 *)X,
                     perm, (u32x4 *)Y, dm.N, vpr, inverse ? 1 : 0);
  return hipGetLastError();
}

}  // namespace svgk
