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

}  // namespace

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
