// Block masks from head labels, and their compaction into kept-block lists.
//
// Token masks (readings of the SVG1 abstract's spatial / temporal heads),
// stated in each head's executing layout:
//   spatial head (frame-major): a video row of frame f keeps the video keys
//     [max(0, f-ks)*S, min(F, f+ks+1)*S);
//   temporal head (position-major): a video row at position p keeps the
//     video keys [max(0, p*F-wt), min(F*S, p*F+F+wt));
//   every row keeps the text keys [F*S, N); a text row keeps every key.
// Each video row's range starts and ends no earlier than the previous
// row's.  Consecutive rows' ranges overlap or touch.  So the union over the
// rows of a q-block is one range: from the first row's start to the last
// row's end.  Tile (qb, kb) is kept iff the key block meets that range, or
// holds a text key, or the q-block holds a text row.
#include "svg_common.h"

namespace svgk {
namespace {

__global__ __launch_bounds__(256)
void block_mask_kernel(const int32_t *__restrict__ labels, int F, int S, int T, int N, int ks,
                       int wt, int bq, int bk, int nqb, int nkb, uint8_t *__restrict__ mask) {
  const int h = blockIdx.y, qb = blockIdx.x;
  const int64_t FS = (int64_t)F * S;
  const int64_t r0 = (int64_t)qb * bq;
  const int64_t r1 = min((int64_t)N, r0 + bq);
  const bool all = r1 > FS;  // the block holds a text row
  int64_t lo = 0, hi = 0;
  if (!all) {
    const int64_t last = r1 - 1;
    if (labels[h] == 0) {
      const int64_t f0 = r0 / S, f1 = last / S;
      lo = max((int64_t)0, f0 - ks) * S;
      hi = min((int64_t)F, f1 + ks + 1) * S;
    } else {
      const int64_t p0 = r0 / F, p1 = last / F;
      lo = max((int64_t)0, p0 * F - wt);
      hi = min(FS, p1 * F + F + wt);
    }
  }
  uint8_t *row = mask + ((int64_t)h * nqb + qb) * nkb;
  for (int kb = threadIdx.x; kb < nkb; kb += blockDim.x) {
    const int64_t c0 = (int64_t)kb * bk;
    const int64_t c1 = min((int64_t)N, c0 + bk);
    const bool keep = all || (c0 < hi && c1 > lo) || (T > 0 && c1 > FS);
    row[kb] = keep ? 1 : 0;
  }
}

// One wave per bitmap row: number of nonzero entries.
__global__ __launch_bounds__(256)
void count_kernel(const uint8_t *__restrict__ mask, int rows, int nkb, int32_t *__restrict__ counts) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint8_t *m = mask + (int64_t)row * nkb;
  int cnt = 0;
  for (int kb = lane; kb < nkb; kb += 64) cnt += m[kb] != 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
  if (lane == 0) counts[row] = cnt;
}

// Exclusive scan of counts[0..rows) into row_ptr[0..rows] by one work-group.
__global__ __launch_bounds__(1024)
void scan_kernel(const int32_t *__restrict__ counts, int rows, int32_t *__restrict__ row_ptr) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (rows + 1023) / 1024;
  const int a = min(rows, tid * per), b = min(rows, a + per);
  int s = 0;
  for (int i = a; i < b; ++i) s += counts[i];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;  // exclusive prefix of this thread's chunk
  for (int i = a; i < b; ++i) {
    row_ptr[i] = run;
    run += counts[i];
  }
  if (tid == 1023) row_ptr[rows] = part[1023];
}

// One wave per row: write the kept column ids in ascending order.
__global__ __launch_bounds__(256)
void fill_kernel(const uint8_t *__restrict__ mask, int rows, int nkb,
                 const int32_t *__restrict__ row_ptr, int32_t *__restrict__ kv_idx) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint8_t *m = mask + (int64_t)row * nkb;
  int32_t *out = kv_idx + row_ptr[row];
  int base_pos = 0;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = 0; base < nkb; base += 64) {
    const int kb = base + lane;
    const bool keep = kb < nkb && m[kb] != 0;
    const uint64_t bal = __ballot(keep);
    if (keep) out[base_pos + __popcll(bal & below)] = kb;
    base_pos += __popcll(bal);
  }
}

}  // namespace

hipError_t launch_block_mask(const Dims &dm, int ks, int wt, const int32_t *labels, int bq, int bk,
                             uint8_t *mask, hipStream_t st) {
  const int nqb = (dm.N + bq - 1) / bq, nkb = (dm.N + bk - 1) / bk;
  if (nqb == 0 || dm.H == 0) return hipSuccess;
  hipLaunchKernelGGL(block_mask_kernel, dim3(nqb, dm.H), dim3(256), 0, st, labels, dm.F, dm.S,
                     dm.T, dm.N, ks, wt, bq, bk, nqb, nkb, mask);
  return hipGetLastError();
}

size_t compact_ws_bytes(int rows) { return ((size_t)rows * 4 + 255) / 256 * 256; }

hipError_t launch_compact(int rows, int nkb, const uint8_t *mask, int32_t *row_ptr,
                          int32_t *kv_idx, void *ws, hipStream_t st) {
  int32_t *counts = (int32_t *)ws;
  if (rows == 0) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, 0, row_ptr);
    return hipGetLastError();
  }
  const int blocks = (rows + 3) / 4;
  hipLaunchKernelGGL(count_kernel, dim3(blocks), dim3(256), 0, st, mask, rows, nkb, counts);
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, st, counts, rows, row_ptr);
  hipLaunchKernelGGL(fill_kernel, dim3(blocks), dim3(256), 0, st, mask, rows, nkb, row_ptr, kv_idx);
  return hipGetLastError();
}

}  // namespace svgk
