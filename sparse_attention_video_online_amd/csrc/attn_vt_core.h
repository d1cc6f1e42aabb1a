// Shared pieces of the attention kernels that read V in the key-tiled
// transposed layout (attn_vt.hip, attn_vt64.hip): LDS swizzles and DMA
// offsets of the K and V^T tiles, the K row order pi, softmax helpers, and the
// per-work-group union of the kept-tile lists.
#pragma once

#include "attn_core.h"

namespace svgk {
namespace core {

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

// Maximum of the lane's 32 scores as a tree of three-input maxima (depth 4).
__device__ __forceinline__ float lane_max_tree(const f32x16 &s0, const f32x16 &s1) {
  float a[11];
#pragma unroll
  for (int k = 0; k < 5; ++k) a[k] = fmaxf(fmaxf(s0[3 * k], s0[3 * k + 1]), s0[3 * k + 2]);
  a[5] = fmaxf(fmaxf(s0[15], s1[0]), s1[1]);
#pragma unroll
  for (int k = 0; k < 4; ++k) a[6 + k] = fmaxf(fmaxf(s1[2 + 3 * k], s1[3 + 3 * k]), s1[4 + 3 * k]);
  a[10] = fmaxf(s1[14], s1[15]);
  const float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]), b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float b2 = fmaxf(fmaxf(a[6], a[7]), a[8]), b3 = fmaxf(a[9], a[10]);
  return fmaxf(fmaxf(b0, b1), fmaxf(b2, b3));
}

// Maximum with the partner lane l ^ 32 (the other half of the same query's
// keys), through v_permlane32_swap instead of an LDS permute.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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
// row d stored at position c ^ ((d >> 1) & 7).  The 16 lanes a ds_read_b128
// serves together (rows d..d+15, one logical chunk) then cover all 64 banks:
// rows of one parity start at the same bank and get 8 distinct positions.
// Operand read of 16-key chunk j for this lane: row d = 32*db + l32, chunk
// 2j + hi; offsets per j, db added as an immediate (32 rows = 4 KB).
__device__ __forceinline__ int swz_vt(int d) { return (d >> 1) & 7; }
__device__ __forceinline__ void vt_offsets(int l32, int hi, int (&off)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) off[j] = l32 * 128 + (((2 * j + hi) ^ swz_vt(l32)) << 4);
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

// Buffer resource over one tile whose first byte is `src`; units at or past
// `bytes` read as zero.  One DMA block (1 KB: 64 lanes x 16 bytes) of it goes
// to LDS block `blk` of `tile` with dma_block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char *src, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(src), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void dma_block(__amdgpu_buffer_rsrc_t rsrc, char *tile, int blk, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(tile + blk * 1024), 16, off, 0, 0, 0);
}

// DMA offsets of the V^T tile: lane's 16-byte unit p = blk*64 + lane lands at
// LDS position p, which holds row p/8, logical chunk (p%8) ^ swz_vt(row).
template <int D, int NW>
__device__ __forceinline__ void vt_dma_offsets(int wave, int lane, int (&off)[DTile<D>::BLOCKS / NW]) {
  constexpr int PER = DTile<D>::BLOCKS / NW;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int p = (wave * PER + i) * 64 + lane;
    const int row = p >> 3;
    off[i] = row * 128 + (((p & 7) ^ swz_vt(row)) << 4);
  }
}


// Union of the kept-tile lists of the G q-blocks grp*G .. grp*G+G-1 of head
// h, ascending, as entries kb | flags << 24 (flag g: q-block g keeps kb), in
// ulist; returns their number.  NT threads; bits and wsum are LDS scratch of
// G*kWords and kWords+1 words.  Needs nkb <= kMaxKb.  Contains barriers: every
// thread of the work-group calls it.
template <int G, int NT>
__device__ __forceinline__ int build_union_list(const int32_t *__restrict__ row_ptr,
                                                const int32_t *__restrict__ kv_idx, int h, int grp, int nqb,
                                                int nkb, int tid, int lane, int wave, int *ulist, uint32_t *bits,
                                                int *wsum) {
  const int nw = (nkb + 31) >> 5;
  for (int i = tid; i < G * kWords; i += NT) bits[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int qb = grp * G + g;
    if (qb < nqb) {
      const int b = row_ptr[h * nqb + qb], e = row_ptr[h * nqb + qb + 1];
      for (int i = b + tid; i < e; i += NT) {
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
  for (int w = tid; w < nw; w += NT) {
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
  const int nt = wsum[kWords];
  __syncthreads();
  return nt;
}

}  // namespace core
}  // namespace svgk
