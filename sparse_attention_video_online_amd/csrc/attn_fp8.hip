// FP8 attention: Q K^T on the gfx950 FP8 matrix cores, P.V in bf16.
//
// The Sparse-VideoGen write-up lists FP8 attention as an open item of its
// plan ("Publication record and the road ahead") without a method, so the
// quantization is this library's definition:
//   - OCP E4M3 codes, round to nearest with ties to even;
//   - one scale per Q token and one per 64-key block of K in the executing
//     layout (the attention's key tile): scale = amax / 448, and a value x
//     becomes round_e4m3(fp32(x * (448 / amax)));
//   - the logit of (query i, key j) is (sum_c q_ic k_jc) * sq_i * sk_b(j) *
//     softmax_scale, accumulated in fp32 on v_mfma_f32_32x32x64_f8f6f4;
//   - the softmax, the bf16 P.V and the output are those of the bf16 kernel.
// The per-token and per-tile scales cost nothing in the softmax: the
// exponent argument is already one FMA per score, whose multiplier becomes
// softmax_scale * log2(e) * sq_i * sk_b per lane and tile.
//
// Kernels:
//   quant_rows_fp8   Q -> codes + per-row scales (any token order);
//   layout_fp8       K -> executing layout (per labels, as the layout
//                    permute) -> codes + per-64-row-block scales;
//   attn_fwd_fp8     the V^T attention of attn_vt.hip with the fp8 QK^T
//                    (d = 128): K tiles of 64 rows x 128 bytes in LDS, four
//                    32x32x64 MFMAs per tile and wave instead of sixteen
//                    32x32x16 bf16 ones.
//
// The FP8 P.V mode codes the other product as well (also this library's
// definition):
//   - V: one scale per channel over the head's tokens, amax_d / 448, codes
//     round_e4m3(fp32(v * (448 / amax_d))), stored key-tiled and transposed
//     (chan_amax, layout_vt_fp8);
//   - P: each probability 2^(y - m) against the lazy reference m (at most
//     2^8, so no scale) coded round_e4m3(fp32(p)) by v_cvt_pk_fp8_f32;
//   - P.V: four 32x32x64 MFMAs per tile and wave over the codes (instead of
//     sixteen bf16 ones), and the row sum as a fifth MFMA of the codes
//     against a block of ones (no vector-ALU sum); the channel scales
//     multiply O once at the end.
#include <type_traits>

#include "attn_vt_core.h"

namespace svgk {
namespace {

using namespace core;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.f;

// fp32 pair -> two E4M3 codes in the low (HI = false) or high half of `old`
// (v_cvt_pk_fp8_f32, round to nearest even).
template <bool HI>
__device__ __forceinline__ int cvt_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// Eight bf16 values (one 16-byte unit) times inv -> eight codes (8 bytes).
__device__ __forceinline__ u32x2 quant8(const u32x4 &w, float inv) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16) * inv;
    f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u) * inv;
  }
  int lo = cvt_fp8x2<false>(f[0], f[1], 0);
  lo = cvt_fp8x2<true>(f[2], f[3], lo);
  int hi = cvt_fp8x2<false>(f[4], f[5], 0);
  hi = cvt_fp8x2<true>(f[6], f[7], hi);
  return u32x2{(uint32_t)lo, (uint32_t)hi};
}

__device__ __forceinline__ float amax8(const u32x4 &w) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(__uint_as_float(w[i] << 16)));
    m = fmaxf(m, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
  }
  return m;
}

// 448 / amax (correctly rounded fp32 division); 0 for an all-zero group.
__device__ __forceinline__ float quant_inv(float amax) { return amax > 0.f ? kE4M3Max / amax : 0.f; }

// One row per group of D/8 lanes (16-byte units), 256 threads.
template <int D>
__global__ __launch_bounds__(256)
void quant_rows_fp8(const u32x4 *__restrict__ X, uint8_t *__restrict__ X8, float *__restrict__ scale, int64_t rows) {
  constexpr int L = D / 8;                       // lanes per row
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / L;
  const int u = (int)(t % L);
  const bool live = row < rows;
  const u32x4 w = live ? X[row * L + u] : u32x4{0, 0, 0, 0};
  float m = amax8(w);
#pragma unroll
  for (int s = 1; s < L; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
  if (!live) return;
  const float inv = quant_inv(m);
  *reinterpret_cast<u32x2 *>(X8 + row * D + u * 8) = quant8(w, inv);
  if (u == 0) scale[row] = m / kE4M3Max;
}

// One work-group per (64-row block of the executing layout, head): rows
// gathered as the layout permute does, amax over the block, codes + scale.
template <int D>
__global__ __launch_bounds__(256)
void layout_fp8(const u32x4 *__restrict__ X, uint8_t *__restrict__ X8, float *__restrict__ scale,
                const int32_t *__restrict__ labels, int F, int S, int N, int nkb) {
  constexpr int CPR = D / 8;                     // 16-byte units per source row
  constexpr int UPT = 64 * CPR / 256;            // units per thread
  __shared__ float red[4];
  const int kb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const bool perm = labels == nullptr || labels[h] == 1;
  const u32x4 *Xh = X + (size_t)h * N * CPR;
  u32x4 w[UPT];
  int rows[UPT];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int unit = tid + 256 * i;
    const int r = kb * 64 + unit / CPR, ch = unit % CPR;
    rows[i] = r;
    w[i] = u32x4{0, 0, 0, 0};
    if (r < N) {
      int src = r;
      if (perm && r < F * S) {
        const int p = r / F, f = r - p * F;
        src = f * S + p;
      }
      w[i] = Xh[(size_t)src * CPR + ch];
    }
    m = fmaxf(m, amax8(w[i]));
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = quant_inv(m);
  uint8_t *Yh = X8 + (size_t)h * N * D;
#pragma unroll
  for (int i = 0; i < UPT; ++i) {
    const int unit = tid + 256 * i;
    if (rows[i] < N) *reinterpret_cast<u32x2 *>(Yh + (size_t)rows[i] * D + (unit % CPR) * 8) = quant8(w[i], inv);
  }
  if (tid == 0) scale[(size_t)h * nkb + kb] = m / kE4M3Max;
}

// ---------------------------------------------------------------------------
// V for the FP8 P.V mode (d = 128).
//
// The V^T code tile of 64 keys is 128 rows (dims) of 64 bytes.  Byte j of a
// row holds key tau(j): j = 32 hi + b holds key 32 (b >> 4) + 16 ((b >> 3) & 1)
// + 8 hi + (b & 7), the order in which a lane of lane half hi holds its 32
// probabilities of a tile after Q K^T (its 16 scores of each 32-key block,
// keys 16 (r >> 3) + 8 hi + (r & 7)).  Then a lane's 32 A-operand bytes (row
// d, bytes 32 hi ..) and its 32 B-operand bytes (its probabilities in
// register order) name the same keys slot by slot.

constexpr int kV8Bytes = 128 * 64;     // V^T code tile: 128 dims x 64 keys
constexpr int kChanRows = 512;         // rows per chan_amax work-group

__device__ __forceinline__ int v8_key(int j) {
  const int hi = j >> 5, b = j & 31;
  return 32 * (b >> 4) + 16 * ((b >> 3) & 1) + 8 * hi + (b & 7);
}

__global__ __launch_bounds__(256)
void zero_f32(float *__restrict__ x, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

// Largest magnitude of each channel (d = 128) over the head's tokens, as
// the bits of a non-negative float (their unsigned order is the float
// order): one work-group per (kChanRows rows, head) takes the maximum of its
// rows and raises amax[h][d] with an atomic maximum (zeroed beforehand).
__global__ __launch_bounds__(256)
void chan_amax(const u32x4 *__restrict__ X, uint32_t *__restrict__ amax, int N) {
  constexpr int D = 128, CPR = D / 8;   // 16 units of 8 dims per row
  __shared__ float red[16][D];
  const int h = blockIdx.y, tid = threadIdx.x;
  const int u = tid & (CPR - 1), r0 = blockIdx.x * kChanRows + (tid >> 4);
  const u32x4 *Xh = X + (size_t)h * N * CPR;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = r0; r < N && r < (int)(blockIdx.x + 1) * kChanRows; r += 16) {
    const u32x4 w = Xh[(size_t)r * CPR + u];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[2 * i] = fmaxf(m[2 * i], fabsf(__uint_as_float(w[i] << 16)));
      m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[tid >> 4][8 * u + i] = m[i];
  __syncthreads();
  if (tid < D) {
    float a = red[0][tid];
    for (int g = 1; g < 16; ++g) a = fmaxf(a, red[g][tid]);
    atomicMax(amax + (size_t)h * D + tid, __float_as_uint(a));
  }
}

// One work-group per (64-key tile of the executing layout, head): the rows
// gathered as the layout permute does, then each 16-byte unit of the code
// tile (row d = u / 4, bytes 16 (u % 4) ..) coded from the channel's amax.
// Keys past N are zero codes.
__global__ __launch_bounds__(256)
void layout_vt_fp8(const u32x4 *__restrict__ X, const float *__restrict__ amax, u32x4 *__restrict__ Y,
                   const int32_t *__restrict__ labels, int F, int S, int N, int nkb) {
  constexpr int D = 128, CPR = D / 8, STR = D + 8;   // padded LDS row (halfwords)
  __shared__ __attribute__((aligned(16))) uint16_t t[64 * STR];
  __shared__ float inv[D];
  const int kb = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const bool perm = labels == nullptr || labels[h] == 1;
  const u32x4 *Xh = X + (size_t)h * N * CPR;
  if (tid < D) inv[tid] = quant_inv(amax[(size_t)h * D + tid]);
  for (int u = tid; u < 64 * CPR; u += 256) {
    const int row = u / CPR, ch = u - row * CPR;
    const int r = kb * 64 + row;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (r < N) {
      int src = r;
      if (perm && r < F * S) {
        const int p = r / F, f = r - p * F;
        src = f * S + p;
      }
      v = Xh[(size_t)src * CPR + ch];
    }
    *reinterpret_cast<u32x4 *>(t + row * STR + ch * 8) = v;
  }
  __syncthreads();
  u32x4 *Yt = Y + ((size_t)h * nkb + kb) * (kV8Bytes / 16);
  for (int u = tid; u < kV8Bytes / 16; u += 256) {
    const int d = u >> 2, j0 = (u & 3) * 16;
    const float s = inv[d];
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = __uint_as_float((uint32_t)t[v8_key(j0 + 4 * i + e) * STR + d] << 16) * s;
      w[i] = (uint32_t)cvt_fp8x2<true>(f[2], f[3], cvt_fp8x2<false>(f[0], f[1], 0));
    }
    Yt[u] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// ---------------------------------------------------------------------------
// The attention (d = 128).

constexpr int kD = 128;
constexpr int kWgRows = 256;
constexpr int kNW = 8;
constexpr int kK8Bytes = 64 * kD;               // fp8 K tile: 64 rows x 128 bytes
constexpr int kVtBytes = DTile<kD>::TBYTES;     // bf16 V^T tile
constexpr int kK8Blocks = kK8Bytes / 1024;      // 1 KB DMA blocks: one per wave
constexpr int kVBlocks = kVtBytes / 1024;       // two per wave
static_assert(kK8Blocks == kNW && kVBlocks == 2 * kNW, "DMA split assumes d = 128 and 8 waves");
static_assert(kV8Bytes / 1024 == kNW, "one DMA block of the V^T code tile per wave");

// K8 tile row r: 16-byte chunk c stored at position c ^ swz8(r).  The 16
// lanes a ds_read_b128 serves (16 keys, one logical chunk) then cover all 64
// banks: rows of one parity share a bank half and get 8 distinct positions.
__device__ __forceinline__ int swz8(int row) { return (row >> 1) & 7; }

// DMA offset (bytes within the tile) of this lane's unit of block `blk`.
__device__ __forceinline__ int k8_dma_offset(int blk, int lane) {
  const int p = blk * 64 + lane;
  const int row = p >> 3, pc = p & 7;
  return row * kD + ((pc ^ swz8(row)) << 4);
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The tile pipeline of vt_attend with the QK^T in fp8: per tile and wave,
// S^T = K8 Q8^T as 2 key blocks x 2 steps of 64 dims.  Operand slot (lane
// half hi, byte b of the 32) of both A (K rows, read from LDS in the order
// pi) and B (the wave's Q rows) holds dim 64*ks + 32*hi + b, so the MFMA's
// reduction pairs equal dims whatever its internal order.  ent_raw / prep
// as vt_attend; tsc(j) gives tile j's K scale (read early, like the entry).
// cq = softmax_scale * log2(e) * this lane's Q scale (> 0).  On return o
// and l_run are the un-normalised output and the lane's partial row sum.
// PV8: V^T is the code tile (Vth points at the head's code tiles), P.V and
// the row sum run on the fp8 matrix cores once the tile's 32 probabilities
// are coded, and l_run is half the row sum (the partner lane holds the same
// sum, and the store adds the two halves).
template <bool PV8, typename EntRaw, typename TileScale, typename Prep>
__device__ __forceinline__ void vt_attend_qk8(int nt, EntRaw ent_raw, TileScale tsc, Prep prep,
                                              const uint8_t *__restrict__ K8h, const void *__restrict__ Vth,
                                              int N, char *k0, char *k1, char *k2, char *v0, char *v1, char *v2,
                                              const i32x8 (&qf)[2], float cq, int wave, int lane,
                                              f32x16 (&o)[kD / 32], float &l_run) {
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
  auto ent = [&](int j) -> int { return __builtin_amdgcn_readfirstlane(ent_raw(j)); };
  const int l32 = lane & 31, hi = lane >> 5;
  // A operand offsets: key row pi(l32) (+32 rows for the second block),
  // logical chunks 4 ks + 2 hi and 4 ks + 2 hi + 1
  const int krow = key_pi(l32);
  int koff[2][2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[ks][u] = krow * kD + (((4 * ks + 2 * hi + u) ^ swz8(krow)) << 4);
  int voff[4], vdma[2];
  if constexpr (PV8) {
    // code tile row d: 16-byte chunk c at position c ^ ((d >> 2) & 3), so the
    // 16 rows of one ds_read_b128 (one logical chunk) cover all 64 banks; a
    // lane reads chunks 2 hi and 2 hi + 1 of row 32 db + l32
    const int sw = (l32 >> 2) & 3;
    voff[0] = l32 * 64 + (((2 * hi) ^ sw) << 4);
    voff[1] = l32 * 64 + (((2 * hi + 1) ^ sw) << 4);
    const int p = wave * 64 + lane;            // DMA unit: LDS position p, row p / 4
    const int row = p >> 2;
    vdma[0] = row * 64 + (((p & 3) ^ ((row >> 2) & 3)) << 4);
  } else {
    vt_offsets(l32, hi, voff);
    vt_dma_offsets<kD, kNW>(wave, lane, vdma);
  }
  const int kdma = k8_dma_offset(wave, lane);
  constexpr int kVTile = PV8 ? kV8Bytes : kVtBytes;
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) o[db] = f32x16{};
  l_run = 0.f;
  f32x16 lsum = f32x16{};     // PV8: the row sum, as the product of the codes with a block of ones
  const i32x8 ones8 = i32x8{0x38383838, 0x38383838, 0x38383838, 0x38383838,
                            0x38383838, 0x38383838, 0x38383838, 0x38383838};   // E4M3 1.0
  float mref_c = -INFINITY;   // reference maximum of the scaled exponent arguments

  auto k_rsrc = [&](int e) {
    const int kb = e & 0xFFFFFF;
    const int left = (N - kb * BK) * kD;
    return tile_rsrc(reinterpret_cast<const char *>(K8h) + (size_t)kb * kK8Bytes, left < kK8Bytes ? left : kK8Bytes);
  };
  auto v_rsrc = [&](int e) {
    const int kb = e & 0xFFFFFF;
    return tile_rsrc(reinterpret_cast<const char *>(Vth) + (size_t)kb * kVTile, kVTile);
  };
  auto dma_k = [&](int e, char *tile) { dma_block(k_rsrc(e), tile, wave, kdma); };
  auto dma_v = [&](int e, char *tile) {
    const auto r = v_rsrc(e);
    if constexpr (PV8) {
      dma_block(r, tile, wave, vdma[0]);
    } else {
      dma_block(r, tile, 2 * wave, vdma[0]);
      dma_block(r, tile, 2 * wave + 1, vdma[1]);
    }
  };
  auto kread = [&](const char *Kt, int ks, int b, i32x8 &a) {
    const i32x4 x = *reinterpret_cast<const i32x4 *>(Kt + koff[ks][0] + b * 32 * kD);
    const i32x4 y = *reinterpret_cast<const i32x4 *>(Kt + koff[ks][1] + b * 32 * kD);
    a = i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  };

  // prologue: K(0..2), V(0..1) in flight; S(0) = K(0) Q^T
  int e0 = ent(0), e1 = ent(1), e2 = ent(2), e3 = ent(3);
  float sc0 = tsc(0), sc1 = tsc(1);
  dma_k(e0, k0);
  dma_k(e1, k1);
  dma_k(e2, k2);
  dma_v(e0, v0);
  dma_v(e1, v1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    i32x8 a0, a1;
    kread(k0, ks, 0, a0);
    kread(k0, ks, 1, a1);
    s0 = mfma_fp8(a0, qf[ks], s0);
    s1 = mfma_fp8(a1, qf[ks], s1);
  }
  __syncthreads();  // every wave is done with K(0) before K(3) overwrites it

  int it = 0;
  auto step = [&](auto st_c) {
    constexpr int ST = decltype(st_c)::value;
    char *const Kdst = kst(std::integral_constant<int, ST>{});            // K(it+3)
    const char *const Kn = kst(std::integral_constant<int, ST + 1>{});    // K(it+1)
    const char *const Vc = vst(std::integral_constant<int, ST>{});        // V(it)
    char *const Vdst = vst(std::integral_constant<int, ST + 2>{});        // V(it+2)
    constexpr int PER = 4;                 // scores of S(it) per sub-step (8 sub-steps)
    const auto rk = k_rsrc(e3);
    const auto rv = v_rsrc(e2);
    const int e4_raw = ent_raw(it + 4);
    const float sc2 = tsc(it + 2);
    f32x16 n0 = f32x16{}, n1 = f32x16{};
    i32x8 a0, a1;
    kread(Kn, 0, 0, a0);
    kread(Kn, 0, 1, a1);
    __builtin_amdgcn_sched_barrier(0);

    // (A) statistics of S(it) behind the first QK MFMAs of S(it+1)
    n0 = mfma_fp8(a0, qf[0], n0);
    const bool own = prep(s0, s1, e0);
    float mx = lane_max_tree(s0, s1);
    __builtin_amdgcn_sched_barrier(0);
    n1 = mfma_fp8(a1, qf[0], n1);
    mx = half_swap_max(mx);
    const float cct = cq * sc0;          // exponent multiplier of this tile and row
    const float mxc = own ? mx * cct : -INFINITY;
    // lazy reference in scaled units: moves when the tile raises the row's
    // maximum by more than 2^8 (from -inf it always moves; -inf - -inf is
    // NaN, so a row with nothing yet kept stays put)
    const bool move = (mxc - mref_c) > kLazyLog2;
    kread(Kn, 1, 0, a0);
    kread(Kn, 1, 1, a1);
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float alpha = move ? fast_exp2(mref_c - mxc) : 1.f;
      mref_c = move ? mxc : mref_c;
      l_run *= alpha;
      if constexpr (PV8) lsum *= alpha;
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) o[db] *= alpha;
    }
    const float cc = own ? cct : 0.f;
    const float mc = own ? mref_c : INFINITY;

    // (B) 8 sub-steps: the second QK step of S(it+1) in the first two, the
    // exponentials of S(it), and each 16-key chunk's P.V one sub-step after
    // its last exponential (V^T operands read two sub-steps ahead); the
    // three DMAs of V(it+2) and K(it+3) spread over sub-steps 0, 3 and 6.
    uint32_t pw[16];
    int pw8[8];                            // PV8: byte b of the 32 = code of score b (s0 then s1)
    float rs = 0.f;
    auto pv_at = [&](int j) { return 2 * j + 2; };
    auto rd_at = [&](int j) { return 2 * j; };
    bf16x8 va[2][kD / 32];
    i32x8 va8[kD / 32];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks == 0) dma_block(rk, Kdst, wave, kdma);
      if constexpr (PV8) {
        if (ks == 4) dma_block(rv, Vdst, wave, vdma[0]);
      } else {
        if (ks == 3) dma_block(rv, Vdst, 2 * wave, vdma[0]);
        if (ks == 6) dma_block(rv, Vdst, 2 * wave + 1, vdma[1]);
      }
      if (ks == 0) n0 = mfma_fp8(a0, qf[1], n0);
      if (ks == 1) n1 = mfma_fp8(a1, qf[1], n1);
#pragma unroll
      for (int e = 0; e < PER; e += 2) {
        const int idx = ks * PER + e;      // 0..31: s0 then s1
        const float x0 = idx < 16 ? s0[idx] : s1[idx - 16];
        const float x1 = idx < 16 ? s0[idx + 1] : s1[idx - 15];
        const float p0 = fast_exp2(__builtin_fmaf(x0, cc, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(x1, cc, -mc));
        if constexpr (PV8) {
          if ((idx & 3) == 0) pw8[idx >> 2] = cvt_fp8x2<false>(p0, p1, 0);
          else pw8[idx >> 2] = cvt_fp8x2<true>(p0, p1, pw8[idx >> 2]);
        } else {
          pw[idx >> 1] = pack_bf16x2(p0, p1);
          rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[idx >> 1]), kOnesBf16x2, rs, false);
        }
      }
      if constexpr (PV8) {
        // the code tile's operands of dim block ks - 4, read in the second
        // half of the step (V(it) stays in its stage for the whole step)
        if (ks >= 4) {
          const int db = ks - 4;
          const i32x4 x = *reinterpret_cast<const i32x4 *>(Vc + voff[0] + db * 32 * 64);
          const i32x4 y = *reinterpret_cast<const i32x4 *>(Vc + voff[1] + db * 32 * 64);
          va8[db] = i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
        }
        __builtin_amdgcn_sched_barrier(0);
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (pv_at(j) != ks) continue;
        const bf16x8 pj = __builtin_bit_cast(bf16x8, u32x4{pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
#pragma unroll
        for (int db = 0; db < kD / 32; ++db) o[db] = mfma32(va[j & 1][db], pj, o[db]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (rd_at(j) != ks) continue;
#pragma unroll
        for (int db = 0; db < kD / 32; ++db)
          va[j & 1][db] = *reinterpret_cast<const bf16x8 *>(Vc + voff[j] + db * 32 * 128);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (PV8) {  // the tile's P.V and row sum on the coded probabilities
      const i32x8 p8 = i32x8{pw8[0], pw8[1], pw8[2], pw8[3], pw8[4], pw8[5], pw8[6], pw8[7]};
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) o[db] = mfma_fp8(va8[db], p8, o[db]);
      lsum = mfma_fp8(ones8, p8, lsum);
    } else {  // the last chunk's P.V, due after the last sub-step
      const bf16x8 pj = __builtin_bit_cast(bf16x8, u32x4{pw[12], pw[13], pw[14], pw[15]});
#pragma unroll
      for (int db = 0; db < kD / 32; ++db) o[db] = mfma32(va[1][db], pj, o[db]);
      l_run += rs;
    }

    // (C) K(it+2) and V(it+1), issued one step ago, have landed once at most
    // this step's DMAs (3; PV8: 2) are outstanding; then every wave's share
    // is in
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(PV8 ? 2 : 3));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    s0 = n0;
    s1 = n1;
    e0 = e1;
    e1 = e2;
    e2 = e3;
    e3 = __builtin_amdgcn_readfirstlane(e4_raw);
    sc0 = sc1;
    sc1 = sc2;
    ++it;
  };

  while (it + 3 <= nt) {
    step(C0{});
    step(C1{});
    step(C2{});
  }
  if (it < nt) step(C0{});
  if (it < nt) step(C1{});
  if constexpr (PV8) l_run = 0.5f * lsum[0];
}

// PV8: Vt holds the V^T code tiles and vamax [H][128] the channels' largest
// magnitudes (the channel scale is amax / 448, applied to O at the end).
template <int BQ, bool DENSE, bool PV8>
__global__ __launch_bounds__(kWgRows * 2, 1)
void attn_fwd_fp8(const uint8_t *__restrict__ Q8, const float *__restrict__ qscale, const uint8_t *__restrict__ K8,
                  const float *__restrict__ kscale, const void *__restrict__ Vt, const float *__restrict__ vamax,
                  bf16_t *__restrict__ O, const int32_t *__restrict__ row_ptr, const int32_t *__restrict__ kv_idx,
                  int N, int nqb, int nkb, int ngrp, float c, const int32_t *__restrict__ labels, int qo_orig, int F,
                  int S) {
  constexpr int G = kWgRows / BQ;
  constexpr int OWN_ALL = (1 << G) - 1;
  constexpr int kVTile = PV8 ? kV8Bytes : kVtBytes;
  // V^T stages first (uppercase names sort first): their reads take
  // immediate offsets below 64 KB
  __shared__ __attribute__((aligned(1024))) char k0[kK8Bytes], k1[kK8Bytes], k2[kK8Bytes], V0[kVTile],
      V1[kVTile], V2[kVTile];
  __shared__ int ulist[DENSE ? 1 : kMaxKb];
  __shared__ float uscale[kMaxKb];
  __shared__ uint32_t bits[DENSE ? 1 : G * kWords];
  __shared__ int wsum[DENSE ? 1 : kWords + 1];

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int nlead = min(ngrp, 512 / kWgRows);
  const int h = work / ngrp, local = work - h * ngrp;
  const int grp = local < nlead ? ngrp - 1 - local : local - nlead;   // text groups first
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int gw = wave * 32 / BQ;
  const size_t hoff = (size_t)h * N * kD;
  const uint8_t *K8h = K8 + hoff;
  const float *ksh = kscale + (size_t)h * nkb;
  const char *Vth = reinterpret_cast<const char *>(Vt) + (size_t)h * nkb * kVTile;
  bf16_t *Oh = O + hoff;
  const int qrow = grp * kWgRows + wave * 32 + l32;
  int qsrc = qrow;
  if (qo_orig && (labels == nullptr || labels[h] == 1) && qrow < F * S) {
    const int p = qrow / F, f = qrow - p * F;
    qsrc = f * S + p;
  }

  int nt = nkb;
  if constexpr (!DENSE)
    nt = build_union_list<G, kWgRows * 2>(row_ptr, kv_idx, h, grp, nqb, nkb, tid, lane, wave, ulist, bits, wsum);
  // each listed tile's K scale next to its entry (1 for an all-zero block:
  // its scores are exactly 0 whatever the multiplier)
  for (int j = tid; j < nt; j += kWgRows * 2) {
    const int kb = DENSE ? j : (ulist[j] & 0xFFFFFF);
    const float s = ksh[kb];
    uscale[j] = s > 0.f ? s : 1.f;
  }
  __syncthreads();

  if (nt == 0) {
    if (qrow < N) {
#pragma unroll
      for (int dd = hi * 8; dd < kD; dd += 16)
        *reinterpret_cast<u32x4 *>(Oh + (size_t)qsrc * kD + dd) = u32x4{0, 0, 0, 0};
    }
    return;
  }
  auto ent_raw = [&](int j) -> int {
    const int i = j < nt ? j : nt - 1;
    if constexpr (DENSE) return i | (OWN_ALL << 24);
    else return ulist[i];
  };
  auto tsc = [&](int j) -> float { return uscale[j < nt ? j : nt - 1]; };
  const int own_bit = 1 << (24 + gw);

  // Q8 operands: dims 64 ks + 32 hi .. + 31 of the lane's query
  i32x8 qf[2];
  float cq = c;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) qf[ks] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  if (qrow < N) {
    const uint8_t *qr = Q8 + hoff + (size_t)qsrc * kD;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const i32x4 x = *reinterpret_cast<const i32x4 *>(qr + 64 * ks + 32 * hi);
      const i32x4 y = *reinterpret_cast<const i32x4 *>(qr + 64 * ks + 32 * hi + 16);
      qf[ks] = i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    }
    const float s = qscale[(size_t)h * N + qsrc];
    cq = s > 0.f ? c * s : c;          // an all-zero row scores 0 whatever the multiplier
  }
  auto prep = [&](f32x16 &s0, f32x16 &s1, int e) -> bool {
    bool own = true;
    if constexpr (!DENSE) own = (e & own_bit) != 0;
    if (own && ((e & 0xFFFFFF) + 1) * BK > N) {
      const int nvh = N - (e & 0xFFFFFF) * BK - 8 * hi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (acc_key_pi(0, r, 0) >= nvh) s0[r] = -INFINITY;
        if (acc_key_pi(1, r, 0) >= nvh) s1[r] = -INFINITY;
      }
    }
    return own;
  };
  f32x16 o[kD / 32];
  float l_run;
  vt_attend_qk8<PV8>(nt, ent_raw, tsc, prep, K8h, Vth, N, k0, k1, k2, V0, V1, V2, qf, cq, wave, lane, o, l_run);
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may land after the work-group ends
  if constexpr (PV8) {  // the channel scales: this lane's dims 32 db + 8 g + 4 hi + 0..3
    const float *va = vamax + (size_t)h * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(va + 32 * db + 8 * g + 4 * hi);
#pragma unroll
        for (int q = 0; q < 4; ++q) o[db][4 * g + q] *= a[q] / kE4M3Max;
      }
  }
  store_o<kD>(qrow < N ? Oh + (size_t)qsrc * kD : nullptr, o, l_run, hi);
}

template <int BQ>
hipError_t launch_fp8(const Dims &dm, const void *Q8, const float *qs, const void *K8, const float *ks,
                      const void *Vt, const float *vamax, void *O, const int32_t *row_ptr, const int32_t *kv_idx,
                      float c, const int32_t *labels, int qo_orig, hipStream_t st) {
  constexpr int G = kWgRows / BQ;
  const int nqb = (dm.N + BQ - 1) / BQ, nkb = (dm.N + BK - 1) / BK;
  const int ngrp = (nqb + G - 1) / G;
  if (dm.H * ngrp == 0) return hipSuccess;
  const int grid = dm.H * ngrp;
#define SVG_FP8_LAUNCH(DENSE, PV8)                                                                              \
  hipLaunchKernelGGL((attn_fwd_fp8<BQ, DENSE, PV8>), dim3(grid), dim3(kWgRows * 2), 0, st, (const uint8_t *)Q8, qs, \
                     (const uint8_t *)K8, ks, Vt, vamax, (bf16_t *)O, row_ptr, kv_idx, dm.N, nqb, nkb, ngrp, c,     \
                     labels, qo_orig, dm.F, dm.S)
  if (vamax != nullptr) {
    if (row_ptr == nullptr) return hipErrorInvalidValue;   // the P.V mode is block-sparse only
    SVG_FP8_LAUNCH(false, true);
  } else if (row_ptr == nullptr) {
    SVG_FP8_LAUNCH(true, false);
  } else {
    SVG_FP8_LAUNCH(false, false);
  }
#undef SVG_FP8_LAUNCH
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows_fp8(const Dims &dm, const void *X, void *X8, float *scale, hipStream_t st) {
  const int64_t rows = (int64_t)dm.H * dm.N;
  if (rows == 0) return hipSuccess;
  const int64_t threads = rows * (dm.d / 8);
  const int blocks = (int)((threads + 255) / 256);
  if (dm.d == 128)
    hipLaunchKernelGGL(quant_rows_fp8<128>, dim3(blocks), dim3(256), 0, st, (const u32x4 *)X, (uint8_t *)X8, scale,
                       rows);
  else
    hipLaunchKernelGGL(quant_rows_fp8<64>, dim3(blocks), dim3(256), 0, st, (const u32x4 *)X, (uint8_t *)X8, scale,
                       rows);
  return hipGetLastError();
}

hipError_t launch_layout_fp8(const Dims &dm, const void *X, void *X8, float *scale, const int32_t *labels,
                             hipStream_t st) {
  const int nkb = (dm.N + 63) / 64;
  if (dm.N == 0 || dm.H == 0) return hipSuccess;
  if (dm.d == 128)
    hipLaunchKernelGGL(layout_fp8<128>, dim3(nkb, dm.H), dim3(256), 0, st, (const u32x4 *)X, (uint8_t *)X8, scale,
                       labels, dm.F, dm.S, dm.N, nkb);
  else
    hipLaunchKernelGGL(layout_fp8<64>, dim3(nkb, dm.H), dim3(256), 0, st, (const u32x4 *)X, (uint8_t *)X8, scale,
                       labels, dm.F, dm.S, dm.N, nkb);
  return hipGetLastError();
}

hipError_t launch_attn_fp8(const Dims &dm, const void *Q8, const float *qscale, const void *K8, const float *kscale,
                           const void *Vt, const float *vamax, void *O, const int32_t *row_ptr,
                           const int32_t *kv_idx, int bq, float scale, const int32_t *labels, bool qo_orig,
                           hipStream_t st) {
  if (dm.d != 128) return hipErrorInvalidValue;
  const float c = scale * kLog2e;
  if (bq == 128)
    return launch_fp8<128>(dm, Q8, qscale, K8, kscale, Vt, vamax, O, row_ptr, kv_idx, c, labels, qo_orig, st);
  if (bq == 64)
    return launch_fp8<64>(dm, Q8, qscale, K8, kscale, Vt, vamax, O, row_ptr, kv_idx, c, labels, qo_orig, st);
  return hipErrorInvalidValue;
}

hipError_t launch_layout_vt_fp8(const Dims &dm, const void *V, void *Vt8, float *vamax, const int32_t *labels,
                                hipStream_t st) {
  if (dm.d != 128) return hipErrorInvalidValue;
  const int nkb = (dm.N + 63) / 64;
  if (dm.N == 0 || dm.H == 0) return hipSuccess;
  const int n = dm.H * 128;
  hipLaunchKernelGGL(zero_f32, dim3((n + 255) / 256), dim3(256), 0, st, vamax, n);
  hipLaunchKernelGGL(chan_amax, dim3((dm.N + kChanRows - 1) / kChanRows, dm.H), dim3(256), 0, st, (const u32x4 *)V,
                     reinterpret_cast<uint32_t *>(vamax), dm.N);
  hipLaunchKernelGGL(layout_vt_fp8, dim3(nkb, dm.H), dim3(256), 0, st, (const u32x4 *)V, vamax, (u32x4 *)Vt8, labels,
                     dm.F, dm.S, dm.N, nkb);
  return hipGetLastError();
}

}  // namespace svgk
