// Building blocks of the gfx950 MFMA flash-attention kernels (internal).
//
// Layout of one wave's work (32 queries, 64-key tiles, head dim D):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16.  A = K rows from LDS.  B =
//   the wave's Q rows, held in registers for the whole key loop.  Lane l
//   serves query (l & 31).  Its 16 accumulator values per 32-key block are
//   keys 8*(r/4) + 4*(l/32) + (r%4), r = 0..15.  So lanes l and l^32 split
//   one query's keys.
//   O^T += V^T P^T.  B = P^T straight from the S^T accumulator registers,
//   rounded to bf16.  A = V^T from LDS, stored with each 16-key chunk's
//   keys in the order {0-3, 8-11 | 4-7, 12-15}: the two lane halves'
//   accumulator key order.  The reduction index of the MFMA then pairs each
//   P value with its own V row.
#pragma once

#include "svg_common.h"

namespace svgk {
namespace core {

constexpr int BK = 64;

template <int D, int NT>
struct Tile {
  static constexpr int KSTR = D * 2 + 16;        // K row stride (bytes): padded against bank conflicts
  static constexpr int KBYTES = BK * KSTR;
  static constexpr int VSTR = BK * 2;            // V^T row stride (bytes): XOR-swizzled 16-byte blocks
  static constexpr int VBYTES = D * VSTR;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int DC = D / 8;               // 16-byte chunks per row
  static constexpr int UNITS = (BK / 4) * DC;    // load unit = 4 consecutive keys x 8 dims
  static constexpr int UPT = (UNITS + NT - 1) / NT;
};

// 16-byte block swizzle of V^T rows: consecutive rows (one MFMA operand
// read) and rows 8 apart (one staging write) land on different banks.
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

__device__ __forceinline__ f32x16 mfma32(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Register staging of one K/V tile.  rowof(key_in_tile) gives the global
// row of a key, or -1 for a key that does not exist (it is zero-filled).
template <int D, int NT>
struct Regs {
  u32x4 k[Tile<D, NT>::UPT][4];
  u32x4 v[Tile<D, NT>::UPT][4];
};

template <int D, int NT, typename RowOf>
__device__ __forceinline__ void load_tile(const bf16_t *__restrict__ Kh, const bf16_t *__restrict__ Vh,
                                          int tid, RowOf rowof, Regs<D, NT> &R) {
  using C = Tile<D, NT>;
#pragma unroll
  for (int i = 0; i < C::UPT; ++i) {
    const int u = tid + i * NT;
    if (C::UNITS % NT == 0 || u < C::UNITS) {
      const int g = u / C::DC, dc = u % C::DC;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rowof(4 * g + r);
        if (row >= 0) {
          R.k[i][r] = *reinterpret_cast<const u32x4 *>(Kh + (size_t)row * D + dc * 8);
          R.v[i][r] = *reinterpret_cast<const u32x4 *>(Vh + (size_t)row * D + dc * 8);
        } else {
          R.k[i][r] = u32x4{0, 0, 0, 0};
          R.v[i][r] = u32x4{0, 0, 0, 0};
        }
      }
    }
  }
}

template <int D, int NT>
__device__ __forceinline__ void store_tile(char *__restrict__ stage, int tid, const Regs<D, NT> &R) {
  using C = Tile<D, NT>;
  char *Ks = stage;
  char *Vs = stage + C::KBYTES;
#pragma unroll
  for (int i = 0; i < C::UPT; ++i) {
    const int u = tid + i * NT;
    if (C::UNITS % NT == 0 || u < C::UNITS) {
      const int g = u / C::DC, dc = u % C::DC;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<u32x4 *>(Ks + (4 * g + r) * C::KSTR + dc * 16) = R.k[i][r];
      // keys 4g..4g+3 -> V^T slots 16*(g/4) + {0, 8, 4, 12}[g%4] .. +3
      const int og = g & 3;
      const int slot = 16 * (g >> 2) + (((og & 1) << 3) | ((og & 2) << 1));
      const int blk = slot >> 3, half = (slot >> 2) & 1;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int d = dc * 8 + 2 * m + e;
          uint32_t lo, hi;
          if (e == 0) {
            lo = (R.v[i][0][m] & 0xFFFFu) | (R.v[i][1][m] << 16);
            hi = (R.v[i][2][m] & 0xFFFFu) | (R.v[i][3][m] << 16);
          } else {
            lo = (R.v[i][0][m] >> 16) | (R.v[i][1][m] & 0xFFFF0000u);
            hi = (R.v[i][2][m] >> 16) | (R.v[i][3][m] & 0xFFFF0000u);
          }
          *reinterpret_cast<u32x2 *>(Vs + d * C::VSTR + ((blk ^ vt_swz(d)) << 4) + half * 8) =
              u32x2{lo, hi};
        }
      }
    }
  }
}

// Q fragment of one wave: row `qrow` (or zeros when qrow < 0).
template <int D>
__device__ __forceinline__ void load_q(const bf16_t *__restrict__ Qh, int qrow, int hi, bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 v = u32x4{0, 0, 0, 0};
    if (qrow >= 0) v = *reinterpret_cast<const u32x4 *>(Qh + (size_t)qrow * D + ks * 16 + hi * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, v);
  }
}

// S^T for the 64 keys of the staged tile: s0 = keys 0-31, s1 = keys 32-63.
template <int D, int NT>
__device__ __forceinline__ void qk_tile(const char *__restrict__ Ks, const bf16x8 (&qf)[D / 16], int l32,
                                        int hi, f32x16 &s0, f32x16 &s1) {
  using C = Tile<D, NT>;
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(Ks + l32 * C::KSTR + (ks * 16 + hi * 8) * 2);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(Ks + (32 + l32) * C::KSTR + (ks * 16 + hi * 8) * 2);
    s0 = mfma32(a0, qf[ks], s0);
    s1 = mfma32(a1, qf[ks], s1);
  }
}

// Key index (0..63, within the tile) of accumulator value r of block b.
__device__ __forceinline__ int acc_key(int b, int r, int hi) { return 32 * b + 8 * (r >> 2) + 4 * hi + (r & 3); }

// Keys at tile positions >= nvalid do not exist: set their scores to -inf.
// acc_key(b, r, hi) = acc_key(b, r, 0) + 4 hi: the constants are compared
// against nvalid - 4 hi, so no per-key offsets stay live across a loop.
__device__ __forceinline__ void mask_tail(f32x16 &s0, f32x16 &s1, int nvalid, int hi) {
  const int nvh = nvalid - 4 * hi;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (acc_key(0, r, 0) >= nvh) s0[r] = -INFINITY;
    if (acc_key(1, r, 0) >= nvh) s1[r] = -INFINITY;
  }
}

constexpr float kLazyLog2 = 8.f;

// IEEE-754 maximum (v_maximum3_f32 on gfx950).  Unlike fmaxf it needs no
// quieting of its operands in IEEE mode; scores and running maxima are
// finite or -inf, never NaN, so the two agree here.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Row maximum of the lane's query over the tile (both lane halves).
__device__ __forceinline__ float row_max(const f32x16 &s0, const f32x16 &s1) {
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = vmax(mx, vmax(s0[r], s1[r]));
  return vmax(mx, __shfl_xor(mx, 32));
}

// Moves the reference maximum if the tile raised the row maximum by more
// than 2^kLazyLog2 (exp2 units), rescales l_run accordingly, and returns the
// factor the accumulated output must be multiplied by.  Branch-free.
__device__ __forceinline__ float update_ref(float mx, float c, float &m_run, float &l_run) {
  const bool move = mx > m_run && (mx - m_run) * c > kLazyLog2;  // m_run = -inf: always moves
  const float a_move = fast_exp2((m_run - mx) * c);
  const float alpha = move ? a_move : 1.f;
  m_run = move ? mx : m_run;
  l_run *= alpha;
  return alpha;
}

// Probabilities of the tile against the reference m_run, packed as bf16 MFMA
// B operands (one per 16-key chunk); their sum is added to l_run.
__device__ __forceinline__ void probs(const f32x16 &s0, const f32x16 &s1, float c, float m_run, float &l_run,
                                      bf16x8 (&pb)[4]) {
  const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
  float rs = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x16 &s = (j < 2) ? s0 : s1;
    const int base = (j & 1) * 8;
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p0 = fast_exp2(__builtin_fmaf(s[base + 2 * i], c, -mc));
      const float p1 = fast_exp2(__builtin_fmaf(s[base + 2 * i + 1], c, -mc));
      rs += p0 + p1;
      w[i] = pack_bf16x2(p0, p1);
    }
    pb[j] = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
  }
  l_run += rs;
}

// One online-softmax step for the lane's query: m_run is the reference
// maximum the exponentials are taken against.  It moves only when the tile
// raises the row maximum by more than 2^kLazyLog2 in exp2 units, so most
// tiles need no rescale of O.  Probabilities then stay <= 2^kLazyLog2, and
// l_run and O share the reference, so O / l is unchanged.  l_run is this
// lane's partial sum.  Returns the rescale factor of the accumulated output.
// c = scale * log2(e).
__device__ __forceinline__ float softmax_step(const f32x16 &s0, const f32x16 &s1, float c, float &m_run,
                                              float &l_run, bf16x8 (&pb)[4]) {
  const float alpha = update_ref(row_max(s0, s1), c, m_run, l_run);
  probs(s0, s1, c, m_run, l_run, pb);
  return alpha;
}

template <int D>
__device__ __forceinline__ void rescale(f32x16 (&o)[D / 32], float alpha) {
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
  }
}

// O^T += V^T P^T for the staged tile.  The four V^T operands of a 16-key
// chunk are read before its MFMAs so the LDS latency overlaps the math.
template <int D, int NT>
__device__ __forceinline__ void pv_tile(const char *__restrict__ Vs, const bf16x8 (&pb)[4], int l32, int hi,
                                        f32x16 (&o)[D / 32]) {
  using C = Tile<D, NT>;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x8 a[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = 32 * db + l32;
      a[db] = *reinterpret_cast<const bf16x8 *>(Vs + d * C::VSTR + (((2 * j + hi) ^ vt_swz(d)) << 4));
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = mfma32(a[db], pb[j], o[db]);
  }
}

// Final O row of the lane's query: O^T / l, written as bf16 (lane holds
// dims 32*db + 8*g + 4*hi + 0..3).
template <int D>
__device__ __forceinline__ void store_o(bf16_t *__restrict__ orow, const f32x16 (&o)[D / 32], float l_run,
                                        int hi) {
  const float lt = l_run + __shfl_xor(l_run, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  if (orow == nullptr) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hi;
      const uint32_t w0 = pack_bf16x2(o[db][4 * g + 0] * inv, o[db][4 * g + 1] * inv);
      const uint32_t w1 = pack_bf16x2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
      *reinterpret_cast<u32x2 *>(orow + d0) = u32x2{w0, w1};
    }
  }
}


// ===========================================================================
// Direct-to-LDS pipeline (gfx950).
//
// K and V tiles are copied from global memory into LDS by the load unit
// itself (global_load_lds_dwordx4: lane l's 16 bytes land at LDS
// base + 16*l), so no registers stage them.  Both tiles are row-major, 64 rows
// of D bf16, and each row's 16-byte chunks are XOR-swizzled:
//   K: chunk ^ swz_k(key)   so the 16 lanes of one ds_read_b128 (16 keys, one
//                           logical chunk) hit 16 different bank groups;
//   V: chunk ^ swz_v(key)   so the ds_read_b64_tr_b16 transposed reads of the
//                           V^T operand are conflict-free.
// The V^T MFMA operand is read transposed from row-major V.  In each 16-lane
// group, ds_read_b64_tr_b16 returns to lane i the i-th halfword of four
// 8-byte rows.  Lane j of the group points at V[key_(j/4)][d0 + 4*(j%4)], so
// lane i receives V[key_0..3][d0 + i]: four keys of its own d.  Two such
// reads give the eight keys an operand lane needs.
// ===========================================================================

template <int D>
struct DTile {
  static constexpr int ROWB = D * 2;          // bytes per row
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int TBYTES = BK * ROWB;    // one K or V tile
  static constexpr int UNITS = BK * CPR;      // 16-byte units per tile
  static constexpr int BLOCKS = UNITS / 64;   // 1 KB DMA blocks per tile
};

template <int D>
__device__ __forceinline__ int swz_k(int key) { return D == 128 ? (key & 15) : ((key >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int key) { return D == 128 ? 4 * (key & 3) : 2 * (key & 3); }

typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4s16 lds_v4s16_t;

// Copy one tile (64 rows) of X into LDS at `tile`.  rowof(r) gives the global
// row of tile row r and must return a readable row (callers clamp rows past
// the end; their scores are masked).  Wave `wave` of NW issues its share of
// the 1 KB blocks.
template <int D, int NW, bool ISV, typename RowOf>
__device__ __forceinline__ void dma_tile(const bf16_t *__restrict__ Xh, char *tile, int wave, int lane,
                                         RowOf rowof) {
  using T = DTile<D>;
  constexpr int PER_WAVE = T::BLOCKS / NW;
  static_assert(T::BLOCKS % NW == 0, "tile blocks must split evenly over the waves");
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int blk = wave * PER_WAVE + i;
    const int p = blk * 64 + lane;                 // 16-byte unit written by this lane
    const int row = p / T::CPR, pc = p % T::CPR;
    const int c = pc ^ (ISV ? swz_v<D>(row) : swz_k<D>(row));
    const bf16_t *src = Xh + (size_t)rowof(row) * D + c * 8;
    __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_t *)(tile + blk * 1024), 16, 0, 0);
  }
}

// Per-lane byte offsets (within a tile) of the 16-byte units this lane's
// DMA instructions copy, for every row inside N.  The tile's global base is
// uniform, so each DMA is "scalar base + vector offset" with no per-tile
// address arithmetic.
template <int D, int NW, bool ISV>
__device__ __forceinline__ void dma_offsets(int wave, int lane, int (&off)[DTile<D>::BLOCKS / NW]) {
  using T = DTile<D>;
  constexpr int PER_WAVE = T::BLOCKS / NW;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int p = (wave * PER_WAVE + i) * 64 + lane;
    const int row = p / T::CPR, pc = p % T::CPR;
    const int c = pc ^ (ISV ? swz_v<D>(row) : swz_k<D>(row));
    off[i] = row * T::ROWB + c * 16;
  }
}

// DMA of a whole tile (every row < N): `src` = the tile's first row in global
// memory, `tile` = its LDS stage, `wave` uniform.
template <int D, int NW>
__device__ __forceinline__ void dma_full(const char *src, char *tile, int wave, const int (&off)[DTile<D>::BLOCKS / NW]) {
  constexpr int PER_WAVE = DTile<D>::BLOCKS / NW;
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i)
    __builtin_amdgcn_global_load_lds((const void *)(src + off[i]), (lds_void_t *)(tile + (wave * PER_WAVE + i) * 1024),
                                     16, 0, 0);
}

// The same through a buffer resource over the head (base = the head's first
// row, `head_bytes` long): the tile's byte offset goes in a scalar, each
// lane's unit offset in one vector register, and no address arithmetic runs
// per tile.
template <int D, int NW>
__device__ __forceinline__ void dma_full_buf(const void *head, int head_bytes, int tile_byte_off, char *tile,
                                             int wave, const int *off) {
  constexpr int PER_WAVE = DTile<D>::BLOCKS / NW;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(head), (short)0, head_bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t *)(tile + (wave * PER_WAVE + i) * 1024), 16, off[i],
                                             tile_byte_off, 0, 0);
}

// Row maximum with three-input maxima (v_maximum3_f32).
__device__ __forceinline__ float row_max3(const f32x16 &s0, const f32x16 &s1) {
  float a = vmax(vmax(s0[0], s0[1]), s0[2]);
  float b = vmax(vmax(s1[0], s1[1]), s1[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) {
    a = vmax(vmax(a, s0[r]), s0[r + 1]);
    b = vmax(vmax(b, s1[r]), s1[r + 1]);
  }
  a = vmax(vmax(a, s0[15]), b);
  a = vmax(a, s1[15]);
  return vmax(a, __shfl_xor(a, 32));
}

// Per-lane byte offsets of the K operand reads (one per 16-dim step; the
// second 32-key block is +32 rows).
template <int D>
__device__ __forceinline__ void k_offsets(int l32, int hi, int (&off)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    off[ks] = l32 * DTile<D>::ROWB + (((2 * ks + hi) ^ swz_k<D>(l32)) << 4);
}

// Per-lane byte offsets of the transposed V reads, one per 32-dim block; the
// chunk (j) and half (s) terms are added as immediates.
template <int D>
__device__ __forceinline__ void v_offsets(int lane, int (&off)[D / 32]) {
  const int G = lane >> 4, r = (lane & 15) >> 2, q = lane & 3;
  const int key = 4 * (G >> 1) + r;  // + 16*j + 8*s, which leaves key & 3 unchanged
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int d = 32 * db + 16 * (G & 1) + 4 * q;
    off[db] = key * DTile<D>::ROWB + (((d >> 3) ^ swz_v<D>(key)) << 4) + (d & 7) * 2;
  }
}

template <int D>
__device__ __forceinline__ void qk_tile_dma(const char *__restrict__ Ks, const bf16x8 (&qf)[D / 16],
                                            const int (&koff)[D / 16], f32x16 &s0, f32x16 &s1) {
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(Ks + koff[ks]);
    const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(Ks + koff[ks] + 32 * DTile<D>::ROWB);
    s0 = mfma32(a0, qf[ks], s0);
    s1 = mfma32(a1, qf[ks], s1);
  }
}

__device__ __forceinline__ v4s16 ds_read_tr16(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16_t *)(p));
}

template <int D>
__device__ __forceinline__ void pv_tile_dma(const char *__restrict__ Vs, const bf16x8 (&pb)[4],
                                            const int (&voff)[D / 32], f32x16 (&o)[D / 32]) {
  constexpr int RB = DTile<D>::ROWB;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x8 a[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const v4s16 lo = ds_read_tr16(Vs + voff[db] + (16 * j) * RB);
      const v4s16 hi = ds_read_tr16(Vs + voff[db] + (16 * j + 8) * RB);
      typedef short v8s16 __attribute__((ext_vector_type(8)));
      const v8s16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      a[db] = __builtin_bit_cast(bf16x8, both);
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = mfma32(a[db], pb[j], o[db]);
  }
}

}  // namespace core
}  // namespace svgk
