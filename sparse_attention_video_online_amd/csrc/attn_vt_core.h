// Shared pieces of the kernels that read V in the key-tiled transposed
// layout (attn_vt.hip, and the profiler's full pass): LDS swizzles and DMA
// offsets of the K and V^T tiles, the K row order pi, softmax helpers, and the
// per-work-group union of the kept-tile lists.
#pragma once

#include <type_traits>

#include "attn_core.h"

namespace svgk {
namespace core {

constexpr int kMaxKb = 8192;     // union-list capacity (kv-blocks per head)
constexpr int kWords = kMaxKb / 32;

// (1, 1) in bf16, the second operand of the row-sum dot products
constexpr bf16x2_t kOnesBf16x2 = {(__bf16)1.0f, (__bf16)1.0f};

// s_waitcnt with vmcnt = n and no wait on the other counters (gfx9 encoding).
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt with lgkmcnt = 0 and no wait on vmcnt or expcnt.
constexpr int kWaitLgkm0 = 0xF | (0x3 << 14) | (0x7 << 4);

// Key (0..63) of accumulator value r of block b (0: keys 0-31, 1: 32-63)
// under the K row order pi.
__device__ __forceinline__ int acc_key_pi(int b, int r, int hi) {
  return 32 * b + 16 * (r >> 3) + 8 * hi + (r & 7);
}

// Scores of keys named by per-lane drop words become -inf.  Bit k0 of d0
// (d1) stands for accumulator value r of s0 (s1), k0 = 16 (r >> 3) + (r & 7),
// i.e. key acc_key_pi(b, r, hi) - 32 b - 8 hi: callers shift their
// wave-uniform key words right by 8 hi first.  Straight-line VALU (a bit test
// and a select per score); written as a lane-varying shift of uniform words
// so that no lane-divergent branch arises.
__device__ __forceinline__ void drop_scores(f32x16 &s0, f32x16 &s1, uint32_t d0, uint32_t d1) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const uint32_t bit = 1u << (16 * (r >> 3) + (r & 7));
    s0[r] = (d0 & bit) ? -INFINITY : s0[r];
    s1[r] = (d1 & bit) ? -INFINITY : s1[r];
  }
}

// Maximum of the lane's 32 scores as a tree of three-input maxima (depth 4).
__device__ __forceinline__ float lane_max_tree(const f32x16 &s0, const f32x16 &s1) {
  float a[11];
#pragma unroll
  for (int k = 0; k < 5; ++k) a[k] = vmax(vmax(s0[3 * k], s0[3 * k + 1]), s0[3 * k + 2]);
  a[5] = vmax(vmax(s0[15], s1[0]), s1[1]);
#pragma unroll
  for (int k = 0; k < 4; ++k) a[6 + k] = vmax(vmax(s1[2 + 3 * k], s1[3 + 3 * k]), s1[4 + 3 * k]);
  a[10] = vmax(s1[14], s1[15]);
  const float b0 = vmax(vmax(a[0], a[1]), a[2]), b1 = vmax(vmax(a[3], a[4]), a[5]);
  const float b2 = vmax(vmax(a[6], a[7]), a[8]), b3 = vmax(a[9], a[10]);
  return vmax(vmax(b0, b1), vmax(b2, b3));
}

// Maximum with the partner lane l ^ 32 (the other half of the same query's
// keys), through v_permlane32_swap instead of an LDS permute.
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Sub-step schedule of the P.V MFMAs: delay after the chunk's last
// exponential, and lead of the V^T operand reads before the MFMAs.
constexpr int kPvDelay = 1;
constexpr int kVLead = 2;
static_assert(kVLead >= 1, "a chunk's V^T operands are read in an earlier sub-step than its P.V");

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
  static_assert(kWords == 4 * 64, "wave 0 scans the bitmap's words four per lane");
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


// The tile pipeline shared by the attention kernels on the V^T layout, for
// one wave of NW: online-softmax attention of the wave's 32 query rows (B
// operands qf, one row per lane pair) over the tiles ent_raw(0..nt-1).
//   ent_raw(j): entry of tile j, kv-block in bits 0-23 and caller flags above;
//               callers repeat the last entry for j >= nt (those DMAs land in
//               free stages and are never read).  Read early, moved to a
//               scalar register late.
//   prep(s0, s1, e): masks the scores of the tile with entry e in place and
//               returns whether the lane's row keeps any key of it.
// K and V^T tiles come from Kh (row-major, N rows; tile e starts at row
// krow(e), by default kv-block * 64) and Vth (key-tiled, every tile full,
// tile e at kv-block e) through three LDS stages each (k0..k2, v0..v2, TB bytes, all
// waves of the work-group call this together: it contains barriers).  On
// return o, m_run and l_run hold the un-normalised output, the reference
// maximum and this lane's partial row sum: of the bf16 probabilities that
// enter the P.V MFMAs (SUM_BF16), or of the fp32 ones.
//
// Per tile it, one wave:
//   (A) the first QK MFMAs of S(it+1), then the statistics of S(it) (masks,
//       row maximum as a max3 tree and a v_permlane32_swap, lazy reference
//       update) behind them;
//   (B) D/16 hand-ordered steps: the MFMAs of S(it+1), the exponentials of
//       S(it), and the O^T += V^T P^T MFMAs of each completed 16-key chunk;
//       the DMAs of V(it+2) and K(it+3) are spread over these steps;
//   (C) wait until only this step's DMAs are in flight, one barrier.
// S^T's rows (keys) are read from K in the order pi, so the accumulator
// layout of S^T is the B-operand layout of P^T with keys in natural order.
// The first K row of the tile with entry e: kv-block e of K.
struct KvBlockRow {
  __device__ int operator()(int e) const { return (e & 0xFFFFFF) * BK; }
};

// K rows gathered from the original token order (the layout permute fused
// into the tile DMA), for a permuted (temporal) head: row r of the executing
// layout is row p*F + f = r of the video, holding original row f*S + p; the
// text rows stay where they are.  Wave 0 writes the source rows of a tile's
// 64 keys to one slot of a four-slot ring in LDS one step before the tile's
// DMA (tiles it .. it+3 in the prologue, tile it+4 during step it); every
// wave then takes its units' rows from the ring and issues the DMA through
// one buffer resource over the head.  Keys past N read row N-1 (their
// scores are masked).
// Lane j of a tile starting at r0: r0 = p0*F + f0 and j = jq*F + jr (jq, jr
// the lane's constants), so r0 + j is position p0 + jq + carry, frame
// f0 + jr - carry*F, with one carry at most.  r0 / F is umulhi(r0, fm) >> fk
// with fk = floor(log2 F), fm = ceil(2^(32+fk) / F): the product overshoots
// r0 / F by less than r0 / 2^(32+fk) < 2^-(8+fk) < 1/F for r0 < 2^24, so the
// floor is exact (a head is under 2 GiB, so N < 2^24).
struct GatherRows {
  int *ring;     // LDS, 4 x 64 ints
  int F, S, N;
  uint32_t fm;
  int fk;
  int jq, jr;    // the lane's j / F and j % F
  __device__ int tile_src(int kb, int lane) const {
    const int r0 = kb * 64;                   // wave-uniform
    const int p0 = (int)(__umulhi((uint32_t)r0, fm) >> fk), f0 = r0 - p0 * F;
    int f = f0 + jr;
    const int cy = f >= F ? 1 : 0;
    f -= cy * F;
    const int r = r0 + lane;
    return r < F * S ? f * S + p0 + jq + cy : min(r, N - 1);
  }
};

// Centroid tiles (the compensation of skipped blocks): an entry with
// kCentFlag set names tile t = e & kCentTileMask of a second pair of tables,
// 64 centroid keys of the head (row-major, like K) and the key-tiled V^T of
// their value sums, each a whole zero-padded tile.  Each centroid stands for
// 64 keys, so the tile's row sum counts 64 times (exact in fp32).  A pass
// with Centroids continues the softmax state of an earlier pass (the caller
// drains that pass's DMAs and passes a barrier between the two).
// NoCentroids (the default) compiles none of it.
constexpr int kCentFlag = 1 << 23;
constexpr int kCentTileMask = 0x1FFF;
struct NoCentroids {
  static constexpr bool kOn = false;
};
struct Centroids {
  static constexpr bool kOn = true;
  const bf16_t *k;     // [tiles * 64][D] of this head
  const bf16_t *vt;    // [tiles][D][64] of this head
};

template <int D, int NW, bool SUM_BF16 = true, typename EntRaw, typename Prep, typename KRow = KvBlockRow,
          typename Cent = NoCentroids>
__device__ __forceinline__ void vt_attend(int nt, EntRaw ent_raw, Prep prep, const bf16_t *__restrict__ Kh,
                                          const bf16_t *__restrict__ Vth, int N, char *k0, char *k1, char *k2,
                                          char *v0, char *v1, char *v2, const bf16x8 (&qf)[D / 16], int wave,
                                          int lane, float c, f32x16 (&o)[D / 32], float &m_run, float &l_run,
                                          KRow krow = KRow{}, Cent cent = Cent{}) {
  using T = DTile<D>;
  constexpr int TB = T::TBYTES;            // K tile bytes == V^T tile bytes
  constexpr int PK = T::BLOCKS / NW;       // DMA instructions per wave per tile
  static_assert(T::BLOCKS % NW == 0, "tile DMA blocks must split over the waves");
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
  int koff[D / 16], voff[4], kdma[PK], vdma[PK];
  k_offsets_pi<D>(l32, hi, koff);
  vt_offsets(l32, hi, voff);
  dma_offsets<D, NW, false>(wave, lane, kdma);
  vt_dma_offsets<D, NW>(wave, lane, vdma);
  constexpr bool kGatherK = std::is_same<KRow, GatherRows>::value;
  int kgr[kGatherK ? PK : 1], kgc[kGatherK ? PK : 1];   // row in the tile, byte in the row, of K unit i
  if constexpr (kGatherK) {
#pragma unroll
    for (int i = 0; i < PK; ++i) {
      kgr[i] = kdma[i] / T::ROWB;
      kgc[i] = kdma[i] % T::ROWB;
    }
  }
  // wave 0: the source rows of the tile with entry e into ring slot `slot`
  auto kfill = [&](int slot, int e) {
    if constexpr (kGatherK)
      if (wave == 0) krow.ring[slot * BK + lane] = krow.tile_src(__builtin_amdgcn_readfirstlane(e) & 0xFFFFFF, lane);
  };
  // a gathered K tile whose rows are in ring slot `slot` (wave's share)
  auto kgoff = [&](int slot, int i) -> int {
    if constexpr (kGatherK) return krow.ring[slot * BK + kgr[i]] * T::ROWB + kgc[i];
    else return 0;
  };
  // A centroid pass continues the softmax state (o, m_run, l_run) of the
  // pass over the exact tiles before it; any other pass starts afresh.
  if constexpr (!Cent::kOn) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
  }
  float mref_c = m_run == -INFINITY ? 0.f : m_run * c;   // m_run * c (0 while m_run is -inf)

  // Tile DMAs through a buffer resource based at the tile: rows past N fall
  // outside the resource's range and read as zero (their scores are masked).
  // (The default keeps the kv-block arithmetic as is: the attention kernels
  // compile to the same code as before the K row became a parameter.)
  constexpr bool kBlockRows = std::is_same<KRow, KvBlockRow>::value;
  auto k_row = [&](int e) -> int {
    if constexpr (kBlockRows || kGatherK) return 0;   // (gathered K takes its rows from the ring)
    else return krow(e);
  };
  auto dma_k = [&](int e, char *tile) {
    if constexpr (Cent::kOn) {
      if (e & kCentFlag) {
        dma_tile_buf<D, NW>(reinterpret_cast<const char *>(cent.k) + (size_t)(e & kCentTileMask) * TB, TB, tile,
                            wave, kdma);
        return;
      }
    }
    if constexpr (kBlockRows) {
      const int kb = e & 0xFFFFFF;
      const int left = (N - kb * BK) * T::ROWB;
      dma_tile_buf<D, NW>(reinterpret_cast<const char *>(Kh) + (size_t)kb * TB, left < TB ? left : TB, tile, wave,
                          kdma);
    } else {
      const int row0 = k_row(e);
      const int left = (N - row0) * T::ROWB;
      dma_tile_buf<D, NW>(reinterpret_cast<const char *>(Kh) + (size_t)row0 * T::ROWB, left < TB ? left : TB, tile,
                          wave, kdma);
    }
  };
  auto dma_v = [&](int e, char *tile) {
    if constexpr (Cent::kOn) {
      if (e & kCentFlag) {
        dma_tile_buf<D, NW>(reinterpret_cast<const char *>(cent.vt) + (size_t)(e & kCentTileMask) * TB, TB, tile,
                            wave, vdma);
        return;
      }
    }
    const int kb = e & 0xFFFFFF;
    dma_tile_buf<D, NW>(reinterpret_cast<const char *>(Vth) + (size_t)kb * TB, TB, tile, wave, vdma);
  };

  // prologue: K(0..2), V(0..1) in flight; S(0) = K(0) Q^T
  int e0 = ent(0), e1 = ent(1), e2 = ent(2), e3 = ent(3);
  if constexpr (kGatherK) {
    kfill(0, e0);
    kfill(1, e1);
    kfill(2, e2);
    kfill(3, e3);
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rh = tile_rsrc(reinterpret_cast<const char *>(Kh), N * T::ROWB);
    char *const kst0[3] = {k0, k1, k2};
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int i = 0; i < PK; ++i) dma_block(rh, kst0[t], wave * PK + i, kgoff(t, i));
  } else {
    dma_k(e0, k0);
    dma_k(e1, k1);
    dma_k(e2, k2);
  }
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
    const int kb_v = e2 & 0xFFFFFF;
    __amdgpu_buffer_rsrc_t rk, rv;
    int kgo[kGatherK ? PK : 1];
    if constexpr (kGatherK) {
      rk = tile_rsrc(reinterpret_cast<const char *>(Kh), N * T::ROWB);
#pragma unroll
      for (int i = 0; i < PK; ++i) kgo[i] = kgoff((it + 3) & 3, i);
    } else if constexpr (kBlockRows) {
      const int kb_k = e3 & 0xFFFFFF;
      const int kleft = (N - kb_k * BK) * T::ROWB;
      rk = tile_rsrc(reinterpret_cast<const char *>(Kh) + (size_t)kb_k * TB, kleft < TB ? kleft : TB);
    } else {
      const int row_k = k_row(e3);
      const int kleft = (N - row_k) * T::ROWB;
      rk = tile_rsrc(reinterpret_cast<const char *>(Kh) + (size_t)row_k * T::ROWB, kleft < TB ? kleft : TB);
    }
    rv = tile_rsrc(reinterpret_cast<const char *>(Vth) + (size_t)kb_v * TB, TB);
    if constexpr (Cent::kOn) {
      if (e3 & kCentFlag)
        rk = tile_rsrc(reinterpret_cast<const char *>(cent.k) + (size_t)(e3 & kCentTileMask) * TB, TB);
      if (e2 & kCentFlag)
        rv = tile_rsrc(reinterpret_cast<const char *>(cent.vt) + (size_t)(e2 & kCentTileMask) * TB, TB);
    }
    auto dma_slot = [&](int ks) {
#pragma unroll
      for (int i = 0; i < 2 * PK; ++i) {
        if (ks != i * (D / 16) / (2 * PK)) continue;
        if (i & 1) dma_block(rv, Vdst, wave * PK + (i >> 1), vdma[i >> 1]);
        else if constexpr (kGatherK) dma_block(rk, Kdst, wave * PK + (i >> 1), kgo[i >> 1]);
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
    // prep masks S(it) and says whether this lane's rows keep the tile at
    // all; a tile they do not keep contributes nothing: its exponentials are
    // taken as exp2(x*0 - inf) = 0 (its scores stay finite).
    n0 = mfma32(kl0[0], qf[0], n0);
    n1 = mfma32(kl1[0], qf[0], n1);
    const bool own = prep(s0, s1, e0);
    float mx = lane_max_tree(s0, s1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 1; q < LEAD; ++q) {
      n0 = mfma32(kl0[q], qf[q], n0);
      n1 = mfma32(kl1[q], qf[q], n1);
    }
    mx = half_swap_max(mx);
    if (!own) mx = -INFINITY;
    // Lazy reference: it moves only when the tile raises the row maximum by
    // more than 2^8 (exp2 units; from -inf it always moves).  A move, rare
    // after the first tiles, rescales l and O in a wave-uniform branch, so
    // the common step computes no rescale factor at all.
    const bool move = mx > m_run && (mx - m_run) * c > kLazyLog2;
    bf16x8 ka0, ka1;
    kread(LEAD, ka0, ka1);
    __builtin_amdgcn_sched_barrier(0);
    if (__builtin_amdgcn_ballot_w64(move)) {
      const float alpha = move ? fast_exp2((m_run - mx) * c) : 1.f;
      m_run = move ? mx : m_run;
      mref_c = m_run == -INFINITY ? 0.f : m_run * c;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
    const float cc = own ? c : 0.f;
    const float mc = own ? mref_c : INFINITY;

    // (B) NKS hand-ordered steps (sched_barrier fences): step ks issues the
    // two MFMAs of S(it+1) for QK step ks + LEAD (K operands read one step
    // ahead), the exponentials of PER scores of S(it), and, once a 16-key
    // chunk of P(it) is complete, its O^T += V^T P^T MFMAs.
    uint32_t pw[16];
    float rs = 0.f;
    // 16-key chunk j of P is complete after sub-step done(j); its P.V MFMAs
    // go kPvDelay sub-steps later (the exponentials and packs have landed)
    // and its V^T operands are read kVLead sub-steps before that.
    constexpr int CPS = 8 / PER;            // sub-steps per chunk
    auto pv_at = [&](int j) { return (j + 1) * CPS - 1 + kPvDelay; };
    auto rd_at = [&](int j) { const int r = pv_at(j) - kVLead; return r < 0 ? 0 : r; };
    bf16x8 va[2][D / 32];
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
      // tile it+4's rows into the slot of tile it (read three steps ago),
      // once the entry's LDS read has surely landed (the K operand reads
      // issued after it have been waited for)
      if (ks == 1) kfill(it & 3, e4_raw);
#pragma unroll
      for (int e = 0; e < PER; e += 2) {
        const int idx = ks * PER + e;      // 0..31: s0 then s1
        const float x0 = idx < 16 ? s0[idx] : s1[idx - 16];
        const float x1 = idx < 16 ? s0[idx + 1] : s1[idx - 15];
        const float p0 = fast_exp2(__builtin_fmaf(x0, cc, -mc));
        const float p1 = fast_exp2(__builtin_fmaf(x1, cc, -mc));
        pw[idx >> 1] = pack_bf16x2(p0, p1);
        if constexpr (SUM_BF16)  // row sum of the probabilities as they enter the MFMA (bf16)
          rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[idx >> 1]), kOnesBf16x2, rs, false);
        else  // row sum of the fp32 probabilities
          rs += p0 + p1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // P.V of the chunks due in this sub-step
        if (pv_at(j) != ks) continue;
        const bf16x8 pj = __builtin_bit_cast(bf16x8, u32x4{pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
#pragma unroll
        for (int db = 0; db < D / 32; ++db) o[db] = mfma32(va[j & 1][db], pj, o[db]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // V^T operands read ahead of their P.V
        if (rd_at(j) != ks) continue;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          va[j & 1][db] = *reinterpret_cast<const bf16x8 *>(Vc + voff[j] + db * 32 * 128);
      }
      ka0 = kn0;
      ka1 = kn1;
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // P.V due after the last sub-step
      if (pv_at(j) < NKS) continue;
      const bf16x8 pj = __builtin_bit_cast(bf16x8, u32x4{pw[4 * j], pw[4 * j + 1], pw[4 * j + 2], pw[4 * j + 3]});
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] = mfma32(va[j & 1][db], pj, o[db]);
    }
    if constexpr (Cent::kOn)   // a centroid stands for 64 keys: its probability counts 64 times (exact)
      l_run += (e0 & kCentFlag) ? 64.f * rs : rs;
    else
      l_run += rs;

    // (C) K(it+2) and V(it+1), issued one step ago, have landed once at most
    // this step's 2*PK DMAs are outstanding; then every wave's share is in
    // (and, gathering K, wave 0's ring writes are done)
    if constexpr (kGatherK) __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
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
}

}  // namespace core
}  // namespace svgk
