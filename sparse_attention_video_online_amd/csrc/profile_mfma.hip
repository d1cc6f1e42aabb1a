// Online head profiling on bf16 inputs with MFMA (gfx950).
//
// Same computation as the vector profiler: for each sampled row, the full,
// spatial-masked and temporal-masked attention outputs, each normalised
// over its own kept keys with its own maximum.  Then per-head MSEs of the
// masked outputs against the full one, and the label (ties -> spatial).
//
// Two passes, both on the attention kernel's V^T tile pipeline (vt_attend:
// 8 waves x 32 sampled rows, K and a key-tiled V^T DMA'd into LDS).  V^T is
// laid out with every frame (then the text) starting a new 64-key tile.
// The full pass walks key chunks that never cross a frame boundary: each is
// one frame, or a part of one, or a part of the text.  A spatial window is a
// run of whole frames plus the text, so the spatial output of a row is the
// merge of the full pass's chunks inside its window: no spatial pass is run.
// The temporal pass takes one work-group per (256 samples in position-major
// order, frame): it walks the frame's tiles that its rows' position windows
// reach, each row masking the keys outside its own window; the text keys,
// kept by every row, come from the full pass's text chunks.  Chunks are
// merged afterwards (flash-decoding style), and the squared errors are
// summed in fp64 in a fixed order.  A narrow temporal window (a few keys
// per frame) goes to a one-wave-per-row vector kernel instead.
#include "attn_vt_core.h"

namespace svgk {
namespace {

using namespace core;

// Both passes: 8 waves = 256 samples per work-group on the V^T tile
// pipeline (vt_attend), one work-group per CU.
constexpr int FNW = 8;
constexpr int FNT = FNW * 64;
constexpr int FQ = FNW * 32;
constexpr int kFullSlots = 256;   // full-pass work-groups resident at once (one per CU, 256 CUs)

// Key chunks of the full pass: each frame in P parts of tpp tiles, the
// text in Pt parts of at most tpp tiles; chunk ch < F*P is part ch % P of
// frame ch / P, the text parts follow.  The pass takes about
// max(total work / resident work-groups, longest work-group), a work-group
// costing its tiles plus a fixed ~8 tiles (Q load, pipeline fill, partial
// store); take the cheapest tpp.  At the HunyuanVideo layer shape: whole
// frames (57 tiles), 34 chunks, 4080 work-groups.
struct FrameGrid { int nqg, nbf, nbt, tpp, P, Pt, nchunks; };

FrameGrid profile_grid_full(const Dims &dm, int n_s) {
  FrameGrid g;
  g.nqg = (n_s + FQ - 1) / FQ;
  g.nbf = (dm.S + BK - 1) / BK;
  g.nbt = (dm.T + BK - 1) / BK;
  double best = -1.0;
  for (int P = 1; P <= g.nbf; ++P) {
    const int tpp = (g.nbf + P - 1) / P;
    const int Pf = (g.nbf + tpp - 1) / tpp, Pt = (g.nbt + tpp - 1) / tpp;
    const double work = (double)dm.H * g.nqg *
                        ((double)dm.F * (g.nbf + 8 * Pf) + (g.nbt + 8 * Pt));
    const double cost = fmax(work / kFullSlots, (double)(tpp + 8));
    if (best < 0.0 || cost < best) {
      best = cost;
      g.tpp = tpp;
      g.P = Pf;
      g.Pt = Pt;
    }
  }
  g.nchunks = dm.F * g.P + g.Pt;
  return g;
}

// Frames per temporal work-group.  Its walk is about (frames) x (tiles that
// a 256-sample group's ranges reach in a frame: the positions the group
// spans, S * 256 / n_s, plus a range on each side) plus ~8 tiles of fixed
// cost; work-groups of one length finish in ceil(count / 256) rounds, so
// take the fewest rounds x length.  At the HunyuanVideo layer shape: 2
// frames (17 chunks, 2,040 work-groups of ~64 tiles).
struct TemporalGrid { int fpc, nchunks; };

TemporalGrid profile_grid_temporal(const Dims &dm, int n_s, int wt) {
  const int nqg = (n_s + FQ - 1) / FQ, nbf = (dm.S + BK - 1) / BK;
  const long long wq = min(wt, dm.N) / dm.F;
  const long long span = min((long long)dm.S, (long long)dm.S * FQ / max(n_s, 1) + 2 * wq + 2);
  const int ntf = min(nbf, (int)((span + BK - 1) / BK) + 1);
  long long best = -1;
  TemporalGrid g{1, dm.F};
  for (int fpc = 1; fpc <= dm.F; ++fpc) {
    const int nch = (dm.F + fpc - 1) / fpc;
    const long long nwg = (long long)dm.H * nqg * nch;
    const long long cost = (nwg + kFullSlots - 1) / kFullSlots * ((long long)fpc * ntf + 8);
    if (best < 0 || cost < best) {
      best = cost;
      g = TemporalGrid{fpc, nch};
    }
  }
  return g;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct Parts {
  float *fo, *fml;  // full pass: [H][n_s][Cf][D], [H][n_s][Cf][2] (O, max, sum)
  float *to, *tml;  // temporal pass: [H][n_s][Ct][D], [H][n_s][Ct][2]
  double *se;       // [H][n_s][2]
  int32_t *ord_t;   // [n_s]
  bf16_t *vt;       // V in its own token order, key-tiled transposed, frames
                    // padded to whole tiles: [H][vt_frame_tiles][D][64]
  size_t bytes;     // workspace size
};

// Workspace layout for Cf full-pass and Ct temporal chunks (ws may be null
// to get the size only).
Parts carve(void *ws, const Dims &dm, int n_s, int Cf, int Ct) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char *q = (char *)((uintptr_t)ws + off);
    off += align256(bytes);
    return q;
  };
  const size_t rows = (size_t)dm.H * n_s;
  Parts r;
  r.fo = (float *)take(rows * Cf * dm.d * sizeof(float));
  r.fml = (float *)take(rows * Cf * 2 * sizeof(float));
  r.to = (float *)take(rows * Ct * dm.d * sizeof(float));
  r.tml = (float *)take(rows * Ct * 2 * sizeof(float));
  r.se = (double *)take(rows * 2 * sizeof(double));
  r.ord_t = (int32_t *)take((size_t)n_s * 4);
  r.vt = (bf16_t *)take((size_t)dm.H * vt_frame_tiles(dm) * BK * dm.d * sizeof(bf16_t));
  r.bytes = off;
  return r;
}

constexpr int kMaxRankSamples = 16384;

// Order of the samples for the work-groups of the temporal pass: by
// position-major index p*F + f (a work-group's samples then share few grid
// positions), text rows last, ties in sample order.  Only the grouping of
// samples into work-groups changes; each sample's result has its own slot.
__global__ __launch_bounds__(256)
void profile_order(const int32_t *__restrict__ sample_idx, int n_s, int F, int S, int32_t *__restrict__ ord_t) {
  __shared__ __attribute__((aligned(16))) int cr[1024];
  const int s = blockIdx.x * 256 + threadIdx.x;
  const bool act = s < n_s;
  if (n_s > kMaxRankSamples) {
    if (act) ord_t[s] = s;
    return;
  }
  const int FS = F * S;
  auto rpos = [&](int i) { return i >= FS ? i : (i % S) * F + i / S; };
  const int i = act ? sample_idx[s] : 0, r = rpos(i);
  int rt = 0;
  for (int base = 0; base < n_s; base += 1024) {
    const int cnt = min(1024, n_s - base);
    __syncthreads();
    for (int u = threadIdx.x; u < cnt; u += 256) cr[u] = rpos(sample_idx[base + u]);
    __syncthreads();
    // four ranks a 16-byte LDS read, several reads in flight
    const int c4 = cnt & ~3;
#pragma unroll 4
    for (int u = 0; u < c4; u += 4) {
      const int4 q = *reinterpret_cast<const int4 *>(cr + u);
      const int us = base + u;
      rt += (q.x < r) || (q.x == r && us < s);
      rt += (q.y < r) || (q.y == r && us + 1 < s);
      rt += (q.z < r) || (q.z == r && us + 2 < s);
      rt += (q.w < r) || (q.w == r && us + 3 < s);
    }
    for (int u = c4; u < cnt; ++u) {
      const int q = cr[u], us = base + u;
      rt += (q < r) || (q == r && us < s);
    }
  }
  if (act) ord_t[rt] = s;
}

// The full pass (no mask) for the work-group's 256 samples, in their given
// order, over one key chunk (a part of a frame, or of the text) on the V^T
// tile pipeline: K and the frame-padded key-tiled V^T DMA'd into three LDS
// stages, MFMA QK and PV, lazy-rescale online softmax.  The partial result
// of the chunk (O unnormalised, reference maximum, row sum) goes to slot
// (h, sample, chunk) of part_o / part_ml.  The work-groups of one chunk
// (the sample groups) are consecutive on one XCD and share its L2.
template <int D>
__global__ __launch_bounds__(FNT, 1)
void profile_full_vt(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ Vt,
                     const int32_t *__restrict__ sample_idx, int n_s, int F, int S, int T, int nqg, int nbf,
                     int nbt, int tpp, int P, int Cf, float c, float *__restrict__ part_o,
                     float *__restrict__ part_ml) {
  constexpr int TB = DTile<D>::TBYTES;
  // V^T stages named to sort first, below 64 KB of LDS (immediate offsets)
  __shared__ __attribute__((aligned(1024))) char k0[TB], k1[TB], k2[TB], V0[TB], V1[TB], V2[TB];
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qg = work % nqg, chunk = (work / nqg) % Cf, h = work / (nqg * Cf);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int N = F * S + T;
  const size_t hoff = (size_t)h * N * D;
  const int pos = qg * FQ + wave * 32 + (lane & 31);
  const bool valid = pos < n_s;
  const int i = valid ? sample_idx[pos] : 0;
  // the chunk's keys: rows krow0 .. krow0 + nrows - 1 (to the end of its
  // frame or of the text), tiles vt0 .. vt0 + nt - 1 of the padded V^T
  int krow0, nrows, vt0, nt;
  if (chunk < F * P) {
    const int f = chunk / P, t0 = (chunk - f * P) * tpp;
    krow0 = f * S + t0 * BK;
    nrows = S - t0 * BK;
    vt0 = f * nbf + t0;
    nt = min(nbf - t0, tpp);
  } else {
    const int t0 = (chunk - F * P) * tpp;
    krow0 = F * S + t0 * BK;
    nrows = T - t0 * BK;
    vt0 = F * nbf + t0;
    nt = min(nbt - t0, tpp);
  }
  auto ent_raw = [&](int j) -> int { return j < nt ? j : nt - 1; };
  auto prep = [&](f32x16 &s0, f32x16 &s1, int e) -> bool {
    if ((e + 1) * BK > nrows) {  // keys past the frame's end: only in its last tile
      const int nvh = nrows - e * BK - 8 * hi;   // acc_key_pi(b, r, hi) = acc_key_pi(b, r, 0) + 8 hi
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (acc_key_pi(0, r, 0) >= nvh) s0[r] = -INFINITY;
        if (acc_key_pi(1, r, 0) >= nvh) s1[r] = -INFINITY;
      }
    }
    return true;
  };
  bf16x8 qf[D / 16];
  load_q<D>(Q + hoff, valid ? i : -1, hi, qf);
  f32x16 o[D / 32];
  float m_run, l_run;
  // Row sums of the fp32 probabilities, as the temporal pass takes them: the
  // three outputs then share one rounding convention, and the small MSEs of
  // heads whose masks both keep nearly all the weight stay comparable.
  const int nkbf = F * nbf + nbt;
  vt_attend<D, FNW, false>(nt, ent_raw, prep, K + hoff + (size_t)krow0 * D,
                           Vt + ((size_t)h * nkbf + vt0) * (BK * D), nrows, k0, k1, k2, V0, V1, V2, qf, wave, lane,
                           c, o, m_run, l_run);
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may land after the work-group ends
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (!valid) return;
  const size_t slot = ((size_t)h * n_s + pos) * Cf + chunk;
  float *dst = part_o + slot * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4 *>(dst + 32 * db + 8 * g + 4 * hi) =
          f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
  if (hi == 0) {
    part_ml[slot * 2] = m_run;
    part_ml[slot * 2 + 1] = lt;
  }
}

// The temporal pass on the V^T tile pipeline: the work-group's 256 samples
// (in position-major order, so they share few grid positions) against the
// video keys of frames fa .. fa + fpc - 1, in one pipeline run.  A row at
// grid position pi keeps, in frame f, the positions pi - floor((w_t + f)/F)
// .. pi + floor((F - 1 + w_t - f)/F) (its rank window p*F + f within
// [pi*F - w_t, pi*F + F - 1 + w_t]); the work-group walks, in each of its
// frames, the tiles that the union of its rows' ranges touches, and each row
// masks the keys outside its own range.  Text rows are skipped (they keep
// every key: their temporal output is the full one) and the text keys, kept
// by every row, come from the full pass's text chunks in the merge.  The
// partial of (sample, frame group) goes to slot (h, sample, chunk).
template <int D>
__global__ __launch_bounds__(FNT, 1)
void profile_temporal_vt(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ Vt,
                         const int32_t *__restrict__ sample_idx, const int32_t *__restrict__ order, int n_s, int F,
                         int S, int T, int wt, int nqg, int nbf, int nbt, int fpc, int Ct, float c,
                         float *__restrict__ part_o, float *__restrict__ part_ml) {
  constexpr int TB = DTile<D>::TBYTES;
  // V^T stages named to sort first, below 64 KB of LDS (immediate offsets)
  __shared__ __attribute__((aligned(1024))) char k0[TB], k1[TB], k2[TB], V0[TB], V1[TB], V2[TB];
  __shared__ int prange[2];   // smallest and largest grid position of the video rows
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int qg = work % nqg, chunk = (work / nqg) % Ct, h = work / (nqg * Ct);
  const int fa = chunk * fpc, nf = min(F, fa + fpc) - fa;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5;
  const int FS = F * S, N = FS + T;
  const size_t hoff = (size_t)h * N * D;
  const int pos = qg * FQ + wave * 32 + (lane & 31);
  const int sidx = pos < n_s ? order[pos] : 0;
  const int i = pos < n_s ? sample_idx[sidx] : FS;
  const bool valid = i < FS;                    // a video row of this work-group
  const int pi = valid ? i % S : 0;
  // w_t clamped to N keeps int32; a row's range in frame f reaches wq or
  // wq + 1 positions to each side
  const int wtc = min(wt, N);
  const int wq = wtc / F, wr = wtc - wq * F;
  if (tid == 0) {
    prange[0] = 0x7fffffff;
    prange[1] = -1;
  }
  __syncthreads();
  if (valid) {
    atomicMin(&prange[0], pi);
    atomicMax(&prange[1], pi);
  }
  __syncthreads();
  const int p_lo = prange[0], p_hi = prange[1];
  if (p_hi < 0) return;   // no video row: nothing to compute (uniform)
  // local tiles t0 .. t0 + ntf - 1 cover the union of the rows' ranges in
  // every frame; tile j of the walk is tile t0 + j % ntf of frame fa + j / ntf
  const int t0 = max(p_lo - wq - 1, 0) / BK, ntf = min(p_hi + wq + 1, S - 1) / BK - t0 + 1;
  const int nt = nf * ntf;
  auto ent_raw = [&](int j) -> int {
    const int jj = j < nt ? j : nt - 1;
    const int fr = jj / ntf;
    return (fa + fr) * nbf + t0 + (jj - fr * ntf);   // tile of the frame-padded V^T
  };
  // K is not padded: the tile's first row is frame f's row 64 t
  auto krow = [=](int e) -> int {
    const int f = e / nbf;
    return f * S + (e - f * nbf) * BK;
  };
  auto prep = [&](f32x16 &s0, f32x16 &s1, int e) -> bool {
    const int f = e / nbf, kb = (e - f * nbf) * BK;
    const int lo = max(pi - (wq + (f + wr >= F)), 0), hk = min(pi + (wq + (f < wr)), S - 1);
    const bool own = valid && lo <= kb + BK - 1 && hk >= kb;
    const bool whole = !valid || (lo <= kb && hk >= kb + BK - 1);
    if (__builtin_amdgcn_ballot_w64(!whole)) {
      // keep offset acc_key_pi(b, r, hi) = acc_key_pi(b, r, 0) + 8 hi iff it
      // lies in [lo, hk] - kb.  A row that keeps none of the tile is left
      // unmasked: the pipeline zeroes it by scaling with 0, and -inf * 0
      // would be NaN.
      const int a = own ? lo - kb - 8 * hi : 0;
      const unsigned span = own ? (unsigned)(hk - lo) : 0xFFFFFFFFu;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if ((unsigned)(acc_key_pi(0, r, 0) - a) > span) s0[r] = -INFINITY;
        if ((unsigned)(acc_key_pi(1, r, 0) - a) > span) s1[r] = -INFINITY;
      }
    }
    return own;
  };
  bf16x8 qf[D / 16];
  load_q<D>(Q + hoff, valid ? i : -1, hi, qf);
  f32x16 o[D / 32];
  float m_run, l_run;
  const int nkbf = F * nbf + nbt;
  vt_attend<D, FNW, false>(nt, ent_raw, prep, K + hoff, Vt + (size_t)h * nkbf * (BK * D), N, k0, k1, k2, V0, V1,
                           V2, qf, wave, lane, c, o, m_run, l_run, krow);
  __builtin_amdgcn_s_waitcnt(0);  // no DMA may land after the work-group ends
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (!valid) return;
  const size_t slot = ((size_t)h * n_s + sidx) * Ct + chunk;
  float *dst = part_o + slot * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<f32x4 *>(dst + 32 * db + 8 * g + 4 * hi) =
          f32x4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
  if (hi == 0) {
    part_ml[slot * 2] = m_run;
    part_ml[slot * 2 + 1] = lt;
  }
}

// The temporal pass for narrow windows (2 w_t + F <= kNarrowKeys video keys
// a row, e.g. w_t = 32 at F = 13: 77), where a tile walk would compute
// whole frames of keys that every row but a few masks.  One wave per sampled
// video row, in float32 on the vector ALUs: each lane takes up to four keys
// of the row's window (executing row r = p F + f is video row f S + p), the
// scores are q.k summed over the dims in order, the wave's maximum and
// sum are reduced, and each lane accumulates one or two dims of O over the
// keys in order.  The partial (O unnormalised, the maximum, the sum) takes
// the row's single temporal slot (Ct = 1), as the tile pass does per chunk.
// Text rows keep every key (their temporal output is the full one) and are
// skipped.
constexpr int kNarrowKeys = 256;

template <int D>
__global__ __launch_bounds__(256)
void profile_temporal_narrow(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K,
                             const bf16_t *__restrict__ V, const int32_t *__restrict__ sample_idx, int n_s, int F,
                             int S, int T, int wt, float c, float *__restrict__ part_o, float *__restrict__ part_ml) {
  __shared__ float qs[4][D];
  __shared__ float ps[4][kNarrowKeys];
  __shared__ int rs[4][kNarrowKeys];
  const int h = blockIdx.y, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + wave;
  const int FS = F * S, N = FS + T;
  const int i = s < n_s ? sample_idx[s] : FS;
  if (i >= FS) return;                         // wave-uniform; no barrier below
  const size_t hoff = (size_t)h * N * D;
  const bf16_t *Kh = K + hoff, *Vh = V + hoff;
  const int p = i % S;
  const int r0 = max(0, p * F - wt), r1 = min(FS - 1, p * F + F - 1 + wt);
  const int nk = r1 - r0 + 1;                  // <= 2 wt + F <= kNarrowKeys (checked by the launch)
  for (int e = lane; e < D; e += 64) qs[wave][e] = bf16_to_f32(Q[hoff + (size_t)i * D + e]);
  __builtin_amdgcn_wave_barrier();
  // scores of the lane's keys j = lane + 64 u
  float sc[4];
  int src[4];
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = lane + 64 * u;
    sc[u] = -INFINITY;
    src[u] = 0;
    if (j < nk) {
      const int r = r0 + j, pp = r / F;
      src[u] = (r - pp * F) * S + pp;
      const u32x4 *kr = reinterpret_cast<const u32x4 *>(Kh + (size_t)src[u] * D);
      float acc = 0.f;
#pragma unroll
      for (int v = 0; v < D / 8; ++v) {
        const u32x4 w = kr[v];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = __builtin_fmaf(qs[wave][8 * v + 2 * q], __uint_as_float(w[q] << 16), acc);
          acc = __builtin_fmaf(qs[wave][8 * v + 2 * q + 1], __uint_as_float(w[q] & 0xFFFF0000u), acc);
        }
      }
      sc[u] = acc;
      mx = fmaxf(mx, acc);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float l = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = lane + 64 * u;
    const float pj = j < nk ? fast_exp2((sc[u] - mx) * c) : 0.f;
    l += pj;
    if (j < nk) {
      ps[wave][j] = pj;
      rs[wave][j] = src[u];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  __builtin_amdgcn_wave_barrier();
  // O: lane's dims lane (+ 64), keys in order, eight rows' loads in flight
  constexpr int DL = D / 64;
  float o[DL];
#pragma unroll
  for (int t = 0; t < DL; ++t) o[t] = 0.f;
  for (int j0 = 0; j0 < nk; j0 += 8) {
    float vv[8][DL];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int t = 0; t < DL; ++t)
        vv[u][t] = j0 + u < nk ? bf16_to_f32(Vh[(size_t)rs[wave][j0 + u] * D + lane + 64 * t]) : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j0 + u < nk)
#pragma unroll
        for (int t = 0; t < DL; ++t) o[t] = __builtin_fmaf(ps[wave][j0 + u], vv[u][t], o[t]);
  }
  const size_t slot = (size_t)h * n_s + s;     // Ct = 1
#pragma unroll
  for (int t = 0; t < DL; ++t) part_o[slot * D + lane + 64 * t] = o[t];
  if (lane == 0) {
    part_ml[slot * 2] = mx;
    part_ml[slot * 2 + 1] = l;
  }
}

// Merge the chunks of one sampled row into its three outputs and take the
// squared errors of the masked ones.  Full: every chunk of the full pass.
// Spatial: the full pass's chunks of the frames within ks of the row's frame
// and the text chunks (a text row keeps every key: its full output).
// Temporal: the temporal pass's chunks.  A mask that keeps every key of
// every row (cover bit 1: spatial, 2: temporal) has the full output as its
// output, exactly: its merge is skipped (the temporal pass was not run).
// One wave per row (four rows per work-group), a lane per dim (two at
// d = 128); the squared errors are summed over the dims by a fixed
// butterfly in float64.
template <int D>
__global__ __launch_bounds__(256)
void profile_combine(const float *__restrict__ fo, const float *__restrict__ fml, int Cf, int P,
                     const float *__restrict__ to, const float *__restrict__ tml, int Ct,
                     const int32_t *__restrict__ sample_idx, int n_s, int F, int S, int ks, int cover,
                     float c, double *__restrict__ se) {
  constexpr int DL = D / 64;
  const int h = blockIdx.y, lane = threadIdx.x & 63, s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= n_s) return;                        // wave-uniform; no barrier below
  const int i = sample_idx[s];
  const bool text_i = i >= F * S;
  const int fi = text_i ? 0 : i / S;
  const bool sp_all = text_i || (cover & 2);
  auto in_window = [&](int ch) { return sp_all || ch >= F * P || abs(ch / P - fi) <= ks; };
  const size_t rf = ((size_t)h * n_s + s) * Cf, rt = ((size_t)h * n_s + s) * Ct;
  // maxima of the full and the spatial merge
  float M0 = -INFINITY, M1 = -INFINITY;
  for (int ch = 0; ch < Cf; ++ch) {
    const float m = fml[(rf + ch) * 2];
    M0 = fmaxf(M0, m);
    if (in_window(ch)) M1 = fmaxf(M1, m);
  }
  const float M0r = M0 == -INFINITY ? 0.f : M0, M1r = M1 == -INFINITY ? 0.f : M1;
  // The merges run in chunk order; the loads of kB chunks go out together
  // (one chunk at a time leaves the loop waiting on memory).
  constexpr int kB = 8;
  double L0 = 0.0, L1 = 0.0, A0[DL], A1[DL];
#pragma unroll
  for (int t = 0; t < DL; ++t) A0[t] = A1[t] = 0.0;
  auto add_full = [&](int ch, float m, float l, const float (&x)[DL]) {
    const float w0 = fast_exp2((m - M0r) * c);
    L0 += (double)w0 * l;
#pragma unroll
    for (int t = 0; t < DL; ++t) A0[t] += (double)w0 * x[t];
    if (in_window(ch)) {
      const float w1 = fast_exp2((m - M1r) * c);
      L1 += (double)w1 * l;
#pragma unroll
      for (int t = 0; t < DL; ++t) A1[t] += (double)w1 * x[t];
    }
  };
  int ch = 0;
  for (; ch + kB <= Cf; ch += kB) {
    float m[kB], l[kB], x[kB][DL];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      m[u] = fml[(rf + ch + u) * 2];
      l[u] = fml[(rf + ch + u) * 2 + 1];
#pragma unroll
      for (int t = 0; t < DL; ++t) x[u][t] = fo[(rf + ch + u) * D + lane + 64 * t];
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) add_full(ch + u, m[u], l[u], x[u]);
  }
  for (; ch < Cf; ++ch) {
    float x[DL];
#pragma unroll
    for (int t = 0; t < DL; ++t) x[t] = fo[(rf + ch) * D + lane + 64 * t];
    add_full(ch, fml[(rf + ch) * 2], fml[(rf + ch) * 2 + 1], x);
  }
  double out0[DL], out1[DL], out2[DL];
#pragma unroll
  for (int t = 0; t < DL; ++t) {
    out0[t] = L0 > 0.0 ? A0[t] / L0 : 0.0;
    out1[t] = L1 > 0.0 ? A1[t] / L1 : 0.0;
    out2[t] = out0[t];
  }
  if (!((cover & 4) || text_i)) {
    // the temporal pass's frame partials, then the full pass's text chunks
    // (every row keeps the text keys)
    float M = -INFINITY;
    for (int ct = 0; ct < Ct; ++ct) M = fmaxf(M, tml[(rt + ct) * 2]);
    for (int cc = F * P; cc < Cf; ++cc) M = fmaxf(M, fml[(rf + cc) * 2]);
    const float Mr = M == -INFINITY ? 0.f : M;
    double L = 0.0, acc[DL];
#pragma unroll
    for (int t = 0; t < DL; ++t) acc[t] = 0.0;
    auto add = [&](float m, float l, const float (&x)[DL]) {
      const float w = fast_exp2((m - Mr) * c);
      L += (double)w * l;
#pragma unroll
      for (int t = 0; t < DL; ++t) acc[t] += (double)w * x[t];
    };
    int ct = 0;
    for (; ct + kB <= Ct; ct += kB) {
      float m[kB], l[kB], x[kB][DL];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        m[u] = tml[(rt + ct + u) * 2];
        l[u] = tml[(rt + ct + u) * 2 + 1];
#pragma unroll
        for (int t = 0; t < DL; ++t) x[u][t] = to[(rt + ct + u) * D + lane + 64 * t];
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) add(m[u], l[u], x[u]);
    }
    for (; ct < Ct; ++ct) {
      float x[DL];
#pragma unroll
      for (int t = 0; t < DL; ++t) x[t] = to[(rt + ct) * D + lane + 64 * t];
      add(tml[(rt + ct) * 2], tml[(rt + ct) * 2 + 1], x);
    }
    for (int cc = F * P; cc < Cf; ++cc) {
      float x[DL];
#pragma unroll
      for (int t = 0; t < DL; ++t) x[t] = fo[(rf + cc) * D + lane + 64 * t];
      add(fml[(rf + cc) * 2], fml[(rf + cc) * 2 + 1], x);
    }
#pragma unroll
    for (int t = 0; t < DL; ++t) out2[t] = L > 0.0 ? acc[t] / L : 0.0;
  }
  double es = 0.0, et = 0.0;
#pragma unroll
  for (int t = 0; t < DL; ++t) {
    const double ds = out1[t] - out0[t], dt = out2[t] - out0[t];
    es += ds * ds;
    et += dt * dt;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    es += __shfl_xor(es, off);
    et += __shfl_xor(et, off);
  }
  if (lane == 0) {
    se[((size_t)h * n_s + s) * 2] = es;
    se[((size_t)h * n_s + s) * 2 + 1] = et;
  }
}

__global__ __launch_bounds__(256)
void profile_label(const double *__restrict__ se, int n_s, int D, int32_t *__restrict__ labels,
                   float *__restrict__ mse) {
  __shared__ double red[2][256];
  const int h = blockIdx.x, tid = threadIdx.x;
  double a = 0.0, b = 0.0;
  for (int s = tid; s < n_s; s += 256) {
    a += se[((size_t)h * n_s + s) * 2];
    b += se[((size_t)h * n_s + s) * 2 + 1];
  }
  red[0][tid] = a;
  red[1][tid] = b;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      red[0][tid] += red[0][tid + off];
      red[1][tid] += red[1][tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const double n = (double)n_s * D;
    const double ms = red[0][0] / n, mt = red[1][0] / n;
    labels[h] = ms <= mt ? 0 : 1;
    if (mse != nullptr) {
      mse[2 * h] = (float)ms;
      mse[2 * h + 1] = (float)mt;
    }
  }
}

}  // namespace

size_t profile_mfma_ws_bytes(const Dims &dm, int n_s) {
  return carve(nullptr, dm, n_s, profile_grid_full(dm, n_s).nchunks, dm.F).bytes;   // temporal chunks <= F
}

hipError_t launch_profile_mfma(const Dims &dm, const void *Q, const void *K, const void *V,
                               const int32_t *sample_idx, int n_s, int ks, int wt, float scale, int32_t *labels,
                               float *mse, void *ws, hipStream_t st) {
  const float c = scale * kLog2e;
  const FrameGrid gf = profile_grid_full(dm, n_s);          // full pass
  const TemporalGrid gt = profile_grid_temporal(dm, n_s, wt);   // temporal pass
  const Parts p = carve(ws, dm, n_s, gf.nchunks, dm.F);       // temporal partials laid out for up to F chunks
  // A mask that keeps every key of every row: the spatial one when every
  // frame lies within ks of every other (ks >= F - 1), the temporal one when
  // the window of position 0 reaches the last video key and that of position
  // S - 1 the first (wt >= (S - 1) * F); text rows and keys are kept anyway.
  const int cover = ((ks >= dm.F - 1) ? 2 : 0) | (((long long)wt >= (long long)(dm.S - 1) * dm.F) ? 4 : 0);
  // a narrow temporal window: one wave per row on the vector ALUs (no
  // sample order, one temporal slot a row); else the tile pass
  const bool narrow = !(cover & 4) && 2LL * wt + dm.F <= kNarrowKeys;
  const int ct = narrow ? 1 : gt.nchunks;
  if (!narrow)
    hipLaunchKernelGGL(profile_order, dim3((n_s + 255) / 256), dim3(256), 0, st, sample_idx, n_s, dm.F, dm.S,
                       p.ord_t);
  // key-tiled V^T of V in its own token order, every frame from a new tile
  const hipError_t ev = launch_layout_vt(dm, V, p.vt, nullptr, st, kVtFrames);
  if (ev != hipSuccess) return ev;
  const dim3 gridf(gf.nqg * gf.nchunks * dm.H), gridt(gf.nqg * gt.nchunks * dm.H);
#define SVG_PROFILE_PASSES(DD)                                                                                   \
  hipLaunchKernelGGL((profile_full_vt<DD>), gridf, dim3(FNT), 0, st, (const bf16_t *)Q, (const bf16_t *)K, p.vt, \
                     sample_idx, n_s, dm.F, dm.S, dm.T, gf.nqg, gf.nbf, gf.nbt, gf.tpp, gf.P, gf.nchunks, c, p.fo, \
                     p.fml);                                                                                     \
  if (narrow)                                                                                                   \
    hipLaunchKernelGGL((profile_temporal_narrow<DD>), dim3((n_s + 3) / 4, dm.H), dim3(256), 0, st,                \
                       (const bf16_t *)Q, (const bf16_t *)K, (const bf16_t *)V, sample_idx, n_s, dm.F, dm.S, dm.T, \
                       wt, c, p.to, p.tml);                                                                     \
  else if (!(cover & 4))                                                                                        \
    hipLaunchKernelGGL((profile_temporal_vt<DD>), gridt, dim3(FNT), 0, st, (const bf16_t *)Q, (const bf16_t *)K,   \
                       p.vt, sample_idx, p.ord_t, n_s, dm.F, dm.S, dm.T, wt, gf.nqg, gf.nbf, gf.nbt, gt.fpc,        \
                       gt.nchunks, c, p.to, p.tml)
  if (dm.d == 128) {
    SVG_PROFILE_PASSES(128);
  } else {
    SVG_PROFILE_PASSES(64);
  }
#undef SVG_PROFILE_PASSES
  const dim3 gridc((n_s + 3) / 4, dm.H);
  if (dm.d == 128)
    hipLaunchKernelGGL(profile_combine<128>, gridc, dim3(256), 0, st, p.fo, p.fml, gf.nchunks, gf.P, p.to, p.tml, ct,
                       sample_idx, n_s, dm.F, dm.S, ks, cover, c, p.se);
  else
    hipLaunchKernelGGL(profile_combine<64>, gridc, dim3(256), 0, st, p.fo, p.fml, gf.nchunks, gf.P, p.to, p.tml, ct,
                       sample_idx, n_s, dm.F, dm.S, ks, cover, c, p.se);
  hipLaunchKernelGGL(profile_label, dim3(dm.H), dim3(256), 0, st, p.se, n_s, dm.d, labels, mse);
  return hipGetLastError();
}

}  // namespace svgk
