// Online head profiling on bf16 inputs with MFMA (gfx950).
//
// Same computation as the vector profiler: for each sampled row, the full,
// spatial-masked and temporal-masked attention outputs, each normalised
// over its own kept keys with its own maximum.  Then per-head MSEs of the
// masked outputs against the full one, and the label (ties -> spatial).
//
// Two passes.  The full pass runs the attention kernel's V^T tile pipeline
// (vt_attend: 8 waves x 32 sampled rows, K and a key-tiled V^T DMA'd into
// LDS) over key chunks that never cross a frame boundary: V^T is laid out
// with every frame (then the text) starting a new 64-key tile, and each
// chunk is one frame, or a part of one, or a part of the text.  A spatial
// window is a run of whole frames plus the text, so the spatial output of a
// row is the merge of the full pass's chunks inside its window: no spatial
// pass is run.  The temporal pass uses the S^T = K Q^T / O^T += V^T P^T
// machinery of attn_core.h on 128 sampled rows (4 waves x 32) grouped by
// grid position, and visits only the key tiles that some sample's window
// (or a text key) reaches.  In a flagged tile each row keeps at most two
// key ranges, one per frame the tile touches: a wave whose rows keep none of
// the tile skips its math, a wave whose rows keep all of it needs no mask,
// and the others test each score's key offset against the two ranges.
// Chunks are merged afterwards (flash-decoding style), and the squared
// errors are summed in fp64 in a fixed order.
#include "attn_vt_core.h"

namespace svgk {
namespace {

using namespace core;

constexpr int PNW = 4;
constexpr int PNT = PNW * 64;
constexpr int PQ = PNW * 32;

struct ProfileGrid { int nqg, nchunks, tiles_per_chunk; };

// The full pass: 8 waves = 256 samples per work-group on the V^T tile
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

// Key chunks of the temporal pass per (head, sample group): about 2048
// work-groups, four rounds of the 512 resident ones.  Fewer chunks leave the
// work in the few work-groups whose chunk holds a sample group's windows;
// more chunks cost merge traffic.
ProfileGrid profile_grid(const Dims &dm, int n_s) {
  const int nkb = (dm.N + BK - 1) / BK;
  const int nqg = (n_s + PQ - 1) / PQ;
  int c = (2048 + dm.H * nqg - 1) / (dm.H * nqg);
  c = max(1, min(c, max(1, nkb / 4)));
  int tpc = (nkb + c - 1) / c;
  tpc = min(tpc, 4096);
  return ProfileGrid{nqg, (nkb + tpc - 1) / tpc, tpc};
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

constexpr int kMaxVisit = 4096;   // visit-list capacity (tiles per chunk)
constexpr int kMaxRankSamples = 16384;

// Order of the samples for the work-groups of the temporal pass: by
// position-major index p*F + f (a work-group's samples then share few grid
// positions), text rows last, ties in sample order.  Only the grouping of
// samples into work-groups changes; each sample's result has its own slot.
__global__ __launch_bounds__(256)
void profile_order(const int32_t *__restrict__ sample_idx, int n_s, int F, int S, int32_t *__restrict__ ord_t) {
  __shared__ int cr[1024];
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
    for (int u = 0; u < cnt; ++u) {
      const int q = cr[u], us = base + u;
      rt += (q < r) || (q == r && us < s);
    }
  }
  if (act) ord_t[rt] = s;
}

// The temporal pass for the work-group's 128 sampled rows over one chunk of
// key tiles.  A prologue lists the chunk's tiles that some sample of the
// work-group keeps (any key), and flags the tiles where some video sample
// does not keep every video key: only those evaluate the token mask.
template <int D>
__global__ __launch_bounds__(PNT, 2)
void profile_temporal_mfma(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ V,
                           const int32_t *__restrict__ sample_idx, const int32_t *__restrict__ order, int n_s,
                           int F, int S, int N, int wt, int nkb, int tpc, int cstride, float c,
                           float *__restrict__ part_o, float *__restrict__ part_ml) {
  using C = Tile<D, PNT>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  __shared__ uint16_t vlist[kMaxVisit];   // tile - t0, bit 15: evaluate the mask
  __shared__ int bnd[5];     // -, video query present, p_lo, p_hi, text query present
  __shared__ int wcount[PNW + 1];
  const int h = blockIdx.z, chunk = blockIdx.y, qg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)h * N * D;
  const bf16_t *Kh = K + hoff, *Vh = V + hoff;

  const int pos = qg * PQ + wave * 32 + l32;
  const bool valid = pos < n_s;
  const int sidx = valid ? order[pos] : 0;
  const int i = valid ? sample_idx[sidx] : 0;
  const int FS = F * S;
  const bool text_i = i >= FS;
  const int fi = text_i ? 0 : i / S;
  const int pi = text_i ? 0 : i - fi * S;
  // temporal window of this row in position-major units (wt clamped so the
  // bounds stay in int32)
  const int wtc = min(wt, N);
  const int tlo = pi * F - wtc, thi = pi * F + F - 1 + wtc;
  // The same window per key frame f: positions pi - floor((wtc + f)/F) ..
  // pi + floor((F - 1 + wtc - f)/F).  With wtc = wq*F + wr (0 <= wr < F) and
  // 0 <= f < F the floors are wq + (f + wr >= F) and wq + (f < wr).
  const int wq = wtc / F, wr = wtc - wq * F;
  // Kept keys of frame f for this row, absolute [lo, hi] (lo > hi: none).
  auto frame_keys = [&](int f, int &lo, int &hk) {
    lo = f * S + max(pi - (wq + (f + wr >= F)), 0);
    hk = f * S + min(pi + (wq + (f < wr)), S - 1);
  };

  // ---- visit list of this chunk
  const int t0 = chunk * tpc, t1 = min(nkb, t0 + tpc);
  if (tid < 5) bnd[tid] = (tid & 1) ? -1 : 0x7fffffff;
  if (tid == 4) bnd[4] = 0;
  __syncthreads();
  if (valid) {
    if (text_i) {
      atomicMax(&bnd[4], 1);
    } else {
      atomicMax(&bnd[1], 1);
      atomicMin(&bnd[2], pi);
      atomicMax(&bnd[3], pi);
    }
  }
  __syncthreads();
  const int p_lo = bnd[2], p_hi = bnd[3];
  const bool any_video = bnd[1] > 0, any_text = bnd[4] != 0;
  // union / intersection of the video samples' windows
  const long long RU_lo = (long long)p_lo * F - wtc, RU_hi = (long long)p_hi * F + F - 1 + wtc;
  const long long RI_lo = (long long)p_hi * F - wtc, RI_hi = (long long)p_lo * F + F - 1 + wtc;
  int nv = 0;
  for (int base = t0; base < t1; base += PNT) {
    const int t = base + tid;
    bool visit = false, needmask = false;
    if (t < t1) {
      const int k0 = t * BK, k1 = min(N, k0 + BK) - 1;
      if (k1 >= FS || any_text) visit = true;   // text keys / text rows keep all
      if (k0 < FS && any_video) {
        const int kv1 = min(k1, FS - 1);
        for (int f = k0 / S; f <= kv1 / S; ++f) {
          const int a = max(k0, f * S) - f * S, b = min(kv1, f * S + S - 1) - f * S;
          // positions p in [a, b] with p*F + f inside [RU_lo, RU_hi]
          const long long plo = (RU_lo - f + F - 1) >= 0 ? (RU_lo - f + F - 1) / F : 0;
          const long long phi = RU_hi - f >= 0 ? (RU_hi - f) / F : -1;
          visit |= max((long long)a, plo) <= min((long long)b, phi);
          needmask |= !((long long)a * F + f >= RI_lo && (long long)b * F + f <= RI_hi);
        }
      }
    }
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(visit);
    if (lane == 0) wcount[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int off = nv;
    for (int w = 0; w < wave; ++w) off += wcount[w];
    int tot = 0;
    for (int w = 0; w < PNW; ++w) tot += wcount[w];
    if (visit) {
      const int rank = __builtin_popcountll(bal & ((1ull << lane) - 1ull));
      vlist[off + rank] = (uint16_t)((t - t0) | (needmask ? 0x8000 : 0));
    }
    nv += tot;
    __syncthreads();
  }

  bf16x8 qf[D / 16];
  load_q<D>(Q + hoff, valid ? i : -1, hi, qf);
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  Regs<D, PNT> R;
  auto rows_of = [&](int t) {
    return [=](int j) { const int key = t * BK + j; return key < N ? key : -1; };
  };
  if (nv > 0) {
    load_tile<D, PNT>(Kh, Vh, tid, rows_of(t0 + (vlist[0] & 0x7FFF)), R);
    store_tile<D, PNT>(smem, tid, R);
  }
  __syncthreads();
  for (int it = 0; it < nv; ++it) {
    const int e = vlist[it];
    const int t = t0 + (e & 0x7FFF);
    const bool more = it + 1 < nv;
    if (more) load_tile<D, PNT>(Kh, Vh, tid, rows_of(t0 + (vlist[it + 1] & 0x7FFF)), R);
    const char *Ks = smem + (it & 1) * C::STAGE;
    const char *Vs = Ks + C::KBYTES;

    const int kbase = t * BK;
    // Token mask of a flagged tile.  With S >= 64 a tile holds keys of at
    // most two frames (f0, then f0 + 1 from offset sp on; past the video the
    // second part is the text keys, all kept), so this row keeps at most two
    // offset ranges [a0, a0 + n0) and [a1, a1 + n1).  A wave none of whose
    // rows keeps a key of the tile skips its math (the tile adds exact
    // zeros); a wave whose rows keep every key needs no mask.
    bool skip = false, ranges = false, perkey = false;
    int a0 = 0, n0 = 0, a1 = 0, n1 = 0;
    if (e & 0x8000) {
      if (S >= BK) {
        const int nvalid = min(BK, N - kbase);
        if (text_i) {
          n0 = nvalid;
        } else {
          const int f0 = min(kbase, FS - 1) / S;
          const int sp = min(max((f0 + 1) * S - kbase, 0), BK);
          int lo, hk;
          frame_keys(f0, lo, hk);
          a0 = max(lo - kbase, 0);
          n0 = max(min(min(hk - kbase, sp - 1), nvalid - 1) - a0 + 1, 0);
          if (f0 + 1 < F) {
            frame_keys(f0 + 1, lo, hk);
          } else {
            lo = FS;
            hk = N - 1;
          }
          a1 = max(lo - kbase, sp);
          n1 = max(min(min(hk - kbase, BK - 1), nvalid - 1) - a1 + 1, 0);
        }
        const int kept = n0 + n1;
        skip = __builtin_amdgcn_ballot_w64(valid && kept > 0) == 0;
        ranges = __builtin_amdgcn_ballot_w64(valid && kept < nvalid) != 0;
      } else {
        perkey = !text_i;
      }
    }
    if (!skip) {
      f32x16 s0, s1;
      qk_tile<D, PNT>(Ks, qf, l32, hi, s0, s1);
      if (kbase + BK > N) mask_tail(s0, s1, N - kbase, hi);
      if (ranges) {
        // offset acc_key(b, r, hi) = acc_key(b, r, 0) + 4 hi
        const int a0h = a0 - 4 * hi, a1h = a1 - 4 * hi;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = acc_key(b, r, 0);
            const bool keep = (unsigned)(off - a0h) < (unsigned)n0 || (unsigned)(off - a1h) < (unsigned)n1;
            if (!keep) {
              if (b == 0) s0[r] = -INFINITY; else s1[r] = -INFINITY;
            }
          }
        }
      } else if (perkey) {
        // S < 64: a tile spans several frames; the mask per key
#pragma unroll
        for (int b = 0; b < 2; ++b) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + acc_key(b, r, hi);
            if (key >= FS) continue;  // text keys are always kept
            const int fk = key / S;
            const int rk = (key - fk * S) * F + fk;
            if (rk < tlo || rk > thi) {
              if (b == 0) s0[r] = -INFINITY; else s1[r] = -INFINITY;
            }
          }
        }
      }
      bf16x8 pb[4];
      const float alpha = softmax_step(s0, s1, c, m_run, l_run, pb);
      rescale<D>(o, alpha);
      pv_tile<D, PNT>(Vs, pb, l32, hi, o);
    }

    if (more) store_tile<D, PNT>(smem + ((it + 1) & 1) * C::STAGE, tid, R);
    __syncthreads();
  }

  // partial result of this chunk: unnormalised O, running max, sum
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (!valid) return;
  const size_t slot = ((size_t)h * n_s + sidx) * cstride + chunk;
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

// Merge the chunks of one sampled row into its three outputs and take the
// squared errors of the masked ones.  Full: every chunk of the full pass.
// Spatial: the full pass's chunks of the frames within ks of the row's frame
// and the text chunks (a text row keeps every key: its full output).
// Temporal: the temporal pass's chunks.  A mask that keeps every key of
// every row (cover bit 1: spatial, 2: temporal) has the full output as its
// output, exactly: its merge is skipped (the temporal pass was not run).
__global__ __launch_bounds__(128)
void profile_combine(const float *__restrict__ fo, const float *__restrict__ fml, int Cf, int P,
                     const float *__restrict__ to, const float *__restrict__ tml, int Ct,
                     const int32_t *__restrict__ sample_idx, int n_s, int F, int S, int ks, int cover, int D,
                     float c, double *__restrict__ se) {
  __shared__ double red[2][128];
  const int h = blockIdx.y, s = blockIdx.x, e = threadIdx.x;
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
  const int De = e < D ? e : 0;
  double L0 = 0.0, A0 = 0.0, L1 = 0.0, A1 = 0.0;
  auto add_full = [&](int ch, float m, float l, float x) {
    const float w0 = fast_exp2((m - M0r) * c);
    L0 += (double)w0 * l;
    A0 += (double)w0 * x;
    if (in_window(ch)) {
      const float w1 = fast_exp2((m - M1r) * c);
      L1 += (double)w1 * l;
      A1 += (double)w1 * x;
    }
  };
  int ch = 0;
  for (; ch + kB <= Cf; ch += kB) {
    float m[kB], l[kB], x[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      m[u] = fml[(rf + ch + u) * 2];
      l[u] = fml[(rf + ch + u) * 2 + 1];
      x[u] = fo[(rf + ch + u) * D + De];
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) add_full(ch + u, m[u], l[u], x[u]);
  }
  for (; ch < Cf; ++ch) add_full(ch, fml[(rf + ch) * 2], fml[(rf + ch) * 2 + 1], fo[(rf + ch) * D + De]);
  double out[3];
  out[0] = L0 > 0.0 ? A0 / L0 : 0.0;
  out[1] = L1 > 0.0 ? A1 / L1 : 0.0;
  if (cover & 4) {
    out[2] = out[0];
  } else {
    float M = -INFINITY;
    for (int ch = 0; ch < Ct; ++ch) M = fmaxf(M, tml[(rt + ch) * 2]);
    const float Mr = M == -INFINITY ? 0.f : M;
    double L = 0.0, acc = 0.0;
    auto add = [&](float m, float l, float x) {
      const float w = fast_exp2((m - Mr) * c);
      L += (double)w * l;
      acc += (double)w * x;
    };
    int ct = 0;
    for (; ct + kB <= Ct; ct += kB) {
      float m[kB], l[kB], x[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        m[u] = tml[(rt + ct + u) * 2];
        l[u] = tml[(rt + ct + u) * 2 + 1];
        x[u] = to[(rt + ct + u) * D + De];
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) add(m[u], l[u], x[u]);
    }
    for (; ct < Ct; ++ct) add(tml[(rt + ct) * 2], tml[(rt + ct) * 2 + 1], to[(rt + ct) * D + De]);
    out[2] = L > 0.0 ? acc / L : 0.0;
  }
  const double ds = out[1] - out[0], dt = out[2] - out[0];
  red[0][e] = e < D ? ds * ds : 0.0;
  red[1][e] = e < D ? dt * dt : 0.0;
  __syncthreads();
  for (int off = 64; off > 0; off >>= 1) {
    if (e < off) {
      red[0][e] += red[0][e + off];
      red[1][e] += red[1][e + off];
    }
    __syncthreads();
  }
  if (e == 0) {
    se[((size_t)h * n_s + s) * 2] = red[0][0];
    se[((size_t)h * n_s + s) * 2 + 1] = red[1][0];
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
  return carve(nullptr, dm, n_s, profile_grid_full(dm, n_s).nchunks, profile_grid(dm, n_s).nchunks).bytes;
}

hipError_t launch_profile_mfma(const Dims &dm, const void *Q, const void *K, const void *V,
                               const int32_t *sample_idx, int n_s, int ks, int wt, float scale, int32_t *labels,
                               float *mse, void *ws, hipStream_t st) {
  const float c = scale * kLog2e;
  const ProfileGrid g = profile_grid(dm, n_s);       // temporal pass
  const FrameGrid gf = profile_grid_full(dm, n_s);   // full pass
  const Parts p = carve(ws, dm, n_s, gf.nchunks, g.nchunks);
  const int nkb = (dm.N + BK - 1) / BK;
  // A mask that keeps every key of every row: the spatial one when every
  // frame lies within ks of every other (ks >= F - 1), the temporal one when
  // the window of position 0 reaches the last video key and that of position
  // S - 1 the first (wt >= (S - 1) * F); text rows and keys are kept anyway.
  const int cover = ((ks >= dm.F - 1) ? 2 : 0) | (((long long)wt >= (long long)(dm.S - 1) * dm.F) ? 4 : 0);
  hipLaunchKernelGGL(profile_order, dim3((n_s + 255) / 256), dim3(256), 0, st, sample_idx, n_s, dm.F, dm.S,
                     p.ord_t);
  // key-tiled V^T of V in its own token order, every frame from a new tile
  const hipError_t ev = launch_layout_vt(dm, V, p.vt, nullptr, st, true);
  if (ev != hipSuccess) return ev;
  const dim3 gridf(gf.nqg * gf.nchunks * dm.H), grid(g.nqg, g.nchunks, dm.H);
#define SVG_PROFILE_PASSES(DD)                                                                                   \
  hipLaunchKernelGGL((profile_full_vt<DD>), gridf, dim3(FNT), 0, st, (const bf16_t *)Q, (const bf16_t *)K, p.vt, \
                     sample_idx, n_s, dm.F, dm.S, dm.T, gf.nqg, gf.nbf, gf.nbt, gf.tpp, gf.P, gf.nchunks, c, p.fo, \
                     p.fml);                                                                                     \
  if (!(cover & 4))                                                                                             \
    hipLaunchKernelGGL((profile_temporal_mfma<DD>), grid, dim3(PNT), 0, st, (const bf16_t *)Q, (const bf16_t *)K, \
                       (const bf16_t *)V, sample_idx, p.ord_t, n_s, dm.F, dm.S, dm.N, wt, nkb, g.tiles_per_chunk,  \
                       g.nchunks, c, p.to, p.tml)
  if (dm.d == 128) {
    SVG_PROFILE_PASSES(128);
  } else {
    SVG_PROFILE_PASSES(64);
  }
#undef SVG_PROFILE_PASSES
  hipLaunchKernelGGL(profile_combine, dim3(n_s, dm.H), dim3(128), 0, st, p.fo, p.fml, gf.nchunks, gf.P, p.to, p.tml,
                     g.nchunks, sample_idx, n_s, dm.F, dm.S, ks, cover, dm.d, c, p.se);
  hipLaunchKernelGGL(profile_label, dim3(dm.H), dim3(256), 0, st, p.se, n_s, dm.d, labels, mse);
  return hipGetLastError();
}

}  // namespace svgk
