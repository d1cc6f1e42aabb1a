// Online head profiling on bf16 inputs with MFMA (gfx950).
//
// Same computation as the vector profiler: for each sampled row, the full,
// spatial-masked and temporal-masked attention outputs, each normalised
// over its own kept keys with its own maximum.  Then per-head MSEs of the
// masked outputs against the full one, and the label (ties -> spatial).
//
// Layout: a work-group gathers 128 sampled rows (4 waves x 32).  It walks one
// chunk of the N keys in 64-key tiles, with the S^T = K Q^T / O^T += V^T P^T
// machinery of attn_core.h.  Each lane owns one sampled row.  Three passes
// (full, spatial, temporal) each keep one online-softmax state, so a wave
// holds one output accumulator and stays at two waves per SIMD.  The masks
// are evaluated per score from the key index.  A tile with a frame boundary
// inside needs one comparison, not a division.  The spatial pass visits
// only the key tiles its samples' frame windows and the text keys can
// reach.  Chunks are merged afterwards (flash-decoding style), and the
// squared errors are summed in fp64 in a fixed order.
#include "attn_core.h"

namespace svgk {
namespace {

using namespace core;

constexpr int PNW = 4;
constexpr int PNT = PNW * 64;
constexpr int PQ = PNW * 32;

struct ProfileGrid { int nqg, nchunks, tiles_per_chunk; };

ProfileGrid profile_grid(const Dims &dm, int n_s) {
  const int nkb = (dm.N + BK - 1) / BK;
  const int nqg = (n_s + PQ - 1) / PQ;
  int c = (1024 + dm.H * nqg - 1) / (dm.H * nqg);
  c = max(1, min(c, max(1, nkb / 4)));
  const int tpc = (nkb + c - 1) / c;
  return ProfileGrid{nqg, (nkb + tpc - 1) / tpc, tpc};
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct Parts {
  float *o;    // [H][n_s][C][3][D]
  float *ml;   // [H][n_s][C][3][2]
  double *se;  // [H][n_s][2]
};

Parts carve(void *ws, const Dims &dm, int n_s, const ProfileGrid &g) {
  char *p = (char *)ws;
  const size_t no = (size_t)dm.H * n_s * g.nchunks * 3 * dm.d * sizeof(float);
  const size_t nml = (size_t)dm.H * n_s * g.nchunks * 3 * 2 * sizeof(float);
  Parts r;
  r.o = (float *)p;
  r.ml = (float *)(p + align256(no));
  r.se = (double *)(p + align256(no) + align256(nml));
  return r;
}

// Frame of key `key` given the tile's first frame f0 and the next frame's
// first key jb (a 64-key tile spans at most two frames when S >= 64).
__device__ __forceinline__ int key_frame(int key, int f0, int jb, int S, bool wide) {
  return wide ? f0 + (key >= jb) : key / S;
}

// One pass of masked attention for the work-group's 128 sampled rows over
// one chunk of key tiles.  KIND 0 = no mask (full), 1 = spatial,
// 2 = temporal.  The spatial pass visits only the tiles that the samples'
// frame windows (and the text keys) can reach.
template <int D, int KIND>
__global__ __launch_bounds__(PNT, 2)
void profile_pass_mfma(const bf16_t *__restrict__ Q, const bf16_t *__restrict__ K, const bf16_t *__restrict__ V,
                       const int32_t *__restrict__ sample_idx, int n_s, int F, int S, int N, int ks, int wt,
                       int nkb, int tpc, int nchunks, float c, float *__restrict__ part_o,
                       float *__restrict__ part_ml) {
  using C = Tile<D, PNT>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  __shared__ int frange[2];
  const int h = blockIdx.z, chunk = blockIdx.y, qg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const size_t hoff = (size_t)h * N * D;
  const bf16_t *Kh = K + hoff, *Vh = V + hoff;

  const int sidx = qg * PQ + wave * 32 + l32;
  const bool valid = sidx < n_s;
  const int i = valid ? sample_idx[sidx] : 0;
  const int FS = F * S;
  const bool text_i = i >= FS;
  const int fi = text_i ? 0 : i / S;
  const int pi = text_i ? 0 : i - fi * S;
  const long long tlo = (long long)pi * F - wt, thi = (long long)pi * F + F - 1 + wt;

  // tiles this pass visits: [t0, t1) of the chunk, and for the spatial pass
  // only the video tiles [va, vb] and the text tiles [tb, nkb)
  int t0 = chunk * tpc, t1 = min(nkb, t0 + tpc);
  int va = 0, vb = nkb - 1, tb = nkb;
  if (KIND == 1) {
    if (tid == 0) {
      frange[0] = F;
      frange[1] = -1;
    }
    __syncthreads();
    if (valid) {
      if (text_i) {
        atomicMin(&frange[0], 0);
        atomicMax(&frange[1], F - 1);
      } else {
        atomicMin(&frange[0], fi);
        atomicMax(&frange[1], fi);
      }
    }
    __syncthreads();
    const int f_lo = max(0, frange[0] - ks), f_hi = min(F - 1, frange[1] + ks);
    if (frange[1] < 0) {
      va = 1;
      vb = 0;  // no valid sample: no video tiles
    } else {
      va = (f_lo * S) / BK;
      vb = ((f_hi + 1) * S - 1) / BK;
    }
    tb = FS / BK;  // first tile holding a text key (== nkb when T == 0 and FS % BK == 0)
    if (FS >= N) tb = nkb;
  }
  auto visit = [&](int t) { return KIND != 1 || (t >= va && t <= vb) || t >= tb; };
  auto next_from = [&](int t) {
    while (t < t1 && !visit(t)) ++t;
    return t;
  };

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
  int t = next_from(t0);
  if (t < t1) {
    load_tile<D, PNT>(Kh, Vh, tid, rows_of(t), R);
    store_tile<D, PNT>(smem, tid, R);
  }
  __syncthreads();
  for (int it = 0; t < t1; ++it) {
    const int tn = next_from(t + 1);
    const bool more = tn < t1;
    if (more) load_tile<D, PNT>(Kh, Vh, tid, rows_of(tn), R);
    const char *Ks = smem + (it & 1) * C::STAGE;
    const char *Vs = Ks + C::KBYTES;

    f32x16 s0, s1;
    qk_tile<D, PNT>(Ks, qf, l32, hi, s0, s1);
    const int kbase = t * BK;
    if (kbase + BK > N) mask_tail(s0, s1, N - kbase, hi);
    if (KIND != 0 && !text_i) {
      const int f0 = kbase < FS ? kbase / S : F;
      const int jb = (f0 + 1) * S;
      const bool wide = S >= BK;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kbase + acc_key(b, r, hi);
          if (key >= FS) continue;  // text keys are always kept
          const int fk = key_frame(key, f0, jb, S, wide);
          bool keep;
          if (KIND == 1) {
            keep = abs(fk - fi) <= ks;
          } else {
            const long long rk = (long long)(key - fk * S) * F + fk;
            keep = rk >= tlo && rk <= thi;
          }
          if (!keep) {
            if (b == 0) s0[r] = -INFINITY; else s1[r] = -INFINITY;
          }
        }
      }
    }
    bf16x8 pb[4];
    const float alpha = softmax_step(s0, s1, c, m_run, l_run, pb);
    rescale<D>(o, alpha);
    pv_tile<D, PNT>(Vs, pb, l32, hi, o);

    if (more) store_tile<D, PNT>(smem + ((it + 1) & 1) * C::STAGE, tid, R);
    __syncthreads();
    t = tn;
  }

  // partial result of this chunk: unnormalised O, running max, sum
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (!valid) return;
  const size_t slot = (((size_t)h * n_s + sidx) * nchunks + chunk) * 3 + KIND;
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

// Merge the chunks of one sampled row; squared errors of the masked outputs.
__global__ __launch_bounds__(128)
void profile_combine(const float *__restrict__ part_o, const float *__restrict__ part_ml, int n_s, int nchunks,
                     int D, float c, double *__restrict__ se) {
  __shared__ double red[2][128];
  const int h = blockIdx.y, s = blockIdx.x, e = threadIdx.x;
  double out[3] = {0.0, 0.0, 0.0};
  for (int m = 0; m < 3; ++m) {
    float M = -INFINITY;
    for (int ch = 0; ch < nchunks; ++ch)
      M = fmaxf(M, part_ml[((((size_t)h * n_s + s) * nchunks + ch) * 3 + m) * 2]);
    const float Mr = M == -INFINITY ? 0.f : M;
    double L = 0.0, acc = 0.0;
    for (int ch = 0; ch < nchunks; ++ch) {
      const size_t slot = (((size_t)h * n_s + s) * nchunks + ch) * 3 + m;
      const float w = fast_exp2((part_ml[slot * 2] - Mr) * c);
      L += (double)w * part_ml[slot * 2 + 1];
      if (e < D) acc += (double)w * part_o[slot * D + e];
    }
    out[m] = L > 0.0 ? acc / L : 0.0;
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
  const ProfileGrid g = profile_grid(dm, n_s);
  return align256((size_t)dm.H * n_s * g.nchunks * 3 * dm.d * sizeof(float)) +
         align256((size_t)dm.H * n_s * g.nchunks * 3 * 2 * sizeof(float)) +
         align256((size_t)dm.H * n_s * 2 * sizeof(double));
}

hipError_t launch_profile_mfma(const Dims &dm, const void *Q, const void *K, const void *V,
                               const int32_t *sample_idx, int n_s, int ks, int wt, float scale, int32_t *labels,
                               float *mse, void *ws, hipStream_t st) {
  const float c = scale * kLog2e;
  const ProfileGrid g = profile_grid(dm, n_s);
  const Parts p = carve(ws, dm, n_s, g);
  const int nkb = (dm.N + BK - 1) / BK;
  const dim3 grid(g.nqg, g.nchunks, dm.H);
#define SVG_PROFILE_PASS(DD, KK)                                                                            \
  hipLaunchKernelGGL((profile_pass_mfma<DD, KK>), grid, dim3(PNT), 0, st, (const bf16_t *)Q, (const bf16_t *)K, \
                     (const bf16_t *)V, sample_idx, n_s, dm.F, dm.S, dm.N, ks, wt, nkb, g.tiles_per_chunk,        \
                     g.nchunks, c, p.o, p.ml)
  if (dm.d == 128) {
    SVG_PROFILE_PASS(128, 0);
    SVG_PROFILE_PASS(128, 1);
    SVG_PROFILE_PASS(128, 2);
  } else {
    SVG_PROFILE_PASS(64, 0);
    SVG_PROFILE_PASS(64, 1);
    SVG_PROFILE_PASS(64, 2);
  }
#undef SVG_PROFILE_PASS
  hipLaunchKernelGGL(profile_combine, dim3(n_s, dm.H), dim3(128), 0, st, p.o, p.ml, n_s, g.nchunks, dm.d, c, p.se);
  hipLaunchKernelGGL(profile_label, dim3(dm.H), dim3(256), 0, st, p.se, n_s, dm.d, labels, mse);
  return hipGetLastError();
}

}  // namespace svgk
