"""Workload table for the sparse video attention path.

Five synthetic workloads stand in for the attention tensors of the video
diffusion transformers that Sparse VideoGen accelerates (the SVG1 abstract on
the arXiv listing page names CogVideoX-v1.5 and HunyuanVideo).  No model
weights, prompts or benchmark items are used: every tensor is drawn from a
seeded generator in ``synth.generators``.

Token order is frame-major video first (token (f, p) at f*S + p), then the T
text tokens.  Tensors are [H][N][d] contiguous, batch 1.

Mask parameters (``ks`` frames either side for the spatial pattern, ``wt``
tokens either side of the own-position run for the temporal pattern) follow
the readings recorded with the oracle: the CogVideoX-shaped rule (own frame
plus text; same position +/-32 tokens across frames) and a widened rule at the
HunyuanVideo shape that gives ~31% tile density.
"""

from dataclasses import dataclass, field
import math


@dataclass(frozen=True)
class Workload:
    name: str
    F: int            # frames
    S: int            # video tokens per frame
    T: int            # text tokens (after the video tokens)
    H: int            # heads
    d: int            # head dimension
    dtype: str        # "f32" or "bf16"
    bq: int           # query block (rows per tile)
    bk: int           # key block (columns per tile)
    ks: int           # spatial mask: frames either side of the query's frame
    wt: int           # temporal mask: tokens either side of the own-position run
    seed: int
    grid: tuple = (0, 0)
    n_samples: int = 0          # profiling sample size (0 = not profiled)
    structure_scale: float = 0.0
    # SVG2 (semantic permutation) parameters
    kq: int = 0
    kk: int = 0
    iters: int = 0
    top_p: float = 0.0
    # HVA-style local-window clustering: window sizes (frames, rows, cols) for
    # Q and K, blob components of the generator, per-step drift
    win_q: tuple = (0, 0, 0)
    win_k: tuple = (0, 0, 0)
    blobs_q: int = 0
    blobs_k: int = 0
    drift: float = 0.0
    notes: str = ""

    @property
    def N(self) -> int:
        return self.F * self.S + self.T

    @property
    def nqb(self) -> int:
        return -(-self.N // self.bq)

    @property
    def nkb(self) -> int:
        return -(-self.N // self.bk)


TINY = Workload(
    name="tiny", F=4, S=64, T=16, H=2, d=64, dtype="f32", bq=16, bk=16,
    ks=0, wt=32, seed=1, grid=(8, 8), n_samples=8, structure_scale=3.0,
    notes="head 0 spatial, head 1 temporal; fp32; checked against brute force")

COG = Workload(
    name="cogvideox_shape", F=13, S=1350, T=224, H=8, d=64, dtype="bf16",
    bq=64, bk=64, ks=0, wt=32, seed=2, grid=(30, 45),
    n_samples=math.ceil(0.01 * (13 * 1350 + 224)), structure_scale=2.0,
    notes="heads 0-3 spatial, 4-7 temporal")

SMALL_FRAMES = Workload(
    name="small_frames", F=8, S=48, T=40, H=4, d=64, dtype="bf16",
    bq=64, bk=64, ks=1, wt=50, seed=11, grid=(6, 8), n_samples=120,
    structure_scale=2.0,
    notes="frames shorter than a 64-key tile (a tile spans up to three "
          "frames); heads alternate spatial / temporal")

HUNYUAN = Workload(
    name="hunyuan_shape", F=33, S=3600, T=256, H=24, d=128, dtype="bf16",
    bq=128, bk=64, ks=5, wt=19800, seed=3, grid=(45, 80), n_samples=0,
    structure_scale=2.0,
    notes="labels Bernoulli(0.5) per head from the seed; attention alone")

HUNYUAN_LAYER = Workload(
    name="hunyuan_layer", F=33, S=3600, T=256, H=24, d=128, dtype="bf16",
    bq=128, bk=64, ks=5, wt=19800, seed=4, grid=(45, 80),
    n_samples=math.ceil(0.01 * (33 * 3600 + 256)),
    notes="end-to-end layer: profile -> masks -> permute -> attention -> "
          "unpermute; mixed head generators, scales 0.5-3")

SVG2_COG = Workload(
    name="svg2_cogvideox_shape", F=13, S=1350, T=224, H=8, d=64, dtype="bf16",
    bq=64, bk=64, ks=0, wt=32, seed=5, grid=(30, 45),
    kq=64, kk=256, iters=10, top_p=0.9,
    notes="Gaussian-mixture Q/K; k-means, cluster permute, top-p pairs, "
          "variable-size block-sparse attention")

HVA_COG = Workload(
    name="hva_cogvideox_shape", F=13, S=1350, T=224, H=8, d=64, dtype="bf16",
    bq=64, bk=64, ks=0, wt=32, seed=7, grid=(30, 45),
    iters=10, top_p=0.9, win_q=(4, 10, 15), win_k=(2, 6, 9), blobs_q=40, blobs_k=160, drift=0.1,
    notes="spatially coherent blob Q/K; 3D local-window clustering (36 + 1 query "
          "clusters, 175 + 1 key clusters), anchor and refresh steps, top-p pairs, "
          "varlen attention")

SMOKE_BF16 = Workload(
    name="smoke_bf16", F=4, S=256, T=32, H=2, d=128, dtype="bf16", bq=128, bk=64,
    ks=1, wt=300, seed=6, grid=(16, 16), n_samples=64, structure_scale=3.0,
    notes="head 0 spatial, head 1 temporal; the bf16 path of the HunyuanVideo layer at a small size")

WORKLOADS = {w.name: w for w in (TINY, COG, SMALL_FRAMES, HUNYUAN, HUNYUAN_LAYER, SVG2_COG, HVA_COG, SMOKE_BF16)}

# Extra mask-width points at the HunyuanVideo shape (density sweep).
# (ks, wt) pairs chosen so that the spatial and temporal tile densities match.
HUNYUAN_DENSITY_POINTS = {
    "k4": (4, 16170),
    "k5": (5, 19800),
    "cog_rule": (0, 32),
}
