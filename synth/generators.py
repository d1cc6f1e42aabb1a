"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This module draws random numbers and converts them to the storage format the
GPU path reads (fp32, or bf16 bits rounded to nearest-even).  It holds none of
the method's arithmetic: no attention, masks, profiling, permutation or
clustering.

Head generator (additive structure).  Q, K, V ~ N(0, 1).  A spatial head adds
a * u_f to Q and K of every video token of frame f (u_f ~ N(0, I_d), one vector
per frame, the same vector for Q and K); a temporal head adds a * u_p per grid
position p; a "both" head adds both.  Text tokens and V carry no structure.
Sharing u between Q and K raises the logits of tokens in the same frame
(position) by about a^2 * d / sqrt(d), which is what makes a head spatial
(temporal) in the sense of the SVG1 abstract.

Mixture generator (semantic clusters).  Per head, Q tokens belong to one of kq
components and K tokens to one of kk components, assigned uniformly at random;
component means ~ N(0, 4 I), tokens = mean + 0.5 * N(0, I).  V ~ N(0, 1).

Blob generator (spatially coherent clusters).  Per head and side, M blob
centres uniform in the (frames, rows, cols) box of the latent grid; a video
token belongs to the blob whose centre is nearest (frame offsets weighted by
4, so blobs are flatter in time than in space); text tokens belong to one of
two more components.  Means ~ N(0, 4 I), tokens = mean + 0.5 * N(0, I).  A
later denoising step s adds s * drift * N(0, I) (its own seeded draw).
V ~ N(0, 1).
"""

import numpy as np

from .configs import Workload

SPATIAL, TEMPORAL, BOTH = 0, 1, 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); return the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return ((b + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _structured_head(rng, F, S, T, d, kind, a):
    N = F * S + T
    q = rng.standard_normal((N, d), dtype=np.float32)
    k = rng.standard_normal((N, d), dtype=np.float32)
    v = rng.standard_normal((N, d), dtype=np.float32)
    if kind in (SPATIAL, BOTH):
        u = rng.standard_normal((F, d), dtype=np.float32) * np.float32(a)
        add = np.repeat(u, S, axis=0)              # token f*S+p gets u[f]
        q[:F * S] += add
        k[:F * S] += add
    if kind in (TEMPORAL, BOTH):
        u = rng.standard_normal((S, d), dtype=np.float32) * np.float32(a)
        add = np.tile(u, (F, 1))                   # token f*S+p gets u[p]
        q[:F * S] += add
        k[:F * S] += add
    return q, k, v


def head_kinds_and_scales(w: Workload, seed: int):
    """Per-head generator kind and structure scale for each workload."""
    if w.name in ("tiny", "smoke_bf16"):
        return [SPATIAL, TEMPORAL], [w.structure_scale] * 2
    if w.name == "small_frames":
        return [SPATIAL, TEMPORAL] * (w.H // 2), [w.structure_scale] * w.H
    if w.name == "cogvideox_shape":
        h2 = w.H // 2
        return [SPATIAL] * h2 + [TEMPORAL] * (w.H - h2), [w.structure_scale] * w.H
    if w.name == "hunyuan_shape":
        rng = np.random.default_rng(seed + 777)
        kinds = [int(x) for x in rng.integers(0, 2, size=w.H)]
        return kinds, [w.structure_scale] * w.H
    if w.name == "hunyuan_layer":
        kinds = [h % 3 for h in range(w.H)]
        scales = [0.5 + 2.5 * (h // 3) / 7.0 for h in range(w.H)]
        return kinds, scales
    raise ValueError(f"no structured-head generator for workload {w.name}")


def structured_qkv(w: Workload, seed: int = None, heads=None):
    """Q, K, V as float32 [H][N][d] (already rounded through bf16 for bf16
    workloads) plus the bf16 bit patterns when the workload is bf16.

    Returns dict(q, k, v, kinds, scales[, q_bits, k_bits, v_bits]).
    ``heads`` restricts generation to a subset of heads (the per-head streams
    are independent, so a subset equals the same heads of the full draw).
    """
    seed = w.seed if seed is None else seed
    kinds, scales = head_kinds_and_scales(w, seed)
    hs = list(range(w.H)) if heads is None else list(heads)
    out_dtype = np.uint16 if w.dtype == "bf16" else np.float32
    Q = np.empty((len(hs), w.N, w.d), dtype=out_dtype)
    K = np.empty_like(Q)
    V = np.empty_like(Q)
    for o, h in enumerate(hs):
        rng = np.random.default_rng([seed, h])
        q, k, v = _structured_head(rng, w.F, w.S, w.T, w.d, kinds[h], scales[h])
        if w.dtype == "bf16":
            Q[o], K[o], V[o] = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        else:
            Q[o], K[o], V[o] = q, k, v
    return dict(q=Q, k=K, v=V, kinds=[kinds[h] for h in hs],
                scales=[scales[h] for h in hs], heads=hs, dtype=w.dtype)


def sample_rows(w: Workload, seed: int = None) -> np.ndarray:
    """Profiling sample: n_s query rows drawn uniformly without replacement from
    [0, N) (text included), sorted, shared by all heads.  int32."""
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng([seed, 99991])
    idx = rng.choice(w.N, size=w.n_samples, replace=False)
    return np.sort(idx).astype(np.int32)


def generator_labels(w: Workload, seed: int = None) -> np.ndarray:
    """Labels known by construction (0 spatial, 1 temporal) where the generator
    fixes them; -1 for heads generated with both structures."""
    kinds, _ = head_kinds_and_scales(w, w.seed if seed is None else seed)
    return np.array([k if k in (SPATIAL, TEMPORAL) else -1 for k in kinds], dtype=np.int32)


def mixture_qkv(w: Workload, seed: int = None):
    """Gaussian-mixture Q and K per head (kq and kk components), V ~ N(0,1).

    Returns dict(q, k, v) as bf16 bits [H][N][d] (uint16) plus the generating
    component of each token (comp_q, comp_k: int32 [H][N]) and the k-means
    initialisation (init_q [H][kq], init_k [H][kk]): one seeded member token of
    each component, in component order.
    """
    seed = w.seed if seed is None else seed
    N, d, H = w.N, w.d, w.H
    Q = np.empty((H, N, d), dtype=np.uint16)
    K = np.empty_like(Q)
    V = np.empty_like(Q)
    comp_q = np.empty((H, N), dtype=np.int32)
    comp_k = np.empty((H, N), dtype=np.int32)
    init_q = np.empty((H, w.kq), dtype=np.int32)
    init_k = np.empty((H, w.kk), dtype=np.int32)
    for h in range(H):
        rng = np.random.default_rng([seed, h, 5])
        for side, kc, X, comp, init in ((0, w.kq, Q, comp_q, init_q), (1, w.kk, K, comp_k, init_k)):
            while True:
                c = rng.integers(0, kc, size=N)
                counts = np.bincount(c, minlength=kc)
                if counts.min() > 0:
                    break
            means = rng.standard_normal((kc, d), dtype=np.float32) * np.float32(2.0)
            x = means[c] + np.float32(0.5) * rng.standard_normal((N, d), dtype=np.float32)
            X[h] = f32_to_bf16_bits(x)
            comp[h] = c
            for j in range(kc):
                members = np.flatnonzero(c == j)
                init[h, j] = members[rng.integers(0, members.size)]
        V[h] = f32_to_bf16_bits(rng.standard_normal((N, d), dtype=np.float32))
    return dict(q=Q, k=K, v=V, comp_q=comp_q, comp_k=comp_k, init_q=init_q, init_k=init_k)


def random_qkv(H, N, d, seed, dtype="f32", scale=1.0):
    """Unstructured N(0, scale^2) tensors for edge-case tests."""
    rng = np.random.default_rng([seed, 31337])
    x = rng.standard_normal((3, H, N, d), dtype=np.float32) * np.float32(scale)
    if dtype == "bf16":
        x = f32_to_bf16_bits(x)
    return x[0], x[1], x[2]


def blob_qkv(w: Workload, seed: int = None, step: int = 0, heads=None):
    """Blob-structured Q and K per head (w.blobs_q / w.blobs_k components),
    V ~ N(0, 1).  Returns dict(q, k, v) as bf16 bits [H][N][d] (uint16) and
    the generating blob of each token (blob_q, blob_k: int32 [H][N], text
    components numbered after the blobs).  step > 0 perturbs Q and K by
    step * w.drift * N(0, I) from a draw of its own (V is kept)."""
    seed = w.seed if seed is None else seed
    heads = range(w.H) if heads is None else heads
    rows, cols = w.grid
    assert rows * cols == w.S
    N, d = w.N, w.d
    f, y, x = np.meshgrid(np.arange(w.F), np.arange(rows), np.arange(cols), indexing="ij")
    pos = np.stack([4.0 * f.ravel(), y.ravel(), x.ravel()], axis=1)
    out = {n: np.empty((len(heads), N, d), dtype=np.uint16) for n in "qkv"}
    blob = {n: np.empty((len(heads), N), dtype=np.int32) for n in "qk"}
    for i, h in enumerate(heads):
        rng = np.random.default_rng([seed, h, 7])
        for side, m in (("q", w.blobs_q), ("k", w.blobs_k)):
            centres = rng.random((m, 3)) * np.array([4.0 * w.F, rows, cols])
            d2 = ((pos[:, None, :] - centres[None, :, :]) ** 2).sum(axis=2)
            comp = np.empty(N, dtype=np.int64)
            comp[:w.F * w.S] = d2.argmin(axis=1)
            comp[w.F * w.S:] = m + rng.integers(0, 2, size=w.T)
            means = rng.standard_normal((m + 2, d), dtype=np.float32) * np.float32(2.0)
            val = means[comp] + np.float32(0.5) * rng.standard_normal((N, d), dtype=np.float32)
            if step > 0:
                srng = np.random.default_rng([seed, h, 7, step, 0 if side == "q" else 1])
                val = val + np.float32(step * w.drift) * srng.standard_normal((N, d), dtype=np.float32)
            out[side][i] = f32_to_bf16_bits(val)
            blob[side][i] = comp
        out["v"][i] = f32_to_bf16_bits(rng.standard_normal((N, d), dtype=np.float32))
    return dict(q=out["q"], k=out["k"], v=out["v"], blob_q=blob["q"], blob_k=blob["k"])
