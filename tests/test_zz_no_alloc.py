"""svg_kmeans_noalloc (scratch in the library's own device array) against
svg_kmeans (caller-owned workspace), through the C ABI.  Three calls in a
row on shrinking problems (the CogVideoX-shaped mixture keys: 8 heads,
N = 17,774, k = 256, d = 64, bf16; then 3 heads, N = 3,000, k = 16, d = 128,
bf16; then 2 heads, N = 1,000, k = 7, d = 64, fp32): assignments, sizes and
float64 centroids equal the workspace entry's bit for bit (the same kernels
on the same inputs), so each call is unaffected by what the previous one
left in the shared array."""

import ctypes

import numpy as np
import pytest
import torch

from _helpers import to_dev, ints
from synth import SVG2_COG
from synth.generators import mixture_qkv, random_qkv

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def kmeans_noalloc(x, k, iters, init):
    """The entry point through ctypes; outputs pre-filled with garbage."""
    H, N, d = x.shape
    dev = x.device
    assign = torch.full((H, N), -7, dtype=torch.int32, device=dev)
    cent = torch.full((H, k, d), float("nan"), dtype=torch.float64, device=dev)
    sizes = torch.full((H, k), -7, dtype=torch.int32, device=dev)
    dm = svg.svg_dims(1, N, 0, H, d)
    dt = svg.SVG_BF16 if x.dtype == torch.bfloat16 else svg.SVG_F32
    st = svg.lib().svg_kmeans_noalloc(ctypes.byref(dm), dt, ptr(x), k, iters, ptr(init), ptr(assign), ptr(cent),
                                      ptr(sizes), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == svg.SVG_OK, svg.last_error()
    return assign, cent, sizes


def small_mixture(H, N, d, k, seed, dtype):
    rng = np.random.default_rng(seed)
    comp = rng.integers(0, k, size=(H, N))
    comp[:, :k] = np.arange(k)
    means = rng.standard_normal((H, k, d)).astype(np.float32) * 4
    x32 = np.take_along_axis(means, comp[:, :, None], axis=1) + \
        0.5 * rng.standard_normal((H, N, d)).astype(np.float32)
    from synth.generators import f32_to_bf16_bits
    x = f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    init = np.stack([[np.flatnonzero(comp[h] == j)[0] for j in range(k)] for h in range(H)]).astype(np.int32)
    return to_dev(x, dtype), ints(init)


def test_kmeans_noalloc_matches_workspace_entry():
    g = mixture_qkv(SVG2_COG)
    x1, i1 = to_dev(g["k"], "bf16"), ints(g["init_k"])
    x2, i2 = small_mixture(3, 3000, 128, 16, 11, "bf16")
    x3, i3 = small_mixture(2, 1000, 64, 7, 12, "f32")
    cases = [(x1, SVG2_COG.kk, SVG2_COG.iters, i1), (x2, 16, 4, i2), (x3, 7, 3, i3)]
    got = [kmeans_noalloc(x, k, it, init) for x, k, it, init in cases]     # back to back on one array
    torch.cuda.synchronize()
    for (x, k, it, init), (a, c, s) in zip(cases, got):
        ra, rc, rs = svg.svg_kmeans(x, k, it, init)
        torch.cuda.synchronize()
        assert torch.equal(a, ra), (x.shape, k)
        assert torch.equal(s, rs), (x.shape, k)
        assert torch.equal(c, rc), (x.shape, k)
        assert int(s.sum()) == x.shape[0] * x.shape[1]
