"""GPU parity of the SVG1 path against the float64 oracle.

Bit-exact: block bitmaps, CSR lists, layout permutations, labels.
Toleranced: attention outputs (bf16: max-abs 2e-2, rel-L2 1e-2; fp32: max-abs
1e-4, rel-L2 1e-5).  Every input is seeded and synthetic (synth/).
"""

import json
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from _helpers import (to_dev, to_host_bits, to_f64, ints, check_close, BF16_MAX_ABS, BF16_REL_L2,
                      F32_MAX_ABS, F32_REL_L2)
from oracle import masks, layout, attention, profile
from oracle.numerics import as_f64
from synth import TINY, COG, SMALL_FRAMES, HUNYUAN, HUNYUAN_LAYER
from synth.generators import structured_qkv, sample_rows, generator_labels, random_qkv

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def sync():
    torch.cuda.synchronize()


_cache = {}


def inputs(w):
    if w.name not in _cache:
        g = structured_qkv(w)
        _cache[w.name] = g
    return _cache[w.name]


def oracle_bitmaps(w, labels, ranges=False):
    out = {}
    for lab in set(int(x) for x in labels):
        f = masks.block_bitmap_ranges if ranges else masks.block_bitmap
        out[lab] = f(lab, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
    return np.stack([out[int(l)] for l in labels])


# ----------------------------------------------------------------------------
# layout permutation

@pytest.mark.parametrize("w", [TINY, COG, HUNYUAN], ids=lambda w: w.name)
def test_layout_permute_bit_exact(w):
    g = inputs(w)
    labels = np.array([1 - (h % 2) for h in range(w.H)], dtype=np.int32)
    x = to_dev(g["q"], w.dtype)
    y = svg.svg_layout_permute(x, w.F, w.S, w.T, ints(labels))
    sync()
    yh = to_host_bits(y)
    # compare against the oracle on 2 heads (one of each label) at full size
    for h in (0, 1):
        ref = layout.permute(g["q"][h:h + 1], w.F, w.S, w.T, labels[h:h + 1])
        np.testing.assert_array_equal(yh[h], ref[0])
    z = svg.svg_layout_unpermute(y, w.F, w.S, w.T, ints(labels))
    sync()
    np.testing.assert_array_equal(to_host_bits(z), g["q"])


def test_layout_all_heads_when_labels_null():
    F, S, T, H, d = 5, 7, 3, 2, 64
    x = torch.arange(H * (F * S + T) * d, dtype=torch.float32, device="cuda:0").reshape(H, F * S + T, d)
    y = svg.svg_layout_permute(x, F, S, T, None)
    sync()
    ref = layout.permute(x.cpu().numpy(), F, S, T, [1, 1])
    np.testing.assert_array_equal(y.cpu().numpy(), ref)


# ----------------------------------------------------------------------------
# block masks and lists

@pytest.mark.parametrize("w", [TINY, COG], ids=lambda w: w.name)
def test_block_mask_bit_exact_elementwise(w):
    labels = np.array([h % 2 for h in range(w.H)], dtype=np.int32)
    bm = svg.svg_build_block_mask(ints(labels), w.F, w.S, w.T, w.H, w.d, w.ks, w.wt, w.bq, w.bk)
    sync()
    np.testing.assert_array_equal(bm.cpu().numpy(), oracle_bitmaps(w, labels))


def test_block_mask_hunyuan_shape():
    w = HUNYUAN
    labels = np.array([0, 1, 1, 0], dtype=np.int32)
    bm = svg.svg_build_block_mask(ints(labels), w.F, w.S, w.T, 4, w.d, w.ks, w.wt, w.bq, w.bk)
    sync()
    got = bm.cpu().numpy()
    ref = oracle_bitmaps(w, labels, ranges=True)
    np.testing.assert_array_equal(got, ref)
    rows = [0, 1, 27, 28, 500, 927, 928, 929, 930]
    for h, lab in enumerate(labels):
        e = masks.block_bitmap(int(lab), w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk, qblocks=rows)
        np.testing.assert_array_equal(got[h][rows], e)


@pytest.mark.parametrize("shape", [(3, 11, 5, 1, 4, 64, 64), (7, 9, 0, 0, 0, 16, 16), (2, 70, 33, 1, 60, 128, 64),
                                   (1, 40, 100, 0, 3, 64, 64)])
def test_block_mask_ragged_shapes(shape):
    F, S, T, ks, wt, bq, bk = shape
    labels = np.array([0, 1], dtype=np.int32)
    bm = svg.svg_build_block_mask(ints(labels), F, S, T, 2, 64, ks, wt, bq, bk)
    sync()
    for h in range(2):
        ref = masks.block_bitmap(int(labels[h]), F, S, T, ks, wt, bq, bk)
        np.testing.assert_array_equal(bm.cpu().numpy()[h], ref)


@pytest.mark.parametrize("rows,nkb,p", [(1, 1, 1.0), (37, 5, 0.5), (300, 1861, 0.3), (0, 4, 0.5), (64, 200, 0.0)])
def test_compact_bit_exact(rows, nkb, p):
    rng = np.random.default_rng(rows * 7 + nkb)
    bm = (rng.random((rows, nkb)) < p).astype(np.uint8)
    t = torch.from_numpy(bm).to("cuda:0") if rows else torch.zeros(0, nkb, dtype=torch.uint8, device="cuda:0")
    ptr, idx = svg.svg_compact_block_mask(t)
    sync()
    rp, ki = masks.compact(bm) if rows else (np.zeros(1, np.int32), np.zeros(0, np.int32))
    np.testing.assert_array_equal(ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(idx.cpu().numpy()[:rp[-1]], ki)


# ----------------------------------------------------------------------------
# attention

def run_sparse(w, g, labels, scale=-1.0):
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    lab = ints(labels)
    qp, kp, vp = (svg.svg_layout_permute(t, w.F, w.S, w.T, lab) for t in (q, k, v))
    bm = svg.svg_build_block_mask(lab, w.F, w.S, w.T, w.H, w.d, w.ks, w.wt, w.bq, w.bk)
    op = svg.svg_block_sparse_attn(qp, kp, vp, bm, w.F, w.S, w.T, w.bq, w.bk, scale)
    o = svg.svg_layout_unpermute(op, w.F, w.S, w.T, lab)
    sync()
    return o, op, bm


def oracle_sparse_head(w, g, h, label, qblocks=None):
    """Oracle output of head h in ORIGINAL order for the given q-blocks of the
    executing layout; returns {qb: (original rows, O rows)}."""
    q, k, v = (as_f64(g[x][h], w.dtype) for x in "qkv")
    xs = layout.permute(np.stack([q, k, v]), w.F, w.S, w.T, [label] * 3)
    bm = masks.block_bitmap_ranges(label, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
    parts = attention.block_sparse_attention(xs[0], xs[1], xs[2], bm, w.bq, w.bk, qblocks=qblocks)
    inv = masks.executing_to_original(label, w.F, w.S, w.T)
    return {qb: (inv[qb * w.bq:qb * w.bq + o.shape[0]], o) for qb, o in parts.items()}


def test_attention_tiny_f32_end_to_end():
    w = TINY
    g = inputs(w)
    labels = generator_labels(w)
    o, _, _ = run_sparse(w, g, labels)
    got = o.double().cpu().numpy()
    for h in range(w.H):
        ref = np.zeros((w.N, w.d))
        for qb, (rows, orow) in oracle_sparse_head(w, g, h, int(labels[h])).items():
            ref[rows] = orow
        check_close(got[h], ref, F32_MAX_ABS, F32_REL_L2, f"tiny head {h}")


def test_attention_cogvideox_bf16_full():
    w = COG
    g = inputs(w)
    labels = generator_labels(w)
    o, _, _ = run_sparse(w, g, labels)
    got = to_f64(o)
    for h in range(w.H):
        ref = np.zeros((w.N, w.d))
        for qb, (rows, orow) in oracle_sparse_head(w, g, h, int(labels[h])).items():
            ref[rows] = orow
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"cog head {h}")


def test_attention_cogvideox_bf16_rowmajor_kernel_full():
    """The row-major MFMA kernel (svg_block_sparse_attn_csr with no
    workspace) at the CogVideoX shape, every row of every head."""
    w = COG
    g = inputs(w)
    labels = generator_labels(w)
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    lab = ints(labels)
    qp, kp, vp = (svg.svg_layout_permute(t, w.F, w.S, w.T, lab) for t in (q, k, v))
    bm = svg.svg_build_block_mask(lab, w.F, w.S, w.T, w.H, w.d, w.ks, w.wt, w.bq, w.bk)
    row_ptr, kv_idx = svg.svg_compact_block_mask(bm)
    op = svg.svg_block_sparse_attn_csr(qp, kp, vp, row_ptr, kv_idx, w.F, w.S, w.T, w.bq, w.bk,
                                       rowmajor_kernel=True)
    o_vt = svg.svg_block_sparse_attn_csr(qp, kp, vp, row_ptr, kv_idx, w.F, w.S, w.T, w.bq, w.bk)
    o = svg.svg_layout_unpermute(op, w.F, w.S, w.T, lab)
    sync()
    got = to_f64(o)
    for h in range(w.H):
        ref = np.zeros((w.N, w.d))
        for qb, (rows, orow) in oracle_sparse_head(w, g, h, int(labels[h])).items():
            ref[rows] = orow
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"cog row-major head {h}")
    # the workspace form of the same call runs the V^T kernel: the bitmap
    # entry's output, bit for bit (same kernel, same lists)
    np.testing.assert_array_equal(to_host_bits(o_vt), to_host_bits(run_sparse(w, g, labels)[1]))


def test_dense_cogvideox_bf16_sampled_rows():
    w = COG
    g = inputs(w)
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    o = svg.svg_dense_attn(q, k, v, w.F, w.S, w.T, w.bq, w.bk)
    sync()
    got = to_f64(o)
    rows = np.r_[0:64, 8000:8064, w.N - 40:w.N]
    for h in (0, 5):
        ref = attention.dense_attention(*(as_f64(g[x][h], w.dtype) for x in "qkv"), rows=rows)
        check_close(got[h][rows], ref, BF16_MAX_ABS, BF16_REL_L2, f"dense head {h}")


def test_attention_hunyuan_sampled_qblocks():
    """Full-size HunyuanVideo shape (N = 119,056, 24 heads, d = 128, 128x64
    tiles, ~31% density) through svg_block_sparse_attn (bitmap in, V
    row-major, run on the V^T kernel); the oracle checks 32 seeded q-blocks
    of every head plus the first, frame-straddling, video/text and tail
    ones."""
    w = HUNYUAN
    g = inputs(w)
    labels = generator_labels(w)
    o, _, _ = run_sparse(w, g, labels)
    got = to_f64(o)
    rng = np.random.default_rng(123)
    vid_qb = (w.F * w.S) // w.bq
    for h in range(w.H):
        qbs = sorted(set([0, 28, vid_qb, w.nqb - 2, w.nqb - 1]) |
                     set(int(x) for x in rng.choice(w.nqb, size=32, replace=False)))
        for qb, (rows, orow) in oracle_sparse_head(w, g, h, int(labels[h]), qblocks=qbs).items():
            check_close(got[h][rows], orow, BF16_MAX_ABS, BF16_REL_L2, f"hunyuan head {h} qb {qb}")


@pytest.mark.parametrize("N,d,bq,bk,dtype", [(75, 64, 64, 64, "bf16"), (300, 128, 128, 64, "bf16"),
                                             (1, 128, 128, 64, "bf16"), (130, 64, 16, 16, "f32"),
                                             (200, 128, 64, 64, "f32"), (77, 64, 64, 64, "f32")])
def test_attention_random_bitmap_ragged(N, d, bq, bk, dtype):
    H = 2
    q, k, v = random_qkv(H, N, d, seed=N + d, dtype=dtype, scale=1.5)
    nqb, nkb = -(-N // bq), -(-N // bk)
    rng = np.random.default_rng(N)
    bm = (rng.random((H, nqb, nkb)) < 0.5).astype(np.uint8)
    bm[:, 0, :] = 0                            # a q-block with no kept tile -> zeros
    bm[0, -1, -1] = 1                          # the ragged tail tile
    o = svg.svg_block_sparse_attn(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype),
                                  torch.from_numpy(bm).cuda(), 1, N, 0, bq, bk)
    outs = [("bitmap entry", o)]
    if dtype == "bf16":   # the row-major MFMA kernel through the list entry with no workspace
        rp, ki = svg.svg_compact_block_mask(torch.from_numpy(bm).cuda())
        outs.append(("row-major kernel", svg.svg_block_sparse_attn_csr(
            to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), rp, ki, 1, N, 0, bq, bk, rowmajor_kernel=True)))
    sync()
    tol = (BF16_MAX_ABS, BF16_REL_L2) if dtype == "bf16" else (F32_MAX_ABS, F32_REL_L2)
    for name, out in outs:
        got = to_f64(out)
        for h in range(H):
            ref = attention.block_sparse_attention_full(as_f64(q[h], dtype), as_f64(k[h], dtype),
                                                        as_f64(v[h], dtype), bm[h], bq, bk)
            check_close(got[h], ref, *tol, f"{name}: random bitmap head {h}")
            if bm[h, 0].sum() == 0:
                assert np.all(got[h][:min(bq, N)] == 0.0)


def test_attention_k_zero_closed_form():
    """K = 0: each row's output is the mean of V over its q-block's kept keys."""
    w = COG
    H, N, d = 2, 600, 64
    rng = np.random.default_rng(9)
    q = rng.standard_normal((H, N, d)).astype(np.float32)
    v = rng.standard_normal((H, N, d)).astype(np.float32)
    from synth.generators import f32_to_bf16_bits
    qb_, vb_ = f32_to_bf16_bits(q), f32_to_bf16_bits(v)
    kb_ = np.zeros_like(qb_)
    nqb = nkb = -(-N // 64)
    bm = (rng.random((H, nqb, nkb)) < 0.4).astype(np.uint8)
    bm[:, :, -1] = 1
    o = svg.svg_block_sparse_attn(to_dev(qb_, "bf16"), to_dev(kb_, "bf16"), to_dev(vb_, "bf16"),
                                  torch.from_numpy(bm).cuda(), 1, N, 0, 64, 64)
    sync()
    got = to_f64(o)
    vv = as_f64(vb_, "bf16")
    for h in range(H):
        for qb in range(nqb):
            keys = [j for j in range(N) if bm[h, qb, j // 64]]
            ref = vv[h][keys].mean(axis=0)
            rows = slice(qb * 64, min(N, qb * 64 + 64))
            check_close(got[h][rows], np.tile(ref, (got[h][rows].shape[0], 1)), 1e-2, 1e-2, f"kzero {h} {qb}")


def test_attention_deterministic():
    w = COG
    g = inputs(w)
    labels = generator_labels(w)
    a = to_host_bits(run_sparse(w, g, labels)[0])
    b = to_host_bits(run_sparse(w, g, labels)[0])
    np.testing.assert_array_equal(a, b)


# ----------------------------------------------------------------------------
# profiling

@pytest.mark.parametrize("w", [TINY, COG], ids=lambda w: w.name)
def test_profile_labels_and_mse(w):
    g = inputs(w)
    si = sample_rows(w)
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    labels, mse = svg.svg_profile_heads(q, k, v, ints(si), w.F, w.S, w.T, w.ks, w.wt)
    sync()
    ol, om = profile.profile_heads(*(as_f64(g[x], w.dtype) for x in "qkv"), w.F, w.S, w.T, si, w.ks, w.wt)
    np.testing.assert_array_equal(labels.cpu().numpy(), ol)
    np.testing.assert_array_equal(labels.cpu().numpy(), generator_labels(w))
    np.testing.assert_allclose(mse.double().cpu().numpy(), om, rtol=2e-2, atol=1e-6)


def test_profile_hunyuan_layer_labels():
    """HunyuanVideo-shaped layer workload (1191 sampled rows, mixed heads):
    labels of the heads the oracle decides with a clear margin are
    bit-exact; the oracle's result is stored in tests/golden."""
    w = HUNYUAN_LAYER
    with open(os.path.join(GOLDEN, "hunyuan_layer_profile.json")) as f:
        gold = json.load(f)
    g = structured_qkv(w)
    si = sample_rows(w)
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    del g
    labels, mse = svg.svg_profile_heads(q, k, v, ints(si), w.F, w.S, w.T, w.ks, w.wt)
    sync()
    lab = labels.cpu().numpy()
    ms = mse.double().cpu().numpy()
    for hd in gold["heads"]:
        h = hd["head"]
        if not hd["ambiguous"]:
            assert lab[h] == hd["label"], (h, lab[h], hd)
        np.testing.assert_allclose(ms[h], [hd["mse_spatial"], hd["mse_temporal"]], rtol=5e-2, atol=1e-6)


def test_profile_sample_order_invariant():
    """The work-groups group samples by frame or by grid position; the labels
    and MSEs do not depend on the order of sample_idx (up to the order of the
    fp64 sums of squared errors)."""
    w = COG
    g = inputs(w)
    si = sample_rows(w)
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    la, ma = svg.svg_profile_heads(q, k, v, ints(si), w.F, w.S, w.T, w.ks, w.wt)
    shuf = np.random.default_rng(4).permutation(si).astype(np.int32)
    lb, mb = svg.svg_profile_heads(q, k, v, ints(shuf), w.F, w.S, w.T, w.ks, w.wt)
    sync()
    np.testing.assert_array_equal(la.cpu().numpy(), lb.cpu().numpy())
    np.testing.assert_allclose(ma.double().cpu().numpy(), mb.double().cpu().numpy(), rtol=1e-6, atol=0)


@pytest.mark.parametrize("d", [64, 128])
def test_profile_small_frames(d):
    """Frames shorter than a 64-key tile (S = 48: a tile spans up to three
    frames), unsorted samples with text rows.  Structured heads: labels and
    MSEs against the oracle.  Gaussian heads (every key matters, so a wrong
    masked key moves both MSEs): MSEs against the oracle."""
    from dataclasses import replace
    w = replace(SMALL_FRAMES, d=d)
    rng = np.random.default_rng(d)
    si = rng.choice(w.N, size=w.n_samples, replace=False).astype(np.int32)
    si[:3] = w.N - 1 - np.arange(3)                       # text rows
    g = structured_qkv(w)
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    labels, mse = svg.svg_profile_heads(q, k, v, ints(si), w.F, w.S, w.T, w.ks, w.wt)
    sync()
    ol, om = profile.profile_heads(*(as_f64(g[x], w.dtype) for x in "qkv"), w.F, w.S, w.T, si, w.ks, w.wt)
    np.testing.assert_array_equal(labels.cpu().numpy(), ol)
    np.testing.assert_allclose(mse.double().cpu().numpy(), om, rtol=2e-2, atol=1e-6)
    qr, kr, vr = random_qkv(w.H, w.N, d, seed=d + 1, dtype="bf16")
    _, mse = svg.svg_profile_heads(*(to_dev(x, "bf16") for x in (qr, kr, vr)), ints(si), w.F, w.S, w.T,
                                   w.ks, w.wt)
    sync()
    _, om = profile.profile_heads(*(as_f64(x, "bf16") for x in (qr, kr, vr)), w.F, w.S, w.T, si, w.ks, w.wt)
    assert om.min() > 1e-3
    np.testing.assert_allclose(mse.double().cpu().numpy(), om, rtol=2e-2, atol=1e-6)


@pytest.mark.parametrize("F,S,T,d", [(5, 200, 0, 64), (3, 128, 64, 128), (9, 70, 5, 64), (2, 1000, 130, 128)])
def test_profile_frame_chunks_ragged(F, S, T, d):
    """The full pass walks key chunks cut at frame boundaries (each frame
    padded to whole 64-key tiles) and takes the spatial outputs from them:
    frames that end mid-tile (S = 200, 70, 1000), whole tiles (S = 128), no
    text (T = 0), a one-key-short text tile (T = 130, 63 + 64 + 3), frames
    split into several parts (S = 1000).  Gaussian heads, so every key
    carries weight: MSEs against the oracle, with samples in every frame and
    in the text."""
    H = 2
    N = F * S + T
    q, k, v = random_qkv(H, N, d, seed=F * S + T + d, dtype="bf16")
    rng = np.random.default_rng(N)
    si = rng.choice(N, size=min(N, 150), replace=False).astype(np.int32)
    if T:
        si[0] = N - 1                                     # a text row
    for ks, wt in ((1 if F > 2 else 0, 3 * F), (0, S * F // 3)):   # windows that keep only some keys
        labels, mse = svg.svg_profile_heads(*(to_dev(x, "bf16") for x in (q, k, v)), ints(si), F, S, T, ks, wt)
        sync()
        ol, om = profile.profile_heads(*(as_f64(x, "bf16") for x in (q, k, v)), F, S, T, si, ks, wt)
        assert om.min() > 1e-4
        np.testing.assert_allclose(mse.double().cpu().numpy(), om, rtol=2e-2, atol=1e-6)


@pytest.mark.parametrize("ks,wt", [(1, 100), (2, 0), (0, 1350 * 13), (0, 121), (0, 122)])
def test_profile_mask_widths_against_oracle(ks, wt):
    """Masks of other widths (a temporal window that is not a multiple of F,
    an empty one, one that covers every key, and the two sides of the
    narrow-window kernel's bound: 2 w_t + F = 255 keys a row on the vector
    path, 257 on the tile pass) on unsorted samples that include text rows:
    MSEs against the oracle, and labels where the oracle's margin is clear."""
    w = COG
    g = inputs(w)
    rng = np.random.default_rng(ks * 1000 + wt)
    si = rng.choice(w.N, size=300, replace=False).astype(np.int32)
    si[:5] = w.N - 1 - np.arange(5)                       # text rows
    q, k, v = (to_dev(g[x], w.dtype) for x in "qkv")
    labels, mse = svg.svg_profile_heads(q, k, v, ints(si), w.F, w.S, w.T, ks, wt)
    sync()
    ol, om = profile.profile_heads(*(as_f64(g[x], w.dtype) for x in "qkv"), w.F, w.S, w.T, si, ks, wt)
    got = mse.double().cpu().numpy()
    np.testing.assert_allclose(got, om, rtol=2e-2, atol=1e-6)
    lab = labels.cpu().numpy()
    for h in range(w.H):
        a, b = om[h]
        if abs(a - b) > 0.05 * max(a, b):
            assert lab[h] == ol[h], (h, lab[h], ol[h], om[h])
    # Gaussian heads: every key carries weight, so a key masked wrongly on the
    # GPU moves both MSEs.  (A window that covers every key leaves nothing
    # to compare: its MSE is 0 on both sides, checked above.)
    if wt < w.F * w.S // 2:
        qr, kr, vr = random_qkv(2, w.N, w.d, seed=ks + wt, dtype="bf16")
        _, mse = svg.svg_profile_heads(*(to_dev(x, "bf16") for x in (qr, kr, vr)), ints(si), w.F, w.S, w.T,
                                       ks, wt)
        sync()
        _, om = profile.profile_heads(*(as_f64(x, "bf16") for x in (qr, kr, vr)), w.F, w.S, w.T, si, ks, wt)
        assert om.min() > 1e-4
        np.testing.assert_allclose(mse.double().cpu().numpy(), om, rtol=2e-2, atol=1e-6)
