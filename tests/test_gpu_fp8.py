"""GPU parity of the FP8 path against the oracle (oracle/fp8.py).

Bit-exact: the E4M3 codes and fp32 scales of both quantizers (per-row for
Q, per-64-row block of the executing layout for K).  Toleranced: the
attention output against the oracle's attention over the same dequantized Q
and K (max-abs 2e-2, rel-L2 1e-2, the bf16 bar: after the quantization the
kernel's arithmetic is the bf16 kernel's).  Inputs are seeded and synthetic.
"""

import concurrent.futures

import numpy as np
import pytest
import torch

from _helpers import to_dev, to_f64, ints, check_close, BF16_MAX_ABS, BF16_REL_L2
from oracle import fp8 as ofp8, layout, masks
from oracle.attention import dense_attention
from oracle.numerics import as_f64
from synth import HUNYUAN_LAYER
from synth.generators import random_qkv, structured_qkv, sample_rows, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def sync():
    torch.cuda.synchronize()


def bf16_tensor(H, N, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((H, N, d)).astype(np.float32) * np.float32(scale)
    x *= np.exp2(rng.integers(-8, 8, size=(H, N, 1))).astype(np.float32)    # rows of very different sizes
    x[:, 3, :] = 0.0                                                       # an all-zero row
    return f32_to_bf16_bits(x)


@pytest.mark.parametrize("N,d", [(300, 128), (1, 128), (517, 64)])
def test_quantize_rows_bit_exact(N, d):
    H = 2 if N > 3 else 1
    x = bf16_tensor(H, N, d, seed=N + d) if N > 3 else f32_to_bf16_bits(np.ones((H, N, d), np.float32))
    codes, scales = svg.svg_quantize_fp8_rows(to_dev(x, "bf16"))
    sync()
    for h in range(H):
        oc, osc = ofp8.quantize_rows(as_f64(x[h], "bf16").astype(np.float32))
        np.testing.assert_array_equal(codes[h].cpu().numpy(), oc)
        np.testing.assert_array_equal(scales[h].cpu().numpy(), osc)


@pytest.mark.parametrize("F,S,T,d,labels", [(5, 70, 13, 128, [0, 1]), (3, 100, 0, 128, None),
                                            (4, 33, 29, 64, [1, 0])])
def test_layout_permute_fp8_bit_exact(F, S, T, d, labels):
    H, N = 2, F * S + T
    x = bf16_tensor(H, N, d, seed=F * S + T)
    x[0, :64, :] = 0                              # (spatial head 0 / temporal): a zero block or rows
    lab = None if labels is None else ints(np.array(labels, np.int32))
    codes, scales = svg.svg_layout_permute_fp8(to_dev(x, "bf16"), F, S, T, lab)
    sync()
    labs = [1, 1] if labels is None else labels
    xp = layout.permute(as_f64(x, "bf16"), F, S, T, labs)
    for h in range(H):
        oc, osc = ofp8.quantize_key_blocks(xp[h].astype(np.float32), 64)
        np.testing.assert_array_equal(codes[h].cpu().numpy(), oc)
        np.testing.assert_array_equal(scales[h].cpu().numpy(), osc)


def fp8_inputs(q, k, v, F, S, T, labels):
    """Device codes, scales and Vt of the FP8 entry (Q in the original order,
    K and V in the executing layout per labels)."""
    lab = None if labels is None else ints(np.asarray(labels, np.int32))
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    q8, qs = svg.svg_quantize_fp8_rows(qd)
    k8, ks = svg.svg_layout_permute_fp8(kd, F, S, T, lab)
    vt = svg.svg_layout_permute_vt(vd, F, S, T, lab)
    return lab, q8, qs, k8, ks, vt


def oracle_fp8_original(q, k, v, F, S, T, label, bm, bq, qblocks=None):
    """Oracle FP8 block-sparse attention of one head, rows in the original
    order: {qb: (original rows, O rows)}."""
    xs = layout.permute(np.stack([as_f64(x, "bf16") for x in (q, k, v)]), F, S, T, [label] * 3)
    parts = ofp8.fp8_block_sparse_attention(xs[0].astype(np.float32), xs[1].astype(np.float32), xs[2], bm, bq, 64,
                                            qblocks=qblocks)
    inv = masks.executing_to_original(label, F, S, T)
    return {qb: (inv[qb * bq:qb * bq + o.shape[0]], o) for qb, o in parts.items()}


@pytest.mark.parametrize("F,S,T,bq", [(5, 60, 7, 128), (3, 100, 0, 64), (7, 64, 33, 128), (9, 450, 51, 64)])
def test_fp8_attention_random_bitmap_ragged(F, S, T, bq):
    """Ragged N, mixed labels, random bitmaps with an empty q-block and the
    ragged tail tile; Q / O in the original order."""
    H, d = 2, 128
    N = F * S + T
    q, k, v = random_qkv(H, N, d, seed=N + bq, dtype="bf16", scale=1.5)
    labels = [0, 1]
    nqb, nkb = -(-N // bq), -(-N // 64)
    rng = np.random.default_rng(N)
    bm = (rng.random((H, nqb, nkb)) < 0.5).astype(np.uint8)
    bm[:, 0, :] = 0
    bm[:, -1, -1] = 1
    row_ptr, kv_idx = svg.svg_compact_block_mask(torch.from_numpy(bm).cuda())
    lab, q8, qs, k8, ks, vt = fp8_inputs(q, k, v, F, S, T, labels)
    o = svg.svg_block_sparse_attn_fp8_vt_layout(q8, qs, k8, ks, vt, row_ptr, kv_idx, lab, F, S, T, bq, 64)
    sync()
    got = to_f64(o)
    for h in range(H):
        for qb, (rows, orow) in oracle_fp8_original(q[h], k[h], v[h], F, S, T, labels[h], bm[h], bq).items():
            check_close(got[h][rows], orow, BF16_MAX_ABS, BF16_REL_L2, f"fp8 head {h} qb {qb}")
            if bm[h, qb].sum() == 0:
                assert np.all(got[h][rows] == 0.0)


def test_fp8_dense_against_oracle():
    H, F, S, T, d = 2, 4, 500, 77, 128
    N = F * S + T
    q, k, v = random_qkv(H, N, d, seed=7, dtype="bf16", scale=1.5)
    _, q8, qs, k8, ks, vt = fp8_inputs(q, k, v, F, S, T, [0, 0])
    o = svg.svg_dense_attn_fp8_vt(q8, qs, k8, ks, vt, F, S, T, 128, 64)
    sync()
    got = to_f64(o)
    for h in range(H):
        qc, qsc = ofp8.quantize_rows(as_f64(q[h], "bf16").astype(np.float32))
        kc, ksc = ofp8.quantize_key_blocks(as_f64(k[h], "bf16").astype(np.float32), 64)
        ref = dense_attention(ofp8.dequantize(qc, qsc, 1), ofp8.dequantize(kc, ksc, 64), as_f64(v[h], "bf16"))
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"fp8 dense head {h}")


def test_fp8_layer_step_hunyuan_sampled_qblocks():
    """The SVG1 layer step with the FP8 attention at the HunyuanVideo layer
    workload (33 x 3600 + 256 tokens, 24 heads, d = 128): labels from the
    profiler, lists, K quantized in the executing layout, Q per token, V^T;
    O against the oracle's FP8 attention on 8 seeded q-blocks per head plus
    the first, video/text and tail ones.  The distance to the unquantized
    (bf16-input) oracle is printed for the record."""
    w = HUNYUAN_LAYER
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        parts = list(ex.map(lambda h: structured_qkv(w, heads=[h]), range(w.H)))
    host = {x: np.concatenate([p[x] for p in parts]) for x in "qkv"}
    q, k, v = (to_dev(host[x], "bf16") for x in "qkv")
    sidx = torch.from_numpy(sample_rows(w)).cuda()
    labels, _ = svg.svg_profile_heads(q, k, v, sidx, w.F, w.S, w.T, w.ks, w.wt)
    bm = svg.svg_build_block_mask(labels, w.F, w.S, w.T, w.H, w.d, w.ks, w.wt, w.bq, w.bk)
    row_ptr, kv_idx = svg.svg_compact_block_mask(bm)
    q8, qs = svg.svg_quantize_fp8_rows(q)
    k8, ks = svg.svg_layout_permute_fp8(k, w.F, w.S, w.T, labels)
    vt = svg.svg_layout_permute_vt(v, w.F, w.S, w.T, labels)
    o = svg.svg_block_sparse_attn_fp8_vt_layout(q8, qs, k8, ks, vt, row_ptr, kv_idx, labels, w.F, w.S, w.T,
                                                w.bq, w.bk)
    sync()
    lab = labels.cpu().numpy()
    got = to_f64(o)
    del q, k, v, q8, k8, vt, o
    rng = np.random.default_rng(77)
    fixed = [0, (w.F * w.S) // w.bq, w.nqb - 2, w.nqb - 1]
    err_bf16 = []
    from oracle.attention import block_sparse_attention
    for h in range(w.H):
        label = int(lab[h])
        obm = masks.block_bitmap_ranges(label, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
        qbs = sorted(set(fixed) | set(int(x) for x in rng.choice(w.nqb, size=8, replace=False)))
        ref = oracle_fp8_original(host["q"][h], host["k"][h], host["v"][h], w.F, w.S, w.T, label, obm, w.bq, qbs)
        for qb, (rows, orow) in ref.items():
            check_close(got[h][rows], orow, BF16_MAX_ABS, BF16_REL_L2, f"fp8 layer head {h} qb {qb}")
        if h < 2:   # distance to attention on the unquantized inputs
            xs = layout.permute(np.stack([as_f64(host[x][h], "bf16") for x in "qkv"]), w.F, w.S, w.T, [label] * 3)
            exact = block_sparse_attention(xs[0], xs[1], xs[2], obm, w.bq, w.bk, qblocks=qbs)
            for qb, (rows, orow) in ref.items():
                e = got[h][rows] - exact[qb]
                err_bf16.append((np.abs(e).max(), np.linalg.norm(e) / np.linalg.norm(exact[qb])))
    print(f"fp8 vs unquantized oracle (heads 0-1): max-abs {max(a for a, _ in err_bf16):.3e}, "
          f"worst q-block rel-L2 {max(b for _, b in err_bf16):.3e}")


# ---------------------------------------------------------------------------
# The FP8 P.V mode: V coded per channel in key-tiled V^T tiles, probabilities
# coded after the lazy reference.  Codes and channel maxima bit-exact; O
# against the oracle within the bf16 bar plus, per row, the oracle's bound on
# what its undecided probability codes (p within a relative 1e-4 of a
# rounding boundary, which the kernel's fp32 logits may round either way)
# can change.

def v8_key(j):
    """Key held by byte j of a V^T code tile row (the layout svg.h states)."""
    hi, b = j >> 5, j & 31
    return 32 * (b >> 4) + 16 * ((b >> 3) & 1) + 8 * hi + (b & 7)


@pytest.mark.parametrize("F,S,T,labels", [(5, 70, 13, [0, 1]), (3, 100, 0, None), (9, 31, 40, [1, 0])])
def test_layout_permute_vt_fp8_bit_exact(F, S, T, labels):
    H, N, d = 2, F * S + T, 128
    x = bf16_tensor(H, N, d, seed=3 * N + 1)
    x[1, :, 7] = 0                                # an all-zero channel
    lab = None if labels is None else ints(np.array(labels, np.int32))
    codes, amax = svg.svg_layout_permute_vt_fp8(to_dev(x, "bf16"), F, S, T, lab)
    sync()
    labs = [1, 1] if labels is None else labels
    xp = layout.permute(as_f64(x, "bf16"), F, S, T, labs)
    nkb = -(-N // 64)
    got = codes.cpu().numpy().reshape(H, nkb, d, 64)
    key = np.array([v8_key(j) for j in range(64)])
    for h in range(H):
        oc, osc = ofp8.quantize_channels(xp[h].astype(np.float32))
        np.testing.assert_array_equal(amax[h].cpu().numpy(), np.abs(xp[h]).max(axis=0).astype(np.float32))
        np.testing.assert_array_equal(amax[h].cpu().numpy() / np.float32(448), osc)
        padded = np.zeros((nkb * 64, d), np.uint8)
        padded[:N] = oc
        want = padded.reshape(nkb, 64, d)[:, key, :].transpose(0, 2, 1)     # [tile][dim][byte]
        np.testing.assert_array_equal(got[h], want)


def pv8_inputs(q, k, v, F, S, T, labels):
    lab = None if labels is None else ints(np.asarray(labels, np.int32))
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    q8, qs = svg.svg_quantize_fp8_rows(qd)
    k8, ks = svg.svg_layout_permute_fp8(kd, F, S, T, lab)
    vt8, vamax = svg.svg_layout_permute_vt_fp8(vd, F, S, T, lab)
    return lab, q8, qs, k8, ks, vt8, vamax


def oracle_pv8_original(q, k, v, F, S, T, label, bm, bq, qblocks=None):
    """Oracle FP8 P.V attention of one head, rows in the original order:
    {qb: (original rows, O rows, bound rows, ambiguous rows)}."""
    xs = layout.permute(np.stack([as_f64(x, "bf16") for x in (q, k, v)]), F, S, T, [label] * 3)
    parts = ofp8.fp8_pv_block_sparse_attention(xs[0].astype(np.float32), xs[1].astype(np.float32),
                                               xs[2].astype(np.float32), bm, bq, 64, qblocks=qblocks)
    inv = masks.executing_to_original(label, F, S, T)
    return {qb: (inv[qb * bq:qb * bq + o.shape[0]], o, b, a) for qb, (o, b, a) in parts.items()}


def check_pv8(got_rows, orow, bound, amb, what):
    """|GPU - oracle| within the bf16 bar plus the row's bound, and rel-L2
    within the bf16 bar over the rows whose bound is below 1e-3.  Rows whose
    lazy-reference move lies within 1e-3 of the threshold (the fp32 logits
    may decide it either way, and then every later code of the row differs)
    are left out, at most 5% of a q-block's rows."""
    keep = ~amb
    assert keep.mean() >= 0.95, f"{what}: {int(amb.sum())} rows with an ambiguous reference move"
    err = np.abs(got_rows - orow)[keep]
    lim = BF16_MAX_ABS + bound[keep][:, None]
    assert np.all(err <= lim), f"{what}: max excess {float((err - lim).max()):.3e}"
    calm = keep & (bound < 1e-3)
    if calm.any():
        num = np.linalg.norm((got_rows - orow)[calm])
        den = max(np.linalg.norm(orow[calm]), 1e-30)
        assert num / den <= BF16_REL_L2, f"{what}: rel-L2 {num / den:.3e}"


@pytest.mark.parametrize("F,S,T,bq", [(5, 60, 7, 128), (3, 100, 0, 64), (7, 64, 33, 128), (9, 450, 51, 64)])
def test_fp8pv_attention_random_bitmap_ragged(F, S, T, bq):
    """Ragged N, mixed labels, random bitmaps with an empty q-block and the
    ragged tail tile; Q / O in the original order."""
    H, d = 2, 128
    N = F * S + T
    q, k, v = random_qkv(H, N, d, seed=N + bq + 1, dtype="bf16", scale=1.5)
    labels = [0, 1]
    nqb, nkb = -(-N // bq), -(-N // 64)
    rng = np.random.default_rng(N + 1)
    bm = (rng.random((H, nqb, nkb)) < 0.5).astype(np.uint8)
    bm[:, 0, :] = 0
    bm[:, -1, -1] = 1
    row_ptr, kv_idx = svg.svg_compact_block_mask(torch.from_numpy(bm).cuda())
    lab, q8, qs, k8, ks, vt8, vamax = pv8_inputs(q, k, v, F, S, T, labels)
    o = svg.svg_block_sparse_attn_fp8pv_vt_layout(q8, qs, k8, ks, vt8, vamax, row_ptr, kv_idx, lab, F, S, T, bq, 64)
    sync()
    got = to_f64(o)
    for h in range(H):
        for qb, (rows, orow, bound, amb) in oracle_pv8_original(q[h], k[h], v[h], F, S, T, labels[h], bm[h],
                                                                 bq).items():
            check_pv8(got[h][rows], orow, bound, amb, f"fp8 P.V head {h} qb {qb}")
            if bm[h, qb].sum() == 0:
                assert np.all(got[h][rows] == 0.0)


def test_fp8pv_layer_step_hunyuan_sampled_qblocks():
    """The SVG1 layer step with the FP8 P.V attention at the HunyuanVideo
    layer workload (33 x 3600 + 256 tokens, 24 heads, d = 128): labels from
    the profiler, lists, Q / K / V coded; O against the oracle on 3 seeded
    q-blocks per head of heads 0-7 plus the first, video/text and tail ones.
    The distance to the FP8 Q K^T entry (bf16 P.V) is printed for the
    record."""
    w = HUNYUAN_LAYER
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        parts = list(ex.map(lambda h: structured_qkv(w, heads=[h]), range(w.H)))
    host = {x: np.concatenate([p[x] for p in parts]) for x in "qkv"}
    q, k, v = (to_dev(host[x], "bf16") for x in "qkv")
    sidx = torch.from_numpy(sample_rows(w)).cuda()
    labels, _ = svg.svg_profile_heads(q, k, v, sidx, w.F, w.S, w.T, w.ks, w.wt)
    bm = svg.svg_build_block_mask(labels, w.F, w.S, w.T, w.H, w.d, w.ks, w.wt, w.bq, w.bk)
    row_ptr, kv_idx = svg.svg_compact_block_mask(bm)
    q8, qs = svg.svg_quantize_fp8_rows(q)
    k8, ks = svg.svg_layout_permute_fp8(k, w.F, w.S, w.T, labels)
    vt8, vamax = svg.svg_layout_permute_vt_fp8(v, w.F, w.S, w.T, labels)
    o = svg.svg_block_sparse_attn_fp8pv_vt_layout(q8, qs, k8, ks, vt8, vamax, row_ptr, kv_idx, labels, w.F, w.S,
                                                  w.T, w.bq, w.bk)
    vt = svg.svg_layout_permute_vt(v, w.F, w.S, w.T, labels)
    o_qk8 = svg.svg_block_sparse_attn_fp8_vt_layout(q8, qs, k8, ks, vt, row_ptr, kv_idx, labels, w.F, w.S, w.T,
                                                    w.bq, w.bk)
    sync()
    rel = float((o.float() - o_qk8.float()).norm() / o_qk8.float().norm())
    lab = labels.cpu().numpy()
    got = to_f64(o)
    del q, k, v, q8, k8, vt8, vt, o, o_qk8
    rng = np.random.default_rng(78)
    fixed = [0, (w.F * w.S) // w.bq, w.nqb - 1]
    qbs_of = [sorted(set(fixed) | set(int(x) for x in rng.choice(w.nqb, size=3, replace=False))) for _ in range(8)]

    def head(h):
        label = int(lab[h])
        obm = masks.block_bitmap_ranges(label, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
        return h, oracle_pv8_original(host["q"][h], host["k"][h], host["v"][h], w.F, w.S, w.T, label, obm, w.bq,
                                      qbs_of[h])

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        refs = list(ex.map(head, range(8)))
    for h, ref in refs:
        for qb, (rows, orow, bound, amb) in ref.items():
            check_pv8(got[h][rows], orow, bound, amb, f"fp8 P.V layer head {h} qb {qb}")
    print(f"fp8 P.V vs fp8 Q K^T with bf16 P.V, whole layer: rel-L2 {rel:.3e}")
