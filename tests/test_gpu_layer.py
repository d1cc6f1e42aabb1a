"""GPU parity of the SVG1 layer step exactly as the bench times it, on the
HunyuanVideo-shaped layer workload: 33 x 3600 video + 256 text tokens
(N = 119,056), 24 heads, d = 128, bf16, 128x64 tiles, masks ks = 5 frames /
wt = 19,800 tokens, 1191 sampled rows, mixed head generators at structure
scales 0.5-3 (some heads near the decision margin).  The chain:

  svg_profile_heads -> svg_build_block_mask -> svg_compact_block_mask
  -> svg_layout_permute (K) and svg_layout_permute_vt (V into Vt)
  -> svg_block_sparse_attn_csr_vt_layout (Q read and O written in the
     original token order; the split-partials workspace as the bench passes)

Checked against the float64 oracle:
- labels: bit-exact on the heads the stored oracle profile decides
  (tests/golden/hunyuan_layer_profile.json, min/max MSE <= 0.9);
- block bitmap and CSR lists of those labels: bit-exact in full;
- O in the original token order: 32 seeded q-blocks per head plus the
  first, frame-straddling, video/text, text and tail q-blocks, within
  max-abs 2e-2 and rel-L2 1e-2 of the oracle's permute -> block-sparse
  attention -> unpermute for the label the GPU chose.
Inputs are seeded and synthetic (synth/)."""

import concurrent.futures
import json
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from _helpers import to_dev, to_f64, check_close, BF16_MAX_ABS, BF16_REL_L2
from oracle import masks, layout, attention
from oracle.numerics import as_f64
from synth import HUNYUAN_LAYER
from synth.generators import structured_qkv, sample_rows

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def layer_inputs(w):
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        parts = list(ex.map(lambda h: structured_qkv(w, heads=[h]), range(w.H)))
    return {x: np.concatenate([p[x] for p in parts]) for x in "qkv"}


def run_layer_step(w, q, k, v, sidx):
    """The bench's step, with the bench's buffers and calls; the attention
    with K gathered in the kernel must give the same O bit for bit."""
    F, S, T, H, d, N, bq, bk = w.F, w.S, w.T, w.H, w.d, w.N, w.bq, w.bk
    dev = q.device
    labels = torch.empty(H, dtype=torch.int32, device=dev)
    mse = torch.empty(H, 2, dtype=torch.float32, device=dev)
    bmask = torch.empty(H, w.nqb, w.nkb, dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(H * w.nqb + 1, dtype=torch.int32, device=dev)
    kv_idx = torch.empty(H * w.nqb * w.nkb, dtype=torch.int32, device=dev)
    kp, o = torch.empty_like(q), torch.empty_like(q)
    vt = torch.empty(svg.svg_vt_elems(H, N, d), dtype=q.dtype, device=dev)
    attn_ws = svg.attn_vt_workspace(q, F, S, T, bq, bk)
    svg.svg_profile_heads(q, k, v, sidx, F, S, T, w.ks, w.wt, labels=labels, mse=mse)
    svg.svg_build_block_mask(labels, F, S, T, H, d, w.ks, w.wt, bq, bk, out=bmask)
    svg.svg_compact_block_mask(bmask, row_ptr=row_ptr, kv_idx=kv_idx)
    svg.svg_layout_permute(k, F, S, T, labels, out=kp)
    svg.svg_layout_permute_vt(v, F, S, T, labels, out=vt)
    svg.svg_block_sparse_attn_csr_vt_layout(q, kp, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, out=o,
                                            ws=attn_ws)
    # the same attention with K's permute fused into the tile DMA: bit for bit
    o2 = svg.svg_block_sparse_attn_csr_vt_fused(q, k, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, ws=attn_ws)
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o.view(torch.int16))
    del o2
    return labels, bmask, row_ptr, kv_idx, o


def layer_qblocks(w, rng, n_random=32):
    """Executing-layout q-blocks: the first two, the two around the frame 0/1
    boundary of a spatial head (3600 = 28.125 x 128), the one holding the
    video/text boundary, the text ones and the ragged tail (16 rows), plus
    n_random seeded ones."""
    fixed = [0, 1, 28, 29, (w.F * w.S) // w.bq, w.nqb - 2, w.nqb - 1]
    return sorted(set(fixed) | set(int(x) for x in rng.choice(w.nqb, size=n_random, replace=False)))


def test_layer_step_hunyuan_against_oracle():
    w = HUNYUAN_LAYER
    with open(os.path.join(GOLDEN, "hunyuan_layer_profile.json")) as f:
        gold = json.load(f)
    host = layer_inputs(w)
    q, k, v = (to_dev(host[x], w.dtype) for x in "qkv")
    sidx = torch.from_numpy(sample_rows(w)).to(q.device)
    labels, bmask, row_ptr, kv_idx, o = run_layer_step(w, q, k, v, sidx)
    lab = labels.cpu().numpy()

    # labels of the decided heads
    for hd in gold["heads"]:
        if not hd["ambiguous"]:
            assert lab[hd["head"]] == hd["label"], (hd["head"], int(lab[hd["head"]]), hd)

    # bitmap and lists of the GPU's labels, in full
    ref_bm = {lb: masks.block_bitmap_ranges(lb, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk) for lb in set(lab.tolist())}
    bm = np.stack([ref_bm[int(x)] for x in lab])
    np.testing.assert_array_equal(bmask.cpu().numpy(), bm)
    flat = bm.reshape(-1, w.nkb)
    ref_ptr = np.concatenate([[0], np.cumsum(flat.sum(axis=1, dtype=np.int64))]).astype(np.int32)
    np.testing.assert_array_equal(row_ptr.cpu().numpy(), ref_ptr)
    np.testing.assert_array_equal(kv_idx[:int(ref_ptr[-1])].cpu().numpy(), np.nonzero(flat)[1].astype(np.int32))

    # O in the original token order against the oracle
    got = to_f64(o)
    del q, k, v, o
    rng = np.random.default_rng(4242)
    checked = 0
    for h in range(w.H):
        label = int(lab[h])
        xs = layout.permute(np.stack([as_f64(host[x][h], w.dtype) for x in "qkv"]), w.F, w.S, w.T, [label] * 3)
        qbs = layer_qblocks(w, rng)
        parts = attention.block_sparse_attention(xs[0], xs[1], xs[2], ref_bm[label], w.bq, w.bk, qblocks=qbs)
        inv = masks.executing_to_original(label, w.F, w.S, w.T)
        for qb, orow in parts.items():
            rows = inv[qb * w.bq:qb * w.bq + orow.shape[0]]
            check_close(got[h][rows], orow, BF16_MAX_ABS, BF16_REL_L2, f"layer head {h} (label {label}) qb {qb}")
            checked += 1
    assert checked >= 32 * w.H
