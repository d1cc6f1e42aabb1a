"""Seeded sweeps of random small configurations through the C ABI, against
the float64 oracle (tests/test_gpu_vt.py, test_gpu_svg2.py hold the
hand-picked cases; these widen them).

- Attention on the key-tiled V^T layout with Q and O in the original order
  (svg_block_sparse_attn_csr_vt_layout) against the oracle's block-sparse
  attention in each head's executing layout, at random frame counts and
  sizes, text lengths, head dims, q-block heights, labels and bitmap
  densities; the K-gathering entry (svg_block_sparse_attn_csr_vt_fused)
  equal to it bit for bit.  Tolerance: max-abs 2e-2, rel-L2 1e-2 (bf16).
- k-means (bf16 at d = 64 and 128, fp32) on well-separated random mixtures:
  assignments and sizes bit-exact, float64 centroids to 1e-12, after the
  oracle's float32 margin audit.
- The SVG2 chain k-means -> cluster sort -> top-p pairs -> varlen attention
  against the oracle's varlen attention on the oracle's clusters and pairs
  (after the top-p margin audit)."""

import numpy as np
import pytest
import torch

from _helpers import to_dev, to_host_bits, to_f64, ints, check_close, BF16_MAX_ABS, BF16_REL_L2
from oracle import layout, attention, svg2 as osvg2
from oracle.numerics import as_f64
from synth.generators import random_qkv, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def sync():
    torch.cuda.synchronize()


def attn_case(seed):
    rng = np.random.default_rng(1000 + seed)
    F = int(rng.integers(1, 13))
    S = int(rng.integers(5, 160))
    T = int(rng.integers(0, 80))
    H = int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    bq = int(rng.choice([64, 128]))
    dens = float(rng.uniform(0.1, 0.9))
    labels = rng.integers(0, 2, size=H).astype(np.int32)
    return F, S, T, H, d, bq, dens, labels


@pytest.mark.parametrize("seed", range(8))
def test_sweep_attention_layout_and_fused(seed):
    F, S, T, H, d, bq, dens, labels = attn_case(seed)
    N, bk = F * S + T, 64
    q, k, v = random_qkv(H, N, d, seed=seed + 77, dtype="bf16", scale=1.5)
    nqb, nkb = -(-N // bq), -(-N // bk)
    bm = (np.random.default_rng(seed + 5).random((H, nqb, nkb)) < dens).astype(np.uint8)
    row_ptr, kv_idx = svg.svg_compact_block_mask(torch.from_numpy(bm).cuda())
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    lab = ints(labels)
    kp = svg.svg_layout_permute(kd, F, S, T, lab)
    vt = svg.svg_layout_permute_vt(vd, F, S, T, lab)
    o = svg.svg_block_sparse_attn_csr_vt_layout(qd, kp, vt, row_ptr, kv_idx, lab, F, S, T, bq, bk)
    of = svg.svg_block_sparse_attn_csr_vt_fused(qd, kd, vt, row_ptr, kv_idx, lab, F, S, T, bq, bk)
    sync()
    np.testing.assert_array_equal(to_host_bits(of), to_host_bits(o))
    got = to_f64(o)
    for h in range(H):
        lb = [int(labels[h])] * 3
        xs = layout.permute(np.stack([as_f64(x[h], "bf16") for x in (q, k, v)]), F, S, T, lb)
        ref_p = attention.block_sparse_attention_full(xs[0], xs[1], xs[2], bm[h], bq, bk)
        ref = layout.unpermute(ref_p[None], F, S, T, [int(labels[h])])[0]
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"sweep {seed} head {h}")


def mixture(rng, H, N, d, k):
    comp = rng.integers(0, k, size=(H, N))
    comp[:, :k] = np.arange(k)
    means = rng.standard_normal((H, k, d)).astype(np.float32) * 4
    x32 = np.take_along_axis(means, comp[:, :, None], axis=1) + 0.5 * rng.standard_normal((H, N, d)).astype(np.float32)
    init = np.stack([[np.flatnonzero(comp[h] == j)[0] for j in range(k)] for h in range(H)]).astype(np.int32)
    return x32, init


@pytest.mark.parametrize("seed", range(6))
def test_sweep_kmeans(seed):
    rng = np.random.default_rng(2000 + seed)
    H = int(rng.integers(1, 3))
    N = int(rng.integers(300, 2500))
    d = int(rng.choice([64, 128]))
    k = int(rng.choice([2, 9, 40, 100, 256]))
    iters = int(rng.integers(1, 4))
    dtype = "f32" if seed == 5 else "bf16"
    x32, init = mixture(rng, H, N, d, k)
    x = f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    a, c, s = svg.svg_kmeans(to_dev(x, dtype), k, iters, ints(init))
    sync()
    for h in range(H):
        oa, oc, os_, margin, ratio = osvg2.kmeans(as_f64(x[h], dtype), init[h], iters, f32_audit=True)
        assert margin > 1e-3 and ratio > 1.01, (margin, ratio)
        np.testing.assert_array_equal(a[h].cpu().numpy(), oa)
        np.testing.assert_array_equal(s[h].cpu().numpy(), os_)
        np.testing.assert_allclose(c[h].cpu().numpy(), oc, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_sweep_svg2_chain(seed):
    rng = np.random.default_rng(3000 + seed)
    H = 2
    N = int(rng.integers(400, 1800))
    d = int(rng.choice([64, 128]))
    kq, kk = int(rng.choice([4, 8, 16])), int(rng.choice([8, 24, 48]))
    top_p = float(rng.choice([0.5, 0.8, 0.95]))
    q32, iq = mixture(rng, H, N, d, kq)
    k32, ik = mixture(rng, H, N, d, kk)
    q, k = f32_to_bf16_bits(q32), f32_to_bf16_bits(k32)
    v = f32_to_bf16_bits(rng.standard_normal((H, N, d)).astype(np.float32))
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    aq, cq, sq = svg.svg_kmeans(qd, kq, 3, ints(iq))
    ak, ck, sk = svg.svg_kmeans(kd, kk, 3, ints(ik))
    pq, oq = svg.svg_cluster_permute(aq, kq, d)
    pk, ok = svg.svg_cluster_permute(ak, kk, d)
    qp, kp, vp = svg.svg_permute_rows(qd, pq), svg.svg_permute_rows(kd, pk), svg.svg_permute_rows(vd, pk)
    ptr, idx = svg.svg_select_pairs(cq, ck, sk, top_p)
    o = svg.svg_varlen_attn(qp, kp, vp, oq, ok, ptr, idx, q_perm=pq)
    sync()
    got = to_f64(o)
    for h in range(H):
        qh, kh, vh = (as_f64(x[h], "bf16") for x in (q, k, v))
        oaq, ocq, osq, _, _ = osvg2.kmeans(qh, iq[h], 3, f32_audit=True)
        oak, ock, osk, _, _ = osvg2.kmeans(kh, ik[h], 3, f32_audit=True)
        np.testing.assert_array_equal(aq[h].cpu().numpy(), oaq)
        np.testing.assert_array_equal(ak[h].cpu().numpy(), oak)
        optr, oidx, margins = osvg2.select_pairs(ocq, ock, osk, top_p)
        assert np.all(margins[:, :2].min(axis=1) > 1e-8) and np.all(margins[:, 2] > 1e-8)
        n = int(ptr[h, -1])
        np.testing.assert_array_equal(ptr[h].cpu().numpy(), optr)
        np.testing.assert_array_equal(idx[h, :n].cpu().numpy(), oidx)
        ref = osvg2.varlen_attention(qh, kh, vh, oaq, oak, optr, oidx)
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"svg2 chain {seed} head {h}")
