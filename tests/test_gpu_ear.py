"""GPU parity of SVG-EAR (oracle/ear.py): block statistics, routing and the
compensated attention.

- Block statistics: float64 centroids and radii within 1e-12 / 1e-10
  relative of the oracle (different summation order); the bf16 centroid
  keys and value sums within one bf16 rounding.
- Routing: the exact sets bit-exact, after a margin audit of the oracle's
  scores at each q-block's cut (both sides decide in float64).
- Attention: O within max-abs 2e-2 / rel-L2 1e-2 of the oracle's
  compensated attention, at ragged shapes (both head dims, both q-block
  heights, mixed labels) and on the HunyuanVideo-shaped layer workload; and
  the closed form: equal keys within each block make the compensation exact,
  so the output is dense attention.
Inputs are seeded and synthetic."""

import concurrent.futures

import numpy as np
import pytest
import torch

from _helpers import to_dev, to_f64, ints, check_close, BF16_MAX_ABS, BF16_REL_L2
from oracle import ear as oear, layout, masks
from oracle.attention import dense_attention
from oracle.numerics import as_f64
from synth import HUNYUAN_LAYER
from synth.generators import random_qkv, structured_qkv, sample_rows, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def sync():
    torch.cuda.synchronize()


def executing(x, F, S, T, label):
    return layout.permute(as_f64(x, "bf16")[None], F, S, T, [label])[0]


def bf16_round(x):
    return as_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32)), "bf16")


def gpu_ear(q, k, v, F, S, T, labels, bm, bq, route_k):
    """The EAR chain on device tensors: K / V^T layouts, statistics, routing,
    lists, compensated attention."""
    lab = ints(np.asarray(labels, np.int32))
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    kp = svg.svg_layout_permute(kd, F, S, T, lab)
    vt = svg.svg_layout_permute_vt(vd, F, S, T, lab)
    kc, vct, kbar, rad = svg.svg_ear_block_stats(kp, vt, F, S, T)
    ex = svg.svg_ear_route(qd, lab, kbar, rad, torch.from_numpy(np.ascontiguousarray(bm)).cuda(), F, S, T, bq, 64,
                           route_k)
    rp, ki = svg.svg_compact_block_mask(ex)
    o = svg.svg_block_sparse_attn_ear_vt_layout(qd, kp, vt, kc, vct, rp, ki, lab, F, S, T, bq, 64)
    sync()
    return dict(kc=kc, vct=vct, kbar=kbar, rad=rad, exact=ex, o=o)


def oracle_head(q, k, v, F, S, T, label, bm, bq, route_k, qblocks=None):
    """Oracle stats, exact sets, scores and O (original row order) of one head."""
    qe, ke, ve = (executing(x, F, S, T, label) for x in (q, k, v))
    n, kbar, vbar, rad = oear.block_stats(ke, ve, 64)
    sc = oear.route_scores(qe, n, kbar, rad, bq)
    ex = oear.exact_sets(bm, sc, qe.shape[0], 64, route_k)
    parts = oear.ear_attention(qe, ke, ve, ex, bq, 64, qblocks=qblocks)
    inv = masks.executing_to_original(label, F, S, T)
    o = {qb: (inv[qb * bq:qb * bq + r.shape[0]], r) for qb, r in parts.items()}
    return dict(n=n, kbar=kbar, vbar=vbar, rad=rad, scores=sc, exact=ex, o=o)


def route_margin_ok(scores, bm, exact, N, route_k, tol=1e-9):
    """Every q-block's cut is clear: the smallest routed score exceeds the
    largest unrouted candidate's by more than tol (relative), or no
    candidate is left out."""
    nkb = bm.shape[1]
    for Q in range(bm.shape[0]):
        cand = np.flatnonzero(bm[Q] == 0)
        if N % 64:
            cand = cand[cand != nkb - 1]
        routed = cand[exact[Q, cand] == 1]
        left = cand[exact[Q, cand] == 0]
        if routed.size == 0 or left.size == 0:
            continue
        a, b = scores[Q, routed].min(), scores[Q, left].max()
        if not (a > b + tol * max(1.0, abs(a))):
            return False
    return True


CASES = [(5, 60, 7, 128, 128, 3), (3, 100, 0, 64, 64, 2), (7, 64, 33, 128, 64, 4), (4, 250, 20, 64, 128, 5)]


@pytest.mark.parametrize("F,S,T,d,bq,route_k", CASES)
def test_ear_chain_against_oracle(F, S, T, d, bq, route_k):
    H = 2
    N = F * S + T
    q, k, v = random_qkv(H, N, d, seed=N + d + bq, dtype="bf16", scale=1.5)
    labels = [0, 1]
    nqb, nkb = -(-N // bq), -(-N // 64)
    rng = np.random.default_rng(N + route_k)
    bm = (rng.random((H, nqb, nkb)) < 0.3).astype(np.uint8)
    bm[:, 0, :] = 0                              # a q-block with nothing kept: all compensated or routed
    g = gpu_ear(q, k, v, F, S, T, labels, bm, bq, route_k)
    for h in range(H):
        o = oracle_head(q[h], k[h], v[h], F, S, T, labels[h], bm[h], bq, route_k)
        np.testing.assert_allclose(g["kbar"][h].cpu().numpy().T, o["kbar"], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(g["rad"][h].cpu().numpy(), o["rad"], rtol=1e-10, atol=1e-12)
        ntc = -(-nkb // 64)
        kc = to_f64(g["kc"]).reshape(H, ntc * 64, d)[h]
        np.testing.assert_allclose(kc[:nkb], bf16_round(o["kbar"]), rtol=2 ** -7, atol=1e-30)
        assert np.all(kc[nkb:] == 0)
        vct = to_f64(g["vct"]).reshape(H, ntc, d, 64)[h]
        vsum = vct.transpose(0, 2, 1).reshape(ntc * 64, d)
        np.testing.assert_allclose(vsum[:nkb], bf16_round(o["vbar"] * o["n"][:, None]), rtol=2 ** -7, atol=1e-6)
        assert route_margin_ok(o["scores"], bm[h], o["exact"], N, route_k)
        np.testing.assert_array_equal(g["exact"][h].cpu().numpy(), o["exact"])
        got = to_f64(g["o"])[h]
        for qb, (rows, orow) in o["o"].items():
            check_close(got[rows], orow, BF16_MAX_ABS, BF16_REL_L2, f"ear head {h} qb {qb}")


def test_ear_route_past_register_capacity():
    """More than 2,048 kv-blocks a head (35 x 3800 + 70 tokens: 2,080 blocks,
    a ragged last one): the routing keeps its candidate scores in LDS
    instead of registers.  Exact sets bit-exact for both heads (after the
    margin audit); O against the oracle on seeded q-blocks plus the first,
    video/text and last ones."""
    H, F, S, T, d, bq, route_k = 2, 35, 3800, 70, 128, 128, 16
    N = F * S + T
    q, k, v = random_qkv(H, N, d, seed=77, dtype="bf16", scale=1.5)
    labels = [0, 1]
    nqb, nkb = -(-N // bq), -(-N // 64)
    assert nkb > 2048
    bm = (np.random.default_rng(78).random((H, nqb, nkb)) < 0.3).astype(np.uint8)
    g = gpu_ear(q, k, v, F, S, T, labels, bm, bq, route_k)
    got = to_f64(g["o"])
    rng = np.random.default_rng(79)
    fixed = [0, (F * S) // bq, nqb - 1]
    for h in range(H):
        qbs = sorted(set(fixed) | set(int(x) for x in rng.choice(nqb, size=5, replace=False)))
        o = oracle_head(q[h], k[h], v[h], F, S, T, labels[h], bm[h], bq, route_k, qblocks=qbs)
        assert route_margin_ok(o["scores"], bm[h], o["exact"], N, route_k)
        np.testing.assert_array_equal(g["exact"][h].cpu().numpy(), o["exact"])
        for qb, (rows, orow) in o["o"].items():
            check_close(got[h][rows], orow, BF16_MAX_ABS, BF16_REL_L2, f"ear wide head {h} qb {qb}")


def test_ear_equal_keys_per_block_is_dense_attention():
    """Keys equal within each 64-key block of the executing layout: the
    centroid stands in exactly, so the compensated output is dense
    attention whatever is skipped."""
    H, F, S, T, d, bq = 2, 4, 128, 64, 128, 128
    N = F * S + T
    q, k, v = random_qkv(H, N, d, seed=3, dtype="bf16", scale=1.0)
    labels = [0, 0]                              # executing layout = original order
    for h in range(H):
        for b in range(-(-N // 64)):
            k[h, b * 64:(b + 1) * 64] = k[h, b * 64]
    nqb, nkb = -(-N // bq), -(-N // 64)
    bm = (np.random.default_rng(4).random((H, nqb, nkb)) < 0.2).astype(np.uint8)
    g = gpu_ear(q, k, v, F, S, T, labels, bm, bq, route_k=0)
    got = to_f64(g["o"])
    for h in range(H):
        ref = dense_attention(*(as_f64(x[h], "bf16") for x in (q, k, v)))
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"equal keys head {h}")


def test_ear_layer_hunyuan_sampled_qblocks():
    """The layer step with SVG-EAR at the HunyuanVideo layer workload (33 x
    3600 + 256 tokens, 24 heads, d = 128): profiler labels, SVG1 masks, block
    statistics, routing 16 blocks per q-block, compensated attention.  Exact
    sets bit-exact for heads 0-7 (after the margin audit); O against the
    oracle on 6 seeded q-blocks per head of those heads plus the first,
    video/text and tail ones."""
    w = HUNYUAN_LAYER
    route_k = 16
    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        parts = list(ex.map(lambda h: structured_qkv(w, heads=[h]), range(w.H)))
    host = {x: np.concatenate([p[x] for p in parts]) for x in "qkv"}
    q, k, v = (to_dev(host[x], "bf16") for x in "qkv")
    sidx = torch.from_numpy(sample_rows(w)).cuda()
    labels, _ = svg.svg_profile_heads(q, k, v, sidx, w.F, w.S, w.T, w.ks, w.wt)
    bm = svg.svg_build_block_mask(labels, w.F, w.S, w.T, w.H, w.d, w.ks, w.wt, w.bq, w.bk)
    kp = svg.svg_layout_permute(k, w.F, w.S, w.T, labels)
    vt = svg.svg_layout_permute_vt(v, w.F, w.S, w.T, labels)
    kc, vct, kbar, rad = svg.svg_ear_block_stats(kp, vt, w.F, w.S, w.T)
    exm = svg.svg_ear_route(q, labels, kbar, rad, bm, w.F, w.S, w.T, w.bq, w.bk, route_k)
    rp, ki = svg.svg_compact_block_mask(exm)
    o = svg.svg_block_sparse_attn_ear_vt_layout(q, kp, vt, kc, vct, rp, ki, labels, w.F, w.S, w.T, w.bq, w.bk)
    sync()
    lab = labels.cpu().numpy()
    got = to_f64(o)
    exh = exm.cpu().numpy()
    bmh = bm.cpu().numpy()
    del q, k, v, kp, vt, o
    rng = np.random.default_rng(99)
    fixed = [0, (w.F * w.S) // w.bq, w.nqb - 2, w.nqb - 1]
    for h in range(8):
        qbs = sorted(set(fixed) | set(int(x) for x in rng.choice(w.nqb, size=6, replace=False)))
        r = oracle_head(host["q"][h], host["k"][h], host["v"][h], w.F, w.S, w.T, int(lab[h]), bmh[h], w.bq, route_k,
                        qblocks=qbs)
        assert route_margin_ok(r["scores"], bmh[h], r["exact"], w.N, route_k)
        np.testing.assert_array_equal(exh[h], r["exact"])
        for qb, (rows, orow) in r["o"].items():
            check_close(got[h][rows], orow, BF16_MAX_ABS, BF16_REL_L2, f"ear layer head {h} qb {qb}")
