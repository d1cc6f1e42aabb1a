"""GPU parity of the HVA-style clustering (oracle/hva.py) through the C ABI.

Bit-exact: assignments, sizes, float64 centroids and the Lowe refresh flags
of the anchor step, and the assignments, sizes and centroids of a refresh
step on the next step's values.  Both sides take the assignment decision in
float32 in the stated order; the member sums are exact in float64, which an
audit of each head's exponent spans confirms first.  Toleranced: the
attention output of the chain HVA clusters -> cluster sort -> top-p pairs ->
varlen attention against the oracle's varlen attention with the oracle's
clusters.  Inputs: the seeded blob workload and seeded random tensors at
ragged shapes (partial windows, no text, one window, one token per window,
several text work-groups)."""

import concurrent.futures

import numpy as np
import pytest
import torch

from _helpers import to_dev, to_f64, ints, check_close, exact_sum_span_ok, BF16_MAX_ABS, BF16_REL_L2
from oracle import hva, svg2 as osvg2
from oracle.numerics import as_f64
from synth import HVA_COG as W
from synth.generators import blob_qkv, random_qkv

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")

ROWS, COLS = W.grid
HEADS = [0, 1, 2, 3]          # heads checked against the oracle (the GPU runs all 8)
_cache = {}


def sync():
    torch.cuda.synchronize()


def data(step):
    if step not in _cache:
        _cache[step] = blob_qkv(W, step=step)
    return _cache[step]


def oracle_side(side, win, h):
    key = ("oracle", side, h)
    if key not in _cache:
        x0 = as_f64(data(0)[side][h], "bf16")
        x1 = as_f64(data(1)[side][h], "bf16")
        assert exact_sum_span_ok(x0, np.zeros(x0.shape[0], np.int64), 1)
        assert exact_sum_span_ok(x1, np.zeros(x1.shape[0], np.int64), 1)
        a, c, s, r = hva.local_kmeans(x0, W.F, ROWS, COLS, W.T, win, W.iters)
        ra, rc, rs = hva.refresh_step(x1, a, c, r, W.F, ROWS, COLS, W.T, win)
        _cache[key] = dict(a=a, c=c, s=s, r=r, ra=ra, rc=rc, rs=rs)
    return _cache[key]


def oracle_all(side, win):
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        return list(ex.map(lambda h: oracle_side(side, win, h), HEADS))


@pytest.mark.parametrize("side,win", [("q", W.win_q), ("k", W.win_k)])
def test_hva_anchor_and_refresh_bit_exact(side, win):
    x0 = to_dev(data(0)[side], "bf16")
    x1 = to_dev(data(1)[side], "bf16")
    a, c, s, r = svg.svg_hva_cluster(x0, W.F, ROWS, COLS, W.T, win, W.iters)
    sync()
    anchor = [t.cpu().numpy() for t in (a, c, s, r)]
    ra, rc, rs = svg.svg_hva_refresh(x1, W.F, ROWS, COLS, W.T, win, r, a, c)
    sync()
    ref = oracle_all(side, win)
    for i, h in enumerate(HEADS):
        o = ref[i]
        np.testing.assert_array_equal(anchor[0][h], o["a"])
        np.testing.assert_array_equal(anchor[2][h], o["s"])
        np.testing.assert_array_equal(anchor[1][h], o["c"])
        np.testing.assert_array_equal(anchor[3][h], o["r"])
        np.testing.assert_array_equal(ra[h].cpu().numpy(), o["ra"])
        np.testing.assert_array_equal(rs[h].cpu().numpy(), o["rs"])
        np.testing.assert_array_equal(rc[h].cpu().numpy(), o["rc"])
    # the flags pick a real subset, and the refresh moved some of it
    assert 0.01 < anchor[3][HEADS].mean() < 0.5
    assert np.any(ra[HEADS].cpu().numpy() != anchor[0][HEADS])


SHAPES = [
    (3, 4, 5, 0, 64, (2, 2, 2), 3),        # partial windows, no text
    (2, 7, 9, 5, 128, (1, 3, 4), 4),       # d = 128, partial windows
    (1, 1, 300, 300, 64, (1, 1, 7), 2),    # one frame, one row, two text work-groups
    (5, 6, 6, 1, 128, (9, 9, 9), 2),       # a single window: one cluster (+ text)
    (4, 8, 8, 40, 64, (1, 1, 1), 1),       # one token per window
]


@pytest.mark.parametrize("F,rows,cols,T,d,win,iters", SHAPES)
def test_hva_small_shapes_bit_exact(F, rows, cols, T, d, win, iters):
    H = 2
    N = F * rows * cols + T
    x0, x1, _ = random_qkv(H, N, d, seed=N + d, dtype="bf16", scale=1.5)
    g0, g1 = to_dev(x0, "bf16"), to_dev(x1, "bf16")
    a, c, s, r = svg.svg_hva_cluster(g0, F, rows, cols, T, win, iters)
    sync()
    anchor = [t.cpu().numpy() for t in (a, c, s, r)]
    ra, rc, rs = svg.svg_hva_refresh(g1, F, rows, cols, T, win, r, a, c)
    sync()
    for h in range(H):
        y0, y1 = as_f64(x0[h], "bf16"), as_f64(x1[h], "bf16")
        oa, oc, os_, orr = hva.local_kmeans(y0, F, rows, cols, T, win, iters)
        np.testing.assert_array_equal(anchor[0][h], oa)
        np.testing.assert_array_equal(anchor[1][h], oc)
        np.testing.assert_array_equal(anchor[2][h], os_)
        np.testing.assert_array_equal(anchor[3][h], orr)
        pa, pc, ps = hva.refresh_step(y1, oa, oc, orr, F, rows, cols, T, win)
        np.testing.assert_array_equal(ra[h].cpu().numpy(), pa)
        np.testing.assert_array_equal(rc[h].cpu().numpy(), pc)
        np.testing.assert_array_equal(rs[h].cpu().numpy(), ps)


def test_hva_refresh_reassigns_tokens_outside_their_candidates():
    """A carried assignment that names a cluster outside a token's candidates
    (here: every video token in cluster 0 of a 3 x 3 x 3 window grid) is
    re-assigned even without a flag, as if flagged."""
    F, rows, cols, T, d, win = 6, 6, 6, 4, 64, (2, 2, 2)
    H, N = 1, F * rows * cols + T
    x = random_qkv(H, N, d, seed=5, dtype="bf16")[0]
    g = to_dev(x, "bf16")
    a, c, s, r = svg.svg_hva_cluster(g, F, rows, cols, T, win, 2)
    k = c.shape[1]
    forced = a.clone()
    forced[:, :F * rows * cols] = 0
    none = torch.zeros_like(r)
    fa, fc, fs = svg.svg_hva_refresh(g, F, rows, cols, T, win, none, forced, c.clone())
    sync()
    y = as_f64(x[0], "bf16")
    cand = hva.candidates(F, rows, cols, win)
    far = np.array([0 not in cand[t] for t in range(F * rows * cols)] + [False] * T)
    flags = far.astype(np.uint8)
    pa, pc, ps = hva.refresh_step(y, forced[0].cpu().numpy(), c[0].cpu().numpy(), flags, F, rows, cols, T, win)
    np.testing.assert_array_equal(fa[0].cpu().numpy(), pa)
    np.testing.assert_array_equal(fc[0].cpu().numpy(), pc)
    np.testing.assert_array_equal(fs[0].cpu().numpy(), ps)
    assert far.sum() > 0 and k == hva.n_clusters(F, rows, cols, T, win)


def test_hva_chain_varlen_attention():
    """HVA clusters of Q and K -> cluster sort -> top-p pairs -> varlen
    attention (V gathered into V^T), against the oracle's varlen attention
    over the oracle's clusters and pairs (the clusters are bit-exact, so the
    pairs are the oracle's exactly when the top-p margins clear)."""
    g = data(0)
    q, k, v = (to_dev(g[x], "bf16") for x in "qkv")
    aq, cq, sq, _ = svg.svg_hva_cluster(q, W.F, ROWS, COLS, W.T, W.win_q, W.iters)
    ak, ck, sk, _ = svg.svg_hva_cluster(k, W.F, ROWS, COLS, W.T, W.win_k, W.iters)
    kq, kk = cq.shape[1], ck.shape[1]
    pq, oq = svg.svg_cluster_permute(aq, kq, W.d)
    pk, ok = svg.svg_cluster_permute(ak, kk, W.d)
    qp, kp = svg.svg_permute_rows(q, pq), svg.svg_permute_rows(k, pk)
    vt = svg.svg_permute_rows_vt(v, pk)
    ptr, idx = svg.svg_select_pairs(cq, ck, sk, W.top_p)
    o = svg.svg_varlen_attn_vt(qp, kp, vt, oq, ok, ptr, idx, q_perm=pq)
    sync()
    got = to_f64(o)
    for h in HEADS[:2]:
        oq_ = oracle_side("q", W.win_q, h)
        ok_ = oracle_side("k", W.win_k, h)
        optr, oidx, margins = osvg2.select_pairs(oq_["c"], ok_["c"], ok_["s"], W.top_p)
        assert np.all(margins[:, :2].min(axis=1) > 1e-8) and np.all(margins[:, 2] > 1e-8)
        n = int(ptr[h, -1])
        np.testing.assert_array_equal(ptr[h].cpu().numpy(), optr)
        np.testing.assert_array_equal(idx[h, :n].cpu().numpy(), oidx)
        qh, kh, vh = (as_f64(g[x][h], "bf16") for x in "qkv")
        ref = osvg2.varlen_attention(qh, kh, vh, oq_["a"], ok_["a"], optr, oidx)
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"hva chain head {h}")
