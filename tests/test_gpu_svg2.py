"""GPU parity of the SVG2 semantic path against the float64 oracle.

Bit-exact: k-means assignments and sizes, centroids (member sums of bf16
values are exact in float64 on both sides), cluster permutations and offsets,
top-p pair lists, the gathered key-tiled V^T.  Toleranced: varlen attention
outputs of both kernels, row-major V and key-tiled V^T (bf16: max-abs 2e-2,
rel-L2 1e-2).  Inputs: the seeded Gaussian-mixture workload (synth/) and
seeded random cluster assignments with skewed sizes.
"""

import json
import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from _helpers import to_dev, to_f64, ints, check_close, exact_sum_span_ok, BF16_MAX_ABS, BF16_REL_L2
from oracle import svg2 as osvg2
from oracle.attention import dense_attention
from oracle.numerics import as_f64
from synth import SVG2_COG
from synth.generators import mixture_qkv, random_qkv

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")

W = SVG2_COG
_cache = {}


def sync():
    torch.cuda.synchronize()


def data():
    if "g" not in _cache:
        _cache["g"] = mixture_qkv(W)
    return _cache["g"]


def oracle_head(h):
    """Oracle k-means (Q and K), sizes, pairs of head h (cached)."""
    key = ("oracle", h)
    if key not in _cache:
        g = data()
        q, k = as_f64(g["q"][h], "bf16"), as_f64(g["k"][h], "bf16")
        aq, cq, sq, _ = osvg2.kmeans(q, g["init_q"][h], W.iters)
        ak, ck, sk, _ = osvg2.kmeans(k, g["init_k"][h], W.iters)
        ptr, idx, _ = osvg2.select_pairs(cq, ck, sk, W.top_p)
        _cache[key] = dict(aq=aq, cq=cq, sq=sq, ak=ak, ck=ck, sk=sk, ptr=ptr, idx=idx)
    return _cache[key]


def gpu_pipeline():
    if "gpu" not in _cache:
        g = data()
        q, k, v = (to_dev(g[x], "bf16") for x in "qkv")
        aq, cq, sq = svg.svg_kmeans(q, W.kq, W.iters, ints(g["init_q"]))
        ak, ck, sk = svg.svg_kmeans(k, W.kk, W.iters, ints(g["init_k"]))
        pq, oq = svg.svg_cluster_permute(aq, W.kq, W.d)
        pk, ok = svg.svg_cluster_permute(ak, W.kk, W.d)
        qp = svg.svg_permute_rows(q, pq)
        kp = svg.svg_permute_rows(k, pk)
        vp = svg.svg_permute_rows(v, pk)
        ptr, idx = svg.svg_select_pairs(cq, ck, sk, W.top_p)
        o = svg.svg_varlen_attn(qp, kp, vp, oq, ok, ptr, idx, q_perm=pq)
        vt = svg.svg_permute_rows_vt(v, pk)
        o_vt = svg.svg_varlen_attn_vt(qp, kp, vt, oq, ok, ptr, idx, q_perm=pq)
        sync()
        _cache["gpu"] = dict(aq=aq, cq=cq, sq=sq, ak=ak, ck=ck, sk=sk, pq=pq, oq=oq, pk=pk, ok=ok,
                             ptr=ptr, idx=idx, o=o, o_vt=o_vt)
    return _cache["gpu"]


def test_kmeans_bit_exact_all_heads():
    """Assignments, sizes and float64 centroids equal the oracle's bit for
    bit; the centroid part rests on the exact-sum bound, checked here on the
    inputs."""
    r = gpu_pipeline()
    g = data()
    for h in range(W.H):
        o = oracle_head(h)
        assert exact_sum_span_ok(as_f64(g["q"][h], "bf16"), o["aq"], W.kq)
        assert exact_sum_span_ok(as_f64(g["k"][h], "bf16"), o["ak"], W.kk)
        np.testing.assert_array_equal(r["aq"][h].cpu().numpy(), o["aq"])
        np.testing.assert_array_equal(r["ak"][h].cpu().numpy(), o["ak"])
        np.testing.assert_array_equal(r["sq"][h].cpu().numpy(), o["sq"])
        np.testing.assert_array_equal(r["sk"][h].cpu().numpy(), o["sk"])
        np.testing.assert_array_equal(r["cq"][h].cpu().numpy(), o["cq"])
        np.testing.assert_array_equal(r["ck"][h].cpu().numpy(), o["ck"])


def test_kmeans_recovers_components():
    r = gpu_pipeline()
    g = data()
    np.testing.assert_array_equal(r["aq"].cpu().numpy(), g["comp_q"])
    np.testing.assert_array_equal(r["ak"].cpu().numpy(), g["comp_k"])


@pytest.mark.parametrize("N,d,k,iters,dtype", [(1000, 64, 7, 3, "bf16"), (700, 64, 45, 2, "bf16"),
                                               (400, 64, 1, 2, "bf16"), (50, 64, 3, 2, "bf16"),
                                               (1500, 64, 256, 2, "bf16"),
                                               (333, 128, 256, 2, "bf16"),
                                               (517, 64, 1, 1, "f32"), (300, 128, 16, 4, "f32")])
def test_kmeans_small_shapes(N, d, k, iters, dtype):
    """Small well-separated mixtures (k components, one seeded member each
    as the initial centroid) at ragged sizes, bf16 and fp32."""
    H = 2
    rng = np.random.default_rng(N + k)
    comp = rng.integers(0, k, size=(H, N))
    comp[:, :k] = np.arange(k)                        # every component has a member
    means = rng.standard_normal((H, k, d)).astype(np.float32) * 4
    x32 = np.take_along_axis(means, comp[:, :, None], axis=1) + \
        0.5 * rng.standard_normal((H, N, d)).astype(np.float32)
    from synth.generators import f32_to_bf16_bits
    x = f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    init = np.stack([[np.flatnonzero(comp[h] == j)[0] for j in range(k)] for h in range(H)]).astype(np.int32)
    a, c, s = svg.svg_kmeans(to_dev(x, dtype), k, iters, ints(init))
    sync()
    for h in range(H):
        oa, oc, os_, margin, ratio = osvg2.kmeans(as_f64(x[h], dtype), init[h], iters, f32_audit=True)
        assert margin > 1e-3 and ratio > 1.01, (margin, ratio)
        np.testing.assert_array_equal(a[h].cpu().numpy(), oa)
        np.testing.assert_array_equal(s[h].cpu().numpy(), os_)
        np.testing.assert_allclose(c[h].cpu().numpy(), oc, rtol=1e-12, atol=1e-12)


# Heads that reach a fixed point of Lloyd's map (an assignment equal to the
# previous one) after different numbers of iterations, or not within the
# run: (sigma, seed) of a 24-component mixture per head, and the iteration
# after which the oracle's assignment stops changing, for the record.
_FIXED_POINT_HEADS = {
    (64, "bf16"): [(0.5, 5), (6.0, 7), (6.0, 6), (6.0, 5)],     # 1, 4, 6, 7
    (64, "f32"): [(0.5, 5), (5.0, 5), (6.0, 5), (6.5, 5)],      # 1, 4, 7, 11
    (128, "bf16"): [(0.5, 5), (5.0, 5), (6.0, 6), (6.0, 7)],    # 1, 3, 5, 7 (sigma x 1.41)
    (128, "f32"): [(0.5, 5), (5.0, 5), (6.0, 7), (7.0, 5)],     # 1, 3, 7, 8 (sigma x 1.41)
}


@pytest.mark.parametrize("iters", [5, 10])
@pytest.mark.parametrize("d,dtype", sorted(_FIXED_POINT_HEADS))
def test_kmeans_heads_reaching_a_fixed_point_at_different_iterations(d, dtype, iters):
    """Each head stops its iterations once its assignment stands still; the
    outputs must still be those of all iterations, head by head.  The second
    call reuses the output buffers (the first iteration compares against
    nothing)."""
    from synth.generators import f32_to_bf16_bits
    N, k = 900, 24
    xs, inits = [], []
    for sig, seed in _FIXED_POINT_HEADS[(d, dtype)]:
        rng = np.random.default_rng(seed)
        comp = rng.integers(0, k, size=N)
        comp[:k] = np.arange(k)
        means = rng.standard_normal((k, d)).astype(np.float32) * 4
        s = sig * (1 if d == 64 else 1.41)
        xs.append(means[comp] + s * rng.standard_normal((N, d)).astype(np.float32))
        inits.append([np.flatnonzero(comp == j)[0] for j in range(k)])
    x32 = np.stack(xs)
    x = f32_to_bf16_bits(x32) if dtype == "bf16" else x32
    init = np.asarray(inits, dtype=np.int32)
    xd = to_dev(x, dtype)
    a, c, s_ = svg.svg_kmeans(xd, k, 10 if iters == 5 else 3, ints(init))
    a, c, s_ = svg.svg_kmeans(xd, k, iters, ints(init), assign=a, centroids=c, sizes=s_)
    sync()
    for h in range(len(inits)):
        oa, oc, os_, margin, ratio = osvg2.kmeans(as_f64(x[h], dtype), init[h], iters, f32_audit=True)
        assert ratio > 1.01, (h, ratio)
        np.testing.assert_array_equal(a[h].cpu().numpy(), oa)
        np.testing.assert_array_equal(s_[h].cpu().numpy(), os_)
        np.testing.assert_allclose(c[h].cpu().numpy(), oc, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kmeans_duplicate_init_tie_goes_to_lower_index(dtype):
    H, N, d = 1, 64, 64
    x, _, _ = random_qkv(H, N, d, seed=5, dtype=dtype)
    init = np.array([[3, 3, 10]], dtype=np.int32)    # clusters 0 and 1 start equal
    a, c, s = svg.svg_kmeans(to_dev(x, dtype), 3, 1, ints(init))
    sync()
    x64 = as_f64(x[0], dtype)
    oa, oc, os_, _ = osvg2.kmeans(x64, init[0], 1)
    np.testing.assert_array_equal(a[0].cpu().numpy(), oa)
    assert s[0, 1].item() == 0                       # the tie never picks cluster 1
    np.testing.assert_array_equal(c[0, 1].cpu().numpy(), x64[3])


def test_cluster_permute_bit_exact():
    r = gpu_pipeline()
    for h in range(W.H):
        for side, kk in (("q", W.kq), ("k", W.kk)):
            perm, offs = osvg2.cluster_permute(r["a" + side][h].cpu().numpy(), kk)
            np.testing.assert_array_equal(r["p" + side][h].cpu().numpy(), perm)
            np.testing.assert_array_equal(r["o" + side][h].cpu().numpy(), offs)


@pytest.mark.parametrize("N,k", [(1, 1), (1023, 5), (1025, 256), (4000, 37)])
def test_cluster_permute_random_with_empty_clusters(N, k):
    rng = np.random.default_rng(N + k)
    H = 3
    a = rng.integers(0, k, size=(H, N)).astype(np.int32)
    if k > 2:
        a[a == 1] = 0                                 # cluster 1 empty
    perm, offs = svg.svg_cluster_permute(ints(a), k)
    sync()
    for h in range(H):
        p, o = osvg2.cluster_permute(a[h], k)
        np.testing.assert_array_equal(perm[h].cpu().numpy(), p)
        np.testing.assert_array_equal(offs[h].cpu().numpy(), o)


def test_permute_rows_gather_and_scatter():
    H, N, d = 2, 777, 64
    x, _, _ = random_qkv(H, N, d, seed=77, dtype="bf16")
    rng = np.random.default_rng(1)
    perm = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    xd = to_dev(x, "bf16")
    y = svg.svg_permute_rows(xd, ints(perm))
    z = svg.svg_permute_rows(y, ints(perm), inverse=True)
    sync()
    yh = y.view(torch.int16).cpu().numpy().view(np.uint16)
    for h in range(H):
        np.testing.assert_array_equal(yh[h], x[h][perm[h]])
    np.testing.assert_array_equal(z.view(torch.int16).cpu().numpy().view(np.uint16), x)


def test_select_pairs_bit_exact_from_oracle_centroids():
    cq = np.stack([oracle_head(h)["cq"] for h in range(W.H)])
    ck = np.stack([oracle_head(h)["ck"] for h in range(W.H)])
    sk = np.stack([oracle_head(h)["sk"] for h in range(W.H)]).astype(np.int32)
    ptr, idx = svg.svg_select_pairs(torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(),
                                    ints(sk), W.top_p)
    sync()
    for h in range(W.H):
        o = oracle_head(h)
        np.testing.assert_array_equal(ptr[h].cpu().numpy(), o["ptr"])
        np.testing.assert_array_equal(idx[h].cpu().numpy()[:o["ptr"][-1]], o["idx"])


def test_select_pairs_hand_cases_and_extremes():
    with open(os.path.join(GOLDEN, "topp_small.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        sizes = np.array([case["sizes"]], dtype=np.int32)
        kk = sizes.shape[1]
        ck = np.random.default_rng(kk).standard_normal((1, kk, 64))
        ptr, idx = svg.svg_select_pairs(torch.zeros(1, 1, 64, dtype=torch.float64, device="cuda:0"),
                                        torch.from_numpy(ck).cuda(), ints(sizes), case["p"])
        sync()
        got = idx[0].cpu().numpy()[:ptr[0, 1].item()]
        np.testing.assert_array_equal(got, case["expect"])
    rng = np.random.default_rng(3)
    cq, ck = rng.standard_normal((2, 5, 64)), rng.standard_normal((2, 40, 64))
    sizes = rng.integers(1, 30, size=(2, 40)).astype(np.int32)
    sizes[:, 7] = 0
    for p in (1.0, 1e-9, 0.5):
        ptr, idx = svg.svg_select_pairs(torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(), ints(sizes), p)
        sync()
        for h in range(2):
            optr, oidx, _ = osvg2.select_pairs(cq[h], ck[h], sizes[h], p)
            np.testing.assert_array_equal(ptr[h].cpu().numpy(), optr)
            np.testing.assert_array_equal(idx[h].cpu().numpy()[:optr[-1]], oidx)


@pytest.mark.parametrize("key", ["o", "o_vt"])
def test_varlen_attention_pipeline_end_to_end(key):
    """GPU pipeline (k-means, permutes, pairs, varlen attention, un-permute)
    against the oracle's varlen attention with the oracle's own clusters and
    pairs, in original token order, all heads; both kernels (row-major V,
    key-tiled V^T gathered in one pass)."""
    r = gpu_pipeline()
    g = data()
    got = to_f64(r[key])
    for h in range(W.H):
        o = oracle_head(h)
        q, k, v = (as_f64(g[x][h], "bf16") for x in "qkv")
        ref = osvg2.varlen_attention(q, k, v, o["aq"], o["ak"], o["ptr"], o["idx"])
        check_close(got[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"svg2 head {h}")


@pytest.mark.parametrize("vt_kernel", [False, True])
@pytest.mark.parametrize("N,d", [(1500, 128), (5000, 128), (9000, 64)])
def test_varlen_all_pairs_equals_dense(vt_kernel, N, d):
    """Every pair selected: varlen attention is dense attention (sampled
    rows).  With N above the gather kernel's row table (2048 keys at
    d = 128, 4096 at d = 64) its walk runs in chunks that carry the softmax
    state."""
    H, kq, kk = 2, 5, 9
    q, k, v = random_qkv(H, N, d, seed=11, dtype="bf16")
    rng = np.random.default_rng(2)
    aq = rng.integers(0, kq, size=(H, N)).astype(np.int32)
    ak = rng.integers(0, kk, size=(H, N)).astype(np.int32)
    pq, oq = svg.svg_cluster_permute(ints(aq), kq, d)
    pk, ok = svg.svg_cluster_permute(ints(ak), kk, d)
    qd, kd, vd = (to_dev(t, "bf16") for t in (q, k, v))
    qp, kp, vp = svg.svg_permute_rows(qd, pq), svg.svg_permute_rows(kd, pk), svg.svg_permute_rows(vd, pk)
    ptr = torch.from_numpy(np.tile(np.arange(0, kq * kk + 1, kk, dtype=np.int32), (H, 1))).cuda()
    idx = torch.from_numpy(np.tile(np.tile(np.arange(kk, dtype=np.int32), kq), (H, 1))).cuda()
    if vt_kernel:
        o = svg.svg_varlen_attn_vt(qp, kp, svg.svg_permute_rows_vt(vd, pk), oq, ok, ptr, idx, q_perm=pq)
    else:
        o = svg.svg_varlen_attn(qp, kp, vp, oq, ok, ptr, idx, q_perm=pq)
    sync()
    got = to_f64(o)
    rows = np.r_[0:100, 700:760, N // 2:N // 2 + 40, N - 50:N]
    for h in range(H):
        ref = dense_attention(as_f64(q[h], "bf16"), as_f64(k[h], "bf16"), as_f64(v[h], "bf16"), rows=rows)
        check_close(got[h][rows], ref, BF16_MAX_ABS, BF16_REL_L2, f"all-pairs head {h}")


@pytest.mark.parametrize("vt_kernel", [False, True])
def test_varlen_k_zero_mean_of_selected_clusters(vt_kernel):
    """K = 0: every selected key scores alike, so a row's output is the mean
    of the values of its selected clusters."""
    H, N, d, kq, kk = 1, 900, 64, 4, 6
    q, v, _ = random_qkv(H, N, d, seed=12, dtype="bf16")
    kz = np.zeros_like(q)
    rng = np.random.default_rng(4)
    aq = rng.integers(0, kq, size=(H, N)).astype(np.int32)
    ak = rng.integers(0, kk, size=(H, N)).astype(np.int32)
    ptr_np = np.array([[0, 2, 3, 5, 6]], dtype=np.int32)
    idx_np = np.zeros((H, kq * kk), dtype=np.int32)
    idx_np[0, :6] = [1, 4, 0, 2, 5, 3]
    pq, oq = svg.svg_cluster_permute(ints(aq), kq, d)
    pk, ok = svg.svg_cluster_permute(ints(ak), kk, d)
    qp = svg.svg_permute_rows(to_dev(q, "bf16"), pq)
    kp = svg.svg_permute_rows(to_dev(kz, "bf16"), pk)
    if vt_kernel:
        vt = svg.svg_permute_rows_vt(to_dev(v, "bf16"), pk)
        o = svg.svg_varlen_attn_vt(qp, kp, vt, oq, ok, ints(ptr_np), ints(idx_np), q_perm=pq)
    else:
        vp = svg.svg_permute_rows(to_dev(v, "bf16"), pk)
        o = svg.svg_varlen_attn(qp, kp, vp, oq, ok, ints(ptr_np), ints(idx_np), q_perm=pq)
    sync()
    got = to_f64(o)[0]
    vv = as_f64(v[0], "bf16")
    for i in range(N):
        sel = idx_np[0, ptr_np[0, aq[0, i]]:ptr_np[0, aq[0, i] + 1]]
        ref = vv[np.isin(ak[0], sel)].mean(axis=0)
        check_close(got[i], ref, 1e-2, 1e-2, f"kzero row {i}")


@pytest.mark.parametrize("N,d", [(1, 64), (63, 64), (200, 128), (4097, 64), (1000, 128)])
def test_permute_rows_vt_bit_exact(N, d):
    """The gathered key-tiled V^T against numpy: tile kb, channel c, key j
    holds V[perm[64 kb + j]][c], zero past N."""
    H = 3
    v = random_qkv(H, N, d, seed=N + d, dtype="bf16")[2]
    rng = np.random.default_rng(N)
    perm = np.stack([rng.permutation(N) for _ in range(H)]).astype(np.int32)
    vt = svg.svg_permute_rows_vt(to_dev(v, "bf16"), ints(perm))
    sync()
    nkb = -(-N // 64)
    want = np.zeros((H, nkb * 64, d), dtype=v.dtype)
    for h in range(H):
        want[h, :N] = v[h][perm[h]]
    want = want.reshape(H, nkb, 64, d).transpose(0, 1, 3, 2)
    got = vt.cpu().view(torch.int16).numpy()
    np.testing.assert_array_equal(got, want.view(np.int16))


def skewed_assign(rng, N, k):
    """Cluster ids with sizes spread over orders of magnitude (some empty):
    small clusters share 64-key windows, large ones span several 128-row
    chunks."""
    w = np.exp(rng.normal(0.0, 1.5, size=k))
    w[rng.random(k) < 0.15] = 0.0
    w[0] = max(w[0], 1e-3)
    return rng.choice(k, size=N, p=w / w.sum()).astype(np.int32)


def random_pairs(rng, H, kq, kk, p):
    """Random ascending pair lists, each query cluster keeping a fraction p
    of the key clusters (cluster 1 keeps none)."""
    ptr = np.zeros((H, kq + 1), np.int32)
    idx = np.zeros((H, kq * kk), np.int32)
    for h in range(H):
        pos = 0
        for i in range(kq):
            sel = np.flatnonzero(rng.random(kk) < p) if i != 1 else np.array([], np.int64)
            idx[h, pos:pos + sel.size] = sel
            pos += sel.size
            ptr[h, i + 1] = pos
    return ptr, idx


@pytest.mark.parametrize("N,d,kq,kk,p", [(777, 64, 6, 40, 0.3), (2500, 128, 9, 200, 0.1), (5000, 64, 20, 256, 0.5),
                                         (3000, 128, 4, 7, 0.6)])
def test_varlen_vt_random_clusters_against_oracle(N, d, kq, kk, p):
    """Both varlen kernels against the oracle's token-exact definition on
    random skewed clusters and random pair lists: empty clusters, clusters
    smaller than a window and larger than a 128-row chunk, a query cluster
    with no pairs (its rows are zero), ragged N."""
    H = 2
    rng = np.random.default_rng(N + kk)
    q, k, v = random_qkv(H, N, d, seed=N + d, dtype="bf16", scale=1.5)
    aq = np.stack([skewed_assign(rng, N, kq) for _ in range(H)])
    ak = np.stack([skewed_assign(rng, N, kk) for _ in range(H)])
    ptr, idx = random_pairs(rng, H, kq, kk, p)
    pq, oq = svg.svg_cluster_permute(ints(aq), kq, d)
    pk, ok = svg.svg_cluster_permute(ints(ak), kk, d)
    qd, kd, vd = (to_dev(t, "bf16") for t in (q, k, v))
    qp, kp = svg.svg_permute_rows(qd, pq), svg.svg_permute_rows(kd, pk)
    o_rm = svg.svg_varlen_attn(qp, kp, svg.svg_permute_rows(vd, pk), oq, ok, ints(ptr), ints(idx), q_perm=pq)
    o_vt = svg.svg_varlen_attn_vt(qp, kp, svg.svg_permute_rows_vt(vd, pk), oq, ok, ints(ptr), ints(idx), q_perm=pq)
    sync()
    for h in range(H):
        ref = osvg2.varlen_attention(*(as_f64(x[h], "bf16") for x in (q, k, v)), aq[h], ak[h], ptr[h], idx[h])
        assert np.all(ref[aq[h] == 1] == 0.0)
        for name, o in (("row-major", o_rm), ("V^T", o_vt)):
            check_close(to_f64(o)[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"{name} varlen head {h}")


@pytest.mark.parametrize("d", [64, 128])
def test_varlen_lists_at_tile_boundaries(d):
    """Selected lists of 1, 64 (one whole tile), 512 (eight), 513 (a 1-key
    last tile), 2,063 and all 3,000 keys, and none, on query clusters of 1
    to 2,049 rows (up to 17 128-row chunks), against the oracle's
    token-exact definition."""
    H = 2
    sizes_k = [512, 1, 63, 64, 2000, 360]                 # N = 3000
    sizes_q = [300, 129, 1, 200, 64, 257, 2049]
    N = sum(sizes_k)
    assert sum(sizes_q) == N
    lists = [[0], [0, 1], [2, 4], [3], [1], list(range(6)), []]
    kq, kk = len(sizes_q), len(sizes_k)
    rng = np.random.default_rng(17)
    aq = np.stack([rng.permutation(np.repeat(np.arange(kq), sizes_q)) for _ in range(H)]).astype(np.int32)
    ak = np.stack([rng.permutation(np.repeat(np.arange(kk), sizes_k)) for _ in range(H)]).astype(np.int32)
    ptr = np.zeros((H, kq + 1), np.int32)
    idx = np.zeros((H, kq * kk), np.int32)
    for h in range(H):
        flat = [j for l in lists for j in l]
        idx[h, :len(flat)] = flat
        ptr[h, 1:] = np.cumsum([len(l) for l in lists])
    q, k, v = random_qkv(H, N, d, seed=d, dtype="bf16", scale=1.5)
    pq, oq = svg.svg_cluster_permute(ints(aq), kq, d)
    pk, ok = svg.svg_cluster_permute(ints(ak), kk, d)
    qd, kd, vd = (to_dev(t, "bf16") for t in (q, k, v))
    qp, kp = svg.svg_permute_rows(qd, pq), svg.svg_permute_rows(kd, pk)
    o = svg.svg_varlen_attn(qp, kp, svg.svg_permute_rows(vd, pk), oq, ok, ints(ptr), ints(idx), q_perm=pq)
    sync()
    for h in range(H):
        ref = osvg2.varlen_attention(*(as_f64(x[h], "bf16") for x in (q, k, v)), aq[h], ak[h], ptr[h], idx[h])
        assert np.all(ref[aq[h] == 6] == 0.0)
        check_close(to_f64(o)[h], ref, BF16_MAX_ABS, BF16_REL_L2, f"varlen tile boundaries head {h}")


def test_varlen_vt_rejects_uncovered_shapes():
    """d outside {64, 128} or more than 2048 windows a head: an error, no
    launch."""
    H, N = 1, 64
    for d, n in ((32, N), (64, 2048 * 64 + 1)):
        x = torch.zeros(H, n, d, dtype=torch.bfloat16, device="cuda")
        vt = torch.zeros(svg.svg_vt_elems(H, n, d), dtype=torch.bfloat16, device="cuda")
        offs = torch.tensor([[0, n]], dtype=torch.int32, device="cuda")
        ptr = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
        idx = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
        with pytest.raises(RuntimeError, match="varlen_attn_vt"):
            svg.svg_varlen_attn_vt(x, x.clone(), vt, offs, offs, ptr, idx)
