"""HIP graph capture of the library's steps: the SVG2 semantic step on two
streams (k-means, cluster sort, gathers, top-p, varlen attention; both
varlen kernels) and the
SVG1 layer step (profile, masks, lists, layouts, attention) are captured
once and replayed three times, with eager work of the program and
synchronizations between the replays; every replay must equal the eager
step bit for bit (the library launches no memset or copy nodes, only its
own kernels).  Small seeded synthetic workloads."""

import numpy as np
import pytest
import torch

from _helpers import to_dev, ints
from synth import SVG2_COG, SMOKE_BF16
from synth.generators import mixture_qkv, structured_qkv, sample_rows

pytestmark = pytest.mark.gpu

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def capture(fn):
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fn()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=cap):
            fn()
    torch.cuda.synchronize()
    return g


def replay_checks(g, outs, want, eager_other, views=None):
    """views(t, i) -> the defined part of output i (default: all of it)."""
    view = views or (lambda t, i: t)
    for _ in range(3):
        for t in outs:
            t.fill_(0) if t.dtype != torch.bfloat16 else t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outs, want)):
            assert torch.equal(view(t, i), view(w, i)), f"output {i} differs after a replay"
        eager_other()                           # the program's own eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("vt_kernel", [False, True])
def test_svg2_step_graph_replays_equal_eager(vt_kernel):
    from dataclasses import replace
    w = replace(SVG2_COG, F=2, S=1500, T=0, H=2)
    g = mixture_qkv(w)
    dev = "cuda:0"
    q, k, v = (to_dev(g[x], "bf16") for x in "qkv")
    iq, ik = ints(g["init_q"]), ints(g["init_k"])
    H, N, d = w.H, w.N, w.d
    i32 = lambda *sh: torch.empty(*sh, dtype=torch.int32, device=dev)
    aq, ak = i32(H, N), i32(H, N)
    cq = torch.empty(H, w.kq, d, dtype=torch.float64, device=dev)
    ck = torch.empty(H, w.kk, d, dtype=torch.float64, device=dev)
    sq, sk = i32(H, w.kq), i32(H, w.kk)
    pq, pk, oq, ok = i32(H, N), i32(H, N), i32(H, w.kq + 1), i32(H, w.kk + 1)
    ptr, idx = i32(H, w.kq + 1), i32(H, w.kq * w.kk)
    qp, kp, vp, o = (torch.empty_like(q) for _ in range(4))
    vt = torch.empty(svg.svg_vt_elems(H, N, d), dtype=q.dtype, device=dev)
    dm = svg.svg_dims(1, N, 0, H, d)
    ws = lambda n: torch.empty(max(1, n), dtype=torch.uint8, device=dev)
    ws_q = ws(svg.workspace_bytes(svg.SVG2_OP_KMEANS, dm, w.kq, svg2=True))
    ws_k = ws(svg.workspace_bytes(svg.SVG2_OP_KMEANS, dm, w.kk, svg2=True))
    ws_c1, ws_c2 = (ws(svg.workspace_bytes(svg.SVG2_OP_CLUSTER_PERMUTE, dm, w.kk, svg2=True)) for _ in range(2))
    ws_v = ws(svg.workspace_bytes(svg.SVG2_OP_VARLEN, dm, w.kq, w.kk, svg2=True))
    side = torch.cuda.Stream()

    def step():
        cur = torch.cuda.current_stream()
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(cur)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            svg.svg_kmeans(k, w.kk, w.iters, ik, assign=ak, centroids=ck, sizes=sk, ws=ws_k)
            svg.svg_cluster_permute(ak, w.kk, d, perm=pk, offs=ok, ws=ws_c2)
            svg.svg_permute_rows(k, pk, out=kp)
            if vt_kernel:
                svg.svg_permute_rows_vt(v, pk, out=vt)
            else:
                svg.svg_permute_rows(v, pk, out=vp)
            join.record(side)
        svg.svg_kmeans(q, w.kq, w.iters, iq, assign=aq, centroids=cq, sizes=sq, ws=ws_q)
        svg.svg_cluster_permute(aq, w.kq, d, perm=pq, offs=oq, ws=ws_c1)
        svg.svg_permute_rows(q, pq, out=qp)
        cur.wait_event(join)
        svg.svg_select_pairs(cq, ck, sk, w.top_p, pair_ptr=ptr, pair_idx=idx)
        if vt_kernel:
            svg.svg_varlen_attn_vt(qp, kp, vt, oq, ok, ptr, idx, q_perm=pq, out=o)
        else:
            svg.svg_varlen_attn(qp, kp, vp, oq, ok, ptr, idx, q_perm=pq, out=o, ws=ws_v)

    step()
    torch.cuda.synchronize()
    outs = [o, idx, ptr, aq, ak, cq, ck]
    want = [t.clone() for t in outs]
    g2 = capture(step)
    other = torch.empty_like(q)
    n_pairs = ptr[:, -1].cpu().tolist()

    def defined(t, i):
        # pair_idx is defined only up to each head's pair count
        if i != 1:
            return t
        return torch.cat([t[h, :n_pairs[h]] for h in range(H)])

    replay_checks(g2, outs, want, lambda: svg.svg_permute_rows(v, pq, out=other), defined)


def test_svg1_layer_step_graph_replays_equal_eager():
    w = SMOKE_BF16
    g = structured_qkv(w)
    q, k, v = (to_dev(g[x], "bf16") for x in "qkv")
    dev = q.device
    sidx = ints(sample_rows(w))
    F, S, T, H, d, N, bq, bk = w.F, w.S, w.T, w.H, w.d, w.N, w.bq, w.bk
    labels = torch.empty(H, dtype=torch.int32, device=dev)
    mse = torch.empty(H, 2, dtype=torch.float32, device=dev)
    prof_ws = torch.empty(svg.workspace_bytes(svg.SVG_OP_PROFILE, svg.dims(F, S, T, H, d), sidx.numel()),
                          dtype=torch.uint8, device=dev)
    bm = torch.empty(H, w.nqb, w.nkb, dtype=torch.uint8, device=dev)
    rp = torch.empty(H * w.nqb + 1, dtype=torch.int32, device=dev)
    ki = torch.empty(H * w.nqb * w.nkb, dtype=torch.int32, device=dev)
    cws = torch.empty(max(1, svg.lib().svg_workspace_bytes(svg.SVG_OP_COMPACT, None, H * w.nqb, w.nkb)),
                      dtype=torch.uint8, device=dev)
    kp, o = torch.empty_like(q), torch.empty_like(q)
    vt = torch.empty(svg.svg_vt_elems(H, N, d), dtype=q.dtype, device=dev)
    aws = svg.attn_vt_workspace(q, F, S, T, bq, bk)

    def step():
        svg.svg_profile_heads(q, k, v, sidx, F, S, T, w.ks, w.wt, labels=labels, mse=mse, ws=prof_ws)
        svg.svg_build_block_mask(labels, F, S, T, H, d, w.ks, w.wt, bq, bk, out=bm)
        svg.svg_compact_block_mask(bm, row_ptr=rp, kv_idx=ki, ws=cws)
        svg.svg_layout_permute(k, F, S, T, labels, out=kp)
        svg.svg_layout_permute_vt(v, F, S, T, labels, out=vt)
        svg.svg_block_sparse_attn_csr_vt_layout(q, kp, vt, rp, ki, labels, F, S, T, bq, bk, out=o, ws=aws)

    step()
    torch.cuda.synchronize()
    outs = [o, labels, bm, rp]
    want = [t.clone() for t in outs]
    g1 = capture(step)
    other = torch.empty_like(q)
    replay_checks(g1, outs, want, lambda: svg.svg_layout_permute(q, F, S, T, labels, out=other))
