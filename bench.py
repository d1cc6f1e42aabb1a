"""Benchmark of the sparse video attention path on one MI355X.

One step = one pass of the whole SVG1 hot path over the HunyuanVideo-shaped
layer workload.  Shape: 33 frames x 3600 tokens + 256 text tokens
(N = 119,056; 118,800 of them video), 24 heads, d = 128, bf16, 128x64 tiles,
masks at ~31% tile density.  The pass:
    profile heads (1191 sampled rows) -> block masks -> CSR lists
    -> permute Q, K, V -> block-sparse attention -> unpermute O
Inputs are synthetic and seeded (synth/), resident in HBM before timing.

Printed metric: effective block-sparse attention TFLOP/s.  The flop count is
4*d per valid (query, key) pair inside the kept tiles, divided by the whole
step time.  Also reported: the attention kernel's own rate (HIP events on
its stream), the speedup over this library's dense attention on the same
tensors, per-stage times, the MFMA roofline fraction, and the CPU oracle's
rate on a bounded sample.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--dense-reps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--density", default="k5", help="mask widths: k5 (31%%), k4 (26%%), cog_rule (~2%%)")
    ap.add_argument("--workload", default="hunyuan_layer", choices=["hunyuan_layer", "cogvideox_shape", "svg2"],
                    help="hunyuan_layer: the SVG1 layer step (default, the headline line); "
                         "cogvideox_shape: the same step at the CogVideoX shape (13 x 1350 + 224 tokens, "
                         "8 heads, d = 64, 64x64 tiles, its own mask rule; --density is ignored); "
                         "svg2: the SVG2 semantic path on the CogVideoX-shaped mixture workload")
    ap.add_argument("--pmc-target", action="store_true",
                    help="launch the block-sparse attention kernel once and a plain 1.46 GB copy "
                         "(layout kernel with every head spatial) once, for hardware-counter runs")
    ap.add_argument("--v-layout", default="vt", choices=["vt", "rowmajor"],
                    help="vt: V permuted straight into the key-tiled transposed layout and the 256-row "
                         "attention kernel (default); rowmajor: row-major V and the 128-row kernel")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: turn the rocprofv3 FETCH_SIZE and WRITE_SIZE counter CSVs of two "
                         "--pmc-target runs into the per-launch HBM traffic record under profiles/")
    return ap.parse_args()


def measured_traffic():
    """HBM bytes per launch of the block-sparse kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE record, scaled by the same counters on a
    copy of known size.  None if that record is missing or was taken on
    different kernel sources than the ones built here."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fwd_vt_hunyuan_layer_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for src in TRAFFIC_SOURCES:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


TRAFFIC_SOURCES = ["sparse_attention_video_online_amd/csrc/attn_vt.hip",
                   "sparse_attention_video_online_amd/csrc/attn_vt_core.h",
                   "sparse_attention_video_online_amd/csrc/attn_core.h",
                   "sparse_attention_video_online_amd/csrc/svg_common.h"]
TRAFFIC_KERNEL = "attn_fwd_vt<128, 128, false>"


def record_traffic(fetch_csv, write_csv):
    """Writes the HBM traffic record of the block-sparse kernel from two
    counter runs of `--pmc-target`.  FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the attention launches are averaged.  Each is scaled by the
    ratio of the known bytes of the plain copy (the last layout launch, which
    reads and writes H*N*d*2 bytes) to what the same counter reads for it."""
    import csv
    import hashlib

    def rows(path, counter):
        att, copy = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                if TRAFFIC_KERNEL in r["Kernel_Name"]:
                    att.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
                elif "layout_kernel" in r["Kernel_Name"]:
                    copy.append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
        att = [v for _, v in sorted(set(att))]
        copy = [v for _, v in sorted(set(copy))]
        return att, copy[-1]

    from synth import HUNYUAN_LAYER as w
    copy_bytes = w.H * w.N * w.d * 2
    fa, fc = rows(fetch_csv, "FETCH_SIZE")
    wa, wc = rows(write_csv, "WRITE_SIZE")
    fs, wsc = copy_bytes / (fc * 1024.0), copy_bytes / (wc * 1024.0)
    fetch = sum(fa) / len(fa) * 1024.0 * fs
    write = sum(wa) / len(wa) * 1024.0 * wsc
    h = hashlib.sha256()
    for src in TRAFFIC_SOURCES:
        h.update(open(os.path.join(ROOT, src), "rb").read())
    rec = {"kernel": TRAFFIC_KERNEL + " block-sparse", "workload": "hunyuan_layer (k5 masks)",
           "source_sha256": h.hexdigest(), "sources": TRAFFIC_SOURCES,
           "fetch_size_kib_per_launch": [round(x, 3) for x in fa],
           "write_size_kib_per_launch": [round(x, 3) for x in wa],
           "copy_kernel_bytes_each_way": copy_bytes,
           "copy_fetch_size_kib": round(fc, 3), "copy_write_size_kib": round(wc, 3),
           "fetch_scale": round(fs, 6), "write_scale": round(wsc, 6),
           "hbm_fetch_bytes_per_launch": int(fetch), "hbm_write_bytes_per_launch": int(write),
           "traffic_bytes_per_launch": int(fetch + write)}
    out = os.path.join(ROOT, "profiles", "attn_fwd_vt_hunyuan_layer_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def gen_inputs(w):
    """Seeded Q, K, V (bf16 bits) for every head, generated in parallel."""
    import concurrent.futures
    import numpy as np
    from synth.generators import structured_qkv

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        parts = list(ex.map(lambda h: structured_qkv(w, heads=[h]), range(w.H)))
    return {x: np.concatenate([p[x] for p in parts]) for x in "qkv"}


def cpu_baseline(w, ks, wt, labels, seconds):
    """The oracle's block-sparse attention on a bounded sample of this
    workload's q-blocks, in TFLOP/s with the same flop accounting."""
    import numpy as np
    from oracle import masks, layout, attention
    from oracle.numerics import as_f64
    from synth.generators import structured_qkv

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = cores
    rng = np.random.default_rng(0)
    # one head of each label present (inputs and layout prepared untimed)
    heads = []
    for lab in (0, 1):
        hs = [h for h in range(w.H) if int(labels[h]) == lab]
        if hs:
            heads.append(hs[0])
    prepared = []
    for h in heads:
        lab = int(labels[h])
        g = structured_qkv(w, heads=[h])
        qd, kd, vd = (as_f64(g[x][0], w.dtype) for x in "qkv")
        xs = layout.permute(np.stack([qd, kd, vd]), w.F, w.S, w.T, [lab] * 3)
        bm = masks.block_bitmap_ranges(lab, w.F, w.S, w.T, ks, wt, w.bq, w.bk)
        prepared.append((h, xs, bm))
    flops = 0.0
    elapsed = 0.0
    blocks = 0
    while elapsed < seconds:
        h, xs, bm = prepared[blocks % len(prepared)]
        qbs = rng.integers(0, w.nqb, size=4)
        ts = time.perf_counter()
        attention.block_sparse_attention(xs[0], xs[1], xs[2], bm, w.bq, w.bk, qblocks=qbs)
        elapsed += time.perf_counter() - ts
        sub = np.zeros_like(bm)
        sub[qbs] = bm[qbs]
        flops += 4.0 * w.d * masks.valid_pairs(sub, w.N, w.bq, w.bk)
        blocks += len(qbs)
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(min(cores, blas_threads)),
            "kind": "oracle",
            "sample": f"float64 numpy block-sparse attention on {blocks} random 128-row q-blocks of heads "
                      f"{heads} of this workload, {elapsed:.1f} s of attention time"}


def bench_svg2(args):
    """SVG2 path on the CogVideoX-shaped mixture workload (13 x 1350 + 224
    tokens, 8 heads, d = 64, bf16; k_q = 64, k_k = 256, 10 Lloyd iterations,
    top-p 0.9).  One step = k-means of Q and K, stable cluster sort of both,
    row gathers of Q, K, V, top-p pair selection, varlen attention written
    back in original order."""
    import numpy as np
    import torch
    from sparse_attention_video_online_amd import svg
    from synth import SVG2_COG as w
    from synth.generators import mixture_qkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g = mixture_qkv(w)
    up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = up(g["q"]), up(g["k"]), up(g["v"])
    iq = torch.from_numpy(g["init_q"]).to(dev)
    ik = torch.from_numpy(g["init_k"]).to(dev)
    H, N, d = w.H, w.N, w.d
    i32 = lambda *shape: torch.empty(*shape, dtype=torch.int32, device=dev)
    aq, ak = i32(H, N), i32(H, N)
    cq = torch.empty(H, w.kq, d, dtype=torch.float64, device=dev)
    ck = torch.empty(H, w.kk, d, dtype=torch.float64, device=dev)
    sq, sk = i32(H, w.kq), i32(H, w.kk)
    pq, pk, oq, ok = i32(H, N), i32(H, N), i32(H, w.kq + 1), i32(H, w.kk + 1)
    ptr, idx = i32(H, w.kq + 1), i32(H, w.kq * w.kk)
    qp, kp, vp, o = (torch.empty_like(q) for _ in range(4))
    dm = svg.svg_dims(1, N, 0, H, d)
    ws_kq = torch.empty(svg.workspace_bytes(svg.SVG2_OP_KMEANS, dm, w.kq, svg2=True), dtype=torch.uint8, device=dev)
    ws_kk = torch.empty(svg.workspace_bytes(svg.SVG2_OP_KMEANS, dm, w.kk, svg2=True), dtype=torch.uint8, device=dev)
    ws_cp, ws_cp2 = (torch.empty(max(1, svg.workspace_bytes(svg.SVG2_OP_CLUSTER_PERMUTE, dm, max(w.kq, w.kk),
                                                             svg2=True)), dtype=torch.uint8, device=dev)
                     for _ in range(2))
    ws_vl = torch.empty(svg.workspace_bytes(svg.SVG2_OP_VARLEN, dm, w.kq, w.kk, svg2=True), dtype=torch.uint8,
                        device=dev)
    stream = torch.cuda.current_stream()
    names = ["kmeans_q", "kmeans_k", "cluster_sort_qk", "gather_qkv", "select_pairs", "varlen_attn"]

    # The query chain (k-means, sort, gather of Q) and the key chain (k-means,
    # sort, gathers of K and V) are independent: the timed step runs the key
    # chain on a second stream (default priority) and joins before the pair
    # selection.  The staged step below runs everything in order on one
    # stream to time each stage.
    side = torch.cuda.Stream()

    def step_overlapped():
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(stream)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            svg.svg_kmeans(k, w.kk, w.iters, ik, assign=ak, centroids=ck, sizes=sk, ws=ws_kk)
            svg.svg_cluster_permute(ak, w.kk, d, perm=pk, offs=ok, ws=ws_cp2)
            svg.svg_permute_rows(k, pk, out=kp)
            svg.svg_permute_rows(v, pk, out=vp)
            join.record(side)
        svg.svg_kmeans(q, w.kq, w.iters, iq, assign=aq, centroids=cq, sizes=sq, ws=ws_kq)
        svg.svg_cluster_permute(aq, w.kq, d, perm=pq, offs=oq, ws=ws_cp)
        svg.svg_permute_rows(q, pq, out=qp)
        stream.wait_event(join)
        svg.svg_select_pairs(cq, ck, sk, w.top_p, pair_ptr=ptr, pair_idx=idx)
        svg.svg_varlen_attn(qp, kp, vp, oq, ok, ptr, idx, q_perm=pq, out=o, ws=ws_vl)

    def step(ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record(stream)
        mark(0)
        svg.svg_kmeans(q, w.kq, w.iters, iq, assign=aq, centroids=cq, sizes=sq, ws=ws_kq)
        mark(1)
        svg.svg_kmeans(k, w.kk, w.iters, ik, assign=ak, centroids=ck, sizes=sk, ws=ws_kk)
        mark(2)
        svg.svg_cluster_permute(aq, w.kq, d, perm=pq, offs=oq, ws=ws_cp)
        svg.svg_cluster_permute(ak, w.kk, d, perm=pk, offs=ok, ws=ws_cp)
        mark(3)
        svg.svg_permute_rows(q, pq, out=qp)
        svg.svg_permute_rows(k, pk, out=kp)
        svg.svg_permute_rows(v, pk, out=vp)
        mark(4)
        svg.svg_select_pairs(cq, ck, sk, w.top_p, pair_ptr=ptr, pair_idx=idx)
        mark(5)
        svg.svg_varlen_attn(qp, kp, vp, oq, ok, ptr, idx, q_perm=pq, out=o, ws=ws_vl)
        mark(6)

    for _ in range(args.warmup):
        step_overlapped()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step_overlapped()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    o_overlapped, idx_overlapped = o.clone(), idx.clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    step(ev)
    torch.cuda.synchronize()
    # the two-stream step computes exactly what the one-stream step does
    if not (torch.equal(o_overlapped, o) and torch.equal(idx_overlapped, idx)):
        raise SystemExit("svg2: two-stream and one-stream steps disagree")
    stage_ms = {n: ev[j].elapsed_time(ev[j + 1]) for j, n in enumerate(names)}

    # work: attention pairs from the selected clusters; bytes of the copies
    optr, oidx = ptr.cpu().numpy(), idx.cpu().numpy()
    qs, ks_ = np.diff(oq.cpu().numpy(), axis=1), np.diff(ok.cpu().numpy(), axis=1)
    pairs = 0
    for h in range(H):
        for i in range(w.kq):
            sel = oidx[h, optr[h, i]:optr[h, i + 1]]
            pairs += int(qs[h, i]) * int(ks_[h, sel].sum())
    attn_flops = 4.0 * d * pairs
    gather_bytes = 3 * 2 * H * N * d * 2
    km_flops = 3.0 * w.iters * H * N * d * (w.kq + w.kk)   # sub + fma per dim per centroid
    result = {
        "metric": "SVG2 semantic path ms per step (k-means, cluster sort, gathers, top-p, varlen attention)",
        "value": round(ms_per_step, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian mixture)",
        "config": {"workload": w.name, "N": N, "H": H, "d": d, "kq": w.kq, "kk": w.kk, "iters": w.iters,
                   "top_p": w.top_p, "pair_density": round(pairs / (H * float(N) * N), 4)},
        "stage_ms": {kk_: round(vv, 4) for kk_, vv in stage_ms.items()},
        "one_stream_ms": round(sum(stage_ms.values()), 4),
        "varlen_tflops": round(attn_flops / (stage_ms["varlen_attn"] * 1e-3) / 1e12, 2),
        "gather_gbs": round(gather_bytes / (stage_ms["gather_qkv"] * 1e-3) / 1e9, 1),
        "kmeans_vector_tflops": round(km_flops / ((stage_ms["kmeans_q"] + stage_ms["kmeans_k"]) * 1e-3) / 1e12, 2),
    }
    if not args.no_cpu_baseline:
        from oracle import svg2 as osvg2
        from oracle.numerics import as_f64
        t0 = time.perf_counter()
        qd, kd, vd = (as_f64(g[x][0], "bf16") for x in "qkv")
        oaq, ocq, osq, _ = osvg2.kmeans(qd, g["init_q"][0], w.iters)
        oak, ock, osk, _ = osvg2.kmeans(kd, g["init_k"][0], w.iters)
        optr0, oidx0, _ = osvg2.select_pairs(ocq, ock, osk, w.top_p)
        osvg2.varlen_attention(qd, kd, vd, oaq, oak, optr0, oidx0)
        t = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(t * H * 1e3, 1), "unit": "ms", "cores": len(os.sched_getaffinity(0)),
                                  "kind": "oracle",
                                  "sample": f"float64 oracle SVG2 pipeline on head 0 ({t:.1f} s), times {H} heads"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.record_traffic:
        return record_traffic(*args.record_traffic)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path shards by head "
              f"with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "svg2":
        return bench_svg2(args)

    import numpy as np
    import torch
    from sparse_attention_video_online_amd import svg
    from synth import COG, HUNYUAN_LAYER
    from synth.configs import HUNYUAN_DENSITY_POINTS
    from synth.generators import sample_rows

    if args.workload == "cogvideox_shape":
        w = COG
        ks, wt = w.ks, w.wt
    else:
        w = HUNYUAN_LAYER
        ks, wt = HUNYUAN_DENSITY_POINTS[args.density]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    host = gen_inputs(w)
    q, k, v = (torch.from_numpy(host[x].view(np.int16)).to(dev).view(torch.bfloat16) for x in "qkv")
    del host
    sidx = torch.from_numpy(sample_rows(w)).to(dev)
    F, S, T, H, d, N, bq, bk = w.F, w.S, w.T, w.H, w.d, w.N, w.bq, w.bk
    nqb, nkb = w.nqb, w.nkb

    # preallocated buffers: nothing is allocated inside the timed region
    labels = torch.empty(H, dtype=torch.int32, device=dev)
    mse = torch.empty(H, 2, dtype=torch.float32, device=dev)
    prof_ws = torch.empty(svg.workspace_bytes(svg.SVG_OP_PROFILE, svg.dims(F, S, T, H, d), sidx.numel()),
                          dtype=torch.uint8, device=dev)
    bmask = torch.empty(H, nqb, nkb, dtype=torch.uint8, device=dev)
    rows = H * nqb
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev)
    kv_idx = torch.empty(rows * nkb, dtype=torch.int32, device=dev)
    comp_ws = torch.empty(max(1, svg.lib().svg_workspace_bytes(svg.SVG_OP_COMPACT, None, rows, nkb)),
                          dtype=torch.uint8, device=dev)
    qp, kp, vp, op, o = (torch.empty_like(q) for _ in range(5))
    use_vt = args.v_layout == "vt"
    vt = torch.empty(svg.svg_vt_elems(H, N, d), dtype=q.dtype, device=dev) if use_vt else None
    attn_ws = svg.attn_vt_workspace(q, F, S, T, bq, bk) if use_vt else None
    stream = torch.cuda.current_stream()
    ev_a0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_a1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def attend():
        if use_vt:
            # Q read and O written in the original token order (the Q permute
            # and the O unpermute happen in the kernel's row indexing)
            svg.svg_block_sparse_attn_csr_vt_layout(q, kp, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, out=o,
                                                    ws=attn_ws)
        else:
            svg.svg_block_sparse_attn_csr(qp, kp, vp, row_ptr, kv_idx, F, S, T, bq, bk, out=op)

    def step(i=None, stage_events=None):
        def mark(j):
            if stage_events is not None:
                stage_events[j].record(stream)
        mark(0)
        svg.svg_profile_heads(q, k, v, sidx, F, S, T, ks, wt, labels=labels, mse=mse, ws=prof_ws)
        mark(1)
        svg.svg_build_block_mask(labels, F, S, T, H, d, ks, wt, bq, bk, out=bmask)
        svg.svg_compact_block_mask(bmask, row_ptr=row_ptr, kv_idx=kv_idx, ws=comp_ws)
        mark(2)
        if not use_vt:
            svg.svg_layout_permute(q, F, S, T, labels, out=qp)
        svg.svg_layout_permute(k, F, S, T, labels, out=kp)
        if use_vt:
            svg.svg_layout_permute_vt(v, F, S, T, labels, out=vt)
        else:
            svg.svg_layout_permute(v, F, S, T, labels, out=vp)
        mark(3)
        if i is not None:
            ev_a0[i].record(stream)
        attend()
        if i is not None:
            ev_a1[i].record(stream)
        mark(4)
        if not use_vt:
            svg.svg_layout_unpermute(op, F, S, T, labels, out=o)
            mark(5)

    if args.pmc_target:
        # the layer's inputs for the attention kernel, then one launch each of
        # the attention kernel and a plain copy of known size (H*N*d*2 bytes
        # read and written)
        step()
        torch.cuda.synchronize()
        attend()
        spatial = torch.zeros(H, dtype=torch.int32, device=dev)
        svg.svg_layout_permute(q, F, S, T, spatial, out=o)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_target": True, "copy_bytes_each_way": q.numel() * 2,
                          "kept_tiles": int(bmask.sum())}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev_a0, ev_a1)]))
    print(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (wall {wall:.2f} s), "
          f"attention {attn_ms:.3f} ms", file=sys.stderr, flush=True)

    # per-stage breakdown (one extra step with events between stages)
    se = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    step(None, se)
    torch.cuda.synchronize()
    if use_vt:  # Q and O stay in the original order: permute K and V (into Vt) only
        names = ["profile", "mask_and_lists", "permute_k_vt", "attention"]
    else:
        names = ["profile", "mask_and_lists", "permute_qkv", "attention", "unpermute_o"]
    stage_ms = {n: se[j].elapsed_time(se[j + 1]) for j, n in enumerate(names)}

    # work done: valid pairs in kept tiles (from the device bitmap)
    rows_valid = torch.clamp(N - torch.arange(nqb, device=dev) * bq, max=bq).double()
    cols_valid = torch.clamp(N - torch.arange(nkb, device=dev) * bk, max=bk).double()
    pairs = float((bmask.double() * rows_valid[None, :, None] * cols_valid[None, None, :]).sum())
    flops = 4.0 * d * pairs
    tiles = int(bmask.sum())
    density = tiles / float(H * nqb * nkb)
    dense_flops = 4.0 * d * float(N) * N * H
    lab_host = labels.cpu().numpy()

    # dense baseline: this library's attention with every tile kept
    dense = torch.empty_like(q)

    def dense_attend():
        if use_vt:
            # every query row attends every key, so Q in its original order
            # is as good as permuted (K and Vt share one key order)
            svg.svg_dense_attn_vt(q, kp, vt, F, S, T, bq, bk, out=dense)
        else:
            svg.svg_dense_attn(qp, kp, vp, F, S, T, bq, bk, out=dense)
    dense_attend()
    torch.cuda.synchronize()
    d0 = torch.cuda.Event(enable_timing=True)
    d1 = torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for _ in range(args.dense_reps):
        dense_attend()
    d1.record(stream)
    torch.cuda.synchronize()
    dense_ms = d0.elapsed_time(d1) / args.dense_reps
    print(f"[bench] dense attention {dense_ms:.3f} ms", file=sys.stderr, flush=True)

    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": f"effective block-sparse attn TFLOP/s (whole SVG1 layer step) + speedup vs dense, N={N:,}",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded structured heads; no model weights)",
        "config": {"workload": w.name, "F": F, "S": S, "T": T, "N": N, "N_video": F * S, "H": H, "d": d,
                   "bq": bq, "bk": bk, "ks_frames": ks, "wt_tokens": wt, "n_samples": int(sidx.numel()),
                   "tile_density": round(density, 4), "kept_tiles": tiles,
                   "labels": "".join(str(int(x)) for x in lab_host), "v_layout": args.v_layout,
                   "qo_layout": "original order, permuted in the attention kernel" if use_vt else "permuted",
                   "parallelism": "single GPU"},
        "attn_ms": round(attn_ms, 4),
        "attn_tflops": round(attn_tflops, 2),
        "dense_ms": round(dense_ms, 4),
        "dense_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense_attn": round(dense_ms / attn_ms, 3),
        "speedup_vs_dense_layer": round(dense_ms / ms_per_step, 3),
        "stage_ms": {kk: round(vv, 4) for kk, vv in stage_ms.items()},
        "roofline": {"bound": "mfma",
                     "kernel": (f"attn_fwd_vt<{d},{bq}>" if use_vt else f"attn_fwd_mfma<{d},{bq}>") + " (block-sparse)",
                     "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (measured_traffic() if (w is HUNYUAN_LAYER and args.density == "k5" and use_vt)
                                 else None),
                     "flop_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, ks, wt, lab_host, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
