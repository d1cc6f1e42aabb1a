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
rate on a bounded sample.  The default run adds, as extra keys of the same
line: the same layer step with the FP8 attention ("fp8": FP8 Q K^T, and in
"fp8.pv" FP8 P.V as well) and with SVG-EAR's
compensation and routing ("ear"), the
CogVideoX-shaped layer step ("cogvideox_shape": 13 x 1350 + 224 tokens, 8
heads, d = 64) and the SVG2 semantic path on the CogVideoX-shaped mixture
workload ("svg2").
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA peak
EAR_ROUTE_K = 16                  # skipped blocks routed to exact per q-block (SVG-EAR leg)
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--dense-reps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the FP8, CogVideoX-shaped and SVG2 legs of the default run")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--density", default="k5", help="mask widths: k5 (31%%), k4 (26%%), cog_rule (~2%%)")
    ap.add_argument("--workload", default="hunyuan_layer",
                    choices=["hunyuan_layer", "cogvideox_shape", "svg2", "hva"],
                    help="hunyuan_layer: the SVG1 layer step (default, the headline line); "
                         "cogvideox_shape: the same step at the CogVideoX shape (13 x 1350 + 224 tokens, "
                         "8 heads, d = 64, 64x64 tiles, its own mask rule; --density is ignored); "
                         "svg2: the SVG2 semantic path on the CogVideoX-shaped mixture workload; "
                         "hva: local-window clustering (anchor and refresh steps) on the blob workload")
    ap.add_argument("--pmc-target", action="store_true",
                    help="launch the block-sparse attention kernel once and a plain 1.46 GB copy "
                         "(layout kernel with every head spatial) once, for hardware-counter runs")
    ap.add_argument("--v-layout", default="vt", choices=["vt", "rowmajor"],
                    help="vt: V permuted straight into the key-tiled transposed layout and the 256-row "
                         "attention kernel (default); rowmajor: row-major V and the 128-row kernel")
    ap.add_argument("--record-counters", metavar="DIR",
                    help="host only: per-kernel HBM traffic / MFMA busy table from rocprofv3 runs under DIR")
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
TRAFFIC_KERNEL = "attn_fwd_vt<128, 128, false, false, false>"


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


COUNTERS_HEADER = """# HBM traffic, achieved bandwidth and MFMA busy time of the path's kernels

Three programs, each run under rocprofv3 four times (kernel trace; FETCH_SIZE; WRITE_SIZE;
SQ_VALU_MFMA_BUSY_CYCLES), from /tmp on the MI355X box (`<repo>` is the repository root,
`<out>` the output folder):

```
# layer: the HunyuanVideo-shaped SVG1 layer step (33 x 3600 + 256 tokens, 24 heads, d = 128)
ARGS="--no-extra --steps 2 --warmup 1 --no-cpu-baseline --dense-reps 1"
# svg2: the SVG2 semantic path on the CogVideoX-shaped mixture workload
ARGS="--workload svg2 --steps 3 --warmup 1 --no-cpu-baseline"
# hva: local-window clustering (anchor and refresh steps) on the CogVideoX-shaped blob workload
ARGS="--workload hva --steps 3 --warmup 1"
rocprofv3 --kernel-trace --stats --output-format csv -d <out>/<prog>_trace -o run -- python3 <repo>/bench.py $ARGS
rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/<prog>_fetch -o run -- python3 <repo>/bench.py $ARGS
rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/<prog>_write -o run -- python3 <repo>/bench.py $ARGS
rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES --output-format csv -d <out>/<prog>_sq -o run -- python3 <repo>/bench.py $ARGS
python3 <repo>/bench.py --record-counters <out>        # writes this table
```

Durations are each dispatch's trace time; counters are joined to it by dispatch id.  Algorithmic
bytes are what a launch must read and write once: a copy reads and writes its tensor; the
profiler's full pass reads K, its V^T copy and the sampled Q rows; a k-means assignment reads the
points and writes the assignment; an update reads the points (gathered through the cluster
order) and the order; the sort reads the assignment and writes the order; a row gather reads
and writes the tensor and reads the order.  The attention kernels are bound by the matrix
cores, not by memory: their line is there for the traffic (the sparse kernel fetches ~18x its
algorithmic bytes, ~78% of it served by the XCD L2s, at ~1.1 TB/s).  The SVG2 workload (36 MB
of Q and K) stays in the L2s and the 256 MB Infinity Cache between launches, so its k-means
kernels run at a few microseconds each and are bound by launch and per-kernel latency.  A
k-means head whose assignment stood still has its later rounds' kernels return at once: their
launches (FETCH_SIZE under 1% of the algorithmic bytes) have rows of their own, "round after the
fixed point".  The
local-window assignment (`hva_assign`) reads each token's row once and runs its distances on the
vector ALUs (a float32 expression the oracle evaluates identically), so its MFMA column is empty.

"""


COUNTER_KERNELS = ["layout_kernel", "vt_kernel", "profile_full_vt", "profile_temporal_vt", "profile_combine",
                   "block_mask_kernel", "fill_kernel", "attn_fwd_vt", "km_assign_bf3", "km_update", "sort_place",
                   "sort_count", "permute_rows_kernel", "select_rows", "varlen_gather", "varlen_vt", "km_prep3",
                   "hva_assign", "hva_finalize", "hva_prep"]


def record_counters(root):
    """Per-kernel HBM traffic, achieved bandwidth and MFMA busy time from
    rocprofv3 runs under `root`: for each of the three programs (layer: the
    HunyuanVideo layer step, bench.py --no-extra; svg2: bench.py --workload
    svg2; hva: bench.py --workload hva) a kernel trace (<prog>_trace) and
    counter runs of FETCH_SIZE
    (<prog>_fetch), WRITE_SIZE (<prog>_write) and SQ_VALU_MFMA_BUSY_CYCLES
    (<prog>_sq), each written with --output-format csv.  Dispatches are
    joined across runs by dispatch id (the programs are deterministic; the
    kernel names must agree).  FETCH_SIZE and WRITE_SIZE are scaled by the
    ratio of known to counted bytes of the layer program's layout_kernel
    launches, plain copies of H*N*d*2 bytes each way.  MFMA busy is
    SQ_VALU_MFMA_BUSY_CYCLES over the launch's SIMD cycles (duration x
    2.4 GHz x 1024 SIMDs).  Writes profiles/path_kernels_hbm_mfma.md."""
    import csv
    import glob
    from collections import defaultdict
    from synth import HUNYUAN_LAYER as L, SVG2_COG as C, HVA_COG as V

    def find(prog, kind, suffix):
        hits = glob.glob(os.path.join(root, f"{prog}_{kind}", "**", f"*{suffix}"), recursive=True)
        if not hits:
            raise SystemExit(f"record-counters: no *{suffix} under {prog}_{kind}")
        return hits[0]

    def trace(prog):
        out = {}
        for r in csv.DictReader(open(find(prog, "trace", "kernel_trace.csv"))):
            out[int(r["Dispatch_Id"])] = (r["Kernel_Name"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
        return out

    def counters(prog, kind):
        vals, names, grids = defaultdict(float), {}, {}
        for r in csv.DictReader(open(find(prog, kind, "counter_collection.csv"))):
            d = int(r["Dispatch_Id"])
            vals[(d, r["Counter_Name"])] += float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
            grids[d] = int(r["Grid_Size"])
        return vals, names, grids

    def short(name):
        for k in COUNTER_KERNELS:
            i = name.find(k)
            if i >= 0:
                j = name.find("(", i)
                return name[i:j] if j > 0 else name[i:]
        return None

    E = L.H * L.N * L.d * 2                   # one [H][N][d] bf16 tensor of the layer workload
    EC = C.H * C.N * C.d * 2                  # one of the SVG2 workload
    vt_attn = L.H * L.nkb * 64 * L.d * 2      # Vt of the attention
    prof_tiles = L.F * -(-L.S // 64) + -(-L.T // 64)
    vt_prof = L.H * prof_tiles * 64 * L.d * 2  # the profiler's Vt (every frame starts a tile)
    attn_vt_grid = L.nkb * L.H * 256
    alg = {   # algorithmic bytes per launch: what the step must read and write once
        ("layer", "layout_kernel"): 2 * E,
        ("layer", "vt_kernel<128> (attention V^T)"): E + vt_attn,
        ("layer", "vt_kernel<128> (profiler V^T)"): E + vt_prof,
        ("layer", "profile_full_vt<128>"): 2 * E + L.H * L.n_samples * L.d * 2,
        ("svg2", "km_assign_bf3<64>"): EC + C.H * C.N * 4,
        ("svg2", "km_update<unsigned short>"): EC + 2 * C.H * C.N * 4,
        ("svg2", "sort_place"): 2 * C.H * C.N * 4,
        ("svg2", "permute_rows_kernel"): 2 * EC + C.H * C.N * 4,
        ("svg2", "vt_kernel<64> (V gather)"): EC + C.H * -(-C.N // 64) * 64 * C.d * 2 + C.H * C.N * 4,
        ("hva", "hva_assign<64>"): V.H * V.N * V.d * 2 + V.H * V.N * 4,
        ("hva", "vt_kernel<64> (V gather)"): V.H * V.N * V.d * 2 + V.H * -(-V.N // 64) * 64 * V.d * 2 + V.H * V.N * 4,
        ("hva", "permute_rows_kernel"): 2 * V.H * V.N * V.d * 2 + V.H * V.N * 4,
    }

    KMEANS_ROUND_KERNELS = {("svg2", "km_assign_bf3<64>"), ("svg2", "km_update<unsigned short>"),
                            ("svg2", "sort_place"), ("hva", "km_assign_bf3<64>"),
                            ("hva", "km_update<unsigned short>"), ("hva", "sort_place")}
    alg[("hva", "km_assign_bf3<64>")] = V.H * V.N * V.d * 2 + V.H * V.N * 4
    alg[("hva", "km_update<unsigned short>")] = V.H * V.N * V.d * 2 + 2 * V.H * V.N * 4
    alg[("hva", "sort_place")] = 2 * V.H * V.N * 4
    fetch_scale = write_scale = None
    rows = []
    for prog in ("layer", "svg2", "hva"):
        tr = trace(prog)
        fv, fnames, grids = counters(prog, "fetch")
        wv, _, _ = counters(prog, "write")
        sv, _, _ = counters(prog, "sq")
        if prog == "layer":
            copies = [d for d, n in fnames.items() if "layout_kernel" in n]
            fetch_scale = E / (sum(fv[(d, "FETCH_SIZE")] for d in copies) / len(copies) * 1024.0)
            write_scale = E / (sum(wv[(d, "WRITE_SIZE")] for d in copies) / len(copies) * 1024.0)
        groups = defaultdict(list)
        for d, (name, dur) in tr.items():
            k = short(name)
            if k is None or d not in fnames or short(fnames[d]) != k:
                continue
            if k.startswith("vt_kernel"):
                if prog in ("svg2", "hva"):
                    k += " (V gather)"
                else:
                    k += " (attention V^T)" if grids[d] == attn_vt_grid else " (profiler V^T)"
            if (prog, k) in KMEANS_ROUND_KERNELS and fv[(d, "FETCH_SIZE")] * 1024.0 < 0.01 * alg[(prog, k)]:
                k += " (round after the fixed point)"   # the head's kernels returned at once
            groups[k].append((d, dur))
        for k, ds in sorted(groups.items()):
            t = sum(dur for _, dur in ds) / len(ds)
            hbm = sum((fv[(d, "FETCH_SIZE")] * fetch_scale + wv[(d, "WRITE_SIZE")] * write_scale) * 1024.0
                      for d, _ in ds) / len(ds)
            busy = sum(sv.get((d, "SQ_VALU_MFMA_BUSY_CYCLES"), 0.0) for d, _ in ds) / len(ds) / (t * 2.4e9 * 1024)
            rows.append((prog, k, len(ds), t, hbm, alg.get((prog, k)), busy))
    out = os.path.join(ROOT, "profiles", "path_kernels_hbm_mfma.md")
    with open(out, "w") as fh:
        fh.write(COUNTERS_HEADER)
        fh.write("| program | kernel | launches | avg ms | HBM GB / launch | HBM GB/s | algorithmic GB / launch | "
                 "algorithmic GB/s | MFMA busy |\n|---|---|---|---|---|---|---|---|---|\n")
        for prog, k, n, t, hbm, a, busy in rows:
            al = "" if a is None else f"{a / 1e9:.4f}"
            ag = "" if a is None else f"{a / t / 1e9:.0f}"
            fh.write(f"| {prog} | `{k}` | {n} | {t * 1e3:.4f} | {hbm / 1e9:.4f} | {hbm / t / 1e9:.0f} | {al} | {ag} | "
                     f"{busy * 100:.1f}% |\n")
        fh.write(f"\nHBM bytes: FETCH_SIZE x {fetch_scale:.4f} + WRITE_SIZE x {write_scale:.4f} (KiB), the scales "
                 f"taken from the layer program's layout_kernel launches ({E:,} bytes each way).\n")
    print(open(out).read())


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


def bench_svg2(args, steps=None, warmup=None, cpu=False):
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
    vt = torch.empty(svg.svg_vt_elems(H, N, d), dtype=q.dtype, device=dev)
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
        cur = torch.cuda.current_stream()      # the capture stream while a graph is recorded
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(cur)
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
        cur.wait_event(join)
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

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    for _ in range(warmup):
        step_overlapped()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step_overlapped()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / steps
    o_eager, idx_eager = o.clone(), idx.clone()

    def pairs_of(ix):
        # the defined part of pair_idx: each head's first ptr[h][kq] entries
        n = ptr[:, -1].cpu().tolist()
        return torch.cat([ix[h, :n[h]] for h in range(H)])

    def same(a, b, ia, ib):
        return torch.equal(a, b) and torch.equal(pairs_of(ia), pairs_of(ib))

    # The same two-stream step captured once in a HIP graph (its ~70
    # dependent launches, most of them a few microseconds long, then go to
    # the GPU in one submission); the timed steps replay it.  Every replay
    # must give the eager step's output bit for bit.
    graph_note = "the timed step replays a HIP graph of the two-stream step (equal to the eager step bit for bit)"
    try:
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        with torch.cuda.stream(cap):
            step_overlapped()          # warm-up on the capture stream
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=cap):
                step_overlapped()
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        if not same(o, o_eager, idx, idx_eager):
            raise SystemExit("svg2: graph replay and eager step disagree")
        e0.record(stream)
        for _ in range(steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_per_step = e0.elapsed_time(e1) / steps
        if not same(o, o_eager, idx, idx_eager):
            raise SystemExit("svg2: graph replay and eager step disagree")
    except RuntimeError as err:           # capture refused: report the eager step
        torch.cuda.synchronize()
        ms_per_step = eager_ms
        graph_note = f"eager two-stream step (graph capture failed: {err})"
        print(f"[bench] svg2: {graph_note}", file=sys.stderr, flush=True)
    o_overlapped, idx_overlapped = o.clone(), idx.clone()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
    step(ev)
    torch.cuda.synchronize()
    # the two-stream step computes exactly what the one-stream step does
    if not same(o_overlapped, o, idx_overlapped, idx):
        raise SystemExit("svg2: two-stream and one-stream steps disagree")
    stage_ms = {n: ev[j].elapsed_time(ev[j + 1]) for j, n in enumerate(names)}
    # the varlen kernel on the key-tiled V^T (64-key windows with key masks)
    # on the same lists, for comparison (same result up to the bf16 rounding
    # of the accumulation order)
    svg.svg_permute_rows_vt(v, pk, out=vt)
    o_vt = torch.empty_like(o)
    for _ in range(3):
        svg.svg_varlen_attn_vt(qp, kp, vt, oq, ok, ptr, idx, q_perm=pq, out=o_vt)
    e0.record(stream)
    for _ in range(10):
        svg.svg_varlen_attn_vt(qp, kp, vt, oq, ok, ptr, idx, q_perm=pq, out=o_vt)
    e1.record(stream)
    torch.cuda.synchronize()
    vt_ms = e0.elapsed_time(e1) / 10
    vt_diff = (o_vt.float() - o.float()).abs().max().item()
    if not vt_diff < 2e-2:
        raise SystemExit(f"svg2: the two varlen kernels disagree (max abs {vt_diff})")

    # The round of each head's k-means whose assignment equals the previous
    # round's (None: none within the run): from there on the library skips
    # the head's kernels, as every later round would repeat that round.
    def fixed_point_round(x, kc, init):
        prev, r = None, [None] * H
        for n in range(1, w.iters + 1):
            a_ = svg.svg_kmeans(x, kc, n, init)[0].cpu()
            if prev is not None:
                for h in range(H):
                    if r[h] is None and torch.equal(a_[h], prev[h]):
                        r[h] = n - 1
            prev = a_
        return r

    fixed_q, fixed_k = fixed_point_round(q, w.kq, iq), fixed_point_round(k, w.kk, ik)

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
    result = {
        "metric": "SVG2 semantic path ms per step (k-means, cluster sort, gathers, top-p, varlen attention)",
        "value": round(ms_per_step, 4), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded Gaussian mixture)",
        "config": {"workload": w.name, "N": N, "H": H, "d": d, "kq": w.kq, "kk": w.kk, "iters": w.iters,
                   "top_p": w.top_p, "pair_density": round(pairs / (H * float(N) * N), 4)},
        "stage_ms": {kk_: round(vv, 4) for kk_, vv in stage_ms.items()},
        "one_stream_ms": round(sum(stage_ms.values()), 4),
        "eager_two_stream_ms": round(eager_ms, 4),
        "graph": graph_note,
        "varlen_tflops": round(attn_flops / (stage_ms["varlen_attn"] * 1e-3) / 1e12, 2),
        "varlen_vt_windows_kernel_ms": round(vt_ms, 4),
        "varlen_kernels_max_abs_diff": vt_diff,
        "gather_gbs": round(gather_bytes / (stage_ms["gather_qkv"] * 1e-3) / 1e9, 1),
        "kmeans_fixed_point_round": {"q": fixed_q, "k": fixed_k},
        "kmeans_note": (f"{w.iters} Lloyd rounds per head; a head whose assignment stands still (the round above, "
                        "0-based) is at a fixed point and its later rounds' kernels return at once: the outputs "
                        f"are those of all {w.iters} rounds, bit for bit"),
    }
    if cpu:
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
    return result


def layer_bench(args, w, ks, wt, use_vt=True, steps=None, warmup=None, fp8_leg=False, cpu=False, pmc=False):
    """The SVG1 layer step on workload w with mask widths (ks, wt): timed
    steps, per-stage times, the dense baseline, and optionally the same
    step with the FP8 attention.  Returns the result dict (the headline
    fields when w is the default workload)."""
    import numpy as np
    import torch
    from sparse_attention_video_online_amd import svg
    from synth import HUNYUAN_LAYER
    from synth.generators import sample_rows

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
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
    vt = torch.empty(svg.svg_vt_elems(H, N, d), dtype=q.dtype, device=dev) if use_vt else None
    attn_ws = svg.attn_vt_workspace(q, F, S, T, bq, bk) if use_vt else None
    # K's permute: at d = 64 gathered by the attention's tile DMA (the whole
    # CogVideoX-shaped step is ~4% faster so), at d = 128 a separate pass (the
    # gathering kernel's attention is ~1.5% slower there than the permute
    # it saves)
    k_gather = use_vt and d == 64
    stream = torch.cuda.current_stream()
    ev_a0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ev_a1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]

    def attend():
        if k_gather:
            # Q, K read and O written in the original token order (the
            # permutes happen in the kernel's row indexing and tile DMA)
            svg.svg_block_sparse_attn_csr_vt_fused(q, k, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, out=o,
                                                   ws=attn_ws)
        elif use_vt:
            # Q read and O written in the original token order (the Q permute
            # and the O unpermute happen in the kernel's row indexing)
            svg.svg_block_sparse_attn_csr_vt_layout(q, kp, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, out=o,
                                                    ws=attn_ws)
        else:
            svg.svg_block_sparse_attn_csr(qp, kp, vp, row_ptr, kv_idx, F, S, T, bq, bk, out=op,
                                          rowmajor_kernel=True)

    def front(mark):
        svg.svg_profile_heads(q, k, v, sidx, F, S, T, ks, wt, labels=labels, mse=mse, ws=prof_ws)
        mark(1)
        svg.svg_build_block_mask(labels, F, S, T, H, d, ks, wt, bq, bk, out=bmask)
        svg.svg_compact_block_mask(bmask, row_ptr=row_ptr, kv_idx=kv_idx, ws=comp_ws)
        mark(2)

    def step(i=None, stage_events=None):
        def mark(j):
            if stage_events is not None:
                stage_events[j].record(stream)
        mark(0)
        front(mark)
        if not use_vt:
            svg.svg_layout_permute(q, F, S, T, labels, out=qp)
        if not k_gather:
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

    if pmc:
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
        return None

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev_a0, ev_a1)]))
    print(f"[bench] {w.name}: {steps} steps: {ms_per_step:.3f} ms/step (wall {wall:.2f} s), "
          f"attention {attn_ms:.3f} ms", file=sys.stderr, flush=True)

    # per-stage breakdown (one extra step with events between stages)
    se = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    step(None, se)
    torch.cuda.synchronize()
    if k_gather:  # Q, K and O stay in the original order: V into Vt only
        names = ["profile", "mask_and_lists", "permute_vt", "attention"]
    elif use_vt:  # Q and O stay in the original order: permute K and V (into Vt) only
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
    if k_gather:   # the executing-layout K of the last step, for the baseline and the comparison below
        svg.svg_layout_permute(k, F, S, T, labels, out=kp)

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
    print(f"[bench] {w.name}: dense attention {dense_ms:.3f} ms", file=sys.stderr, flush=True)

    # the two forms of K's permute side by side: gathered by the attention's
    # tile DMA (K read from the original rows) and a separate pass before
    # the attention on the permuted copy; the step uses the one k_gather names
    fused = None
    if use_vt:
        o_f = torch.empty_like(q)

        def timed(fn, reps):
            fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps
        reps = max(steps, 2)
        f_ms = timed(lambda: svg.svg_block_sparse_attn_csr_vt_fused(q, k, vt, row_ptr, kv_idx, labels, F, S, T, bq,
                                                                     bk, out=o_f, ws=attn_ws), reps)
        l_ms = timed(lambda: svg.svg_block_sparse_attn_csr_vt_layout(q, kp, vt, row_ptr, kv_idx, labels, F, S, T, bq,
                                                                      bk, out=o_f, ws=attn_ws), reps)
        kperm_ms = timed(lambda: svg.svg_layout_permute(k, F, S, T, labels, out=kp), reps)
        o_l = torch.empty_like(q)
        svg.svg_block_sparse_attn_csr_vt_fused(q, k, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, out=o_f,
                                               ws=attn_ws)
        svg.svg_block_sparse_attn_csr_vt_layout(q, kp, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, out=o_l,
                                                ws=attn_ws)
        torch.cuda.synchronize()
        fused = {"used_in_step": k_gather, "attn_ms": round(f_ms, 4), "layout_attn_ms": round(l_ms, 4),
                 "k_permute_ms": round(kperm_ms, 4), "separate_ms": round(l_ms + kperm_ms, 4),
                 "same_output": bool(torch.equal(o_f.view(torch.int16), o_l.view(torch.int16)))}
        del o_f, o_l
        print(f"[bench] {w.name}: attention with K gathered in the kernel {f_ms:.3f} ms, on the permuted K "
              f"{l_ms:.3f} ms + K permute {kperm_ms:.3f} ms", file=sys.stderr, flush=True)

    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    result = {
        "metric": f"effective block-sparse attn TFLOP/s (whole SVG1 layer step) + speedup vs dense, N={N:,}",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded structured heads; no model weights)",
        "config": {"workload": w.name, "F": F, "S": S, "T": T, "N": N, "N_video": F * S, "H": H, "d": d,
                   "bq": bq, "bk": bk, "ks_frames": ks, "wt_tokens": wt, "n_samples": int(sidx.numel()),
                   "tile_density": round(density, 4), "kept_tiles": tiles,
                   "labels": "".join(str(int(x)) for x in lab_host), "v_layout": "vt" if use_vt else "rowmajor",
                   "qo_layout": "original order, permuted in the attention kernel" if use_vt else "permuted",
                   "k_layout": ("original order, gathered by the attention's tile DMA" if k_gather
                                else "permuted by a separate pass"),
                   "parallelism": "single GPU"},
        "attn_ms": round(attn_ms, 4),
        "attn_tflops": round(attn_tflops, 2),
        "dense_ms": round(dense_ms, 4),
        "dense_tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 2),
        "speedup_vs_dense_attn": round(dense_ms / attn_ms, 3),
        "speedup_vs_dense_layer": round(dense_ms / ms_per_step, 3),
        "stage_ms": {kk: round(vv, 4) for kk, vv in stage_ms.items()},
        "k_gather_fused": fused,
        "roofline": {"bound": "mfma",
                     "kernel": (f"attn_fwd_vt<{d},{bq}>" if use_vt else f"attn_fwd_mfma<{d},{bq}>") + " (block-sparse)",
                     "achieved": round(attn_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": (measured_traffic() if (w is HUNYUAN_LAYER and ks == w.ks and wt == w.wt and use_vt)
                                 else None),
                     "flop_per_launch": flops},
    }

    if fp8_leg and use_vt and d == 128:
        # The same step with the FP8 attention: K quantized in the executing
        # layout (per 64-key block), Q per token in the original order, V^T
        # as before; Q K^T on the FP8 matrix cores, P.V in bf16.
        q8 = torch.empty(H, N, d, dtype=torch.uint8, device=dev)
        k8 = torch.empty(H, N, d, dtype=torch.uint8, device=dev)
        qsc = torch.empty(H, N, dtype=torch.float32, device=dev)
        ksc = torch.empty(H, nkb, dtype=torch.float32, device=dev)
        o8 = torch.empty_like(q)
        f0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        f1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]

        def step8(i=None, stage_events=None):
            def mark(j):
                if stage_events is not None:
                    stage_events[j].record(stream)
            mark(0)
            front(mark)
            svg.svg_layout_permute_fp8(k, F, S, T, labels, out=k8, scale=ksc)
            svg.svg_quantize_fp8_rows(q, out=q8, scale=qsc)
            svg.svg_layout_permute_vt(v, F, S, T, labels, out=vt)
            mark(3)
            if i is not None:
                f0[i].record(stream)
            svg.svg_block_sparse_attn_fp8_vt_layout(q8, qsc, k8, ksc, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk,
                                                    out=o8)
            if i is not None:
                f1[i].record(stream)
            mark(4)

        for _ in range(warmup):
            step8()
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(steps):
            step8(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        ms8 = t_start.elapsed_time(t_end) / steps
        attn8 = float(np.mean([a.elapsed_time(b) for a, b in zip(f0, f1)]))
        step8(None, se)
        torch.cuda.synchronize()
        st8 = {n: se[j].elapsed_time(se[j + 1]) for j, n in
               enumerate(["profile", "mask_and_lists", "quantize_qk_permute_k_vt", "attention"])}
        diff = (o8.float() - o.float())
        result["fp8"] = {
            "qk": "fp8 e4m3 (per-token Q, per-64-key K scales), P.V bf16",
            "ms_per_step": round(ms8, 4), "value": round(flops / (ms8 * 1e-3) / 1e12, 3),
            "attn_ms": round(attn8, 4), "attn_tflops": round(flops / (attn8 * 1e-3) / 1e12, 2),
            "speedup_vs_bf16_attn": round(attn_ms / attn8, 3), "speedup_vs_dense_bf16_attn": round(dense_ms / attn8, 3),
            "stage_ms": {kk: round(vv, 4) for kk, vv in st8.items()},
            "rel_l2_vs_bf16_output": round(float(diff.norm() / o.float().norm()), 4)}
        print(f"[bench] {w.name}: fp8 step {ms8:.3f} ms, fp8 attention {attn8:.3f} ms", file=sys.stderr, flush=True)

        # The FP8 P.V mode: V coded per channel into key-tiled V^T code tiles
        # (instead of the bf16 V^T), probabilities coded after the lazy
        # reference, P.V and the row sum on the FP8 matrix cores.
        vt8 = torch.empty(svg.svg_vt_elems(H, N, d), dtype=torch.uint8, device=dev)
        vam = torch.empty(H, d, dtype=torch.float32, device=dev)
        o8p = torch.empty_like(q)

        def step8p(i=None, stage_events=None):
            def mark(j):
                if stage_events is not None:
                    stage_events[j].record(stream)
            mark(0)
            front(mark)
            svg.svg_layout_permute_fp8(k, F, S, T, labels, out=k8, scale=ksc)
            svg.svg_quantize_fp8_rows(q, out=q8, scale=qsc)
            svg.svg_layout_permute_vt_fp8(v, F, S, T, labels, out=vt8, amax=vam)
            mark(3)
            if i is not None:
                f0[i].record(stream)
            svg.svg_block_sparse_attn_fp8pv_vt_layout(q8, qsc, k8, ksc, vt8, vam, row_ptr, kv_idx, labels, F, S, T,
                                                      bq, bk, out=o8p)
            if i is not None:
                f1[i].record(stream)
            mark(4)

        for _ in range(warmup):
            step8p()
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(steps):
            step8p(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        ms8p = t_start.elapsed_time(t_end) / steps
        attn8p = float(np.mean([a.elapsed_time(b) for a, b in zip(f0, f1)]))
        step8p(None, se)
        torch.cuda.synchronize()
        st8p = {n: se[j].elapsed_time(se[j + 1]) for j, n in
                enumerate(["profile", "mask_and_lists", "quantize_qkv_permute_k_vt", "attention"])}
        diffp = (o8p.float() - o.float())
        result["fp8"]["pv"] = {
            "mode": "fp8 e4m3 Q K^T as above; V per-channel codes, P coded after the lazy reference, P.V fp8",
            "ms_per_step": round(ms8p, 4), "value": round(flops / (ms8p * 1e-3) / 1e12, 3),
            "attn_ms": round(attn8p, 4), "attn_tflops": round(flops / (attn8p * 1e-3) / 1e12, 2),
            "speedup_vs_bf16_attn": round(attn_ms / attn8p, 3),
            "speedup_vs_dense_bf16_attn": round(dense_ms / attn8p, 3),
            "stage_ms": {kk: round(vv, 4) for kk, vv in st8p.items()},
            "rel_l2_vs_bf16_output": round(float(diffp.norm() / o.float().norm()), 4)}
        del vt8, o8p
        print(f"[bench] {w.name}: fp8 P.V step {ms8p:.3f} ms, attention {attn8p:.3f} ms", file=sys.stderr,
              flush=True)
    if fp8_leg and use_vt:
        # The same step with SVG-EAR: block statistics of K / V^T, routing of
        # EAR_ROUTE_K skipped blocks per q-block into the exact sets, their
        # lists, and the attention with the centroid compensation of every
        # other block.  Also the distance of both outputs to dense attention
        # on the same tensors (what the compensation is for).
        exm = torch.empty(H, nqb, nkb, dtype=torch.uint8, device=dev)
        ne = svg.svg_ear_centroid_elems(H, N, d)
        kc = torch.empty(ne, dtype=torch.bfloat16, device=dev)
        vct = torch.empty(ne, dtype=torch.bfloat16, device=dev)
        kbar = torch.empty(H, d, nkb, dtype=torch.float64, device=dev)
        rad = torch.empty(H, nkb, dtype=torch.float64, device=dev)
        oe = torch.empty_like(q)
        g0 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        g1 = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]

        def step_ear(i=None, stage_events=None):
            def mark(j):
                if stage_events is not None:
                    stage_events[j].record(stream)
            mark(0)
            svg.svg_profile_heads(q, k, v, sidx, F, S, T, ks, wt, labels=labels, mse=mse, ws=prof_ws)
            svg.svg_build_block_mask(labels, F, S, T, H, d, ks, wt, bq, bk, out=bmask)
            svg.svg_layout_permute(k, F, S, T, labels, out=kp)
            svg.svg_layout_permute_vt(v, F, S, T, labels, out=vt)
            mark(1)
            svg.svg_ear_block_stats(kp, vt, F, S, T, kc=kc, vct=vct, kbar=kbar, radius=rad)
            mark(2)
            svg.svg_ear_route(q, labels, kbar, rad, bmask, F, S, T, bq, bk, EAR_ROUTE_K, out=exm)
            svg.svg_compact_block_mask(exm, row_ptr=row_ptr, kv_idx=kv_idx, ws=comp_ws)
            mark(3)
            if i is not None:
                g0[i].record(stream)
            svg.svg_block_sparse_attn_ear_vt_layout(q, kp, vt, kc, vct, row_ptr, kv_idx, labels, F, S, T, bq, bk,
                                                    out=oe)
            if i is not None:
                g1[i].record(stream)
            mark(4)

        for _ in range(warmup):
            step_ear()
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(steps):
            step_ear(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        mse_ = t_start.elapsed_time(t_end) / steps
        attn_e = float(np.mean([a.elapsed_time(b) for a, b in zip(g0, g1)]))
        step_ear(None, se)
        torch.cuda.synchronize()
        ste = {n: se[j].elapsed_time(se[j + 1]) for j, n in
               enumerate(["profile_masks_layouts", "block_stats", "route_and_lists", "attention"])}
        # o still holds the SVG1 output of the staged step above
        dn = dense.float().norm()
        result["ear"] = {
            "route_k": EAR_ROUTE_K, "ms_per_step": round(mse_, 4), "attn_ms": round(attn_e, 4),
            "exact_tile_density": round(float(exm.float().mean()), 4),
            "stage_ms": {kk: round(vv, 4) for kk, vv in ste.items()},
            "rel_l2_vs_dense": round(float((oe.float() - dense.float()).norm() / dn), 5),
            "svg1_rel_l2_vs_dense": round(float((o.float() - dense.float()).norm() / dn), 5)}
        print(f"[bench] {w.name}: ear step {mse_:.3f} ms, ear attention {attn_e:.3f} ms", file=sys.stderr, flush=True)
    if cpu:
        result["cpu_baseline"] = cpu_baseline(w, ks, wt, lab_host, args.cpu_seconds)
    return result


def bench_hva(args, steps=None, warmup=None):
    """HVA-style clustering in the SVG2 step, on the CogVideoX-shaped blob
    workload (13 x 1350 + 224 tokens, 8 heads, d = 64, bf16; windows of
    4 x 10 x 15 tokens for Q (36 + 1 clusters) and 2 x 6 x 9 for K (175 + 1),
    10 iterations, top-p 0.9).  Anchor step = local-window clustering of Q
    and K, cluster sort, gathers of Q, K and V, top-p pairs, varlen attention;
    refresh step = the same with the Lowe-flagged subset re-assigned on the
    next step's values instead of a full clustering.  Both run the key chain
    on a second stream.  For comparison: SVG2 k-means with as many clusters
    (from one seed token per window) on the same tensors, its clustering
    time and objective at 10 and 50 iterations, and each path's output
    against dense attention."""
    import numpy as np
    import torch
    from sparse_attention_video_online_amd import svg
    from synth import HVA_COG as w
    from synth.generators import blob_qkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rows, cols = w.grid
    H, N, d = w.H, w.N, w.d
    up = lambda x: torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    g0, g1 = blob_qkv(w, step=0), blob_qkv(w, step=1)
    q0, k0, v = up(g0["q"]), up(g0["k"]), up(g0["v"])
    q1, k1 = up(g1["q"]), up(g1["k"])
    kq = svg.svg_hva_clusters(w.F, rows, cols, w.T, w.win_q, H, d)
    kk = svg.svg_hva_clusters(w.F, rows, cols, w.T, w.win_k, H, d)
    i32 = lambda *sh: torch.empty(*sh, dtype=torch.int32, device=dev)
    aq, ak = i32(H, N), i32(H, N)
    cq = torch.empty(H, kq, d, dtype=torch.float64, device=dev)
    ck = torch.empty(H, kk, d, dtype=torch.float64, device=dev)
    sq, sk = i32(H, kq), i32(H, kk)
    rq, rk = (torch.empty(H, N, dtype=torch.uint8, device=dev) for _ in range(2))
    pq, pk, oq, ok = i32(H, N), i32(H, N), i32(H, kq + 1), i32(H, kk + 1)
    ptr, idx = i32(H, kq + 1), i32(H, kq * kk)
    qp, kp, vp, o = (torch.empty_like(q0) for _ in range(4))
    dm = svg.svg_dims(w.F, w.S, w.T, H, d)
    ws = lambda n: torch.empty(max(1, n), dtype=torch.uint8, device=dev)
    ws_q, ws_k = ws(svg.workspace_bytes(svg.SVG2_OP_HVA, dm, kq, svg2=True)), \
        ws(svg.workspace_bytes(svg.SVG2_OP_HVA, dm, kk, svg2=True))
    ws_c1, ws_c2 = (ws(svg.workspace_bytes(svg.SVG2_OP_CLUSTER_PERMUTE, dm, max(kq, kk), svg2=True))
                    for _ in range(2))
    side = torch.cuda.Stream()
    stream = torch.cuda.current_stream()

    def attention_tail(q, k):
        svg.svg_select_pairs(cq, ck, sk, w.top_p, pair_ptr=ptr, pair_idx=idx)
        svg.svg_varlen_attn(qp, kp, vp, oq, ok, ptr, idx, q_perm=pq, out=o)

    def step(anchor):
        q, k = (q0, k0) if anchor else (q1, k1)
        cur = torch.cuda.current_stream()
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(cur)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            if anchor:
                svg.svg_hva_cluster(k, w.F, rows, cols, w.T, w.win_k, w.iters, assign=ak, centroids=ck, sizes=sk,
                                    refresh=rk, ws=ws_k)
            else:
                svg.svg_hva_refresh(k, w.F, rows, cols, w.T, w.win_k, rk, ak, ck, sizes=sk, ws=ws_k)
            svg.svg_cluster_permute(ak, kk, d, perm=pk, offs=ok, ws=ws_c2)
            svg.svg_permute_rows(k, pk, out=kp)
            svg.svg_permute_rows(v, pk, out=vp)
            join.record(side)
        if anchor:
            svg.svg_hva_cluster(q, w.F, rows, cols, w.T, w.win_q, w.iters, assign=aq, centroids=cq, sizes=sq,
                                refresh=rq, ws=ws_q)
        else:
            svg.svg_hva_refresh(q, w.F, rows, cols, w.T, w.win_q, rq, aq, cq, sizes=sq, ws=ws_q)
        svg.svg_cluster_permute(aq, kq, d, perm=pq, offs=oq, ws=ws_c1)
        svg.svg_permute_rows(q, pq, out=qp)
        cur.wait_event(join)
        attention_tail(q, k)

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup

    def timed(fn, n, reps_warm):
        for _ in range(reps_warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # an anchor step, then refresh steps from its state (the refresh reads and
    # writes the carried clusters, so each timed refresh starts from the last)
    anchor_ms = timed(lambda: step(True), steps, warmup)
    o_anchor = o.clone()
    lists_anchor = [t.clone() for t in (ptr, idx, oq, ok)]
    state = [t.clone() for t in (aq, cq, ak, ck)]
    refresh_ms = timed(lambda: step(False), steps, warmup)
    for t, s_ in zip((aq, cq, ak, ck), state):
        t.copy_(s_)
    # clustering alone, one stream
    clus = {
        "hva_anchor_q": timed(lambda: svg.svg_hva_cluster(q0, w.F, rows, cols, w.T, w.win_q, w.iters, assign=aq,
                                                          centroids=cq, sizes=sq, refresh=rq, ws=ws_q), steps, 2),
        "hva_anchor_k": timed(lambda: svg.svg_hva_cluster(k0, w.F, rows, cols, w.T, w.win_k, w.iters, assign=ak,
                                                          centroids=ck, sizes=sk, refresh=rk, ws=ws_k), steps, 2),
    }
    a_q, c_q, a_k, c_k = aq.clone(), cq.clone(), ak.clone(), ck.clone()
    flag_frac = {"q": float(rq.float().mean()), "k": float(rk.float().mean())}
    # (each call refreshes the state the previous one left: same work)
    clus["hva_refresh_q"] = timed(lambda: svg.svg_hva_refresh(q1, w.F, rows, cols, w.T, w.win_q, rq, aq, cq,
                                                               sizes=sq, ws=ws_q), steps, 2)
    clus["hva_refresh_k"] = timed(lambda: svg.svg_hva_refresh(k1, w.F, rows, cols, w.T, w.win_k, rk, ak, ck,
                                                               sizes=sk, ws=ws_k), steps, 2)

    # objective per token (float64, mean squared distance to the centroid)
    def sse(x, a, c):
        xf = x.double()
        return float(((xf - torch.gather(c, 1, a.long()[..., None].expand(-1, -1, d))) ** 2).sum() / (H * N))

    # SVG2 k-means on the same tensors, as many clusters, one seed token per
    # window (its first token) and the text cluster's first token
    def window_seeds(win):
        wf, wy, wx = win
        first = [(a * wf) * w.S + (b * wy) * cols + c * wx
                 for a in range(-(-w.F // wf)) for b in range(-(-rows // wy)) for c in range(-(-cols // wx))]
        if w.T:
            first.append(w.F * w.S)
        return torch.tensor([first] * H, dtype=torch.int32, device=dev)

    km, kmc = {}, {}
    for name, x, win, kc, a_h, c_h in (("q", q0, w.win_q, kq, a_q, c_q), ("k", k0, w.win_k, kk, a_k, c_k)):
        seeds = window_seeds(win)
        r = {"hva_sse": sse(x, a_h, c_h)}
        for it in (50, w.iters):
            a_, c_, s_ = svg.svg_kmeans(x, kc, it, seeds)
            r[f"kmeans{it}_sse"] = sse(x, a_, c_)
        kmc[name] = (a_, c_, s_)                # 10 iterations, for the attention below
        r["kmeans_ms"] = timed(lambda: svg.svg_kmeans(x, kc, w.iters, seeds), steps, 2)
        km[name] = r
    # the same attention tail over the k-means clusters
    (ka, kc_, ks), (kka, kkc, kks) = kmc["q"], kmc["k"]
    kpq, koq = svg.svg_cluster_permute(ka, kq, d)
    kpk, kok = svg.svg_cluster_permute(kka, kk, d)
    kptr, kidx = svg.svg_select_pairs(kc_, kkc, kks, w.top_p)
    o_km = svg.svg_varlen_attn(svg.svg_permute_rows(q0, kpq), svg.svg_permute_rows(k0, kpk),
                               svg.svg_permute_rows(v, kpk), koq, kok, kptr, kidx, q_perm=kpq)

    # attention quality: each path's output against dense attention
    vt_id = svg.svg_layout_permute_vt(v, 1, N, 0, torch.zeros(H, dtype=torch.int32, device=dev))
    dense = svg.svg_dense_attn_vt(q0, k0, vt_id, 1, N, 0, 64, 64)
    rel = lambda a, b: float((a.float() - b.float()).norm() / b.float().norm())

    def pair_density(p_, i_, qo, ko):
        # selected (query, key) token pairs over H N^2
        p_, i_ = p_.cpu().numpy(), i_.cpu().numpy()
        qs, ks_ = np.diff(qo.cpu().numpy(), axis=1), np.diff(ko.cpu().numpy(), axis=1)
        tot = sum(int(qs[h, i]) * int(ks_[h, i_[h, p_[h, i]:p_[h, i + 1]]].sum())
                  for h in range(H) for i in range(p_.shape[1] - 1))
        return tot / (H * float(N) * N)
    torch.cuda.synchronize()
    return {
        "workload": w.name, "kq": kq, "kk": kk, "iters": w.iters,
        "anchor_step_ms": round(anchor_ms, 4), "refresh_step_ms": round(refresh_ms, 4),
        "clustering_ms": {k_: round(v_, 4) for k_, v_ in clus.items()},
        "kmeans_same_k_ms": {"q": round(km["q"]["kmeans_ms"], 4), "k": round(km["k"]["kmeans_ms"], 4)},
        "refresh_fraction": {k_: round(v_, 4) for k_, v_ in flag_frac.items()},
        "sse_per_token": {s_: {k_: round(v_, 3) for k_, v_ in km[s_].items() if k_.endswith("sse")} for s_ in km},
        "rel_l2_vs_dense": round(rel(o_anchor, dense), 5),
        "kmeans_rel_l2_vs_dense": round(rel(o_km, dense), 5),
        "pair_density": round(pair_density(*lists_anchor), 4),
        "kmeans_pair_density": round(pair_density(kptr, kidx, koq, kok), 4),
    }


def main():
    args = parse()
    if args.record_traffic:
        return record_traffic(*args.record_traffic)
    if args.record_counters:
        return record_counters(args.record_counters)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the path shards by head "
              f"with no exchange, see the design notes.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "svg2":
        print(json.dumps(bench_svg2(args, cpu=not args.no_cpu_baseline)), flush=True)
        return
    if args.workload == "hva":
        print(json.dumps(bench_hva(args)), flush=True)
        return

    from synth import COG, HUNYUAN_LAYER
    from synth.configs import HUNYUAN_DENSITY_POINTS

    use_vt = args.v_layout == "vt"
    if args.workload == "cogvideox_shape":
        result = layer_bench(args, COG, COG.ks, COG.wt, use_vt, cpu=not args.no_cpu_baseline, pmc=args.pmc_target)
        if result is not None:
            print(json.dumps(result), flush=True)
        return
    ks, wt = HUNYUAN_DENSITY_POINTS[args.density]
    default = args.density == "k5" and use_vt and not args.pmc_target
    result = layer_bench(args, HUNYUAN_LAYER, ks, wt, use_vt, fp8_leg=default and not args.no_extra,
                         pmc=args.pmc_target)
    if result is None:
        return
    if default and not args.no_extra:
        # the other two workloads of the path, for the record: the
        # CogVideoX-shaped layer step and the SVG2 semantic path
        import torch
        torch.cuda.empty_cache()
        cog = layer_bench(args, COG, COG.ks, COG.wt, True, steps=20, warmup=3)
        result["cogvideox_shape"] = {k_: cog[k_] for k_ in ("ms_per_step", "value", "attn_ms", "attn_tflops",
                                                             "dense_ms", "speedup_vs_dense_attn", "stage_ms",
                                                             "k_gather_fused")}
        result["cogvideox_shape"]["tile_density"] = cog["config"]["tile_density"]
        torch.cuda.empty_cache()
        s2 = bench_svg2(args, steps=20, warmup=3)
        result["svg2"] = {k_: s2[k_] for k_ in ("ms_per_step", "stage_ms", "one_stream_ms", "eager_two_stream_ms",
                                                 "varlen_tflops", "gather_gbs", "kmeans_fixed_point_round")}
        result["svg2"]["pair_density"] = s2["config"]["pair_density"]
        torch.cuda.empty_cache()
        result["hva"] = bench_hva(args, steps=20, warmup=3)
    if not args.no_cpu_baseline:
        lab = [int(c) for c in result["config"]["labels"]]
        result["cpu_baseline"] = cpu_baseline(HUNYUAN_LAYER, ks, wt, lab, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
