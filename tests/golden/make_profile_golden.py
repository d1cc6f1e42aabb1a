"""Writes the oracle's head-profiling result for the HunyuanVideo-shaped layer
workload (33 x 3600 video + 256 text tokens, 24 heads, d = 128, 1191 sampled
rows) to hunyuan_layer_profile.json.

It calls only the oracle and the seeded generators.  The oracle needs a few
minutes on 8 cores, so the GPU tests read the stored result instead of
recomputing it.  Re-run after any change to the oracle's profiling, the masks
or the generator:

    python tests/golden/make_profile_golden.py
"""

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from synth import HUNYUAN_LAYER  # noqa: E402
from synth.generators import structured_qkv, sample_rows  # noqa: E402
from oracle import profile, numerics  # noqa: E402

AMBIGUOUS_RATIO = 0.9


def main():
    w = HUNYUAN_LAYER
    si = sample_rows(w)
    out = dict(workload=w.name, seed=w.seed, n_samples=int(si.size), ks=w.ks, wt=w.wt,
               ambiguous_ratio=AMBIGUOUS_RATIO, heads=[])
    t0 = time.time()
    for h in range(w.H):
        g = structured_qkv(w, heads=[h])
        q, k, v = (numerics.as_f64(g[x], w.dtype)[0] for x in "qkv")
        lab, ms, mt = profile.profile_head(q, k, v, w.F, w.S, w.T, si, w.ks, w.wt)
        ratio = min(ms, mt) / max(ms, mt) if max(ms, mt) > 0 else 1.0
        out["heads"].append(dict(head=h, kind=int(g["kinds"][0]), scale=float(g["scales"][0]),
                                 label=int(lab), mse_spatial=ms, mse_temporal=mt,
                                 ratio=ratio, ambiguous=bool(ratio > AMBIGUOUS_RATIO)))
        print(f"head {h}: label {lab} mse_s {ms:.6e} mse_t {mt:.6e} ratio {ratio:.4f} "
              f"({time.time() - t0:.0f}s)", flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hunyuan_layer_profile.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
