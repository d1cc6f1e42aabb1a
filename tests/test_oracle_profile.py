"""Pins for the oracle's head profiling (CPU only).

* K = 0 closed form: each masked output is the plain mean of V over the
  mask's keys, so both MSEs have values computed here with no softmax.
* Masks that keep everything give MSE 0, and the tie goes to spatial.
* Heads built with a known structure get that label, by a clear margin.
"""

import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import profile, masks, numerics
from synth import TINY, COG
from synth.generators import structured_qkv, sample_rows, generator_labels


def test_k_zero_closed_form():
    F, S, T, ks, wt = 4, 6, 3, 0, 2
    N, d = F * S + T, 5
    rng = np.random.default_rng(11)
    q = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    rows = np.array([0, 5, 7, 13, 22, 25])
    lab, ms, mt = profile.profile_head(q, np.zeros((N, d)), v, F, S, T, rows, ks, wt)
    full = v.mean(axis=0)
    se_s = se_t = 0.0
    for i in rows:
        keys_s = [j for j in range(N) if j >= F * S or i >= F * S or abs(j // S - i // S) <= ks]
        p = i % S
        keys_t = [j for j in range(N)
                  if j >= F * S or i >= F * S or p * F - wt <= (j % S) * F + j // S <= p * F + F - 1 + wt]
        se_s += ((v[keys_s].mean(axis=0) - full) ** 2).sum()
        se_t += ((v[keys_t].mean(axis=0) - full) ** 2).sum()
    assert ms == pytest.approx(se_s / (rows.size * d), rel=1e-12)
    assert mt == pytest.approx(se_t / (rows.size * d), rel=1e-12)
    assert lab == (0 if ms <= mt else 1)


def test_full_masks_tie_goes_to_spatial():
    F, S, T = 3, 5, 2
    N, d = F * S + T, 4
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    lab, ms, mt = profile.profile_head(q, k, v, F, S, T, np.arange(N), ks=F, wt=F * S)
    assert ms == 0.0 and mt == 0.0 and lab == 0


def test_text_rows_do_not_contribute():
    F, S, T = 3, 5, 4
    N, d = F * S + T, 4
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    lab, ms, mt = profile.profile_head(q, k, v, F, S, T, np.arange(F * S, N), ks=0, wt=0)
    assert ms == 0.0 and mt == 0.0


@pytest.mark.parametrize("w", [TINY, COG], ids=lambda w: w.name)
def test_generated_heads_get_their_label_with_margin(w):
    g = structured_qkv(w)
    q, k, v = (numerics.as_f64(g[x], w.dtype) for x in "qkv")
    si = sample_rows(w)
    assert si.size == w.n_samples and np.all(np.diff(si) > 0)
    labels, mse = profile.profile_heads(q, k, v, w.F, w.S, w.T, si, w.ks, w.wt)
    np.testing.assert_array_equal(labels, generator_labels(w))
    ratio = mse.min(axis=1) / mse.max(axis=1)
    assert np.all(ratio <= 0.9), ratio         # decided heads (clear margins)


def test_hunyuan_layer_golden_is_consistent():
    """The stored profile of the HunyuanVideo-shaped layer workload: heads
    generated purely spatial (temporal) at scale >= 1 get label 0 (1), and at
    least one head is decided per label.  (The file is written by
    tests/golden/make_profile_golden.py from the oracle.)"""
    path = os.path.join(GOLDEN, "hunyuan_layer_profile.json")
    if not os.path.exists(path):
        pytest.skip("golden profile not generated")
    with open(path) as f:
        g = json.load(f)
    assert len(g["heads"]) == 24
    for h in g["heads"]:
        ratio = min(h["mse_spatial"], h["mse_temporal"]) / max(h["mse_spatial"], h["mse_temporal"])
        assert ratio == pytest.approx(h["ratio"])
        assert h["label"] == (0 if h["mse_spatial"] <= h["mse_temporal"] else 1)
        if h["kind"] in (0, 1) and h["scale"] >= 1.0:
            assert h["label"] == h["kind"] and not h["ambiguous"]
    labels = [h["label"] for h in g["heads"] if not h["ambiguous"]]
    assert 0 in labels and 1 in labels
