"""Pins for the oracle's token masks, block bitmaps, lists and layout (CPU only).

Every check comes from outside the oracle's own code: hand-enumerated masks
and permutations under tests/golden/, counts derived by hand, and the
element-wise bitmap against the range form on several shapes.
"""

import json
import os

import numpy as np
import pytest

from conftest import GOLDEN
from oracle import masks, layout
from synth import TINY, COG, HUNYUAN


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_token_masks_match_hand_enumeration():
    g = load("masks_small.json")
    F, S, T = g["F"], g["S"], g["T"]
    i = np.arange(F * S + T)[:, None]
    j = np.arange(F * S + T)[None, :]
    np.testing.assert_array_equal(masks.spatial_keep(i, j, F, S, g["ks"]).astype(int), g["spatial"])
    np.testing.assert_array_equal(masks.temporal_keep(i, j, F, S, g["wt"]).astype(int), g["temporal"])


@pytest.mark.parametrize("F,S,T,ks,wt", [(4, 64, 16, 0, 32), (5, 7, 3, 1, 4), (13, 30, 9, 2, 40), (3, 11, 0, 0, 0)])
def test_per_query_kept_counts(F, S, T, ks, wt):
    """Spatial: (frames within ks, clipped) * S + T.  Temporal: the widened
    own-position run clipped to [0, FS), plus T.  Text queries keep N."""
    N = F * S + T
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    cs = masks.spatial_keep(i, j, F, S, ks).sum(axis=1)
    ct = masks.temporal_keep(i, j, F, S, wt).sum(axis=1)
    for t in range(N):
        if t >= F * S:
            assert cs[t] == N and ct[t] == N
            continue
        f, p = t // S, t % S
        frames = min(F - 1, f + ks) - max(0, f - ks) + 1
        assert cs[t] == frames * S + T
        lo, hi = max(0, p * F - wt), min(F * S - 1, p * F + F - 1 + wt)
        assert ct[t] == hi - lo + 1 + T


def test_tiny_bitmap_counts_by_hand():
    """Tiny (F=4, S=64, T=16, 16x16 tiles).  Spatial, own frame: each video
    q-block keeps its frame's S/bk = 4 blocks and the one text block; the text
    q-block keeps all 17: 16*5 + 17 = 97.  Temporal (position-major, wt=32):
    q-block qb spans positions 4qb..4qb+3, its rows keep keys
    [max(0,16qb-32), min(256, 16qb+48)), i.e. blocks max(0,qb-2)..min(15,qb+2),
    plus the text block; the text q-block keeps all 17: 4+5+12*6+5+4+17 = 107."""
    w = TINY
    bs = masks.block_bitmap(0, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
    bt = masks.block_bitmap(1, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
    assert bs.shape == (17, 17)
    assert bs.sum() == 97 and bt.sum() == 107
    for qb in range(16):
        f = qb // 4
        expect = np.zeros(17, dtype=np.uint8)
        expect[4 * f:4 * f + 4] = 1
        expect[16] = 1
        np.testing.assert_array_equal(bs[qb], expect)
        expect = np.zeros(17, dtype=np.uint8)
        expect[max(0, qb - 2):min(15, qb + 2) + 1] = 1
        expect[16] = 1
        np.testing.assert_array_equal(bt[qb], expect)
    assert bs[16].all() and bt[16].all()


@pytest.mark.parametrize("F,S,T,ks,wt,bq,bk", [
    (4, 64, 16, 0, 32, 16, 16), (5, 7, 3, 1, 4, 4, 8), (6, 13, 10, 0, 9, 8, 8),
    (3, 40, 0, 2, 30, 16, 32), (7, 9, 5, 0, 0, 16, 4), (2, 50, 17, 1, 120, 32, 16)])
def test_range_form_equals_elementwise(F, S, T, ks, wt, bq, bk):
    for label in (0, 1):
        a = masks.block_bitmap(label, F, S, T, ks, wt, bq, bk)
        b = masks.block_bitmap_ranges(label, F, S, T, ks, wt, bq, bk)
        np.testing.assert_array_equal(a, b)


def test_range_form_equals_elementwise_cogvideox_shape():
    w = COG
    for label in (0, 1):
        a = masks.block_bitmap(label, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
        b = masks.block_bitmap_ranges(label, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
        np.testing.assert_array_equal(a, b)


def test_hunyuan_shape_density_and_sampled_rows():
    """At 33 x 3600 + 256 with ks = 5 and wt = 19800 the two patterns keep ~31%
    of the 128 x 64 tiles; sampled rows (first, tail, text) match the
    element-wise definition."""
    w = HUNYUAN
    for label in (0, 1):
        b = masks.block_bitmap_ranges(label, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk)
        assert b.shape == (931, 1861)
        assert 0.30 < b.mean() < 0.32
        rows = [0, 27, 28, 464, 927, 928, 929, 930]
        e = masks.block_bitmap(label, w.F, w.S, w.T, w.ks, w.wt, w.bq, w.bk, qblocks=rows)
        np.testing.assert_array_equal(e, b[rows])
        assert b[930].all()                    # text-only q-block keeps all


def test_compact_csr():
    bm = np.array([[1, 0, 1, 1], [0, 0, 0, 0], [0, 1, 0, 0]], dtype=np.uint8)
    ptr, idx = masks.compact(bm)
    np.testing.assert_array_equal(ptr, [0, 3, 3, 4])
    np.testing.assert_array_equal(idx, [0, 2, 3, 1])


def test_valid_pairs_with_tails():
    bm = np.ones((3, 2), dtype=np.uint8)       # N = 10, bq = 4 (rows 4,4,2), bk = 8 (cols 8,2)
    assert masks.valid_pairs(bm, 10, 4, 8) == 100
    bm[2, 0] = 0
    assert masks.valid_pairs(bm, 10, 4, 8) == 100 - 2 * 8


def test_permute_hand_example():
    g = load("permute_small.json")
    F, S, T = g["F"], g["S"], g["T"]
    np.testing.assert_array_equal(masks.position_major_index(F, S, T), g["executing_index_of_original"])
    x = np.arange(F * S + T, dtype=np.float64)[None, :, None] * np.ones((2, 1, 3))
    y = layout.permute(x, F, S, T, [0, 1])
    np.testing.assert_array_equal(y[0, :, 0], np.arange(F * S + T))        # spatial head copied
    np.testing.assert_array_equal(y[1, :, 0], g["original_at_executing_position"])


@pytest.mark.parametrize("F,S,T", [(4, 64, 16), (1, 9, 3), (7, 1, 2), (13, 30, 0)])
def test_unpermute_inverts_permute(F, S, T):
    rng = np.random.default_rng(F * 100 + S)
    x = rng.standard_normal((3, F * S + T, 4))
    labels = [1, 0, 1]
    y = layout.permute(x, F, S, T, labels)
    np.testing.assert_array_equal(layout.unpermute(y, F, S, T, labels), x)
    if F == 1 or S == 1:
        np.testing.assert_array_equal(y, x)    # one frame or one position: identity
    else:
        assert not np.array_equal(y[0], x[0])
    np.testing.assert_array_equal(y[1], x[1])


def test_temporal_pattern_is_banded_after_permute():
    """In the executing layout each video row of a temporal head keeps one
    contiguous range of video keys (plus text)."""
    F, S, T, wt = 5, 12, 4, 7
    N = F * S + T
    inv = masks.executing_to_original(1, F, S, T)
    keep = masks.temporal_keep(inv[:, None], inv[None, :], F, S, wt)
    lo, hi = masks.row_kept_ranges(1, F, S, T, 0, wt)
    for x in range(F * S):
        cols = np.flatnonzero(keep[x, :F * S])
        assert cols[0] == lo[x] and cols[-1] == hi[x] - 1 and cols.size == hi[x] - lo[x]
