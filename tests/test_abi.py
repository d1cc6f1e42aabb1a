"""The C ABI library loads, exports every function include/*.h declares, and
rejects bad arguments on the host with the documented status (CPU only: every
call here returns from host validation before any HIP call)."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")


def declared_functions():
    names = []
    for h in ("svg.h", "svg2.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(svg2?_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "svg_block_sparse_attn" in names and "svg_varlen_attn" in names and len(names) >= 17
    lib = ctypes.CDLL(svg.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) <= set(svg.SIGNATURES), set(names) - set(svg.SIGNATURES)


def test_version_string():
    assert b"gfx950" in svg.lib().svg_version()


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE2 = ctypes.c_void_p(0x20000000)
FAKE3 = ctypes.c_void_p(0x40000000)


def dims(F=4, S=64, T=16, H=2, d=64):
    return ctypes.byref(svg.svg_dims(F, S, T, H, d))


def status(name, *args):
    return getattr(svg.lib(), name)(*args)


def test_null_and_shape_errors():
    L = svg.lib()
    assert L.svg_dense_attn(None, 0, FAKE, FAKE, FAKE, 16, 16, -1.0, FAKE2, None) == svg.SVG_ERR_NULL
    assert "dims" in svg.last_error()
    assert L.svg_dense_attn(dims(), 0, None, FAKE, FAKE, 16, 16, -1.0, FAKE2, None) == svg.SVG_ERR_NULL
    assert L.svg_dense_attn(dims(d=96), 0, FAKE, FAKE, FAKE, 16, 16, -1.0, FAKE2, None) == svg.SVG_ERR_UNSUPPORTED
    assert L.svg_dense_attn(dims(H=0), 0, FAKE, FAKE, FAKE, 16, 16, -1.0, FAKE2, None) == svg.SVG_ERR_SHAPE
    assert L.svg_dense_attn(dims(), 7, FAKE, FAKE, FAKE, 16, 16, -1.0, FAKE2, None) == svg.SVG_ERR_DTYPE
    assert L.svg_dense_attn(dims(), 0, FAKE, FAKE, FAKE, 32, 32, -1.0, FAKE2, None) == svg.SVG_ERR_UNSUPPORTED
    assert "block shape" in svg.last_error()


def test_aliasing_and_workspace_errors():
    L = svg.lib()
    assert L.svg_dense_attn(dims(), 0, FAKE, FAKE2, FAKE2, 16, 16, -1.0, FAKE, None) == svg.SVG_ERR_RANGE
    assert L.svg_layout_permute(dims(), 1, FAKE, FAKE, None, None) == svg.SVG_ERR_RANGE
    mp = svg.svg_mask_params(0, 32)
    assert L.svg_profile_heads(dims(), 0, FAKE, FAKE, FAKE, FAKE, 8, ctypes.byref(mp), -1.0, FAKE2, None,
                               FAKE2, 16, None) == svg.SVG_ERR_WORKSPACE
    assert L.svg_profile_heads(dims(), 0, FAKE, FAKE, FAKE, FAKE, 0, ctypes.byref(mp), -1.0, FAKE2, None,
                               FAKE2, 1 << 30, None) == svg.SVG_ERR_RANGE
    bad = svg.svg_mask_params(-1, 0)
    assert L.svg_build_block_mask(dims(), ctypes.byref(bad), FAKE, 16, 16, FAKE2, None) == svg.SVG_ERR_RANGE
    assert L.svg_block_sparse_attn(dims(), 0, FAKE, FAKE, FAKE, FAKE, 16, 16, -1.0, FAKE2, FAKE2, 8, None) \
        == svg.SVG_ERR_WORKSPACE
    assert L.svg_compact_block_mask(10, 0, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == svg.SVG_ERR_SHAPE


def test_workspace_sizes():
    L = svg.lib()
    d = dims(F=13, S=1350, T=224, H=8, d=64)
    ws = L.svg_workspace_bytes(svg.SVG_OP_BLOCK_SPARSE, d, 64, 64)
    rows, nkb = 8 * 278, 278
    assert ws >= rows * 4 + (rows + 1) * 4 + rows * nkb * 4
    assert L.svg_workspace_bytes(svg.SVG_OP_BLOCK_SPARSE, d, 32, 32) == 0
    assert L.svg_workspace_bytes(svg.SVG_OP_PROFILE, d, 178, 0) >= 3 * 8 * 178 * 64 * 4
    # split text groups of the sparse V^T attention: 278 kv-blocks -> 6 parts
    # of the 2 leading groups, 256 rows of d + 4 floats each; none at <= 48
    assert L.svg_workspace_bytes(svg.SVG_OP_ATTN_VT, d, 64, 64) == 8 * 2 * 6 * 256 * (64 + 4) * 4
    assert L.svg_workspace_bytes(svg.SVG_OP_ATTN_VT, dims(F=2, S=1536, T=0, H=2, d=128), 128, 64) == 0


def test_svg2_validation():
    L = svg.lib()
    flat = dims(F=1, S=1000, T=0, H=2, d=64)
    assert L.svg_kmeans(flat, 1, FAKE, 300, 10, FAKE, FAKE, FAKE, FAKE, FAKE2, 1 << 30, None) == svg.SVG_ERR_RANGE
    assert L.svg_kmeans(flat, 1, FAKE, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE2, 1 << 30, None) == svg.SVG_ERR_RANGE
    assert L.svg_select_pairs(flat, FAKE, FAKE, FAKE, 64, 256, 1.5, -1.0, FAKE, FAKE, None) == svg.SVG_ERR_RANGE
    assert L.svg_select_pairs(flat, FAKE, FAKE, FAKE, 64, 512, 0.9, -1.0, FAKE, FAKE, None) == svg.SVG_ERR_RANGE
    assert L.svg_permute_rows(flat, 1, FAKE, FAKE2, FAKE, 0, None) == svg.SVG_ERR_RANGE
    assert L.svg_varlen_attn(flat, 1, FAKE, FAKE, FAKE, None, FAKE, 64, 256, FAKE, FAKE, None, -1.0, FAKE2,
                             FAKE2, 1 << 30, None) == svg.SVG_ERR_NULL


def test_vt_entry_points_validate_on_host():
    L = svg.lib()
    # Vt element count: H * ceil(N/64) * 64 * d
    assert L.svg_vt_elems(dims(F=4, S=64, T=16, H=2, d=64)) == 2 * 5 * 64 * 64
    assert L.svg_vt_elems(None) == 0
    bf16 = svg.SVG_BF16
    assert L.svg_dense_attn_vt(dims(), 0, FAKE, FAKE, FAKE, 64, 64, -1.0, FAKE2, None) == svg.SVG_ERR_UNSUPPORTED
    assert "bf16" in svg.last_error()
    assert L.svg_dense_attn_vt(dims(), bf16, FAKE, FAKE, FAKE, 16, 16, -1.0, FAKE2, None) == svg.SVG_ERR_UNSUPPORTED
    assert L.svg_dense_attn_vt(dims(), bf16, FAKE, None, FAKE, 64, 64, -1.0, FAKE2, None) == svg.SVG_ERR_NULL
    # more than 8192 kv-blocks per head
    big = dims(F=1, S=8192 * 64 + 1, T=0, H=1, d=64)
    assert L.svg_dense_attn_vt(big, bf16, FAKE, FAKE, FAKE, 128, 64, -1.0, FAKE2, None) == svg.SVG_ERR_UNSUPPORTED
    assert "kv-blocks" in svg.last_error()
    assert L.svg_block_sparse_attn_csr_vt(dims(), bf16, FAKE, FAKE, FAKE, None, FAKE, 64, 64, -1.0, FAKE2,
                                          None, 0, None) == svg.SVG_ERR_NULL
    # the original-order variant: same checks (NULL lists, NULL tensors, unsupported shapes)
    assert L.svg_block_sparse_attn_csr_vt_layout(dims(), bf16, FAKE, FAKE, FAKE, FAKE, None, None, 64, 64, -1.0,
                                                 FAKE2, None, 0, None) == svg.SVG_ERR_NULL
    assert L.svg_block_sparse_attn_csr_vt_layout(dims(), bf16, None, FAKE, FAKE, FAKE, FAKE, None, 64, 64, -1.0,
                                                 FAKE2, None, 0, None) == svg.SVG_ERR_NULL
    assert L.svg_block_sparse_attn_csr_vt_layout(dims(), bf16, FAKE, FAKE, FAKE, FAKE, FAKE, None, 128, 128, -1.0,
                                                 FAKE2, None, 0, None) == svg.SVG_ERR_UNSUPPORTED
    assert L.svg_block_sparse_attn_csr_vt_layout(dims(), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, 64, 64, -1.0,
                                                 FAKE2, None, 0, None) == svg.SVG_ERR_UNSUPPORTED
    # the split-partials workspace: too small, or overlapping a tensor
    big_w = dims(F=4, S=64 * 40, T=64, H=2, d=128)       # 161 kv-blocks: split
    need = L.svg_workspace_bytes(svg.SVG_OP_ATTN_VT, big_w, 128, 64)
    assert L.svg_block_sparse_attn_csr_vt(big_w, bf16, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 64, -1.0, FAKE2,
                                          FAKE3, need - 1, None) == svg.SVG_ERR_WORKSPACE
    assert L.svg_block_sparse_attn_csr_vt_layout(big_w, bf16, FAKE, FAKE, FAKE, FAKE, FAKE, None, 128, 64, -1.0,
                                                 FAKE2, FAKE, need, None) == svg.SVG_ERR_RANGE
    # O overlapping an input
    assert L.svg_dense_attn_vt(dims(), bf16, FAKE, FAKE2, FAKE, 64, 64, -1.0, FAKE, None) == svg.SVG_ERR_RANGE
    assert L.svg_layout_permute_vt(dims(), 0, FAKE, FAKE2, None, None) == svg.SVG_ERR_UNSUPPORTED
    assert L.svg_layout_permute_vt(dims(), bf16, FAKE, FAKE, None, None) == svg.SVG_ERR_RANGE
    assert L.svg_layout_permute_vt(dims(), bf16, None, FAKE2, None, None) == svg.SVG_ERR_NULL


def test_kmeans_noalloc_rejects_problems_beyond_its_scratch():
    """The allocation-free k-means refuses, on the host, a problem whose
    scratch exceeds the library's array, and checks its arguments like
    svg_kmeans."""
    L = svg.lib()
    big = svg.svg_dims(1, 1 << 20, 0, 24, 128)      # ~100 MB of cluster order alone
    need = L.svg2_workspace_bytes(svg.SVG2_OP_KMEANS, ctypes.byref(big), 256, 0)
    assert need > (32 << 20)
    assert L.svg_kmeans_noalloc(ctypes.byref(big), 1, FAKE, 256, 10, FAKE, FAKE2, FAKE3, FAKE2, None) \
        == svg.SVG_ERR_WORKSPACE
    assert "scratch" in svg.last_error()
    small = svg.svg_dims(1, 1000, 0, 2, 64)
    assert L.svg_kmeans_noalloc(ctypes.byref(small), 1, FAKE, 0, 10, FAKE, FAKE2, FAKE3, FAKE2, None) \
        == svg.SVG_ERR_RANGE
    assert L.svg_kmeans_noalloc(ctypes.byref(small), 1, None, 8, 10, FAKE, FAKE2, FAKE3, FAKE2, None) \
        == svg.SVG_ERR_NULL


def test_hva_cluster_count_and_host_checks():
    """svg_hva_clusters agrees with the oracle's count (windows plus the text
    cluster); the HVA entries reject bad geometry, dtype and workspace on
    the host."""
    from oracle import hva
    win = lambda *w: (ctypes.c_int32 * 3)(*w)
    for F, rows, cols, T, w in ((13, 30, 45, 224, (2, 6, 9)), (13, 30, 45, 224, (4, 10, 15)), (3, 4, 5, 0, (2, 2, 2)),
                                (1, 1, 7, 3, (1, 1, 7)), (5, 6, 6, 1, (9, 9, 9))):
        got = svg.lib().svg_hva_clusters(dims(F=F, S=rows * cols, T=T), rows, cols, win(*w))
        assert got == hva.n_clusters(F, rows, cols, T, w)
    L = svg.lib()
    d0 = dims(F=13, S=1350, T=224, H=2, d=64)
    assert L.svg_hva_clusters(d0, 30, 44, win(2, 6, 9)) == 0                 # rows * cols != S
    assert L.svg_hva_clusters(d0, 30, 45, win(0, 6, 9)) == 0
    assert L.svg_hva_clusters(d0, 30, 45, None) == 0
    o1, o2, o3, o4 = (ctypes.c_void_p(a) for a in (0x100000000, 0x200000000, 0x300000000, 0x400000000))
    wsp = ctypes.c_void_p(0x500000000)

    def cl(dt=1, x=FAKE, rows=30, w=(2, 6, 9), iters=10, r2=0.64, ws=wsp, wsb=1 << 30, outs=(o1, o2, o3, o4)):
        return L.svg_hva_cluster(d0, dt, x, rows, 45, win(*w), iters, ctypes.c_float(r2), *outs, ws, wsb, None)

    assert cl(dt=0) == svg.SVG_ERR_UNSUPPORTED                               # fp32
    assert cl(x=None) == svg.SVG_ERR_NULL
    assert cl(rows=29) == svg.SVG_ERR_SHAPE
    assert cl(w=(2, 0, 9)) == svg.SVG_ERR_RANGE
    assert cl(iters=0) == svg.SVG_ERR_RANGE
    assert cl(r2=1.5) == svg.SVG_ERR_RANGE
    assert cl(wsb=16) == svg.SVG_ERR_WORKSPACE
    assert cl(outs=(o1, o1, o3, o4)) == svg.SVG_ERR_RANGE                    # two outputs share memory
    assert L.svg_hva_refresh(d0, 1, FAKE, 30, 45, win(2, 6, 9), None, o1, o2, o3, wsp, 1 << 30,
                             None) == svg.SVG_ERR_NULL
    need = svg.lib().svg2_workspace_bytes(svg.SVG2_OP_HVA, d0, 176, 0)
    assert need >= 2 * 176 * 64 * 12
