"""The Python binding rejects a wrong dtype, size or device of every tensor
argument before anything reaches the library (CPU only: each call here raises
in the binding's own checks, so no HIP call is made).

A torch.tensor([0, 1]) is int64, and float32 centroids are half the bytes of
the float64 ones a kernel reads: without these checks such arguments would
make a kernel read the wrong words or past the end of a buffer."""

import pytest
import torch

svg = pytest.importorskip("sparse_attention_video_online_amd.svg")

F, S, T, H, d = 3, 20, 4, 2, 64
N = F * S + T


def bf16(*shape):
    return torch.zeros(*shape, dtype=torch.bfloat16)


def i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def raises(exc, match, fn, *args, **kw):
    with pytest.raises(exc, match=match):
        fn(*args, **kw)


def test_layout_labels_dtype_and_size():
    x = bf16(H, N, d)
    raises(TypeError, "labels must be torch.int32", svg.svg_layout_permute, x, F, S, T, torch.tensor([0, 1]))
    raises(ValueError, "labels must have 2 elements", svg.svg_layout_unpermute, x, F, S, T, i32(3))
    raises(TypeError, "labels must be torch.int32", svg.svg_layout_permute_vt, x, F, S, T, torch.tensor([0, 1]))
    raises(TypeError, "labels must be torch.int32", svg.svg_build_block_mask, torch.tensor([0, 1]),
           F, S, T, H, d, 0, 32, 64, 64)


def test_layout_shape_and_output():
    raises(ValueError, r"N=65 != F\*S\+T=64", svg.svg_layout_permute, bf16(H, N + 1, d), F, S, T)
    raises(ValueError, "out must have", svg.svg_layout_permute, bf16(H, N, d), F, S, T, None, bf16(H, N - 1, d))
    raises(TypeError, "out must be torch.bfloat16", svg.svg_layout_unpermute, bf16(H, N, d), F, S, T, None,
           torch.zeros(H, N, d))
    raises(ValueError, "contiguous", svg.svg_layout_permute, bf16(H, d, N).transpose(1, 2), F, S, T)
    raises(ValueError, "Vt must have", svg.svg_layout_permute_vt, bf16(H, N, d), F, S, T, None, bf16(10))


def test_attention_lists_outputs_and_workspaces():
    q, k, v = bf16(H, N, d), bf16(H, N, d), bf16(H, N, d)
    nqb = -(-N // 64)
    raises(ValueError, "K must have", svg.svg_dense_attn, q, bf16(H, N, d + 64), v, F, S, T, 64, 64)
    raises(TypeError, "V must be torch.bfloat16", svg.svg_dense_attn, q, k, torch.zeros(H, N, d), F, S, T, 64, 64)
    raises(TypeError, "row_ptr must be torch.int32", svg.svg_block_sparse_attn_csr, q, k, v,
           torch.zeros(H * nqb + 1, dtype=torch.int64), i32(4), F, S, T, 64, 64)
    raises(ValueError, "row_ptr must have", svg.svg_block_sparse_attn_csr, q, k, v, i32(H * nqb), i32(4),
           F, S, T, 64, 64)
    raises(ValueError, "block_mask must have", svg.svg_block_sparse_attn, q, k, v,
           torch.zeros(H, nqb, nqb + 1, dtype=torch.uint8), F, S, T, 64, 64)
    vt = bf16(svg.svg_vt_elems(H, N, d))
    raises(TypeError, "labels must be torch.int32", svg.svg_block_sparse_attn_csr_vt_layout, q, k, vt,
           i32(H * nqb + 1), i32(4), torch.tensor([1, 1]), F, S, T, 64, 64)
    raises(ValueError, "Vt must have", svg.svg_dense_attn_vt, q, k, bf16(7), F, S, T, 64, 64)
    raises(ValueError, "out must have", svg.svg_block_sparse_attn_csr_vt, q, k, vt, i32(H * nqb + 1), i32(4),
           F, S, T, 64, 64, out=bf16(H, N, 8))
    raises(TypeError, "ws must be torch.uint8", svg.svg_block_sparse_attn, q, k, v,
           torch.zeros(H, nqb, nqb, dtype=torch.uint8), F, S, T, 64, 64, ws=torch.zeros(1 << 20))
    raises(ValueError, "ws must have at least", svg.svg_block_sparse_attn, q, k, v,
           torch.zeros(H, nqb, nqb, dtype=torch.uint8), F, S, T, 64, 64, ws=torch.zeros(4, dtype=torch.uint8))


def test_profile_and_compaction():
    q, k, v = bf16(H, N, d), bf16(H, N, d), bf16(H, N, d)
    raises(TypeError, "sample_idx must be torch.int32", svg.svg_profile_heads, q, k, v, torch.tensor([1, 2]),
           F, S, T, 0, 32)
    raises(ValueError, "sample_idx must hold", svg.svg_profile_heads, q, k, v, i32(N + 1), F, S, T, 0, 32)
    raises(TypeError, "mse must be torch.float32", svg.svg_profile_heads, q, k, v, i32(4), F, S, T, 0, 32,
           mse=torch.zeros(H, 2, dtype=torch.float64))
    bm = torch.zeros(H, 3, 5, dtype=torch.uint8)
    raises(ValueError, "kv_idx must have at least 30", svg.svg_compact_block_mask, bm, None, i32(29))
    raises(TypeError, "block_mask must be torch.uint8", svg.svg_compact_block_mask, torch.zeros(H, 3, 5))


def test_svg2_arguments():
    x = bf16(H, N, d)
    raises(ValueError, "init_idx must have", svg.svg_kmeans, x, 8, 2, i32(H * 7))
    raises(TypeError, "centroids must be torch.float64", svg.svg_kmeans, x, 8, 2, i32(H * 8),
           centroids=torch.zeros(H, 8, d))
    raises(TypeError, "assign must be torch.int32", svg.svg_cluster_permute, torch.zeros(H, N, dtype=torch.int64), 8)
    raises(ValueError, "perm must have", svg.svg_permute_rows, x, i32(H * N - 1))
    raises(TypeError, "perm must be torch.int32", svg.svg_permute_rows, x, torch.zeros(H, N, dtype=torch.int64))
    cq, ck = torch.zeros(H, 4, d, dtype=torch.float64), torch.zeros(H, 6, d, dtype=torch.float64)
    raises(TypeError, "cq must be torch.float64", svg.svg_select_pairs, cq.float(), ck, i32(H, 6), 0.9)
    raises(TypeError, "ck must be torch.float64", svg.svg_select_pairs, cq, ck.float(), i32(H, 6), 0.9)
    raises(ValueError, "size_k must have", svg.svg_select_pairs, cq, ck, i32(H, 5), 0.9)
    qo, ko = i32(H, 5), i32(H, 7)
    raises(ValueError, "pair_idx must have", svg.svg_varlen_attn, x, x, x, qo, ko, i32(H, 5), i32(H, 4 * 5))
    raises(ValueError, "q_perm must have", svg.svg_varlen_attn, x, x, x, qo, ko, i32(H, 5), i32(H, 4 * 6),
           q_perm=i32(H, N - 1))


def test_right_arguments_on_the_host_are_refused_as_host_tensors():
    """dtype and sizes right, but host memory: refused before any library
    call (the pointer of a host tensor would fault a kernel)."""
    x = bf16(H, N, d)
    raises(ValueError, "device tensors", svg.svg_layout_permute, x, F, S, T, i32(H))
    raises(ValueError, "device tensors", svg.svg_permute_rows, x, i32(H, N))


def test_fused_ear_and_fp8_attention_arguments():
    q, k = bf16(H, N, d), bf16(H, N, d)
    nqb, nkb = -(-N // 64), -(-N // 64)
    vt = bf16(svg.svg_vt_elems(H, N, d))
    rp, ki = i32(H * nqb + 1), i32(4)
    raises(TypeError, "labels must be torch.int32", svg.svg_block_sparse_attn_csr_vt_fused, q, k, vt, rp, ki,
           torch.tensor([1, 1]), F, S, T, 64, 64)
    raises(ValueError, "Vt must have", svg.svg_block_sparse_attn_csr_vt_fused, q, k, bf16(9), rp, ki, i32(H),
           F, S, T, 64, 64)
    raises(TypeError, "row_ptr must be torch.int32", svg.svg_block_sparse_attn_csr_vt_fused, q, k, vt,
           torch.zeros(H * nqb + 1, dtype=torch.int64), ki, i32(H), F, S, T, 64, 64)
    ne = svg.svg_ear_centroid_elems(H, N, d)
    raises(ValueError, "Vt must have", svg.svg_ear_block_stats, k, bf16(5), F, S, T)
    raises(TypeError, "kbar must be torch.float64", svg.svg_ear_block_stats, k, vt, F, S, T,
           kbar=torch.zeros(H, d, nkb))
    raises(ValueError, "block_mask must have", svg.svg_ear_route, q, i32(H), torch.zeros(H, d, nkb, dtype=torch.float64),
           torch.zeros(H, nkb, dtype=torch.float64), torch.zeros(H, nqb, nkb - 1, dtype=torch.uint8), F, S, T, 64, 64, 16)
    raises(ValueError, "Kc must have", svg.svg_block_sparse_attn_ear_vt_layout, q, k, vt, bf16(ne - 1), bf16(ne), rp,
           ki, i32(H), F, S, T, 64, 64)
    q8, k8 = torch.zeros(H, N, d, dtype=torch.uint8), torch.zeros(H, N, d, dtype=torch.uint8)
    qs, ks = torch.zeros(H, N), torch.zeros(H, nkb)
    raises(TypeError, "X must be torch.bfloat16", svg.svg_quantize_fp8_rows, torch.zeros(H, N, d))
    raises(ValueError, "scale must have", svg.svg_layout_permute_fp8, k, F, S, T, None, None, torch.zeros(H, nkb + 1))
    raises(TypeError, "Q8 must be torch.uint8", svg.svg_block_sparse_attn_fp8_vt_layout, q, qs, k8, ks, vt, rp, ki,
           i32(H), F, S, T, 64, 64)
    raises(ValueError, "kscale must have", svg.svg_dense_attn_fp8_vt, q8, qs, k8, torch.zeros(H, nkb - 1), vt,
           F, S, T, 64, 64)
    vt8, va = torch.zeros(svg.svg_vt_elems(H, N, d), dtype=torch.uint8), torch.zeros(H, d)
    raises(TypeError, "V must be torch.bfloat16", svg.svg_layout_permute_vt_fp8, torch.zeros(H, N, d), F, S, T)
    raises(ValueError, "vamax must have", svg.svg_layout_permute_vt_fp8, k, F, S, T, None, None, torch.zeros(H, d - 1))
    raises(TypeError, "Vt8 must be torch.uint8", svg.svg_block_sparse_attn_fp8pv_vt_layout, q8, qs, k8, ks, vt, va,
           rp, ki, i32(H), F, S, T, 64, 64)
    raises(ValueError, "vamax must have", svg.svg_block_sparse_attn_fp8pv_vt_layout, q8, qs, k8, ks, vt8,
           torch.zeros(H, d + 1), rp, ki, i32(H), F, S, T, 64, 64)


def test_varlen_vt_and_hva_arguments():
    x = bf16(H, N, d)
    raises(TypeError, "perm must be torch.int32", svg.svg_permute_rows_vt, x, torch.zeros(H, N, dtype=torch.int64))
    raises(ValueError, "Vt must have", svg.svg_permute_rows_vt, x, i32(H, N), bf16(7))
    qo, ko = i32(H, 5), i32(H, 7)
    raises(ValueError, "Vt must have", svg.svg_varlen_attn_vt, x, x, bf16(3), qo, ko, i32(H, 5), i32(H, 4 * 6))
    raises(ValueError, "pair_idx must have", svg.svg_varlen_attn_vt, x, x, bf16(svg.svg_vt_elems(H, N, d)), qo, ko,
           i32(H, 5), i32(H, 4 * 5))
    rows, cols, win = 4, 4, (2, 2, 2)
    raises(ValueError, r"F\*S\+T", svg.svg_hva_cluster, bf16(H, N, d), F, rows, cols, T, win, 2)
    n = F * rows * cols + T
    y = bf16(H, n, d)
    k = svg.svg_hva_clusters(F, rows, cols, T, win, H, d)
    raises(TypeError, "assign must be torch.int32", svg.svg_hva_cluster, y, F, rows, cols, T, win, 2,
           assign=torch.zeros(H, n, dtype=torch.int64))
    raises(ValueError, "centroids must have", svg.svg_hva_refresh, y, F, rows, cols, T, win,
           torch.zeros(H, n, dtype=torch.uint8), i32(H, n), torch.zeros(H, k - 1, d, dtype=torch.float64))
    raises(TypeError, "refresh must be torch.uint8", svg.svg_hva_refresh, y, F, rows, cols, T, win,
           i32(H, n), i32(H, n), torch.zeros(H, k, d, dtype=torch.float64))
