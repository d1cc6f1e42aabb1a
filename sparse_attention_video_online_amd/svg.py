"""Thin Python binding of libsvg_hip.so (the C ABI in include/svg.h, svg2.h).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory (tensors) and the current HIP stream.  The
functions keep the C names.  Outputs and workspaces the caller does not pass
are allocated as torch tensors.

Importing this module raises if the built library is missing.  There is no
fallback path.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsvg_hip.so")

SVG_OK, SVG_ERR_NULL, SVG_ERR_SHAPE, SVG_ERR_DTYPE, SVG_ERR_UNSUPPORTED, SVG_ERR_RANGE, \
    SVG_ERR_WORKSPACE, SVG_ERR_HIP = range(8)
SVG_F32, SVG_BF16 = 0, 1
SVG_OP_PROFILE, SVG_OP_BLOCK_SPARSE, SVG_OP_COMPACT, SVG_OP_ATTN_VT, SVG_OP_ATTN_CSR = 0, 1, 2, 3, 4
SVG2_OP_KMEANS, SVG2_OP_CLUSTER_PERMUTE, SVG2_OP_VARLEN, SVG2_OP_HVA = 0, 1, 2, 3


class svg_dims(ctypes.Structure):
    _fields_ = [("F", ctypes.c_int32), ("S", ctypes.c_int32), ("T", ctypes.c_int32),
                ("H", ctypes.c_int32), ("d", ctypes.c_int32)]


class svg_mask_params(ctypes.Structure):
    _fields_ = [("ks_frames", ctypes.c_int32), ("wt_tokens", ctypes.c_int32)]


class SvgError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"svg status {status}: {message}")
        self.status = status


_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_D = ctypes.c_double
_Z = ctypes.c_size_t
_DIMS = ctypes.POINTER(svg_dims)
_MASK = ctypes.POINTER(svg_mask_params)

# name -> argtypes (all return int32 status unless listed in _RESTYPES)
SIGNATURES = {
    "svg_workspace_bytes": [_I, _DIMS, _I, _I],
    "svg_last_error": [],
    "svg_version": [],
    "svg_profile_heads": [_DIMS, _I, _P, _P, _P, _P, _I, _MASK, _F, _P, _P, _P, _Z, _P],
    "svg_layout_permute": [_DIMS, _I, _P, _P, _P, _P],
    "svg_layout_unpermute": [_DIMS, _I, _P, _P, _P, _P],
    "svg_build_block_mask": [_DIMS, _MASK, _P, _I, _I, _P, _P],
    "svg_compact_block_mask": [_I, _I, _P, _P, _P, _P, _Z, _P],
    "svg_block_sparse_attn": [_DIMS, _I, _P, _P, _P, _P, _I, _I, _F, _P, _P, _Z, _P],
    "svg_block_sparse_attn_csr": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P, _Z, _P],
    "svg_dense_attn": [_DIMS, _I, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg_vt_elems": [_DIMS],
    "svg_layout_permute_vt": [_DIMS, _I, _P, _P, _P, _P],
    "svg_block_sparse_attn_csr_vt": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P, _Z, _P],
    "svg_block_sparse_attn_csr_vt_layout": [_DIMS, _I, _P, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P, _Z, _P],
    "svg_block_sparse_attn_csr_vt_fused": [_DIMS, _I, _P, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P, _Z, _P],
    "svg_dense_attn_vt": [_DIMS, _I, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg_ear_centroid_elems": [_DIMS],
    "svg_ear_block_stats": [_DIMS, _I, _P, _P, _P, _P, _P, _P, _P],
    "svg_ear_route": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _I, _F, _P, _P],
    "svg_block_sparse_attn_ear_vt_layout": [_DIMS, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg_quantize_fp8_rows": [_DIMS, _I, _P, _P, _P, _P],
    "svg_layout_permute_fp8": [_DIMS, _I, _P, _P, _P, _P, _P],
    "svg_block_sparse_attn_fp8_vt_layout": [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg_dense_attn_fp8_vt": [_DIMS, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg_layout_permute_vt_fp8": [_DIMS, _I, _P, _P, _P, _P, _P],
    "svg_block_sparse_attn_fp8pv_vt_layout": [_DIMS, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg2_workspace_bytes": [_I, _DIMS, _I, _I],
    "svg_kmeans": [_DIMS, _I, _P, _I, _I, _P, _P, _P, _P, _P, _Z, _P],
    "svg_kmeans_noalloc": [_DIMS, _I, _P, _I, _I, _P, _P, _P, _P, _P],
    "svg_cluster_permute": [_DIMS, _P, _I, _P, _P, _P, _Z, _P],
    "svg_permute_rows": [_DIMS, _I, _P, _P, _P, _I, _P],
    "svg_select_pairs": [_DIMS, _P, _P, _P, _I, _I, _D, _F, _P, _P, _P],
    "svg_varlen_attn": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _F, _P, _P, _Z, _P],
    "svg_permute_rows_vt": [_DIMS, _I, _P, _P, _P, _P],
    "svg_hva_clusters": [_DIMS, _I, _I, _P],
    "svg_hva_cluster": [_DIMS, _I, _P, _I, _I, _P, _I, _F, _P, _P, _P, _P, _P, _Z, _P],
    "svg_hva_refresh": [_DIMS, _I, _P, _I, _I, _P, _P, _P, _P, _P, _P, _Z, _P],
    "svg_varlen_attn_vt": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _F, _P, _P],
}
_RESTYPES = {"svg_hva_clusters": _I, "svg_workspace_bytes": _Z, "svg2_workspace_bytes": _Z, "svg_vt_elems": _Z, "svg_ear_centroid_elems": _Z,
             "svg_last_error": ctypes.c_char_p, "svg_version": ctypes.c_char_p}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          f"or python sparse_attention_video_online_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name, None)
        if fn is None:
            continue
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, ctypes.c_int32)
    return lib


_lib = _load()


def lib():
    return _lib


def last_error() -> str:
    return _lib.svg_last_error().decode()


def _check(status, name):
    if status != SVG_OK:
        raise SvgError(status, f"{name}: {last_error()}")


def _ptr(t):
    """Device pointer of a tensor argument (None -> NULL).  Every argument
    check of a call runs before its first pointer is taken, so a CPU tensor
    is reported only once its dtype and size are right."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor arguments must be device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return SVG_BF16
    if t.dtype == torch.float32:
        return SVG_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, numel=None, min_numel=None):
    """Checks a tensor argument before anything reaches the library: its
    dtype, its element count (exact, or a capacity) and contiguity (_ptr
    then requires a device tensor).  Every tensor the C ABI receives goes
    through here, so a wrong dtype or size raises instead of letting a kernel
    read or write past a buffer."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name} must have at least {min_numel} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _opt(t, name, **kw):
    if t is not None:
        _need(t, name, **kw)


def _bytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def dims(F, S, T, H, d):
    return svg_dims(F, S, T, H, d)


def _shape3(x, name):
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError(f"{name} must be a [H][N][d] tensor")
    return x.shape


def _video_dims(x, F, S, T, name="X"):
    H, N, d = _shape3(x, name)
    if N != F * S + T:
        raise ValueError(f"{name}: N={N} != F*S+T={F * S + T}")
    return svg_dims(F, S, T, H, d)


def _qkv(q, k, v, F, S, T):
    dm = _video_dims(q, F, S, T, "Q")
    H, N, d = q.shape
    dt = _dtype(q)
    for t, n in ((q, "Q"), (k, "K"), (v, "V")):
        _need(t, n, q.dtype, H * N * d)
    return dm, dt


def _out_like(out, x, name="out"):
    if out is None:
        return torch.empty_like(x)
    _need(out, name, x.dtype, x.numel())
    return out


def _labels(labels, H):
    _opt(labels, "labels", dtype=torch.int32, numel=H)


def workspace_bytes(op, dm, a=0, b=0, svg2=False):
    fn = _lib.svg2_workspace_bytes if svg2 else _lib.svg_workspace_bytes
    return fn(op, ctypes.byref(dm), a, b)


def _ws(nbytes, device, ws=None, name="ws"):
    if ws is not None:
        _need(ws, name, torch.uint8, min_numel=int(nbytes))
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# SVG1 path

def svg_profile_heads(q, k, v, sample_idx, F, S, T, ks, wt, scale=-1.0, labels=None, mse=None, ws=None):
    dm, dt = _qkv(q, k, v, F, S, T)
    H, N = q.shape[0], q.shape[1]
    _need(sample_idx, "sample_idx", torch.int32)
    if not 1 <= sample_idx.numel() <= N:
        raise ValueError(f"sample_idx must hold 1..N={N} rows, got {sample_idx.numel()}")
    labels = torch.empty(H, dtype=torch.int32, device=q.device) if labels is None else labels
    mse = torch.empty(H, 2, dtype=torch.float32, device=q.device) if mse is None else mse
    _need(labels, "labels", torch.int32, H)
    _need(mse, "mse", torch.float32, 2 * H)
    mp = svg_mask_params(ks, wt)
    ws = _ws(workspace_bytes(SVG_OP_PROFILE, dm, sample_idx.numel()), q.device, ws)
    _check(_lib.svg_profile_heads(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(sample_idx),
                                  sample_idx.numel(), ctypes.byref(mp), scale, _ptr(labels), _ptr(mse),
                                  _ptr(ws), _bytes(ws), _stream()), "svg_profile_heads")
    return labels, mse


def _layout(fn, name, x, F, S, T, labels, out):
    dm = _video_dims(x, F, S, T)
    dt = _dtype(x)
    _need(x, "X", x.dtype, x.numel())
    _labels(labels, x.shape[0])
    out = _out_like(out, x)
    _check(fn(ctypes.byref(dm), dt, _ptr(x), _ptr(out), _ptr(labels), _stream()), name)
    return out


def svg_layout_permute(x, F, S, T, labels=None, out=None):
    return _layout(_lib.svg_layout_permute, "svg_layout_permute", x, F, S, T, labels, out)


def svg_layout_unpermute(x, F, S, T, labels=None, out=None):
    return _layout(_lib.svg_layout_unpermute, "svg_layout_unpermute", x, F, S, T, labels, out)


def svg_build_block_mask(labels, F, S, T, H, d, ks, wt, bq, bk, out=None):
    dm = svg_dims(F, S, T, H, d)
    N = F * S + T
    nqb, nkb = -(-N // bq), -(-N // bk)
    _need(labels, "labels", torch.int32, H)
    out = torch.empty(H, nqb, nkb, dtype=torch.uint8, device=labels.device) if out is None else out
    _need(out, "block_mask", torch.uint8, H * nqb * nkb)
    mp = svg_mask_params(ks, wt)
    _check(_lib.svg_build_block_mask(ctypes.byref(dm), ctypes.byref(mp), _ptr(labels), bq, bk, _ptr(out),
                                     _stream()), "svg_build_block_mask")
    return out


def svg_compact_block_mask(block_mask, row_ptr=None, kv_idx=None, ws=None):
    if not isinstance(block_mask, torch.Tensor) or block_mask.dim() < 1:
        raise ValueError("block_mask must be a tensor whose last dimension is nKB")
    nkb = block_mask.shape[-1]
    rows = block_mask.numel() // nkb if nkb else 0
    _need(block_mask, "block_mask", torch.uint8)
    dev = block_mask.device
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev) if row_ptr is None else row_ptr
    kv_idx = torch.empty(max(rows * nkb, 1), dtype=torch.int32, device=dev) if kv_idx is None else kv_idx
    _need(row_ptr, "row_ptr", torch.int32, rows + 1)
    _need(kv_idx, "kv_idx", torch.int32, min_numel=rows * nkb)
    ws = _ws(_lib.svg_workspace_bytes(SVG_OP_COMPACT, None, rows, nkb), dev, ws)
    _check(_lib.svg_compact_block_mask(rows, nkb, _ptr(block_mask), _ptr(row_ptr), _ptr(kv_idx), _ptr(ws),
                                       _bytes(ws), _stream()), "svg_compact_block_mask")
    return row_ptr, kv_idx


def _lists(row_ptr, kv_idx, H, N, bq):
    nqb = -(-N // bq)
    _need(row_ptr, "row_ptr", torch.int32, H * nqb + 1)
    _need(kv_idx, "kv_idx", torch.int32)


def svg_block_sparse_attn(q, k, v, block_mask, F, S, T, bq, bk, scale=-1.0, out=None, ws=None):
    dm, dt = _qkv(q, k, v, F, S, T)
    H, N = q.shape[0], q.shape[1]
    _need(block_mask, "block_mask", torch.uint8, H * (-(-N // bq)) * (-(-N // bk)))
    out = _out_like(out, q)
    ws = _ws(workspace_bytes(SVG_OP_BLOCK_SPARSE, dm, bq, bk), q.device, ws)
    _check(_lib.svg_block_sparse_attn(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), bq, bk,
                                      scale, _ptr(out), _ptr(ws), _bytes(ws), _stream()), "svg_block_sparse_attn")
    return out


def attn_csr_workspace(q, F, S, T, bq, bk):
    """Workspace of svg_block_sparse_attn_csr's V^T path (None when that
    kernel does not cover the shape)."""
    n = workspace_bytes(SVG_OP_ATTN_CSR, svg_dims(F, S, T, q.shape[0], q.shape[2]), bq, bk)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None


def svg_block_sparse_attn_csr(q, k, v, row_ptr, kv_idx, F, S, T, bq, bk, scale=-1.0, out=None, ws=None,
                              rowmajor_kernel=False):
    """ws: from attn_csr_workspace (allocated here when None).
    rowmajor_kernel: pass no workspace, so the row-major MFMA kernel runs."""
    dm, dt = _qkv(q, k, v, F, S, T)
    _lists(row_ptr, kv_idx, q.shape[0], q.shape[1], bq)
    out = _out_like(out, q)
    if rowmajor_kernel:
        ws = None
    elif ws is None:
        ws = attn_csr_workspace(q, F, S, T, bq, bk)
    else:
        _need(ws, "ws", torch.uint8, min_numel=workspace_bytes(SVG_OP_ATTN_CSR, dm, bq, bk))
    _check(_lib.svg_block_sparse_attn_csr(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                          _ptr(kv_idx), bq, bk, scale, _ptr(out), _ptr(ws), _bytes(ws),
                                          _stream()),
           "svg_block_sparse_attn_csr")
    return out


def svg_dense_attn(q, k, v, F, S, T, bq, bk, scale=-1.0, out=None):
    dm, dt = _qkv(q, k, v, F, S, T)
    out = _out_like(out, q)
    _check(_lib.svg_dense_attn(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(v), bq, bk, scale, _ptr(out),
                               _stream()), "svg_dense_attn")
    return out


def svg_vt_elems(H, N, d):
    """Elements of the key-tiled transposed V of a [H][N][d] tensor."""
    dm = svg_dims(1, N, 0, H, d)
    return int(_lib.svg_vt_elems(ctypes.byref(dm)))


def svg_layout_permute_vt(v, F, S, T, labels=None, out=None):
    """Vt (key-tiled transposed layout, shape [H][nKB][d][64]) of the
    executing-layout V."""
    dm = _video_dims(v, F, S, T, "V")
    H, N, d = v.shape
    dt = _dtype(v)
    _need(v, "V", v.dtype, v.numel())
    _labels(labels, H)
    nkb = -(-N // 64)
    out = torch.empty(H, nkb, d, 64, dtype=v.dtype, device=v.device) if out is None else out
    _need(out, "Vt", v.dtype, svg_vt_elems(H, N, d))
    _check(_lib.svg_layout_permute_vt(ctypes.byref(dm), dt, _ptr(v), _ptr(out), _ptr(labels), _stream()),
           "svg_layout_permute_vt")
    return out


def _qk_vt(q, k, vt, F, S, T):
    dm = _video_dims(q, F, S, T, "Q")
    H, N, d = q.shape
    dt = _dtype(q)
    for t, n in ((q, "Q"), (k, "K")):
        _need(t, n, q.dtype, H * N * d)
    _need(vt, "Vt", q.dtype, svg_vt_elems(H, N, d))
    return dm, dt


def attn_vt_workspace(q, F, S, T, bq, bk):
    """Workspace for the split text groups of the sparse V^T attention
    entries (None when no split applies)."""
    n = workspace_bytes(SVG_OP_ATTN_VT, svg_dims(F, S, T, q.shape[0], q.shape[2]), bq, bk)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None


def _vt_ws(ws, q, dm, F, S, T, bq, bk):
    if ws is None:
        return attn_vt_workspace(q, F, S, T, bq, bk)
    _need(ws, "ws", torch.uint8, min_numel=workspace_bytes(SVG_OP_ATTN_VT, dm, bq, bk))
    return ws


def svg_block_sparse_attn_csr_vt(q, k, vt, row_ptr, kv_idx, F, S, T, bq, bk, scale=-1.0, out=None, ws=None):
    """ws: from attn_vt_workspace (allocated here when None)."""
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    _lists(row_ptr, kv_idx, q.shape[0], q.shape[1], bq)
    out = _out_like(out, q)
    ws = _vt_ws(ws, q, dm, F, S, T, bq, bk)
    _check(_lib.svg_block_sparse_attn_csr_vt(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt), _ptr(row_ptr),
                                             _ptr(kv_idx), bq, bk, scale, _ptr(out), _ptr(ws), _bytes(ws),
                                             _stream()),
           "svg_block_sparse_attn_csr_vt")
    return out


def svg_block_sparse_attn_csr_vt_layout(q, k, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, scale=-1.0,
                                        out=None, ws=None):
    """Q and the returned O in the original token order; K, Vt and the lists
    in each head's executing layout per labels (None: every head temporal).
    ws: from attn_vt_workspace (allocated here when None)."""
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    _lists(row_ptr, kv_idx, q.shape[0], q.shape[1], bq)
    _labels(labels, q.shape[0])
    out = _out_like(out, q)
    ws = _vt_ws(ws, q, dm, F, S, T, bq, bk)
    _check(_lib.svg_block_sparse_attn_csr_vt_layout(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt),
                                                    _ptr(row_ptr), _ptr(kv_idx), _ptr(labels), bq, bk, scale,
                                                    _ptr(out), _ptr(ws), _bytes(ws), _stream()),
           "svg_block_sparse_attn_csr_vt_layout")
    return out


def svg_block_sparse_attn_csr_vt_fused(q, k, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, scale=-1.0,
                                       out=None, ws=None):
    """Q, K and the returned O in the original token order; Vt and the lists
    in each head's executing layout per labels (None: every head temporal)."""
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    _lists(row_ptr, kv_idx, q.shape[0], q.shape[1], bq)
    _labels(labels, q.shape[0])
    out = _out_like(out, q)
    ws = _vt_ws(ws, q, dm, F, S, T, bq, bk)
    _check(_lib.svg_block_sparse_attn_csr_vt_fused(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt),
                                                   _ptr(row_ptr), _ptr(kv_idx), _ptr(labels), bq, bk, scale,
                                                   _ptr(out), _ptr(ws), _bytes(ws), _stream()),
           "svg_block_sparse_attn_csr_vt_fused")
    return out


def svg_dense_attn_vt(q, k, vt, F, S, T, bq, bk, scale=-1.0, out=None):
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    out = _out_like(out, q)
    _check(_lib.svg_dense_attn_vt(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt), bq, bk, scale, _ptr(out),
                                  _stream()), "svg_dense_attn_vt")
    return out


# ----------------------------------------------------------------------------
# SVG-EAR

def svg_ear_centroid_elems(H, N, d):
    dm = svg_dims(1, N, 0, H, d)
    return int(_lib.svg_ear_centroid_elems(ctypes.byref(dm)))


def svg_ear_block_stats(k, vt, F, S, T, kc=None, vct=None, kbar=None, radius=None):
    """Centroid tables (bf16 centroid keys, key-tiled bf16 value sums) and the
    double centroids (dim-major, [H][d][nKB]) and radii of the kv-blocks of
    K / Vt (executing layout)."""
    dm = _video_dims(k, F, S, T, "K")
    H, N, d = k.shape
    dt = _dtype(k)
    _need(k, "K", torch.bfloat16, k.numel())
    _need(vt, "Vt", torch.bfloat16, svg_vt_elems(H, N, d))
    ne = svg_ear_centroid_elems(H, N, d)
    nkb = -(-N // 64)
    dev = k.device
    kc = torch.empty(ne, dtype=torch.bfloat16, device=dev) if kc is None else kc
    vct = torch.empty(ne, dtype=torch.bfloat16, device=dev) if vct is None else vct
    kbar = torch.empty(H, d, nkb, dtype=torch.float64, device=dev) if kbar is None else kbar
    radius = torch.empty(H, nkb, dtype=torch.float64, device=dev) if radius is None else radius
    _need(kc, "Kc", torch.bfloat16, ne)
    _need(vct, "Vct", torch.bfloat16, ne)
    _need(kbar, "kbar", torch.float64, H * nkb * d)
    _need(radius, "radius", torch.float64, H * nkb)
    _check(_lib.svg_ear_block_stats(ctypes.byref(dm), dt, _ptr(k), _ptr(vt), _ptr(kc), _ptr(vct), _ptr(kbar),
                                    _ptr(radius), _stream()), "svg_ear_block_stats")
    return kc, vct, kbar, radius


def svg_ear_route(q, labels, kbar, radius, block_mask, F, S, T, bq, bk, route_k, scale=-1.0, out=None):
    """The exact sets (uint8 [H][nQB][nKB]) from the block mask, the ragged
    last block and the route_k routed blocks per q-block."""
    dm = _video_dims(q, F, S, T, "Q")
    H, N, d = q.shape
    dt = _dtype(q)
    _need(q, "Q", torch.bfloat16, q.numel())
    _labels(labels, H)
    nqb, nkb = -(-N // bq), -(-N // 64)
    _need(kbar, "kbar", torch.float64, H * nkb * d)
    _need(radius, "radius", torch.float64, H * nkb)
    _need(block_mask, "block_mask", torch.uint8, H * nqb * nkb)
    out = torch.empty(H, nqb, nkb, dtype=torch.uint8, device=q.device) if out is None else out
    _need(out, "exact_mask", torch.uint8, H * nqb * nkb)
    _check(_lib.svg_ear_route(ctypes.byref(dm), dt, _ptr(q), _ptr(labels), _ptr(kbar), _ptr(radius),
                              _ptr(block_mask), bq, bk, int(route_k), scale, _ptr(out), _stream()), "svg_ear_route")
    return out


def svg_block_sparse_attn_ear_vt_layout(q, k, vt, kc, vct, row_ptr, kv_idx, labels, F, S, T, bq, bk, scale=-1.0,
                                        out=None):
    """Attention over the exact lists plus the centroid compensation of every
    other block; Q and O in the original order, K / Vt / lists / tables in the
    executing layout."""
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    H, N, d = q.shape
    ne = svg_ear_centroid_elems(H, N, d)
    _need(kc, "Kc", torch.bfloat16, ne)
    _need(vct, "Vct", torch.bfloat16, ne)
    _lists(row_ptr, kv_idx, H, N, bq)
    _labels(labels, H)
    out = _out_like(out, q)
    _check(_lib.svg_block_sparse_attn_ear_vt_layout(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt), _ptr(kc),
                                                    _ptr(vct), _ptr(row_ptr), _ptr(kv_idx), _ptr(labels), bq, bk,
                                                    scale, _ptr(out), _stream()),
           "svg_block_sparse_attn_ear_vt_layout")
    return out


# ----------------------------------------------------------------------------
# FP8 attention

def svg_quantize_fp8_rows(x, out=None, scale=None):
    """E4M3 codes (uint8 [H][N][d]) and per-row scales (float32 [H][N]) of a
    bf16 [H][N][d] tensor."""
    dm = _flat_dims(x)
    H, N, d = x.shape
    dt = _dtype(x)
    _need(x, "X", torch.bfloat16, x.numel())
    out = torch.empty(H, N, d, dtype=torch.uint8, device=x.device) if out is None else out
    scale = torch.empty(H, N, dtype=torch.float32, device=x.device) if scale is None else scale
    _need(out, "X8", torch.uint8, x.numel())
    _need(scale, "scale", torch.float32, H * N)
    _check(_lib.svg_quantize_fp8_rows(ctypes.byref(dm), dt, _ptr(x), _ptr(out), _ptr(scale), _stream()),
           "svg_quantize_fp8_rows")
    return out, scale


def svg_layout_permute_fp8(x, F, S, T, labels=None, out=None, scale=None):
    """x (bf16 [H][N][d]) in each head's executing layout as E4M3 codes, with
    one float32 scale per 64-row block ([H][ceil(N/64)])."""
    dm = _video_dims(x, F, S, T)
    H, N, d = x.shape
    dt = _dtype(x)
    _need(x, "X", torch.bfloat16, x.numel())
    _labels(labels, H)
    nkb = -(-N // 64)
    out = torch.empty(H, N, d, dtype=torch.uint8, device=x.device) if out is None else out
    scale = torch.empty(H, nkb, dtype=torch.float32, device=x.device) if scale is None else scale
    _need(out, "X8", torch.uint8, x.numel())
    _need(scale, "scale", torch.float32, H * nkb)
    _check(_lib.svg_layout_permute_fp8(ctypes.byref(dm), dt, _ptr(x), _ptr(out), _ptr(scale), _ptr(labels),
                                       _stream()), "svg_layout_permute_fp8")
    return out, scale


def _fp8_args(q8, qs, k8, ks, vt, F, S, T):
    dm = _video_dims(q8, F, S, T, "Q8")
    H, N, d = q8.shape
    _need(q8, "Q8", torch.uint8, H * N * d)
    _need(k8, "K8", torch.uint8, H * N * d)
    _need(qs, "qscale", torch.float32, H * N)
    _need(ks, "kscale", torch.float32, H * (-(-N // 64)))
    _need(vt, "Vt", torch.bfloat16, svg_vt_elems(H, N, d))
    return dm


def svg_block_sparse_attn_fp8_vt_layout(q8, qs, k8, ks, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk,
                                        scale=-1.0, out=None):
    """FP8 Q K^T (codes + scales from the two quantizers), bf16 P.V; Q8 and
    the returned O in the original token order, K8 / Vt / lists in the
    executing layout."""
    dm = _fp8_args(q8, qs, k8, ks, vt, F, S, T)
    H, N, d = q8.shape
    _lists(row_ptr, kv_idx, H, N, bq)
    _labels(labels, H)
    out = torch.empty(H, N, d, dtype=torch.bfloat16, device=q8.device) if out is None else out
    _need(out, "out", torch.bfloat16, H * N * d)
    _check(_lib.svg_block_sparse_attn_fp8_vt_layout(ctypes.byref(dm), _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks),
                                                    _ptr(vt), _ptr(row_ptr), _ptr(kv_idx), _ptr(labels), bq, bk,
                                                    scale, _ptr(out), _stream()),
           "svg_block_sparse_attn_fp8_vt_layout")
    return out


def svg_dense_attn_fp8_vt(q8, qs, k8, ks, vt, F, S, T, bq, bk, scale=-1.0, out=None):
    dm = _fp8_args(q8, qs, k8, ks, vt, F, S, T)
    H, N, d = q8.shape
    out = torch.empty(H, N, d, dtype=torch.bfloat16, device=q8.device) if out is None else out
    _need(out, "out", torch.bfloat16, H * N * d)
    _check(_lib.svg_dense_attn_fp8_vt(ctypes.byref(dm), _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks), _ptr(vt), bq, bk,
                                      scale, _ptr(out), _stream()), "svg_dense_attn_fp8_vt")
    return out


def svg_layout_permute_vt_fp8(v, F, S, T, labels=None, out=None, amax=None):
    """V (bf16 [H][N][128]) for the FP8 P.V mode: each channel's largest
    magnitude (float32 [H][128]) and the key-tiled V^T codes of the executing
    layout (uint8, ceil(N/64) tiles of 128 x 64 per head)."""
    dm = _video_dims(v, F, S, T, "V")
    H, N, d = v.shape
    dt = _dtype(v)
    _need(v, "V", torch.bfloat16, v.numel())
    _labels(labels, H)
    nt = svg_vt_elems(H, N, d)
    out = torch.empty(nt, dtype=torch.uint8, device=v.device) if out is None else out
    amax = torch.empty(H, d, dtype=torch.float32, device=v.device) if amax is None else amax
    _need(out, "Vt8", torch.uint8, nt)
    _need(amax, "vamax", torch.float32, H * d)
    _check(_lib.svg_layout_permute_vt_fp8(ctypes.byref(dm), dt, _ptr(v), _ptr(out), _ptr(amax), _ptr(labels),
                                          _stream()), "svg_layout_permute_vt_fp8")
    return out, amax


def svg_block_sparse_attn_fp8pv_vt_layout(q8, qs, k8, ks, vt8, vamax, row_ptr, kv_idx, labels, F, S, T, bq, bk,
                                          scale=-1.0, out=None):
    """The FP8 P.V mode: FP8 Q K^T as svg_block_sparse_attn_fp8_vt_layout,
    then probabilities coded after the lazy reference and P.V on the V codes
    (svg_layout_permute_vt_fp8); O bf16 in the original token order."""
    dm = _video_dims(q8, F, S, T, "Q8")
    H, N, d = q8.shape
    _need(q8, "Q8", torch.uint8, H * N * d)
    _need(k8, "K8", torch.uint8, H * N * d)
    _need(qs, "qscale", torch.float32, H * N)
    _need(ks, "kscale", torch.float32, H * (-(-N // 64)))
    _need(vt8, "Vt8", torch.uint8, svg_vt_elems(H, N, d))
    _need(vamax, "vamax", torch.float32, H * d)
    _lists(row_ptr, kv_idx, H, N, bq)
    _labels(labels, H)
    out = torch.empty(H, N, d, dtype=torch.bfloat16, device=q8.device) if out is None else out
    _need(out, "out", torch.bfloat16, H * N * d)
    _check(_lib.svg_block_sparse_attn_fp8pv_vt_layout(ctypes.byref(dm), _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks),
                                                      _ptr(vt8), _ptr(vamax), _ptr(row_ptr), _ptr(kv_idx),
                                                      _ptr(labels), bq, bk, scale, _ptr(out), _stream()),
           "svg_block_sparse_attn_fp8pv_vt_layout")
    return out


# ----------------------------------------------------------------------------
# SVG2 path

def _flat_dims(x, name="X"):
    H, N, d = _shape3(x, name)
    return svg_dims(1, N, 0, H, d)


def svg_kmeans(x, k, iters, init_idx, assign=None, centroids=None, sizes=None, ws=None):
    dm = _flat_dims(x)
    H, N, d = x.shape
    dt = _dtype(x)
    _need(x, "X", x.dtype, x.numel())
    dev = x.device
    _need(init_idx, "init_idx", torch.int32, H * k)
    assign = torch.empty(H, N, dtype=torch.int32, device=dev) if assign is None else assign
    centroids = torch.empty(H, k, d, dtype=torch.float64, device=dev) if centroids is None else centroids
    sizes = torch.empty(H, k, dtype=torch.int32, device=dev) if sizes is None else sizes
    _need(assign, "assign", torch.int32, H * N)
    _need(centroids, "centroids", torch.float64, H * k * d)
    _need(sizes, "sizes", torch.int32, H * k)
    ws = _ws(workspace_bytes(SVG2_OP_KMEANS, dm, k, svg2=True), dev, ws)
    _check(_lib.svg_kmeans(ctypes.byref(dm), dt, _ptr(x), k, iters, _ptr(init_idx), _ptr(assign),
                           _ptr(centroids), _ptr(sizes), _ptr(ws), _bytes(ws), _stream()), "svg_kmeans")
    return assign, centroids, sizes


def svg_cluster_permute(assign, k, d=64, perm=None, offs=None, ws=None):
    if not isinstance(assign, torch.Tensor) or assign.dim() != 2:
        raise ValueError("assign must be an int32 [H][N] tensor")
    H, N = assign.shape
    _need(assign, "assign", torch.int32, H * N)
    dm = svg_dims(1, N, 0, H, d)
    dev = assign.device
    perm = torch.empty(H, N, dtype=torch.int32, device=dev) if perm is None else perm
    offs = torch.empty(H, k + 1, dtype=torch.int32, device=dev) if offs is None else offs
    _need(perm, "perm", torch.int32, H * N)
    _need(offs, "offs", torch.int32, H * (k + 1))
    ws = _ws(workspace_bytes(SVG2_OP_CLUSTER_PERMUTE, dm, k, svg2=True), dev, ws)
    _check(_lib.svg_cluster_permute(ctypes.byref(dm), _ptr(assign), k, _ptr(perm), _ptr(offs), _ptr(ws),
                                    _bytes(ws), _stream()), "svg_cluster_permute")
    return perm, offs


def svg_permute_rows(x, perm, inverse=False, out=None):
    dm = _flat_dims(x)
    H, N, d = x.shape
    dt = _dtype(x)
    _need(x, "X", x.dtype, x.numel())
    _need(perm, "perm", torch.int32, H * N)
    out = _out_like(out, x)
    _check(_lib.svg_permute_rows(ctypes.byref(dm), dt, _ptr(x), _ptr(perm), _ptr(out), int(inverse),
                                 _stream()), "svg_permute_rows")
    return out


def svg_select_pairs(cq, ck, size_k, top_p, scale=-1.0, pair_ptr=None, pair_idx=None):
    H, kq, d = _shape3(cq, "cq")
    kk = _shape3(ck, "ck")[1]
    _need(cq, "cq", torch.float64, H * kq * d)
    _need(ck, "ck", torch.float64, H * kk * d)
    _need(size_k, "size_k", torch.int32, H * kk)
    dm = svg_dims(1, 1, 0, H, d)
    dev = cq.device
    pair_ptr = torch.empty(H, kq + 1, dtype=torch.int32, device=dev) if pair_ptr is None else pair_ptr
    pair_idx = torch.empty(H, kq * kk, dtype=torch.int32, device=dev) if pair_idx is None else pair_idx
    _need(pair_ptr, "pair_ptr", torch.int32, H * (kq + 1))
    _need(pair_idx, "pair_idx", torch.int32, H * kq * kk)
    _check(_lib.svg_select_pairs(ctypes.byref(dm), _ptr(cq), _ptr(ck), _ptr(size_k), kq, kk, float(top_p),
                                 scale, _ptr(pair_ptr), _ptr(pair_idx), _stream()), "svg_select_pairs")
    return pair_ptr, pair_idx


def _varlen_lists(qp, q_offs, k_offs, pair_ptr, pair_idx, q_perm):
    H, N, _ = qp.shape
    if not isinstance(q_offs, torch.Tensor) or q_offs.dim() != 2 or not isinstance(k_offs, torch.Tensor) \
            or k_offs.dim() != 2:
        raise ValueError("q_offs and k_offs must be int32 [H][k+1] tensors")
    kq, kk = q_offs.shape[1] - 1, k_offs.shape[1] - 1
    _need(q_offs, "q_offs", torch.int32, H * (kq + 1))
    _need(k_offs, "k_offs", torch.int32, H * (kk + 1))
    _need(pair_ptr, "pair_ptr", torch.int32, H * (kq + 1))
    _need(pair_idx, "pair_idx", torch.int32, H * kq * kk)
    _opt(q_perm, "q_perm", dtype=torch.int32, numel=H * N)
    return kq, kk


def svg_varlen_attn(qp, kp, vp, q_offs, k_offs, pair_ptr, pair_idx, q_perm=None, scale=-1.0, out=None, ws=None):
    dm = _flat_dims(qp, "Qp")
    H, N, d = qp.shape
    dt = _dtype(qp)
    for t, n in ((qp, "Qp"), (kp, "Kp"), (vp, "Vp")):
        _need(t, n, qp.dtype, H * N * d)
    kq, kk = _varlen_lists(qp, q_offs, k_offs, pair_ptr, pair_idx, q_perm)
    out = _out_like(out, qp)
    ws = _ws(workspace_bytes(SVG2_OP_VARLEN, dm, kq, kk, svg2=True), qp.device, ws)
    _check(_lib.svg_varlen_attn(ctypes.byref(dm), dt, _ptr(qp), _ptr(kp), _ptr(vp), _ptr(q_offs),
                                _ptr(k_offs), kq, kk, _ptr(pair_ptr), _ptr(pair_idx), _ptr(q_perm), scale,
                                _ptr(out), _ptr(ws), _bytes(ws), _stream()), "svg_varlen_attn")
    return out


def svg_permute_rows_vt(v, perm, out=None):
    """Key-tiled V^T ([H][nKB][d][64]) of the rows of v gathered by perm
    (row r of head h is v[h][perm[h][r]])."""
    dm = _flat_dims(v, "V")
    H, N, d = v.shape
    dt = _dtype(v)
    _need(v, "V", v.dtype, v.numel())
    _need(perm, "perm", torch.int32, H * N)
    out = torch.empty(H, -(-N // 64), d, 64, dtype=v.dtype, device=v.device) if out is None else out
    _need(out, "Vt", v.dtype, svg_vt_elems(H, N, d))
    _check(_lib.svg_permute_rows_vt(ctypes.byref(dm), dt, _ptr(v), _ptr(perm), _ptr(out), _stream()),
           "svg_permute_rows_vt")
    return out


def svg_varlen_attn_vt(qp, kp, vt, q_offs, k_offs, pair_ptr, pair_idx, q_perm=None, scale=-1.0, out=None):
    """svg_varlen_attn with V given as the key-tiled V^T of Vp."""
    dm = _flat_dims(qp, "Qp")
    H, N, d = qp.shape
    dt = _dtype(qp)
    for t, n in ((qp, "Qp"), (kp, "Kp")):
        _need(t, n, qp.dtype, H * N * d)
    _need(vt, "Vt", qp.dtype, svg_vt_elems(H, N, d))
    kq, kk = _varlen_lists(qp, q_offs, k_offs, pair_ptr, pair_idx, q_perm)
    out = _out_like(out, qp)
    _check(_lib.svg_varlen_attn_vt(ctypes.byref(dm), dt, _ptr(qp), _ptr(kp), _ptr(vt), _ptr(q_offs),
                                   _ptr(k_offs), kq, kk, _ptr(pair_ptr), _ptr(pair_idx), _ptr(q_perm), scale,
                                   _ptr(out), _stream()), "svg_varlen_attn_vt")
    return out


# ----------------------------------------------------------------------------
# HVA-style local-window clustering

def _win(win):
    w = (ctypes.c_int32 * 3)(*[int(v) for v in win])
    return w


def svg_hva_clusters(F, rows, cols, T, win, H=1, d=64):
    """Number of clusters of the window grid (windows plus the text cluster)."""
    return int(_lib.svg_hva_clusters(ctypes.byref(svg_dims(F, rows * cols, T, H, d)), rows, cols, _win(win)))


def svg_hva_cluster(x, F, rows, cols, T, win, iters, lowe_r2=0.64, assign=None, centroids=None, sizes=None,
                    refresh=None, ws=None):
    """Anchor step: local-window k-means of x [H][N][d] (bf16).  Returns
    assign [H][N], centroids [H][k][d] (float64), sizes [H][k], refresh
    flags [H][N] (uint8)."""
    dm = _video_dims(x, F, rows * cols, T)
    H, N, d = x.shape
    dt = _dtype(x)
    _need(x, "X", x.dtype, x.numel())
    k = svg_hva_clusters(F, rows, cols, T, win, H, d)
    if k < 1:
        raise SvgError(-1, f"svg_hva_clusters: {last_error()}")
    dev = x.device
    assign = torch.empty(H, N, dtype=torch.int32, device=dev) if assign is None else assign
    centroids = torch.empty(H, k, d, dtype=torch.float64, device=dev) if centroids is None else centroids
    sizes = torch.empty(H, k, dtype=torch.int32, device=dev) if sizes is None else sizes
    refresh = torch.empty(H, N, dtype=torch.uint8, device=dev) if refresh is None else refresh
    _need(assign, "assign", torch.int32, H * N)
    _need(centroids, "centroids", torch.float64, H * k * d)
    _need(sizes, "sizes", torch.int32, H * k)
    _need(refresh, "refresh", torch.uint8, H * N)
    ws = _ws(workspace_bytes(SVG2_OP_HVA, dm, k, svg2=True), dev, ws)
    _check(_lib.svg_hva_cluster(ctypes.byref(dm), dt, _ptr(x), rows, cols, _win(win), iters, float(lowe_r2),
                                _ptr(assign), _ptr(centroids), _ptr(sizes), _ptr(refresh), _ptr(ws), _bytes(ws),
                                _stream()), "svg_hva_cluster")
    return assign, centroids, sizes, refresh


def svg_hva_refresh(x, F, rows, cols, T, win, refresh, assign, centroids, sizes=None, ws=None):
    """Non-anchor step: flagged tokens re-assigned against the carried
    centroids, then one update from x; assign and centroids in place.
    Returns (assign, centroids, sizes)."""
    dm = _video_dims(x, F, rows * cols, T)
    H, N, d = x.shape
    dt = _dtype(x)
    _need(x, "X", x.dtype, x.numel())
    k = svg_hva_clusters(F, rows, cols, T, win, H, d)
    if k < 1:
        raise SvgError(-1, f"svg_hva_clusters: {last_error()}")
    sizes = torch.empty(H, k, dtype=torch.int32, device=x.device) if sizes is None else sizes
    _need(refresh, "refresh", torch.uint8, H * N)
    _need(assign, "assign", torch.int32, H * N)
    _need(centroids, "centroids", torch.float64, H * k * d)
    _need(sizes, "sizes", torch.int32, H * k)
    ws = _ws(workspace_bytes(SVG2_OP_HVA, dm, k, svg2=True), x.device, ws)
    _check(_lib.svg_hva_refresh(ctypes.byref(dm), dt, _ptr(x), rows, cols, _win(win), _ptr(refresh), _ptr(assign),
                                _ptr(centroids), _ptr(sizes), _ptr(ws), _bytes(ws), _stream()), "svg_hva_refresh")
    return assign, centroids, sizes
