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
SVG_OP_PROFILE, SVG_OP_BLOCK_SPARSE, SVG_OP_COMPACT, SVG_OP_ATTN_VT = 0, 1, 2, 3
SVG2_OP_KMEANS, SVG2_OP_CLUSTER_PERMUTE, SVG2_OP_VARLEN = 0, 1, 2


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
    "svg_block_sparse_attn_csr": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg_dense_attn": [_DIMS, _I, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg_vt_elems": [_DIMS],
    "svg_layout_permute_vt": [_DIMS, _I, _P, _P, _P, _P],
    "svg_block_sparse_attn_csr_vt": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P, _Z, _P],
    "svg_block_sparse_attn_csr_vt_layout": [_DIMS, _I, _P, _P, _P, _P, _P, _P, _I, _I, _F, _P, _P, _Z, _P],
    "svg_dense_attn_vt": [_DIMS, _I, _P, _P, _P, _I, _I, _F, _P, _P],
    "svg2_workspace_bytes": [_I, _DIMS, _I, _I],
    "svg_kmeans": [_DIMS, _I, _P, _I, _I, _P, _P, _P, _P, _P, _Z, _P],
    "svg_cluster_permute": [_DIMS, _P, _I, _P, _P, _P, _Z, _P],
    "svg_permute_rows": [_DIMS, _I, _P, _P, _P, _I, _P],
    "svg_select_pairs": [_DIMS, _P, _P, _P, _I, _I, _D, _F, _P, _P, _P],
    "svg_varlen_attn": [_DIMS, _I, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P, _F, _P, _P, _Z, _P],
}
_RESTYPES = {"svg_workspace_bytes": _Z, "svg2_workspace_bytes": _Z, "svg_vt_elems": _Z,
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
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype(t):
    if t.dtype == torch.bfloat16:
        return SVG_BF16
    if t.dtype == torch.float32:
        return SVG_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t, name, dtype=None, numel=None):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


def dims(F, S, T, H, d):
    return svg_dims(F, S, T, H, d)


def _qkv(q, k, v, F, S, T):
    H, N, d = q.shape
    if N != F * S + T:
        raise ValueError(f"N={N} != F*S+T={F * S + T}")
    for t, n in ((q, "Q"), (k, "K"), (v, "V")):
        _need(t, n, q.dtype, H * N * d)
    return svg_dims(F, S, T, H, d), _dtype(q)


def workspace_bytes(op, dm, a=0, b=0, svg2=False):
    fn = _lib.svg2_workspace_bytes if svg2 else _lib.svg_workspace_bytes
    return fn(op, ctypes.byref(dm), a, b)


def _ws(nbytes, device, ws=None):
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------
# SVG1 path

def svg_profile_heads(q, k, v, sample_idx, F, S, T, ks, wt, scale=-1.0, labels=None, mse=None, ws=None):
    dm, dt = _qkv(q, k, v, F, S, T)
    H = q.shape[0]
    _need(sample_idx, "sample_idx", torch.int32)
    labels = torch.empty(H, dtype=torch.int32, device=q.device) if labels is None else labels
    mse = torch.empty(H, 2, dtype=torch.float32, device=q.device) if mse is None else mse
    mp = svg_mask_params(ks, wt)
    need = workspace_bytes(SVG_OP_PROFILE, dm, sample_idx.numel())
    ws = _ws(need, q.device, ws)
    _check(_lib.svg_profile_heads(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(sample_idx),
                                  sample_idx.numel(), ctypes.byref(mp), scale, _ptr(labels), _ptr(mse),
                                  _ptr(ws), ws.numel(), _stream()), "svg_profile_heads")
    return labels, mse


def svg_layout_permute(x, F, S, T, labels=None, out=None):
    H, N, d = x.shape
    dm = svg_dims(F, S, T, H, d)
    out = torch.empty_like(x) if out is None else out
    _check(_lib.svg_layout_permute(ctypes.byref(dm), _dtype(x), _ptr(x), _ptr(out), _ptr(labels), _stream()),
           "svg_layout_permute")
    return out


def svg_layout_unpermute(x, F, S, T, labels=None, out=None):
    H, N, d = x.shape
    dm = svg_dims(F, S, T, H, d)
    out = torch.empty_like(x) if out is None else out
    _check(_lib.svg_layout_unpermute(ctypes.byref(dm), _dtype(x), _ptr(x), _ptr(out), _ptr(labels), _stream()),
           "svg_layout_unpermute")
    return out


def svg_build_block_mask(labels, F, S, T, H, d, ks, wt, bq, bk, out=None):
    dm = svg_dims(F, S, T, H, d)
    N = F * S + T
    nqb, nkb = -(-N // bq), -(-N // bk)
    out = torch.empty(H, nqb, nkb, dtype=torch.uint8, device=labels.device) if out is None else out
    mp = svg_mask_params(ks, wt)
    _check(_lib.svg_build_block_mask(ctypes.byref(dm), ctypes.byref(mp), _ptr(labels), bq, bk, _ptr(out),
                                     _stream()), "svg_build_block_mask")
    return out


def svg_compact_block_mask(block_mask, row_ptr=None, kv_idx=None, ws=None):
    nkb = block_mask.shape[-1]
    rows = block_mask.numel() // nkb
    dev = block_mask.device
    row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=dev) if row_ptr is None else row_ptr
    kv_idx = torch.empty(max(rows * nkb, 1), dtype=torch.int32, device=dev) if kv_idx is None else kv_idx
    ws = _ws(_lib.svg_workspace_bytes(SVG_OP_COMPACT, None, rows, nkb), dev, ws)
    _check(_lib.svg_compact_block_mask(rows, nkb, _ptr(block_mask), _ptr(row_ptr), _ptr(kv_idx), _ptr(ws),
                                       ws.numel(), _stream()), "svg_compact_block_mask")
    return row_ptr, kv_idx


def svg_block_sparse_attn(q, k, v, block_mask, F, S, T, bq, bk, scale=-1.0, out=None, ws=None):
    dm, dt = _qkv(q, k, v, F, S, T)
    out = torch.empty_like(q) if out is None else out
    ws = _ws(workspace_bytes(SVG_OP_BLOCK_SPARSE, dm, bq, bk), q.device, ws)
    _check(_lib.svg_block_sparse_attn(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(block_mask), bq, bk,
                                      scale, _ptr(out), _ptr(ws), ws.numel(), _stream()), "svg_block_sparse_attn")
    return out


def svg_block_sparse_attn_csr(q, k, v, row_ptr, kv_idx, F, S, T, bq, bk, scale=-1.0, out=None):
    dm, dt = _qkv(q, k, v, F, S, T)
    out = torch.empty_like(q) if out is None else out
    _check(_lib.svg_block_sparse_attn_csr(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(v), _ptr(row_ptr),
                                          _ptr(kv_idx), bq, bk, scale, _ptr(out), _stream()),
           "svg_block_sparse_attn_csr")
    return out


def svg_dense_attn(q, k, v, F, S, T, bq, bk, scale=-1.0, out=None):
    dm, dt = _qkv(q, k, v, F, S, T)
    out = torch.empty_like(q) if out is None else out
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
    H, N, d = v.shape
    dm = svg_dims(F, S, T, H, d)
    nkb = -(-N // 64)
    out = torch.empty(H, nkb, d, 64, dtype=v.dtype, device=v.device) if out is None else out
    _need(out, "Vt", v.dtype, svg_vt_elems(H, N, d))
    _check(_lib.svg_layout_permute_vt(ctypes.byref(dm), _dtype(v), _ptr(v), _ptr(out), _ptr(labels), _stream()),
           "svg_layout_permute_vt")
    return out


def _qk_vt(q, k, vt, F, S, T):
    H, N, d = q.shape
    if N != F * S + T:
        raise ValueError(f"N={N} != F*S+T={F * S + T}")
    for t, n in ((q, "Q"), (k, "K")):
        _need(t, n, q.dtype, H * N * d)
    _need(vt, "Vt", q.dtype, svg_vt_elems(H, N, d))
    return svg_dims(F, S, T, H, d), _dtype(q)


def attn_vt_workspace(q, F, S, T, bq, bk):
    """Workspace for the split text groups of the sparse V^T attention
    entries (None when no split applies)."""
    n = workspace_bytes(SVG_OP_ATTN_VT, svg_dims(F, S, T, q.shape[0], q.shape[2]), bq, bk)
    return torch.empty(n, dtype=torch.uint8, device=q.device) if n > 0 else None


def svg_block_sparse_attn_csr_vt(q, k, vt, row_ptr, kv_idx, F, S, T, bq, bk, scale=-1.0, out=None, ws=None):
    """ws: from attn_vt_workspace (allocated here when None)."""
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    out = torch.empty_like(q) if out is None else out
    ws = attn_vt_workspace(q, F, S, T, bq, bk) if ws is None else ws
    _check(_lib.svg_block_sparse_attn_csr_vt(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt), _ptr(row_ptr),
                                             _ptr(kv_idx), bq, bk, scale, _ptr(out), _ptr(ws),
                                             0 if ws is None else ws.numel() * ws.element_size(), _stream()),
           "svg_block_sparse_attn_csr_vt")
    return out


def svg_block_sparse_attn_csr_vt_layout(q, k, vt, row_ptr, kv_idx, labels, F, S, T, bq, bk, scale=-1.0,
                                        out=None, ws=None):
    """Q and the returned O in the original token order; K, Vt and the lists
    in each head's executing layout per labels (None: every head temporal).
    ws: from attn_vt_workspace (allocated here when None)."""
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    out = torch.empty_like(q) if out is None else out
    ws = attn_vt_workspace(q, F, S, T, bq, bk) if ws is None else ws
    _check(_lib.svg_block_sparse_attn_csr_vt_layout(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt),
                                                    _ptr(row_ptr), _ptr(kv_idx), _ptr(labels), bq, bk, scale,
                                                    _ptr(out), _ptr(ws),
                                                    0 if ws is None else ws.numel() * ws.element_size(),
                                                    _stream()),
           "svg_block_sparse_attn_csr_vt_layout")
    return out


def svg_dense_attn_vt(q, k, vt, F, S, T, bq, bk, scale=-1.0, out=None):
    dm, dt = _qk_vt(q, k, vt, F, S, T)
    out = torch.empty_like(q) if out is None else out
    _check(_lib.svg_dense_attn_vt(ctypes.byref(dm), dt, _ptr(q), _ptr(k), _ptr(vt), bq, bk, scale, _ptr(out),
                                  _stream()), "svg_dense_attn_vt")
    return out


# ----------------------------------------------------------------------------
# SVG2 path

def _flat_dims(x):
    H, N, d = x.shape
    return svg_dims(1, N, 0, H, d)


def svg_kmeans(x, k, iters, init_idx, assign=None, centroids=None, sizes=None, ws=None):
    H, N, d = x.shape
    dm = _flat_dims(x)
    dev = x.device
    _need(init_idx, "init_idx", torch.int32, H * k)
    assign = torch.empty(H, N, dtype=torch.int32, device=dev) if assign is None else assign
    centroids = torch.empty(H, k, d, dtype=torch.float64, device=dev) if centroids is None else centroids
    sizes = torch.empty(H, k, dtype=torch.int32, device=dev) if sizes is None else sizes
    ws = _ws(workspace_bytes(SVG2_OP_KMEANS, dm, k, svg2=True), dev, ws)
    _check(_lib.svg_kmeans(ctypes.byref(dm), _dtype(x), _ptr(x), k, iters, _ptr(init_idx), _ptr(assign),
                           _ptr(centroids), _ptr(sizes), _ptr(ws), ws.numel(), _stream()), "svg_kmeans")
    return assign, centroids, sizes


def svg_cluster_permute(assign, k, d=64, perm=None, offs=None, ws=None):
    H, N = assign.shape
    dm = svg_dims(1, N, 0, H, d)
    dev = assign.device
    perm = torch.empty(H, N, dtype=torch.int32, device=dev) if perm is None else perm
    offs = torch.empty(H, k + 1, dtype=torch.int32, device=dev) if offs is None else offs
    ws = _ws(workspace_bytes(SVG2_OP_CLUSTER_PERMUTE, dm, k, svg2=True), dev, ws)
    _check(_lib.svg_cluster_permute(ctypes.byref(dm), _ptr(assign), k, _ptr(perm), _ptr(offs), _ptr(ws),
                                    ws.numel(), _stream()), "svg_cluster_permute")
    return perm, offs


def svg_permute_rows(x, perm, inverse=False, out=None):
    dm = _flat_dims(x)
    out = torch.empty_like(x) if out is None else out
    _check(_lib.svg_permute_rows(ctypes.byref(dm), _dtype(x), _ptr(x), _ptr(perm), _ptr(out), int(inverse),
                                 _stream()), "svg_permute_rows")
    return out


def svg_select_pairs(cq, ck, size_k, top_p, scale=-1.0, pair_ptr=None, pair_idx=None):
    H, kq, d = cq.shape
    kk = ck.shape[1]
    dm = svg_dims(1, 1, 0, H, d)
    dev = cq.device
    pair_ptr = torch.empty(H, kq + 1, dtype=torch.int32, device=dev) if pair_ptr is None else pair_ptr
    pair_idx = torch.empty(H, kq * kk, dtype=torch.int32, device=dev) if pair_idx is None else pair_idx
    _check(_lib.svg_select_pairs(ctypes.byref(dm), _ptr(cq), _ptr(ck), _ptr(size_k), kq, kk, float(top_p),
                                 scale, _ptr(pair_ptr), _ptr(pair_idx), _stream()), "svg_select_pairs")
    return pair_ptr, pair_idx


def svg_varlen_attn(qp, kp, vp, q_offs, k_offs, pair_ptr, pair_idx, q_perm=None, scale=-1.0, out=None, ws=None):
    H, N, d = qp.shape
    kq, kk = q_offs.shape[1] - 1, k_offs.shape[1] - 1
    dm = _flat_dims(qp)
    out = torch.empty_like(qp) if out is None else out
    ws = _ws(workspace_bytes(SVG2_OP_VARLEN, dm, kq, kk, svg2=True), qp.device, ws)
    _check(_lib.svg_varlen_attn(ctypes.byref(dm), _dtype(qp), _ptr(qp), _ptr(kp), _ptr(vp), _ptr(q_offs),
                                _ptr(k_offs), kq, kk, _ptr(pair_ptr), _ptr(pair_idx), _ptr(q_perm), scale,
                                _ptr(out), _ptr(ws), ws.numel(), _stream()), "svg_varlen_attn")
    return out
