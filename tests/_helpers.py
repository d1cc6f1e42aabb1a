"""Shared helpers for the GPU parity tests: upload seeded inputs, download
outputs, and the tolerance checks."""

import numpy as np
import torch

from oracle.numerics import as_f64

DEV = "cuda:0"

# bf16 attention outputs against the float64 oracle
BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 1e-2
# fp32 attention outputs against the float64 oracle: one fp32 rounding per
# accumulated term over <= a few thousand terms
F32_MAX_ABS, F32_REL_L2 = 1e-4, 1e-5


def to_dev(x: np.ndarray, dtype: str):
    """Stored tensor (bf16 bits as uint16, or float32) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def to_host_bits(t):
    """Device tensor -> stored form (uint16 bits for bf16, float32 otherwise)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def to_f64(t):
    if t.dtype == torch.bfloat16:
        return as_f64(to_host_bits(t), "bf16")
    return t.double().cpu().numpy()


def ints(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(DEV)


def check_close(got, ref, max_abs, rel_l2, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    rl2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    assert mx <= max_abs and rl2 <= rel_l2, f"{what}: max-abs {mx:.3e} rel-L2 {rl2:.3e}"
    return mx, rl2


def exact_sum_span_ok(x64, assign, k):
    """Whether every cluster's member sums are exact in float64 in any order:
    for bf16 members (8-bit significands) the exponent span of a dimension's
    nonzero values must be at most 45 - log2(cluster size)."""
    e = np.frexp(x64)[1]
    nz = x64 != 0
    for j in range(k):
        m = assign == j
        n = int(m.sum())
        if n == 0:
            continue
        ej, nzj = e[m], nz[m]
        hi = np.where(nzj, ej, -10 ** 6).max(axis=0)
        lo = np.where(nzj, ej, 10 ** 6).min(axis=0)
        span = np.where(hi >= lo, hi - lo, 0)
        if span.max() > 45 - np.log2(n):
            return False
    return True
