"""MI355X (gfx950) sparse video attention: Sparse VideoGen's hot path as
hand-written HIP kernels behind a C ABI (include/svg.h, include/svg2.h).

The Python side is the ctypes binding in ``svg`` (argument marshalling only).
"""
from . import svg  # noqa: F401  (raises if libsvg_hip.so is not built)
