"""CPU oracle for the sparse video attention path (TEST INFRASTRUCTURE).

This package is test infrastructure.  Only the tests, the smoke check and the
bench's CPU-baseline leg may import or call it.  The GPU library never routes
through it.  It shares no code with the HIP path.

It is a plain, slow, float64 restatement of what the path computes.  The
sources are:

* the SVG1 abstract ("Sparse VideoGen: Accelerating Video Diffusion
  Transformers with Spatial-Temporal Sparsity", English abstract on the
  arxivdaily listing).  It says attention heads fall into a spatial group
  (tokens of the query's own frame dominate) and a temporal group (tokens at
  the same place in other frames dominate).  An online profiling step predicts
  each head's group.  A tensor layout transformation and custom kernels
  exploit the pattern.
* the Sparse-VideoGen project write-up ("Sparse-VideoGen and the sparsity
  hiding inside video diffusion attention"):
  - its section "Three generations of the same idea" covers SVG1 profiling
    and layout.  It also covers SVG2: semantic-aware permutation, a dynamic
    attention kernel and flash k-means.
  - its install section covers block-sparse attention with varied block sizes
    and the bundled batched k-means.

Where the pages leave a step open, the oracle takes the readings stated in
the design notes.  Each function's docstring names the reading it uses.

Modules:
  attention -- dense, masked and block-sparse softmax attention
  masks     -- spatial / temporal token masks, block bitmaps, CSR lists
  layout    -- frame-major <-> position-major permutation
  profile   -- online head profiling (sampled-row MSE, label)
  svg2      -- k-means, cluster permutation, top-p pairs, varlen attention
  fp8       -- E4M3 quantization (per-token Q, per-key-block K scales) and
               block-sparse attention over the dequantized values
  ear       -- SVG-EAR: block centroids, error-aware routing, compensated
               attention
"""

from . import attention, masks, layout, profile, svg2, fp8, ear  # noqa: F401
from .numerics import bf16_bits_to_f64  # noqa: F401
