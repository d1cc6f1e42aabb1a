"""Seeded synthetic inputs (shapes and value distributions only)."""
from .configs import Workload, WORKLOADS, TINY, COG, HUNYUAN, HUNYUAN_LAYER, SVG2_COG, SMOKE_BF16  # noqa: F401
