"""Seeded synthetic inputs (shapes and value distributions only)."""
from .configs import Workload, WORKLOADS, TINY, COG, SMALL_FRAMES, HUNYUAN, HUNYUAN_LAYER, SVG2_COG, HVA_COG, SMOKE_BF16  # noqa: F401
