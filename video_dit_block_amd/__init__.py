"""MI355X (gfx950) Video Sparse Attention hot path: cube tiling, coarse
selector, fine block-sparse attention, the coarse-stage output and the gated
combine, in HIP kernels behind the C ABI of include/vsa.h. This package holds
the kernels' sources (csrc/), the build script and a thin torch/ctypes
binding."""
from .ops import (coarse, coarse_workspace_bytes, cube_order, default_scale, fwd,  # noqa: F401
                  fwd_lut, fwd_splits, fwd_workspace_bytes, gate_combine, mask_to_lut,
                  num_cubes, select, select_cdf, select_noalloc, select_noalloc_max_bytes,
                  select_workspace_bytes, tile, untile, validate_topk, vbs_host)
