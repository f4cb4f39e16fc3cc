"""MI355X (gfx950) Video Sparse Attention hot path: cube tiling, coarse
selector and fine block-sparse attention, in HIP kernels behind the C ABI of
include/vsa.h. This package holds the kernels' sources (csrc/), the build
script and a thin torch/ctypes binding."""
from .ops import (default_scale, fwd, fwd_lut, fwd_workspace_bytes, num_cubes, select, select_cdf,
                  select_workspace_bytes,  # noqa: F401
                  tile, untile, validate_topk, vbs_host)
