"""Python binding of libvsa: argument marshalling only.

Each function takes torch tensors on the GPU, checks dtypes/shapes, allocates
outputs with torch (device memory is PyTorch's job here) and calls the C ABI
on torch's current stream. Every step of the computation runs in libvsa's HIP
kernels.
"""
from __future__ import annotations

import math

import torch

from . import _lib

CUBE = 64


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _bf16(t: torch.Tensor, name: str, ndim: int = 4) -> None:
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != ndim:
        raise ValueError(f"{name} must be a contiguous {ndim}-d bfloat16 CUDA tensor, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def _i32(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 CUDA tensor")


def _shape(t: torch.Tensor, shape: tuple, name: str) -> None:
    """Caller-supplied buffers must have exactly the shape the C call writes
    (a smaller one would be written past its end on the device)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _numel(t: torch.Tensor, n: int, name: str) -> None:
    if t.numel() != n:
        raise ValueError(f"{name} must hold {n} entries, got {t.numel()}")


def num_cubes(T: int, H: int, W: int) -> int:
    n = _lib.load().vsa_num_cubes(T, H, W)
    if n < 0:
        raise ValueError(f"bad grid {T}x{H}x{W}")
    return n


def vbs_host(T: int, H: int, W: int) -> torch.Tensor:
    """Real tokens per cube, computed on the host (int32 CPU tensor)."""
    n = num_cubes(T, H, W)
    out = torch.empty(n, dtype=torch.int32)
    _lib.check(_lib.load().vsa_vbs_host(T, H, W, out.data_ptr(), n), "vsa_vbs_host")
    return out


def cube_order(T: int, H: int, W: int, kind: str = "hilbert") -> torch.Tensor:
    """Cube order table (int32 CPU tensor (Nc,)): entry p is the row-major id of
    the cube placed at tiled position p. kind: "row_major" or "hilbert"."""
    kinds = {"row_major": _lib.VSA_ORDER_ROW_MAJOR, "hilbert": _lib.VSA_ORDER_HILBERT}
    if kind not in kinds:
        raise ValueError(f"kind must be one of {sorted(kinds)}")
    n = num_cubes(T, H, W)
    out = torch.empty(n, dtype=torch.int32)
    _lib.check(_lib.load().vsa_cube_order_host(T, H, W, kinds[kind], out.data_ptr(), n),
               "vsa_cube_order_host")
    return out


def _order(order: torch.Tensor | None, nc: int) -> None:
    if order is not None:
        _i32(order, "order")
        if order.numel() != nc:
            raise ValueError(f"order must hold Nc = {nc} entries")


def tile(x: torch.Tensor, T: int, H: int, W: int, out: torch.Tensor | None = None,
         vbs: torch.Tensor | None = None,
         order: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """(B, T*H*W, NH, D) natural order -> ((B, Nc*64, NH, D) tiled, vbs int32 (Nc,)).
    ``order`` (device int32 (Nc,), from ``cube_order``) places row-major cube
    order[p] at tiled position p."""
    _bf16(x, "x")
    B, N, NH, D = x.shape
    if N != T * H * W:
        raise ValueError(f"x has {N} tokens, grid {T}x{H}x{W} has {T * H * W}")
    nc = num_cubes(T, H, W)
    if out is None:
        out = torch.empty((B, nc * CUBE, NH, D), dtype=torch.bfloat16, device=x.device)
    _bf16(out, "out")
    _shape(out, (B, nc * CUBE, NH, D), "out")
    if vbs is None:
        vbs = torch.empty(nc, dtype=torch.int32, device=x.device)
    _i32(vbs, "vbs")
    _numel(vbs, nc, "vbs")
    _order(order, nc)
    if order is None:
        _lib.check(_lib.load().vsa_tile(x.data_ptr(), out.data_ptr(), vbs.data_ptr(), B, T, H, W,
                                        NH, D, _stream()), "vsa_tile")
    else:
        _lib.check(_lib.load().vsa_tile_ordered(x.data_ptr(), out.data_ptr(), vbs.data_ptr(),
                                                order.data_ptr(), B, T, H, W, NH, D, _stream()),
                   "vsa_tile_ordered")
    return out, vbs


def untile(y: torch.Tensor, T: int, H: int, W: int, out: torch.Tensor | None = None,
           order: torch.Tensor | None = None) -> torch.Tensor:
    """(B, Nc*64, NH, D) tiled -> (B, T*H*W, NH, D) natural order (``order``: the
    table the tensor was tiled with)."""
    _bf16(y, "y")
    B, S, NH, D = y.shape
    if S != num_cubes(T, H, W) * CUBE:
        raise ValueError("tiled length does not match the grid")
    if out is None:
        out = torch.empty((B, T * H * W, NH, D), dtype=torch.bfloat16, device=y.device)
    _bf16(out, "out")
    _shape(out, (B, T * H * W, NH, D), "out")
    _order(order, S // CUBE)
    if order is None:
        _lib.check(_lib.load().vsa_untile(y.data_ptr(), out.data_ptr(), B, T, H, W, NH, D,
                                          _stream()), "vsa_untile")
    else:
        _lib.check(_lib.load().vsa_untile_ordered(y.data_ptr(), out.data_ptr(), order.data_ptr(),
                                                  B, T, H, W, NH, D, _stream()),
                   "vsa_untile_ordered")
    return out


def select_workspace_bytes(B: int, NH: int, Nc: int, D: int) -> int:
    return int(_lib.load().vsa_select_workspace_bytes(B, NH, Nc, D))


def select(q_t: torch.Tensor, k_t: torch.Tensor, vbs: torch.Tensor, topk: int,
           workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """Coarse selector: topk_idx int32 (B, NH, Nc, topk)."""
    _bf16(q_t, "q_t")
    _bf16(k_t, "k_t")
    _i32(vbs, "vbs")
    B, S, NH, D = q_t.shape
    Nc = S // CUBE
    if k_t.shape != q_t.shape or S % CUBE:
        raise ValueError("q_t and k_t must both be (B, Nc*64, NH, D)")
    _numel(vbs, Nc, "vbs")
    need = select_workspace_bytes(B, NH, Nc, D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q_t.device)
    if out is None:
        out = torch.empty((B, NH, Nc, topk), dtype=torch.int32, device=q_t.device)
    _i32(out, "out")
    _shape(out, (B, NH, Nc, topk), "out")
    _lib.check(_lib.load().vsa_select(q_t.data_ptr(), k_t.data_ptr(), vbs.data_ptr(), B, Nc, NH,
                                      D, topk, out.data_ptr(), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), _stream()),
               "vsa_select")
    return out


def select_noalloc(q_t: torch.Tensor, k_t: torch.Tensor, vbs: torch.Tensor, topk: int,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """The coarse selector without a workspace (vsa_select_noalloc): the same
    topk_idx int32 (B, NH, Nc, topk) as ``select``, computed in the library's
    static per-GPU scratch. With ``out`` given, nothing is allocated."""
    _bf16(q_t, "q_t")
    _bf16(k_t, "k_t")
    _i32(vbs, "vbs")
    B, S, NH, D = q_t.shape
    Nc = S // CUBE
    if k_t.shape != q_t.shape or S % CUBE:
        raise ValueError("q_t and k_t must both be (B, Nc*64, NH, D)")
    _numel(vbs, Nc, "vbs")
    if out is None:
        out = torch.empty((B, NH, Nc, topk), dtype=torch.int32, device=q_t.device)
    _i32(out, "out")
    _shape(out, (B, NH, Nc, topk), "out")
    _lib.check(_lib.load().vsa_select_noalloc(q_t.data_ptr(), k_t.data_ptr(), vbs.data_ptr(), B,
                                              Nc, NH, D, topk, out.data_ptr(), _stream()),
               "vsa_select_noalloc")
    return out


def select_noalloc_max_bytes() -> int:
    """Size of the static per-GPU scratch of select_noalloc."""
    return int(_lib.load().vsa_select_noalloc_max_bytes())


def select_cdf(q_t: torch.Tensor, k_t: torch.Tensor, vbs: torch.Tensor, max_k: int, tau: float,
               sm_scale: float | None = None, workspace: torch.Tensor | None = None):
    """Coarse selector with a cumulative softmax-mass threshold: returns
    (kv_block_idx int32 (B, NH, Nc, max_k), valid_block_num int32 (B, NH, Nc))."""
    _bf16(q_t, "q_t")
    _bf16(k_t, "k_t")
    _i32(vbs, "vbs")
    B, S, NH, D = q_t.shape
    Nc = S // CUBE
    if k_t.shape != q_t.shape or S % CUBE:
        raise ValueError("q_t and k_t must both be (B, Nc*64, NH, D)")
    _numel(vbs, Nc, "vbs")
    if workspace is None:
        workspace = torch.empty(select_workspace_bytes(B, NH, Nc, D), dtype=torch.uint8,
                                device=q_t.device)
    idx = torch.empty((B, NH, Nc, max_k), dtype=torch.int32, device=q_t.device)
    valid = torch.empty((B, NH, Nc), dtype=torch.int32, device=q_t.device)
    scale = 0.0 if sm_scale is None else float(sm_scale)
    _lib.check(_lib.load().vsa_select_cdf(q_t.data_ptr(), k_t.data_ptr(), vbs.data_ptr(), B, Nc,
                                          NH, D, max_k, float(tau), scale, idx.data_ptr(),
                                          valid.data_ptr(), workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(),
                                          _stream()),
               "vsa_select_cdf")
    return idx, valid


def fwd_workspace_bytes(B: int, Nq: int, Nkv: int, NH: int, D: int, topk: int,
                        kv_splits: int = 0) -> int:
    return int(_lib.load().vsa_fwd_workspace_bytes_ex(B, Nq, Nkv, NH, D, topk, kv_splits))


def fwd_splits(Nkv: int, D: int, topk: int, kv_splits: int = 0) -> int:
    """Key-range splits the fine stage uses (0 = invalid arguments)."""
    return int(_lib.load().vsa_fwd_splits(Nkv, D, topk, kv_splits))


def fwd(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, topk_idx: torch.Tensor,
        vbs: torch.Tensor, sm_scale: float | None = None,
        out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Fine block-sparse attention: (B, Nq*64, NH, D) bf16."""
    for t, n in ((q_t, "q_t"), (k_t, "k_t"), (v_t, "v_t")):
        _bf16(t, n)
    _i32(topk_idx, "topk_idx")
    _i32(vbs, "vbs")
    B, Sq, NH, D = q_t.shape
    Skv = k_t.shape[1]
    if v_t.shape != k_t.shape or k_t.shape[0] != B or k_t.shape[2:] != q_t.shape[2:]:
        raise ValueError("k_t and v_t must be (B, Nkv*64, NH, D) matching q_t")
    if Sq % CUBE or Skv % CUBE:
        raise ValueError("sequence lengths must be multiples of 64")
    Nq, Nkv = Sq // CUBE, Skv // CUBE
    if topk_idx.dim() != 4 or tuple(topk_idx.shape[:3]) != (B, NH, Nq):
        raise ValueError(f"topk_idx must be (B, NH, Nq, topk) = ({B}, {NH}, {Nq}, k)")
    if vbs.numel() != Nkv:
        raise ValueError(f"vbs must hold Nkv = {Nkv} entries")
    topk = topk_idx.shape[3]
    if out is None:
        out = torch.empty_like(q_t)
    _bf16(out, "out")
    _shape(out, tuple(q_t.shape), "out")
    scale = 0.0 if sm_scale is None else float(sm_scale)
    if workspace is None:
        workspace = torch.empty(fwd_workspace_bytes(B, Nq, Nkv, NH, D, topk),
                                dtype=torch.uint8, device=q_t.device)
    _lib.check(_lib.load().vsa_fwd(q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(),
                                   topk_idx.data_ptr(), vbs.data_ptr(), out.data_ptr(), B, Nq,
                                   Nkv, NH, D, topk, scale, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), _stream()),
               "vsa_fwd")
    return out


def fwd_lut(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor,
            kv_block_idx: torch.Tensor, valid_block_num: torch.Tensor | None, vbs: torch.Tensor,
            sm_scale: float | None = None, stats: bool = False,
            workspace: torch.Tensor | None = None, kv_splits: int = 0):
    """Fine attention over the first valid_block_num[b, h, c] ids of each
    kv_block_idx row (B, NH, Nq, max_kv); valid_block_num (B, NH, Nq) or None
    for all. Returns out, or (out, lse, max_prob) with the per-row statistics
    (B, NH, Nq*64) float32 when stats is true. kv_splits: key-range splits
    (0 = chosen from the sizes, 1 = none, 2..16 = that many)."""
    for t, n in ((q_t, "q_t"), (k_t, "k_t"), (v_t, "v_t")):
        _bf16(t, n)
    _i32(kv_block_idx, "kv_block_idx")
    _i32(vbs, "vbs")
    B, Sq, NH, D = q_t.shape
    Skv = k_t.shape[1]
    if v_t.shape != k_t.shape or k_t.shape[0] != B or k_t.shape[2:] != q_t.shape[2:]:
        raise ValueError("k_t and v_t must be (B, Nkv*64, NH, D) matching q_t")
    if Sq % CUBE or Skv % CUBE:
        raise ValueError("sequence lengths must be multiples of 64")
    Nq, Nkv = Sq // CUBE, Skv // CUBE
    if kv_block_idx.dim() != 4 or tuple(kv_block_idx.shape[:3]) != (B, NH, Nq):
        raise ValueError(f"kv_block_idx must be (B, NH, Nq, max_kv) = ({B}, {NH}, {Nq}, m)")
    if valid_block_num is not None:
        _i32(valid_block_num, "valid_block_num")
        if tuple(valid_block_num.shape) != (B, NH, Nq):
            raise ValueError(f"valid_block_num must be (B, NH, Nq) = ({B}, {NH}, {Nq})")
    if vbs.numel() != Nkv:
        raise ValueError(f"vbs must hold Nkv = {Nkv} entries")
    max_kv = kv_block_idx.shape[3]
    out = torch.empty_like(q_t)
    lse = mp = None
    if stats:
        lse = torch.empty((B, NH, Sq), dtype=torch.float32, device=q_t.device)
        mp = torch.empty((B, NH, Sq), dtype=torch.float32, device=q_t.device)
    scale = 0.0 if sm_scale is None else float(sm_scale)
    if workspace is None:
        workspace = torch.empty(fwd_workspace_bytes(B, Nq, Nkv, NH, D, max_kv, kv_splits),
                                dtype=torch.uint8, device=q_t.device)
    ptr = lambda t: None if t is None else t.data_ptr()
    _lib.check(_lib.load().vsa_fwd_lut_ex(q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(),
                                          kv_block_idx.data_ptr(), ptr(valid_block_num),
                                          vbs.data_ptr(), out.data_ptr(), ptr(lse), ptr(mp), B,
                                          Nq, Nkv, NH, D, max_kv, scale, int(kv_splits),
                                          workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(),
                                          _stream()),
               "vsa_fwd_lut_ex")
    return (out, lse, mp) if stats else out


def coarse_workspace_bytes(B: int, NH: int, Nc: int, D: int) -> int:
    return int(_lib.load().vsa_coarse_workspace_bytes(B, NH, Nc, D))


def coarse(q_t: torch.Tensor, k_t: torch.Tensor, v_t: torch.Tensor, vbs: torch.Tensor,
           topk: int | None = None, sm_scale: float | None = None,
           workspace: torch.Tensor | None = None):
    """Coarse stage over mean-pooled cubes: o_coarse float32 (B, NH, Nc, D),
    and with ``topk`` also the selector's ids (B, NH, Nc, topk) from the same
    scores, returned as (o_coarse, topk_idx)."""
    for t, n in ((q_t, "q_t"), (k_t, "k_t"), (v_t, "v_t")):
        _bf16(t, n)
    _i32(vbs, "vbs")
    B, S, NH, D = q_t.shape
    Nc = S // CUBE
    if k_t.shape != q_t.shape or v_t.shape != q_t.shape or S % CUBE:
        raise ValueError("q_t, k_t and v_t must all be (B, Nc*64, NH, D)")
    _numel(vbs, Nc, "vbs")
    if workspace is None:
        workspace = torch.empty(coarse_workspace_bytes(B, NH, Nc, D), dtype=torch.uint8,
                                device=q_t.device)
    oc = torch.empty((B, NH, Nc, D), dtype=torch.float32, device=q_t.device)
    idx = None
    if topk is not None:
        idx = torch.empty((B, NH, Nc, topk), dtype=torch.int32, device=q_t.device)
    scale = 0.0 if sm_scale is None else float(sm_scale)
    _lib.check(_lib.load().vsa_coarse(q_t.data_ptr(), k_t.data_ptr(), v_t.data_ptr(),
                                      vbs.data_ptr(), B, Nc, NH, D, 0 if topk is None else topk,
                                      _ptr(idx), scale, oc.data_ptr(), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), _stream()),
               "vsa_coarse")
    return oc if topk is None else (oc, idx)


def gate_combine(o_fine: torch.Tensor, o_coarse: torch.Tensor, gate_coarse: torch.Tensor,
                 gate_fine: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """out = gate_coarse * o_coarse[cube of the row] + gate_fine * o_fine, bf16
    (B, Nc*64, NH, D); ``out`` may be ``o_fine`` itself."""
    for t, n in ((o_fine, "o_fine"), (gate_coarse, "gate_coarse"), (gate_fine, "gate_fine")):
        _bf16(t, n)
    B, S, NH, D = o_fine.shape
    Nc = S // CUBE
    if S % CUBE or gate_coarse.shape != o_fine.shape or gate_fine.shape != o_fine.shape:
        raise ValueError("o_fine and both gates must be (B, Nc*64, NH, D)")
    if (o_coarse.dtype != torch.float32 or not o_coarse.is_cuda or not o_coarse.is_contiguous()
            or tuple(o_coarse.shape) != (B, NH, Nc, D)):
        raise ValueError(f"o_coarse must be a contiguous float32 CUDA tensor ({B}, {NH}, {Nc}, {D})")
    if out is None:
        out = torch.empty_like(o_fine)
    _bf16(out, "out")
    if out.shape != o_fine.shape:
        raise ValueError("out must match o_fine")
    _lib.check(_lib.load().vsa_gate_combine(o_fine.data_ptr(), o_coarse.data_ptr(),
                                            gate_coarse.data_ptr(), gate_fine.data_ptr(),
                                            out.data_ptr(), B, Nc, NH, D, _stream()),
               "vsa_gate_combine")
    return out


def mask_to_lut(block_mask: torch.Tensor, max_kv: int | None = None,
                count_truncated: bool = False):
    """Block mask (B, NH, Nq, Nkv) bool/uint8 -> (kv_block_idx int32 (B, NH, Nq,
    max_kv), valid_block_num int32 (B, NH, Nq)), ids ascending; with
    ``count_truncated`` also the number of rows with more than max_kv set cells.
    Entries past a row's count are left as allocated (zero here)."""
    if block_mask.dtype == torch.bool:
        block_mask = block_mask.view(torch.uint8)
    if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda or not block_mask.is_contiguous()
            or block_mask.dim() != 4):
        raise ValueError("block_mask must be a contiguous 4-d bool/uint8 CUDA tensor")
    B, NH, Nq, Nkv = block_mask.shape
    max_kv = Nkv if max_kv is None else int(max_kv)
    idx = torch.zeros((B, NH, Nq, max_kv), dtype=torch.int32, device=block_mask.device)
    cnt = torch.empty((B, NH, Nq), dtype=torch.int32, device=block_mask.device)
    trunc = torch.zeros(1, dtype=torch.int32, device=block_mask.device) if count_truncated else None
    _lib.check(_lib.load().vsa_mask_to_lut(block_mask.data_ptr(), B, NH, Nq, Nkv, max_kv,
                                           idx.data_ptr(), cnt.data_ptr(), _ptr(trunc), _stream()),
               "vsa_mask_to_lut")
    return (idx, cnt, int(trunc.item())) if count_truncated else (idx, cnt)


def validate_topk(topk_idx: torch.Tensor, Nkv: int) -> int:
    """Number of out-of-range or repeated ids in topk_idx (B, NH, Nq, topk)."""
    _i32(topk_idx, "topk_idx")
    B, NH, Nq, topk = topk_idx.shape
    bad = torch.zeros(1, dtype=torch.int32, device=topk_idx.device)
    _lib.check(_lib.load().vsa_validate_topk(topk_idx.data_ptr(), B, NH, Nq, Nkv, topk,
                                             bad.data_ptr(), _stream()), "vsa_validate_topk")
    return int(bad.item())


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
