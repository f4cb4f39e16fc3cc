"""GPU parity of the space-filling-curve cube order (vsa_tile_ordered,
vsa_untile_ordered; VSA blog, "Two-Stage Architecture", pre-stage) and of the
block mask -> lookup table compaction (vsa_mask_to_lut; VSA blog, "Sparse
Encoding in CK Tile"). Both are integer / copy work: compared bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import assert_fine_ok, from_gpu_bf16, to_gpu_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


@pytest.mark.parametrize("grid,NH,D", [((5, 6, 7), 2, 64), ((9, 5, 6), 3, 128),
                                       ((17, 3, 90), 1, 64), ((21, 30, 52), 4, 128)])
def test_tile_ordered_bit_exact_and_roundtrip(grid, NH, D):
    T, H, W = grid
    rng = np.random.default_rng(sum(grid))
    x = synth.bf16_bits_from_f32(rng.standard_normal((2, T * H * W, NH, D), dtype=np.float32))
    order = oracle.cube_order(T, H, W)
    assert np.array_equal(vsa.cube_order(T, H, W).numpy(), order)
    order_t = torch.from_numpy(order).cuda()
    print(f"[tile_ordered] grid {grid} NH={NH} D={D} Nc={order.size}", flush=True)
    xt, vbs = vsa.tile(to_gpu_bf16(x), T, H, W, order=order_t)
    ref, vbs_o = oracle.tile(x, T, H, W, order)
    np.testing.assert_array_equal(from_gpu_bf16(xt), ref)
    np.testing.assert_array_equal(vbs.cpu().numpy(), vbs_o)
    back = vsa.untile(xt, T, H, W, order=order_t)
    np.testing.assert_array_equal(from_gpu_bf16(back), x)


def test_pipeline_in_hilbert_order_tiny():
    """tile (Hilbert order) -> select -> fwd -> untile against the oracle's
    chain in the same order, every row."""
    c = synth.tiny()
    T, H, W = c.T, c.H, c.W
    order = oracle.cube_order(T, H, W)
    order_t = torch.from_numpy(order).cuda()
    qt, vbs = vsa.tile(to_gpu_bf16(c.q), T, H, W, order=order_t)
    kt, _ = vsa.tile(to_gpu_bf16(c.k), T, H, W, order=order_t)
    vt, _ = vsa.tile(to_gpu_bf16(c.v), T, H, W, order=order_t)
    idx = vsa.select(qt, kt, vbs, c.topk)
    out = from_gpu_bf16(vsa.untile(vsa.fwd(qt, kt, vt, idx, vbs), T, H, W, order=order_t))
    q64, k64, v64 = (oracle.decode_bf16(oracle.tile(x, T, H, W, order)[0]) for x in (c.q, c.k, c.v))
    vbs_o = oracle.tile(c.q, T, H, W, order)[1]
    idx_o, _ = oracle.select(q64, k64, vbs_o, c.topk)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    ref = oracle.untile(oracle.fwd(q64, k64, v64, idx_o, vbs_o), T, H, W, order)
    assert_fine_ok({h: out[:, :, h] for h in range(c.NH)}, {h: ref[:, :, h] for h in range(c.NH)},
                   "hilbert-order tiny pipeline")


def _check_mask(M, max_kv, label):
    Mt = torch.from_numpy(M).cuda()
    idx, cnt, trunc = vsa.mask_to_lut(Mt, max_kv, count_truncated=True)
    ids_o, cnt_o, trunc_o = oracle.mask_to_lut(M, max_kv)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    np.testing.assert_array_equal(cnt, cnt_o)
    assert trunc == trunc_o
    used = np.arange(max_kv) < cnt[..., None]
    np.testing.assert_array_equal(np.where(used, idx, -1), ids_o)
    print(f"[{label}] shape {M.shape} max_kv {max_kv}: mean count {cnt.mean():.1f}, "
          f"truncated rows {trunc}", flush=True)


@pytest.mark.parametrize("shape,density", [((1, 2, 8, 8), 0.0), ((1, 2, 8, 8), 1.0),
                                           ((2, 3, 37, 77), 0.05), ((2, 3, 37, 77), 0.5),
                                           ((1, 4, 96, 1000), 0.3)])
def test_mask_to_lut_bit_exact(shape, density):
    rng = np.random.default_rng(int(1000 * density) + shape[-1])
    M = (rng.random(shape) < density).astype(np.uint8) * rng.integers(1, 256, size=shape,
                                                                       dtype=np.uint8)
    _check_mask(M, shape[-1], f"mask density {density}")
    _check_mask(M, max(1, shape[-1] // 7), f"mask density {density}, capped")


def test_mask_from_selection_drives_fwd_lut_bitwise_like_fwd():
    """The small workload: the selector's top-187 as a block mask, compacted to
    a LUT (ids ascending, count 187 on every row), gives vsa_fwd_lut an output
    bit-identical to vsa_fwd on the top-k ids (the fine kernel orders every
    row's list by id itself)."""
    c = synth.small()
    T, H, W = c.T, c.H, c.W
    qt, vbs = vsa.tile(to_gpu_bf16(c.q), T, H, W)
    kt, _ = vsa.tile(to_gpu_bf16(c.k), T, H, W)
    vt, _ = vsa.tile(to_gpu_bf16(c.v), T, H, W)
    idx = vsa.select(qt, kt, vbs, c.topk)
    B, NH, Nc, _ = idx.shape
    M = torch.zeros((B, NH, Nc, Nc), dtype=torch.uint8, device="cuda")
    M.scatter_(3, idx.long(), 1)
    lut, cnt = vsa.mask_to_lut(M)
    torch.cuda.synchronize()
    assert bool((cnt == c.topk).all())
    assert torch.equal(lut[..., :c.topk], torch.sort(idx, dim=-1).values)
    a = vsa.fwd_lut(qt, kt, vt, lut, cnt, vbs)
    b = vsa.fwd(qt, kt, vt, idx, vbs)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
