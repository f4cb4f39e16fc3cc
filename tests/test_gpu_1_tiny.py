"""GPU parity on the tiny workload (grid 5x6x7, 2 heads, D = 64, topk 3):
every row of every stage against the oracle, plus the device-side invariants."""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import (assert_fine_ok, from_gpu_bf16, to_gpu_bf16, topk_check)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tiny():
    c = synth.tiny()
    print(f"[tiny] B={c.B} grid={c.T}x{c.H}x{c.W} NH={c.NH} D={c.D} topk={c.topk}", flush=True)
    qt_o, vbs_o = oracle.tile(c.q, c.T, c.H, c.W)
    kt_o, _ = oracle.tile(c.k, c.T, c.H, c.W)
    vt_o, _ = oracle.tile(c.v, c.T, c.H, c.W)
    q64, k64, v64 = (oracle.decode_bf16(a) for a in (qt_o, kt_o, vt_o))
    idx_o, S = oracle.select(q64, k64, vbs_o, c.topk)
    return dict(case=c, qt_o=qt_o, kt_o=kt_o, vt_o=vt_o, vbs_o=vbs_o, q64=q64, k64=k64,
                v64=v64, idx_o=idx_o, S=S)


def test_tile_bit_exact(tiny):
    c = tiny["case"]
    for name in ("q", "k", "v"):
        xt, vbs = vsa.tile(to_gpu_bf16(getattr(c, name)), c.T, c.H, c.W)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(from_gpu_bf16(xt), tiny[name + "t_o"])
        np.testing.assert_array_equal(vbs.cpu().numpy(), tiny["vbs_o"])
        back = vsa.untile(xt, c.T, c.H, c.W)
        np.testing.assert_array_equal(from_gpu_bf16(back), getattr(c, name))


def test_select_matches_oracle(tiny):
    c = tiny["case"]
    qt, vbs = vsa.tile(to_gpu_bf16(c.q), c.T, c.H, c.W)
    kt, _ = vsa.tile(to_gpu_bf16(c.k), c.T, c.H, c.W)
    idx = vsa.select(qt, kt, vbs, c.topk).cpu().numpy()
    Qc = oracle.mean_pool(tiny["q64"], tiny["vbs_o"])
    Kc = oracle.mean_pool(tiny["k64"], tiny["vbs_o"])
    Qa = oracle.mean_pool(np.abs(tiny["q64"]), tiny["vbs_o"])
    Ka = oracle.mean_pool(np.abs(tiny["k64"]), tiny["vbs_o"])
    ok, n_diff, worst = topk_check(idx, tiny["idx_o"], tiny["S"], Qc, Kc, Qa, Ka, 64)
    print(f"[tiny select] differing positions {n_diff}, worst {worst:.3g}", flush=True)
    assert ok
    assert vsa.validate_topk(torch.from_numpy(idx).cuda(), 8) == 0


def test_fwd_every_row(tiny):
    c = tiny["case"]
    qt, kt, vt = (to_gpu_bf16(tiny[n]) for n in ("qt_o", "kt_o", "vt_o"))
    vbs = torch.from_numpy(tiny["vbs_o"]).cuda()
    idx = torch.from_numpy(tiny["idx_o"]).cuda()
    out = from_gpu_bf16(vsa.fwd(qt, kt, vt, idx, vbs))
    ref = oracle.fwd(tiny["q64"], tiny["k64"], tiny["v64"], tiny["idx_o"], tiny["vbs_o"])
    assert_fine_ok({h: out[:, :, h] for h in range(c.NH)},
                   {h: ref[:, :, h] for h in range(c.NH)}, "tiny fwd")


def test_pipeline_end_to_end(tiny):
    """tile -> select -> fwd -> untile on the device vs the oracle pipeline."""
    c = tiny["case"]
    qt, vbs = vsa.tile(to_gpu_bf16(c.q), c.T, c.H, c.W)
    kt, _ = vsa.tile(to_gpu_bf16(c.k), c.T, c.H, c.W)
    vt, _ = vsa.tile(to_gpu_bf16(c.v), c.T, c.H, c.W)
    idx = vsa.select(qt, kt, vbs, c.topk)
    out = from_gpu_bf16(vsa.untile(vsa.fwd(qt, kt, vt, idx, vbs), c.T, c.H, c.W))
    np.testing.assert_array_equal(idx.cpu().numpy(), tiny["idx_o"])
    ref = oracle.untile(oracle.fwd(tiny["q64"], tiny["k64"], tiny["v64"], tiny["idx_o"],
                                   tiny["vbs_o"]), c.T, c.H, c.W)
    assert_fine_ok({h: out[:, :, h] for h in range(c.NH)},
                   {h: ref[:, :, h] for h in range(c.NH)}, "tiny pipeline")


def test_fwd_ignores_nan_padding_and_is_deterministic(tiny):
    qt, kt, vt = (to_gpu_bf16(tiny[n]) for n in ("qt_o", "kt_o", "vt_o"))
    vbs = torch.from_numpy(tiny["vbs_o"]).cuda()
    idx = torch.from_numpy(tiny["idx_o"]).cuda()
    a = from_gpu_bf16(vsa.fwd(qt, kt, vt, idx, vbs))
    b = from_gpu_bf16(vsa.fwd(qt, kt, vt, idx, vbs))
    np.testing.assert_array_equal(a, b)
    kp, vp = kt.clone(), vt.clone()
    for cc, n in enumerate(tiny["vbs_o"]):
        kp[:, 64 * cc + n:64 * (cc + 1)] = float("nan")
        vp[:, 64 * cc + n:64 * (cc + 1)] = float("inf")
    c2 = from_gpu_bf16(vsa.fwd(qt, kp, vp, idx, vbs))
    np.testing.assert_array_equal(c2, a)


def test_fwd_order_invariance(tiny):
    c = tiny["case"]
    qt, kt, vt = (to_gpu_bf16(tiny[n]) for n in ("qt_o", "kt_o", "vt_o"))
    vbs = torch.from_numpy(tiny["vbs_o"]).cuda()
    perm = tiny["idx_o"][..., ::-1].copy()
    out = from_gpu_bf16(vsa.fwd(qt, kt, vt, torch.from_numpy(perm).cuda(), vbs))
    ref = oracle.fwd(tiny["q64"], tiny["k64"], tiny["v64"], tiny["idx_o"], tiny["vbs_o"])
    assert_fine_ok({h: out[:, :, h] for h in range(c.NH)},
                   {h: ref[:, :, h] for h in range(c.NH)}, "tiny reversed topk")


def test_fwd_guard_band_untouched(tiny):
    qt, kt, vt = (to_gpu_bf16(tiny[n]) for n in ("qt_o", "kt_o", "vt_o"))
    vbs = torch.from_numpy(tiny["vbs_o"]).cuda()
    idx = torch.from_numpy(tiny["idx_o"]).cuda()
    full = torch.full((3,) + tuple(qt.shape[1:]), 7.0, dtype=torch.bfloat16, device="cuda")
    vsa.fwd(qt, kt, vt, idx, vbs, out=full[1:2])
    torch.cuda.synchronize()
    assert bool((full[0] == 7.0).all()) and bool((full[2] == 7.0).all())
    np.testing.assert_array_equal(from_gpu_bf16(full[1:2]), from_gpu_bf16(vsa.fwd(qt, kt, vt, idx, vbs)))


def test_validate_topk_counts_bad_ids():
    idx = torch.tensor([[[[0, 1, 2], [3, 3, 1], [7, 8, -1]]]], dtype=torch.int32, device="cuda")
    assert vsa.validate_topk(idx, 8) == 3       # one repeat, two out of range


def test_select_ties_to_lower_id():
    """All cubes identical: every score ties, so the selection is 0..k-1."""
    T, H, W, NH, D = 8, 8, 8, 2, 64
    x = torch.ones(1, T * H * W, NH, D, dtype=torch.bfloat16, device="cuda") * 0.5
    qt, vbs = vsa.tile(x, T, H, W)
    idx = vsa.select(qt, qt, vbs, 5).cpu().numpy()
    np.testing.assert_array_equal(idx, np.broadcast_to(np.arange(5), idx.shape))
