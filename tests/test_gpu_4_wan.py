"""GPU parity on the Wan2.2-A14B shape: q, k, v (1, 39936, 40, 128) bf16, 624
cubes, topk 78 (87.5% sparse), heavy-tailed q/k with one outlier head whose
logits reach about +-2000. Tiling bit-exact; the selector on every row; the
fine stage (oracle indices) finite everywhere and checked on every head x 32
seeded query cubes plus all 624 cubes of the outlier head; the sparsity sweep
topk in {624, 312, 187, 78, 31} on 2 query cubes per head; the coarse-stage
output on every (head, cube) and the gated combine on sampled token rows."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import (ConfigRun, assert_fine_ok, check_coarse, combine_check, from_gpu_bf16,
                      sample_units, topk_check)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(scope="module")
def run():
    return ConfigRun(synth.wan())


def test_tile_bit_exact(run):
    for name, t in (("q", run.qt), ("k", run.kt), ("v", run.vt)):
        np.testing.assert_array_equal(from_gpu_bf16(t), run.tiled_oracle(name))


def test_select_every_row(run):
    idx_o, S, Qc, Kc, Qa, Ka = run.oracle_select()
    idx = run.vsa.select(run.qt, run.kt, run.vbs, run.case.topk).cpu().numpy()
    ok, n_diff, worst = topk_check(idx, idx_o, S, Qc, Kc, Qa, Ka, 64)
    print(f"[wan select] differing positions {n_diff} of {idx.size}, worst {worst:.3g}",
          flush=True)
    assert ok


def test_fwd_sampled_and_outlier_head(run):
    idx_o = run.oracle_select()[0]
    out = run.vsa.fwd(run.qt, run.kt, run.vt, torch.from_numpy(idx_o).cuda(), run.vbs)
    assert bool(torch.isfinite(out.float()).all()), "non-finite output"
    bits = from_gpu_bf16(out)
    h_star = run.case.outlier_head
    units = sample_units(run.vbs_o, run.case.NH, 32, seed=202, extra_heads=(h_star,))
    dev, ref = run.device_rows(bits, units), run.oracle_rows(units, idx_o)
    assert_fine_ok(dev, ref, "wan fwd")
    assert_fine_ok({h_star: dev[h_star]}, {h_star: ref[h_star]}, "wan outlier head")


@pytest.mark.parametrize("k", synth.SWEEP_TOPK)
def test_sweep_sampled(run, k):
    S = run.oracle_select()[1]
    idx_k = oracle.topk_select(S, k)
    out = run.vsa.fwd(run.qt, run.kt, run.vt, torch.from_numpy(idx_k).cuda(), run.vbs)
    assert bool(torch.isfinite(out.float()).all())
    units = sample_units(run.vbs_o, run.case.NH, 2, seed=300 + k)
    units = [u for i, u in enumerate(units) if i % 4 == 0 or k <= 78]
    bits = from_gpu_bf16(out)
    assert_fine_ok(run.device_rows(bits, units), run.oracle_rows(units, idx_k), f"wan k={k}")


def test_coarse_every_row_and_combine_sampled(run):
    oc, idx = run.vsa.coarse(run.qt, run.kt, run.vt, run.vbs, topk=run.case.topk)
    ref_idx = run.vsa.select(run.qt, run.kt, run.vbs, run.case.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    oc_h = oc.cpu().numpy()
    check_coarse(oc_h, run.head64, run.vbs_o, run.case.NH, None, "wan coarse")

    rng = np.random.default_rng(29)
    shape = tuple(run.qt.shape)
    of = run.vsa.fwd(run.qt, run.kt, run.vt, idx, run.vbs)
    gen = torch.Generator(device="cuda").manual_seed(29)
    gc = torch.rand(shape, device="cuda", generator=gen).to(torch.bfloat16)
    gf = torch.rand(shape, device="cuda", generator=gen).to(torch.bfloat16)
    out = run.vsa.gate_combine(of, oc, gc, gf)
    torch.cuda.synchronize()
    cubes = np.sort(rng.choice(run.Nc, size=32, replace=False))   # 2048 token rows
    rows = (64 * cubes[:, None] + np.arange(64)[None, :]).reshape(-1)
    sel = lambda t: from_gpu_bf16(t)[:, rows]
    combine_check(sel(out), sel(of), oc_h[:, :, cubes, :], sel(gc), sel(gf),
                  "wan combine, 32 cubes")
