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


def test_cdf_lut_and_mask_bench_config(run):
    """The lookup-table legs as bench.py runs them on this workload: the
    0.9-mass selector capped at Nc/2 on every row (counts checked against the
    fp64 scores), vsa_fwd_lut with its row statistics on the oracle's own
    table (every head x 8 query cubes plus 64 of the outlier head), and the
    oracle's top-78 as a block mask through vsa_mask_to_lut (bit-equal LUT,
    and vsa_fwd_lut bit-equal to vsa_fwd)."""
    import math

    from gpu_util import stat_tolerance_rows
    from test_gpu_7_cdf import _check_counts, _score_err

    idx_o, S, Qc, Kc, Qa, Ka = run.oracle_select()
    D, NH, Nc = run.case.D, run.case.NH, run.Nc
    scale, max_k, tau = 1 / math.sqrt(D), Nc // 2, 0.9
    gidx, gcnt = run.vsa.select_cdf(run.qt, run.kt, run.vbs, max_k, tau)
    gidx, gcnt = gidx.cpu().numpy(), gcnt.cpu().numpy()
    ora_idx, ora_cnt = oracle.cdf_counts(S, max_k, tau, scale)
    ok, n_diff, _ = topk_check(gidx, ora_idx, S, Qc, Kc, Qa, Ka, 64)
    bad = _check_counts(gidx, gcnt, S, _score_err(Qc, Kc, Qa, Ka, 64), tau, scale, max_k)
    print(f"[wan cdf] mean count {gcnt.mean():.1f} (oracle {ora_cnt.mean():.1f}), equal counts "
          f"{int((gcnt == ora_cnt).sum())}/{gcnt.size}, invalid {bad}, id positions differing "
          f"{n_diff}", flush=True)
    assert ok and bad == 0

    out, lse, mp = run.vsa.fwd_lut(run.qt, run.kt, run.vt, torch.from_numpy(ora_idx).cuda(),
                                   torch.from_numpy(ora_cnt).cuda(), run.vbs, stats=True)
    assert bool(torch.isfinite(out.float()).all())
    bits, lse, mp = from_gpu_bf16(out), lse.cpu().numpy(), mp.cpu().numpy()
    h_star = run.case.outlier_head
    rng = np.random.default_rng(505)
    units = [(0, h, int(c)) for h in range(NH) for c in rng.choice(Nc, size=8, replace=False)]
    units += [(0, h_star, int(c)) for c in rng.choice(Nc, size=64, replace=False)]
    dev, ref = {}, {}
    worst = 0.0
    for b, h, c in units:
        q, k, v = run.head64("q", h), run.head64("k", h), run.head64("v", h)
        ids = ora_idx[b, h, c, :ora_cnt[b, h, c]]
        o, e, x = oracle.fwd_unit_stats(q, k, v, ids, run.vbs_o, b, 0, c)
        dev.setdefault(h, []).append(bits[b, 64 * c:64 * (c + 1), h])
        ref.setdefault(h, []).append(o)
        tol = stat_tolerance_rows(q[b, 64 * c:64 * (c + 1), 0], k[b, :, 0], ids, run.vbs_o, scale)
        rows = slice(64 * c, 64 * (c + 1))
        d_lse = np.abs(lse[b, h, rows] - e)
        d_mp = np.abs(mp[b, h, rows] / x - 1)
        assert np.all(d_lse <= tol + 8 * 2.0 ** -24 * np.abs(e)), (h, c)
        assert np.all(d_mp <= 2 * tol + 8 * 2.0 ** -24), (h, c)
        worst = max(worst, float(np.max(d_lse / (tol + 8 * 2.0 ** -24 * np.abs(e)))))
    print(f"[wan lut] lse worst |d| / bound {worst:.3g}", flush=True)
    assert_fine_ok({h: np.stack(v) for h, v in dev.items()}, {h: np.stack(v) for h, v in ref.items()},
                   "wan fwd_lut (oracle table)")

    idx_t = torch.from_numpy(idx_o).cuda()
    M = torch.zeros((1, NH, Nc, Nc), dtype=torch.uint8, device="cuda")
    M.scatter_(3, idx_t.long(), 1)
    lut, cnt = run.vsa.mask_to_lut(M, run.case.topk)
    torch.cuda.synchronize()
    assert bool((cnt == run.case.topk).all())
    assert np.array_equal(lut.cpu().numpy(), np.sort(idx_o, axis=-1))
    a = run.vsa.fwd_lut(run.qt, run.kt, run.vt, lut, cnt, run.vbs)
    b2 = run.vsa.fwd(run.qt, run.kt, run.vt, idx_t, run.vbs)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b2.view(torch.int16))
