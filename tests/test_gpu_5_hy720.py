"""GPU parity on the 720p HunyuanVideo-like workload: latent grid 30x48x80
(115,200 tokens, FastVideo STA guide, "The 115K Token Sequence Wall"), 24
heads, D = 128, 1,920 cubes (S_padded = 122,880), topk 192 (90% sparse),
heavy-tailed q/k with one high-logit head. The whole path runs on the device:
tiling (bit-exact), the selector (every row), the fine stage on the oracle's
indices (finite everywhere; every head x 16 seeded query cubes plus 64 cubes of
the outlier head against the oracle) and untiling (the exact inverse of the
tiling on every real token); the cumulative-mass selector and the coarse
output on every row."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import ConfigRun, assert_fine_ok, from_gpu_bf16, sample_units, topk_check

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


@pytest.fixture(scope="module")
def run():
    return ConfigRun(synth.hy720())


def test_tile_bit_exact(run):
    for name, t in (("q", run.qt), ("k", run.kt), ("v", run.vt)):
        np.testing.assert_array_equal(from_gpu_bf16(t), run.tiled_oracle(name))


def test_select_every_row(run):
    idx_o, S, Qc, Kc, Qa, Ka = run.oracle_select()
    idx = run.vsa.select(run.qt, run.kt, run.vbs, run.case.topk).cpu().numpy()
    ok, n_diff, worst = topk_check(idx, idx_o, S, Qc, Kc, Qa, Ka, 64)
    print(f"[hy720 select] differing positions {n_diff} of {idx.size}, worst {worst:.3g}",
          flush=True)
    assert ok


def test_fwd_sampled_and_outlier_head(run):
    idx_o = run.oracle_select()[0]
    out = run.vsa.fwd(run.qt, run.kt, run.vt, torch.from_numpy(idx_o).cuda(), run.vbs)
    assert bool(torch.isfinite(out.float()).all()), "non-finite output"
    bits = from_gpu_bf16(out)
    h_star = run.case.outlier_head
    units = sample_units(run.vbs_o, run.case.NH, 16, seed=720)
    units += [u for u in sample_units(run.vbs_o, run.case.NH, 64, seed=721) if u[1] == h_star]
    units = sorted(set(units))
    dev, ref = run.device_rows(bits, units), run.oracle_rows(units, idx_o)
    assert_fine_ok(dev, ref, "hy720 fwd")
    assert_fine_ok({h_star: dev[h_star]}, {h_star: ref[h_star]}, "hy720 outlier head")


def test_untile_inverts_tile(run):
    c = run.case
    back = run.vsa.untile(run.vt, c.T, c.H, c.W)
    np.testing.assert_array_equal(from_gpu_bf16(back), c.v)


def test_cdf_counts_and_coarse_every_row(run):
    """The cumulative-mass selector (tau 0.9, at most half of the cubes) on
    every one of the 46,080 rows against the fp64 scores, and the coarse
    output on every (head, cube)."""
    import math

    import oracle
    from gpu_util import check_coarse
    from test_gpu_7_cdf import _check_counts, _score_err

    idx_o, S, Qc, Kc, Qa, Ka = run.oracle_select()
    D, Nc = run.case.D, run.Nc
    scale, max_k, tau = 1 / math.sqrt(D), Nc // 2, 0.9
    gidx, gcnt = run.vsa.select_cdf(run.qt, run.kt, run.vbs, max_k, tau)
    gidx, gcnt = gidx.cpu().numpy(), gcnt.cpu().numpy()
    _, ora_cnt = oracle.cdf_counts(S, max_k, tau, scale)
    bad = _check_counts(gidx, gcnt, S, _score_err(Qc, Kc, Qa, Ka, 64), tau, scale, max_k)
    print(f"[hy720 cdf] mean count {gcnt.mean():.1f} (oracle {ora_cnt.mean():.1f}), equal "
          f"counts {int((gcnt == ora_cnt).sum())}/{gcnt.size}, invalid {bad}", flush=True)
    assert bad == 0
    oc = run.vsa.coarse(run.qt, run.kt, run.vt, run.vbs)
    check_coarse(oc.cpu().numpy(), run.head64, run.vbs_o, run.case.NH, None, "hy720 coarse")
