"""GPU parity of vsa_select_cdf: the cube selector with a cumulative-mass
threshold (Wan INT8 blog, "Decoupling Block Selection from Sparse CUDA
Kernels"), and the lookup table it produces driving vsa_fwd_lut.

The ids are compared like vsa_select's (tie-tolerant, gpu_util.topk_check).
A count is a decision taken in fp32 on the device and in fp64 by the oracle,
so the test accepts the device's count n when, with the oracle's fp64 scores
taken in the device's id order, C(n-1) < tau Z + eps and C(n) >= tau Z - eps
(C(n) the sum of the n leading weights, Z the total), or n = max_k with
C(max_k) < tau Z + eps. eps bounds the fp32 error of the weights and sums:
each score is off by at most e_i (the pooling and dot-product bound that
topk_check uses), so each weight by a factor exp(2 e_max scale) - 1, plus the
fp32 exp and summation roundoff (Nc 2^-23 of Z).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import ConfigRun, gamma, topk_check

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _score_err(Qc, Kc, Qa, Ka, n_pool):
    """Per (b, h, i) the largest fp32 error bound over the row's scores."""
    D = Qc.shape[-1]
    aQ, aK = np.abs(Qc), np.abs(Kc)
    e = gamma(D) * np.einsum("bhid,bhjd->bhij", aQ, aK)
    e += gamma(n_pool + 1) * (np.einsum("bhid,bhjd->bhij", Qa, aK)
                              + np.einsum("bhid,bhjd->bhij", aQ, Ka))
    return e.max(axis=-1)


def _check_counts(gidx, gcnt, S, err, tau, scale, max_k):
    """Validity of every device count against the fp64 scores; returns the
    number of rows whose count differs from the oracle's."""
    B, NH, Nc = gcnt.shape
    bad = 0
    for b in range(B):
        for h in range(NH):
            for i in range(Nc):
                n = int(gcnt[b, h, i])
                assert 1 <= n <= max_k, n
                s = S[b, h, i]
                full = np.argsort(-s, kind="stable")          # fp64 order of all cubes
                head = gidx[b, h, i]
                rest = np.setdiff1d(full, head, assume_unique=True)
                order = np.concatenate([head, rest])
                w = np.exp((s[order] - s.max()) * scale)
                C = np.concatenate([[0.0], np.cumsum(w)])
                Z = C[-1]
                eps = (math.expm1(2 * err[b, h, i] * scale) + Nc * 2.0 ** -23) * Z
                lo_ok = C[n - 1] < tau * Z + eps
                hi_ok = C[n] >= tau * Z - eps or (n == max_k and C[max_k] < tau * Z + eps)
                if not (lo_ok and hi_ok):
                    bad += 1
    return bad


@pytest.fixture(scope="module")
def small():
    return ConfigRun(synth.small())


@pytest.mark.parametrize("tau,max_k", [(0.5, 624), (0.9, 312), (0.99, 187), (0.5, 128), (0.9, 100)])
def test_select_cdf_small_every_row(small, tau, max_k):
    idx_o, S, Qc, Kc, Qa, Ka = small.oracle_select()
    D = Qc.shape[-1]
    scale = 1 / math.sqrt(D)
    gidx_t, gcnt_t = vsa.select_cdf(small.qt, small.kt, small.vbs, max_k, tau)
    gidx, gcnt = gidx_t.cpu().numpy(), gcnt_t.cpu().numpy()
    ora_idx, ora_cnt = oracle.cdf_counts(S, max_k, tau, scale)
    ok, n_diff, worst = topk_check(gidx, ora_idx, S, Qc, Kc, Qa, Ka, 64)
    assert ok, (n_diff, worst)
    err = _score_err(Qc, Kc, Qa, Ka, 64)
    bad = _check_counts(gidx, gcnt, S, err, tau, scale, max_k)
    n_same = int((gcnt == ora_cnt).sum())
    print(f"[cdf tau={tau} max_k={max_k}] mean count {gcnt.mean():.1f} (oracle {ora_cnt.mean():.1f}); "
          f"equal counts {n_same}/{gcnt.size}; invalid {bad}; id positions differing {n_diff}",
          flush=True)
    assert bad == 0


def test_select_cdf_tiny_and_constructed_threshold():
    """Tiny workload at several thresholds, every row against the oracle;
    tau = 1 keeps max_k unless trailing weights underflow."""
    c = synth.tiny()
    run = ConfigRun(c)
    idx_o, S, Qc, Kc, Qa, Ka = run.oracle_select()
    scale = 1 / math.sqrt(c.D)
    err = _score_err(Qc, Kc, Qa, Ka, 64)
    for tau in (0.2, 0.7, 0.95, 1.0):
        for max_k in (3, run.Nc):
            gidx_t, gcnt_t = vsa.select_cdf(run.qt, run.kt, run.vbs, max_k, tau)
            gidx, gcnt = gidx_t.cpu().numpy(), gcnt_t.cpu().numpy()
            ora_idx, ora_cnt = oracle.cdf_counts(S, max_k, tau, scale)
            ok, _, _ = topk_check(gidx, ora_idx, S, Qc, Kc, Qa, Ka, 64)
            assert ok
            assert _check_counts(gidx, gcnt, S, err, tau, scale, max_k) == 0
            print(f"[cdf tiny tau={tau} max_k={max_k}] counts {gcnt.ravel().tolist()} "
                  f"oracle {ora_cnt.ravel().tolist()}", flush=True)


def test_cdf_lut_drives_fwd(small):
    """select_cdf's table fed to vsa_fwd_lut: sampled units against the
    oracle over the same (device-chosen) ids and counts."""
    gidx_t, gcnt_t = vsa.select_cdf(small.qt, small.kt, small.vbs, 312, 0.9)
    out = vsa.fwd_lut(small.qt, small.kt, small.vt, gidx_t, gcnt_t, small.vbs)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out.float()).all())
    gidx, gcnt = gidx_t.cpu().numpy(), gcnt_t.cpu().numpy()
    bits = out.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    got = oracle.decode_bf16(bits)
    rng = np.random.default_rng(17)
    worst_max = worst_mean = 0.0
    for h in range(small.case.NH):
        q, k, v = small.head64("q", h), small.head64("k", h), small.head64("v", h)
        for qc in rng.choice(small.Nc, size=3, replace=False):
            ids = gidx[0, h, qc, :gcnt[0, h, qc]]
            o, _, _ = oracle.fwd_unit_stats(q, k, v, ids, small.vbs_o, 0, 0, qc)
            d = np.abs(got[0, 64 * qc:64 * (qc + 1), h] - oracle.round_to_bf16(o))
            worst_max, worst_mean = max(worst_max, d.max()), max(worst_mean, d.mean())
    print(f"[cdf -> fwd_lut] worst max|d| {worst_max:.3g}, worst unit mean|d| {worst_mean:.3g}",
          flush=True)
    assert worst_max <= 3e-2 and worst_mean <= 2e-4
