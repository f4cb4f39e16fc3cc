"""GPU parity of vsa_fwd_lut: the fine stage over the first valid_block_num
ids of each index row (VSA blog, "Block-Sparse Encoding" and "Sparse
Traversal"), with the per-row log-sum-exp and max_prob = 1 / l (Wan INT8 blog,
"Dynamic Sparsity Budgeting via Softmax Normalizer Registers").

Tolerances of the statistics, per row, from the kernel's arithmetic:
* l is the fp32 sum of the fp16-rounded weights: relative error <= 2^-11
  (+ fp32 summation), so |d ln l| <= 2^-11 + n 2^-24;
* each score is an fp32 MFMA dot product of bf16 inputs: |d s| <= gamma_D
  sum_d |q_d k_d| (Higham), scaled by sm_scale, which moves lse and the
  exponent of max_prob by at most twice that over the row's keys;
* the final fp32 expression adds a few ulps of |lse|.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import assert_fine_ok, from_gpu_bf16, gamma, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _case(B, Nq, Nkv, NH, D, max_kv, seed, vbs=None, scale_qk=1.0):
    rng = np.random.default_rng(seed)
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D) * scale_qk)
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D) * scale_qk)
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    if vbs is None:
        vbs = rng.integers(0, 65, size=Nkv).astype(np.int32)
    idx = np.stack([np.stack([np.stack([rng.permutation(Nkv)[:max_kv] for _ in range(Nq)])
                              for _ in range(NH)]) for _ in range(B)]).astype(np.int32)
    valid = rng.integers(0, max_kv + 1, size=(B, NH, Nq)).astype(np.int32)
    valid.flat[0] = 0
    valid.flat[-1] = max_kv
    return q, k, v, np.asarray(vbs, np.int32), idx, valid


def _stat_tolerances(q64, k64, idx, valid, vbs, scale):
    """Per-row bounds (B, NH, S) on |d lse| and on |d max_prob| / max_prob."""
    B, S, NH, D = q64.shape
    tol_lse = np.zeros((B, NH, S))
    for b in range(B):
        for h in range(NH):
            for c in range(S // 64):
                ids = idx[b, h, c, :valid[b, h, c]]
                rows = np.concatenate([64 * j + np.arange(vbs[j]) for j in ids]) if ids.size else []
                if len(rows) == 0:
                    continue
                a = np.abs(q64[b, 64 * c:64 * (c + 1), h]) @ np.abs(k64[b, rows, h]).T
                tol_lse[b, h, 64 * c:64 * (c + 1)] = (2.0 ** -11 + len(rows) * 2.0 ** -24
                                                       + 2 * gamma(D) * scale * a.max(axis=1))
    return tol_lse


def _check(q, k, v, vbs, idx, valid, label, sm_scale=None, kv_splits=0):
    B, S, NH, D = q.shape
    print(f"[{label}] B={B} Nq={S // 64} Nkv={vbs.size} NH={NH} D={D} max_kv={idx.shape[-1]} "
          f"splits={vsa.fwd_splits(vbs.size, D, idx.shape[-1], kv_splits)}", flush=True)
    out_t, lse_t, mp_t = vsa.fwd_lut(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v),
                                     torch.from_numpy(idx).cuda(), torch.from_numpy(valid).cuda(),
                                     torch.from_numpy(vbs).cuda(), sm_scale=sm_scale, stats=True,
                                     kv_splits=kv_splits)
    out = from_gpu_bf16(out_t)
    lse, mp = lse_t.cpu().numpy().astype(np.float64), mp_t.cpu().numpy().astype(np.float64)
    q64, k64, v64 = (oracle.decode_bf16(a) for a in (q, k, v))
    ref, ref_lse, ref_mp = oracle.fwd_lut(q64, k64, v64, idx, valid, vbs, sm_scale=sm_scale)
    assert_fine_ok({h: out[:, :, h] for h in range(NH)}, {h: ref[:, :, h] for h in range(NH)},
                   label)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), "rows without keys differ"
    assert np.all(mp[empty] == 0.0)
    scale = 1 / math.sqrt(D) if sm_scale is None else sm_scale
    tol = _stat_tolerances(q64, k64, idx, valid, vbs, scale)
    tol_abs = tol + 8 * 2.0 ** -24 * np.abs(np.where(empty, 0, ref_lse))
    # rows without keys hold -inf on both sides (checked above): mask before subtracting
    d_lse = np.abs(np.where(empty, 0.0, lse) - np.where(empty, 0.0, ref_lse))
    d_mp = np.abs(np.where(empty, 0, mp / np.where(empty, 1, ref_mp) - 1))
    print(f"[{label}] max |d lse| {d_lse.max():.2e} (worst / bound {np.max(d_lse / np.maximum(tol_abs, 1e-30)):.3f});"
          f" max rel d max_prob {d_mp.max():.2e}", flush=True)
    assert np.all(np.isfinite(lse[~empty])) and np.all(np.isfinite(mp))
    assert np.all(d_lse <= tol_abs)
    assert np.all(d_mp <= 2 * tol + 8 * 2.0 ** -24)
    return out, lse, mp


@pytest.mark.parametrize("D", [64, 128])
def test_lut_counts_and_stats_ragged(D):
    vbs = np.array([0, 1, 3, 17, 31, 32, 33, 63, 64, 64, 5, 48], np.int32)
    q, k, v, vbs, idx, valid = _case(2, 12, 12, 3, D, 6, seed=31 + D, vbs=vbs)
    _check(q, k, v, vbs, idx, valid, f"lut ragged D={D}")


def test_lut_huge_logits_stats():
    q, k, v, vbs, idx, valid = _case(1, 8, 8, 2, 128, 4, seed=9, scale_qk=12.0)
    _, lse, _ = _check(q, k, v, vbs, idx, valid, "lut huge logits")
    assert np.nanmax(np.abs(lse[np.isfinite(lse)])) > 100


def test_lut_null_counts_equal_fwd_bitwise():
    q, k, v, vbs, idx, _ = _case(1, 10, 10, 2, 128, 5, seed=12)
    args = [to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(idx).cuda()]
    vb = torch.from_numpy(vbs).cuda()
    a = vsa.fwd_lut(*args, None, vb)
    b = vsa.fwd(*args, vb)
    full = torch.full(idx.shape[:3], idx.shape[3], dtype=torch.int32, device="cuda")
    c = vsa.fwd_lut(*args, full, vb)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c.view(torch.int16), b.view(torch.int16))


def test_lut_small_workload_sampled_units():
    """The small workload (12 heads, 624 cubes) with the selector's top-187
    rows cut to a random count per row; 3 seeded query cubes per head."""
    c = synth.small()
    dev = torch.device("cuda:0")
    qt, vbs_t = vsa.tile(to_gpu_bf16(c.q), c.T, c.H, c.W)
    kt, _ = vsa.tile(to_gpu_bf16(c.k), c.T, c.H, c.W)
    vt, _ = vsa.tile(to_gpu_bf16(c.v), c.T, c.H, c.W)
    idx_t = vsa.select(qt, kt, vbs_t, c.topk)
    B, S, NH, D = qt.shape
    Nq = S // 64
    rng = np.random.default_rng(3)
    valid = rng.integers(1, c.topk + 1, size=(B, NH, Nq)).astype(np.int32)
    out_t, lse_t, mp_t = vsa.fwd_lut(qt, kt, vt, idx_t, torch.from_numpy(valid).to(dev), vbs_t,
                                     stats=True)
    torch.cuda.synchronize()
    q64 = oracle.decode_bf16(from_gpu_bf16(qt))
    k64 = oracle.decode_bf16(from_gpu_bf16(kt))
    v64 = oracle.decode_bf16(from_gpu_bf16(vt))
    idx, vbs = idx_t.cpu().numpy(), vbs_t.cpu().numpy()
    out = oracle.decode_bf16(from_gpu_bf16(out_t))
    lse, mp = lse_t.cpu().numpy(), mp_t.cpu().numpy()
    worst_lse = worst_mp = 0.0
    for h in range(NH):
        for qc in rng.choice(Nq, size=3, replace=False):
            n = int(valid[0, h, qc])
            o, e, x = oracle.fwd_unit_stats(q64, k64, v64, idx[0, h, qc, :n], vbs, 0, h, qc)
            rows = slice(64 * qc, 64 * (qc + 1))
            ref = oracle.round_to_bf16(o)
            d = np.abs(out[0, rows, h] - ref)
            assert d.max() <= 3e-2 and d.mean() <= 2e-4, (h, qc, d.max(), d.mean())
            worst_lse = max(worst_lse, float(np.abs(lse[0, h, rows] - e).max()))
            worst_mp = max(worst_mp, float(np.abs(mp[0, h, rows] / x - 1).max()))
    print(f"[lut small] max |d lse| {worst_lse:.2e}; max rel d max_prob {worst_mp:.2e}", flush=True)
    assert worst_lse <= 2e-3 and worst_mp <= 2e-3
