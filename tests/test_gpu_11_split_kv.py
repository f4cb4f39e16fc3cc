"""GPU parity of the fine stage's key-range splits (split-KV): every (b, h,
query cube) computed as S items, item s over its selected cubes with
id * S / Nkv == s, and the merge pass combining their partial softmax states
(VSA blog, "Kernel Architecture": the running max and sum of the online
softmax, here carried across items instead of across tiles).

Forced split counts on small ragged inputs, every row against the oracle
under the fine stage's acceptance rule, with the per-row statistics under the
bounds of test_gpu_6_lut: splits that no selected cube falls in, more splits
than key cubes, rows with no keys, per-row counts, B = 2, both D. A split
count of 1 is the unsplit stage bit for bit. The 720p workload takes 2 splits
by itself (test_gpu_5_hy720 runs it)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import assert_fine_ok, from_gpu_bf16, to_gpu_bf16
from test_gpu_6_lut import _case, _check

pytestmark = pytest.mark.gpu

RAGGED_VBS = np.array([0, 1, 3, 17, 31, 32, 33, 63, 64, 64, 5, 48], np.int32)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [2, 3, 7, 16])
def test_forced_splits_counts_and_stats(D, splits):
    q, k, v, vbs, idx, valid = _case(2, 12, 12, 3, D, 6, seed=50 + D + splits, vbs=RAGGED_VBS)
    _check(q, k, v, vbs, idx, valid, f"splits={splits} D={D}", kv_splits=splits)


def test_splits_with_selections_inside_one_range():
    """Half of the rows select only among the first 8 of 64 key cubes, so 7 of
    their 8 splits are empty; the others select across all ranges."""
    rng = np.random.default_rng(61)
    B, Nq, Nkv, NH, D, topk = 1, 16, 64, 2, 128, 5
    q, k, v, vbs, idx, valid = _case(B, Nq, Nkv, NH, D, topk, seed=61)
    for c in range(0, Nq, 2):
        for h in range(NH):
            idx[0, h, c] = rng.permutation(8)[:topk]
    valid[:] = topk
    out8, _, _ = _check(q, k, v, vbs, idx, valid, "one range", kv_splits=8)
    out1, _, _ = _check(q, k, v, vbs, idx, valid, "one range unsplit", kv_splits=1)
    d = np.abs(oracle.decode_bf16(out8) - oracle.decode_bf16(out1))
    print(f"[one range] split vs unsplit: max {d.max():.3g} mean {d.mean():.3g}", flush=True)


def test_splits_huge_logits():
    """Scores of several hundred: the merge weights exp2((m_s - M) c) span the
    whole fp32 range across splits."""
    q, k, v, vbs, idx, valid = _case(1, 8, 8, 2, 128, 4, seed=62, scale_qk=12.0)
    _, lse, _ = _check(q, k, v, vbs, idx, valid, "splits huge logits", kv_splits=4)
    assert np.nanmax(np.abs(lse[np.isfinite(lse)])) > 100


def test_split_count_one_is_the_unsplit_stage():
    q, k, v, vbs, idx, valid = _case(1, 10, 10, 2, 128, 5, seed=63)
    args = [to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(idx).cuda(),
            torch.from_numpy(valid).cuda(), torch.from_numpy(vbs).cuda()]
    assert vsa.fwd_splits(10, 128, 5) == 1
    a = vsa.fwd_lut(*args)
    b = vsa.fwd_lut(*args, kv_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_small_workload_forced_splits_sampled_units():
    """The small workload (12 heads, 624 cubes, top-187 from the oracle's
    selector) in 6 splits: 4 seeded query cubes per head against the oracle."""
    c = synth.small()
    q_t, vbs = oracle.tile(c.q, c.T, c.H, c.W)
    k_t, _ = oracle.tile(c.k, c.T, c.H, c.W)
    v_t, _ = oracle.tile(c.v, c.T, c.H, c.W)
    q64, k64, v64 = (oracle.decode_bf16(a) for a in (q_t, k_t, v_t))
    idx, _ = oracle.select(q64, k64, vbs, c.topk)
    idx = idx.astype(np.int32)
    print(f"[small splits] topk={c.topk} splits={vsa.fwd_splits(vbs.size, c.D, c.topk, 6)}",
          flush=True)
    out = from_gpu_bf16(vsa.fwd_lut(to_gpu_bf16(q_t), to_gpu_bf16(k_t), to_gpu_bf16(v_t),
                                    torch.from_numpy(idx).cuda(), None,
                                    torch.from_numpy(vbs).cuda(), kv_splits=6))
    rng = np.random.default_rng(64)
    gpu, ref = {}, {}
    for h in range(c.NH):
        cubes = rng.choice(vbs.size, size=4, replace=False)
        gpu[h] = np.stack([out[0, u * 64:(u + 1) * 64, h] for u in cubes])
        ref[h] = np.stack([oracle.fwd_unit(q64, k64, v64, idx, vbs, 0, h, u) for u in cubes])
    assert_fine_ok(gpu, ref, "small splits")


@pytest.mark.parametrize("D, Nkv, topk", [(128, 1100, 100), (64, 2100, 40)])
def test_splits_chosen_by_the_library(D, Nkv, topk):
    """Key/value heads just above the 32 MiB the library splits at (1,100
    cubes at D = 128, 2,100 at D = 64: 36 and 34 MB of K plus fp16 V): vsa_fwd
    itself takes 2 splits. Every query cube (Nq = 40, two heads, ragged vbs)
    against the oracle."""
    rng = np.random.default_rng(65 + D)
    B, Nq, NH = 1, 40, 2
    assert vsa.fwd_splits(Nkv, D, topk) == 2
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    vbs = rng.integers(0, 65, size=Nkv).astype(np.int32)
    idx = np.stack([np.stack([rng.choice(Nkv, size=topk, replace=False) for _ in range(Nq)])
                    for _ in range(NH)])[None].astype(np.int32)
    print(f"[auto splits D={D}] Nkv={Nkv} topk={topk} splits={vsa.fwd_splits(Nkv, D, topk)}",
          flush=True)
    out = from_gpu_bf16(vsa.fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v),
                                torch.from_numpy(idx).cuda(), torch.from_numpy(vbs).cuda()))
    q64, k64, v64 = (oracle.decode_bf16(a) for a in (q, k, v))
    gpu = {h: out[0, :, h].reshape(Nq, 64, D) for h in range(NH)}
    ref = {h: np.stack([oracle.fwd_unit(q64, k64, v64, idx, vbs, 0, h, c) for c in range(Nq)])
           for h in range(NH)}
    assert_fine_ok(gpu, ref, f"auto splits D={D}")
