"""GPU parity of vsa_coarse (the coarse stage's own output, and the top-k ids
from the same scores) and vsa_gate_combine (VSA blog, "Two-Stage
Architecture": the final output mixes the coarse and fine outputs through
gates). Tolerances are derived from the kernels' fp32 arithmetic in
gpu_util.coarse_tolerance and gpu_util.combine_check."""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import (ConfigRun, assert_fine_ok, check_coarse, combine_check, from_gpu_bf16,
                      to_gpu_bf16)

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _random_case(B, Nc, NH, D, vbs, seed, scale_qk=1.0):
    rng = np.random.default_rng(seed)
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nc * 64, NH, D) * scale_qk)
    k = synth.bf16_bits_from_f32(f32(B, Nc * 64, NH, D) * scale_qk)
    v = synth.bf16_bits_from_f32(f32(B, Nc * 64, NH, D))
    return q, k, v, np.asarray(vbs, np.int32)


def _heads(arrays):
    dec = {n: oracle.decode_bf16(a) for n, a in arrays.items()}
    return lambda name, h: dec[name][:, :, h:h + 1, :]


@pytest.mark.parametrize("D", [64, 128])
def test_coarse_ragged_with_empty_cubes(D):
    vbs = [0, 1, 3, 17, 31, 64, 0, 63, 64, 64, 5, 48, 2]
    q, k, v, vbs = _random_case(2, len(vbs), 3, D, vbs, seed=40 + D)
    print(f"[coarse ragged D={D}] B=2 Nc={vbs.size} NH=3", flush=True)
    oc = vsa.coarse(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(vbs).cuda())
    check_coarse(oc.cpu().numpy(), _heads({"q": q, "k": k, "v": v}), vbs, 3, None,
                 f"coarse ragged D={D}")
    oc2 = vsa.coarse(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(vbs).cuda(),
                     sm_scale=0.05)
    check_coarse(oc2.cpu().numpy(), _heads({"q": q, "k": k, "v": v}), vbs, 3, 0.05,
                 f"coarse ragged D={D} scale 0.05")


def test_coarse_large_logits_and_no_real_key():
    vbs = [64, 64, 12, 0, 40, 7]
    q, k, v, vbs = _random_case(1, len(vbs), 2, 128, vbs, seed=8, scale_qk=30.0)
    oc = vsa.coarse(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(vbs).cuda())
    check_coarse(oc.cpu().numpy(), _heads({"q": q, "k": k, "v": v}), vbs, 2, None,
                 "coarse large logits")
    empty = np.zeros(4, np.int32)
    q, k, v, _ = _random_case(1, 4, 2, 64, empty, seed=9)
    oc = vsa.coarse(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(empty).cuda())
    torch.cuda.synchronize()
    assert torch.equal(oc, torch.zeros_like(oc))


@pytest.fixture(scope="module")
def small():
    return ConfigRun(synth.small())


def test_coarse_small_every_row_and_topk_equals_select(small):
    """The small workload (12 heads, 624 cubes, D 128): every o_coarse element;
    the ids written from the same scores are those of vsa_select, bit for bit."""
    oc, idx = vsa.coarse(small.qt, small.kt, small.vt, small.vbs, topk=small.case.topk)
    ref_idx = vsa.select(small.qt, small.kt, small.vbs, small.case.topk)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref_idx)
    check_coarse(oc.cpu().numpy(), small.head64, small.vbs_o, small.case.NH, None, "coarse small")


def test_gate_combine_and_in_place(small):
    rng = np.random.default_rng(21)
    shape = tuple(small.qt.shape)
    of = synth.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    gc = synth.bf16_bits_from_f32(rng.uniform(-1, 1, size=shape).astype(np.float32))
    gf = synth.bf16_bits_from_f32(rng.uniform(-1, 1, size=shape).astype(np.float32))
    gc.reshape(-1)[:4096] = 0                     # gates that switch a branch off
    gf.reshape(-1)[4096:8192] = 0
    oc = vsa.coarse(small.qt, small.kt, small.vt, small.vbs)
    of_t, gc_t, gf_t = to_gpu_bf16(of), to_gpu_bf16(gc), to_gpu_bf16(gf)
    out = vsa.gate_combine(of_t, oc, gc_t, gf_t)
    combine_check(from_gpu_bf16(out), of, oc.cpu().numpy(), gc, gf, "combine small")
    vsa.gate_combine(of_t, oc, gc_t, gf_t, out=of_t)   # in place over o_fine
    torch.cuda.synchronize()
    assert torch.equal(of_t.view(torch.int16), out.view(torch.int16))


def test_two_stage_pipeline_tiny():
    """tile -> coarse (+ top-k) -> fine -> gated combine -> untile on the tiny
    workload, against the oracle's chain on every row. The fine output crosses
    the boundary as bf16, so the oracle's chain rounds it to bf16 (nearest
    even) before the combine; the result is held to the fine stage's
    acceptance rules."""
    run = ConfigRun(synth.tiny())
    c = run.case
    T, H, W = c.T, c.H, c.W
    rng = np.random.default_rng(4)
    oc, idx = vsa.coarse(run.qt, run.kt, run.vt, run.vbs, topk=c.topk)
    of = vsa.fwd(run.qt, run.kt, run.vt, idx, run.vbs)
    shape = tuple(run.qt.shape)
    gc = synth.bf16_bits_from_f32(rng.uniform(0, 1, size=shape).astype(np.float32))
    gf = synth.bf16_bits_from_f32(rng.uniform(0, 1, size=shape).astype(np.float32))
    out = vsa.untile(vsa.gate_combine(of, oc, to_gpu_bf16(gc), to_gpu_bf16(gf)), T, H, W)
    got = from_gpu_bf16(out)

    idx_o = run.oracle_select()[0]
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_o)
    qo, ko, vo = (oracle.decode_bf16(run.tiled_oracle(n)) for n in ("q", "k", "v"))
    vbs = run.vbs_o
    fine = oracle.round_to_bf16(oracle.fwd(qo, ko, vo, idx_o, vbs))
    ref_t = oracle.gated_combine(fine, oracle.coarse_output(qo, ko, vo, vbs),
                                 oracle.decode_bf16(gc), oracle.decode_bf16(gf))
    ref = oracle.untile(ref_t, T, H, W)
    assert_fine_ok({h: got[:, :, h] for h in range(c.NH)}, {h: ref[:, :, h] for h in range(c.NH)},
                   "two-stage tiny")
