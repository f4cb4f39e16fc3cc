"""Seeded random configurations of the fine stage against the oracle.

Each case draws its own shape (batch, heads, head size 64 or 128, query and
key cube counts), a row length, a vbs per key cube in [0, 64], optional
per-row counts (the lookup-table form), and a key-range split count (chosen
by the library, none, or forced to 2, 3 or 5, even beyond the key cube
count, which leaves empty splits). Every row of every case is compared with
the oracle (Wan card, "Operator contract": softmax over the real tokens of
the selected cubes) under the acceptance rule of the other fine-stage tests.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import assert_fine_ok, from_gpu_bf16, to_gpu_bf16

pytestmark = pytest.mark.gpu

N_CASES = 20


def _draw(seed):
    rng = np.random.default_rng(9000 + seed)
    D = int(rng.choice([64, 128]))
    B = int(rng.integers(1, 3))
    NH = int(rng.integers(1, 4))
    Nkv = int(rng.integers(1, 49))
    Nq = int(rng.integers(1, 25))
    topk = int(rng.integers(1, Nkv + 1))
    vbs = rng.integers(0, 65, size=Nkv).astype(np.int32)
    vbs[rng.random(Nkv) < 0.5] = 64  # about half the cubes full
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    idx = np.stack([np.stack([np.stack([rng.permutation(Nkv)[:topk] for _ in range(Nq)])
                              for _ in range(NH)]) for _ in range(B)]).astype(np.int32)
    valid = (rng.integers(0, topk + 1, size=(B, NH, Nq)).astype(np.int32)
             if rng.random() < 0.5 else None)
    splits = int(rng.choice([0, 1, 2, 3, 5]))
    return dict(D=D, B=B, NH=NH, Nkv=Nkv, Nq=Nq, topk=topk, vbs=vbs, q=q, k=k, v=v, idx=idx,
                valid=valid, splits=splits)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_fuzz_fine_stage_against_oracle(seed):
    c = _draw(seed)
    label = (f"fuzz {seed}: B={c['B']} NH={c['NH']} D={c['D']} Nq={c['Nq']} Nkv={c['Nkv']} "
             f"topk={c['topk']} counts={c['valid'] is not None} splits={c['splits']}")
    print(f"[{label}]", flush=True)
    valid_t = None if c["valid"] is None else torch.from_numpy(c["valid"]).cuda()
    out = from_gpu_bf16(vsa.fwd_lut(to_gpu_bf16(c["q"]), to_gpu_bf16(c["k"]), to_gpu_bf16(c["v"]),
                                    torch.from_numpy(c["idx"]).cuda(), valid_t,
                                    torch.from_numpy(c["vbs"]).cuda(), kv_splits=c["splits"]))
    ref, _, _ = oracle.fwd_lut(oracle.decode_bf16(c["q"]), oracle.decode_bf16(c["k"]),
                               oracle.decode_bf16(c["v"]), c["idx"], c["valid"], c["vbs"])
    NH = c["NH"]
    assert_fine_ok({h: out[:, :, h] for h in range(NH)}, {h: ref[:, :, h] for h in range(NH)},
                   label)
