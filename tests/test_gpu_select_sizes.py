"""The selector's top-k across row lengths: both device paths (one wave per
row up to 2048 cubes, a workgroup-wide sort beyond), every KPL size class and
its edges, heavy ties, topk from 1 to Nc, and the CDF count on a long row.

Cube-constant inputs with entries in {-1/2, 0, 1/2} make the fp32 pooling
and dot products exact, so the device scores equal the oracle's and its ids
must match the oracle's bit for bit, ties included (VSA blog, "Generating
Sparsity Patterns": top-k along the key axis, largest first; equal scores go
to the lower cube id)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import to_gpu_bf16
from test_gpu_7_cdf import _check_counts, _score_err

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(600)]


def _cube_constant(Nc, NH, D, levels, rng):
    """bf16 bits (1, Nc*64, NH, D) whose 64 rows per cube repeat one vector."""
    vec = rng.integers(-levels, levels + 1, size=(Nc, NH, D)).astype(np.float32) * 0.5
    return synth.bf16_bits_from_f32(np.repeat(vec, 64, axis=0)[None])


@pytest.mark.parametrize("Nc", [1, 8, 64, 65, 128, 129, 256, 640, 1024, 1025, 2048, 2049, 2100,
                                4096, 8192])
def test_topk_exact_scores_every_size(Nc):
    rng = np.random.default_rng(Nc)
    NH, D = 2, 64
    q = _cube_constant(Nc, NH, D, 1, rng)
    k = _cube_constant(Nc, NH, D, 1, rng)
    vbs = rng.integers(0, 65, size=Nc).astype(np.int32)
    q64, k64 = oracle.decode_bf16(q), oracle.decode_bf16(k)
    S = oracle.cube_scores(oracle.mean_pool(q64, vbs), oracle.mean_pool(k64, vbs))
    n_ties = int(sum(len(r) - len(np.unique(r)) for r in S.reshape(-1, Nc)))
    for topk in sorted({1, min(3, Nc), max(1, Nc // 8), max(1, Nc // 2), Nc}):
        print(f"[topk sizes] Nc={Nc} topk={topk} tied scores {n_ties}", flush=True)
        idx = vsa.select(to_gpu_bf16(q), to_gpu_bf16(k), torch.from_numpy(vbs).cuda(), topk)
        np.testing.assert_array_equal(idx.cpu().numpy(), oracle.topk_select(S, topk))


@pytest.mark.parametrize("Nc", [1500, 2100])
def test_cdf_count_long_rows(Nc):
    rng = np.random.default_rng(7 + Nc)
    NH, D = 2, 64
    f32 = lambda: rng.standard_normal((1, Nc * 64, NH, D), dtype=np.float32)
    q, k = synth.bf16_bits_from_f32(f32()), synth.bf16_bits_from_f32(f32())
    vbs = rng.integers(1, 65, size=Nc).astype(np.int32)
    q64, k64 = oracle.decode_bf16(q), oracle.decode_bf16(k)
    Qc, Kc = oracle.mean_pool(q64, vbs), oracle.mean_pool(k64, vbs)
    Qa, Ka = oracle.mean_pool(np.abs(q64), vbs), oracle.mean_pool(np.abs(k64), vbs)
    S = oracle.cube_scores(Qc, Kc)
    scale = 1 / math.sqrt(D)
    err = _score_err(Qc, Kc, Qa, Ka, 64)
    for tau, max_k in ((0.5, Nc), (0.9, Nc // 3)):
        gidx, gcnt = vsa.select_cdf(to_gpu_bf16(q), to_gpu_bf16(k), torch.from_numpy(vbs).cuda(),
                                    max_k, tau)
        gidx, gcnt = gidx.cpu().numpy(), gcnt.cpu().numpy()
        _, ora_cnt = oracle.cdf_counts(S, max_k, tau, scale)
        bad = _check_counts(gidx, gcnt, S, err, tau, scale, max_k)
        print(f"[cdf long rows] Nc={Nc} tau={tau} max_k={max_k}: mean count {gcnt.mean():.1f} "
              f"(oracle {ora_cnt.mean():.1f}), invalid {bad}", flush=True)
        assert bad == 0
