"""The path under HIP graph capture. No entry point allocates, sets memory or
synchronises, so a whole step (tile x 3 -> select -> fwd -> untile) can be
captured into one graph and replayed. Each replay, with eager work on the
same stream between replays (a fill of the outputs and unrelated torch
kernels), must reproduce the eager step's bits exactly; so must a captured
fine stage in key-range splits (fwd_lut_ex, with the merge pass) and the
allocation-free selector."""
import numpy as np
import pytest
import torch

import synth
import video_dit_block_amd as vsa
from gpu_util import to_gpu_bf16

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_whole_step_graph_replays_match_eager():
    c = synth.small()
    T, H, W, NH, D, B, topk = c.T, c.H, c.W, c.NH, c.D, c.B, c.topk
    q, k, v = to_gpu_bf16(c.q), to_gpu_bf16(c.k), to_gpu_bf16(c.v)
    Nc = vsa.num_cubes(T, H, W)
    qt, kt, vt = (torch.empty((B, Nc * 64, NH, D), dtype=torch.bfloat16, device="cuda")
                  for _ in range(3))
    vbs = torch.empty(Nc, dtype=torch.int32, device="cuda")
    ws = torch.empty(vsa.select_workspace_bytes(B, NH, Nc, D), dtype=torch.uint8, device="cuda")
    wsf = torch.empty(vsa.fwd_workspace_bytes(B, Nc, Nc, NH, D, topk), dtype=torch.uint8,
                      device="cuda")
    idx = torch.empty((B, NH, Nc, topk), dtype=torch.int32, device="cuda")
    idx_na = torch.empty_like(idx)
    out_t = torch.empty_like(qt)
    out = torch.empty_like(q)

    def step():
        vsa.tile(q, T, H, W, out=qt, vbs=vbs)
        vsa.tile(k, T, H, W, out=kt, vbs=vbs)
        vsa.tile(v, T, H, W, out=vt, vbs=vbs)
        vsa.select(qt, kt, vbs, topk, workspace=ws, out=idx)
        vsa.select_noalloc(qt, kt, vbs, topk, out=idx_na)
        vsa.fwd(qt, kt, vt, idx, vbs, out=out_t, workspace=wsf)
        vsa.untile(out_t, T, H, W, out=out)

    step()  # eager, which also sets up the allocation-free selector's scratch
    torch.cuda.synchronize()
    ref = {n: _bits(t).clone() for n, t in (("qt", qt), ("idx", idx), ("idx_na", idx_na),
                                            ("out_t", out_t), ("out", out))}
    assert torch.equal(ref["idx"], ref["idx_na"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on a side stream, as torch asks before a capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    noise = torch.randn(1 << 20, device="cuda")
    for replay in range(4):
        for t in (qt, out_t, out):
            t.zero_()
        idx.fill_(-1)
        idx_na.fill_(-1)
        noise = torch.tanh(noise) * 1.5 + 0.1  # unrelated eager kernels between replays
        g.replay()
        torch.cuda.synchronize()
        print(f"[graph] replay {replay}", flush=True)
        for n, t in (("qt", qt), ("idx", idx), ("idx_na", idx_na), ("out_t", out_t),
                     ("out", out)):
            assert torch.equal(_bits(t), ref[n]), (replay, n)


def test_split_fine_stage_graph_replays_match_eager():
    """vsa_fwd_lut in 3 key-range splits (the fine kernel, then the merge),
    with per-row counts and the row statistics, captured and replayed."""
    rng = np.random.default_rng(90)
    B, Nq, Nkv, NH, D, max_kv = 2, 20, 20, 3, 128, 7
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = to_gpu_bf16(synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D)))
    k = to_gpu_bf16(synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D)))
    v = to_gpu_bf16(synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D)))
    vbs = torch.from_numpy(rng.integers(0, 65, size=Nkv).astype(np.int32)).cuda()
    idx = torch.from_numpy(np.stack([np.stack([np.stack([rng.permutation(Nkv)[:max_kv]
                                                         for _ in range(Nq)])
                                               for _ in range(NH)]) for _ in range(B)])
                           .astype(np.int32)).cuda()
    cnt = torch.from_numpy(rng.integers(0, max_kv + 1, size=(B, NH, Nq)).astype(np.int32)).cuda()
    ws = torch.empty(vsa.fwd_workspace_bytes(B, Nq, Nkv, NH, D, max_kv, 3), dtype=torch.uint8,
                     device="cuda")
    run = lambda: vsa.fwd_lut(q, k, v, idx, cnt, vbs, stats=True, workspace=ws, kv_splits=3)
    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    for replay in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, ref):
            assert torch.equal(_bits(a), _bits(b)), replay
