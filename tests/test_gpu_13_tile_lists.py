"""The fine stage's tile lists, read back from the workspace after a call.

vsa_fwd's list pre-pass turns each (b, h, query cube)'s selected ids into
16-row quarters (a uint32: byte offset from the head's first key row | real
rows) paired into 32-row tiles, per key-range split, each split followed by
zero tiles; include/vsa.h gives the workspace layout. A quarter lost or
repeated would move the output by less than the acceptance rule can see, so
this test checks the lists themselves: for every unit and split, the
quarters are exactly those of its selected cubes in that split (ceil(vbs/16)
per cube, min(16, vbs - 16k) rows each), each once, in an ascending sweep of
the cube ids that wraps around at most once (a rotated sweep), with one zero
quarter at most (completing the last tile) and the zero tiles after it."""
import numpy as np
import pytest
import torch

import synth
import video_dit_block_amd as vsa
from gpu_util import to_gpu_bf16

pytestmark = pytest.mark.gpu

LIST_PAD = 4  # zero tiles after each split's tiles


def _up(n):
    return (n + 255) & ~255


def _check_lists(ws, B, Nq, Nkv, NH, D, row_len, idx, valid, vbs, splits):
    units = B * NH * Nq
    stride = 2 * row_len + LIST_PAD + (splits * (LIST_PAD + 1) if splits > 1 else 0)
    list_off = _up(B * Nkv * 64 * NH * D * 2)
    sbeg_off = list_off + _up(units * stride * 8)
    raw = ws.cpu().numpy()
    lists = raw[list_off:list_off + units * stride * 8].view(np.uint32).reshape(units, stride * 2)
    sbeg = raw[sbeg_off:sbeg_off + units * (splits + 1) * 4].view(np.int32).reshape(units,
                                                                                 splits + 1)
    rs2 = NH * D * 2
    rotated = 0
    for u in range(units):
        b, h, c = u // (NH * Nq), (u // Nq) % NH, u % Nq
        n_ids = row_len if valid is None else int(np.clip(valid[b, h, c], 0, row_len))
        ids = idx[b, h, c, :n_ids]
        for s in range(splits):
            t0, t1 = sbeg[u, s], sbeg[u, s + 1] - LIST_PAD
            assert 0 <= t0 <= t1, (u, s, t0, t1)
            q = lists[u, 2 * t0:2 * t1]
            pad = lists[u, 2 * t1:2 * (t1 + LIST_PAD)]
            assert not pad.any(), (u, s, "padding tiles")
            zero = np.nonzero(q == 0)[0]
            assert zero.size == 0 or (zero.size == 1 and zero[0] == q.size - 1), (u, s, zero)
            q = q[q != 0]
            cube = (q & ~np.uint32(31)) // np.uint32(64 * rs2)
            part = ((q & ~np.uint32(31)) % np.uint32(64 * rs2)) // np.uint32(16 * rs2)
            rows = q & np.uint32(31)
            mine = [j for j in ids if (j * splits) // Nkv == s] if splits > 1 else list(ids)
            want = sorted((j, k, min(16, vbs[j] - 16 * k)) for j in mine
                          for k in range((vbs[j] + 15) // 16))
            got = sorted(zip(cube.tolist(), part.tolist(), rows.tolist()))
            assert got == want, (u, s)
            assert (q.size + 1) // 2 == t1 - t0, (u, s, "tile count")
            # one ascending sweep of the cubes, wrapped at most once
            seq = [j for i, j in enumerate(cube.tolist()) if i == 0 or j != cube[i - 1]]
            drops = sum(1 for a, b2 in zip(seq, seq[1:]) if b2 < a)
            assert drops <= 1 and len(set(seq)) == len(seq), (u, s, seq)
            if drops == 1:
                assert seq[-1] < seq[0], (u, s, seq)
                rotated += 1
    return rotated


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("counts", [False, True])
def test_tile_lists_hold_every_selected_quarter_once(splits, counts):
    rng = np.random.default_rng(70 + splits + 10 * counts)
    B, Nq, Nkv, NH, D, topk = 2, 40, 40, 3, 64, 12
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    vbs = rng.choice([0, 1, 8, 15, 16, 17, 31, 32, 33, 48, 63, 64], size=Nkv).astype(np.int32)
    idx = np.stack([np.stack([np.stack([rng.permutation(Nkv)[:topk] for _ in range(Nq)])
                              for _ in range(NH)]) for _ in range(B)]).astype(np.int32)
    valid = rng.integers(0, topk + 1, size=(B, NH, Nq)).astype(np.int32) if counts else None
    assert vsa.fwd_splits(Nkv, D, topk, splits) == splits
    ws = torch.zeros(vsa.fwd_workspace_bytes(B, Nq, Nkv, NH, D, topk, splits), dtype=torch.uint8,
                     device="cuda")
    vsa.fwd_lut(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(idx).cuda(),
                None if valid is None else torch.from_numpy(valid).cuda(),
                torch.from_numpy(vbs).cuda(), workspace=ws, kv_splits=splits)
    torch.cuda.synchronize()
    rotated = _check_lists(ws, B, Nq, Nkv, NH, D, topk, idx, valid, vbs, splits)
    print(f"[tile lists splits={splits} counts={counts}] rotated sweeps: {rotated}", flush=True)
    assert rotated > 0  # most units start their sweep past their smallest id


def test_tile_lists_of_dense_rows_are_not_rotated():
    """Rows that select every key cube keep the plain ascending sweep."""
    rng = np.random.default_rng(75)
    B, Nq, Nkv, NH, D = 1, 12, 12, 2, 64
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    vbs = rng.integers(1, 65, size=Nkv).astype(np.int32)
    idx = np.stack([np.stack([rng.permutation(Nkv) for _ in range(Nq)])
                    for _ in range(NH)])[None].astype(np.int32)
    ws = torch.zeros(vsa.fwd_workspace_bytes(B, Nq, Nkv, NH, D, Nkv), dtype=torch.uint8,
                     device="cuda")
    vsa.fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(idx).cuda(),
            torch.from_numpy(vbs).cuda(), workspace=ws)
    torch.cuda.synchronize()
    assert _check_lists(ws, B, Nq, Nkv, NH, D, Nkv, idx, None, vbs, 1) == 0


@pytest.mark.parametrize("topk", [64, 65, 128, 129, 256, 257])
@pytest.mark.parametrize("splits", [1, 2])
def test_tile_lists_across_the_sort_paths(topk, splits):
    """Rows of up to 64, 128 and 256 ids are sorted in registers (1, 2 or 4
    keys per lane), longer ones through LDS: every path gives the same
    lists (each selected quarter once, one wrapped ascending sweep)."""
    rng = np.random.default_rng(80 + topk + splits)
    B, Nq, Nkv, NH, D = 1, 8, 300, 2, 64
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    vbs = rng.choice([1, 8, 16, 17, 33, 48, 64], size=Nkv).astype(np.int32)
    idx = np.stack([np.stack([rng.permutation(Nkv)[:topk] for _ in range(Nq)])
                    for _ in range(NH)])[None].astype(np.int32)
    assert vsa.fwd_splits(Nkv, D, topk, splits) == splits
    ws = torch.zeros(vsa.fwd_workspace_bytes(B, Nq, Nkv, NH, D, topk, splits), dtype=torch.uint8,
                     device="cuda")
    vsa.fwd_lut(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v), torch.from_numpy(idx).cuda(),
                None, torch.from_numpy(vbs).cuda(), workspace=ws, kv_splits=splits)
    torch.cuda.synchronize()
    rotated = _check_lists(ws, B, Nq, Nkv, NH, D, topk, idx, None, vbs, splits)
    print(f"[tile lists topk={topk} splits={splits}] rotated sweeps: {rotated}", flush=True)
