"""GPU parity of the fine stage at the edges of its input ranges.

* V magnitudes outside fp16's normal range: heads whose v reach |v| >= 1e5, or
  stay below 2^-14, and a head with a few huge rows among N(0, 1) values. The
  Wan2.2 Production Values dataset card's "Operator contract" takes bf16 v
  with no range limit, so the output must match the oracle there too.
* Index rows longer than the list pre-pass sorts (more than 1024 ids): the
  tile list then keeps the given id order.
* More than 4096 query cubes: the dispatch-order pass is skipped (also with
  key-range splits).

Every unit of the first case is checked; the other two check sampled units
against ``oracle.fwd_unit`` (plus the first and last units)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import video_dit_block_amd as vsa
from gpu_util import COS_MIN, MAX_ABS, MEAN_ABS, assert_fine_ok, cosine, from_gpu_bf16, to_gpu_bf16

pytestmark = pytest.mark.gpu


def _idx(rng, B, NH, Nq, Nkv, topk):
    return np.stack([np.stack([np.stack([rng.permutation(Nkv)[:topk] for _ in range(Nq)])
                               for _ in range(NH)]) for _ in range(B)]).astype(np.int32)


def _gpu_fwd(q, k, v, idx, vbs):
    return from_gpu_bf16(vsa.fwd(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v),
                                 torch.from_numpy(idx).cuda(), torch.from_numpy(vbs).cuda()))


@pytest.mark.parametrize("D", [64, 128])
def test_v_beyond_fp16_range(D):
    """Head 0: v ~ N(0,1); head 1: v * 2^17 (|v| up to ~5e5); head 2:
    v * 2^-20 (|v| below 2^-14 almost everywhere); head 3: N(0,1) with three
    key rows of magnitude 3e5. Heads 1 and 2 are compared after dividing by
    their power-of-two scale (bf16 rounding commutes with it). Head 3 is checked
    element by element against the unrounded oracle with the bound the
    arithmetic gives: |delta| <= 3e-2 + 2^-8 |ref| + 2^-9 A. The bf16 output
    rounds to 8 significant bits (relative error <= 2^-8); the weights enter
    the P.V product rounded to fp16 (relative error <= 2^-11 each, so at most
    2^-10 A on the normalised sum, A = sum_j w_j |v_j| the softmax-weighted
    magnitude of the values; the bound keeps a factor 2 on that term). A can
    be far above |ref| where large rows of opposite sign cancel. The oracle
    gives A exactly as its output on |v|."""
    rng = np.random.default_rng(40 + D)
    B, Nq, Nkv, NH, topk = 1, 6, 6, 4, 4
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    vf = f32(B, Nkv * 64, NH, D)
    scale = np.array([1.0, 2.0 ** 17, 2.0 ** -20, 1.0])
    vf[:, :, 1] *= np.float32(scale[1])
    vf[:, :, 2] *= np.float32(scale[2])
    for row in (3, 70, 200):          # real rows of cubes 0, 1, 3
        vf[0, row, 3, :] = np.float32(3e5) * np.sign(vf[0, row, 3, :])
    v = synth.bf16_bits_from_f32(vf)
    vbs = np.array([64, 40, 17, 64, 8, 33], np.int32)
    idx = _idx(rng, B, NH, Nq, Nkv, topk)
    print(f"[v range D={D}] max|v| per head "
          f"{[float(np.abs(oracle.decode_bf16(v[..., h, :])).max()) for h in range(NH)]}",
          flush=True)
    out = _gpu_fwd(q, k, v, idx, vbs)
    ref = oracle.fwd(oracle.decode_bf16(q), oracle.decode_bf16(k), oracle.decode_bf16(v), idx, vbs)
    g = oracle.decode_bf16(out)
    assert np.all(np.isfinite(g))
    # heads 0-2: the acceptance rule on the values divided by the head's scale
    norm_g = {h: g[:, :, h] / scale[h] for h in range(3)}
    norm_r = {h: ref[:, :, h] / scale[h] for h in range(3)}
    for h in range(3):
        d = np.abs(norm_g[h] - oracle.round_to_bf16(norm_r[h]))
        cos = cosine(norm_g[h], oracle.round_to_bf16(norm_r[h]))
        print(f"[v range D={D}] head {h}: cos {cos:.8f} max {d.max():.3g} mean {d.mean():.3g}",
              flush=True)
        assert cos >= COS_MIN and d.max() <= MAX_ABS and d.mean() <= MEAN_ABS, h
    # head 3: mixed magnitudes
    r3 = ref[:, :, 3]
    a3 = oracle.fwd(oracle.decode_bf16(q), oracle.decode_bf16(k), np.abs(oracle.decode_bf16(v)),
                    idx, vbs)[:, :, 3]
    d3 = np.abs(g[:, :, 3] - r3)
    bound = MAX_ABS + 2.0 ** -8 * np.abs(r3) + 2.0 ** -9 * a3
    print(f"[v range D={D}] head 3: worst |delta| / bound {(d3 / bound).max():.3g}, "
          f"worst |delta| / A {(d3 / a3).max():.3g}", flush=True)
    assert np.all(d3 <= bound)
    assert cosine(g[:, :, 3], oracle.round_to_bf16(r3)) >= COS_MIN
    # the huge head really exceeds fp16: a saturating conversion would fail above
    assert np.abs(oracle.decode_bf16(v[..., 1, :])).max() > 65504


def test_index_rows_longer_than_the_sorted_list():
    """1100 ids per row (every key cube, shuffled), ragged vbs including empty
    cubes: the list pre-pass keeps the row's order above 1024 ids."""
    rng = np.random.default_rng(77)
    B, Nq, Nkv, NH, D, topk = 1, 3, 1100, 2, 64, 1100
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    vbs = rng.integers(0, 65, size=Nkv).astype(np.int32)
    idx = _idx(rng, B, NH, Nq, Nkv, topk)
    print(f"[long rows] Nkv={Nkv} topk={topk} real keys {int(vbs.sum())}", flush=True)
    out = _gpu_fwd(q, k, v, idx, vbs)
    q64, k64, v64 = (oracle.decode_bf16(a) for a in (q, k, v))
    gpu, ref = {}, {}
    for h in range(NH):
        gpu[h] = np.stack([out[0, c * 64:(c + 1) * 64, h] for c in range(Nq)])
        ref[h] = np.stack([oracle.fwd_unit(q64, k64, v64, idx, vbs, 0, h, c) for c in range(Nq)])
    assert_fine_ok(gpu, ref, "long rows")


@pytest.mark.parametrize("splits", [0, 3])
def test_more_query_cubes_than_the_dispatch_order_ranks(splits):
    """Nq = Nkv = 4100 (above the 4096 cubes the dispatch-order pass ranks),
    topk = 4, ragged vbs: sampled units plus the first and last; also in 3
    key-range splits (items in plain rank order)."""
    rng = np.random.default_rng(78)
    B, Nq, Nkv, NH, D, topk = 1, 4100, 4100, 1, 64, 4
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    q = synth.bf16_bits_from_f32(f32(B, Nq * 64, NH, D))
    k = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    v = synth.bf16_bits_from_f32(f32(B, Nkv * 64, NH, D))
    vbs = rng.integers(1, 65, size=Nkv).astype(np.int32)
    idx = np.stack([rng.choice(Nkv, size=topk, replace=False) for _ in range(Nq)])
    idx = idx.reshape(B, NH, Nq, topk).astype(np.int32)
    print(f"[Nq>4096] Nq={Nq} topk={topk} splits={vsa.fwd_splits(Nkv, D, topk, splits)}",
          flush=True)
    if splits == 0:
        out = _gpu_fwd(q, k, v, idx, vbs)
    else:
        out = from_gpu_bf16(vsa.fwd_lut(to_gpu_bf16(q), to_gpu_bf16(k), to_gpu_bf16(v),
                                        torch.from_numpy(idx).cuda(), None,
                                        torch.from_numpy(vbs).cuda(), kv_splits=splits))
    q64, k64, v64 = (oracle.decode_bf16(a) for a in (q, k, v))
    cubes = sorted(set(rng.choice(Nq, size=64, replace=False).tolist()) | {0, Nq - 1})
    gpu = {0: np.stack([out[0, c * 64:(c + 1) * 64, 0] for c in cubes])}
    ref = {0: np.stack([oracle.fwd_unit(q64, k64, v64, idx, vbs, 0, 0, c) for c in cubes])}
    assert_fine_ok(gpu, ref, "Nq>4096")
