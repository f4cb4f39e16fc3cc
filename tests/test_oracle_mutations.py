"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin fails.

Each mutation replaces one oracle function with a wrong variant for the length
of one check; the pin it is paired with must notice.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import vsa_oracle as vo

from test_oracle_pins import (_dense_masked, _random_topk, _tiled_case, coarse_sdpa_error,
                              combine_pin, hilbert_pin, mask_lut_pin, tile_order_pin,
                              topk_tie_pin)


def _fwd_no_vbs(q_t, k_t, v_t, topk_idx, vbs, b, h, c, sm_scale=None):
    full = np.full_like(np.asarray(vbs), 64)          # padding not masked
    return _orig_fwd_unit(q_t, k_t, v_t, topk_idx, full, b, h, c, sm_scale)


def _fwd_wrong_scale(q_t, k_t, v_t, topk_idx, vbs, b, h, c, sm_scale=None):
    return _orig_fwd_unit(q_t, k_t, v_t, topk_idx, vbs, b, h, c, 1.0 / q_t.shape[-1])


def _fwd_transposed_kv(q_t, k_t, v_t, topk_idx, vbs, b, h, c, sm_scale=None):
    return _orig_fwd_unit(q_t, v_t, k_t, topk_idx, vbs, b, h, c, sm_scale)


_orig_fwd_unit = vo.fwd_unit


def _pin_dense(monkeypatch, mutant):
    monkeypatch.setattr(vo, "fwd_unit", mutant)
    q, k, v, vbs = _tiled_case(5, 6, 7, NH=2, D=16)
    idx = _random_topk(1, 2, 8, 3)
    got = vo.fwd(q, k, v, idx, vbs)
    ref = _dense_masked(q, k, v, idx, vbs, 1 / math.sqrt(16))
    return np.max(np.abs(got - ref))


@pytest.mark.parametrize("mutant", [_fwd_no_vbs, _fwd_wrong_scale, _fwd_transposed_kv])
def test_dense_pin_catches_fwd_mutations(monkeypatch, mutant):
    assert _pin_dense(monkeypatch, mutant) > 1e-6


def test_dense_pin_passes_unmutated(monkeypatch):
    assert _pin_dense(monkeypatch, _orig_fwd_unit) < 1e-12


def test_pool_pin_catches_denominator_64(monkeypatch):
    orig = vo.mean_pool

    def pool64(x_t, vbs):
        return orig(x_t, vbs) * (np.asarray(vbs, np.float64)[None, None, :, None] / 64.0)

    monkeypatch.setattr(vo, "mean_pool", pool64)
    vbs = oracle.cube_sizes(5, 6, 7)
    const = np.full((1, 8 * 64, 1, 3), 0.7)
    assert np.max(np.abs(vo.mean_pool(const, vbs) - 0.7)) > 0.1


def test_topk_pin_catches_ties_to_the_higher_id(monkeypatch):
    """A top-k that breaks equal scores toward the higher id fails the tie pin
    (the unmutated oracle passes it)."""
    def topk_ties_high(S, k):
        order = np.argsort(-S[..., ::-1], axis=-1, kind="stable")
        return (S.shape[-1] - 1 - order[..., :k]).astype(np.int32)

    monkeypatch.setattr(vo, "topk_select", topk_ties_high)
    assert not topk_tie_pin(vo.topk_select)
    monkeypatch.undo()
    assert topk_tie_pin(vo.topk_select)


def test_tile_pin_catches_w_slowest_cube_order(monkeypatch):
    """slot_tokens with the cubes enumerated w-slowest instead of t-slowest
    fails the independent-derivation pin."""
    orig = vo.slot_tokens

    def w_slowest(T, H, W):
        good = orig(T, H, W)
        Nt, Nh, Nw = vo.cube_grid(T, H, W)
        perm = [((cw * Nh + ch) * Nt + ct) for ct in range(Nt) for ch in range(Nh)
                for cw in range(Nw)]
        return good[np.argsort(perm)]

    monkeypatch.setattr(vo, "slot_tokens", w_slowest)
    assert not tile_order_pin(vo.slot_tokens, (5, 6, 7))
    monkeypatch.undo()
    assert tile_order_pin(vo.slot_tokens, (5, 6, 7))


_orig_coarse = vo.coarse_output


def _coarse_all_cubes(q_t, k_t, v_t, vbs, sm_scale=None):
    # empty cubes kept as keys (their pooled vectors are 0)
    Qc, Kc, Vc = (vo.mean_pool(x, vbs) for x in (q_t, k_t, v_t))
    s = Qc @ np.swapaxes(Kc, -1, -2) / math.sqrt(q_t.shape[-1])
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    return (p @ Vc) / p.sum(axis=-1, keepdims=True)


def _coarse_scale_1_over_d(q_t, k_t, v_t, vbs, sm_scale=None):
    return _orig_coarse(q_t, k_t, v_t, vbs, 1.0 / q_t.shape[-1])


def _coarse_swapped_kv(q_t, k_t, v_t, vbs, sm_scale=None):
    return _orig_coarse(q_t, v_t, k_t, vbs, sm_scale)


def _coarse_pool_64(q_t, k_t, v_t, vbs, sm_scale=None):
    scale = np.asarray(vbs, np.float64)[None, :, None, None].repeat(64, axis=1).reshape(1, -1, 1, 1)
    f = scale / 64.0      # mean over 64 slots of zero-padded cubes
    return _orig_coarse(q_t * f, k_t * f, v_t * f, vbs, sm_scale)


@pytest.mark.parametrize("mutant", [_coarse_all_cubes, _coarse_scale_1_over_d, _coarse_swapped_kv,
                                    _coarse_pool_64])
def test_sdpa_pin_catches_coarse_mutations(mutant):
    assert coarse_sdpa_error(mutant) > 1e-6


def test_combine_pin_catches_swapped_gates(monkeypatch):
    orig = vo.gated_combine
    monkeypatch.setattr(vo, "gated_combine", lambda of, oc, gc, gf: orig(of, oc, gf, gc))
    assert not combine_pin(vo.gated_combine)


def test_hilbert_pin_catches_a_missing_gray_encode(monkeypatch):
    def no_gray(x0, x1, x2, bits):
        # the same construction without the Gray-encode step
        X = [x0, x1, x2]
        q = 1 << (bits - 1)
        while q > 1:
            low = q - 1
            for i in range(3):
                if X[i] & q:
                    X[0] ^= low
                else:
                    t = (X[0] ^ X[i]) & low
                    X[0] ^= t
                    X[i] ^= t
            q >>= 1
        h = 0
        for plane in range(bits - 1, -1, -1):
            for v in X:
                h = 2 * h + ((v >> plane) & 1)
        return h

    monkeypatch.setattr(vo, "hilbert_index_3d", no_gray)
    assert not hilbert_pin(vo.hilbert_index_3d, 2)


def test_mask_pin_catches_keeping_the_highest_ids():
    orig = vo.mask_to_lut

    def keep_highest(block_mask, max_kv):
        m = np.asarray(block_mask) != 0
        full, cnt_all, _ = orig(m, m.shape[-1])
        ids, cnt, tr = orig(m, max_kv)
        for r in np.ndindex(*m.shape[:-1]):
            n = cnt_all[r]
            if n > max_kv:
                ids[r][:max_kv] = full[r][n - max_kv:n]
        return ids, cnt, tr

    assert not mask_lut_pin(keep_highest)
