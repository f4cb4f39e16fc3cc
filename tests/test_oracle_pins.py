"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each test ties one oracle function to something other than itself: numbers the
pages print, closed forms derived by hand, an independent formulation (brute
force, a library routine), or an invariant of the mathematics. Run on the CPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle

RNG = np.random.default_rng(1234)


def _randn(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ------------------------------------------------------------------ tiling

def test_printed_counts_wan_grid():
    """Dataset card "Shapes": S_padded = 39936 = 624 x 64, real = 32760 = 21x30x52,
    Nq = Nkv = 624 = 6 x 8 x 13."""
    assert oracle.cube_grid(21, 30, 52) == (6, 8, 13)
    vbs = oracle.cube_sizes(21, 30, 52)
    assert vbs.shape == (624,)
    assert vbs.size * 64 == 39936
    assert int(vbs.sum()) == 32760


def test_printed_counts_720p_grid():
    """FastVideo STA guide, "The 115K Token Sequence Wall": latent (30, 48, 80)
    gives N = 115,200 tokens."""
    vbs = oracle.cube_sizes(30, 48, 80)
    assert vbs.size == 8 * 12 * 20
    assert int(vbs.sum()) == 115200


@pytest.mark.parametrize("grid,hist", [
    # 21 = 5*4 + 1, 30 = 7*4 + 2, 52 = 13*4: cube sizes are et*eh*4 with
    # et in {4 (5 cubes), 1 (1 cube)}, eh in {4 (7 cubes), 2 (1 cube)}, 13 cw.
    ((21, 30, 52), {64: 5 * 7 * 13, 32: 5 * 1 * 13, 16: 1 * 7 * 13, 8: 1 * 1 * 13}),
    # 30 = 7*4 + 2, 48 = 12*4, 80 = 20*4
    ((30, 48, 80), {64: 7 * 12 * 20, 32: 1 * 12 * 20}),
])
def test_vbs_histogram_closed_form(grid, hist):
    vbs = oracle.cube_sizes(*grid)
    vals, counts = np.unique(vbs, return_counts=True)
    assert dict(zip(vals.tolist(), counts.tolist())) == hist


def test_vbs_tiny_row_major_order():
    """5x6x7: extents t (4, 1), h (4, 2), w (4, 3); cube id (ct*Nh + ch)*Nw + cw."""
    expect = [4 * 4 * 4, 4 * 4 * 3, 4 * 2 * 4, 4 * 2 * 3,
              1 * 4 * 4, 1 * 4 * 3, 1 * 2 * 4, 1 * 2 * 3]
    assert oracle.cube_sizes(5, 6, 7).tolist() == expect


def tile_order_pin(slot_tokens_fn, grid) -> bool:
    """Token -> slot by sorting tokens on (cube id, t, h, w): an independent
    formulation of the cube-major order with real tokens first, row-major inside
    the clipped cube. True when slot_tokens_fn agrees with it."""
    T, H, W = grid
    Nt, Nh, Nw = -(-T // 4), -(-H // 4), -(-W // 4)
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    t, y, x = t.ravel(), y.ravel(), x.ravel()
    nat = (t * H + y) * W + x
    cube = ((t // 4) * Nh + y // 4) * Nw + x // 4
    order = np.lexsort((x, y, t, cube))          # primary key: cube
    expect = np.full((Nt * Nh * Nw, 64), -1)
    for c in range(Nt * Nh * Nw):
        members = nat[order][cube[order] == c]
        expect[c, :members.size] = members
    return np.array_equal(slot_tokens_fn(T, H, W), expect)


@pytest.mark.parametrize("grid", [(5, 6, 7), (4, 4, 4), (1, 1, 1), (9, 3, 5), (8, 13, 2)])
def test_tile_permutation_independent_derivation(grid):
    assert tile_order_pin(oracle.slot_tokens, grid)


def test_tile_untile_roundtrip_bitwise_and_zero_pads():
    T, H, W = 5, 6, 7
    x = RNG.integers(0, 2 ** 16, size=(2, T * H * W, 3, 8), dtype=np.uint16)
    xt, vbs = oracle.tile(x, T, H, W)
    assert xt.shape == (2, 8 * 64, 3, 8) and xt.dtype == np.uint16
    for c in range(8):
        assert np.all(xt[:, 64 * c + vbs[c]:64 * (c + 1)] == 0)
    np.testing.assert_array_equal(oracle.untile(xt, T, H, W), x)


# ---------------------------------------------------------------- bf16 values

def test_decode_bf16_known_values():
    bits = np.array([0x3F80, 0xBF80, 0x4000, 0x0000, 0x8000, 0x7F7F, 0x0001], np.uint16)
    expect = [1.0, -1.0, 2.0, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133]
    np.testing.assert_array_equal(oracle.decode_bf16(bits), expect)


def test_round_to_bf16_ties_and_library():
    # ties to even at 1 + 2^-8 (halfway between 1 and 1 + 2^-7)
    cases = {1 + 2 ** -8: 1.0, 1 + 3 * 2 ** -8: 1 + 2 ** -6, -(1 + 2 ** -8): -1.0,
             1 + 2 ** -8 + 2 ** -30: 1 + 2 ** -7,
             2.0 ** -140: 0.0,                 # below half the smallest subnormal
             3 * 2.0 ** -134: 2.0 ** -132,     # subnormal tie -> even multiple
             (2 - 2 ** -9) * 2.0 ** 127: math.inf}
    for x, r in cases.items():
        got = float(oracle.round_to_bf16(np.array([x]))[0])
        assert got == r, (x, got, r)
    # float32-representable inputs: torch's float32 -> bfloat16 conversion
    x = (RNG.standard_normal(20000) * np.exp(RNG.uniform(-30, 30, 20000))).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_to_bf16(x.astype(np.float64)), lib)


# ------------------------------------------------------------- fine stage

def _dense_masked(q_t, k_t, v_t, topk_idx, vbs, scale):
    """Brute force: full S_padded x S_padded score matrix with the block mask
    M[i, j] = cube(j) in sel(cube(i)) and slot(j) < vbs[cube(j)]."""
    B, S, NH, D = q_t.shape
    cube_of = np.arange(S) // 64
    slot_of = np.arange(S) % 64
    out = np.zeros_like(q_t)
    for b in range(B):
        for h in range(NH):
            sel = np.zeros((S // 64, S // 64), bool)
            for c in range(S // 64):
                sel[c, topk_idx[b, h, c]] = True
            M = sel[cube_of][:, cube_of] & (slot_of < vbs[cube_of])[None, :]
            s = q_t[b, :, h] @ k_t[b, :, h].T * scale
            s = np.where(M, s, -np.inf)
            s -= s.max(axis=1, keepdims=True)
            p = np.where(M, np.exp(s), 0.0)
            out[b, :, h] = p @ v_t[b, :, h] / p.sum(axis=1, keepdims=True)
    return out


def _tiled_case(T, H, W, NH, D, B=1, rng=RNG):
    vbs = oracle.cube_sizes(T, H, W)
    Nc = vbs.size
    q = _randn(B, Nc * 64, NH, D, rng=rng)
    k = _randn(B, Nc * 64, NH, D, rng=rng)
    v = _randn(B, Nc * 64, NH, D, rng=rng)
    return q, k, v, vbs


def _random_topk(B, NH, Nc, k, rng=RNG):
    return np.stack([np.stack([np.stack([rng.permutation(Nc)[:k] for _ in range(Nc)])
                               for _ in range(NH)]) for _ in range(B)]).astype(np.int32)


@pytest.mark.parametrize("grid,k,D", [((5, 6, 7), 3, 16), ((9, 5, 6), 4, 8), ((4, 8, 4), 1, 8)])
def test_fwd_equals_dense_masked_softmax(grid, k, D):
    q, kk, v, vbs = _tiled_case(*grid, NH=2, D=D, B=2)
    idx = _random_topk(2, 2, vbs.size, k)
    got = oracle.fwd(q, kk, v, idx, vbs)
    ref = _dense_masked(q, kk, v, idx, vbs, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_fwd_topk_all_full_cubes_equals_sdpa():
    """8x8x8 grid: all cubes full; topk = all cubes is dense attention over the
    tiled sequence (torch CPU float64 scaled_dot_product_attention)."""
    T = H = W = 8
    q, k, v, vbs = _tiled_case(T, H, W, NH=2, D=32)
    assert np.all(vbs == 64)
    idx = np.tile(np.arange(8, dtype=np.int32), (1, 2, 8, 1))
    got = oracle.fwd(q, k, v, idx, vbs)
    tq, tk, tv = (torch.from_numpy(a).permute(0, 2, 1, 3) for a in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3)
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_fwd_topk_all_partial_cubes_equals_sdpa_on_real_tokens():
    """With partial cubes, topk = all equals dense attention over the real
    tokens in natural order (the padding deleted), for every real row."""
    T, H, W = 5, 6, 7
    NH, D = 3, 16
    qn, kn, vn = (_randn(1, T * H * W, NH, D) for _ in range(3))
    qt, vbs = oracle.tile(qn, T, H, W)
    kt, _ = oracle.tile(kn, T, H, W)
    vt, _ = oracle.tile(vn, T, H, W)
    idx = np.tile(np.arange(8, dtype=np.int32)[::-1], (1, NH, 8, 1))
    got = oracle.untile(oracle.fwd(qt, kt, vt, idx, vbs), T, H, W)
    tq, tk, tv = (torch.from_numpy(a).permute(0, 2, 1, 3) for a in (qn, kn, vn))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3)
    np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("poison", [np.nan, 1e30, -np.inf])
def test_fwd_ignores_padding_values(poison):
    """Masking by vbs is the same as deleting the padding: poisoned padding
    slots of k and v leave every output row unchanged (bit for bit)."""
    q, k, v, vbs = _tiled_case(5, 6, 7, NH=2, D=16)
    idx = _random_topk(1, 2, 8, 5)
    ref = oracle.fwd(q, k, v, idx, vbs)
    k2, v2 = k.copy(), v.copy()
    for c in range(8):
        k2[:, 64 * c + vbs[c]:64 * (c + 1)] = poison
        v2[:, 64 * c + vbs[c]:64 * (c + 1)] = poison
    got = oracle.fwd(q, k2, v2, idx, vbs)
    np.testing.assert_array_equal(got, ref)


def test_fwd_order_invariance():
    q, k, v, vbs = _tiled_case(9, 5, 6, NH=2, D=16)
    Nc = vbs.size
    idx = _random_topk(1, 2, Nc, 5)
    perm = np.array([[[RNG.permutation(row) for row in head] for head in b] for b in idx])
    a = oracle.fwd(q, k, v, idx, vbs)
    b = oracle.fwd(q, k, v, perm.astype(np.int32), vbs)
    np.testing.assert_allclose(b, a, rtol=1e-14, atol=1e-15)


def test_fwd_convex_hull_of_selected_values():
    q, k, v, vbs = _tiled_case(5, 6, 7, NH=2, D=16)
    q *= 3.0
    idx = _random_topk(1, 2, 8, 3)
    out = oracle.fwd(q, k, v, idx, vbs)
    for h in range(2):
        for c in range(8):
            rows = np.concatenate([64 * j + np.arange(vbs[j]) for j in idx[0, h, c]])
            lo = v[0, rows, h].min(axis=0)
            hi = v[0, rows, h].max(axis=0)
            o = out[0, 64 * c:64 * (c + 1), h]
            assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def test_fwd_single_token_selection_returns_that_row():
    """topk = 1 onto a cube with vbs = 1: every row's output is that v row."""
    T, H, W = 5, 5, 5     # last cube along each axis has extent 1 -> vbs 1 corner
    vbs = oracle.cube_sizes(T, H, W)
    j = int(np.where(vbs == 1)[0][0])
    q, k, v, _ = _tiled_case(T, H, W, NH=1, D=8)
    idx = np.full((1, 1, vbs.size, 1), j, dtype=np.int32)
    out = oracle.fwd(q, k, v, idx, vbs)
    np.testing.assert_array_equal(out[0, :, 0], np.broadcast_to(v[0, 64 * j, 0], out[0, :, 0].shape))


def test_fwd_zero_query_is_mean_of_selected_values():
    q, k, v, vbs = _tiled_case(5, 6, 7, NH=1, D=8)
    q[:] = 0.0
    idx = _random_topk(1, 1, 8, 3)
    out = oracle.fwd(q, k, v, idx, vbs)
    for c in range(8):
        rows = np.concatenate([64 * j + np.arange(vbs[j]) for j in idx[0, 0, c]])
        np.testing.assert_allclose(out[0, 64 * c:64 * (c + 1), 0],
                                   np.broadcast_to(v[0, rows, 0].mean(axis=0), (64, 8)),
                                   rtol=0, atol=1e-14)


def test_fwd_huge_logits_finite_and_argmax():
    """Logits of order +-2000 (exp overflows without the row max): output is
    finite and equals the v row of the largest logit when the gap is large."""
    q, k, v, vbs = _tiled_case(5, 6, 7, NH=1, D=8)
    q *= 40.0
    k *= 40.0
    idx = _random_topk(1, 1, 8, 4)
    out = oracle.fwd(q, k, v, idx, vbs)
    assert np.all(np.isfinite(out))
    checked = 0
    for c in range(8):
        rows = np.concatenate([64 * j + np.arange(vbs[j]) for j in idx[0, 0, c]])
        s = q[0, 64 * c:64 * (c + 1), 0] @ k[0, rows, 0].T / math.sqrt(8)
        assert np.abs(s).max() > 500
        srt = np.sort(s, axis=1)
        for r in range(64):
            if srt[r, -1] - srt[r, -2] > 50:
                np.testing.assert_allclose(out[0, 64 * c + r, 0], v[0, rows[np.argmax(s[r])], 0],
                                           rtol=0, atol=1e-15)
                checked += 1
    assert checked > 100


def test_fwd_no_real_token_row_is_zero():
    q, k, v, vbs = _tiled_case(5, 6, 7, NH=1, D=8)
    vbs = vbs.copy()
    vbs[3] = 0
    idx = np.zeros((1, 1, 8, 1), dtype=np.int32)
    idx[..., 0] = 3
    out = oracle.fwd(q, k, v, idx, vbs)
    assert np.all(out == 0)


# ---------------------------------------------------------------- selector

def test_mean_pool_closed_forms_and_padding_excluded():
    T, H, W = 5, 6, 7
    vbs = oracle.cube_sizes(T, H, W)
    x = np.full((1, 8 * 64, 2, 4), 1e30)          # padding poisoned
    means = RNG.standard_normal((8, 2, 4))
    for c in range(8):
        n = int(vbs[c])
        # arithmetic progression around the mean: exact mean by symmetry
        offs = (np.arange(n) - (n - 1) / 2.0)[:, None, None] * 0.25
        x[0, 64 * c:64 * c + n] = means[c][None] + offs
    got = oracle.mean_pool(x, vbs)
    np.testing.assert_allclose(got[0], np.transpose(means, (1, 0, 2)), rtol=0, atol=1e-14)
    const = np.full((1, 8 * 64, 1, 3), 0.7)
    np.testing.assert_allclose(oracle.mean_pool(const, vbs), 0.7, rtol=0, atol=1e-15)


def test_cube_scores_constructed_ranking():
    """Orthonormal Kc and Qc = sum_j a_j Kc_j give scores exactly a (rotation
    of a known coefficient vector), so the ranking is known by construction."""
    n, D = 6, 6
    Qm, _ = np.linalg.qr(RNG.standard_normal((D, D)))
    Kc = Qm.T[None, None]                          # rows orthonormal
    a = RNG.standard_normal((1, 1, 3, n))
    Qc = a @ Kc[0, 0]
    S = oracle.cube_scores(Qc, Kc)
    np.testing.assert_allclose(S, a, rtol=0, atol=1e-13)
    idx = oracle.topk_select(S, 3)
    np.testing.assert_array_equal(idx[0, 0], np.argsort(-a[0, 0], axis=1)[:, :3])


def _rank_count_topk(row, k):
    """Brute force: id j's rank = #{i: s_i > s_j} + #{i < j: s_i == s_j}."""
    n = row.size
    out = np.empty(k, dtype=np.int64)
    for j in range(n):
        r = sum(1 for i in range(n) if row[i] > row[j] or (row[i] == row[j] and i < j))
        if r < k:
            out[r] = j
    return out


def topk_tie_pin(topk_fn) -> bool:
    """Rows full of ties (integer scores in [-3, 3]): topk_fn must give, for
    k = 1, 5, 17, exactly the brute-force rank count (score descending, equal
    scores by ascending id)."""
    S = np.random.default_rng(77).integers(-3, 4, size=(1, 2, 12, 17)).astype(np.float64)
    for k in (1, 5, 17):
        idx = topk_fn(S, k)
        for h in range(2):
            for i in range(12):
                if not np.array_equal(idx[0, h, i], _rank_count_topk(S[0, h, i], k)):
                    return False
    return True


def test_topk_matches_rank_counting_with_ties():
    assert topk_tie_pin(oracle.topk_select)


def test_topk_all_is_permutation_and_descending():
    S = RNG.standard_normal((2, 3, 9, 9))
    idx = oracle.topk_select(S, 9)
    for row_ids, row in zip(idx.reshape(-1, 9), S.reshape(-1, 9)):
        assert sorted(row_ids.tolist()) == list(range(9))
        assert np.all(np.diff(row[row_ids]) <= 0)


def test_select_end_to_end_tiny():
    """Selector output fed to the fine stage reproduces the brute-force dense
    masked attention built from the same selection (tiny grid)."""
    T, H, W = 5, 6, 7
    qn, kn, vn = (_randn(1, T * H * W, 2, 16) for _ in range(3))
    qt, vbs = oracle.tile(qn, T, H, W)
    kt, _ = oracle.tile(kn, T, H, W)
    vt, _ = oracle.tile(vn, T, H, W)
    idx, S = oracle.select(qt, kt, vbs, 3)
    # the selection is the top-3 of brute-force per-cube means dotted together
    for h in range(2):
        for i in range(8):
            qm = qn[0, oracle.slot_tokens(T, H, W)[i][:vbs[i]], h].mean(axis=0)
            sc = [qm @ kn[0, oracle.slot_tokens(T, H, W)[j][:vbs[j]], h].mean(axis=0)
                  for j in range(8)]
            np.testing.assert_array_equal(idx[0, h, i], _rank_count_topk(np.array(sc), 3))
    got = oracle.fwd(qt, kt, vt, idx, vbs)
    np.testing.assert_allclose(got, _dense_masked(qt, kt, vt, idx, vbs, 0.25), rtol=0, atol=1e-12)


def test_fwd_rejects_bad_indices():
    q, k, v, vbs = _tiled_case(5, 6, 7, NH=1, D=8)
    idx = np.zeros((1, 1, 8, 2), dtype=np.int32)      # duplicate id 0
    with pytest.raises(AssertionError):
        oracle.fwd(q, k, v, idx, vbs)
    idx[..., 1] = 8                                     # out of range
    with pytest.raises(AssertionError):
        oracle.fwd(q, k, v, idx, vbs)


# ---------------------------------------------- lookup table and row statistics

def test_fwd_lut_full_counts_equals_fwd():
    q, kk, v, vbs = _tiled_case(5, 6, 7, NH=2, D=16, B=2)
    idx = _random_topk(2, 2, vbs.size, 4)
    out, _, _ = oracle.fwd_lut(q, kk, v, idx, None, vbs)
    np.testing.assert_array_equal(out, oracle.fwd(q, kk, v, idx, vbs))
    full = np.full(idx.shape[:3], 4, np.int32)
    out2, _, _ = oracle.fwd_lut(q, kk, v, idx, full, vbs)
    np.testing.assert_array_equal(out2, out)


def test_fwd_lut_counts_equal_truncated_rows_and_dense_mask():
    """valid_block_num = n uses exactly the first n ids of each row: equal to
    the brute-force masked attention over those ids (rows with n = 0 are 0)."""
    rng = np.random.default_rng(7)
    q, kk, v, vbs = _tiled_case(9, 5, 6, NH=2, D=8, B=1, rng=rng)
    Nc = vbs.size
    idx = _random_topk(1, 2, Nc, 5, rng=rng)
    valid = rng.integers(1, 6, size=(1, 2, Nc)).astype(np.int32)
    valid[0, 0, 0] = 0
    out, lse, mp = oracle.fwd_lut(q, kk, v, idx, valid, vbs)
    scale = 1 / math.sqrt(8)
    for h in range(2):
        for c in range(Nc):
            n = int(valid[0, h, c])
            rows = slice(64 * c, 64 * (c + 1))
            if n == 0:
                assert np.all(out[0, rows, h] == 0) and np.all(np.isneginf(lse[0, h, rows]))
                assert np.all(mp[0, h, rows] == 0)
                continue
            # a row-specific dense reference: only row (h, c) matters here
            sub_full = np.repeat(idx[:, :, :, :1], n, axis=3)
            sub_full[0, h, c] = idx[0, h, c, :n]
            ref = _dense_masked(q, kk, v, sub_full, vbs, scale)
            np.testing.assert_allclose(out[0, rows, h], ref[0, rows, h], rtol=0, atol=1e-12)


def test_lse_and_max_prob_against_dense_logsumexp():
    """lse equals scipy's logsumexp over the brute-force masked score row, and
    max_prob equals the largest entry of the dense softmax row."""
    from scipy.special import logsumexp, softmax
    rng = np.random.default_rng(11)
    q, kk, v, vbs = _tiled_case(5, 6, 7, NH=1, D=16, B=1, rng=rng)
    Nc = vbs.size
    idx = _random_topk(1, 1, Nc, 3, rng=rng)
    _, lse, mp = oracle.fwd_lut(q, kk, v, idx, None, vbs)
    scale = 1 / math.sqrt(16)
    S = Nc * 64
    cube_of = np.arange(S) // 64
    slot_of = np.arange(S) % 64
    sel = np.zeros((Nc, Nc), bool)
    for c in range(Nc):
        sel[c, idx[0, 0, c]] = True
    M = sel[cube_of][:, cube_of] & (slot_of < vbs[cube_of])[None, :]
    s = np.where(M, q[0, :, 0] @ kk[0, :, 0].T * scale, -np.inf)
    np.testing.assert_allclose(lse[0, 0], logsumexp(s, axis=1), rtol=0, atol=1e-12)
    np.testing.assert_allclose(mp[0, 0], softmax(s, axis=1).max(axis=1), rtol=1e-12, atol=0)


def test_stats_closed_forms():
    """One key: max_prob = 1 and lse = its scaled score. n keys with equal
    scores: max_prob = 1/n and lse = s + log n."""
    D = 8
    vbs = np.array([1, 64, 0, 5], np.int32)
    q = np.zeros((1, 4 * 64, 1, D))
    k = np.zeros((1, 4 * 64, 1, D))
    v = RNG.standard_normal((1, 4 * 64, 1, D))
    q[0, :, 0, 0] = 1.0
    k[0, 0, 0, 0] = 3.0                     # cube 0: one real token, score 3/sqrt(8)
    k[0, 64:128, 0, 0] = 2.0                # cube 1: 64 equal scores 2/sqrt(8)
    idx = np.array([[[[0, 1], [1, 2], [2, 3], [3, 0]]]], np.int32)
    valid = np.array([[[1, 1, 1, 1]]], np.int32)
    _, lse, mp = oracle.fwd_lut(q, k, v, idx, valid, vbs)
    r = lambda c: slice(64 * c, 64 * (c + 1))
    np.testing.assert_allclose(mp[0, 0, r(0)], 1.0, rtol=1e-15)
    np.testing.assert_allclose(lse[0, 0, r(0)], 3 / math.sqrt(D), rtol=1e-15)
    np.testing.assert_allclose(mp[0, 0, r(1)], 1 / 64, rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0, r(1)], 2 / math.sqrt(D) + math.log(64), rtol=1e-14)
    assert np.all(np.isneginf(lse[0, 0, r(2)])) and np.all(mp[0, 0, r(2)] == 0)  # cube 2 empty
    np.testing.assert_allclose(mp[0, 0, r(3)], 1 / 5, rtol=1e-14)   # 5 zero scores
    np.testing.assert_allclose(lse[0, 0, r(3)], math.log(5), rtol=1e-14)


# ------------------------------------------------ cumulative-mass selector

def test_cdf_counts_constructed_weights():
    """Scores log(8), log(4), log(2), 0, 0 at scale 1 give weights 8, 4, 2, 1, 1
    (total 16): cumulative shares 0.5, 0.75, 0.875, 0.9375, 1."""
    S = np.array([[0.0, math.log(2), math.log(8), 0.0, math.log(4)]])
    for tau, n in [(0.3, 1), (0.5, 1), (0.51, 2), (0.75, 2), (0.76, 3), (0.875, 3),
                   (0.9, 4), (0.95, 5), (1.0, 5)]:
        ids, cnt = oracle.cdf_counts(S, 5, tau, 1.0)
        assert cnt[0] == n, (tau, cnt[0], n)
        assert list(ids[0]) == [2, 4, 1, 0, 3]   # descending, ties by lower id
    _, cnt = oracle.cdf_counts(S, 2, 0.99, 1.0)
    assert cnt[0] == 2                            # capped at max_k


def test_cdf_counts_uniform_rows_and_monotone():
    N = 37
    S = np.full((3, N), 1.5)
    for tau in (0.1, 0.33, 0.5, 0.8, 1.0):
        _, cnt = oracle.cdf_counts(S, N, tau, 0.7)
        assert np.all(cnt == math.ceil(round(tau * N, 9))), (tau, cnt)
    rng = np.random.default_rng(5)
    S = rng.standard_normal((20, 50)) * 3
    prev = np.zeros(20, np.int32)
    for tau in np.linspace(0.05, 1.0, 20):
        ids, cnt = oracle.cdf_counts(S, 50, tau, 0.5)
        assert np.all(cnt >= prev) and np.all((cnt >= 1) & (cnt <= 50))
        prev = cnt
        np.testing.assert_array_equal(ids, oracle.topk_select(S, 50))


def test_cdf_counts_brute_force_definition():
    """The count is the smallest n whose leading weights reach tau of the total,
    checked by direct summation over each candidate n."""
    rng = np.random.default_rng(8)
    S = rng.standard_normal((30, 12)) * 2
    for tau in (0.2, 0.6, 0.9, 0.999):
        ids, cnt = oracle.cdf_counts(S, 12, tau, 1.3)
        for r in range(S.shape[0]):
            w = [math.exp((S[r, j] - S[r].max()) * 1.3) for j in ids[r]]
            total = math.fsum(w)
            n = next(n for n in range(1, 13) if math.fsum(w[:n]) >= tau * total - 1e-12 * total)
            assert cnt[r] == n, (tau, r, cnt[r], n)


# ------------------------------------------------------ coarse output, combine

def _pool_matrix(vbs):
    """(Nc, Nc*64) matrix whose row c averages the real slots of cube c: an
    independent (matrix) form of the mean-pool."""
    Nc = vbs.size
    M = np.zeros((Nc, Nc * 64))
    for c in range(Nc):
        if vbs[c] > 0:
            M[c, 64 * c:64 * c + vbs[c]] = 1.0 / vbs[c]
    return M


def coarse_sdpa_error(coarse_fn=None):
    """Largest |coarse_fn - SDPA| on a ragged case with empty cubes: torch's
    fp64 scaled_dot_product_attention on means formed by a pooling matrix, the
    empty cubes masked out as keys."""
    coarse_fn = coarse_fn or oracle.coarse_output
    rng = np.random.default_rng(77)
    vbs = np.array([64, 0, 17, 5, 64, 1, 0, 40, 33], np.int32)
    B, NH, D = 2, 3, 16
    S = vbs.size * 64
    q, k, v = (rng.standard_normal((B, S, NH, D)) for _ in range(3))
    got = coarse_fn(q, k, v, vbs)
    M = torch.from_numpy(_pool_matrix(vbs))
    pool = lambda x: torch.einsum("cs,bshd->bhcd", M, torch.from_numpy(x))
    mask = torch.from_numpy(vbs > 0)[None, None, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(pool(q), pool(k), pool(v),
                                                           attn_mask=mask).numpy()
    return float(np.max(np.abs(got - ref)))


def test_coarse_output_equals_sdpa_on_pooled_cubes():
    """VSA blog, "Two-Stage Architecture": coarse attention over mean-pooled
    cubes, against an independent formulation (pooling matrix + library SDPA)."""
    assert coarse_sdpa_error() < 1e-13
    vbs = np.array([64, 0, 17, 5], np.int32)
    q, k, v = (_randn(1, 4 * 64, 2, 8) for _ in range(3))
    # the scale is 1/sqrt(D) by default; an explicit scale is honoured
    got2 = oracle.coarse_output(q, k, v, vbs, sm_scale=0.3)
    M = torch.from_numpy(_pool_matrix(vbs))
    pool = lambda x: torch.einsum("cs,bshd->bhcd", M, torch.from_numpy(x))
    mask = torch.from_numpy(vbs > 0)[None, None, None, :]
    ref2 = torch.nn.functional.scaled_dot_product_attention(pool(q), pool(k), pool(v),
                                                            attn_mask=mask, scale=0.3).numpy()
    assert np.allclose(got2, ref2, rtol=1e-12, atol=1e-13)


def test_coarse_output_closed_forms():
    """q = 0: every score is 0, so each row is the plain average of the real
    cubes' mean v. One key cube far ahead of the rest: each row is that cube's
    mean v. Padding slots never matter."""
    vbs = np.array([64, 3, 0, 20, 64], np.int32)
    D = 8
    S = vbs.size * 64
    v = _randn(1, S, 1, D)
    k = _randn(1, S, 1, D)
    means = np.stack([v[0, 64 * c:64 * c + vbs[c], 0].mean(axis=0) for c in (0, 1, 3, 4)])
    got = oracle.coarse_output(np.zeros((1, S, 1, D)), k, v, vbs)
    assert np.allclose(got[0, 0], means.mean(axis=0)[None, :], rtol=0, atol=1e-14)

    u = np.ones(D)
    q = np.tile(u, (1, S, 1, 1))
    k = np.zeros((1, S, 1, D))
    k[0, 64 * 3:64 * 3 + 20, 0] = 40.0 * u            # cube 3 dominates: score 40 D
    got = oracle.coarse_output(q, k, v, vbs)
    real = vbs > 0
    assert np.allclose(got[0, 0][real], means[2][None, :], rtol=0, atol=1e-12)
    # the empty query cube pools to 0, so its row is again the plain average
    assert np.allclose(got[0, 0][~real], means.mean(axis=0)[None, :], rtol=0, atol=1e-14)

    poisoned = v.copy()
    for c in range(vbs.size):
        poisoned[0, 64 * c + vbs[c]:64 * (c + 1)] = 1e30
    q = _randn(1, S, 1, D)
    assert np.array_equal(oracle.coarse_output(q, k, v, vbs), oracle.coarse_output(q, k, poisoned, vbs))


def test_coarse_output_no_real_key_cube_is_zero():
    vbs = np.zeros(3, np.int32)
    x = _randn(1, 3 * 64, 2, 4)
    assert np.array_equal(oracle.coarse_output(x, x, x, vbs), np.zeros((1, 2, 3, 4)))


def combine_pin(combine_fn) -> bool:
    """VSA blog, "Two-Stage Architecture": out = g_c * Oc + g_f * O_fine with
    the coarse row broadcast to its cube's 64 rows; checked element by element,
    and gates (1, 0) / (0, 1) give the branches themselves."""
    rng = np.random.default_rng(21)
    B, Nc, NH, D = 2, 3, 2, 4
    S = Nc * 64
    of, gc, gf = (rng.standard_normal((B, S, NH, D)) for _ in range(3))
    oc = rng.standard_normal((B, NH, Nc, D))
    got = combine_fn(of, oc, gc, gf)
    for b in range(B):
        for s in range(0, S, 7):
            for h in range(NH):
                for d in range(D):
                    want = gc[b, s, h, d] * oc[b, h, s // 64, d] + gf[b, s, h, d] * of[b, s, h, d]
                    if got[b, s, h, d] != want:
                        return False
    one, zero = np.ones_like(of), np.zeros_like(of)
    if not np.array_equal(combine_fn(of, oc, zero, one), of):
        return False
    bc = combine_fn(of, oc, one, zero)
    return all(np.array_equal(bc[:, s], oc[:, :, s // 64]) for s in range(S))


def test_gated_combine_brute_force_and_special_gates():
    assert combine_pin(oracle.gated_combine)


# --------------------------------------------- cube order (SFC), mask -> LUT

def hilbert_pin(index_fn, bits) -> bool:
    """Defining properties of the 3D Hilbert curve on a 2^b box: the indices are
    a permutation of [0, 8^b); the path starts at the origin; consecutive cells
    are face neighbours; every aligned 2^k sub-box is visited contiguously."""
    n = 1 << bits
    cells = [(x, y, z) for x in range(n) for y in range(n) for z in range(n)]
    idx = [index_fn(*c, bits) for c in cells]
    if sorted(idx) != list(range(n ** 3)):
        return False
    path = [cells[i] for i in np.argsort(idx)]
    if path[0] != (0, 0, 0):
        return False
    steps = np.abs(np.diff(np.asarray(path), axis=0)).sum(axis=1)
    if not np.all(steps == 1):
        return False
    for k in range(1, bits):
        blocks = [tuple(v >> k for v in c) for c in path]
        runs = [b for i, b in enumerate(blocks) if i == 0 or b != blocks[i - 1]]
        if not len(runs) == len(set(runs)) == (n >> k) ** 3:
            return False
    return True


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_hilbert_box_order_is_a_unit_step_hierarchical_path(bits):
    assert hilbert_pin(oracle.hilbert_index_3d, bits)


def test_cube_order_restricts_the_box_curve():
    """On a non-power-of-two grid the order is the box curve's order with the
    cells outside the grid skipped; a permutation; row_major is the identity."""
    Nt, Nh, Nw = 6, 8, 13                     # the Wan grid 21x30x52
    order = oracle.cube_order(21, 30, 52)
    assert np.array_equal(np.sort(order), np.arange(Nt * Nh * Nw))
    n = 16
    box = [(t, h, w) for t in range(n) for h in range(n) for w in range(n)]
    walk = [box[i] for i in np.argsort([oracle.hilbert_index_3d(*c, 4) for c in box])]
    inside = [(t * Nh + h) * Nw + w for t, h, w in walk if t < Nt and h < Nh and w < Nw]
    assert np.array_equal(order, inside)
    assert np.array_equal(oracle.cube_order(21, 30, 52, "row_major"), np.arange(624))
    # locality: the mean step between consecutive cubes is close to 1
    xyz = np.stack([order // (Nh * Nw), (order // Nw) % Nh, order % Nw], axis=1)
    assert np.abs(np.diff(xyz, axis=0)).sum(axis=1).mean() < 1.1


def test_tile_with_order_permutes_whole_cubes_and_roundtrips():
    rng = np.random.default_rng(3)
    T, H, W = 9, 5, 6
    x = rng.integers(0, 65535, size=(2, T * H * W, 2, 4), dtype=np.uint16)
    order = oracle.cube_order(T, H, W)
    plain, vbs = oracle.tile(x, T, H, W)
    xt, vbs_o = oracle.tile(x, T, H, W, order)
    for p, c in enumerate(order):
        assert np.array_equal(xt[:, 64 * p:64 * (p + 1)], plain[:, 64 * c:64 * (c + 1)])
        assert vbs_o[p] == vbs[c]
    assert np.array_equal(oracle.untile(xt, T, H, W, order), x)


def mask_lut_pin(fn=None) -> bool:
    """Brute force over a random mask with an empty and a full row: each row's
    ids are its set cells in ascending order and give the mask back; with a
    cap of 4 the counts, the truncated-row tally and the kept (lowest) ids."""
    fn = fn or oracle.mask_to_lut
    rng = np.random.default_rng(11)
    M = rng.random((2, 3, 7, 19)) < 0.3
    M[0, 0, 0] = False                           # an empty row
    M[1, 2, 6] = True                            # a full row
    ids, cnt, trunc = fn(M, 19)
    ok = trunc == 0
    for r in np.ndindex(2, 3, 7):
        want = [j for j in range(19) if M[r][j]]
        ok &= bool(cnt[r] == len(want) and list(ids[r][:cnt[r]]) == want)
        back = np.zeros(19, bool)
        back[ids[r][:cnt[r]]] = True
        ok &= bool(np.array_equal(back, M[r]))
    ids4, cnt4, trunc4 = fn(M, 4)
    ok &= trunc4 == int((M.sum(axis=-1) > 4).sum())
    ok &= bool(np.array_equal(cnt4, np.minimum(M.sum(axis=-1), 4)))
    for r in np.ndindex(2, 3, 7):
        ok &= list(ids4[r][:cnt4[r]]) == [j for j in range(19) if M[r][j]][:4]
    return bool(ok)


def test_mask_to_lut_brute_force_and_roundtrip():
    assert mask_lut_pin()


def test_mask_lut_drives_fwd_lut_like_the_dense_mask():
    """A block mask turned into the LUT gives, through fwd_lut, the brute-force
    dense attention under that block mask (and the real-token mask)."""
    rng = np.random.default_rng(12)
    q, kk, v, vbs = _tiled_case(9, 5, 6, NH=2, D=8, B=1, rng=rng)
    Nc = vbs.size
    M = rng.random((1, 2, Nc, Nc)) < 0.35
    M[..., 0] = True                             # every row attends cube 0 (64 real tokens)
    ids, cnt, _ = oracle.mask_to_lut(M, Nc)
    out, _, _ = oracle.fwd_lut(q, kk, v, np.maximum(ids, 0), cnt, vbs)
    S = Nc * 64
    cube_of, slot_of = np.arange(S) // 64, np.arange(S) % 64
    scale = 1 / math.sqrt(8)
    for h in range(2):
        tok = M[0, h][cube_of][:, cube_of] & (slot_of < vbs[cube_of])[None, :]
        s = np.where(tok, q[0, :, h] @ kk[0, :, h].T * scale, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = p @ v[0, :, h] / p.sum(axis=1, keepdims=True)
        np.testing.assert_allclose(out[0, :, h], ref, rtol=0, atol=1e-12)
