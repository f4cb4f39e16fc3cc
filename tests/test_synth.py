"""Seeded generators: determinism, shapes and the structure they promise."""
import math

import numpy as np

import oracle
import synth


def test_tiny_deterministic_and_shaped():
    a, b = synth.tiny(), synth.tiny()
    assert a.q.shape == (1, 210, 2, 64) and a.q.dtype == np.uint16
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        np.testing.assert_array_equal(x, y)
    assert not np.array_equal(a.q, a.k)


def test_seed_changes_draws():
    cfg = dict(synth.CONFIGS["tiny"])
    cfg["seed"] = 7
    c = synth.make_case("tiny7", **cfg)
    assert not np.array_equal(c.q, synth.tiny().q)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, 3.0e38], np.float32)
    np.testing.assert_array_equal(synth.bf16_bits_from_f32(x),
                                  np.array([0x3F80, 0x3F82, 0xC020, 0x7F62], np.uint16))


def test_outlier_head_reaches_2000():
    """A reduced grid with the Wan recipe: the outlier head's logits reach
    about +-2000 and the other heads stay far below."""
    c = synth.make_case("mini", B=1, T=8, H=8, W=12, NH=4, D=128, topk=4, seed=3,
                        qk="field", heavy=True, outlier=True)
    assert 0 <= c.outlier_head < 4
    q = oracle.decode_bf16(c.q)[0]
    k = oracle.decode_bf16(c.k)[0]
    peak = [np.abs(q[:, h] @ k[:, h].T).max() / math.sqrt(128) for h in range(4)]
    assert 1500 < peak[c.outlier_head] < 2600
    assert peak[c.outlier_head] > math.log(np.finfo(np.float32).max)  # one-pass exp overflows


def test_field_gives_spatially_local_scores():
    """q and k of a head share a smooth field: a query cube scores its own
    neighbourhood above the median cube (what makes the selection local)."""
    c = synth.make_case("mini", B=1, T=8, H=8, W=8, NH=2, D=128, topk=4, seed=5,
                        qk="field", heavy=False, outlier=False)
    qt, vbs = oracle.tile(oracle.decode_bf16(c.q), 8, 8, 8)
    kt, _ = oracle.tile(oracle.decode_bf16(c.k), 8, 8, 8)
    S = oracle.cube_scores(oracle.mean_pool(qt, vbs), oracle.mean_pool(kt, vbs))
    diag = np.einsum("hii->hi", S[0])
    assert np.mean(diag > np.median(S[0], axis=-1)) > 0.9
