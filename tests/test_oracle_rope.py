"""Pins of the QK-norm + RoPE + append oracle (oracle/rope.py) to facts that do not come from the
oracle itself: rotation by a hand-computed angle, complex multiplication, the group and
relative-position properties of rotations, the two pairings being one permutation apart, the RMS of
a normalised row, hand-computed bf16 roundings, and the append's slot arithmetic on a tiny pool."""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import rope as R


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_position_zero_is_identity():
    x = _rand((3, 64), 1)
    for inter in (False, True):
        np.testing.assert_array_equal(R.rope(x, 0, 10000.0, 64, inter), x)


def test_first_pair_turns_by_position_radians():
    """Pair 0 has frequency 1: at position t, e_0 turns to (cos t, sin t) — counter-clockwise from
    the first element of the pair towards the second."""
    D = 16
    for inter, second in ((False, 8), (True, 1)):
        e0 = np.zeros(D)
        e0[0] = 1.0
        y = R.rope(e0, 3, 10000.0, D, inter)
        assert y[0] == pytest.approx(-0.9899924966004454, abs=1e-15)   # cos 3
        assert y[second] == pytest.approx(0.1411200080598672, abs=1e-15)  # sin 3
        assert np.count_nonzero(y) == 2


def test_pair_frequency_hand_value():
    """theta 10000, 128 rotated dims: pair 32 turns 10000^(-64/128) = 0.01 rad per position; with
    the exponent spaced over 512 dims (a partial rotation of a 512-wide head) it turns
    10000^(-64/512) = 10^(-1/2) rad per position."""
    x = np.zeros(128)
    x[32] = 1.0
    y = R.rope(x, 5, 10000.0, 128, False)
    assert y[32] == pytest.approx(math.cos(0.05), abs=1e-14)
    assert y[96] == pytest.approx(math.sin(0.05), abs=1e-14)
    y = R.rope(x, 1, 10000.0, 128, False, freq_dim=512)
    assert y[32] == pytest.approx(math.cos(0.31622776601683794), abs=1e-14)
    assert y[96] == pytest.approx(math.sin(0.31622776601683794), abs=1e-14)


def test_neox_equals_complex_multiplication():
    """NeoX pairing: z_j = x_j + i x_{j+R/2} is multiplied by exp(i t f_j)."""
    D, Rd = 96, 64
    x = _rand(D, 2)
    t, theta = 1234, 500000.0
    f = np.array([theta ** (-2.0 * j / Rd) for j in range(Rd // 2)])
    z = (x[:Rd // 2] + 1j * x[Rd // 2:Rd]) * np.exp(1j * t * f)
    y = R.rope(x, t, theta, Rd, False)
    np.testing.assert_allclose(y[:Rd // 2], z.real, atol=1e-12)
    np.testing.assert_allclose(y[Rd // 2:Rd], z.imag, atol=1e-12)
    np.testing.assert_array_equal(y[Rd:], x[Rd:])  # partial rotation leaves the tail


def test_interleaved_is_neox_under_the_pair_permutation():
    D = 64
    x = _rand((5, D), 3)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])  # interleaved -> halves
    pos = np.arange(5) * 37
    a = R.rope(x, pos, 10000.0, D, True)
    b = R.rope(x[:, perm], pos, 10000.0, D, False)
    np.testing.assert_allclose(a[:, perm], b, atol=1e-12)


@pytest.mark.parametrize("inter", [False, True])
def test_rotation_properties(inter):
    """Pair norms are kept; rotating by m then n equals rotating by m + n; scores of rotated q and
    k depend only on the position difference."""
    D = 32
    q, k = _rand(D, 4), _rand(D, 5)
    th = 10000.0
    y = R.rope(q, 77, th, D, inter)
    pairs = (lambda v: np.hypot(v[0:D:2], v[1:D:2])) if inter else (
        lambda v: np.hypot(v[:D // 2], v[D // 2:]))
    np.testing.assert_allclose(pairs(y), pairs(q), rtol=1e-12)
    np.testing.assert_allclose(R.rope(R.rope(q, 40, th, D, inter), 37, th, D, inter), y,
                               atol=1e-12)
    s1 = R.rope(q, 1000, th, D, inter) @ R.rope(k, 990, th, D, inter)
    s2 = R.rope(q, 70000, th, D, inter) @ R.rope(k, 69990, th, D, inter)
    assert s1 == pytest.approx(s2, abs=1e-9)


def test_rms_norm_hand_values():
    y = R.rms_norm(np.array([3.0, 4.0]), None, 0.0)  # mean square 12.5
    np.testing.assert_allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=1e-15)
    y = R.rms_norm(np.array([1.0, -1.0, 1.0, -1.0]), np.array([2.0, 1.0, 0.5, 0.0]), 1.0)
    np.testing.assert_allclose(y, np.array([2.0, -1.0, 0.5, 0.0]) / math.sqrt(2.0), rtol=1e-15)


def test_rms_norm_unit_rms_and_scale_invariance():
    x = _rand((4, 256), 6)
    y = R.rms_norm(x, None, 1e-6)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-5)
    y0 = R.rms_norm(x, None, 0.0)
    np.testing.assert_allclose(R.rms_norm(1000.0 * x, None, 0.0), y0, rtol=1e-12)
    np.testing.assert_allclose(y, y0, rtol=1e-5)  # eps only matters for tiny rows


def test_bf16_rounding_hand_values():
    vals = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                     0.0])
    bits = R._f64_to_bf16(vals)
    # exact; tie to even (down); tie to even (up); exact negative; just above a tie (up); zero
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F81, 0x0000]
    np.testing.assert_array_equal(R._bf16_to_f64(np.array([0x3F80, 0xC020], np.uint16)),
                                  [1.0, -2.5])


def _bits(x):
    return R._f64_to_bf16(np.asarray(x, dtype=np.float64))


def test_prepare_and_append_slots_and_skips():
    """Tiny pool by hand: pages of 4 slots, two sequences with two new tokens each; the second
    sequence's first token is at position -1 (skipped) and a token past max_position is skipped
    (q row untouched); values pass bitwise without a v norm; one pool given twice takes k only."""
    B, L, Hq, Hkv, D, S, P = 3, 2, 2, 1, 8, 4, 6
    rng = np.random.default_rng(7)
    q = _bits(rng.standard_normal((B, L, Hq, D)))
    k = _bits(rng.standard_normal((B, L, Hkv, D)))
    v = _bits(rng.standard_normal((B, L, Hkv, D)))
    bt = np.array([[2, 5], [4, 1], [3, 0]], dtype=np.int32)
    ctx = np.array([6, 1, 12], dtype=np.int32)  # positions [4, 5], [-1, 0], [10, 11]
    kp = np.zeros((P, Hkv, S, D), np.uint16)
    vp = np.zeros((P, Hkv, S, D), np.uint16)
    qb = R.prepare_and_append(q, k, v, kp, vp, bt, ctx, 11, False, False, None, None, None, 1e-6,
                              10000.0, D, False)
    # seq 0: positions 4, 5 -> page bt[0,1] = 5, slots 0, 1
    kr = R.rope(R._bf16_to_f64(k[0, :, 0]), np.array([4, 5]), 10000.0, D, False)
    np.testing.assert_array_equal(kp[5, 0, 0], _bits(kr[0]))
    np.testing.assert_array_equal(kp[5, 0, 1], _bits(kr[1]))
    np.testing.assert_array_equal(vp[5, 0, :2], v[0, :, 0])
    # seq 1: token 0 at -1 skipped (q row kept); token 1 at position 0 -> page 4 slot 0, unrotated
    np.testing.assert_array_equal(qb[1, 0], q[1, 0])
    np.testing.assert_array_equal(qb[1, 1], q[1, 1])
    np.testing.assert_array_equal(kp[4, 0, 0], k[1, 1, 0])
    # seq 2: position 10 -> column 2, past the 2-column table row: q rotated, nothing written;
    # position 11 >= max_position: q row kept
    assert not np.array_equal(qb[2, 0], q[2, 0])
    np.testing.assert_array_equal(qb[2, 1], q[2, 1])
    written = {(5, 0), (5, 1), (4, 0)}
    for p in range(P):
        for s in range(S):
            if (p, s) not in written:
                assert not kp[p, 0, s].any() and not vp[p, 0, s].any()
    # one pool for both: the k row goes in, the value row is not written
    kp2 = np.zeros_like(kp)
    R.prepare_and_append(q, k, None, kp2, kp2, bt, ctx, 11, False, False, None, None, None, 1e-6,
                         10000.0, D, False)
    np.testing.assert_array_equal(kp2, kp)


def test_prepare_norm_then_rotate():
    """With norm_qk, k is normalised (unit RMS, times the weight) and then rotated; norm_v
    normalises v without rotating it."""
    rng = np.random.default_rng(8)
    D = 16
    q = _bits(rng.standard_normal((1, 1, 2, D)) * 3)
    k = _bits(rng.standard_normal((1, 1, 1, D)) * 3)
    v = _bits(rng.standard_normal((1, 1, 1, D)) * 3)
    w = rng.uniform(0.5, 1.5, D)
    qo, ko, vo = R.prepare(q, k, v, np.array([9]), True, True, None, w, w, 1e-6, 10000.0, D, True)
    k64 = R._bf16_to_f64(k[0, 0, 0])
    kn = k64 / math.sqrt(np.mean(k64 ** 2) + 1e-6) * w
    np.testing.assert_allclose(ko[0, 0, 0], R.rope(kn, 8, 10000.0, D, True), rtol=1e-12)
    v64 = R._bf16_to_f64(v[0, 0, 0])
    np.testing.assert_allclose(vo[0, 0, 0], v64 / math.sqrt(np.mean(v64 ** 2) + 1e-6) * w,
                               rtol=1e-12)
    # q with a unit scale: each head has RMS ~1 after the norm, and rotation keeps it
    np.testing.assert_allclose(np.sqrt(np.mean(qo[0, 0] ** 2, axis=-1)), 1.0, rtol=1e-5)
