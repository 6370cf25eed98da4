"""Pins of the fp64 CPU oracle against facts fixed by the mathematics of decode attention.

The pages print no worked example, so each test below checks the oracle against something other
than its own formula: closed forms (one key, identical keys, scale 0, two keys, window bounds with
counting values), invariances (physical-page permutation, score shift, GQA vs replicated MHA,
sliding = global over the truncated context), the split/merge identity, and brute force against an
independently written numpy twin on tiny shapes. Each is chosen so that a plausible slip in the
oracle (a wrong head mapping, page/slot swap, off-by-one window, sign error, missing max or lse
term) fails at least one of them. CPU only.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import twin
from paged_gqa_kv_attn_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits, make_layer_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    """bf16 bits of values that are exactly representable in bf16 (asserted)."""
    x = np.asarray(x, dtype=np.float32)
    bits = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(bits), x), "test value not exact in bf16"
    return bits


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def paged(keys, values, S, rng=None, spare=3):
    """Pools and block table for per-sequence logical arrays keys[b]/values[b] of shape
    [n_b, Hkv, D] (bf16 bits). Pages are placed at random physical ids when rng is given."""
    B = len(keys)
    Hkv, D = keys[0].shape[1], keys[0].shape[2]
    npages = [(k.shape[0] + S - 1) // S for k in keys]
    total = sum(npages) + spare
    ids = np.arange(total) if rng is None else rng.permutation(total)
    width = max(1, max(npages))
    table = np.full((B, width), -1, dtype=np.int32)
    kp = np.full((total, Hkv, S, D), 0x7FC0, dtype=np.uint16)
    vp = np.full((total, Hkv, S, D), 0x7FC0, dtype=np.uint16)
    c = 0
    for b in range(B):
        n = keys[b].shape[0]
        for j in range(npages[b]):
            p = int(ids[c])
            c += 1
            table[b, j] = p
            seg = slice(j * S, min(n, (j + 1) * S))
            cnt = seg.stop - seg.start
            kp[p, :, :cnt] = np.transpose(keys[b][seg], (1, 0, 2))
            vp[p, :, :cnt] = np.transpose(values[b][seg], (1, 0, 2))
    return kp, vp, table


def rand_bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits(np.float32(scale) * rng.standard_normal(shape, dtype=np.float32))


# ----------------------------------------------------------------------------- closed forms


def test_single_key_returns_its_value():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, D, S = 2, 4, 2, 16, 16
    keys = [rand_bits(rng, (1, Hkv, D)) for _ in range(B)]
    vals = [rand_bits(rng, (1, Hkv, D)) for _ in range(B)]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (B, Hq, D))
    out, lse = oracle.decode_attn(q, kp, vp, table, [1, 1], 0.25)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            assert np.array_equal(out[b, h], f64(vals[b][0, g]))  # exp(0)/exp(0) = 1 exactly
            s = 0.25 * float(np.dot(f64(q[b, h]), f64(keys[b][0, g])))
            assert lse[b, h] == pytest.approx(s, rel=1e-15, abs=1e-15)


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    Hq, Hkv, D, S, n = 2, 1, 8, 16, 37
    k1 = rand_bits(rng, (1, Hkv, D))
    keys = [np.repeat(k1, n, axis=0)]
    vals = [rand_bits(rng, (n, Hkv, D))]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (1, Hq, D))
    scale = 0.7
    out, lse = oracle.decode_attn(q, kp, vp, table, [n], scale)
    mean_v = f64(vals[0][:, 0]).mean(axis=0)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], mean_v, rtol=0, atol=1e-12)
        s = scale * float(np.dot(f64(q[0, h]), f64(k1[0, 0])))
        assert lse[0, h] == pytest.approx(s + math.log(n), abs=1e-12)


def test_scale_zero_gives_mean_of_values_and_log_count():
    rng = np.random.default_rng(3)
    Hq, Hkv, D, S, n = 4, 2, 8, 16, 50
    keys = [rand_bits(rng, (n, Hkv, D))]
    vals = [rand_bits(rng, (n, Hkv, D))]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (1, Hq, D))
    out, lse = oracle.decode_attn(q, kp, vp, table, [n], 0.0)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], f64(vals[0][:, h // 2]).mean(axis=0), atol=1e-12)
        assert lse[0, h] == pytest.approx(math.log(n), abs=1e-14)


@pytest.mark.parametrize("a,b,scale", [(0.0, 1.0, 1.0), (2.0, -1.5, 0.5), (-3.0, 4.0, 0.125)])
def test_two_keys_closed_form(a, b, scale):
    """q = e0, K_0[0] = a, K_1[0] = b: s = scale*(a, b); weights are a logistic pair."""
    D, S = 4, 16
    q = bf(np.array([[[1, 0, 0, 0]]], dtype=np.float32))
    keys = [bf(np.array([[[a, 5, -7, 9]], [[b, 3, 1, -2]]], dtype=np.float32))]
    v0, v1 = np.array([1.0, -2.0, 0.5, 8.0]), np.array([-4.0, 3.0, 0.25, 16.0])
    vals = [bf(np.stack([v0, v1])[:, None, :])]
    kp, vp, table = paged(keys, vals, S)
    out, lse = oracle.decode_attn(q, kp, vp, table, [2], scale)
    w1 = 1.0 / (1.0 + math.exp(scale * (a - b)))  # weight of key 1
    np.testing.assert_allclose(out[0, 0], (1 - w1) * v0 + w1 * v1, rtol=0, atol=1e-14)
    expect_lse = math.log(math.exp(scale * a) + math.exp(scale * b))
    assert lse[0, 0] == pytest.approx(expect_lse, abs=1e-14)


def test_dominant_key_wins_without_overflow():
    """Scores near 1e4: exp without the max shift would overflow; the output is the top key's V."""
    D, S, n = 4, 16, 20
    rng = np.random.default_rng(4)
    k = np.zeros((n, 1, D), dtype=np.float32)
    k[:, 0, 0] = np.arange(n, dtype=np.float32) * 64.0  # s_t = 64 t * 8
    k[7, 0, 0] = 2048.0                                 # key 7 dominates: s = 16384
    keys = [bf(k)]
    vals = [rand_bits(rng, (n, 1, D))]
    kp, vp, table = paged(keys, vals, S, rng)
    q = bf(np.array([[[8, 0, 0, 0]]], dtype=np.float32))
    out, lse = oracle.decode_attn(q, kp, vp, table, [n], 1.0)
    assert np.all(np.isfinite(out))
    np.testing.assert_allclose(out[0, 0], f64(vals[0][7, 0]), atol=1e-12)
    assert lse[0, 0] == pytest.approx(16384.0, abs=1e-9)


def _count_values(n_max, D=4):
    """V_t = (t % 16, t // 16, 1, -t % 7): small integers, exact in bf16."""
    t = np.arange(n_max)
    v = np.zeros((n_max, 1, D), dtype=np.float32)
    v[:, 0, 0] = t % 16
    v[:, 0, 1] = t // 16
    v[:, 0, 2] = 1
    v[:, 0, 3] = -(t % 7)
    return v


@pytest.mark.parametrize("window", [0, 1, 15, 16, 17, 31, 32, 33, 1024])
def test_window_bounds_with_counting_values(window):
    """scale 0: out = mean of V over exactly the attended keys; V_t encodes t, so the mean pins
    both ends of the range [max(0, n - W), n) for every n % 32 alignment."""
    S, D = 16, 4
    rng = np.random.default_rng(5)
    for n in range(1, 81):
        v = _count_values(n, D)
        keys = [rand_bits(rng, (n, 1, D))]
        kp, vp, table = paged(keys, [bf(v)], S, rng)
        q = rand_bits(rng, (1, 1, D))
        out, lse = oracle.decode_attn(q, kp, vp, table, [n], 0.0, window=window)
        lo = max(0, n - window) if window else 0
        t = np.arange(lo, n)
        expect = np.array([np.mean(t % 16), np.mean(t // 16), 1.0, -np.mean(t % 7)])
        np.testing.assert_allclose(out[0, 0], expect, atol=1e-12, err_msg="n=%d W=%d" % (n, window))
        assert lse[0, 0] == pytest.approx(math.log(n - lo), abs=1e-13)


def test_window_one_returns_last_value():
    rng = np.random.default_rng(6)
    S, D, Hq, Hkv = 16, 8, 4, 2
    ns = [1, 16, 17, 45]
    keys = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    vals = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (len(ns), Hq, D))
    out, _ = oracle.decode_attn(q, kp, vp, table, ns, 0.3, window=1)
    for b, n in enumerate(ns):
        for h in range(Hq):
            assert np.array_equal(out[b, h], f64(vals[b][n - 1, h // 2]))


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_head_mapping_closed_form(G):
    """V of KV head g is the constant g + 1, so out[b, h, :] = h // G + 1 exactly: query heads map
    to KV heads in contiguous groups."""
    rng = np.random.default_rng(7)
    Hkv, D, S, n = 3, 8, 16, 21
    Hq = G * Hkv
    keys = [rand_bits(rng, (n, Hkv, D))]
    v = np.broadcast_to(np.arange(1, Hkv + 1, dtype=np.float32)[None, :, None], (n, Hkv, D))
    kp, vp, table = paged(keys, [bf(v)], S, rng)
    q = rand_bits(rng, (1, Hq, D))
    out, _ = oracle.decode_attn(q, kp, vp, table, [n], 0.4)
    for h in range(Hq):
        np.testing.assert_allclose(out[0, h], np.full(D, h // G + 1.0), rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------- invariances


def test_gqa_equals_replicated_mha():
    rng = np.random.default_rng(8)
    B, Hkv, G, D, S = 2, 2, 4, 16, 16
    Hq = Hkv * G
    ns = [33, 50]
    keys = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    vals = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    q = rand_bits(rng, (B, Hq, D))
    kp, vp, table = paged(keys, vals, S, rng)
    out, lse = oracle.decode_attn(q, kp, vp, table, ns, 0.2)
    rep = lambda a: np.repeat(a, G, axis=1)  # KV head g -> query heads g*G .. g*G+G-1
    kp2, vp2, table2 = paged([rep(k) for k in keys], [rep(v) for v in vals], S, rng)
    out2, lse2 = oracle.decode_attn(q, kp2, vp2, table2, ns, 0.2)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_page_permutation_invariance_is_bitwise():
    inp = make_layer_inputs([100, 37, 64], 8, 2, 32, page_size=16, seed=9)
    out, lse = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                                  inp.scale)
    rng = np.random.default_rng(10)
    P = inp.k_pool.shape[0]
    perm = rng.permutation(P)            # new id of old page p is perm[p]
    kp2 = np.empty_like(inp.k_pool)
    vp2 = np.empty_like(inp.v_pool)
    kp2[perm] = inp.k_pool
    vp2[perm] = inp.v_pool
    table2 = np.where(inp.block_table >= 0, perm[np.maximum(inp.block_table, 0)], -1)
    out2, lse2 = oracle.decode_attn(inp.q, kp2, vp2, table2, inp.ctx_lens, inp.scale)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_score_shift_invariance():
    """An extra dimension with q = c and every K = 1 adds scale*c to all scores: out unchanged,
    lse shifted by scale*c."""
    rng = np.random.default_rng(11)
    D, S, n, Hkv, Hq = 8, 16, 40, 1, 2
    keys = rand_bits(rng, (n, Hkv, D))
    vals = rand_bits(rng, (n, Hkv, D))
    q = rand_bits(rng, (1, Hq, D))
    kp, vp, table = paged([keys], [vals], S)
    out, lse = oracle.decode_attn(q, kp, vp, table, [n], 0.5)
    ext = lambda a, val: np.concatenate([a, np.full(a.shape[:-1] + (1,), val, np.uint16)], -1)
    c = 6.0
    q2 = ext(q, bf(np.float32(c)))
    k2 = ext(keys, bf(np.float32(1.0)))
    v2 = ext(vals, bf(np.float32(0.0)))
    kp2, vp2, table2 = paged([k2], [v2], S)
    out2, lse2 = oracle.decode_attn(q2, kp2, vp2, table2, [n], 0.5)
    np.testing.assert_allclose(out2[..., :D], out, atol=1e-12)
    np.testing.assert_allclose(lse2, lse + 0.5 * c, atol=1e-12)


def test_linearity_in_values():
    rng = np.random.default_rng(12)
    D, S, n = 8, 16, 29
    keys = rand_bits(rng, (n, 1, D))
    v1 = rng.integers(-8, 9, size=(n, 1, D)).astype(np.float32)
    v2 = rng.integers(-8, 9, size=(n, 1, D)).astype(np.float32)
    q = rand_bits(rng, (1, 1, D))
    res = []
    for v in (v1, v2, v1 + 2 * v2):
        kp, vp, table = paged([keys], [bf(v)], S)
        res.append(oracle.decode_attn(q, kp, vp, table, [n], 0.9)[0])
    np.testing.assert_allclose(res[2], res[0] + 2 * res[1], atol=1e-12)


@pytest.mark.parametrize("window", [1, 17, 32, 100])
def test_sliding_equals_global_over_truncated_context(window):
    """A sliding layer equals a global layer run on the last min(W, n) keys laid out afresh."""
    rng = np.random.default_rng(13)
    S, D, Hkv, Hq = 16, 16, 2, 4
    ns = [5, 31, 77, 130]
    keys = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    vals = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    q = rand_bits(rng, (len(ns), Hq, D))
    kp, vp, table = paged(keys, vals, S, rng)
    out, lse = oracle.decode_attn(q, kp, vp, table, ns, 0.3, window=window)
    lo = [max(0, n - window) for n in ns]
    kp2, vp2, table2 = paged([k[l:] for k, l in zip(keys, lo)], [v[l:] for v, l in zip(vals, lo)],
                             S, rng)
    out2, lse2 = oracle.decode_attn(q, kp2, vp2, table2, [n - l for n, l in zip(ns, lo)], 0.3)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_window_at_least_context_equals_global():
    inp = make_layer_inputs([40, 64, 65], 4, 2, 16, page_size=16, seed=14)
    g = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens, inp.scale)
    s = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens, inp.scale,
                           window=65)
    np.testing.assert_array_equal(g[0], s[0])
    np.testing.assert_array_equal(g[1], s[1])


# ----------------------------------------------------------------------------- sink + window views


@pytest.mark.parametrize("window,sink", [(1, 1), (16, 4), (17, 16), (32, 33), (5, 40)])
def test_sink_window_bounds_with_counting_values(window, sink):
    """scale 0: out = mean of V over exactly the attended keys [0, min(sink, n)) u [n - W, n);
    V_t encodes t, so the mean pins both ranges (and that overlapping keys count once)."""
    S, D = 16, 4
    rng = np.random.default_rng(15)
    for n in range(1, 81):
        v = _count_values(n, D)
        keys = [rand_bits(rng, (n, 1, D))]
        kp, vp, table = paged(keys, [bf(v)], S, rng)
        q = rand_bits(rng, (1, 1, D))
        out, lse = oracle.decode_attn_sink(q, kp, vp, table, [n], 0.0, window, sink)
        t = np.array(sorted(set(range(min(sink, n))) | set(range(max(0, n - window), n))))
        expect = np.array([np.mean(t % 16), np.mean(t // 16), 1.0, -np.mean(t % 7)])
        np.testing.assert_allclose(out[0, 0], expect, atol=1e-12,
                                   err_msg="n=%d W=%d sink=%d" % (n, window, sink))
        assert lse[0, 0] == pytest.approx(math.log(len(t)), abs=1e-13)


@pytest.mark.parametrize("seed", range(4))
def test_sink_window_equals_global_over_the_concatenated_view(seed):
    """Attention over [0, sink) u [n - W, n) equals global attention over a new cache holding
    exactly those keys, in order, on fresh pages: the view is a concatenation."""
    rng = np.random.default_rng(40 + seed)
    S, D, Hq, Hkv = 16, 32, 4, 2
    ns = [int(x) for x in rng.integers(1, 140, size=3)]
    window, sink = int(rng.integers(1, 60)), int(rng.integers(1, 40))
    keys = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    vals = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (len(ns), Hq, D))
    out, lse = oracle.decode_attn_sink(q, kp, vp, table, ns, 0.3, window, sink)
    kept = [sorted(set(range(min(sink, n))) | set(range(max(0, n - window), n))) for n in ns]
    kp2, vp2, table2 = paged([k[idx] for k, idx in zip(keys, kept)],
                             [v[idx] for v, idx in zip(vals, kept)], S, rng)
    out2, lse2 = oracle.decode_attn(q, kp2, vp2, table2, [len(i) for i in kept], 0.3)
    np.testing.assert_allclose(out, out2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=1e-12)


def test_sink_reduces_to_sliding_and_global():
    """sink 0 is the sliding layer; window 0, or sink + window covering the context, is global."""
    rng = np.random.default_rng(44)
    S, D, Hq, Hkv = 16, 16, 2, 1
    ns = [1, 31, 64, 99]
    keys = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    vals = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (len(ns), Hq, D))
    glob = oracle.decode_attn(q, kp, vp, table, ns, 0.2)
    slid = oracle.decode_attn(q, kp, vp, table, ns, 0.2, window=20)
    for got, want in ((oracle.decode_attn_sink(q, kp, vp, table, ns, 0.2, 20, 0), slid),
                      (oracle.decode_attn_sink(q, kp, vp, table, ns, 0.2, 0, 7), glob),
                      (oracle.decode_attn_sink(q, kp, vp, table, ns, 0.2, 20, 80), glob)):
        np.testing.assert_allclose(got[0], want[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(got[1], want[1], rtol=0, atol=1e-12)


def test_sink_pages_outside_the_view_are_never_read():
    """Pages holding no attended key may be invalid ids: they are not dereferenced."""
    rng = np.random.default_rng(45)
    S, D = 16, 8
    n, window, sink = 100, 20, 10
    keys = [rand_bits(rng, (n, 1, D))]
    vals = [rand_bits(rng, (n, 1, D))]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (1, 1, D))
    want = oracle.decode_attn_sink(q, kp, vp, table, [n], 0.5, window, sink)
    table[0, 1:5] = -1  # keys 16..79: neither sink nor window
    got = oracle.decode_attn_sink(q, kp, vp, table, [n], 0.5, window, sink)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


# ----------------------------------------------------------------------------- multi-token decode


@pytest.mark.parametrize("L,window,sink", [(2, 0, 0), (3, 0, 0), (4, 17, 0), (7, 16, 4),
                                           (5, 1, 0), (8, 33, 40)])
def test_multi_token_bounds_with_counting_values(L, window, sink):
    """scale 0: each query's output is the mean of V over exactly its key set, whose upper end
    moves with the query (t <= n - L + i) and whose window moves with it."""
    S, D = 16, 4
    rng = np.random.default_rng(60 + L)
    for n in range(1, 75):
        v = _count_values(n, D)
        kp, vp, table = paged([rand_bits(rng, (n, 1, D))], [bf(v)], S, rng)
        q = rand_bits(rng, (1, L, 1, D))
        out, lse = oracle.decode_attn_multi(q, kp, vp, table, [n], 0.0, window, sink)
        for i in range(L):
            p = n - L + i
            if p < 0:
                assert np.all(out[0, i, 0] == 0) and lse[0, i, 0] == -np.inf
                continue
            lo = max(0, p + 1 - window) if window else 0
            sk = min(sink, lo) if window else 0
            t = np.array(list(range(sk)) + list(range(lo, p + 1)))
            expect = np.array([np.mean(t % 16), np.mean(t // 16), 1.0, -np.mean(t % 7)])
            np.testing.assert_allclose(out[0, i, 0], expect, atol=1e-12,
                                       err_msg="n=%d L=%d i=%d" % (n, L, i))
            assert lse[0, i, 0] == pytest.approx(math.log(len(t)), abs=1e-13)


@pytest.mark.parametrize("G,L,window", [(1, 2, 0), (2, 4, 0), (4, 3, 9), (8, 2, 0), (2, 8, 20)])
def test_multi_token_equals_masked_sdpa(G, L, window):
    """Against torch's scaled_dot_product_attention in fp64 on the dense keys with an explicit
    causal (and window) mask: the prefill-style formulation of the same queries."""
    import torch
    rng = np.random.default_rng(70 + G + L)
    S, D, Hkv = 16, 32, 2
    Hq = G * Hkv
    ns = [L, 17, 50, 97]
    keys = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    vals = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (len(ns), L, Hq, D))
    scale = 0.2
    out, lse = oracle.decode_attn_multi(q, kp, vp, table, ns, scale, window)
    for b, n in enumerate(ns):
        qt = torch.from_numpy(f64(q[b])).permute(1, 0, 2)                    # [Hq, L, D]
        kt = torch.from_numpy(f64(keys[b])).permute(1, 0, 2).repeat_interleave(G, 0)
        vt = torch.from_numpy(f64(vals[b])).permute(1, 0, 2).repeat_interleave(G, 0)
        pos = torch.arange(n - L, n)[:, None]
        t = torch.arange(n)[None, :]
        mask = (t <= pos) & ((t > pos - window) if window else True)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                               scale=scale)
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        s = scale * (qt @ kt.transpose(1, 2))
        ref_lse = torch.logsumexp(s.masked_fill(~mask, -np.inf), dim=-1).T.numpy()
        np.testing.assert_allclose(lse[b], ref_lse, rtol=0, atol=1e-12)


def test_multi_token_one_query_is_single_token_decode():
    rng = np.random.default_rng(80)
    S, D, Hq, Hkv = 16, 16, 4, 2
    ns = [1, 31, 64, 99]
    keys = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    vals = [rand_bits(rng, (n, Hkv, D)) for n in ns]
    kp, vp, table = paged(keys, vals, S, rng)
    q = rand_bits(rng, (len(ns), 1, Hq, D))
    for window, sink in ((0, 0), (20, 0), (20, 6)):
        got = oracle.decode_attn_multi(q, kp, vp, table, ns, 0.3, window, sink)
        want = oracle.decode_attn_sink(q[:, 0], kp, vp, table, ns, 0.3, window, sink)
        assert np.array_equal(got[0][:, 0], want[0]) and np.array_equal(got[1][:, 0], want[1])


def test_empty_context_gives_zero_and_minus_inf():
    inp = make_layer_inputs([0, 3], 2, 1, 16, page_size=16, seed=15)
    out, lse = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                                  inp.scale)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


def test_out_of_range_page_is_an_error():
    inp = make_layer_inputs([20], 2, 1, 16, page_size=16, seed=16)
    table = inp.block_table.copy()
    table[0, 1] = inp.k_pool.shape[0]
    with pytest.raises(ValueError):
        oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, table, inp.ctx_lens, inp.scale)


# ----------------------------------------------------------------------------- split / merge


def test_merge_two_parts_closed_form():
    o = np.array([[[1.0, 2.0], [3.0, -1.0]]])
    a, b = 0.3, -1.2
    out, lse = oracle.lse_merge(o, np.array([[a, b]]))
    wa, wb = math.exp(a), math.exp(b)
    np.testing.assert_allclose(out[0], (wa * o[0, 0] + wb * o[0, 1]) / (wa + wb), atol=1e-15)
    assert lse[0] == pytest.approx(math.log(wa + wb), abs=1e-15)


def test_merge_of_empty_parts():
    o = np.zeros((2, 3, 4))
    l = np.array([[-np.inf] * 3, [-np.inf, 0.5, -np.inf]])
    o[1, 1] = [1, 2, 3, 4]
    out, lse = oracle.lse_merge(o, l)
    assert np.all(out[0] == 0) and np.isneginf(lse[0])
    np.testing.assert_array_equal(out[1], [1, 2, 3, 4])
    assert lse[1] == 0.5


@pytest.mark.parametrize("seed", range(6))
def test_split_then_merge_equals_unsplit(seed):
    """Softmax over a union of disjoint key ranges is the LSE-weighted mix of the per-range
    softmaxes, for any chunking (empty chunks included)."""
    rng = np.random.default_rng(100 + seed)
    inp = make_layer_inputs(rng.integers(1, 300, size=3), 8, 2, 32, page_size=16, seed=seed,
                            window=int(rng.choice([0, 40])))
    B = len(inp.ctx_lens)
    ref, ref_lse = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                      inp.ctx_lens, inp.scale, window=inp.window)
    splits = int(rng.integers(1, 9))
    parts = np.zeros((B, 8, splits, 32))
    lses = np.zeros((B, 8, splits))
    bounds = []
    for n in inp.ctx_lens:
        lo, hi = oracle.key_range(int(n), inp.window)
        cuts = np.sort(rng.integers(lo, hi + 1, size=splits - 1))
        bounds.append(np.concatenate([[lo], cuts, [hi]]))
    for s in range(splits):
        klo = [bd[s] for bd in bounds]
        khi = [bd[s + 1] for bd in bounds]
        o, l = oracle.decode_attn_ranges(inp.q, inp.k_pool, inp.v_pool, inp.block_table, klo, khi,
                                         inp.scale)
        parts[:, :, s] = o
        lses[:, :, s] = l
    out, lse = oracle.lse_merge(parts.reshape(B * 8, splits, 32), lses.reshape(B * 8, splits))
    np.testing.assert_allclose(out.reshape(B, 8, 32), ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse.reshape(B, 8), ref_lse, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- brute force


@pytest.mark.parametrize("G,window", [(1, 0), (2, 0), (4, 0), (2, 7), (4, 16), (1, 33)])
def test_matches_independent_numpy_twin(G, window):
    """Every n % 16 alignment and several pools/page sizes, tiny D, against the numpy twin."""
    rng = np.random.default_rng(200 + G + window)
    Hkv, D = 2, 8
    for S in (16, 32):
        ns = list(range(1, 49))
        inp = make_layer_inputs(ns, G * Hkv, Hkv, D, page_size=S, window=window,
                                seed=int(rng.integers(1 << 30)), scale=float(rng.uniform(0.1, 1)))
        a = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                               inp.scale, window=window)
        b = twin.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                             inp.scale, window=window)
        np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_poisoned_slots_are_never_read():
    """The generator fills every slot outside [lo, n) with NaN; a finite result shows the oracle
    reads only attended keys, for global and sliding layers."""
    for window in (0, 24):
        inp = make_layer_inputs([1, 15, 16, 17, 33, 47], 4, 2, 16, page_size=16, window=window,
                                seed=17)
        out, lse = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                                      inp.scale, window=window)
        assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


def test_golden_regression_cases():
    """Stored oracle outputs for tiny seeded cases (written by tests/golden/make_golden.py from
    the oracle alone) still reproduce: guards later changes to the oracle."""
    with open(os.path.join(GOLDEN, "oracle_tiny_cases.json")) as f:
        cases = json.load(f)["cases"]
    assert cases
    for case in cases:
        sink, q_len = case.get("sink", 0), case.get("q_len", 1)
        inp = make_layer_inputs(case["ctx_lens"], case["Hq"], case["Hkv"], case["D"],
                                page_size=case["S"], window=case["window"], seed=case["seed"],
                                q_mult=case["q_mult"], sink=sink, q_len=q_len)
        if sink or q_len > 1:
            out, lse = oracle.decode_attn_multi(inp.q if q_len > 1 else inp.q[:, None],
                                                inp.k_pool, inp.v_pool, inp.block_table,
                                                inp.ctx_lens, inp.scale, case["window"], sink)
        else:
            out, lse = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                          inp.ctx_lens, inp.scale, window=case["window"])
        np.testing.assert_allclose(out, np.array(case["out"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, np.array(case["lse"]), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- paged KV append


def test_append_writes_exactly_the_newest_slot():
    rng = np.random.default_rng(40)
    inp = make_layer_inputs([5, 16, 17, 33], 4, 2, 16, page_size=16, seed=41, poison=False)
    k0, v0 = inp.k_pool.copy(), inp.v_pool.copy()
    k_new = rand_bits(rng, (4, 2, 16))
    v_new = rand_bits(rng, (4, 2, 16))
    oracle.append_kv(k_new, v_new, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens)
    expect_k, expect_v = k0.copy(), v0.copy()
    for b, n in enumerate(inp.ctx_lens):
        t = int(n) - 1
        page = inp.block_table[b, t // 16]
        expect_k[page, :, t % 16] = k_new[b]
        expect_v[page, :, t % 16] = v_new[b]
    np.testing.assert_array_equal(inp.k_pool, expect_k)
    np.testing.assert_array_equal(inp.v_pool, expect_v)


def test_append_round_trip_restores_attention():
    """Removing each sequence's newest key/value (NaN) and appending it back gives the original
    attention output bitwise."""
    inp = make_layer_inputs([1, 20, 64, 65], 8, 2, 32, page_size=16, seed=42)
    ref = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                             inp.scale)
    k_new = np.zeros((4, 2, 32), np.uint16)
    v_new = np.zeros((4, 2, 32), np.uint16)
    for b, n in enumerate(inp.ctx_lens):
        t = int(n) - 1
        page = inp.block_table[b, t // 16]
        k_new[b] = inp.k_pool[page, :, t % 16]
        v_new[b] = inp.v_pool[page, :, t % 16]
        inp.k_pool[page, :, t % 16] = 0x7FC0
        inp.v_pool[page, :, t % 16] = 0x7FC0
    oracle.append_kv(k_new, v_new, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens)
    out = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                             inp.scale)
    np.testing.assert_array_equal(out[0], ref[0])
    np.testing.assert_array_equal(out[1], ref[1])


def test_append_one_pool_writes_keys_only():
    rng = np.random.default_rng(43)
    inp = make_layer_inputs([9], 2, 1, 16, page_size=16, seed=44, poison=False)
    k_new = rand_bits(rng, (1, 1, 16))
    pool = inp.k_pool
    oracle.append_kv(k_new, None, pool, pool, inp.block_table, inp.ctx_lens)
    page = inp.block_table[0, 0]
    np.testing.assert_array_equal(pool[page, 0, 8], k_new[0, 0])


def test_append_rejects_positions_outside_the_table():
    inp = make_layer_inputs([16], 2, 1, 16, page_size=16, seed=45)
    ctx = np.array([17], np.int32)  # position 16 needs a second table column that is absent
    with pytest.raises(ValueError):
        oracle.append_kv(np.zeros((1, 1, 16), np.uint16), np.zeros((1, 1, 16), np.uint16),
                         inp.k_pool, inp.v_pool, inp.block_table, ctx)


def _row_code(b, i, g, D, sign=1.0):
    """A row whose every element names (sequence b, new token i, KV head g): 16 b + 4 i + g, plus
    d % 4 quarters so a row read at a shifted column also fails. Exact in bf16 (at most 8
    significant bits)."""
    return bf([sign * (16 * b + 4 * i + g + 0.25 * (d % 4)) for d in range(D)])


# Slots of the L = 3 newest tokens, placed by hand from the block table below (page size 4):
#   b0: ctx 6  -> positions 3, 4, 5:   column 0 (page 5) slot 3, column 1 (page 2) slots 0 and 1
#   b1: ctx 2  -> positions -1, 0, 1:  token 0 skipped, column 0 (page 1) slots 0 and 1
#   b2: ctx 12 -> positions 9, 10, 11: column 2 (page 4) slots 1, 2, 3
_APPEND_TABLE = [[5, 2, 7], [1, 6, -1], [3, 0, 4]]
_APPEND_CTX = [6, 2, 12]
_APPEND_SLOTS = {  # (b, i) -> (page, slot)
    (0, 0): (5, 3), (0, 1): (2, 0), (0, 2): (2, 1),
    (1, 1): (1, 0), (1, 2): (1, 1),
    (2, 0): (4, 1), (2, 1): (4, 2), (2, 2): (4, 3),
}


@pytest.mark.parametrize("one_pool", [False, True])
def test_append_several_tokens_lands_in_hand_placed_slots(one_pool):
    """L = 3 new tokens per sequence, across a page boundary, with a position below 0 skipped:
    every (b, i, g) row lands in the slot worked out by hand above and no other slot changes. A
    reversed token order, a swapped b / i stride or a page / slot mix-up moves some row."""
    B, L, Hkv, D, S, P = 3, 3, 2, 8, 4, 8
    k_new = np.stack([np.stack([np.stack([_row_code(b, i, g, D) for g in range(Hkv)])
                                for i in range(L)]) for b in range(B)])
    v_new = np.stack([np.stack([np.stack([_row_code(b, i, g, D, -1.0) for g in range(Hkv)])
                                for i in range(L)]) for b in range(B)])
    sentinel = bf([-3.5])[0]
    k_pool = np.full((P, Hkv, S, D), sentinel, np.uint16)
    v_pool = k_pool if one_pool else np.full((P, Hkv, S, D), sentinel, np.uint16)
    table = np.array(_APPEND_TABLE, np.int32)
    ctx = np.array(_APPEND_CTX, np.int32)
    oracle.append_kv(k_new, None if one_pool else v_new, k_pool, v_pool, table, ctx)

    expect_k = np.full((P, Hkv, S, D), sentinel, np.uint16)
    expect_v = np.full((P, Hkv, S, D), sentinel, np.uint16)
    for (b, i), (page, slot) in _APPEND_SLOTS.items():
        for g in range(Hkv):
            expect_k[page, g, slot] = _row_code(b, i, g, D)
            expect_v[page, g, slot] = _row_code(b, i, g, D, -1.0)
    np.testing.assert_array_equal(k_pool, expect_k)
    if not one_pool:
        np.testing.assert_array_equal(v_pool, expect_v)
    # The skipped token (b1, i0) was written nowhere.
    for g in range(Hkv):
        assert not (k_pool == _row_code(1, 0, g, D)).all(axis=-1).any()
