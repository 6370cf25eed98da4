"""GPU parity of multi-token decode (L query tokens per sequence, causal: query i sits at position
n - L + i), against the fp64 oracle: every compiled (head_dim, group) pair, several L (one and
several query blocks), windows, sinks, contexts shorter than L, K = V pools, append of the L new
tokens followed by attention, and a full-size 32K layer."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import WORKLOADS, make_layer_inputs, workload_ctx_lens

pytestmark = pytest.mark.gpu

SWEEP = [(D, G, L) for D in (256, 512) for G in (1, 2, 4, 8, 16) for L in (2, 3, 8)]


@pytest.mark.parametrize("D,G,L", SWEEP)
@pytest.mark.parametrize("window", [0, 37])
def test_multi_small_shapes(D, G, L, window):
    """Ragged contexts, including ones shorter than L (queries before position 0 attend
    nothing), several splits per sequence."""
    print("multi D=%d G=%d L=%d W=%d" % (D, G, L, window), flush=True)
    Hkv = 2 if G < 16 else 1
    ctx = [1, 2, 15, 17, 100, 333, 520]
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, D, page_size=16, window=window,
                            seed=[61, D, G, L, window], q_mult=1.5, q_len=L)
    out, lse = gu.run(inp, force_splits=5)
    gu.compare(out, lse, *gu.reference(inp), "multi D%d G%d L%d W%d" % (D, G, L, window))


@pytest.mark.parametrize("L,window,sink", [(4, 0, 0), (4, 17, 0), (5, 33, 0), (16, 16, 4),
                                           (3, 20, 40)])
def test_multi_every_alignment(L, window, sink):
    """Contexts 1..90 in one batch: every alignment of each query's end and window edge."""
    print("multi alignment L=%d W=%d sink=%d" % (L, window, sink), flush=True)
    ctx = list(range(1, 91))
    inp = make_layer_inputs(ctx, 4, 2, 256, page_size=16, window=window, sink=sink,
                            seed=[62, L, window, sink], q_len=L)
    for splits in (0, 3):
        out, lse = gu.run(inp, force_splits=splits)
        gu.compare(out, lse, *gu.reference(inp), "L%d W%d sink%d ns%d" % (L, window, sink,
                                                                          splits))


@pytest.mark.parametrize("S", [32, 64, 256])
def test_multi_larger_pages(S):
    """Several query tokens and a sliding window with sinks over pages of 32-256 keys (tiles are
    16-key slices of a page)."""
    print("multi pages S=%d" % S, flush=True)
    ctx = [3, 100, 517, 1300]
    inp = make_layer_inputs(ctx, 16, 2, 512, page_size=S, window=300, sink=8, seed=[67, S],
                            q_len=3)
    out, lse = gu.run(inp, force_splits=4)
    gu.compare(out, lse, *gu.reference(inp), "multi S%d" % S)


def test_multi_one_query_is_bitwise_single_token():
    """A plan with q_len 1 and q given as [B, 1, Hq, D] is the single-token path, bit for bit."""
    inp = make_layer_inputs([1000, 77, 2049], 16, 2, 512, page_size=16, seed=63)
    a = gu.run(inp)
    b = gu.run(inp, q_len=1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("window", [0, 300])
def test_multi_values_equal_keys(window):
    inp = make_layer_inputs([1000, 77, 2049], 16, 2, 512 if window == 0 else 256, page_size=16,
                            window=window, seed=[64, window], q_len=4)
    inp.v_pool = inp.k_pool
    t = gu.upload(inp)
    t["v"] = t["k"]
    out, lse = gu.run(inp, dev_bufs=t, values_are_keys=True)
    gu.compare(out, lse, *gu.reference(inp), "multi k=v W%d" % window)


@pytest.mark.parametrize("window", [0, 100])
def test_multi_append_then_attend(window):
    """Poison the L newest slots, append the L new tokens' K/V through the library, attend: the
    result equals the oracle on the original cache."""
    import torch
    import oracle
    import paged_gqa_kv_attn_amd as pda
    L = 4
    inp = make_layer_inputs([500, 64, 999], 8, 2, 512 if window == 0 else 256, page_size=16,
                            window=window, seed=[65, window], q_len=L)
    d = inp.dims
    rng = np.random.default_rng(66)
    k_new = rng.integers(0, 2**16, size=(d["B"], L, d["Hkv"], d["D"]), dtype=np.uint16) & 0x3FFF
    v_new = rng.integers(0, 2**16, size=(d["B"], L, d["Hkv"], d["D"]), dtype=np.uint16) & 0x3FFF
    oracle.append_kv(k_new, v_new, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens)
    ref = gu.reference(inp)
    poisoned_k, poisoned_v = inp.k_pool.copy(), inp.v_pool.copy()
    S = d["S"]
    for b, n in enumerate(inp.ctx_lens):
        for t in range(n - L, n):
            p = inp.block_table[b, t // S]
            poisoned_k[p, :, t % S] = 0x7FC0
            poisoned_v[p, :, t % S] = 0x7FC0
    inp.k_pool, inp.v_pool = poisoned_k, poisoned_v
    t = gu.upload(inp)
    plan = gu.make_plan(inp)
    dev = gu.device()
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    pda.decode_attn_append_kv(plan, bf(k_new), bf(v_new), t["k"], t["v"], t["bt"], t["ctx"],
                              d["B"])
    out, lse = gu.run(inp, plan=plan, dev_bufs=t)
    gu.compare(out, lse, *ref, "multi append+attend W%d" % window)


def test_multi_workload_global_layer():
    """The 32K global layer (batch 4, 16/2 heads, D 512) verifying 4 tokens per sequence."""
    print("multi workload long_ctx global L=4", flush=True)
    wl = WORKLOADS["long_ctx"]
    spec = wl.layers["global"]
    inp = make_layer_inputs(workload_ctx_lens(wl), spec.num_q_heads, spec.num_kv_heads,
                            spec.head_dim, page_size=wl.page_size, scale=spec.scale,
                            num_pages=wl.num_pages, pool_factor=wl.pool_factor, q_mult=spec.q_mult,
                            seed=[wl.index, 3], q_len=4)
    out, lse = gu.run(inp)
    err, cos = gu.compare(out, lse, *gu.reference(inp), "long_ctx global L4")
    print("  max_abs_err %.3g  min_cos %.7f" % (err, cos), flush=True)
