"""GPU tests of the paged KV append: bit-exact against the oracle's append (byte work), K = V
pools, skipped positions, and append followed by attention against the oracle."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
import oracle
import paged_gqa_kv_attn_amd as pda
from paged_gqa_kv_attn_amd.workloads import f32_to_bf16_bits, make_layer_inputs

pytestmark = pytest.mark.gpu


def _bf(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(gu.device()).view(
        torch.bfloat16)


def _host(t):
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("D,Hkv,S", [(512, 2, 16), (256, 8, 16), (256, 4, 64)])
def test_append_bit_exact(D, Hkv, S):
    gu.ensure_library()
    rng = np.random.default_rng(D + Hkv + S)
    ctx = [1, 16, 17, 200, 1023]
    inp = make_layer_inputs(ctx, 2 * Hkv, Hkv, D, page_size=S, seed=[50, D, S], poison=False)
    k_new = f32_to_bf16_bits(rng.standard_normal((len(ctx), Hkv, D), dtype=np.float32))
    v_new = f32_to_bf16_bits(rng.standard_normal((len(ctx), Hkv, D), dtype=np.float32))
    t = gu.upload(inp)
    plan = gu.make_plan(inp)
    pda.decode_attn_append_kv(plan, _bf(k_new), _bf(v_new), t["k"], t["v"], t["bt"], t["ctx"],
                              len(ctx))
    __import__("torch").cuda.synchronize()
    oracle.append_kv(k_new, v_new, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens)
    np.testing.assert_array_equal(_host(t["k"]), inp.k_pool)
    np.testing.assert_array_equal(_host(t["v"]), inp.v_pool)


def test_append_one_pool_and_skips():
    """K = V layers write only K; n = 0, positions past the table and invalid page ids are
    skipped; batch below the plan's leaves the rest alone."""
    gu.ensure_library()
    rng = np.random.default_rng(51)
    ctx = [0, 40, 33, 90, 7]
    inp = make_layer_inputs(ctx, 8, 1, 512, page_size=16, seed=52, poison=False)
    inp.ctx_lens[3] = 10 ** 6                       # past the table row: skipped
    inp.block_table[2, 2] = inp.k_pool.shape[0]     # invalid page id: skipped
    k_new = f32_to_bf16_bits(rng.standard_normal((5, 1, 512), dtype=np.float32))
    t = gu.upload(inp)
    plan = gu.make_plan(inp, max_ctx_len=100)
    before = inp.k_pool.copy()
    pda.decode_attn_append_kv(plan, _bf(k_new), None, t["k"], t["k"], t["bt"], t["ctx"], 4)
    __import__("torch").cuda.synchronize()
    expect = before.copy()
    page = inp.block_table[1, 39 // 16]
    expect[page, 0, 39 % 16] = k_new[1, 0]          # only sequence 1 is written
    np.testing.assert_array_equal(_host(t["k"]), expect)


@pytest.mark.parametrize("window", [0, 100])
def test_append_then_attend(window):
    """The decode step's order: write the new token, then attend over all keys including it."""
    import torch
    gu.ensure_library()
    D = 512 if window == 0 else 256
    ctx = [130, 47, 1000]
    inp = make_layer_inputs(ctx, 16, 2 if window == 0 else 8, D, page_size=16, window=window,
                            seed=[53, window])
    Hkv = inp.k_pool.shape[1]
    rng = np.random.default_rng(54)
    k_new = f32_to_bf16_bits(rng.standard_normal((3, Hkv, D), dtype=np.float32))
    v_new = f32_to_bf16_bits(rng.standard_normal((3, Hkv, D), dtype=np.float32))
    t = gu.upload(inp)
    plan = gu.make_plan(inp)
    pda.decode_attn_append_kv(plan, _bf(k_new), _bf(v_new), t["k"], t["v"], t["bt"], t["ctx"], 3)
    out, lse = gu.run(inp, plan=plan, dev_bufs=t)
    oracle.append_kv(k_new, v_new, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens)
    gu.compare(out, lse, *gu.reference(inp), "append+attend W%d" % window)
    torch.cuda.synchronize()
