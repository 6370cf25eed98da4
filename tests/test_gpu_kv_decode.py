"""GPU parity of single-token decode at head_dim 512 when the values are the keys (one pool passed
as K and V, each tile read once and parked in LDS for both products): every group size, windows
that cut tiles, contexts of 1 to a few thousand keys ending inside a page, invalid block-table
entries, page sizes from 16 to 64 keys, split counts from the planner's to more splits than tiles
(workgroups without a tile), and the full-size K = V global layers of the 32K-128K workloads, each
against the fp64 oracle with V := K. Unused pool slots hold NaN: a kernel that let one into P.V
would fail."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import make_layer_inputs, make_workload_layer

pytestmark = pytest.mark.gpu


def _one_pool(inp):
    inp.v_pool = inp.k_pool
    t = gu.upload(inp)
    t["v"] = t["k"]
    return t


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("S,window", [(16, 0), (64, 0), (16, 37), (32, 300)])
def test_kv_decode_small_shapes(G, S, window):
    print("k=v decode G=%d S=%d W=%d" % (G, S, window), flush=True)
    Hkv = 2 if G < 16 else 1
    ctx = [1, 15, 16, 17, 100, 333, 1000, 2049]
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, 512, page_size=S, window=window,
                            seed=[90, G, S, window], q_mult=1.5)
    t = _one_pool(inp)
    ref = gu.reference(inp)
    for splits in (0, 1, 3, 7, 64):
        out, lse = gu.run(inp, dev_bufs=t, values_are_keys=True, force_splits=splits)
        gu.compare(out, lse, *ref, "k=v G%d S%d W%d ns%d" % (G, S, window, splits))


def test_kv_decode_planned_splits():
    """The planner's pick for a K = V layer at head_dim 512: two workgroups per CU."""
    inp = make_layer_inputs([5000, 3000], 16, 2, 512, page_size=16, seed=91)
    plan = gu.make_plan(inp, values_are_keys=True, num_cus=256)
    assert plan.num_splits == 128
    t = _one_pool(inp)
    out, lse = gu.run(inp, plan=plan, dev_bufs=t)
    gu.compare(out, lse, *gu.reference(inp), "k=v planned")


def test_kv_decode_invalid_pages_and_extreme_scores():
    """Block-table entries outside [0, P) are skipped (their keys masked), and q scaled so scores
    reach the hundreds."""
    import oracle
    inp = make_layer_inputs([400, 300, 90], 16, 2, 512, page_size=16, seed=92, q_mult=30.0)
    inp.block_table[0, 0] = inp.k_pool.shape[0] + 5
    inp.block_table[1, 0] = -7
    inp.block_table[2, 0] = -1
    inp.v_pool = inp.k_pool
    ref = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool,
                             np.ascontiguousarray(inp.block_table[:, 1:]), inp.ctx_lens - 16,
                             inp.scale)
    t = _one_pool(inp)
    for splits in (0, 5):
        out, lse = gu.run(inp, dev_bufs=t, values_are_keys=True, force_splits=splits)
        gu.compare(out, lse, *ref, "k=v invalid first page ns%d" % splits)


@pytest.mark.parametrize("name", ["long_ctx", "very_long_b2", "very_long_b1"])
def test_kv_decode_workload_global_layer(name):
    """The global layers of the 4 x 32K, 2 x 64K and 1 x 128K workloads with one pool."""
    print("k=v workload", name, flush=True)
    inp = make_workload_layer(name, "global")
    t = _one_pool(inp)
    out, lse = gu.run(inp, dev_bufs=t, values_are_keys=True)
    err, cos = gu.compare(out, lse, *gu.reference(inp), "k=v %s" % name)
    print("  max_abs_err %.3g  min_cos %.7f" % (err, cos), flush=True)
