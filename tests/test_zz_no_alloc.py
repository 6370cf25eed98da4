"""GPU parity of the allocation-free layer call (decode_attn_layer_noalloc, the library's static
device array as workspace) against the layer call with a caller workspace (the same kernels, so
bit for bit) and against the fp64 oracle. Each test makes two calls in a row, the second with a
smaller input, so the array still holds the first call's partials when the second runs."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import make_layer_inputs, make_workload_layer

pytestmark = pytest.mark.gpu


def _noalloc(inp, plan, batch=None):
    import torch
    import paged_gqa_kv_attn_amd as pda
    gu.ensure_library()
    t = gu.upload(inp)
    d = inp.dims
    B = d["B"] if batch is None else batch
    lead = (d["B"],) if inp.q_len == 1 else (d["B"], inp.q_len)
    out = torch.full(lead + (d["Hq"], d["D"]), float("nan"), device=gu.device())
    lse = torch.full(lead + (d["Hq"],), float("nan"), device=gu.device())
    pda.decode_attn_layer_noalloc(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], B, inp.window,
                                  inp.scale, out, lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _check(inp, what, batch=None, **plan_kw):
    plan = gu.make_plan(inp, **plan_kw)
    print("noalloc %s: %r" % (what, plan), flush=True)
    got = _noalloc(inp, plan, batch)
    want = gu.run(inp, plan=plan, batch=batch)
    B = inp.dims["B"] if batch is None else batch
    np.testing.assert_array_equal(got[0][:B], want[0][:B])
    np.testing.assert_array_equal(got[1][:B], want[1][:B])
    ref_out, ref_lse = gu.reference(inp)
    gu.compare(got[0][:B], got[1][:B], ref_out[:B], ref_lse[:B], "noalloc " + what)
    return plan


@pytest.mark.parametrize("kind", ["global", "sliding"])
def test_noalloc_full_size_then_smaller(kind):
    """The 4 x 33792 layer at full size, then a batch of 3 short sequences (splits capped by their
    tiles, so a smaller partial buffer) called with batch 2 of the plan's 3."""
    first = make_workload_layer("long_ctx", kind)
    p1 = _check(first, "long_ctx %s" % kind)
    if kind == "global":
        second = make_layer_inputs([500, 333, 77], 16, 2, 512, seed=[90, 0], q_mult=2.0)
    else:
        second = make_layer_inputs([300, 77, 33], 16, 8, 256, window=1024, seed=[90, 1])
    p2 = _check(second, "ragged %s" % kind, batch=2)
    assert p2.layer_workspace_bytes < p1.layer_workspace_bytes


def test_noalloc_multi_token_then_one_split_chunk():
    """Four causal query tokens per sequence (row groups, 2 workgroups per CU), then a one-split
    prefill chunk whose layer call keeps only its lse plane in the array."""
    first = make_layer_inputs([5000, 6001], 16, 2, 512, seed=91, q_len=4)
    p1 = _check(first, "q_len 4")
    second = make_layer_inputs([1100, 1313], 16, 2, 512, seed=92, q_len=1100)
    p2 = _check(second, "prefill chunk")
    assert p2.num_splits == 1 and p2.layer_workspace_bytes < p1.layer_workspace_bytes
