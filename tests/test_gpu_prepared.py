"""GPU: prepared calls (arguments checked and converted once, one ctypes call per use) give the
same results as ordinary calls, and read the device data current at each call (lengths, block
tables, K/V), as a serving loop that rewrites its buffers in place needs."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import make_layer_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window", [0, 1024])
def test_prepared_layer_call_matches_and_follows_device_data(window):
    import torch
    import paged_gqa_kv_attn_amd as pda
    gu.ensure_library()
    D, Hkv = (512, 2) if window == 0 else (256, 8)
    # Every page allocated (drawn as a global layer), so the shorter contexts below still find
    # theirs; a sliding call then reads only its window.
    inp = make_layer_inputs([3000, 1777, 64], 16, Hkv, D, page_size=16, seed=[130, window])
    inp.window = window
    plan = gu.make_plan(inp)
    t = gu.upload(inp)
    d = inp.dims
    out = torch.full((d["B"], d["Hq"], d["D"]), float("nan"), device=gu.device())
    lse = torch.full((d["B"], d["Hq"]), float("nan"), device=gu.device())
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=gu.device())
    if window:
        call = pda.decode_attn_sliding(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], d["B"],
                                       window, inp.scale, out, lse, ws, prepare=True)
    else:
        call = pda.decode_attn_global(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], d["B"],
                                      inp.scale, out, lse, ws, prepare=True)
    call()
    torch.cuda.synchronize()
    want = gu.run(inp, plan=plan)
    np.testing.assert_array_equal(out.cpu().numpy(), want[0])
    np.testing.assert_array_equal(lse.cpu().numpy(), want[1])
    # Shorter contexts written in place: the same prepared call attends the new lengths.
    inp.ctx_lens = np.array([2999, 1000, 17], np.int32)
    t["ctx"].copy_(torch.from_numpy(inp.ctx_lens))
    call()
    torch.cuda.synchronize()
    gu.compare(out.cpu().numpy(), lse.cpu().numpy(), *gu.reference(inp), "prepared W%d" % window)


def test_prepared_stage_calls_and_append():
    """Stage 1, stage 2 and the paged append as prepared calls, against the ordinary layer call."""
    import torch
    import paged_gqa_kv_attn_amd as pda
    gu.ensure_library()
    inp = make_layer_inputs([5000, 4321], 16, 2, 512, page_size=16, seed=131)
    plan = gu.make_plan(inp)
    t = gu.upload(inp)
    d = inp.dims
    B = d["B"]
    pos = inp.ctx_lens - 1
    pages = inp.block_table[np.arange(B), pos // d["S"]]
    k_new = torch.from_numpy(np.ascontiguousarray(inp.k_pool[pages, :, pos % d["S"], :])
                             .view(np.int16)).to(gu.device()).view(torch.bfloat16)
    v_new = torch.from_numpy(np.ascontiguousarray(inp.v_pool[pages, :, pos % d["S"], :])
                             .view(np.int16)).to(gu.device()).view(torch.bfloat16)
    out = torch.full((B, d["Hq"], d["D"]), float("nan"), device=gu.device())
    lse = torch.full((B, d["Hq"]), float("nan"), device=gu.device())
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=gu.device())
    # The newest slots are poisoned, then written back by the prepared append.
    for b in range(B):
        t["k"][int(pages[b]), :, int(pos[b] % d["S"])] = float("nan")
        t["v"][int(pages[b]), :, int(pos[b] % d["S"])] = float("nan")
    calls = [
        pda.decode_attn_append_kv(plan, k_new, v_new, t["k"], t["v"], t["bt"], t["ctx"], B,
                                  prepare=True),
        pda.decode_attn_stage1(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], B, inp.scale, ws,
                               prepare=True),
        pda.decode_attn_stage2(plan, B, ws, out, lse, prepare=True),
    ]
    for c in calls:
        c()
    torch.cuda.synchronize()
    want = gu.run(inp, plan=plan)
    np.testing.assert_array_equal(out.cpu().numpy(), want[0])
    np.testing.assert_array_equal(lse.cpu().numpy(), want[1])
