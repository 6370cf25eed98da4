"""GPU parity of prefill chunks: L from 17 up to the 8192-token maximum new query tokens per
sequence (causal, query i at position n - L + i), against the fp64 oracle. Covers pure prefill
(ctx = L: the prompt's first chunk), chunks appended to an existing context, sliding windows with
sinks, every compiled (head_dim, group) pair, the one-split path (the planner's pick for large L,
where stage 1 writes the output directly and no merge runs) next to forced split counts, and a
chunk of the 32K global layer."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import WORKLOADS, make_layer_inputs, workload_ctx_lens

pytestmark = pytest.mark.gpu

SWEEP = [(D, G) for D in (256, 512) for G in (1, 2, 4, 8, 16)]


@pytest.mark.parametrize("D,G", SWEEP)
@pytest.mark.parametrize("L,window", [(33, 0), (100, 0), (100, 64)])
def test_prefill_small_shapes(D, G, L, window):
    """Pure prefill (ctx = L), ctx shorter than L (leading queries attend nothing) and chunks
    on top of an existing context, with the planner's split count and with 3 forced splits."""
    print("prefill D=%d G=%d L=%d W=%d" % (D, G, L, window), flush=True)
    Hkv = 2 if G < 16 else 1
    ctx = [L, L - 7, L + 5, 3 * L + 1, 700]
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, D, page_size=16, window=window,
                            seed=[71, D, G, L, window], q_mult=1.5, q_len=L)
    ref = gu.reference(inp)
    for splits in (0, 3):
        out, lse = gu.run(inp, force_splits=splits)
        gu.compare(out, lse, *ref, "prefill D%d G%d L%d W%d ns%d" % (D, G, L, window, splits))


@pytest.mark.parametrize("L", [1024, 1280])
def test_prefill_one_split_chunks(L):
    """Chunks large enough that the query blocks fill the GPU: the plan has one split, stage 1
    writes out and lse in place and stage 2 is skipped."""
    print("prefill one-split L=%d" % L, flush=True)
    inp = make_layer_inputs([L, 2000], 16, 2, 512, page_size=16, seed=[72, L], q_len=L)
    plan = gu.make_plan(inp)
    assert plan.num_splits == 1
    out, lse = gu.run(inp, plan=plan)
    gu.compare(out, lse, *gu.reference(inp), "prefill one-split L%d" % L)


def test_prefill_one_split_without_lse_output():
    """With one split and lse_out NULL the chunk's lse goes to the workspace, which then needs only
    the [B, L, Hq] lse plane (plan.layer_workspace_bytes); out is unchanged."""
    import torch
    import paged_gqa_kv_attn_amd as pda
    gu.ensure_library()
    inp = make_layer_inputs([1100, 1313], 16, 2, 512, page_size=16, seed=73, q_len=1100)
    plan = gu.make_plan(inp)
    assert plan.num_splits == 1
    d = inp.dims
    rows = d["B"] * inp.q_len * d["Hq"]
    assert plan.layer_workspace_bytes == -(-rows * 4 // 256) * 256 < plan.workspace_bytes
    t = gu.upload(inp)
    out = torch.full((d["B"], inp.q_len, d["Hq"], d["D"]), float("nan"), device=gu.device())
    ws = torch.full((plan.layer_workspace_bytes // 4,), float("nan"), device=gu.device())
    pda.decode_attn_global(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], d["B"], inp.scale,
                           out, None, ws)
    torch.cuda.synchronize()
    ref_out, ref_lse = gu.reference(inp)
    lse_ws = ws[:rows].view(d["B"], inp.q_len, d["Hq"]).cpu().numpy()
    gu.compare(out.cpu().numpy(), lse_ws, ref_out, ref_lse, "prefill no lse")


@pytest.mark.parametrize("window,sink", [(128, 0), (128, 4), (1024, 16)])
def test_prefill_sliding_with_sinks(window, sink):
    print("prefill sliding W=%d sink=%d" % (window, sink), flush=True)
    inp = make_layer_inputs([300, 1500, 77], 16, 8, 256, page_size=16, window=window, sink=sink,
                            seed=[74, window, sink], q_len=300)
    for splits in (0, 2):
        out, lse = gu.run(inp, force_splits=splits)
        gu.compare(out, lse, *gu.reference(inp), "prefill W%d sink%d ns%d" % (window, sink,
                                                                             splits))


def test_prefill_values_equal_keys():
    inp = make_layer_inputs([600, 1100], 16, 2, 512, page_size=16, seed=75, q_len=512)
    inp.v_pool = inp.k_pool
    t = gu.upload(inp)
    t["v"] = t["k"]
    out, lse = gu.run(inp, dev_bufs=t, values_are_keys=True)
    gu.compare(out, lse, *gu.reference(inp), "prefill k=v")


@pytest.mark.parametrize("window,sink", [(0, 0), (300, 4)])
def test_prefill_values_equal_keys_forced_splits(window, sink):
    """K = V at head_dim 512 (one pool for both, each tile staged once) with split counts that
    leave 1 to 3 tile-list entries per split, so the last step of a split stages clamped re-reads,
    on lengths that end inside a page; a windowed variant with sinks."""
    print("prefill k=v forced splits W=%d sink=%d" % (window, sink), flush=True)
    ctx = [197, 250, 83]
    inp = make_layer_inputs(ctx, 16, 2, 512, page_size=16, window=window, sink=sink,
                            seed=[77, window, sink], q_mult=1.5, q_len=80)
    inp.v_pool = inp.k_pool
    t = gu.upload(inp)
    t["v"] = t["k"]
    ref = gu.reference(inp)
    for splits in (0, 7, 11, 16):
        out, lse = gu.run(inp, dev_bufs=t, values_are_keys=True, force_splits=splits)
        gu.compare(out, lse, *ref, "prefill k=v W%d sink%d ns%d" % (window, sink, splits))


def test_prefill_longest_chunk():
    """The largest chunk a plan accepts: 8192 queries, pure prefill of an 8192-token prompt, with
    pages of 64 keys."""
    print("prefill L=8192", flush=True)
    inp = make_layer_inputs([8192], 2, 1, 256, page_size=64, seed=76, q_len=8192)
    out, lse = gu.run(inp)
    gu.compare(out, lse, *gu.reference(inp), "prefill L8192")


def test_prefill_workload_global_chunk():
    """A 256-token chunk at the end of each 33792-token context of the 32K global layer (batch 4,
    16/2 heads, D 512)."""
    print("prefill workload long_ctx global L=256", flush=True)
    wl = WORKLOADS["long_ctx"]
    spec = wl.layers["global"]
    inp = make_layer_inputs(workload_ctx_lens(wl), spec.num_q_heads, spec.num_kv_heads,
                            spec.head_dim, page_size=wl.page_size, scale=spec.scale,
                            num_pages=wl.num_pages, pool_factor=wl.pool_factor, q_mult=spec.q_mult,
                            seed=[wl.index, 4], q_len=256)
    out, lse = gu.run(inp)
    err, cos = gu.compare(out, lse, *gu.reference(inp), "long_ctx global L256")
    print("  max_abs_err %.3g  min_cos %.7f" % (err, cos), flush=True)


@pytest.mark.parametrize("S", [32, 48, 256, 1008, 1024])
@pytest.mark.parametrize("D,G,window,sink", [(512, 8, 0, 0), (256, 2, 200, 8)])
def test_prefill_pages_empty_and_short_sequences(S, D, G, window, sink):
    """Pages of 32 to 1024 keys (tiles are 16-key slices of a page; 48 and 1008 give 3 and 63
    tiles per page, which the kernel's page-of-tile reciprocal must divide exactly), an empty
    sequence (all its queries attend nothing: out = 0, lse = -inf), sequences shorter than the
    chunk, a window with sinks, and 64 forced splits (most of them empty for the short
    sequences)."""
    print("prefill pages S=%d D=%d G=%d W=%d sink=%d" % (S, D, G, window, sink), flush=True)
    Hkv = 2
    inp = make_layer_inputs([0, 5, 300, 1200], G * Hkv, Hkv, D, page_size=S, window=window,
                            sink=sink, seed=[77, S, D, window], q_mult=1.5, q_len=100)
    for splits in (0, 3, 64):
        out, lse = gu.run(inp, force_splits=splits)
        gu.compare(out, lse, *gu.reference(inp), "prefill S%d D%d ns%d" % (S, D, splits))


def test_prefill_sliding_values_equal_keys():
    inp = make_layer_inputs([900, 64], 16, 8, 256, page_size=16, window=300, sink=4, seed=78,
                            q_len=200)
    inp.v_pool = inp.k_pool
    t = gu.upload(inp)
    t["v"] = t["k"]
    out, lse = gu.run(inp, dev_bufs=t, values_are_keys=True)
    gu.compare(out, lse, *gu.reference(inp), "prefill sliding k=v")


@pytest.mark.parametrize("D,G,L", [(512, 8, 64), (512, 2, 40), (256, 2, 64)])
def test_prefill_invalid_first_page_is_skipped(D, G, L):
    """A block-table entry outside [0, P) on the first page of a sequence: its 16 keys are
    skipped, so the chunk equals the same queries over the sequence without that page (block
    table shifted by one page, context 16 keys shorter: the same keys at the same causal offsets).
    Covers the zero-filled tiles of the direct-to-LDS fetch (head_dim 512, 128-row workgroups)
    and of the register-staged paths."""
    import oracle
    print("prefill invalid first page D=%d G=%d L=%d" % (D, G, L), flush=True)
    Hkv = 2
    inp = make_layer_inputs([400, 300], G * Hkv, Hkv, D, page_size=16, seed=[79, D, G, L],
                            q_mult=1.5, q_len=L)
    inp.block_table[0, 0] = inp.k_pool.shape[0] + 5
    inp.block_table[1, 0] = -7
    ref = oracle.decode_attn_multi(inp.q, inp.k_pool, inp.v_pool,
                                   np.ascontiguousarray(inp.block_table[:, 1:]),
                                   inp.ctx_lens - 16, inp.scale)
    for splits in (0, 3):
        out, lse = gu.run(inp, force_splits=splits)
        gu.compare(out, lse, *ref, "prefill invalid page D%d G%d L%d ns%d" % (D, G, L, splits))


@pytest.mark.parametrize("scale", [-0.06, 0.0])
@pytest.mark.parametrize("D,G,window", [(512, 8, 0), (512, 2, 0), (256, 4, 300)])
def test_prefill_negative_and_zero_scale(scale, D, G, window):
    """A negative scale (the kernel flips q's sign and scales by |scale|, so that the softmax
    maximum is taken over the raw scores) and a zero scale (uniform weights over the attended
    keys), on the 128-row kernel (D 512, G 8) and the 64-row ones, with planned and 3 splits."""
    print("prefill scale=%g D=%d G=%d W=%d" % (scale, D, G, window), flush=True)
    Hkv = 2
    inp = make_layer_inputs([130, 700, 1500], G * Hkv, Hkv, D, page_size=16, window=window,
                            scale=scale, seed=[80, D, G, window, int(scale < 0)], q_len=100)
    ref = gu.reference(inp)
    for splits in (0, 3):
        out, lse = gu.run(inp, force_splits=splits)
        gu.compare(out, lse, *ref, "prefill scale %g D%d G%d ns%d" % (scale, D, G, splits))
