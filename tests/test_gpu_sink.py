"""GPU parity of sliding layers with attention sinks (StreamingLLM-style views: the first `sink`
keys plus the last `window` keys) and of sparse block-table views, against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import WORKLOADS, make_layer_inputs, make_workload_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("window,sink", [(1, 1), (16, 4), (17, 16), (33, 17), (5, 40), (64, 64)])
def test_sink_every_alignment(window, sink):
    """Contexts 1..120 in one batch: every alignment of n, of the window edge and of the sink
    edge mod 32, including windows that overlap the sink keys."""
    print("sink alignment W=%d sink=%d" % (window, sink), flush=True)
    ctx = list(range(1, 121))
    inp = make_layer_inputs(ctx, 4, 2, 256, page_size=16, window=window, sink=sink,
                            seed=[51, window, sink])
    for splits in (0, 3):  # planner's count, then several chunks per sequence
        out, lse = gu.run(inp, force_splits=splits)
        gu.compare(out, lse, *gu.reference(inp), "W%d sink%d ns%d" % (window, sink, splits))


@pytest.mark.parametrize("D,G,S", [(256, 2, 16), (256, 8, 64), (512, 8, 32), (512, 16, 16)])
def test_sink_small_shapes(D, G, S):
    print("sink small D=%d G=%d S=%d" % (D, G, S), flush=True)
    Hkv = 2 if G < 16 else 1
    ctx = [1, 3, 20, 100, 333, 520, 1500]
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, D, page_size=S, window=200, sink=4,
                            seed=[52, D, G, S], q_mult=1.5)
    out, lse = gu.run(inp, force_splits=5)
    gu.compare(out, lse, *gu.reference(inp), "sink D%d G%d S%d" % (D, G, S))


@pytest.mark.parametrize("name", [n for n, wl in WORKLOADS.items() if "sliding" in wl.layers])
def test_sink_workload_sliding_layers(name):
    """Each workload's sliding layer at full size with 4 sink keys."""
    print("sink workload", name, flush=True)
    wl = WORKLOADS[name]
    spec = wl.layers["sliding"]
    base = make_workload_layer(name, "sliding")
    inp = make_layer_inputs(base.ctx_lens, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                            page_size=wl.page_size, window=spec.window, scale=spec.scale,
                            num_pages=wl.num_pages, pool_factor=wl.pool_factor,
                            q_mult=spec.q_mult, seed=[wl.index, 2], sink=4)
    out, lse = gu.run(inp)
    err, cos = gu.compare(out, lse, *gu.reference(inp), "%s sliding sink 4" % name)
    print("  max_abs_err %.3g  min_cos %.7f" % (err, cos), flush=True)


def test_sparse_view_equals_sink_window():
    """A sparse block-table view (a table naming only the sink pages and the window pages of each
    sequence, with n counting the keys they hold) attended as a global layer gives the same
    result as the sliding layer with page-aligned sinks over the full table."""
    import torch
    S, window, sink = 16, 64, 32
    ctx = [704, 128, 96, 2000, 48]  # multiples of S: the window starts on a page boundary
    inp = make_layer_inputs(ctx, 8, 1, 512, page_size=S, window=window, sink=sink, seed=53)
    out, lse = gu.run(inp)
    gu.compare(out, lse, *gu.reference(inp), "sink view")

    view = np.full_like(inp.block_table, -1)
    lens = []
    for b, n in enumerate(ctx):
        lo = max(0, n - window)
        cols = sorted(set(range(0, min(sink, lo) // S)) | set(range(lo // S, (n - 1) // S + 1)))
        view[b, :len(cols)] = inp.block_table[b, cols]
        lens.append(min(sink, lo) + (n - lo))
    vinp = make_layer_inputs(ctx, 8, 1, 512, page_size=S, seed=53)  # shape donor
    vinp.q, vinp.k_pool, vinp.v_pool = inp.q, inp.k_pool, inp.v_pool
    vinp.block_table, vinp.ctx_lens = view, np.asarray(lens, dtype=np.int32)
    vout, vlse = gu.run(vinp)
    gu.compare(vout, vlse, *gu.reference(vinp), "sparse view")
    gu.compare(vout, vlse, out.astype(np.float64), lse.astype(np.float64), "view vs sink",
               max_abs=2e-3)
    torch.cuda.synchronize()


def test_sink_zero_is_bitwise_the_sliding_layer():
    inp = make_layer_inputs([1000, 77, 2049], 16, 2, 256, page_size=16, window=300, seed=54)
    a = gu.run(inp)
    b = gu.run(inp, sink=0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
