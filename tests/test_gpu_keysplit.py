"""GPU parity of single-token decode at head_dim 256 with G <= 4 (the sliding-window layers' shape)
with one split, which runs on the key-split stage-1 kernel (the 8 waves of a workgroup take turns
over the tiles and merge their softmax states once at the end), next to more splits on the
column-split kernel. Covers every group size, page sizes, windows, ragged and very short contexts,
waves with more than 64 tiles (the page-id vector refetched), plans whose context length differs
from the real ones, invalid page ids, and a batch large enough that the planner picks one split
itself."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import make_layer_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("S,window", [(16, 0), (16, 64), (64, 1024), (32, 33)])
def test_keysplit_forced_splits(G, S, window):
    print("keysplit G=%d S=%d W=%d" % (G, S, window), flush=True)
    ctx = [1, 15, 16, 17, 100, 1031, 2049, 777]
    inp = make_layer_inputs(ctx, 2 * G, 2, 256, page_size=S, window=window,
                            seed=[120, G, S, window], q_mult=1.5)
    ref = gu.reference(inp)
    for ns in (0, 1, 2, 3, 7, 16):
        out, lse = gu.run(inp, force_splits=ns)
        gu.compare(out, lse, *ref, "keysplit G%d S%d W%d ns%d" % (G, S, window, ns))


@pytest.mark.parametrize("ns", [1, 2, 5])
def test_keysplit_more_than_64_tiles_per_wave(ns):
    """A 20000-key global layer at head_dim 256: with one split each of the 8 waves walks 157
    tiles, so its vector of page ids is fetched three times."""
    print("keysplit long ns=%d" % ns, flush=True)
    inp = make_layer_inputs([20000, 9001], 4, 2, 256, page_size=16, seed=[121, ns])
    out, lse = gu.run(inp, force_splits=ns)
    gu.compare(out, lse, *gu.reference(inp), "keysplit long ns%d" % ns)


@pytest.mark.parametrize("hint", ["exact", "longer", "ragged"])
def test_keysplit_plan_length_is_only_a_hint(hint):
    """The plan's max_ctx_len sizes the split count only: equal lengths at the planned length, a plan
    for longer contexts and a ragged batch under it all give the oracle's result."""
    ctx = {"exact": [4000] * 4, "longer": [4000] * 4, "ragged": [4000, 3999, 1234, 17]}[hint]
    inp = make_layer_inputs(ctx, 16, 8, 256, page_size=16, window=1024, seed=[122, ["exact", "longer", "ragged"].index(hint)],
                            max_pages_per_seq=400)
    plan = gu.make_plan(inp, max_ctx_len=5000 if hint == "longer" else 4000, force_splits=1)
    out, lse = gu.run(inp, plan=plan)
    gu.compare(out, lse, *gu.reference(inp), "keysplit hint %s" % hint)


def test_keysplit_invalid_pages_are_skipped():
    """Block-table entries outside [0, P) are never dereferenced: their keys are skipped. One on the
    first page of each sequence (global layer at head_dim 256); the result equals attention over
    the keys after that page."""
    import oracle
    inp = make_layer_inputs([100, 64, 700], 8, 2, 256, page_size=16, seed=123)
    inp.block_table[0, 0] = inp.k_pool.shape[0] + 5
    inp.block_table[1, 0] = -7
    inp.block_table[2, 0] = -1
    for ns in (0, 1):
        out, lse = gu.run(inp, force_splits=ns)
        ref = oracle.decode_attn_ranges(inp.q, inp.k_pool, inp.v_pool,
                                        np.maximum(inp.block_table, 0), [16, 16, 16],
                                        [100, 64, 700], inp.scale)
        gu.compare(out, lse, *ref, "keysplit invalid page ns%d" % ns)


def test_keysplit_planner_picks_one_split_for_a_large_batch():
    """32 sequences x 8 KV heads (256 pairs, one per CU): the planner's own pick is one split."""
    inp = make_layer_inputs([1500 + 7 * b for b in range(32)], 16, 8, 256, page_size=16,
                            window=1024, seed=124)
    plan = gu.make_plan(inp)
    assert plan.num_splits == 1
    out, lse = gu.run(inp, plan=plan)
    gu.compare(out, lse, *gu.reference(inp), "keysplit planner one split")
