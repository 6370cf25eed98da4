"""GPU tests of the two stages on their own, of graph capture, and of the tensor-level binding
checks. Stage 1's partials are compared with the oracle over the documented chunk ranges; stage 2
is fed synthetic partials (empty chunks included) and compared with the oracle's merge."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
import oracle
import paged_gqa_kv_attn_amd as pda
from paged_gqa_kv_attn_amd.workloads import make_layer_inputs

pytestmark = pytest.mark.gpu


def chunk_ranges(n, window, ns):
    """Key range of each split, as the header documents it."""
    lo = max(0, n - window) if window > 0 else 0
    tlo, thi = lo // 16, (n + 15) // 16
    T = max(0, thi - tlo)
    out = []
    for s in range(ns):
        a = (tlo + s * T // ns) * 16
        b = (tlo + (s + 1) * T // ns) * 16
        out.append((max(a, lo), min(b, n)) if b > a else (0, 0))
    return out


@pytest.mark.parametrize("D,G,window", [(512, 8, 0), (256, 2, 100), (512, 4, 0)])
def test_stage1_partials_match_oracle_chunks(D, G, window):
    import torch
    gu.ensure_library()
    ctx = [1, 250, 611]
    inp = make_layer_inputs(ctx, 2 * G, 2, D, page_size=16, window=window, seed=[21, D, G])
    plan = gu.make_plan(inp, force_splits=6)
    t = gu.upload(inp)
    ws = torch.full((plan.workspace_bytes // 4,), float("nan"), device=gu.device())
    pda.decode_attn_stage1(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], len(ctx), inp.scale,
                           ws)
    torch.cuda.synchronize()
    ns, Hq = plan.num_splits, 2 * G
    rows = len(ctx) * Hq
    o_part = ws[: rows * ns * D].view(len(ctx), Hq, ns, D).cpu().numpy()
    off = plan.partial_lse_offset // 4
    lse_part = ws[off: off + rows * ns].view(len(ctx), Hq, ns).cpu().numpy()
    for s in range(ns):
        rng = [chunk_ranges(n, window, ns)[s] for n in ctx]
        ref = oracle.decode_attn_ranges(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                        [r[0] for r in rng], [r[1] for r in rng], inp.scale)
        gu.compare(o_part[:, :, s], lse_part[:, :, s], ref[0], ref[1], "split %d" % s)


def split_keysets(n_ctx, L, G, window, sink, ns):
    """Keys each (query, split) attends in stage 1, as the header documents it: queries in blocks
    of 16 / G (32 / G when G * L > 16); a block walks the sink tiles, then its window's tiles, and
    split s takes list entries [floor(s T / ns), floor((s + 1) T / ns)); a query keeps the keys of
    those tiles that it attends."""
    per = (32 if G * L > 16 and L > 1 else 16) // G
    sink = sink if window > 0 else 0
    end = lambda i: max(0, n_ctx - L + i + 1)
    wlo = lambda e: e - window if window > 0 and e > window else 0
    sets = {}
    for first in range(0, L, per):
        last = min(L, first + per) - 1
        n, lo = end(last), wlo(end(first))
        sk = min(sink, lo)
        st = -(-sk // 16)
        w0 = max(st, lo // 16)
        T = st + max(0, -(-n // 16) - w0)
        for sp in range(ns):
            tiles = [e if e < st else e - st + w0 for e in range(sp * T // ns, (sp + 1) * T // ns)]
            keys = {t for p in tiles for t in range(16 * p, 16 * p + 16)}
            for i in range(first, last + 1):
                ni, li = end(i), wlo(end(i))
                sets[i, sp] = sorted(t for t in keys if t < ni and (t >= li or t < sink))
    return sets


def runs(keys):
    out = []
    for t in keys:
        if out and out[-1][1] == t:
            out[-1][1] = t + 1
        else:
            out.append([t, t + 1])
    return out


@pytest.mark.parametrize("D,G,L,window,sink", [(256, 2, 3, 40, 20), (512, 8, 3, 0, 0),
                                               (256, 2, 1, 33, 17), (512, 8, 4, 100, 5)])
def test_stage1_partials_follow_the_documented_tile_list(D, G, L, window, sink):
    """Stage-1 partials with sinks and several query tokens: each (query, split) equals the
    oracle over the keys the documented tile list gives it (sink and window parts merged by the
    oracle's LSE merge)."""
    import torch
    gu.ensure_library()
    ctx = [1, 30, 70, 130, 300]
    inp = make_layer_inputs(ctx, 2 * G, 2, D, page_size=16, window=window, sink=sink,
                            seed=[27, D, G, L], q_len=L)
    plan = gu.make_plan(inp, force_splits=5)
    t = gu.upload(inp)
    ws = torch.full((plan.workspace_bytes // 4,), float("nan"), device=gu.device())
    pda.decode_attn_stage1(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], len(ctx), inp.scale,
                           ws)
    torch.cuda.synchronize()
    ns, Hq, B = plan.num_splits, 2 * G, len(ctx)
    rows = B * L * Hq
    o_part = ws[: rows * ns * D].view(B, L, Hq, ns, D).cpu().numpy()
    off = plan.partial_lse_offset // 4
    lse_part = ws[off: off + rows * ns].view(B, L, Hq, ns).cpu().numpy()
    q4 = inp.q if L > 1 else inp.q[:, None]
    sets = [split_keysets(n, L, G, window, sink, ns) for n in ctx]
    for i in range(L):
        for sp in range(ns):
            parts = []
            for r in range(2):  # at most a sink run and a window run
                lo_hi = [runs(sets[b][i, sp])[r] if len(runs(sets[b][i, sp])) > r else [0, 0]
                         for b in range(B)]
                parts.append(oracle.decode_attn_ranges(
                    np.ascontiguousarray(q4[:, i]), inp.k_pool, inp.v_pool, inp.block_table,
                    [x[0] for x in lo_hi], [x[1] for x in lo_hi], inp.scale))
            assert all(len(runs(sets[b][i, sp])) <= 2 for b in range(B))
            o = np.stack([p[0] for p in parts], axis=2).reshape(B * Hq, 2, D)
            l = np.stack([p[1] for p in parts], axis=2).reshape(B * Hq, 2)
            ref_o, ref_l = oracle.lse_merge(o, l)
            gu.compare(o_part[:, i, :, sp], lse_part[:, i, :, sp], ref_o.reshape(B, Hq, D),
                       ref_l.reshape(B, Hq), "query %d split %d" % (i, sp))


@pytest.mark.parametrize("D", [256, 512])
@pytest.mark.parametrize("ns", [1, 3, 16, 17, 32, 33, 64, 257])
def test_stage2_merge_matches_oracle(ns, D):
    """Split counts below, at and above the 16 split groups of the merge, and head dims 256, 512."""
    import torch
    gu.ensure_library()
    B, Hq = 2, 4
    inp = make_layer_inputs([40, 40], Hq, 1, D, page_size=16, seed=22)
    plan = gu.make_plan(inp, force_splits=ns)
    rng = np.random.default_rng(ns)
    o = rng.standard_normal((B, Hq, ns, D)).astype(np.float32)
    lse = (rng.standard_normal((B, Hq, ns)) * 3).astype(np.float32)
    lse[rng.random((B, Hq, ns)) < 0.3] = -np.inf   # empty chunks
    lse[1, 2, :] = -np.inf                          # a row with every chunk empty
    o[np.isneginf(lse)] = 0.0
    ws = torch.zeros(plan.workspace_bytes // 4, dtype=torch.float32, device=gu.device())
    ws[: o.size] = torch.from_numpy(o.ravel()).to(gu.device())
    off = plan.partial_lse_offset // 4
    ws[off: off + lse.size] = torch.from_numpy(lse.ravel()).to(gu.device())
    out = torch.empty((B, Hq, D), device=gu.device())
    lse_out = torch.empty((B, Hq), device=gu.device())
    pda.decode_attn_stage2(plan, B, ws, out, lse_out)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.lse_merge(o.reshape(B * Hq, ns, D).astype(np.float64),
                                    lse.reshape(B * Hq, ns).astype(np.float64))
    np.testing.assert_allclose(out.cpu().numpy().reshape(B * Hq, D), ref_o, atol=2e-5, rtol=1e-5)
    l = lse_out.cpu().numpy().ravel()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l))
    fin = ~np.isneginf(ref_l)
    np.testing.assert_allclose(l[fin], ref_l[fin], atol=1e-5)
    assert np.all(out.cpu().numpy()[1, 2] == 0)


def test_graph_capture_replays_with_new_step_data():
    """Both entry points captured in one HIP graph; per-step data (lengths, block tables) change
    between replays through the same buffers; each replay matches an eager call."""
    import torch
    gu.ensure_library()
    dev = gu.device()
    g_inp = make_layer_inputs([500, 1000], 16, 2, 512, page_size=16, seed=23, pool_factor=3)
    s_inp = make_layer_inputs([500, 1000], 16, 8, 256, page_size=16, window=300, seed=24,
                              pool_factor=3)
    gp = gu.make_plan(g_inp, max_ctx_len=1200)
    sp = gu.make_plan(s_inp, max_ctx_len=1200)
    gt, st = gu.upload(g_inp), gu.upload(s_inp)
    g_out = torch.zeros((2, 16, 512), device=dev)
    s_out = torch.zeros((2, 16, 256), device=dev)
    g_ws = torch.empty(gp.workspace_bytes, dtype=torch.uint8, device=dev)
    s_ws = torch.empty(sp.workspace_bytes, dtype=torch.uint8, device=dev)

    def step():
        pda.decode_attn_global(gp, gt["q"], gt["k"], gt["v"], gt["bt"], gt["ctx"], 2,
                               g_inp.scale, g_out, None, g_ws)
        pda.decode_attn_sliding(sp, st["q"], st["k"], st["v"], st["bt"], st["ctx"], 2, 300,
                                s_inp.scale, s_out, None, s_ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    rng = np.random.default_rng(25)
    for it in range(4):
        ctx = rng.integers(1, 1009, size=2).astype(np.int32)  # table holds 63 pages
        for inp, t in ((g_inp, gt), (s_inp, st)):
            fresh = make_layer_inputs(ctx, inp.q.shape[1], inp.k_pool.shape[1], inp.q.shape[2],
                                      page_size=16, window=inp.window, seed=[26, it],
                                      num_pages=inp.k_pool.shape[0],
                                      max_pages_per_seq=inp.block_table.shape[1])
            inp.block_table[:] = fresh.block_table
            inp.ctx_lens[:] = fresh.ctx_lens
            inp.k_pool[:] = fresh.k_pool
            inp.v_pool[:] = fresh.v_pool
            u = gu.upload(inp)
            for key in ("k", "v", "bt", "ctx"):
                t[key].copy_(u[key])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_g, got_s = g_out.cpu().numpy(), s_out.cpu().numpy()
        eager_g, _ = gu.run(g_inp, plan=gp)
        eager_s, _ = gu.run(s_inp, plan=sp)
        np.testing.assert_array_equal(got_g, eager_g)
        np.testing.assert_array_equal(got_s, eager_s)
        gu.compare(got_g, None, *gu.reference(g_inp), "graph global %d" % it)
        gu.compare(got_s, None, *gu.reference(s_inp), "graph sliding %d" % it)


def test_binding_rejects_wrong_tensors():
    import torch
    gu.ensure_library()
    inp = make_layer_inputs([20], 4, 1, 256, page_size=16, seed=27)
    plan = gu.make_plan(inp)
    t = gu.upload(inp)
    out = torch.empty((1, 4, 256), device=gu.device())
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=gu.device())
    with pytest.raises(ValueError):
        pda.decode_attn_global(plan, t["q"].float(), t["k"], t["v"], t["bt"], t["ctx"], 1,
                               inp.scale, out, None, ws)
    with pytest.raises(ValueError):
        pda.decode_attn_global(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], 1, inp.scale,
                               out.cpu(), None, ws)
    with pytest.raises(pda.DecodeAttnError):
        pda.decode_attn_global(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], 1, inp.scale,
                               out, None, ws[:16])
