"""GPU parity of the step before attention: the rotation table (decode_attn_rope_cache) against
cos/sin in fp64, and the fused QK-norm + RoPE + paged append (decode_attn_append_kv_rope) against
the fp64 oracle in oracle/rope.py, then attention over the appended cache against the attention
oracle.

Bar for a bf16 output y of the fused step (fp32 arithmetic, one rounding): |y - y64| <= ulp(y64) +
2^-20 * max|row of y64|, where y64 is the oracle's fp64 value and ulp is the bf16 spacing at y64:
half an ulp for the rounding, the rest for fp32 error (a few 2^-24 of the row's magnitude, the
extra term covering outputs that are small next to their row after the rotation's cancellation).
At least 99% of the outputs must also equal the oracle's own nearest-even rounding, which a
truncating or biased rounding fails. Values copied without a norm, untouched slots and untouched
q rows are compared bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
import oracle
from oracle import rope as orope
import paged_gqa_kv_attn_amd as pda
from paged_gqa_kv_attn_amd.workloads import (WORKLOADS, make_layer_inputs, make_new_tokens,
                                              workload_ctx_lens)

pytestmark = pytest.mark.gpu

NAN_BITS = 0xFFFF  # a NaN pattern no output of the step can have


def _torch():
    import torch
    return torch


def _bf(a):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(gu.device()).view(
        torch.bfloat16)


def _f32(a):
    return _torch().from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(gu.device())


def _host(t):
    return t.view(_torch().int16).cpu().numpy().view(np.uint16)


def _bf16_ulp(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax >= 2.0 ** -126, 2.0 ** (e - 7), 2.0 ** -133)


def check_bf16(got_bits, ref64, what):
    """The bar above, over rows of the last axis."""
    got = orope._bf16_to_f64(got_bits)
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    rowmax = np.abs(ref64).max(axis=-1, keepdims=True)
    tol = _bf16_ulp(ref64) + 2.0 ** -20 * rowmax
    err = np.abs(got - ref64)
    bad = err > tol
    assert not bad.any(), "%s: %d outputs off, worst %g (tol %g)" % (
        what, bad.sum(), err[bad].max(), tol[bad][np.argmax(err[bad])])
    same = np.mean(got_bits == orope._f64_to_bf16(ref64)) if got_bits.size else 1.0
    assert same >= 0.99, "%s: only %.4f of the outputs round as the oracle's" % (what, same)
    return float(same)


@pytest.mark.parametrize("max_pos,rot,freq_dim,theta", [
    (40000, 512, 0, 1e6), (4096, 128, 512, 1e4), (70000, 64, 0, 5e5), (3, 2, 0, 1e4)])
def test_rope_cache(max_pos, rot, freq_dim, theta):
    """Each entry is cos / sin of t f_j in fp64 rounded to fp32: within 2^-24 of the fp64 value
    (the fp32 rounding) plus 1e-10 (the device's double-precision angle)."""
    print("rope cache P=%d R=%d F=%d theta=%g" % (max_pos, rot, freq_dim, theta), flush=True)
    gu.ensure_library()
    torch = _torch()
    cs = torch.full((max_pos, rot), float("nan"), device=gu.device())
    pda.decode_attn_rope_cache(cs, max_pos, rot, theta, freq_dim)
    got = cs.cpu().numpy().astype(np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * orope.inv_freq(theta, rot,
                                                                         freq_dim or None)
    ref = np.concatenate([np.cos(ang), np.sin(ang)], axis=1)
    np.testing.assert_allclose(got, ref, rtol=0, atol=2.0 ** -24 + 1e-10)


def _written_slots(inp, ctx, L, max_position, pool_shape):
    """(b, i, page, slot) of every append the oracle makes: it is run on pools filled with a NaN
    pattern and the slots it changed are read back."""
    probe = np.full(pool_shape, NAN_BITS, dtype=np.uint16)
    B = len(ctx)
    Hq, Hkv, D = inp["q"].shape[2], inp["k"].shape[2], inp["q"].shape[3]
    orope.prepare_and_append(np.zeros((B, L, Hq, D), np.uint16), np.zeros((B, L, Hkv, D),
                             np.uint16), None, probe, probe, inp["bt"], ctx, max_position, False,
                             False, None, None, None, 1e-6, 1e4, 0, False)
    pos = orope.positions_of(ctx, L)
    out = []
    S = pool_shape[2]
    for b in range(B):
        for i in range(L):
            t = int(pos[b, i])
            if t < 0 or t >= max_position or t // S >= inp["bt"].shape[1]:
                continue
            page = int(inp["bt"][b, t // S])
            if 0 <= page < pool_shape[0] and probe[page, 0, t % S, 0] != NAN_BITS:
                out.append((b, i, page, t % S))
    return out


def _f32_offset(a, misalign):
    """a on the device; with misalign, as a view 4 bytes past a 16-byte boundary."""
    if not misalign:
        return _f32(a)
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    big = _f32(np.concatenate([np.zeros(1, np.float32), flat]))
    return big[1:].view(a.shape)


def run_case(D, Hq, Hkv, S, ctx, L, rot, interleaved, norm_qk, norm_v, same_pool, seed,
             max_position=None, freq_dim=0, theta=1e4, batch=None, in_place=False,
             weights=True, pool=None, misalign=False):
    """One fused step on the GPU and in the oracle; checks q_out and both pools. Returns the GPU
    buffers, the oracle's q bits and pools, and the step's inputs for an attention check."""
    torch = _torch()
    gu.ensure_library()
    ctx = np.asarray(ctx, dtype=np.int32)
    B = len(ctx)
    batch = B if batch is None else batch
    inp = pool if pool is not None else make_layer_inputs(ctx, Hq, Hkv, D, page_size=S,
                                                          seed=[seed, 1], poison=False)
    if same_pool:
        inp.v_pool = inp.k_pool
    new = make_new_tokens(B, L, Hq, Hkv, D, seed=[seed, 2])
    max_position = int(ctx.max()) + 5 if max_position is None else max_position
    qw, kw, vw = ((new["q_weight"], new["k_weight"], new["v_weight"]) if weights else
                  (None, None, None))
    flags = (pda.NORM_QK if norm_qk else 0) | (pda.NORM_V if norm_v else 0)

    t = gu.upload(inp)
    if same_pool:
        t["v"] = t["k"]
    q_dev = _bf(new["q"])
    q_out = q_dev if in_place else _bf(np.full(new["q"].shape, NAN_BITS, np.uint16))
    cs = None
    if rot > 0:
        cs = _f32_offset(np.zeros((max_position, rot), np.float32), misalign)
        pda.decode_attn_rope_cache(cs, max_position, rot, theta, freq_dim)
    plan = gu.make_plan(inp, q_len=L) if pool is None else gu.make_plan(inp)
    pda.decode_attn_append_kv_rope(
        plan, q_dev, q_out, _bf(new["k"]), None if same_pool else _bf(new["v"]), t["k"], t["v"],
        t["bt"], t["ctx"], batch, cs, max_position, rot, interleaved, flags,
        _f32_offset(qw, misalign) if qw is not None else None,
        _f32_offset(kw, misalign) if kw is not None else None,
        _f32_offset(vw, misalign) if vw is not None else None, 1e-6)
    torch.cuda.synchronize()

    # Oracle on the first `batch` sequences.
    k_ref = inp.k_pool.copy()
    v_ref = k_ref if same_pool else inp.v_pool.copy()
    sel = slice(0, batch)
    q_bits_ref = orope.prepare_and_append(
        new["q"][sel], new["k"][sel], None if same_pool else new["v"][sel], k_ref, v_ref,
        inp.block_table[sel], ctx[sel], max_position, norm_qk, norm_v, qw, kw, vw, 1e-6, theta,
        rot, interleaved, freq_dim or None)
    qo64, ko64, vo64 = orope.prepare(new["q"][sel], new["k"][sel], new["v"][sel], ctx[sel],
                                     norm_qk, norm_v, qw, kw, vw, 1e-6, theta, rot, interleaved,
                                     freq_dim or None)
    what = "D%d Hq%d Hkv%d S%d L%d R%d il%d nqk%d nv%d same%d" % (
        D, Hq, Hkv, S, L, rot, interleaved, norm_qk, norm_v, same_pool)

    # q_out: rows at positions in range are checked against fp64; the others are untouched.
    got_q = _host(q_out).reshape(B, L, Hq, D)
    pos = orope.positions_of(ctx, L)
    live = (pos >= 0) & (pos < max_position)
    live[batch:] = False
    untouched = new["q"] if in_place else np.full_like(new["q"], NAN_BITS)
    np.testing.assert_array_equal(got_q[~live], untouched[~live], err_msg=what + " q skipped")
    check_bf16(got_q[live], qo64[live[sel]], what + " q")

    # Pools: appended slots against fp64, everything else bit for bit.
    got_k = _host(t["k"])
    got_v = got_k if same_pool else _host(t["v"])
    slots = _written_slots(dict(q=new["q"][sel], k=new["k"][sel], bt=inp.block_table[sel]),
                           ctx[sel], L, max_position, inp.k_pool.shape)
    mask = np.zeros(inp.k_pool.shape[:3], dtype=bool)
    k_rows, k_ref64, v_rows, v_ref64 = [], [], [], []
    for b, i, page, s in slots:
        mask[page, :, s] = True
        k_rows.append(got_k[page, :, s])
        k_ref64.append(ko64[b, i])
        v_rows.append(got_v[page, :, s])
        v_ref64.append(vo64[b, i])
    np.testing.assert_array_equal(got_k[~mask], inp.k_pool[~mask], err_msg=what + " k untouched")
    if not same_pool:
        np.testing.assert_array_equal(got_v[~mask], inp.v_pool[~mask],
                                      err_msg=what + " v untouched")
    if slots:
        check_bf16(np.stack(k_rows), np.stack(k_ref64), what + " k")
        if not same_pool:
            if norm_v:
                check_bf16(np.stack(v_rows), np.stack(v_ref64), what + " v")
            else:
                np.testing.assert_array_equal(np.stack(v_rows),
                                              np.stack([new["v"][b, i] for b, i, _, _ in slots]),
                                              err_msg=what + " v copy")
    return dict(inp=inp, t=t, plan=plan, q_out=q_out, q_bits_ref=q_bits_ref, k_ref=k_ref,
                v_ref=v_ref, n_slots=len(slots))


# (D, Hq, Hkv, S): the two Gemma-4 layer shapes and smaller group sizes, pages of 16 to 256 keys.
SHAPES = [(512, 16, 2, 16), (256, 16, 8, 16), (512, 4, 4, 64), (256, 2, 1, 256)]


@pytest.mark.parametrize("D,Hq,Hkv,S", SHAPES)
@pytest.mark.parametrize("rot_frac,interleaved", [(1.0, False), (1.0, True), (0.25, False),
                                                  (0.5, True)])
@pytest.mark.parametrize("L", [1, 7])
def test_append_kv_rope_parity(D, Hq, Hkv, S, rot_frac, interleaved, L):
    """Full and partial rotation in both pairings, QK-norm with weights, decode (L = 1) and a
    7-token chunk; ragged contexts incl. 0 and shorter than L (leading tokens skipped)."""
    rot = int(D * rot_frac)
    print("rope D=%d Hq=%d Hkv=%d S=%d R=%d il=%d L=%d" % (D, Hq, Hkv, S, rot, interleaved, L),
          flush=True)
    run_case(D, Hq, Hkv, S, [0, 3, 129, 1000, 4097], L, rot, interleaved, True, False, False,
             seed=[80, D, Hq, S, rot, int(interleaved), L])


@pytest.mark.parametrize("norm_qk,norm_v,weights", [(False, False, True), (True, True, True),
                                                    (True, True, False), (False, True, True)])
def test_append_kv_rope_norm_modes(norm_qk, norm_v, weights):
    """RoPE alone, QK-norm + V-norm with and without weights, V-norm alone."""
    print("rope norm qk=%d v=%d w=%d" % (norm_qk, norm_v, weights), flush=True)
    run_case(256, 16, 8, 16, [40, 1, 777], 3, 256, False, norm_qk, norm_v, False,
             seed=[81, norm_qk, norm_v, weights], weights=weights)


@pytest.mark.parametrize("D,rot,interleaved,misalign", [
    (512, 40, False, False), (512, 2, True, False), (256, 36, False, False),
    (256, 12, True, False), (256, 256, True, True), (512, 512, False, True),
    (512, 128, False, True)])
def test_append_kv_rope_general_path(D, rot, interleaved, misalign):
    """The per-element path: rotated widths that split a lane's elements (R not a multiple of
    2 * D / 64) or a table and weights only 4-byte aligned."""
    print("rope general D=%d R=%d il=%d mis=%d" % (D, rot, interleaved, misalign), flush=True)
    Hq, Hkv = (16, 2) if D == 512 else (16, 8)
    run_case(D, Hq, Hkv, 16, [9, 260, 1], 3, rot, interleaved, True, True, False,
             seed=[88, D, rot, int(interleaved), int(misalign)], misalign=misalign)


def test_append_kv_rope_no_rotation_and_in_place():
    """rotary_dim 0 (norm only, no table) with q normalised in place."""
    run_case(512, 8, 1, 32, [5, 64, 65], 2, 0, False, True, False, False, seed=82, in_place=True)


@pytest.mark.parametrize("rot,interleaved", [(512, False), (128, True)])
def test_append_kv_rope_one_pool(rot, interleaved):
    """Layers whose values are their keys: one pool, only k written (v_new NULL)."""
    run_case(512, 16, 2, 16, [17, 300, 2], 4, rot, interleaved, True, False, True,
             seed=[83, rot])


def test_append_kv_rope_skips():
    """A token at or past max_position is skipped whole; a page column past the table row or an
    invalid page id skips the append but not q; batch below the plan's leaves the last sequence
    alone."""
    ctx = [20, 50, 90, 33, 61, 45]
    inp = make_layer_inputs(ctx, 8, 2, 256, page_size=16, seed=[84, 1], poison=False)
    assert inp.block_table.shape[1] == 6
    inp.ctx_lens[1] = 250                               # t 249 >= max_position: skipped whole
    inp.ctx_lens[2] = 150                               # t 149: column 9 past the 6-column row
    inp.block_table[3, 2] = inp.k_pool.shape[0] + 3     # t 32: invalid page id
    r = run_case(256, 8, 2, 16, inp.ctx_lens, 1, 256, False, True, True, False, seed=84,
                 max_position=200, batch=5, pool=inp)
    assert r["n_slots"] == 2  # sequences 0 (t 19) and 4 (t 60); sequence 5 is not in the batch


def test_append_kv_rope_partial_rotation_with_full_spacing():
    """A partial rotation that keeps the full head's frequency spacing (freq_dim = D)."""
    run_case(512, 16, 2, 16, [100, 2000], 5, 128, False, True, False, False, seed=85,
             freq_dim=512, theta=1e6)


def test_append_kv_rope_longest_chunk():
    """The largest chunk a plan accepts: 8192 new tokens of one sequence (pure prefill), pages of
    64 keys, both pairings' fast path (R = D) and a partial one."""
    print("rope L=8192", flush=True)
    for rot, inter in ((256, False), (64, True)):
        run_case(256, 2, 1, 64, [8192], 8192, rot, inter, True, True, False, seed=[89, rot])


@pytest.mark.parametrize("L,window", [(1, 0), (24, 0), (1, 300), (64, 300)])
def test_append_kv_rope_then_attention(L, window):
    """The decode step's order: norm + rotate + append the new tokens, then attend with the
    rotated q over the cache including them; against the oracle step then the oracle attention."""
    print("rope+attend L=%d W=%d" % (L, window), flush=True)
    D, Hq, Hkv = (512, 16, 2) if window == 0 else (256, 16, 8)
    ctx = [L + 3, 700, 1500]
    inp = make_layer_inputs(ctx, Hq, Hkv, D, page_size=16, window=window, seed=[86, L, window],
                            q_len=L)
    r = run_case(D, Hq, Hkv, 16, ctx, L, D, False, True, False, False, seed=[86, L, window],
                 pool=inp, theta=1e6 if window == 0 else 1e4)
    t = r["t"]
    t["q"] = r["q_out"]
    out, lse = gu.run(inp, plan=r["plan"], dev_bufs=t)
    inp.q = r["q_bits_ref"] if L > 1 else r["q_bits_ref"][:, 0]
    inp.k_pool, inp.v_pool = r["k_ref"], r["v_ref"]
    gu.compare(out, lse, *gu.reference(inp), "rope+attend L%d W%d" % (L, window))


@pytest.mark.parametrize("L", [1, 256])
def test_append_kv_rope_workload_global(L):
    """The 32K global layer (batch 4, 16/2 heads, D 512, 33792-token contexts): the step for L new
    tokens per sequence, then attention, against the oracle."""
    print("rope workload long_ctx global L=%d" % L, flush=True)
    wl = WORKLOADS["long_ctx"]
    spec = wl.layers["global"]
    ctx = workload_ctx_lens(wl)
    inp = make_layer_inputs(ctx, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                            page_size=wl.page_size, scale=spec.scale, num_pages=wl.num_pages,
                            pool_factor=wl.pool_factor, q_mult=spec.q_mult, seed=[wl.index, 87, L],
                            q_len=L)
    r = run_case(512, 16, 2, wl.page_size, ctx, L, 512, False, True, False, False,
                 seed=[87, L], pool=inp, max_position=int(ctx.max()) + 4096, theta=1e6)
    t = r["t"]
    t["q"] = r["q_out"]
    out, lse = gu.run(inp, plan=r["plan"], dev_bufs=t)
    inp.q = r["q_bits_ref"] if L > 1 else r["q_bits_ref"][:, 0]
    inp.k_pool, inp.v_pool = r["k_ref"], r["v_ref"]
    err, cos = gu.compare(out, lse, *gu.reference(inp), "rope+attend long_ctx L%d" % L)
    print("  max_abs_err %.3g  min_cos %.7f" % (err, cos), flush=True)


def test_decode_loop_in_a_graph():
    """A decode loop: the fused step then attention captured once in a HIP graph; each replay
    appends the next token of every sequence (ctx_lens advance by one through the same buffer,
    with fresh q, k and v), and is compared bit for bit with the same calls made eagerly on a
    second set of buffers, and with the oracle's step followed by the attention oracle."""
    torch = _torch()
    gu.ensure_library()
    dev = gu.device()
    D, Hq, Hkv, B, steps, max_pos = 512, 16, 2, 2, 4, 2048
    ctx0 = np.array([100, 517], dtype=np.int32)
    inp = make_layer_inputs(ctx0 + steps, Hq, Hkv, D, page_size=16, seed=90, poison=False)
    inp.ctx_lens[:] = ctx0
    plan = gu.make_plan(inp)
    cs = torch.empty((max_pos, D), dtype=torch.float32, device=dev)
    pda.decode_attn_rope_cache(cs, max_pos, D, 1e6)
    w = make_new_tokens(B, 1, Hq, Hkv, D, seed=[91, 0])
    wq, wk = _f32(w["q_weight"]), _f32(w["k_weight"])

    def buffers():
        t = gu.upload(inp)
        t.update(q_raw=_bf(w["q"]), q=_bf(w["q"]), k_new=_bf(w["k"]), v_new=_bf(w["v"]),
                 out=torch.zeros((B, Hq, D), device=dev),
                 ws=torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev))
        return t

    def step(t):
        pda.decode_attn_append_kv_rope(plan, t["q_raw"], t["q"], t["k_new"], t["v_new"], t["k"],
                                       t["v"], t["bt"], t["ctx"], B, cs, max_pos, D, False,
                                       pda.NORM_QK, wq, wk, None, 1e-6)
        pda.decode_attn_global(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], B, inp.scale,
                               t["out"], None, t["ws"])

    host_k, host_v = inp.k_pool.copy(), inp.v_pool.copy()
    tg, te = buffers(), buffers()

    def feed(t, new, ctx):
        for key, src in (("q_raw", new["q"]), ("k_new", new["k"]), ("v_new", new["v"])):
            t[key].copy_(_bf(src))
        t["ctx"].copy_(torch.from_numpy(ctx).to(dev))

    # Warm up on the capture stream with the first replay's data (the replay rewrites the same
    # slot with the same values), then capture.
    first = make_new_tokens(B, 1, Hq, Hkv, D, seed=[92, 0])
    feed(tg, first, ctx0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(tg)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(tg)
    torch.cuda.synchronize()

    for it in range(steps):
        print("graph decode step %d" % it, flush=True)
        new = make_new_tokens(B, 1, Hq, Hkv, D, seed=[92, it])
        ctx = (ctx0 + it).astype(np.int32)
        feed(tg, new, ctx)
        feed(te, new, ctx)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(te)
        torch.cuda.synchronize()
        for key in ("q", "k", "v"):
            np.testing.assert_array_equal(_host(tg[key]), _host(te[key]), err_msg="%s %d" % (key, it))
        got = tg["out"].cpu().numpy()
        np.testing.assert_array_equal(got, te["out"].cpu().numpy())
        q_bits = orope.prepare_and_append(new["q"], new["k"], new["v"], host_k, host_v,
                                          inp.block_table, ctx, max_pos, True, False,
                                          w["q_weight"], w["k_weight"], None, 1e-6, 1e6, D, False)
        ref = oracle.decode_attn(q_bits[:, 0], host_k, host_v, inp.block_table, ctx, inp.scale)
        gu.compare(got, None, *ref, "graph decode step %d" % it)


def _random_rope_cases(n=40):
    rng = np.random.default_rng(2026)
    cases = []
    for i in range(n):
        D = int(rng.choice([256, 512]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        S = int(rng.choice([16, 32, 64, 128]))
        L = int(rng.choice([1, 1, 2, 3, 5, 16, 40]))
        B = int(rng.integers(1, 5))
        ctx = [int(x) for x in rng.integers(0, 700, size=B)]
        rot = int(rng.choice([0, 2, D // 4, D // 2, D, 2 * int(rng.integers(1, D // 2 + 1))]))
        cases.append(dict(D=D, Hq=G * Hkv, Hkv=Hkv, S=S, L=L, ctx=ctx, rot=rot,
                          interleaved=bool(rng.integers(0, 2)), norm_qk=bool(rng.integers(0, 2)),
                          norm_v=bool(rng.integers(0, 2)), same_pool=bool(rng.integers(0, 4) == 0),
                          in_place=bool(rng.integers(0, 2)), weights=bool(rng.integers(0, 3) > 0),
                          misalign=bool(rng.integers(0, 4) == 0),
                          max_position=(None if rng.integers(0, 3) > 0 else
                                        int(rng.integers(1, 700))),
                          batch=int(rng.integers(1, B + 1)), freq_dim=int(rng.choice([0, 0, D])),
                          theta=float(rng.choice([1e4, 5e5, 1e6]))))
    return cases


@pytest.mark.parametrize("i,case", list(enumerate(_random_rope_cases())))
def test_append_kv_rope_random(i, case):
    """Seeded random combinations of every option of the step: head dim, group, KV heads, page
    size, new tokens per sequence, ragged contexts (shorter than L included), rotated width (0,
    2, partial, odd multiples of 2, full), pairing, norm flags, weights or none, one pool, in place,
    4-byte-aligned tables and weights, a max_position that skips tokens, batch below the plan's,
    frequency spacing and theta."""
    c = case
    print("rope random %d %s" % (i, c), flush=True)
    run_case(c["D"], c["Hq"], c["Hkv"], c["S"], c["ctx"], c["L"], c["rot"], c["interleaved"],
             c["norm_qk"], c["norm_v"], c["same_pool"], seed=[93, i],
             max_position=c["max_position"], freq_dim=c["freq_dim"] if c["rot"] else 0,
             theta=c["theta"], batch=c["batch"], in_place=c["in_place"], weights=c["weights"],
             misalign=c["misalign"])
