"""Helpers of the GPU tests: upload seeded host inputs, call the library through its C ABI, and
compare with the fp64 oracle to the stated tolerance."""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import paged_gqa_kv_attn_amd as pda  # noqa: E402
from paged_gqa_kv_attn_amd.workloads import LayerInputs  # noqa: E402

# Parity bar for fp32 outputs of bf16 inputs with fp32 accumulation.
MAX_ABS = 1e-2
MIN_COS = 0.9999
LSE_ABS = 2e-3   # fp32 scores: |error| <~ 1e-4 * |s| for |s| up to ~20, plus exp/log rounding


def ensure_library():
    if not os.path.exists(pda.library_path()):
        from paged_gqa_kv_attn_amd import build
        build.build()
    return pda.load_library()


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda:0")


def upload(inp: LayerInputs):
    import torch
    dev = device()
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
        torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    return dict(q=bf(inp.q), k=bf(inp.k_pool), v=bf(inp.v_pool), bt=i32(inp.block_table),
                ctx=i32(inp.ctx_lens))


def make_plan(inp: LayerInputs, **kw):
    d = inp.dims
    args = dict(batch=d["B"], num_q_heads=d["Hq"], num_kv_heads=d["Hkv"], head_dim=d["D"],
                page_size=d["S"], max_pages_per_seq=d["M"], num_pages=d["P"],
                max_ctx_len=int(inp.ctx_lens.max()) if len(inp.ctx_lens) else 0,
                window=inp.window, sink=inp.sink, q_len=inp.q_len)
    args.update(kw)
    return pda.decode_attn_plan(**args)


def run(inp: LayerInputs, plan=None, dev_bufs=None, batch=None, **plan_kw):
    """Run the layer on the GPU; returns (out [B,Hq,D] f32, lse [B,Hq] f32) as numpy, with an
    extra query axis after B ([B,L,Hq,D], [B,L,Hq]) when the inputs hold L > 1 queries."""
    import torch
    ensure_library()
    plan = plan or make_plan(inp, **plan_kw)
    t = dev_bufs or upload(inp)
    d = inp.dims
    B = d["B"] if batch is None else batch
    lead = (d["B"],) if inp.q_len == 1 else (d["B"], inp.q_len)
    out = torch.full(lead + (d["Hq"], d["D"]), float("nan"), device=device())
    lse = torch.full(lead + (d["Hq"],), float("nan"), device=device())
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=device())
    if inp.window > 0:
        pda.decode_attn_sliding(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], B, inp.window,
                                inp.scale, out, lse, ws)
    else:
        pda.decode_attn_global(plan, t["q"], t["k"], t["v"], t["bt"], t["ctx"], B, inp.scale,
                               out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def reference(inp: LayerInputs):
    if inp.q_len > 1:
        return oracle.decode_attn_multi(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                        inp.ctx_lens, inp.scale, inp.window, inp.sink)
    if inp.sink > 0:
        return oracle.decode_attn_sink(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                       inp.ctx_lens, inp.scale, inp.window, inp.sink)
    return oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table, inp.ctx_lens,
                              inp.scale, window=inp.window)


def compare(out, lse, ref_out, ref_lse, what="", max_abs=MAX_ABS, min_cos=MIN_COS):
    """Assert the parity bar: max |gpu - oracle| <= max_abs, per-(b,h) cosine >= min_cos, and
    lse within LSE_ABS (equal -inf where the oracle has -inf)."""
    out = np.asarray(out, dtype=np.float64)
    assert np.all(np.isfinite(out)), "%s: non-finite output" % what
    err = np.abs(out - ref_out)
    assert err.max(initial=0.0) <= max_abs, "%s: max abs err %g" % (what, err.max())
    num = (out * ref_out).sum(-1)
    den = np.linalg.norm(out, axis=-1) * np.linalg.norm(ref_out, axis=-1)
    nz = den > 0
    cos = np.where(nz, num / np.where(nz, den, 1), 1.0)
    # rows whose reference is exactly zero (empty ranges) must be exactly zero too
    assert np.all(out[~nz & (np.linalg.norm(ref_out, axis=-1) == 0)] == 0), what
    assert cos.min(initial=1.0) >= min_cos, "%s: min cosine %.7f" % (what, cos.min())
    if lse is not None:
        lse = np.asarray(lse, dtype=np.float64)
        inf_ref = np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(lse), inf_ref), "%s: -inf lse mismatch" % what
        if (~inf_ref).any():
            lerr = np.abs(lse[~inf_ref] - ref_lse[~inf_ref]).max()
            assert lerr <= LSE_ABS, "%s: lse err %g" % (what, lerr)
    return float(err.max(initial=0.0)), float(cos.min(initial=1.0))
