"""The C-ABI library loads, exports every symbol its header declares, plans on the host, and
rejects bad arguments before launching anything. CPU only: no call here reaches a kernel launch
or a device query (plans pass num_cus explicitly)."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

from paged_gqa_kv_attn_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decode_attn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_PLAN, ERR_HIP, ERR_ALIGN = range(8)


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(decode_attn_\w+)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("decode_attn_plan", "decode_attn_global", "decode_attn_sliding",
                     "decode_attn_stage1", "decode_attn_stage2", "decode_attn_append_kv",
                     "decode_attn_rope_cache", "decode_attn_append_kv_rope",
                     "decode_attn_status_str", "decode_attn_version"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_plan_struct_layout_matches_header():
    # 15 int32 problem fields, 4 int32, 2 uint64, uint32 magic, int32, uint64, 4 int32 reserved
    assert ctypes.sizeof(binding.Problem) == 60
    assert binding.Plan.workspace_bytes.offset == 80
    assert binding.Plan.magic.offset == 96
    assert binding.Plan.layer_workspace_bytes.offset == 104
    assert ctypes.sizeof(binding.Plan) == 128


def plan(**kw):
    base = dict(batch=4, num_q_heads=16, num_kv_heads=2, head_dim=512, page_size=16,
                max_pages_per_seq=2112, num_pages=16896, max_ctx_len=33792, window=0,
                num_cus=256)
    base.update(kw)
    return binding.decode_attn_plan(**base)


def expected_workspace(B, Hq, ns, D, L=1):
    rows = B * L * Hq * ns
    lse_off = -(-rows * D * 4 // 256) * 256
    return lse_off, -(-(lse_off + rows * 4) // 256) * 256


@pytest.mark.parametrize("kw,splits", [
    (dict(), 32),                                                     # 4 x 33792 global
    (dict(batch=1, max_pages_per_seq=8256, num_pages=16384, max_ctx_len=132096), 128),
    (dict(batch=2, max_pages_per_seq=4160, num_pages=16384, max_ctx_len=66560), 64),
    (dict(batch=8, max_pages_per_seq=80, max_ctx_len=1280), 16),      # 16 pairs
    (dict(num_kv_heads=8, head_dim=256, window=1024), 8),             # 32 pairs: key split, 1/CU
    (dict(num_kv_heads=8, head_dim=256, window=1024, sink=4), 16),    # + 1 sink tile
    (dict(batch=32, num_kv_heads=8, head_dim=256, window=1024), 1),   # 256 pairs: key split
    (dict(batch=32, num_kv_heads=8, head_dim=256, window=1024, values_are_keys=1), 2),
    (dict(batch=32, num_kv_heads=8, head_dim=256, window=1024, sink=4), 2),
    (dict(batch=1, num_kv_heads=8, head_dim=256, window=64, max_ctx_len=8192), 5),  # 5 tiles
    (dict(batch=1, num_kv_heads=8, head_dim=256, window=64, max_ctx_len=8192, sink=40), 8),
    (dict(q_len=4), 64),                                              # 32 rows: 1 block, 2/CU
    (dict(q_len=8), 32),                                              # 2 blocks of 4 queries
    (dict(q_len=2), 32),                                              # 1 block: as q_len 1
    (dict(batch=1, num_q_heads=4, num_kv_heads=1, max_pages_per_seq=64, max_ctx_len=1024,
          q_len=8), 64),                                              # G 4: capped by tiles
    (dict(batch=1, num_q_heads=4, num_kv_heads=1, max_pages_per_seq=64, max_ctx_len=1024), 64),
    (dict(batch=1, max_pages_per_seq=4, max_ctx_len=64), 4),          # capped: >= 1 tile/split
    (dict(q_len=16), 32),                                             # 1 prefill block of 16
    (dict(q_len=512), 1),                                             # prefill chunk: 32 blocks
    (dict(batch=1, q_len=64, max_ctx_len=4096), 32),                  # 4 blocks of 128 rows
    (dict(batch=1, num_kv_heads=8, head_dim=256, window=1024, q_len=256), 8),  # 8 x 8 blocks
    (dict(num_q_heads=8, num_kv_heads=1), 64),                        # TP2 share of 4 x 33792
    (dict(num_q_heads=8, num_kv_heads=4, head_dim=256, window=1024), 16),  # its sliding layer
    (dict(batch=1, num_q_heads=8, num_kv_heads=1, max_pages_per_seq=8256, num_pages=16384,
          max_ctx_len=132096), 256),                                  # TP2 share of 1 x 132096
])
def test_plan_split_counts(kw, splits):
    p = plan(**kw)
    assert p.num_splits == splits
    assert p.kind == (2 if p.problem.window else 1)
    assert p.group_size == p.problem.num_q_heads // p.problem.num_kv_heads
    off, total = expected_workspace(p.problem.batch, p.problem.num_q_heads, splits,
                                    p.problem.head_dim, p.problem.q_len)
    assert p.partial_lse_offset == off and p.workspace_bytes == total
    rows = p.problem.batch * max(1, p.problem.q_len) * p.problem.num_q_heads
    assert p.layer_workspace_bytes == (total if splits > 1 else -(-rows * 4 // 256) * 256)
    assert p.magic == binding.PLAN_MAGIC


def test_plan_long_context_split_counts_meet_chunk_rules():
    # 32K global layer, batch 4: 16-64 chunks per sequence; 128K batch 1: >= 128 chunks; 64K batch
    # 2: >= 128 chunks in the launch (64 per sequence)
    assert 16 <= plan().num_splits <= 64
    assert plan(batch=1, max_pages_per_seq=8256, num_pages=16384,
                max_ctx_len=132096).num_splits >= 128
    assert 2 * plan(batch=2, max_pages_per_seq=4160, num_pages=16384,
                    max_ctx_len=66560).num_splits >= 128


def test_plan_values_are_keys_doubles_the_workgroups():
    assert plan(values_are_keys=True).num_splits == 64
    assert plan(batch=1, max_pages_per_seq=8256, num_pages=16384, max_ctx_len=132096,
                values_are_keys=True).num_splits == 256
    prob = binding.Problem(4, 16, 2, 512, 16, 2112, 16896, 33792, 0, 256, 0, 0, 2, 0, 0)
    out = binding.Plan()
    assert binding.load_library().decode_attn_plan(ctypes.byref(prob), ctypes.byref(out)) == \
        ERR_SHAPE


def test_values_are_keys_plan_needs_one_pool(lib):
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600, values_are_keys=True)
    assert call_global(lib, p, k=A, v=A + 4096) == ERR_SHAPE


def test_plan_force_and_cap():
    assert plan(force_splits=7).num_splits == 7
    assert plan(max_splits=5).num_splits == 5
    assert plan(batch=1, max_ctx_len=16, max_pages_per_seq=1).num_splits == 1


@pytest.mark.parametrize("kw,status", [
    (dict(num_q_heads=15), ERR_SHAPE),           # Hq % Hkv
    (dict(batch=0), ERR_SHAPE),
    (dict(num_pages=0), ERR_SHAPE),
    (dict(window=-1), ERR_SHAPE),
    (dict(window=64, sink=-1), ERR_SHAPE),
    (dict(q_len=-1), ERR_SHAPE),
    (dict(q_len=8193), ERR_SHAPE),
    (dict(num_q_heads=65536 * 2, num_kv_heads=2), ERR_SHAPE),  # heads past a grid dimension
    (dict(batch=4096, q_len=16), ERR_SHAPE),     # 65536 (sequence, token) pairs
    (dict(force_splits=1025), ERR_SHAPE),
    (dict(max_splits=2000), ERR_SHAPE),
    (dict(head_dim=128), ERR_UNSUPPORTED),
    (dict(num_q_heads=6), ERR_UNSUPPORTED),      # G = 3
    (dict(num_q_heads=64), ERR_UNSUPPORTED),     # G = 32
    (dict(page_size=24), ERR_UNSUPPORTED),
    (dict(page_size=8), ERR_UNSUPPORTED),
    (dict(page_size=2048, max_pages_per_seq=8), ERR_UNSUPPORTED),
])
def test_plan_rejects(kw, status):
    with pytest.raises(binding.DecodeAttnError) as e:
        plan(**kw)
    assert e.value.status == status


def test_plan_null_pointers(lib):
    assert lib.decode_attn_plan(None, None) == ERR_NULL


# Fake, aligned, never-dereferenced addresses: every call below must fail validation first.
A = 1 << 20


def call_global(lib, p, q=A, k=A, v=A, bt=A, ctx=A, batch=1, scale=0.1, out=A, lse=None, ws=A,
                wsb=None):
    wsb = p.workspace_bytes if wsb is None else wsb
    return lib.decode_attn_global(ctypes.byref(p), q, k, v, bt, ctx, batch, scale, out, lse, ws,
                                  wsb, None)


def test_entry_validation_before_launch(lib):
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600)
    assert call_global(lib, p, q=None) == ERR_NULL
    assert call_global(lib, p, out=None) == ERR_NULL
    assert call_global(lib, p, ws=None) == ERR_NULL
    assert call_global(lib, p, q=A + 8) == ERR_ALIGN
    assert call_global(lib, p, k=A + 2) == ERR_ALIGN
    assert call_global(lib, p, out=A + 4) == ERR_ALIGN
    assert call_global(lib, p, bt=A + 1) == ERR_ALIGN
    assert call_global(lib, p, wsb=p.workspace_bytes - 1) == ERR_WORKSPACE
    assert call_global(lib, p, batch=3) == ERR_SHAPE
    assert call_global(lib, p, batch=-1) == ERR_SHAPE
    assert call_global(lib, p, scale=math.nan) == ERR_SHAPE
    assert call_global(lib, p, scale=math.inf) == ERR_SHAPE
    # batch 0 is a no-op: no pointer is needed and nothing is launched
    assert call_global(lib, p, q=None, k=None, v=None, bt=None, ctx=None, out=None, ws=None,
                       wsb=0, batch=0) == OK


def test_one_split_layer_call_needs_only_the_lse_plane(lib):
    """A one-split plan (a prefill chunk) asks the layer calls for the [B, L, Hq] lse plane only,
    and the stage calls still for the whole partial buffer."""
    p = plan(batch=1, q_len=8192, max_pages_per_seq=600, max_ctx_len=9000)
    assert p.num_splits == 1
    rows = 1 * 8192 * 16
    assert p.layer_workspace_bytes == rows * 4 < p.workspace_bytes // 100
    assert call_global(lib, p, wsb=p.layer_workspace_bytes - 1) == ERR_WORKSPACE
    assert lib.decode_attn_stage1(ctypes.byref(p), A, A, A, A, A, 1, 0.1, A,
                                  p.layer_workspace_bytes, None) == ERR_WORKSPACE
    bad = binding.Plan.from_buffer_copy(p)
    bad.layer_workspace_bytes -= 256
    assert call_global(lib, bad) == ERR_PLAN


def test_noalloc_rejects_before_touching_the_device(lib):
    """The allocation-free layer call checks the plan, the window and the scratch limit before it
    looks up its device array."""
    f = lib.decode_attn_layer_noalloc
    args = (A, A, A, A, A, 1)
    big = plan(force_splits=1024)  # 4 x 16 heads x 1024 splits x 513 x 4 B > 64 MiB
    assert big.layer_workspace_bytes > binding.NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), *args, 0, 0.1, A, None, None) == ERR_WORKSPACE
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600)
    assert f(None, *args, 0, 0.1, A, None, None) == ERR_NULL
    assert f(ctypes.byref(p), *args, 1024, 0.1, A, None, None) == ERR_SHAPE  # global plan
    bad = binding.Plan.from_buffer_copy(p)
    bad.magic = 0
    assert f(ctypes.byref(bad), *args, 0, 0.1, A, None, None) == ERR_PLAN
    assert f(ctypes.byref(p), A, A, A, A, A, 0, 0, 0.1, A, None, None) == OK  # batch 0: no-op
    s = plan(batch=2, num_kv_heads=8, head_dim=256, window=1024, max_pages_per_seq=100,
             max_ctx_len=1600)
    assert f(ctypes.byref(s), *args, 512, 0.1, A, None, None) == ERR_SHAPE


def test_prepared_call_checks_once_and_reports_status(lib):
    """A prepared call converts its arguments once and reports the library's status when called."""
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600)
    ok = binding.decode_attn_global(p, A, A, A, A, A, 0, 0.1, A, None, A, p.workspace_bytes,
                                    prepare=True)
    assert isinstance(ok, binding.PreparedCall)
    ok()  # batch 0: nothing launched
    ok()
    bad = binding.decode_attn_global(p, None, A, A, A, A, 1, 0.1, A, None, A, p.workspace_bytes,
                                     prepare=True)
    with pytest.raises(binding.DecodeAttnError) as e:
        bad()
    assert e.value.status == ERR_NULL
    s = plan(batch=2, num_kv_heads=8, head_dim=256, window=1024, max_pages_per_seq=100,
             max_ctx_len=1600)
    wrong = binding.decode_attn_sliding(s, A, A, A, A, A, 1, 512, 0.1, A, None, A,
                                        s.workspace_bytes, prepare=True)
    with pytest.raises(binding.DecodeAttnError) as e:
        wrong()
    assert e.value.status == ERR_SHAPE


def test_plan_tampering_and_kind(lib):
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600)
    bad = binding.Plan.from_buffer_copy(p)
    bad.magic = 0
    assert call_global(lib, bad) == ERR_PLAN
    bad = binding.Plan.from_buffer_copy(p)
    bad.num_splits += 1                        # workspace no longer matches
    assert call_global(lib, bad) == ERR_PLAN
    bad = binding.Plan.from_buffer_copy(p)
    bad.problem.head_dim = 384
    assert call_global(lib, bad) == ERR_PLAN
    assert lib.decode_attn_global(None, A, A, A, A, A, 1, 0.1, A, None, A, 1 << 30, None) == \
        ERR_NULL
    s = plan(batch=2, num_kv_heads=8, head_dim=256, window=1024, max_pages_per_seq=100,
             max_ctx_len=1600)
    assert call_global(lib, s) == ERR_PLAN     # sliding plan on the global entry point
    args = (A, A, A, A, A, 1)
    assert lib.decode_attn_sliding(ctypes.byref(p), *args, 1024, 0.1, A, None, A,
                                   p.workspace_bytes, None) == ERR_PLAN
    assert lib.decode_attn_sliding(ctypes.byref(s), *args, 512, 0.1, A, None, A,
                                   s.workspace_bytes, None) == ERR_SHAPE


def test_stage_entry_validation(lib):
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600)
    assert lib.decode_attn_stage1(ctypes.byref(p), A, A, A, A, A, 1, 0.1, None, 0, None) == \
        ERR_NULL
    assert lib.decode_attn_stage1(ctypes.byref(p), A, A, A, A, A, 1, 0.1, A, 16, None) == \
        ERR_WORKSPACE
    assert lib.decode_attn_stage2(ctypes.byref(p), 1, A, p.workspace_bytes, None, None, None) == \
        ERR_NULL
    assert lib.decode_attn_stage2(ctypes.byref(p), 1, A, p.workspace_bytes, A, A + 2, None) == \
        ERR_ALIGN
    assert lib.decode_attn_stage2(ctypes.byref(p), 0, None, 0, None, None, None) == OK


def test_append_validation(lib):
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600)
    bp = ctypes.byref(p)
    assert lib.decode_attn_append_kv(bp, None, A, A, A, A, A, 1, None) == ERR_NULL
    assert lib.decode_attn_append_kv(bp, A, None, A, A + 64, A, A, 1, None) == ERR_NULL
    assert lib.decode_attn_append_kv(bp, A + 2, A, A, A + 64, A, A, 1, None) == ERR_ALIGN
    assert lib.decode_attn_append_kv(bp, A, A, A, A + 64, A, A, 3, None) == ERR_SHAPE
    assert lib.decode_attn_append_kv(bp, None, None, None, None, None, None, 0, None) == OK
    bad = binding.Plan.from_buffer_copy(p)
    bad.magic = 1
    assert lib.decode_attn_append_kv(ctypes.byref(bad), A, A, A, A + 64, A, A, 1, None) == \
        ERR_PLAN


def test_rope_entry_validation(lib):
    """decode_attn_rope_cache and decode_attn_append_kv_rope reject bad arguments on the host."""
    c = lib.decode_attn_rope_cache
    assert c(None, 16, 64, 0, 1e4, None) == ERR_NULL
    assert c(A + 2, 16, 64, 0, 1e4, None) == ERR_ALIGN
    for mp, r, fd, th in ((0, 64, 0, 1e4), (16, 63, 0, 1e4), (16, 0, 0, 1e4), (16, 64, -1, 1e4),
                          (16, 64, 0, 0.0), (16, 64, 0, -5.0), (16, 64, 0, math.inf),
                          (16, 64, 0, math.nan)):
        assert c(A, mp, r, fd, th, None) == ERR_SHAPE, (mp, r, fd, th)
    p = plan(batch=2, max_pages_per_seq=100, max_ctx_len=1600)
    bp = ctypes.byref(p)
    f = lib.decode_attn_append_kv_rope

    def call(**kw):
        a = dict(q=A, q_out=A, k_new=A, v_new=A, k_pool=A, v_pool=A + 64, bt=A, ctx=A, batch=1,
                 cs=A, max_pos=4096, rot=512, inter=0, flags=3, qw=A, kw=A, vw=A, eps=1e-6)
        a.update(kw)
        return f(bp, a["q"], a["q_out"], a["k_new"], a["v_new"], a["k_pool"], a["v_pool"], a["bt"],
                 a["ctx"], a["batch"], a["cs"], a["max_pos"], a["rot"], a["inter"], a["flags"],
                 a["qw"], a["kw"], a["vw"], a["eps"], None)

    assert call(batch=3) == ERR_SHAPE
    assert call(batch=-1) == ERR_SHAPE
    assert call(rot=513) == ERR_SHAPE      # odd
    assert call(rot=514) == ERR_SHAPE      # past D
    assert call(rot=-2) == ERR_SHAPE
    assert call(max_pos=0) == ERR_SHAPE
    assert call(inter=2) == ERR_SHAPE
    assert call(flags=4) == ERR_SHAPE
    assert call(eps=0.0) == ERR_SHAPE
    assert call(eps=math.nan) == ERR_SHAPE
    assert call(batch=0) == OK             # nothing to do, nothing launched
    assert call(q=None) == ERR_NULL
    assert call(q_out=None) == ERR_NULL
    assert call(k_new=None) == ERR_NULL
    assert call(v_new=None) == ERR_NULL    # separate pools need v_new
    assert call(cs=None) == ERR_NULL       # a rotation needs the table
    assert call(bt=None) == ERR_NULL
    assert call(q_out=A + 2) == ERR_ALIGN
    assert call(v_new=A + 8) == ERR_ALIGN
    assert call(cs=A + 2) == ERR_ALIGN
    assert call(kw=A + 1) == ERR_ALIGN
    bad = binding.Plan.from_buffer_copy(p)
    bad.magic = 1
    assert f(ctypes.byref(bad), A, A, A, A, A, A + 64, A, A, 1, A, 16, 64, 0, 0, None, None, None,
             1e-6, None) == ERR_PLAN


def test_status_strings(lib):
    for code in range(8):
        assert binding.decode_attn_status_str(code).startswith(binding.STATUS_NAMES[code])
    assert "unknown" in binding.decode_attn_status_str(99)
    assert binding.decode_attn_version() == binding.ABI_VERSION == 300


def test_binding_rejects_tensors_smaller_than_the_plan():
    """The C side takes raw pointers and cannot see tensor sizes; the binding checks element
    counts against the plan before anything reaches the library (CPU tensors suffice: the size
    check runs first)."""
    import torch
    p = plan(batch=2, max_pages_per_seq=8, num_pages=16, max_ctx_len=128, q_len=3)
    L, Hq, Hkv, D, S = 3, 16, 2, 512, 16
    q = torch.zeros((2, L, Hq, D), dtype=torch.bfloat16)
    pool = torch.zeros((16, Hkv, S, D), dtype=torch.bfloat16)
    bt = torch.zeros((2, 8), dtype=torch.int32)
    ctx = torch.zeros((2,), dtype=torch.int32)
    out = torch.zeros((2, L, Hq, D))
    short = dict(q=q[:, :2].contiguous(), k_pool=pool[:15].contiguous(), block_table=bt[:, :7],
                 ctx_lens=ctx[:1], out=out[:1])
    for name, bad in short.items():
        args = dict(q=q, k_pool=pool, v_pool=pool, block_table=bt, ctx_lens=ctx, out=out)
        args[name] = bad
        with pytest.raises(ValueError, match=name):
            binding.decode_attn_global(p, args["q"], args["k_pool"], args["v_pool"],
                                       args["block_table"], args["ctx_lens"], 2, 0.1,
                                       args["out"])
    with pytest.raises(ValueError, match="lse_out"):
        binding.decode_attn_global(p, q, pool, pool, bt, ctx, 2, 0.1, out,
                                   torch.zeros((2, L, Hq - 1)))
    with pytest.raises(ValueError, match="k_new"):
        binding.decode_attn_append_kv(p, torch.zeros((2, L - 1, Hkv, D), dtype=torch.bfloat16),
                                      None, pool, pool, bt, ctx, 2)
    # a smaller batch needs fewer elements: passes the size check, then fails as a host tensor
    with pytest.raises(ValueError, match="device memory"):
        binding.decode_attn_global(p, q[:1].contiguous(), pool, pool, bt[:1], ctx[:1], 1, 0.1,
                                   out[:1])
