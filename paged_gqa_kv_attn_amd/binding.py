"""ctypes binding of ``libdecode_attn.so`` (declared in ``include/decode_attn.h``).

Argument marshalling only: every step of decode attention runs in the library's HIP kernels.
Device buffers are passed either as torch CUDA tensors (their ``data_ptr()``) or as raw integer
device addresses; the stream defaults to torch's current stream. A nonzero status from the
library raises :class:`DecodeAttnError`. The library is loaded on first use; if it has not been
built (``python -c "import __graft_entry__ as g; g.build()"``) loading raises, there is no fallback.

Every call function also takes ``prepare=True``: it then checks and converts its arguments once
and returns a :class:`PreparedCall`, which a serving loop calls with one ctypes call and no torch
queries (about 1 us of host time instead of about 9).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libdecode_attn.so"
_lib = None

PLAN_MAGIC = 0x44415431  # "DAT1", set by decode_attn_plan

STATUS_NAMES = {
    0: "DECODE_ATTN_OK",
    1: "DECODE_ATTN_ERR_NULL",
    2: "DECODE_ATTN_ERR_SHAPE",
    3: "DECODE_ATTN_ERR_UNSUPPORTED",
    4: "DECODE_ATTN_ERR_WORKSPACE",
    5: "DECODE_ATTN_ERR_PLAN",
    6: "DECODE_ATTN_ERR_HIP",
    7: "DECODE_ATTN_ERR_ALIGN",
}


class DecodeAttnError(RuntimeError):
    """A nonzero decode_attn_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__("%s: %s (%d)" % (where, STATUS_NAMES.get(self.status, "unknown"),
                                          self.status))


class Problem(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "max_pages_per_seq",
        "num_pages", "max_ctx_len", "window", "num_cus", "max_splits", "force_splits",
        "values_are_keys", "sink", "q_len")]


class Plan(ctypes.Structure):
    _fields_ = [
        ("problem", Problem),
        ("num_splits", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_uint64),
        ("partial_lse_offset", ctypes.c_uint64),
        ("magic", ctypes.c_uint32),
        ("reserved0", ctypes.c_int32),
        ("layer_workspace_bytes", ctypes.c_uint64),
        ("reserved", ctypes.c_int32 * 4),
    ]

    def __repr__(self):
        p = self.problem
        return ("Plan(kind=%s, B=%d, Hq=%d, Hkv=%d, D=%d, S=%d, window=%d, num_splits=%d, "
                "chunk_tokens=%d, workspace_bytes=%d)" % (
                    {1: "global", 2: "sliding"}.get(self.kind, "?"), p.batch, p.num_q_heads,
                    p.num_kv_heads, p.head_dim, p.page_size, p.window, self.num_splits,
                    self.chunk_tokens, self.workspace_bytes))


def library_path() -> str:
    """The in-tree library, or the file named by PAGED_GQA_KV_ATTN_LIB (for A/B builds)."""
    return os.environ.get("PAGED_GQA_KV_ATTN_LIB") or os.path.join(_HERE, _LIB_NAME)


# decode_attn_version() of the library whose struct layouts Problem and Plan mirror.
ABI_VERSION = 300


def load_library():
    """Load ``libdecode_attn.so`` from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError("%s is not built; run __graft_entry__.build() first" % path)
    # PyTorch ships its own HIP runtime. Loading torch first makes the dynamic linker resolve this
    # library's libamdhip64.so.7 to that same runtime, so torch's streams, events and device memory
    # and this library's launches belong to one runtime (loading this library first would map a
    # second HIP/HSA runtime into the process).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    _check_single_runtime()
    vp, i32, u64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64, ctypes.c_float
    pplan = ctypes.POINTER(Plan)
    lib.decode_attn_plan.argtypes = [ctypes.POINTER(Problem), pplan]
    lib.decode_attn_global.argtypes = [pplan, vp, vp, vp, vp, vp, i32, f32, vp, vp, vp, u64, vp]
    lib.decode_attn_sliding.argtypes = [pplan, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp, vp, u64,
                                        vp]
    lib.decode_attn_stage1.argtypes = [pplan, vp, vp, vp, vp, vp, i32, f32, vp, u64, vp]
    lib.decode_attn_stage2.argtypes = [pplan, i32, vp, u64, vp, vp, vp]
    lib.decode_attn_append_kv.argtypes = [pplan, vp, vp, vp, vp, vp, vp, i32, vp]
    lib.decode_attn_rope_cache.argtypes = [vp, i32, i32, i32, ctypes.c_double, vp]
    lib.decode_attn_append_kv_rope.argtypes = [pplan, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32,
                                               i32, i32, i32, vp, vp, vp, f32, vp]
    lib.decode_attn_layer_noalloc.argtypes = [pplan, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp,
                                              vp]
    for fn in ("decode_attn_plan", "decode_attn_global", "decode_attn_sliding",
               "decode_attn_stage1", "decode_attn_stage2", "decode_attn_append_kv",
               "decode_attn_rope_cache", "decode_attn_append_kv_rope",
               "decode_attn_layer_noalloc"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.decode_attn_status_str.argtypes = [ctypes.c_int]
    lib.decode_attn_status_str.restype = ctypes.c_char_p
    lib.decode_attn_version.argtypes = []
    lib.decode_attn_version.restype = ctypes.c_int
    if lib.decode_attn_version() != ABI_VERSION:
        raise RuntimeError("%s reports version %d; this binding's structs match version %d "
                           "(rebuild the library)" % (path, lib.decode_attn_version(), ABI_VERSION))
    _lib = lib
    return lib


def _check_single_runtime() -> None:
    """Raise if more than one HIP runtime is mapped into this process."""
    try:
        with open("/proc/self/maps") as f:
            libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    if len(libs) > 1:
        raise RuntimeError("two HIP runtimes are loaded (%s); import torch before loading %s"
                           % (sorted(libs), _LIB_NAME))


def _check(status: int, where: str) -> None:
    if status != 0:
        raise DecodeAttnError(status, where)


_raw_lib = None


def _raw(name: str):
    """The library function without ctypes argument conversion (for prepared calls, whose
    arguments are ctypes values already)."""
    global _raw_lib
    if _raw_lib is None:
        _raw_lib = ctypes.CDLL(library_path())
    return getattr(_raw_lib, name)


class PreparedCall:
    """One library call whose arguments were checked and converted once: calling it makes a
    single ctypes call with no torch queries. It keeps the tensors it was made from alive. The
    device addresses, the batch and the stream are fixed at preparation; what the kernels read
    from device memory (q, the pools, block tables, lengths) may change between calls, as in
    HIP-graph replay. Made by passing ``prepare=True`` to a call function."""

    __slots__ = ("name", "_fn", "_args", "_keep")

    def __init__(self, fn, name, args, keep):
        self.name = name
        self._keep = keep
        types = fn.argtypes
        conv = []
        for t, a in zip(types, args):
            if isinstance(a, ctypes._SimpleCData) or type(a).__name__ == "CArgObject":
                conv.append(a)
            elif t is ctypes.c_void_p:
                conv.append(ctypes.c_void_p(a))
            else:
                conv.append(t(a))
        self._args = tuple(conv)
        self._fn = _raw(name)

    def __call__(self) -> None:
        status = self._fn(*self._args)
        if status != 0:
            raise DecodeAttnError(status, self.name)


def _keep(scope: dict):
    """The tensors among a call's arguments (kept alive by a prepared call)."""
    return tuple(v for v in scope.values() if hasattr(v, "data_ptr"))


def _call(fn, name: str, prepare: bool, keep, *args):
    if prepare:
        return PreparedCall(fn, name, args, keep)
    _check(fn(*args), name)
    return None


def _dev_ptr(x, name: str, dtype=None, device: Optional[int] = None) -> Optional[int]:
    """Device address of a torch CUDA tensor (checked, on ``device`` when given) or a raw integer
    address; None -> NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError("%s must be a torch CUDA tensor or an integer device address" % name)
    if not x.is_cuda:
        raise ValueError("%s must live in device memory" % name)
    if device is not None and x.get_device() != device:
        raise ValueError("%s lives on cuda:%d; the call launches on the current device cuda:%d"
                         % (name, x.get_device(), device))
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and x.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, x.dtype))
    return x.data_ptr()


def _nbytes(x) -> int:
    return x.numel() * x.element_size()


def _need(x, name: str, elems: int) -> None:
    """Reject a tensor with fewer elements than the call reads or writes through it (integer
    addresses are passed through unchecked)."""
    if x is None or isinstance(x, int):
        return
    if x.numel() < elems:
        raise ValueError("%s holds %d elements, the call needs %d" % (name, x.numel(), elems))


def _check_sizes(plan, batch, q=None, k_pool=None, v_pool=None, block_table=None, ctx_lens=None,
                 out=None, lse_out=None) -> None:
    p = plan.problem
    L = max(1, p.q_len)
    rows = int(batch) * L * p.num_q_heads
    pool = p.num_pages * p.num_kv_heads * p.page_size * p.head_dim
    _need(q, "q", rows * p.head_dim)
    _need(k_pool, "k_pool", pool)
    _need(v_pool, "v_pool", pool)
    _need(block_table, "block_table", int(batch) * p.max_pages_per_seq)
    _need(ctx_lens, "ctx_lens", int(batch))
    _need(out, "out", rows * p.head_dim)
    _need(lse_out, "lse_out", rows)


def _current_device() -> Optional[int]:
    import torch
    return torch.cuda.current_device() if torch.cuda.is_available() else None


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream  # torch.cuda.Stream


def decode_attn_plan(batch, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_seq,
                     num_pages, max_ctx_len=0, window=0, num_cus=0, max_splits=0,
                     force_splits=0, values_are_keys=False, sink=0, q_len=0) -> Plan:
    """Host-only planning (see decode_attn_plan in the header). Returns the plan struct."""
    lib = load_library()
    prob = Problem(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(page_size),
                   int(max_pages_per_seq), int(num_pages), int(max_ctx_len), int(window),
                   int(num_cus), int(max_splits), int(force_splits), int(bool(values_are_keys)),
                   int(sink), int(q_len))
    plan = Plan()
    _check(lib.decode_attn_plan(ctypes.byref(prob), ctypes.byref(plan)), "decode_attn_plan")
    return plan


def _bf16():
    import torch
    return torch.bfloat16


def _i32():
    import torch
    return torch.int32


def _f32():
    import torch
    return torch.float32


def _ws(workspace, workspace_bytes, device=None):
    if workspace_bytes is None:
        raw = workspace is None or isinstance(workspace, int)
        workspace_bytes = 0 if raw else _nbytes(workspace)
    return _dev_ptr(workspace, "workspace", None, device), int(workspace_bytes)


def decode_attn_global(plan: Plan, q, k_pool, v_pool, block_table, ctx_lens, batch, scale, out,
                       lse_out=None, workspace=None, workspace_bytes=None, stream=None,
                       prepare=False) -> Optional[PreparedCall]:
    lib = load_library()
    dev = _current_device()
    _check_sizes(plan, batch, q, k_pool, v_pool, block_table, ctx_lens, out, lse_out)
    ws, wsb = _ws(workspace, workspace_bytes, dev)
    return _call(lib.decode_attn_global, "decode_attn_global", prepare, _keep(locals()),
        ctypes.byref(plan), _dev_ptr(q, "q", _bf16(), dev),
        _dev_ptr(k_pool, "k_pool", _bf16(), dev), _dev_ptr(v_pool, "v_pool", _bf16(), dev),
        _dev_ptr(block_table, "block_table", _i32(), dev),
        _dev_ptr(ctx_lens, "ctx_lens", _i32(), dev), int(batch), float(scale),
        _dev_ptr(out, "out", _f32(), dev), _dev_ptr(lse_out, "lse_out", _f32(), dev), ws, wsb,
        _stream_handle(stream))


def decode_attn_sliding(plan: Plan, q, k_pool, v_pool, block_table, ctx_lens, batch, window, scale,
                        out, lse_out=None, workspace=None, workspace_bytes=None,
                        stream=None, prepare=False) -> Optional[PreparedCall]:
    lib = load_library()
    dev = _current_device()
    _check_sizes(plan, batch, q, k_pool, v_pool, block_table, ctx_lens, out, lse_out)
    ws, wsb = _ws(workspace, workspace_bytes, dev)
    return _call(lib.decode_attn_sliding, "decode_attn_sliding", prepare, _keep(locals()),
        ctypes.byref(plan), _dev_ptr(q, "q", _bf16(), dev),
        _dev_ptr(k_pool, "k_pool", _bf16(), dev), _dev_ptr(v_pool, "v_pool", _bf16(), dev),
        _dev_ptr(block_table, "block_table", _i32(), dev),
        _dev_ptr(ctx_lens, "ctx_lens", _i32(), dev), int(batch), int(window), float(scale),
        _dev_ptr(out, "out", _f32(), dev), _dev_ptr(lse_out, "lse_out", _f32(), dev), ws, wsb,
        _stream_handle(stream))


NOALLOC_SCRATCH_BYTES = 64 << 20  # DECODE_ATTN_NOALLOC_SCRATCH_BYTES


def decode_attn_layer_noalloc(plan: Plan, q, k_pool, v_pool, block_table, ctx_lens, batch, window,
                              scale, out, lse_out=None, stream=None,
                              prepare=False) -> Optional[PreparedCall]:
    """The layer call (global for window 0, else sliding) with the partials in the library's
    static device array instead of a caller workspace: nothing is allocated. Calls that may
    overlap on one device share that array and must be ordered by the caller."""
    lib = load_library()
    dev = _current_device()
    _check_sizes(plan, batch, q, k_pool, v_pool, block_table, ctx_lens, out, lse_out)
    return _call(lib.decode_attn_layer_noalloc, "decode_attn_layer_noalloc", prepare,
                 _keep(locals()),
        ctypes.byref(plan), _dev_ptr(q, "q", _bf16(), dev),
        _dev_ptr(k_pool, "k_pool", _bf16(), dev), _dev_ptr(v_pool, "v_pool", _bf16(), dev),
        _dev_ptr(block_table, "block_table", _i32(), dev),
        _dev_ptr(ctx_lens, "ctx_lens", _i32(), dev), int(batch), int(window), float(scale),
        _dev_ptr(out, "out", _f32(), dev), _dev_ptr(lse_out, "lse_out", _f32(), dev),
        _stream_handle(stream))


def decode_attn_stage1(plan: Plan, q, k_pool, v_pool, block_table, ctx_lens, batch, scale,
                       workspace, workspace_bytes=None, stream=None,
                       prepare=False) -> Optional[PreparedCall]:
    lib = load_library()
    dev = _current_device()
    _check_sizes(plan, batch, q, k_pool, v_pool, block_table, ctx_lens)
    ws, wsb = _ws(workspace, workspace_bytes, dev)
    return _call(lib.decode_attn_stage1, "decode_attn_stage1", prepare, _keep(locals()),
        ctypes.byref(plan), _dev_ptr(q, "q", _bf16(), dev),
        _dev_ptr(k_pool, "k_pool", _bf16(), dev), _dev_ptr(v_pool, "v_pool", _bf16(), dev),
        _dev_ptr(block_table, "block_table", _i32(), dev),
        _dev_ptr(ctx_lens, "ctx_lens", _i32(), dev), int(batch), float(scale), ws, wsb,
        _stream_handle(stream))


def decode_attn_stage2(plan: Plan, batch, workspace, out, lse_out=None, workspace_bytes=None,
                       stream=None, prepare=False) -> Optional[PreparedCall]:
    lib = load_library()
    dev = _current_device()
    _check_sizes(plan, batch, out=out, lse_out=lse_out)
    ws, wsb = _ws(workspace, workspace_bytes, dev)
    return _call(lib.decode_attn_stage2, "decode_attn_stage2", prepare, _keep(locals()),
        ctypes.byref(plan), int(batch), ws, wsb, _dev_ptr(out, "out", _f32(), dev),
        _dev_ptr(lse_out, "lse_out", _f32(), dev), _stream_handle(stream))


def decode_attn_append_kv(plan: Plan, k_new, v_new, k_pool, v_pool, block_table, ctx_lens, batch,
                          stream=None, prepare=False) -> Optional[PreparedCall]:
    """Write each sequence's L = plan q_len newest K/V (positions ctx_lens[b] - L ..) into the
    pools. Passing the same tensor as k_pool and v_pool writes K only (v_new may be None)."""
    lib = load_library()
    dev = _current_device()
    p = plan.problem
    new = int(batch) * max(1, p.q_len) * p.num_kv_heads * p.head_dim
    _need(k_new, "k_new", new)
    if v_pool is not k_pool:
        _need(v_new, "v_new", new)
    _check_sizes(plan, batch, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                 ctx_lens=ctx_lens)
    return _call(lib.decode_attn_append_kv, "decode_attn_append_kv", prepare, _keep(locals()),
        ctypes.byref(plan), _dev_ptr(k_new, "k_new", _bf16(), dev),
        _dev_ptr(v_new, "v_new", _bf16(), dev),
        _dev_ptr(k_pool, "k_pool", _bf16(), dev), _dev_ptr(v_pool, "v_pool", _bf16(), dev),
        _dev_ptr(block_table, "block_table", _i32(), dev),
        _dev_ptr(ctx_lens, "ctx_lens", _i32(), dev),
        int(batch), _stream_handle(stream))


NORM_QK = 1  # RMSNorm q and the new k heads before the rotation
NORM_V = 2   # RMSNorm the new v heads


def decode_attn_rope_cache(cos_sin, max_position, rotary_dim, theta, freq_dim=0,
                           stream=None, prepare=False) -> Optional[PreparedCall]:
    """Fill cos_sin [max_position, rotary_dim] fp32 with cos(t f_j) then sin(t f_j), f_j =
    theta^(-2j / (freq_dim or rotary_dim)), computed on the device in double precision."""
    lib = load_library()
    dev = _current_device()
    _need(cos_sin, "cos_sin", int(max_position) * int(rotary_dim))
    return _call(lib.decode_attn_rope_cache, "decode_attn_rope_cache", prepare, _keep(locals()),
                 _dev_ptr(cos_sin, "cos_sin", _f32(), dev), int(max_position), int(rotary_dim),
                 int(freq_dim), float(theta), _stream_handle(stream))


def decode_attn_append_kv_rope(plan: Plan, q, q_out, k_new, v_new, k_pool, v_pool, block_table,
                               ctx_lens, batch, cos_sin, max_position, rotary_dim,
                               interleaved=False, norm_flags=0, q_norm_weight=None,
                               k_norm_weight=None, v_norm_weight=None, eps=1e-6,
                               stream=None, prepare=False) -> Optional[PreparedCall]:
    """QK-norm + RoPE of the new tokens' q (into q_out, which may be q) and k, and the paged append
    of k and v (v optionally normalised), in one launch. Passing the same tensor as k_pool and
    v_pool writes K only (v_new may be None)."""
    lib = load_library()
    dev = _current_device()
    p = plan.problem
    L = max(1, p.q_len)
    new = int(batch) * L * p.num_kv_heads * p.head_dim
    _need(q_out, "q_out", int(batch) * L * p.num_q_heads * p.head_dim)
    _need(k_new, "k_new", new)
    if v_pool is not k_pool:
        _need(v_new, "v_new", new)
    if int(rotary_dim) > 0:
        _need(cos_sin, "cos_sin", int(max_position) * int(rotary_dim))
    for w, name in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight"),
                    (v_norm_weight, "v_norm_weight")):
        _need(w, name, p.head_dim)
    _check_sizes(plan, batch, q=q, k_pool=k_pool, v_pool=v_pool, block_table=block_table,
                 ctx_lens=ctx_lens)
    return _call(lib.decode_attn_append_kv_rope, "decode_attn_append_kv_rope", prepare,
                 _keep(locals()),
        ctypes.byref(plan), _dev_ptr(q, "q", _bf16(), dev), _dev_ptr(q_out, "q_out", _bf16(), dev),
        _dev_ptr(k_new, "k_new", _bf16(), dev), _dev_ptr(v_new, "v_new", _bf16(), dev),
        _dev_ptr(k_pool, "k_pool", _bf16(), dev), _dev_ptr(v_pool, "v_pool", _bf16(), dev),
        _dev_ptr(block_table, "block_table", _i32(), dev),
        _dev_ptr(ctx_lens, "ctx_lens", _i32(), dev), int(batch),
        _dev_ptr(cos_sin, "cos_sin", _f32(), dev), int(max_position), int(rotary_dim),
        int(bool(interleaved)), int(norm_flags),
        _dev_ptr(q_norm_weight, "q_norm_weight", _f32(), dev),
        _dev_ptr(k_norm_weight, "k_norm_weight", _f32(), dev),
        _dev_ptr(v_norm_weight, "v_norm_weight", _f32(), dev), float(eps),
        _stream_handle(stream))


def decode_attn_status_str(status: int) -> str:
    return load_library().decode_attn_status_str(int(status)).decode()


def decode_attn_version() -> int:
    return int(load_library().decode_attn_version())
