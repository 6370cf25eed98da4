"""fp64 CPU oracle for paged GQA single-token decode attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()`` and by the
CPU-baseline leg of ``bench.py``. The product package never imports it, and it imports nothing from
the product package. The arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over (b, h));
this module only builds/loads it and marshals numpy arrays.

Definition (see ``oracle.c`` for the citations): for sequence ``b``, query head ``h``, KV head
``g = h // G``, keys ``t`` in ``[lo, n)`` gathered from page ``block_table[b, t // S]``, slot
``t % S``::

    s_t = scale * <q[b, h], K_t>,   out = sum_t softmax(s)_t V_t,   lse = logsumexp(s)

with ``lo = 0`` for a global layer and ``max(0, n - W)`` for a sliding window of ``W`` keys.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc (fp64, no fast-math, OpenMP)."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    i32, f64, vp = ctypes.c_int32, ctypes.c_double, ctypes.c_void_p
    lib.oracle_decode_attn_ranges.argtypes = [i32] * 7 + [vp] * 6 + [f64, vp, vp, i32]
    lib.oracle_decode_attn_ranges.restype = ctypes.c_int
    lib.oracle_decode_attn.argtypes = [i32] * 7 + [vp] * 5 + [i32, f64, vp, vp, i32]
    lib.oracle_decode_attn.restype = ctypes.c_int
    lib.oracle_lse_merge.argtypes = [i32, i32, i32, vp, vp, vp, vp]
    lib.oracle_lse_merge.restype = ctypes.c_int
    lib.oracle_key_range.argtypes = [i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.oracle_key_range.restype = None
    lib.oracle_decode_attn_sink.argtypes = [i32] * 7 + [vp] * 5 + [i32, i32, f64, vp, vp, i32]
    lib.oracle_decode_attn_sink.restype = ctypes.c_int
    lib.oracle_decode_attn_multi.argtypes = [i32] * 8 + [vp] * 5 + [i32, i32, f64, vp, vp, i32]
    lib.oracle_decode_attn_multi.restype = ctypes.c_int
    lib.oracle_append_kv.argtypes = [i32] * 7 + [vp] * 6
    lib.oracle_append_kv.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns, got %s" % a.dtype)
    return a


def _check_shapes(q, k_pool, v_pool, block_table):
    if q.ndim != 3 or k_pool.ndim != 4 or k_pool.shape != v_pool.shape or block_table.ndim != 2:
        raise ValueError("expected q[B,Hq,D], pools[P,Hkv,S,D], block_table[B,M]")
    B, Hq, D = q.shape
    P, Hkv, S, D2 = k_pool.shape
    if D2 != D or block_table.shape[0] != B or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes q%s pool%s table%s" % (q.shape, k_pool.shape,
                                                                      block_table.shape))
    return B, Hq, Hkv, D, S, P, block_table.shape[1]


def key_range(n: int, window: int) -> tuple[int, int]:
    """Key range ``[lo, hi)`` attended by a sequence of ``n`` cached keys (window 0 = all)."""
    lib = _load()
    lo, hi = ctypes.c_int32(), ctypes.c_int32()
    lib.oracle_key_range(int(n), int(window), ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


def decode_attn(q, k_pool, v_pool, block_table, ctx_lens, scale, window=0, num_threads=0):
    """Oracle output ``(out[B,Hq,D] fp64, lse[B,Hq] fp64)`` of a global (window 0) or sliding layer."""
    lib = _load()
    q, k_pool, v_pool = _bits(q), _bits(k_pool), _bits(v_pool)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, Hq, Hkv, D, S, P, M = _check_shapes(q, k_pool, v_pool, block_table)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    rc = lib.oracle_decode_attn(B, Hq, Hkv, D, S, M, P, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_table), _ptr(ctx_lens), int(window), float(scale),
                                _ptr(out), _ptr(lse), int(num_threads))
    if rc != 0:
        raise ValueError("oracle_decode_attn failed with code %d" % rc)
    return out, lse


def decode_attn_sink(q, k_pool, v_pool, block_table, ctx_lens, scale, window, sink,
                     num_threads=0):
    """Oracle output of a sliding layer that also attends the first ``sink`` keys."""
    lib = _load()
    q, k_pool, v_pool = _bits(q), _bits(k_pool), _bits(v_pool)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    B, Hq, Hkv, D, S, P, M = _check_shapes(q, k_pool, v_pool, block_table)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    rc = lib.oracle_decode_attn_sink(B, Hq, Hkv, D, S, M, P, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                     _ptr(block_table), _ptr(ctx_lens), int(window), int(sink),
                                     float(scale), _ptr(out), _ptr(lse), int(num_threads))
    if rc != 0:
        raise ValueError("oracle_decode_attn_sink failed with code %d" % rc)
    return out, lse


def decode_attn_multi(q, k_pool, v_pool, block_table, ctx_lens, scale, window=0, sink=0,
                      num_threads=0):
    """Oracle output ``(out[B,L,Hq,D], lse[B,L,Hq])`` of L new tokens per sequence (``q`` is
    [B, L, Hq, D]); query i sits at position ctx_lens[b] - L + i and attends causally."""
    lib = _load()
    q, k_pool, v_pool = _bits(q), _bits(k_pool), _bits(v_pool)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    if q.ndim != 4:
        raise ValueError("q must be [B, L, Hq, D]")
    B, L, Hq, D = q.shape
    _, _, Hkv, _, S, P, M = _check_shapes(q[:, 0], k_pool, v_pool, block_table)
    out = np.zeros((B, L, Hq, D), dtype=np.float64)
    lse = np.zeros((B, L, Hq), dtype=np.float64)
    rc = lib.oracle_decode_attn_multi(B, L, Hq, Hkv, D, S, M, P, _ptr(q), _ptr(k_pool),
                                      _ptr(v_pool), _ptr(block_table), _ptr(ctx_lens), int(window),
                                      int(sink), float(scale), _ptr(out), _ptr(lse),
                                      int(num_threads))
    if rc != 0:
        raise ValueError("oracle_decode_attn_multi failed with code %d" % rc)
    return out, lse


def decode_attn_ranges(q, k_pool, v_pool, block_table, key_lo, key_hi, scale, num_threads=0):
    """Oracle output over explicit per-sequence key ranges ``[key_lo[b], key_hi[b])``."""
    lib = _load()
    q, k_pool, v_pool = _bits(q), _bits(k_pool), _bits(v_pool)
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    key_lo = np.ascontiguousarray(key_lo, dtype=np.int32)
    key_hi = np.ascontiguousarray(key_hi, dtype=np.int32)
    B, Hq, Hkv, D, S, P, M = _check_shapes(q, k_pool, v_pool, block_table)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    rc = lib.oracle_decode_attn_ranges(B, Hq, Hkv, D, S, M, P, _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(block_table), _ptr(key_lo), _ptr(key_hi), float(scale),
                                       _ptr(out), _ptr(lse), int(num_threads))
    if rc != 0:
        raise ValueError("oracle_decode_attn_ranges failed with code %d" % rc)
    return out, lse


def lse_merge(o_parts, lses):
    """Merge partials ``o_parts[R, splits, D]`` with log-sum-exps ``lses[R, splits]``."""
    lib = _load()
    o_parts = np.ascontiguousarray(o_parts, dtype=np.float64)
    lses = np.ascontiguousarray(lses, dtype=np.float64)
    R, splits, D = o_parts.shape
    if lses.shape != (R, splits):
        raise ValueError("lses must be [R, splits]")
    out = np.zeros((R, D), dtype=np.float64)
    lse = np.zeros((R,), dtype=np.float64)
    rc = lib.oracle_lse_merge(R, splits, D, _ptr(o_parts), _ptr(lses), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_lse_merge failed with code %d" % rc)
    return out, lse


def append_kv(k_new, v_new, k_pool, v_pool, block_table, ctx_lens):
    """Write each sequence's newest token (position ctx_lens[b] - 1) into the pools, in place;
    ``k_new`` [B, Hkv, D], or [B, L, Hkv, D] for the L newest tokens (positions n - L .. n - 1).
    ``v_pool is k_pool`` writes K only (layers whose values are their keys)."""
    lib = _load()
    same = v_pool is k_pool
    for a in (k_new, k_pool) + (() if same else (v_new, v_pool)):
        if a.dtype != np.uint16 or not a.flags.c_contiguous:
            raise TypeError("bf16 bit patterns (uint16), C-contiguous, expected")
    block_table = np.ascontiguousarray(block_table, dtype=np.int32)
    ctx_lens = np.ascontiguousarray(ctx_lens, dtype=np.int32)
    if k_new.ndim == 3:
        B, Hkv, D = k_new.shape
        L = 1
    else:
        B, L, Hkv, D = k_new.shape
    if not same and v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new differ in shape")
    P, Hkv2, S, D2 = k_pool.shape
    if Hkv2 != Hkv or D2 != D or block_table.shape[0] != B:
        raise ValueError("inconsistent shapes")
    rc = lib.oracle_append_kv(B, L, Hkv, D, S, block_table.shape[1], P, _ptr(k_new),
                              _ptr(k_new if same else v_new), _ptr(k_pool),
                              _ptr(k_pool if same else v_pool), _ptr(block_table), _ptr(ctx_lens))
    if rc != 0:
        raise ValueError("oracle_append_kv failed with code %d" % rc)


def max_threads() -> int:
    """Threads the oracle's OpenMP runtime uses by default."""
    return int(_load().oracle_max_threads())
