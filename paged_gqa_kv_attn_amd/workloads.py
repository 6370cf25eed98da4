"""Seeded synthetic workloads for paged decode attention: shapes, page tables and bf16 values.

This module only draws inputs; it contains none of the attention arithmetic, so both the GPU
tests/benchmark and the CPU oracle can be fed from it. Everything is numpy on the host; values
are bf16 bit patterns in ``uint16`` arrays.

Workloads follow the serving shapes the pages measure (Gemma 4 26B-A4B decode at 1K to 128K
input tokens and batch 1 to 8: Sparse-vLLM PR #27 "feat: support Gemma 4 and native multimodal
inference", section "性能结果" / performance results) with the two Gemma-4 layer kinds (global,
head_dim 512; sliding window, head_dim 256: same page, section "Gemma 4 文本推理"). No dataset is
involved; these arrays stand in for the KV caches of those runs.

Structure:
* pool ``[P, Hkv, S, D]``; a sequence's pages are drawn at random (without replacement) from the
  pool, so logical neighbours are scattered physically;
* pool slots that hold no attended key (unused pages, the tail of a partial last page, keys before
  a sliding window) are filled with a quiet-NaN pattern when ``poison`` is set, so any stray read
  turns the output into NaN;
* sliding layers only keep the pages that intersect their window; block-table entries of older
  pages (and past the last page) are -1.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

BF16_QNAN = 0x7FC0  # quiet NaN bit pattern used to poison unused slots


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.asarray(x, dtype=np.float32)
    u = np.ascontiguousarray(x).view(np.uint32).reshape(x.shape)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    kind: str            # "global" or "sliding"
    num_q_heads: int     # Hq
    num_kv_heads: int    # Hkv
    head_dim: int        # D
    window: int = 0      # 0 for global layers
    q_mult: float = 1.0  # q ~ q_mult * N(0, 1)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                         # seed root of the workload
    batch: int
    ctx: Sequence[int] | str           # fixed lengths, or "ragged" (drawn, see ragged_ctx_lens)
    layers: Dict[str, LayerSpec]
    page_size: int = 16
    num_pages: Optional[int] = None    # pool pages; None = pool_factor * pages needed
    pool_factor: int = 2
    description: str = ""


def _global(hq: int, hkv: int, q_mult: float = 1.0) -> LayerSpec:
    return LayerSpec("global", hq, hkv, 512, 0, q_mult)


def _sliding(hq: int = 16, hkv: int = 8, q_mult: float = 1.0) -> LayerSpec:
    return LayerSpec("sliding", hq, hkv, 256, 1024, q_mult)


WORKLOADS: Dict[str, Workload] = {
    "tiny_global": Workload(
        "tiny_global", 0, 1, [1024], {"global": _global(4, 1)}, num_pages=128,
        description="batch 1, 4 q heads on 1 KV head, D 512, ctx 1024, 64 pages shuffled in a "
                    "128-page pool"),
    "short_batch": Workload(
        "short_batch", 1, 8, [1280] * 8, {"global": _global(16, 2), "sliding": _sliding()},
        description="batch 8, ctx 1280; global 16/2 heads D 512 and sliding 16/8 heads D 256, W 1024"),
    "ragged_batch": Workload(
        "ragged_batch", 2, 8, "ragged", {"global": _global(16, 2), "sliding": _sliding()},
        description="batch 8, ctx uniform in [3800, 4608] and never a multiple of 32; layers as "
                    "short_batch"),
    "long_ctx": Workload(
        "long_ctx", 3, 4, [32768 + 1024] * 4,
        {"global": _global(16, 2, q_mult=2.0), "sliding": _sliding(q_mult=2.0)},
        description="batch 4, ctx 33792; global D 512 GQA 8 and sliding D 256 W 1024; q ~ 2 N(0,1)"),
    "very_long_b1": Workload(
        "very_long_b1", 4, 1, [131072 + 1024], {"global": _global(16, 2)}, num_pages=16384,
        description="batch 1, ctx 132096, global 16/2 heads D 512, 16384-page pool"),
    "very_long_b2": Workload(
        "very_long_b2", 5, 2, [65536 + 1024] * 2, {"global": _global(16, 2)}, num_pages=16384,
        description="batch 2, ctx 66560, global 16/2 heads D 512, 16384-page pool"),
    # One GPU's share under 2-way tensor parallelism over KV heads: each GPU holds half the KV
    # heads, their query heads and their own pools; attention itself needs no exchange.
    "long_ctx_tp2": Workload(
        "long_ctx_tp2", 6, 4, [32768 + 1024] * 4,
        {"global": _global(8, 1, q_mult=2.0), "sliding": _sliding(8, 4, q_mult=2.0)},
        description="one GPU's share of long_ctx at 2-way KV-head tensor parallelism: batch 4, "
                    "ctx 33792; global 8/1 heads D 512 and sliding 8/4 heads D 256 W 1024"),
    "very_long_b1_tp2": Workload(
        "very_long_b1_tp2", 7, 1, [131072 + 1024], {"global": _global(8, 1)}, num_pages=16384,
        description="one GPU's share of very_long_b1 at 2-way KV-head tensor parallelism: "
                    "batch 1, ctx 132096, global 8/1 heads D 512, 16384-page pool"),
}


def ragged_ctx_lens(rng: np.random.Generator, batch: int, low: int = 3800,
                    high: int = 4608) -> np.ndarray:
    """Uniform integer lengths in [low, high], none a multiple of 32, at least one with a partial
    last page (n % 16 != 0) and one whose 1024-key window starts 16 keys past a 32-key boundary
    (n % 32 == 16). Draws again until these hold."""
    while True:
        n = rng.integers(low, high + 1, size=batch)
        while np.any(n % 32 == 0):
            bad = n % 32 == 0
            n[bad] = rng.integers(low, high + 1, size=int(bad.sum()))
        if np.any(n % 16 != 0) and np.any(n % 32 == 16):
            return n.astype(np.int32)


@dataclasses.dataclass
class LayerInputs:
    """Host arrays for one layer call."""
    q: np.ndarray            # uint16 [B, Hq, D], or [B, L, Hq, D] for L > 1 query tokens
    k_pool: np.ndarray       # uint16 [P, Hkv, S, D]
    v_pool: np.ndarray       # uint16 [P, Hkv, S, D]
    block_table: np.ndarray  # int32  [B, max_pages_per_seq]
    ctx_lens: np.ndarray     # int32  [B]
    scale: float
    window: int
    page_size: int
    sink: int = 0            # leading keys a sliding layer also attends
    q_len: int = 1           # query tokens per sequence

    @property
    def dims(self):
        B, Hq, D = (self.q.shape[0],) + self.q.shape[-2:]
        P, Hkv, S, _ = self.k_pool.shape
        return dict(B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, P=P, M=self.block_table.shape[1])


def attended_range(n: int, window: int) -> tuple[int, int]:
    """Keys [lo, n) a layer reads (used only to decide which pages to allocate and poison)."""
    return (max(0, n - window) if window > 0 else 0), n


def attended_spans(n: int, window: int, sink: int = 0) -> list[tuple[int, int]]:
    """Disjoint key spans a layer reads: [0, min(sink, lo)) for a sliding layer with sinks, then
    [lo, n). Used only to decide which pages to allocate and poison."""
    lo, hi = attended_range(n, window)
    sk = min(sink, lo) if window > 0 else 0
    return ([(0, sk)] if sk > 0 else []) + ([(lo, hi)] if hi > lo else [])


def make_layer_inputs(ctx_lens: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                      page_size: int = 16, window: int = 0, scale: Optional[float] = None,
                      num_pages: Optional[int] = None, pool_factor: int = 2, q_mult: float = 1.0,
                      seed=0, poison: bool = True, max_pages_per_seq: Optional[int] = None,
                      value_dist: str = "normal", sink: int = 0,
                      q_len: int = 1) -> LayerInputs:
    """Draw one layer's inputs. ``seed`` is anything ``np.random.SeedSequence`` accepts.

    Pages are allocated only for the logical pages holding attended keys; all other block-table
    entries are -1. ``value_dist`` "normal" draws N(0,1) values, "zero" leaves them 0. ``sink``
    (sliding layers) also attends the first ``sink`` keys of each sequence. ``q_len`` > 1 draws
    q as [B, L, Hq, D]: the last L cached keys are the new tokens, each query attending causally
    (so a window reaches L - 1 keys further back for the first of them)."""
    ctx = np.asarray(ctx_lens, dtype=np.int32)
    B, S, D = len(ctx), int(page_size), int(head_dim)
    ss = np.random.SeedSequence(seed)
    rq, rk, rv, rp = (np.random.default_rng(s) for s in ss.spawn(4))

    reach = window + q_len - 1 if window > 0 else 0
    spans = [attended_spans(int(n), reach, sink) for n in ctx]
    pages = [sorted({j for a, e in sp for j in range(a // S, (e - 1) // S + 1)}) for sp in spans]
    total = int(sum(len(pg) for pg in pages))
    P = int(num_pages) if num_pages is not None else max(1, pool_factor * total)
    if P < total:
        raise ValueError("pool of %d pages cannot hold %d pages" % (P, total))
    width = max_pages_per_seq or max(1, max((int(n) + S - 1) // S for n in ctx) if B else 1)

    perm = rp.permutation(P).astype(np.int32)
    table = np.full((B, width), -1, dtype=np.int32)
    logical = []  # (b, logical page) for each allocated page, in allocation order
    cursor = 0
    for b in range(B):
        for j in pages[b]:
            table[b, j] = perm[cursor]
            logical.append((b, j))
            cursor += 1
    used = perm[:total]

    fill = BF16_QNAN if poison else 0
    k_pool = np.full((P, num_kv_heads, S, D), fill, dtype=np.uint16)
    v_pool = np.full((P, num_kv_heads, S, D), fill, dtype=np.uint16)
    if total:
        shape = (total, num_kv_heads, S, D)
        if value_dist == "normal":
            k_pool[used] = f32_to_bf16_bits(rk.standard_normal(shape, dtype=np.float32))
            v_pool[used] = f32_to_bf16_bits(rv.standard_normal(shape, dtype=np.float32))
        elif value_dist == "zero":
            k_pool[used] = 0
            v_pool[used] = 0
        else:
            raise ValueError(value_dist)
        if poison:
            # Slots of allocated pages holding no attended key: before the window (or between
            # the sink keys and the window), after the last key.
            for (b, j), p in zip(logical, used):
                t0 = j * S
                if any(a <= t0 and t0 + S <= e for a, e in spans[b]):
                    continue
                t = np.arange(t0, t0 + S)
                keep = np.zeros(S, dtype=bool)
                for a, e in spans[b]:
                    keep |= (t >= a) & (t < e)
                k_pool[p, :, ~keep] = BF16_QNAN
                v_pool[p, :, ~keep] = BF16_QNAN

    q_shape = (B, num_q_heads, D) if q_len == 1 else (B, q_len, num_q_heads, D)
    q = f32_to_bf16_bits(np.float32(q_mult) * rq.standard_normal(q_shape, dtype=np.float32))
    return LayerInputs(q=q, k_pool=k_pool, v_pool=v_pool, block_table=table, ctx_lens=ctx,
                       scale=float(scale if scale is not None else 1.0 / math.sqrt(D)),
                       window=int(window), page_size=S, sink=int(sink) if window > 0 else 0,
                       q_len=int(q_len))


def make_new_tokens(batch: int, q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                    seed=0, scale: float = 3.0) -> dict:
    """Pre-norm q, k and v of a step's new tokens ([B, L, H, D] bf16 bits drawn from
    N(0, scale^2)) and per-channel norm weights for q, k and v ([D] fp32, uniform in [0.5, 1.5]).
    Inputs of the QK-norm + RoPE + append step."""
    rq, rk, rv, rw = (np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(4))
    shape = lambda h: (batch, q_len, h, head_dim)
    draw = lambda r, h: f32_to_bf16_bits(np.float32(scale) * r.standard_normal(shape(h),
                                                                                dtype=np.float32))
    w = rw.uniform(0.5, 1.5, (3, head_dim)).astype(np.float32)
    return dict(q=draw(rq, num_q_heads), k=draw(rk, num_kv_heads), v=draw(rv, num_kv_heads),
                q_weight=w[0], k_weight=w[1], v_weight=w[2])


def workload_ctx_lens(wl: Workload) -> np.ndarray:
    if isinstance(wl.ctx, str):
        rng = np.random.default_rng(np.random.SeedSequence([wl.index, 99]))
        return ragged_ctx_lens(rng, wl.batch)
    return np.asarray(wl.ctx, dtype=np.int32)


def make_workload_layer(name: str, kind: str, poison: bool = True, sink: int = 0,
                        q_len: int = 1) -> LayerInputs:
    """Inputs of layer ``kind`` ("global"/"sliding") of workload ``name``; seed = (index, kind),
    extended by (sink, q_len) when either differs from the plain single-token layer."""
    wl = WORKLOADS[name]
    spec = wl.layers[kind]
    ctx = workload_ctx_lens(wl)
    seed = [wl.index, 0 if kind == "global" else 1]
    if sink or q_len != 1:
        seed += [sink, q_len]
    return make_layer_inputs(ctx, spec.num_q_heads, spec.num_kv_heads, spec.head_dim,
                             page_size=wl.page_size, window=spec.window, scale=spec.scale,
                             num_pages=wl.num_pages, pool_factor=wl.pool_factor, q_mult=spec.q_mult,
                             seed=seed, poison=poison, sink=sink, q_len=q_len)


def algorithmic_bytes(ctx_lens: Sequence[int], num_q_heads: int, num_kv_heads: int, head_dim: int,
                      page_size: int = 16, window: int = 0, k_eq_v: bool = False, sink: int = 0,
                      q_len: int = 1) -> int:
    """Bytes the method must move for one layer call: K and V (bf16; K only when the values are
    the keys) of every key some query attends, each once, q (bf16), out (fp32) and the
    block-table entries of the pages touched (int32)."""
    reach = window + q_len - 1 if window > 0 else 0
    kv = 0
    table = 0
    for n in ctx_lens:
        spans = attended_spans(int(n), reach, sink)
        kv += sum(e - a for a, e in spans) * num_kv_heads * head_dim * 2 * (1 if k_eq_v else 2)
        pages = {j for a, e in spans for j in range(a // page_size, (e - 1) // page_size + 1)}
        table += len(pages) * 4
    rows = len(ctx_lens) * q_len * num_q_heads
    return kv + rows * head_dim * 2 + rows * head_dim * 4 + table


def algorithmic_flops(ctx_lens: Sequence[int], num_q_heads: int, head_dim: int,
                      window: int = 0, sink: int = 0, q_len: int = 1) -> int:
    """4 * D flops (q.k and p.v, multiply and add) per query head and key it attends."""
    total = 0
    for n in ctx_lens:
        for i in range(q_len):
            total += sum(e - a for a, e in attended_spans(int(n) - q_len + 1 + i, window, sink))
    return 4 * head_dim * num_q_heads * total
