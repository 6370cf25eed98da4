"""fp64 oracle of the step before attention: per-head RMSNorm of the new tokens' q and k (QK-norm),
rotary position embedding (RoPE) at each token's position, and the paged append of k and v.

TEST INFRASTRUCTURE ONLY: imported by the tests (never by the product package, and it imports
nothing from it).

Sources (cited by page and section):

- Sparse-vLLM PR #27 "feat: support Gemma 4 and native multimodal inference", section
  "Gemma 4 文本推理": the two Gemma 4 layer kinds carry their own RoPE parameters, with a RoPE cache
  kept per layer configuration; section "专用算子与性能优化" lists a dedicated QKV-norm + RoPE kernel.
- vLLM learning notes "模型库与算子层 — 概念": section "自定义 Inductor 融合 pass" fuses norm/RoPE with
  the paged KV-cache write (no launch and no intermediate tensor between them); section
  "内核框架（Helion）" fuses the q/k RMSNorm with RoPE in place, for both pairings (NeoX halves and
  GPT-J interleaved pairs); section "旋转位置编码（RoPE）" lists the default RoPE among the variants.

Definitions (written out here from the standard formulations; the pages name the operations
without formulas):

    rms_norm(x; w, eps) = x / sqrt(mean_d x_d^2 + eps) * w            (w = None: no scaling)
    rope(x, t): for pair j < R/2 of the first R dims (R = rotary_dim), angle a = t * theta^(-2j/R),
        (x1, x2) -> (x1 cos a - x2 sin a, x2 cos a + x1 sin a)
    where the pair is (x_j, x_{j+R/2}) (NeoX) or (x_{2j}, x_{2j+1}) (interleaved); dims >= R pass.
"""
from __future__ import annotations

import numpy as np


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def _f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bf16, ties to even (via fp32: the fp64 value is first rounded to fp32,
    which can move a value sitting within 2^-24 relative of a bf16 tie; such cases are covered by
    the one-ulp tolerance of the comparisons)."""
    f = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (f + 0x7FFF + ((f >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def rms_norm(x: np.ndarray, weight, eps: float) -> np.ndarray:
    """RMSNorm over the last axis, fp64 (weight None: no per-channel scale)."""
    x = np.asarray(x, dtype=np.float64)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if weight is None else y * np.asarray(weight, dtype=np.float64)


def inv_freq(theta: float, rotary_dim: int, freq_dim: int | None = None) -> np.ndarray:
    """Angular frequency of each rotated pair j < rotary_dim / 2: theta^(-2j / freq_dim), where
    freq_dim is rotary_dim unless given (a partial rotation can keep the full head's spacing)."""
    fd = rotary_dim if freq_dim is None else freq_dim
    j = np.arange(rotary_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / fd)


def rope(x: np.ndarray, positions, theta: float, rotary_dim: int, interleaved: bool,
         freq_dim: int | None = None) -> np.ndarray:
    """Rotate the first rotary_dim dims of x[..., D] by position (positions broadcast against
    x[..., 0]); dims at or past rotary_dim pass unchanged."""
    x = np.asarray(x, dtype=np.float64)
    half = rotary_dim // 2
    if half == 0:
        return x.copy()
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq(theta, rotary_dim, freq_dim)
    c, s = np.cos(ang), np.sin(ang)
    out = x.copy()
    if interleaved:
        x1, x2 = x[..., 0:rotary_dim:2], x[..., 1:rotary_dim:2]
        out[..., 0:rotary_dim:2] = x1 * c - x2 * s
        out[..., 1:rotary_dim:2] = x2 * c + x1 * s
    else:
        x1, x2 = x[..., :half], x[..., half:rotary_dim]
        out[..., :half] = x1 * c - x2 * s
        out[..., half:rotary_dim] = x2 * c + x1 * s
    return out


def positions_of(ctx_lens: np.ndarray, q_len: int) -> np.ndarray:
    """[B, L] positions of the new tokens: token i of sequence b sits at ctx_lens[b] - L + i."""
    ctx = np.asarray(ctx_lens, dtype=np.int64)
    return ctx[:, None] - q_len + np.arange(q_len, dtype=np.int64)[None, :]


def prepare(q, k_new, v_new, ctx_lens, norm_qk, norm_v, q_weight, k_weight, v_weight, eps, theta,
            rotary_dim, interleaved, freq_dim=None):
    """fp64 q, k and v of the new tokens after the pre-attention step.

    q: [B, L, Hq, D], k_new and v_new: [B, L, Hkv, D], all bf16 bits. With norm_qk, q and k get
    RMSNorm before RoPE (scaled by q_weight / k_weight; None means a unit scale); with norm_v, v
    gets RMSNorm (scaled by v_weight) and no rotation. v_new may be None (values are the keys)."""
    q64, k64 = _bf16_to_f64(q), _bf16_to_f64(k_new)
    v64 = None if v_new is None else _bf16_to_f64(v_new)
    pos = positions_of(ctx_lens, q64.shape[1])[:, :, None]
    if norm_qk:
        q64 = rms_norm(q64, q_weight, eps)
        k64 = rms_norm(k64, k_weight, eps)
    if norm_v and v64 is not None:
        v64 = rms_norm(v64, v_weight, eps)
    qo = rope(q64, pos, theta, rotary_dim, interleaved, freq_dim)
    ko = rope(k64, pos, theta, rotary_dim, interleaved, freq_dim)
    return qo, ko, v64


def prepare_and_append(q, k_new, v_new, k_pool, v_pool, block_table, ctx_lens, max_position,
                       norm_qk, norm_v, q_weight, k_weight, v_weight, eps, theta, rotary_dim,
                       interleaved, freq_dim=None):
    """The whole step on host arrays. Returns q_out as bf16 bits: rows of tokens whose position t
    is outside [0, max_position) keep their input bits. For every token with t in range, writes
    bf16(k) and bf16(v) into slot t % S of page block_table[b, t // S] (in place; a pool passed as
    both k_pool and v_pool receives k only); a page column past the table row or a page id outside
    [0, P) skips the write."""
    qo, ko, vo = prepare(q, k_new, v_new, ctx_lens, norm_qk, norm_v, q_weight, k_weight, v_weight,
                         eps, theta, rotary_dim, interleaved, freq_dim)
    q_bits = np.array(q, dtype=np.uint16, copy=True)
    pos = positions_of(ctx_lens, q_bits.shape[1])
    B, L = pos.shape
    P, _, S, _ = k_pool.shape
    same = v_pool is k_pool
    for b in range(B):
        for i in range(L):
            t = int(pos[b, i])
            if t < 0 or t >= max_position:
                continue
            q_bits[b, i] = _f64_to_bf16(qo[b, i])
            col = t // S
            if col >= block_table.shape[1]:
                continue
            page = int(block_table[b, col])
            if page < 0 or page >= P:
                continue
            k_pool[page, :, t % S] = _f64_to_bf16(ko[b, i])
            if not same:
                v_pool[page, :, t % S] = _f64_to_bf16(vo[b, i])
    return q_bits
