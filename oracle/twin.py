"""A second, pure-numpy fp64 implementation of the oracle's definition, for tiny shapes only.

TEST INFRASTRUCTURE ONLY. It is written independently of ``oracle.c`` (page-at-a-time gather into
a dense per-sequence array, then numpy's vectorised softmax) so that a pointer or indexing slip in
the C code shows up as a mismatch on brute-force sweeps of tiny inputs. It is not a pin on its
own; the pins are the closed forms and invariants in the oracle tests.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def decode_attn(q, k_pool, v_pool, block_table, ctx_lens, scale, window=0):
    qf = bf16_bits_to_f64(np.asarray(q))
    kf = bf16_bits_to_f64(np.asarray(k_pool))
    vf = bf16_bits_to_f64(np.asarray(v_pool))
    B, Hq, D = qf.shape
    _, Hkv, S, _ = kf.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(ctx_lens[b])
        lo = max(0, n - window) if window > 0 else 0
        if n <= lo:
            continue
        # Dense [Hkv, pages * S, D] copy of the pages holding keys lo..n-1, in logical order.
        first, last = lo // S, (n - 1) // S
        pages = [int(block_table[b, j]) for j in range(first, last + 1)]
        start = lo - first * S
        dense_k = np.concatenate([kf[p] for p in pages], axis=1)[:, start:start + (n - lo)]
        dense_v = np.concatenate([vf[p] for p in pages], axis=1)[:, start:start + (n - lo)]
        for h in range(Hq):
            g = h // G
            s = scale * (dense_k[g] @ qf[b, h])
            m = s.max()
            w = np.exp(s - m)
            out[b, h] = (w @ dense_v[g]) / w.sum()
            lse[b, h] = m + np.log(w.sum())
    return out, lse
