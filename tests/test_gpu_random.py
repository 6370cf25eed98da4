"""GPU parity on a fixed list of seeded random configurations: every option of the path combined at
random (head_dim, group size, page size, window, sink keys, query tokens, split count, one pool for
K and V, ragged contexts including ones shorter than the query count, query scales up to scores in
the hundreds), each against the fp64 oracle. The list is generated from a fixed seed, so every run checks the same cases."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import make_layer_inputs

pytestmark = pytest.mark.gpu


def _cases(count=120, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        D = int(rng.choice([256, 512]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = 1 if G == 16 else int(rng.choice([1, 2]))
        S = int(rng.choice([16, 32, 64, 128]))
        window = int(rng.choice([0, 0, int(rng.integers(1, 400))]))
        sink = int(rng.integers(0, 40)) if window and rng.random() < 0.5 else 0
        q_len = int(rng.choice([1, 1, 2, 3, 5, 8, 16]))
        B = int(rng.integers(1, 5))
        ctx = [int(x) for x in rng.integers(1, 900, size=B)]
        splits = int(rng.choice([0, 1, 3, 7]))
        kv = bool(rng.random() < 0.25)
        q_mult = float(rng.choice([1.0, 1.0, 4.0, 30.0]))  # 30: scores in the hundreds
        out.append((k, D, G, Hkv, S, window, sink, q_len, ctx, splits, kv, q_mult))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "case%d" % c[0])
def test_random_configuration(case):
    k, D, G, Hkv, S, window, sink, q_len, ctx, splits, kv, q_mult = case
    print("random case", case, flush=True)
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, D, page_size=S, window=window, sink=sink,
                            q_len=q_len, seed=[70, k], q_mult=q_mult)
    t = None
    if kv:
        inp.v_pool = inp.k_pool
        t = gu.upload(inp)
        t["v"] = t["k"]
    out, lse = gu.run(inp, dev_bufs=t, force_splits=splits, values_are_keys=kv)
    gu.compare(out, lse, *gu.reference(inp), "random case %d" % k)


def _prefill_cases(count=60, seed=2025):
    """Long query chunks (the prefill kernel from 64 rows per kv head) combined at random with the
    other options."""
    rng = np.random.default_rng(seed)
    out = []
    for k in range(count):
        D = int(rng.choice([256, 512]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        Hkv = 1 if G == 16 else int(rng.choice([1, 2]))
        S = int(rng.choice([16, 32, 64, 128]))
        window = int(rng.choice([0, 0, int(rng.integers(1, 400))]))
        sink = int(rng.integers(0, 40)) if window and rng.random() < 0.5 else 0
        q_len = int(rng.choice([64, 100, 257])) if G < 4 else int(rng.choice([20, 64, 100, 257]))
        B = int(rng.integers(1, 4))
        ctx = [int(x) for x in rng.integers(1, 1500, size=B)]
        splits = int(rng.choice([0, 1, 3, 7]))
        kv = bool(rng.random() < 0.25)
        q_mult = float(rng.choice([1.0, 1.0, 4.0, 30.0]))
        out.append((k, D, G, Hkv, S, window, sink, q_len, ctx, splits, kv, q_mult))
    return out


@pytest.mark.parametrize("case", _prefill_cases(), ids=lambda c: "prefill%d" % c[0])
def test_random_prefill_configuration(case):
    k, D, G, Hkv, S, window, sink, q_len, ctx, splits, kv, q_mult = case
    print("random prefill case", case, flush=True)
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, D, page_size=S, window=window, sink=sink,
                            q_len=q_len, seed=[71, k], q_mult=q_mult)
    t = None
    if kv:
        inp.v_pool = inp.k_pool
        t = gu.upload(inp)
        t["v"] = t["k"]
    out, lse = gu.run(inp, dev_bufs=t, force_splits=splits, values_are_keys=kv)
    gu.compare(out, lse, *gu.reference(inp), "random prefill case %d" % k)
