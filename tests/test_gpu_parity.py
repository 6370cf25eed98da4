"""GPU parity: the HIP path, called through the C ABI, against the fp64 CPU oracle on the same
seeded inputs. Full-size workloads are compared on every output element (the C oracle is fast
enough); smaller sweeps span several tiles, splits and ragged tails for every compiled
(head_dim, group) pair and several page sizes."""
from __future__ import annotations

import numpy as np
import pytest

import gpu_util as gu
from paged_gqa_kv_attn_amd.workloads import WORKLOADS, make_layer_inputs, make_workload_layer

pytestmark = pytest.mark.gpu

CASES = [(name, kind) for name, wl in WORKLOADS.items() for kind in wl.layers]


@pytest.mark.parametrize("name,kind", CASES, ids=["%s-%s" % c for c in CASES])
def test_workload_parity(name, kind):
    print("workload", name, kind, flush=True)
    inp = make_workload_layer(name, kind)
    out, lse = gu.run(inp)
    ref_out, ref_lse = gu.reference(inp)
    err, cos = gu.compare(out, lse, ref_out, ref_lse, "%s/%s" % (name, kind))
    print("  max_abs_err %.3g  min_cos %.7f" % (err, cos), flush=True)


SWEEP = []
for D in (256, 512):
    for G in (1, 2, 4, 8, 16):
        for S in (16, 32, 64):
            SWEEP.append((D, G, S))


@pytest.mark.parametrize("D,G,S", SWEEP)
@pytest.mark.parametrize("window", [0, 37, 200])
def test_small_shapes(D, G, S, window):
    """Ragged contexts (1 key, partial tiles, partial pages, several splits) for each variant."""
    print("small D=%d G=%d S=%d W=%d" % (D, G, S, window), flush=True)
    Hkv = 2 if G < 16 else 1
    ctx = [1, 15, 16, 17, 100, 333, 520]
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, D, page_size=S, window=window,
                            seed=[D, G, S, window], q_mult=1.5)
    out, lse = gu.run(inp, force_splits=5)  # several splits per sequence, some empty
    gu.compare(out, lse, *gu.reference(inp), "D%d G%d S%d W%d" % (D, G, S, window))


@pytest.mark.parametrize("window", [0, 1, 15, 16, 17, 31, 32, 33, 1024])
def test_every_alignment(window):
    """Contexts 1..80 in one batch: every alignment of n and of the window edge mod 32."""
    print("alignment W=%d" % window, flush=True)
    ctx = list(range(1, 81))
    inp = make_layer_inputs(ctx, 4, 2, 256, page_size=16, window=window, seed=[7, window])
    out, lse = gu.run(inp)
    gu.compare(out, lse, *gu.reference(inp), "W%d" % window)


def test_forced_split_counts_agree():
    inp = make_layer_inputs([700, 129, 64], 16, 2, 512, page_size=16, seed=11)
    ref = gu.reference(inp)
    outs = []
    for ns in (1, 2, 3, 5, 8, 13, 44, 100):
        print("splits", ns, flush=True)
        out, lse = gu.run(inp, force_splits=ns)
        gu.compare(out, lse, *ref, "splits=%d" % ns)
        outs.append(out)
    # P is rounded to bf16 before P.V (relative error <= 2^-9 per weight). Different split
    # counts subtract different running maxima, so the roundings differ and two results may
    # differ by up to about 2 * 2^-9 * max|V| (~1.6e-2 for |V| <= 4); each one already meets the
    # oracle bar above, so require mutual agreement at that bar.
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], atol=gu.MAX_ABS, rtol=0)


@pytest.mark.parametrize("D,G,window", [(512, 8, 0), (512, 4, 200), (256, 2, 1024), (256, 8, 300)])
def test_plan_length_other_than_the_contexts(D, G, window):
    """The plan's max_ctx_len only sizes the split count, and the kernels fetch the first page ids
    of the chunk it gives before the sequences' lengths arrive: every sequence at that length
    (kept), none (fetched again), some, a plan length below the contexts and none (0) all give
    the same results. Covers the column-split kernel (head_dim 512, and head_dim 256 with G = 8)
    and the key-split kernel (head_dim 256, G = 2)."""
    print("plan length D=%d G=%d W=%d" % (D, G, window), flush=True)
    Hkv = 2
    ctx = [3000, 3000, 2100, 3000]
    inp = make_layer_inputs(ctx, G * Hkv, Hkv, D, page_size=16, window=window,
                            seed=[34, D, G, window], q_mult=1.5)
    ref = gu.reference(inp)
    t = gu.upload(inp)
    for max_ctx in (3000, 4096, 2100, 1000, 0):
        for splits in (0, 5):
            out, lse = gu.run(inp, dev_bufs=t, max_ctx_len=max_ctx, force_splits=splits)
            gu.compare(out, lse, *ref, "plan length %d ns%d" % (max_ctx, splits))


def test_page_permutation_is_bitwise_invariant():
    inp = make_layer_inputs([900, 333], 8, 1, 512, page_size=16, seed=12)
    out, lse = gu.run(inp)
    rng = np.random.default_rng(13)
    perm = rng.permutation(inp.k_pool.shape[0])
    inp2 = make_layer_inputs([900, 333], 8, 1, 512, page_size=16, seed=12)
    inp2.k_pool[perm] = inp.k_pool
    inp2.v_pool[perm] = inp.v_pool
    inp2.block_table[:] = np.where(inp.block_table >= 0, perm[np.maximum(inp.block_table, 0)], -1)
    out2, lse2 = gu.run(inp2)
    np.testing.assert_array_equal(out, out2)
    np.testing.assert_array_equal(lse, lse2)


def test_repeat_calls_are_bitwise_identical():
    inp = make_layer_inputs([2000, 1], 16, 8, 256, page_size=16, window=1024, seed=14)
    a = gu.run(inp)
    b = gu.run(inp)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_single_key_returns_value_exactly():
    inp = make_layer_inputs([1, 1], 8, 1, 512, page_size=16, seed=15)
    out, lse = gu.run(inp)
    p = inp.block_table[:, 0]
    from paged_gqa_kv_attn_amd.workloads import bf16_bits_to_f32
    for b in range(2):
        v0 = bf16_bits_to_f32(inp.v_pool[p[b], 0, 0])
        for h in range(8):
            np.testing.assert_array_equal(out[b, h], v0)


def test_empty_context_and_clamped_context():
    inp = make_layer_inputs([0, 40, 48], 4, 2, 256, page_size=16, seed=16)
    out, lse = gu.run(inp)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    ref = gu.reference(inp)
    gu.compare(out, lse, *ref, "empty")
    # a length past the block table's capacity is clamped to max_pages_per_seq * S
    inp.ctx_lens[2] = 10 ** 6
    cap = inp.block_table.shape[1] * 16
    out2, lse2 = gu.run(inp, max_ctx_len=cap)
    inp.ctx_lens[2] = cap
    gu.compare(out2, lse2, *gu.reference(inp), "clamped")


def test_invalid_page_ids_are_skipped():
    """A block-table entry outside [0, P) is never dereferenced: its keys are skipped. Put one on
    the first page of a sequence; the result equals attention over the keys after that page."""
    import oracle
    inp = make_layer_inputs([100, 64], 8, 2, 512, page_size=16, seed=17)
    inp.block_table[0, 0] = inp.k_pool.shape[0] + 5
    inp.block_table[1, 0] = -7
    out, lse = gu.run(inp)
    ref = oracle.decode_attn_ranges(inp.q, inp.k_pool, inp.v_pool, np.maximum(inp.block_table, 0),
                                    [16, 16], [100, 64], inp.scale)
    gu.compare(out, lse, *ref, "invalid page")


def test_batch_smaller_than_plan():
    inp = make_layer_inputs([300, 200, 100], 8, 1, 512, page_size=16, seed=18)
    plan = gu.make_plan(inp)
    out, lse = gu.run(inp, plan=plan, batch=2)
    ref_out, ref_lse = gu.reference(inp)
    gu.compare(out[:2], lse[:2], ref_out[:2], ref_lse[:2], "batch 2 of 3")
    assert np.all(np.isnan(out[2]))  # row past `batch` untouched


def test_extreme_scores_stay_finite():
    """q scaled so scores reach the hundreds: the running max keeps exp2 in range."""
    inp = make_layer_inputs([777, 90], 16, 2, 512, page_size=16, seed=19, q_mult=40.0)
    out, lse = gu.run(inp)
    gu.compare(out, lse, *gu.reference(inp), "extreme")


@pytest.mark.parametrize("window", [0, 300])
def test_values_equal_keys_one_pool(window):
    """Layers whose values are their keys pass the same pool as K and V."""
    inp = make_layer_inputs([1000, 77, 2049], 16, 2, 512 if window == 0 else 256, page_size=16,
                            window=window, seed=[31, window])
    inp.v_pool = inp.k_pool
    t = gu.upload(inp)
    t["v"] = t["k"]
    for flag in (True, False):  # planned as such, or only passed one pool
        out, lse = gu.run(inp, dev_bufs=t, values_are_keys=flag)
        gu.compare(out, lse, *gu.reference(inp), "k=v W%d planned %s" % (window, flag))


@pytest.mark.parametrize("S,ns", [(256, 3), (1024, 2), (16, 1024)])
def test_large_pages_and_max_splits(S, ns):
    """Page sizes up to 1024 keys and the largest split count."""
    inp = make_layer_inputs([3000, 1, 2500], 8, 2, 512, page_size=S, seed=[32, S])
    out, lse = gu.run(inp, force_splits=ns)
    gu.compare(out, lse, *gu.reference(inp), "S%d ns%d" % (S, ns))


def test_many_sequences():
    """A large batch of short ragged sequences (more workgroups than fit the GPU at once)."""
    rng = np.random.default_rng(33)
    ctx = rng.integers(1, 700, size=96)
    inp = make_layer_inputs(ctx, 16, 8, 256, page_size=16, window=512, seed=34)
    out, lse = gu.run(inp)
    gu.compare(out, lse, *gu.reference(inp), "batch 96")


@pytest.mark.parametrize("D,G,window,L", [(512, 8, 0, 1), (512, 8, 0, 128), (256, 2, 300, 1),
                                          (256, 2, 300, 96)])
def test_pools_beyond_4gib(D, G, window, L):
    """Pools of 4.6 GB whose used pages sit past the first 4 GiB: every K/V address is a 64-bit
    offset. The attended pages of a compact layer are copied to high page ids of a large pool
    (the rest of the pool is left uninitialised and never read) and the result must equal the
    oracle on the compact layer, for decode and for a prefill chunk."""
    import torch
    print("big pools D=%d G=%d W=%d L=%d" % (D, G, window, L), flush=True)
    Hkv = 2
    inp = make_layer_inputs([1000, 777], G * Hkv, Hkv, D, page_size=16, window=window,
                            seed=[81, D, L], q_len=L)
    ref = gu.reference(inp)
    d = inp.dims
    page_bytes = Hkv * 16 * D * 2
    big = (9 << 29) // page_bytes              # ~4.8 GB per pool
    first_high = (4 << 30) // page_bytes + 1   # page ids from here start past 4 GiB
    rng = np.random.default_rng(82)
    high = rng.choice(np.arange(first_high, big), size=d["P"], replace=False)
    table = inp.block_table.copy()
    valid = (table >= 0) & (table < d["P"])
    table[valid] = high[table[valid]]
    dev = gu.device()
    t = gu.upload(inp)
    idx = torch.from_numpy(high).to(dev)
    kb = torch.empty((big, Hkv, 16, D), dtype=torch.bfloat16, device=dev)
    vb = torch.empty((big, Hkv, 16, D), dtype=torch.bfloat16, device=dev)
    kb[idx] = t["k"]
    vb[idx] = t["v"]
    t["k"], t["v"] = kb, vb
    t["bt"] = torch.from_numpy(table).to(dev)
    plan = gu.make_plan(inp, num_pages=big)
    out, lse = gu.run(inp, plan=plan, dev_bufs=t)
    gu.compare(out, lse, *ref, "big pools D%d L%d" % (D, L))
    del kb, vb, t
    torch.cuda.empty_cache()


def test_append_beyond_4gib():
    """The paged append into a 4.8 GB pool whose target pages lie past the first 4 GiB: the new
    tokens land in their slots, bit for bit."""
    import torch
    import paged_gqa_kv_attn_amd as pda
    gu.ensure_library()
    D, Hkv, S, L = 512, 2, 16, 3
    ctx = np.array([1000, 77], dtype=np.int32)
    page_bytes = Hkv * S * D * 2
    big = (9 << 29) // page_bytes
    first_high = (4 << 30) // page_bytes + 1
    M = 64
    rng = np.random.default_rng(83)
    table = rng.choice(np.arange(first_high, big), size=(2, M), replace=False).astype(np.int32)
    dev = gu.device()
    kb = torch.zeros((big, Hkv, S, D), dtype=torch.bfloat16, device=dev)
    vb = torch.zeros((big, Hkv, S, D), dtype=torch.bfloat16, device=dev)
    k_new = torch.randn((2, L, Hkv, D), device=dev).to(torch.bfloat16)
    v_new = torch.randn((2, L, Hkv, D), device=dev).to(torch.bfloat16)
    plan = pda.decode_attn_plan(2, 8 * Hkv, Hkv, D, S, M, big, max_ctx_len=1000, q_len=L)
    pda.decode_attn_append_kv(plan, k_new, v_new, kb, vb, torch.from_numpy(table).to(dev),
                              torch.from_numpy(ctx).to(dev), 2)
    torch.cuda.synchronize()
    for b in range(2):
        for i in range(L):
            tpos = int(ctx[b]) - L + i
            page = int(table[b, tpos // S])
            assert torch.equal(kb[page, :, tpos % S], k_new[b, i])
            assert torch.equal(vb[page, :, tpos % S], v_new[b, i])
    del kb, vb
    torch.cuda.empty_cache()
