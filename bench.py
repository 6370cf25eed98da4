#!/usr/bin/env python3
"""Benchmark of paged GQA split-KV decode attention on one MI355X.

One step = one decode-attention call of each layer kind of the workload (plan made once, then
stage 1 + stage 2 of the global layer and the sliding-window layer), with inputs already resident
in HBM. Default workload: long_ctx (batch 4, 33792 keys per sequence; global layer 16 q / 2 KV
heads, head_dim 512; sliding layer 16 q / 8 KV heads, head_dim 256, window 1024).

Prints one JSON line: whole-step algorithmic HBM GB/s (value), ms per step, the roofline of the
dominant kernel (global stage 1: HIP events on its stream around every timed launch), per-layer
event medians (cold: the caches flushed before each call; hot: back to back), and the fp64 CPU
oracle timed on this host's cores on the same inputs (which also checks the step's outputs).
Steps rotate over copies of the KV pools so that no step finds its K/V in the L2s or the MALL.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
    python bench.py --copy-calibration     # plain 1 GiB device copy, for counter scaling
    python bench.py --copy-rate            # copy and read bandwidth of hand-written kernels
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attention µs/call and achieved HBM GB/s (% of peak) at 1K–128K ctx"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
# fp64 oracle sample budgets (flops per pass): ~1-2 s on 16 host cores, ~2 s on one.
CPU_SAMPLE_FLOPS = 60e9
CPU_ONE_THREAD_FLOPS = 6e9


def _fatbin() -> bytes:
    """The library's device code: its .hip_fatbin ELF section."""
    import paged_gqa_kv_attn_amd as pda
    with open(pda.library_path(), "rb") as f:
        elf = f.read()
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    sections = [struct.unpack_from("<IIQQQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    names = sections[shstrndx][4]
    for name, _, _, _, offset, size in sections:
        if elf[names + name:elf.index(b"\0", names + name)] == b".hip_fatbin":
            return elf[offset:offset + size]
    raise RuntimeError("no device code section in %s" % pda.library_path())


# Kernel families whose code-object bundles are hashed on their own (one bundle per source file).
KERNEL_FAMILIES = ("stage1_kernel", "stage1_ks_kernel", "prefill_kernel", "stage2_kernel",
                   "append_kernel", "append_rope_kernel")


def kernel_code_hash(kernel: str = "") -> str:
    """First 16 hex digits of the SHA-256 of the library's device code: the whole .hip_fatbin
    section, or with ``kernel`` only the offload bundles (one per source file) whose code object
    names that kernel, so a profile of one kernel stays valid while other sources change.
    Host-side edits and comment edits leave either unchanged, kernel edits do not."""
    data = _fatbin()
    if not kernel:
        return hashlib.sha256(data).hexdigest()[:16]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = []
    i = data.find(magic)
    while i >= 0:
        starts.append(i)
        i = data.find(magic, i + 1)
    h = hashlib.sha256()
    found = False
    needle = kernel.encode()
    for k, a in enumerate(starts):
        b = starts[k + 1] if k + 1 < len(starts) else len(data)
        if needle not in data[a:b]:
            continue
        # Bundle: magic, entry count, then (offset, size, triple length, triple) per entry, offsets
        # from the magic. Only the entries' bytes are hashed (not the alignment padding after them).
        count, = struct.unpack_from("<Q", data, a + len(magic))
        pos = a + len(magic) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", data, pos)
            h.update(data[pos + 24:pos + 24 + tlen])
            h.update(data[a + off:a + off + size])
            pos += 24 + tlen
        found = True
    if not found:
        raise RuntimeError("no code object names %s" % kernel)
    return h.hexdigest()[:16]


def load_traffic(workload: str, num_splits: int):
    """HBM bytes per stage-1 launch from the committed counter summary, if it was taken with the
    same device code and split count as now (else None)."""
    path = os.path.join(ROOT, "profiles", "stage1_global_%s_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_code_sha256_16") != kernel_code_hash("stage1_kernel"):
        return None
    if fields.get("num_splits") != str(num_splits):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def load_trace_mean_us(workload: str):
    """Mean duration (us) of the global stage-1 kernel in the committed rocprofv3 kernel-trace
    summary of this workload, if it was taken with the same device code as now (else None)."""
    import re
    path = os.path.join(ROOT, "profiles", "stage1_global_%s_kernel_trace.txt" % workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"^kernel_code_sha256_16:\s*(\S+)", text, re.M)
    m = re.search(r"^(?:dominant kernel|global stage 1) stage1_kernel.*mean ([0-9.]+) us", text,
                  re.M)
    if h is None or m is None or h.group(1) != kernel_code_hash("stage1_kernel"):
        return None
    return float(m.group(1))


def provenance() -> dict:
    """Where the numbers come from: the source revision the library was built from, the ROCm and
    torch versions, the device."""
    import subprocess
    info = {}
    try:
        sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True,
                             text=True, timeout=10)
        if sha.returncode == 0:
            dirty = subprocess.run(["git", "-C", ROOT, "status", "--porcelain",
                                    "--untracked-files=no"], capture_output=True, text=True,
                                   timeout=10)
            info["git_sha"] = sha.stdout.strip()
            info["git_dirty"] = bool(dirty.stdout.strip())
            info["git_source"] = "working tree"
    except (OSError, subprocess.SubprocessError):
        pass
    if "git_sha" not in info:
        # No repository here (a copied tree): the revision recorded when the library was built.
        try:
            with open(os.path.join(ROOT, "paged_gqa_kv_attn_amd", "_build_info.json")) as f:
                b = json.load(f)
            info.update(git_sha=b.get("git_sha"), git_dirty=b.get("git_dirty"),
                        git_source="recorded at library build")
        except (OSError, ValueError):
            info.update(git_sha=None, git_dirty=None, git_source="unavailable")
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm_version"] = f.read().strip()
    except OSError:
        info["rocm_version"] = None
    import torch
    info["torch_version"] = torch.__version__
    info["torch_hip_version"] = getattr(torch.version, "hip", None)
    if torch.cuda.is_available():
        props = torch.cuda.get_device_properties(0)
        info["device"] = "%s (%s), %d CUs" % (props.name, getattr(props, "gcnArchName", "?"),
                                             props.multi_processor_count)
    return info


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_ctx")
    ap.add_argument("--copies", type=int, default=0,
                    help="distinct copies of the KV pools, used in rotation across steps; 0 = "
                         "enough that a step re-reads a copy only after ~768 MB of other K/V "
                         "(more than the L2s and the 256 MB MALL hold)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--copy-rate", action="store_true",
                    help="run the copy-rate program (1 GiB device copies by hand-written kernels "
                         "with and without non-temporal loads/stores, and the runtime's copy; "
                         "1 GiB read-only passes, one-pass grids and streams of 1-4 workgroups "
                         "per CU): the ceilings of a kernel that reads each byte once and writes "
                         "it once, and of one that only streams its inputs")
    ap.add_argument("--k-eq-v", action="store_true",
                    help="layers whose values are their keys: one pool passed as both K and V")
    ap.add_argument("--q-len", type=int, default=1,
                    help="query tokens per sequence (causal multi-token decode), both layers")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed steps for this long before the warmup steps (clock ramp-up)")
    ap.add_argument("--append", action="store_true",
                    help="each layer call first appends the step's new tokens' K/V to the pools")
    ap.add_argument("--rope", action="store_true",
                    help="each layer call first runs the fused QK-norm + RoPE + paged append of the "
                         "step's new tokens, then attends with the rotated q")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the two extra lines of the default run: the global layer on a "
                         "512-token prefill chunk per sequence (MFMA-bound) and the fused QK-norm "
                         "+ RoPE + append of a 2048-token chunk per sequence")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replay diagnostic after the timed region")
    ap.add_argument("--sink", type=int, default=0,
                    help="sink keys the sliding layer also attends (StreamingLLM-style view)")
    ap.add_argument("--range", default="very_long_b2,very_long_b1",
                    help="further workloads whose global layer is timed after the step (cold and "
                         "hot call medians, back-to-back stage-1 launches): by default the 2 x 64K "
                         "and 1 x 128K ends of the 32K-128K range; '' for none")
    args = ap.parse_args()

    if args.append and args.rope:
        print("--append and --rope are alternatives (--rope appends too)", flush=True)
        return 2
    if args.gpus != 1:
        print("bench.py measures a single GPU; --gpus %d is not supported (the decode-attention "
              "path has no cross-GPU step; run with --gpus 1)" % args.gpus, flush=True)
        return 2

    if args.copy_rate:
        # A child process of its own, started before this process touches the GPU.
        import subprocess
        from paged_gqa_kv_attn_amd import build as hip_build
        if not os.path.exists(hip_build.COPY_RATE):
            print("copy_rate is not built (python -m paged_gqa_kv_attn_amd.build)", flush=True)
            return 2
        return subprocess.run([hip_build.COPY_RATE]).returncode

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(5)]
        for ea, eb in evs:
            ea.record(stream)
            dst.copy_(src)
            eb.record(stream)
        torch.cuda.synchronize()
        us = sorted(1e3 * ea.elapsed_time(eb) for ea, eb in evs)
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "launches": 5, "median_us": round(us[2], 1),
                          "read_plus_write_GB_per_s": round(2 * n / (us[2] * 1e-6) / 1e9, 1)}),
              flush=True)
        return 0

    import paged_gqa_kv_attn_amd as pda
    from paged_gqa_kv_attn_amd import workloads as wl_mod

    if not os.path.exists(pda.library_path()):
        from paged_gqa_kv_attn_amd import build
        build.build()
    pda.load_library()

    wl = wl_mod.WORKLOADS[args.workload]
    copies = args.copies
    if copies <= 0:
        step_kv = sum(wl_mod.algorithmic_bytes(wl_mod.workload_ctx_lens(wl), sp.num_q_heads,
                                               sp.num_kv_heads, sp.head_dim, wl.page_size,
                                               sp.window, k_eq_v=args.k_eq_v, sink=args.sink,
                                               q_len=args.q_len) for sp in wl.layers.values())
        copies = int(min(256, max(2, -(-(768 << 20) // step_kv))))
    t_gen = time.time()
    layers = []
    for kind in ("global", "sliding"):
        if kind not in wl.layers:
            continue
        sink = args.sink if kind == "sliding" else 0
        inp = wl_mod.make_workload_layer(args.workload, kind, sink=sink, q_len=args.q_len)
        lead = (inp.dims["B"],) if args.q_len == 1 else (inp.dims["B"], args.q_len)
        d = inp.dims
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)
        if args.k_eq_v:
            inp.v_pool = inp.k_pool
        k0 = bf(inp.k_pool)
        v0 = k0 if args.k_eq_v else bf(inp.v_pool)
        plan = pda.decode_attn_plan(d["B"], d["Hq"], d["Hkv"], d["D"], d["S"], d["M"], d["P"],
                                    max_ctx_len=int(inp.ctx_lens.max()), window=inp.window,
                                    values_are_keys=args.k_eq_v, sink=sink, q_len=args.q_len)
        spec = wl.layers[kind]
        rope = None
        if args.rope:
            # Pre-norm q, k and v of the step's new tokens, RMSNorm weights and the rotation table
            # (full rotation, NeoX pairs; theta 1e6 for the global layer, 1e4 for the sliding one).
            # The step is run once before the pool copies are made, so every copy already holds
            # the rotated keys the timed steps write again.
            new = wl_mod.make_new_tokens(d["B"], args.q_len, d["Hq"], d["Hkv"], d["D"],
                                         seed=[wl.index, 0 if kind == "global" else 1, 7])
            theta = 1e6 if kind == "global" else 1e4
            max_pos = int(inp.ctx_lens.max()) + 1
            cs = torch.empty((max_pos, d["D"]), dtype=torch.float32, device=dev)
            pda.decode_attn_rope_cache(cs, max_pos, d["D"], theta)
            f32 = lambda a: torch.from_numpy(a).to(dev)
            rope = dict(new=new, theta=theta, max_pos=max_pos, cs=cs, q=bf(new["q"]),
                        k=bf(new["k"]), v=None if args.k_eq_v else bf(new["v"]),
                        qw=f32(new["q_weight"]), kw=f32(new["k_weight"]), eps=1e-6)
            rope["q_out"] = torch.empty_like(rope["q"])
            pda.decode_attn_append_kv_rope(plan, rope["q"], rope["q_out"], rope["k"], rope["v"],
                                           k0, v0, torch.from_numpy(inp.block_table).to(dev),
                                           torch.from_numpy(inp.ctx_lens).to(dev), d["B"], cs,
                                           max_pos, d["D"], False, pda.NORM_QK, rope["qw"],
                                           rope["kw"], None, rope["eps"])
        ks, vs = [k0], [v0]
        for _ in range(1, copies):
            ks.append(k0.clone())
            vs.append(ks[-1] if args.k_eq_v else v0.clone())
        # The newest q_len tokens' K/V as the append's input: the values already in the pools, so the
        # appended cache (and the oracle check) is unchanged while the copy does its full work.
        S, Lq = d["S"], args.q_len
        pos = inp.ctx_lens[:, None] - Lq + np.arange(Lq)[None, :]
        pages = inp.block_table[np.arange(d["B"])[:, None], pos // S]
        k_new = np.ascontiguousarray(inp.k_pool[pages, :, pos % S, :])  # [B, L, Hkv, D]
        v_new = np.ascontiguousarray(inp.v_pool[pages, :, pos % S, :])
        # Per new token: q read and written, k (and v) read and written to its slot, one table row.
        rope_bytes = (d["B"] * Lq * (4 * d["Hq"] * d["D"] + 4 * d["Hkv"] * d["D"] *
                                     (1 if args.k_eq_v else 2) + 4 * d["D"]))
        layers.append(dict(
            spec=wl.layers[kind], sink=sink,
            k_new=bf(k_new), v_new=bf(v_new),
            append_bytes=(rope_bytes if args.rope else
                          2 * k_new.size * 2 * (1 if args.k_eq_v else 2)),
            rope=rope,
            kind=kind, inp=inp, dims=d, plan=plan,
            q=rope["q_out"] if rope else bf(inp.q), k=ks, v=vs,
            bt=torch.from_numpy(inp.block_table).to(dev),
            ctx=torch.from_numpy(inp.ctx_lens).to(dev),
            out=torch.empty(lead + (d["Hq"], d["D"]), device=dev),
            lse=torch.empty(lead + (d["Hq"],), device=dev),
            ws=torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev),
            bytes=wl_mod.algorithmic_bytes(inp.ctx_lens, spec.num_q_heads, spec.num_kv_heads,
                                           spec.head_dim, wl.page_size, spec.window,
                                           k_eq_v=args.k_eq_v, sink=sink, q_len=args.q_len),
            flops=wl_mod.algorithmic_flops(inp.ctx_lens, spec.num_q_heads, spec.head_dim,
                                           spec.window, sink=sink, q_len=args.q_len)))
        del inp.k_pool, inp.v_pool  # host copies are regenerated for the CPU leg if needed
    torch.cuda.synchronize()
    print("# inputs ready in %.1f s: %s" % (time.time() - t_gen, ", ".join(
        "%s %r" % (L["kind"], L["plan"]) for L in layers)), file=sys.stderr, flush=True)

    dominant = layers[0]  # the global layer's stage 1 moves ~all of the bytes
    B = dominant["plan"].problem.batch

    def append(L, r):
        ro = L["rope"]
        if ro is not None:
            pda.decode_attn_append_kv_rope(
                L["plan"], ro["q"], ro["q_out"], ro["k"], ro["v"], L["k"][r], L["v"][r], L["bt"],
                L["ctx"], L["plan"].problem.batch, ro["cs"], ro["max_pos"],
                L["plan"].problem.head_dim, False, pda.NORM_QK, ro["qw"], ro["kw"], None,
                ro["eps"])
        else:
            pda.decode_attn_append_kv(L["plan"], L["k_new"], L["v_new"], L["k"][r], L["v"][r],
                                      L["bt"], L["ctx"], L["plan"].problem.batch)

    appends = args.append or args.rope

    # The step's calls prepared once per layer and pool copy (arguments checked and converted once,
    # one ctypes call each), as a serving loop with fixed buffers makes them. The graph-replay
    # diagnostic below uses the ordinary calls, which follow torch's current (capture) stream.
    def prepare_calls(L, r):
        p = L["plan"]
        c = {}
        if L["rope"] is not None:
            ro = L["rope"]
            c["append"] = pda.decode_attn_append_kv_rope(
                p, ro["q"], ro["q_out"], ro["k"], ro["v"], L["k"][r], L["v"][r], L["bt"],
                L["ctx"], p.problem.batch, ro["cs"], ro["max_pos"], p.problem.head_dim, False,
                pda.NORM_QK, ro["qw"], ro["kw"], None, ro["eps"], prepare=True)
        else:
            c["append"] = pda.decode_attn_append_kv(p, L["k_new"], L["v_new"], L["k"][r],
                                                    L["v"][r], L["bt"], L["ctx"],
                                                    p.problem.batch, prepare=True)
        if L is dominant:
            c["layer"] = pda.decode_attn_global(p, L["q"], L["k"][r], L["v"][r], L["bt"],
                                                L["ctx"], p.problem.batch, L["inp"].scale,
                                                L["out"], L["lse"], L["ws"], prepare=True)
            if p.num_splits > 1:
                c["s1"] = pda.decode_attn_stage1(p, L["q"], L["k"][r], L["v"][r], L["bt"],
                                                 L["ctx"], p.problem.batch, L["inp"].scale,
                                                 L["ws"], prepare=True)
                c["s2"] = pda.decode_attn_stage2(p, p.problem.batch, L["ws"], L["out"], L["lse"],
                                                 prepare=True)
        else:
            c["layer"] = pda.decode_attn_sliding(p, L["q"], L["k"][r], L["v"][r], L["bt"],
                                                 L["ctx"], p.problem.batch, p.problem.window,
                                                 L["inp"].scale, L["out"], L["lse"], L["ws"],
                                                 prepare=True)
        return c

    for L in layers:
        L["pc"] = [prepare_calls(L, r) for r in range(len(L["k"]))]

    def run_layer(L, r, ev_s1=None, prepared=True):
        p = L["plan"]
        if prepared:
            c = L["pc"][r]
            if appends:
                c["append"]()
            if ev_s1 is not None:
                ev_s1[0].record(stream)
            if L is dominant and p.num_splits > 1:
                c["s1"]()
                if ev_s1 is not None:
                    ev_s1[1].record(stream)
                c["s2"]()
            else:
                c["layer"]()
                if ev_s1 is not None:
                    ev_s1[1].record(stream)
            return
        if appends:
            append(L, r)
        if L is dominant and p.num_splits == 1:
            # One split: the layer call is stage 1 alone, writing out and lse in place.
            if ev_s1 is not None:
                ev_s1[0].record(stream)
            pda.decode_attn_global(p, L["q"], L["k"][r], L["v"][r], L["bt"], L["ctx"],
                                   p.problem.batch, L["inp"].scale, L["out"], L["lse"], L["ws"])
            if ev_s1 is not None:
                ev_s1[1].record(stream)
        elif L is dominant:
            if ev_s1 is not None:
                ev_s1[0].record(stream)
            pda.decode_attn_stage1(p, L["q"], L["k"][r], L["v"][r], L["bt"], L["ctx"],
                                   p.problem.batch, L["inp"].scale, L["ws"])
            if ev_s1 is not None:
                ev_s1[1].record(stream)
            pda.decode_attn_stage2(p, p.problem.batch, L["ws"], L["out"], L["lse"])
        else:
            pda.decode_attn_sliding(p, L["q"], L["k"][r], L["v"][r], L["bt"], L["ctx"],
                                    p.problem.batch, p.problem.window, L["inp"].scale, L["out"],
                                    L["lse"], L["ws"])

    R = len(dominant["k"])
    # Clock settle: a fresh GPU ramps its clocks over the first few hundred milliseconds of load, so
    # steps run untimed for --settle-ms before the warmup steps (the timed region is unchanged).
    t_settle = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(20):
            for L in layers:
                run_layer(L, settle_steps % R)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        for L in layers:
            run_layer(L, i % R)
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        for L in layers:
            run_layer(L, i % R, ev[i] if L is dominant else None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    ms_per_step = (t1 - t0) * 1e3 / K

    # Graph replay, a diagnostic after the timed region: the same step captured once per pool copy
    # in a HIP graph, as a serving loop runs it, which removes the host's launch gaps between the
    # kernels. The kernels and their arguments are the eager step's.
    graph_us = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for r in range(R):
                for L in layers:
                    run_layer(L, r, prepared=False)
        stream.wait_stream(side)
        graphs = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for L in layers:
                    run_layer(L, r, prepared=False)
            graphs.append(g)
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[i % R].replay()
        ga, gb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ga.record(stream)
        for i in range(K):
            graphs[i % R].replay()
        gb.record(stream)
        torch.cuda.synchronize()
        graph_us = 1e3 * ga.elapsed_time(gb) / K
        del graphs

    # The dominant kernel on its own: back-to-back stage-1 launches of the global layer (rotating
    # pool copies) between one event pair on the launch stream; the average per launch includes
    # the dispatch gap between kernels but not an event pair's own overhead per launch.
    def stage1_only(L, r):
        p = L["plan"]
        if p.num_splits == 1:
            pda.decode_attn_global(p, L["q"], L["k"][r], L["v"][r], L["bt"], L["ctx"],
                                   p.problem.batch, L["inp"].scale, L["out"], L["lse"], L["ws"])
        else:
            pda.decode_attn_stage1(p, L["q"], L["k"][r], L["v"][r], L["bt"], L["ctx"],
                                   p.problem.batch, L["inp"].scale, L["ws"])

    def back_to_back_us(L, n, fn, batches=5):
        """Mean launch duration of n back-to-back launches between one HIP event pair; the median
        over `batches` such batches (one batch can catch a clock or memory-controller hiccup)."""
        for i in range(3):
            fn(L, i % len(L["k"]))
        per = []
        for _ in range(batches):
            ba, bb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ba.record(stream)
            for i in range(n):
                fn(L, i % len(L["k"]))
            bb.record(stream)
            torch.cuda.synchronize()
            per.append(1e3 * ba.elapsed_time(bb) / n)
        return sorted(per)[len(per) // 2]

    s1_b2b_us = back_to_back_us(dominant, K, stage1_only)

    # Per-layer breakdown, after (outside) the timed region: events around each layer call.
    # Cold: before every call a 512 MB buffer is written (outside the event pair), which evicts
    # the L2s and the MALL, so the call reads its K/V from HBM whatever the workload's size.
    # Hot (a diagnostic): the same call on the same pool copy back to back, so a layer small
    # enough to stay in the L2s and the MALL shows it (GB/s above the HBM peak). Fills queued in
    # front keep the GPU busy while the host enqueues the calls, so short calls are not timed
    # waiting for the host.
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def timed_calls(L, n, flush):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        if not flush:
            for i in range(8):
                flush_buf.fill_(i)
        for i, (ea, eb) in enumerate(evs):
            if flush:
                flush_buf.fill_(i & 0xFF)
            ea.record(stream)
            run_layer(L, i % R if flush else 0)
            eb.record(stream)
        torch.cuda.synchronize()
        return sorted(1e3 * ea.elapsed_time(eb) for ea, eb in evs)

    detail = {}
    for L in layers:
        us = timed_calls(L, 50, flush=True)
        hot = timed_calls(L, 50, flush=False)
        med = us[len(us) // 2]
        if appends:
            # The append alone, prepared, behind a queue of fills (as for the hot calls), so that
            # a short append is not timed waiting for the host to enqueue it.
            eva = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(20)]
            for i in range(8):
                flush_buf.fill_(i)
            for i, (ea, eb) in enumerate(eva):
                ea.record(stream)
                L["pc"][i % R]["append"]()
                eb.record(stream)
            torch.cuda.synchronize()
            ua = sorted(1e3 * ea.elapsed_time(eb) for ea, eb in eva)
            L["append_us"] = ua[len(ua) // 2]
        detail[L["kind"]] = {"us_per_call_median": round(med, 2),
                             "us_per_call_p10": round(us[len(us) // 10], 2),
                             "us_per_call_p90": round(us[(9 * len(us)) // 10], 2),
                             "hot_us_per_call_median": round(hot[len(hot) // 2], 2),
                             "GB_per_s": round(L["bytes"] / (med * 1e-6) / 1e9, 1),
                             "pct_of_hbm_peak": round(100 * L["bytes"] / (med * 1e-6) / 1e9 /
                                                      PEAK_HBM_GBS, 2)}
        if appends:
            detail[L["kind"]].update(append_us_median=round(L["append_us"], 2),
                                     append_bytes=L["append_bytes"],
                                     append_GB_per_s=round(L["append_bytes"] /
                                                           (L["append_us"] * 1e-6) / 1e9, 1))
    # The other ends of the 32K-128K range: each workload's global layer on its own (inputs made
    # here, two pool copies rotated), timed like the step's layers: back-to-back stage-1 launches,
    # then cold and hot calls.
    range_detail = {}
    for name in [w for w in args.range.split(",") if w and w != args.workload]:
        rw = wl_mod.WORKLOADS[name]
        if "global" not in rw.layers:
            continue
        t_r = time.time()
        rinp = wl_mod.make_workload_layer(name, "global")
        rd = rinp.dims
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(
            torch.bfloat16)
        rk0, rv0 = bf(rinp.k_pool), bf(rinp.v_pool)
        del rinp.k_pool, rinp.v_pool
        rplan = pda.decode_attn_plan(rd["B"], rd["Hq"], rd["Hkv"], rd["D"], rd["S"], rd["M"],
                                     rd["P"], max_ctx_len=int(rinp.ctx_lens.max()))
        rspec = rw.layers["global"]
        rbytes = wl_mod.algorithmic_bytes(rinp.ctx_lens, rspec.num_q_heads, rspec.num_kv_heads,
                                          rspec.head_dim, rw.page_size, 0)
        RL = dict(kind="global", inp=rinp, dims=rd, plan=rplan, q=bf(rinp.q),
                  k=[rk0, rk0.clone()], v=[rv0, rv0.clone()],
                  bt=torch.from_numpy(rinp.block_table).to(dev),
                  ctx=torch.from_numpy(rinp.ctx_lens).to(dev),
                  out=torch.empty((rd["B"], rd["Hq"], rd["D"]), device=dev),
                  lse=torch.empty((rd["B"], rd["Hq"]), device=dev),
                  ws=torch.empty(rplan.workspace_bytes, dtype=torch.uint8, device=dev))
        torch.cuda.synchronize()

        def rcall(L, r):
            p = L["plan"]
            pda.decode_attn_global(p, L["q"], L["k"][r], L["v"][r], L["bt"], L["ctx"],
                                   p.problem.batch, L["inp"].scale, L["out"], L["lse"], L["ws"])

        t_s = time.perf_counter()
        while (time.perf_counter() - t_s) * 1e3 < args.settle_ms / 2:
            for i in range(20):
                rcall(RL, i % 2)
            torch.cuda.synchronize()
        rs1_bytes = rbytes - rd["B"] * rd["Hq"] * rd["D"] * 4
        rs1_us = back_to_back_us(RL, K, stage1_only)
        rcall_us = back_to_back_us(RL, K, rcall)
        cold = []
        for i in range(50):
            flush_buf.fill_(i & 0xFF)
            ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea.record(stream)
            rcall(RL, i % 2)
            eb.record(stream)
            cold.append((ea, eb))
        torch.cuda.synchronize()
        cold = sorted(1e3 * a.elapsed_time(b) for a, b in cold)
        rtrace = load_trace_mean_us(name)
        med = cold[len(cold) // 2]
        range_detail[name] = {
            "description": rw.description, "num_splits": rplan.num_splits,
            "layer_algorithmic_bytes": rbytes,
            "stage1_back_to_back_us": round(rs1_us, 2),
            "stage1_pct_of_hbm_peak": round(100 * rs1_bytes / (rs1_us * 1e-6) / 1e9 /
                                            PEAK_HBM_GBS, 2),
            "stage1_trace_mean_us": rtrace,
            "stage1_trace_pct_of_hbm_peak": (round(100 * rs1_bytes / (rtrace * 1e-6) / 1e9 /
                                                   PEAK_HBM_GBS, 2) if rtrace else None),
            "layer_back_to_back_us": round(rcall_us, 2),
            "layer_back_to_back_pct_of_hbm_peak": round(100 * rbytes / (rcall_us * 1e-6) / 1e9 /
                                                        PEAK_HBM_GBS, 2),
            "us_per_call_median": round(med, 2),
            "us_per_call_p10": round(cold[len(cold) // 10], 2),
            "us_per_call_p90": round(cold[(9 * len(cold)) // 10], 2),
            "pct_of_hbm_peak": round(100 * rbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
            "setup_s": round(time.time() - t_r, 1)}
        del RL, rk0, rv0
        torch.cuda.empty_cache()
        print("# range %s: %s" % (name, range_detail[name]), file=sys.stderr, flush=True)

    # Extras of the plain run, on the global layer's pools (after the step's timing): a prefill
    # chunk of 512 tokens per sequence (the layer call: one split, stage 1 writes out and lse
    # in place) and the fused QK-norm + RoPE + append of 2048 tokens per sequence (into copies of
    # the pools), each timed over back-to-back launches between one HIP event pair.
    extras = {}
    if not args.no_extras and args.q_len == 1 and not appends and not args.k_eq_v and \
            args.sink == 0 and dominant["kind"] == "global":
        t_x = time.time()
        gL = dominant
        gd, ginp0 = gL["dims"], gL["inp"]
        B_, Hq_, Hkv_, D_ = gd["B"], gd["Hq"], gd["Hkv"], gd["D"]
        mx = int(ginp0.ctx_lens.max())

        def b2b(fn, n, warm_ms=300.0):
            # Run the call for warm_ms first: the clocks settle differently under MFMA-bound work
            # than under the memory-bound step just timed.
            t_w = time.perf_counter()
            while (time.perf_counter() - t_w) * 1e3 < warm_ms:
                for _ in range(4):
                    fn()
                torch.cuda.synchronize()
            xa, xb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            xa.record(stream)
            for _ in range(n):
                fn()
            xb.record(stream)
            torch.cuda.synchronize()
            return 1e3 * xa.elapsed_time(xb) / n

        PLq = 512
        pplan = pda.decode_attn_plan(B_, Hq_, Hkv_, D_, gd["S"], gd["M"], gd["P"],
                                     max_ctx_len=mx, q_len=PLq)
        pq = bf(wl_mod.make_new_tokens(B_, PLq, Hq_, Hkv_, D_, seed=[wl.index, 11],
                                       scale=wl.layers["global"].q_mult)["q"])
        pout = torch.empty((B_, PLq, Hq_, D_), device=dev)
        plse = torch.empty((B_, PLq, Hq_), device=dev)
        pws = torch.empty(max(pplan.layer_workspace_bytes, 256), dtype=torch.uint8, device=dev)
        pcall = pda.decode_attn_global(pplan, pq, gL["k"][0], gL["v"][0], gL["bt"], gL["ctx"], B_,
                                       ginp0.scale, pout, plse, pws, prepare=True)
        p_us = b2b(pcall, 5)
        p_flops = wl_mod.algorithmic_flops(ginp0.ctx_lens, Hq_, D_, 0, 0, q_len=PLq)
        extras["prefill_chunk"] = {
            "description": "global layer, %d causal query tokens per sequence at the end of each "
                           "context (layer call)" % PLq,
            "num_splits": pplan.num_splits, "us_per_call": round(p_us, 1),
            "algorithmic_flops": p_flops,
            "TFLOP_per_s": round(p_flops / (p_us * 1e-6) / 1e12, 1),
            "pct_of_bf16_mfma_peak": round(100 * p_flops / (p_us * 1e-6) / 1e12 /
                                           PEAK_BF16_TFLOPS, 2)}
        del pq, pout, plse, pws, pcall
        RLq = 2048
        rplan_x = pda.decode_attn_plan(B_, Hq_, Hkv_, D_, gd["S"], gd["M"], gd["P"],
                                       max_ctx_len=mx, q_len=RLq)
        nt = wl_mod.make_new_tokens(B_, RLq, Hq_, Hkv_, D_, seed=[wl.index, 12])
        cs = torch.empty((mx + 1, D_), dtype=torch.float32, device=dev)
        pda.decode_attn_rope_cache(cs, mx + 1, D_, 1e6)
        f32 = lambda a: torch.from_numpy(a).to(dev)
        rq_in, rk_in, rv_in = bf(nt["q"]), bf(nt["k"]), bf(nt["v"])
        rq_out = torch.empty_like(rq_in)
        kc, vc = gL["k"][0].clone(), gL["v"][0].clone()
        rcall_x = pda.decode_attn_append_kv_rope(
            rplan_x, rq_in, rq_out, rk_in, rv_in, kc, vc, gL["bt"], gL["ctx"], B_, cs, mx + 1, D_,
            False, pda.NORM_QK, f32(nt["q_weight"]), f32(nt["k_weight"]), None, 1e-6,
            prepare=True)
        r_us = b2b(rcall_x, 10)
        r_bytes = B_ * RLq * (4 * Hq_ * D_ + 8 * Hkv_ * D_ + 4 * D_)
        extras["rope_append_chunk"] = {
            "description": "fused QK-norm + RoPE + paged append of %d new tokens per sequence "
                           "(global layer: q, k and v rows, full NeoX rotation)" % RLq,
            "us_per_call": round(r_us, 2), "algorithmic_bytes": r_bytes,
            "GB_per_s": round(r_bytes / (r_us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * r_bytes / (r_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2)}
        del rq_in, rk_in, rv_in, rq_out, kc, vc, cs, rcall_x
        torch.cuda.empty_cache()
        extras["setup_and_timing_s"] = round(time.time() - t_x, 1)
        print("# extras: %s" % extras, file=sys.stderr, flush=True)

    step_bytes = sum(L["bytes"] + (L["append_bytes"] if appends else 0) for L in layers)
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    s1_ms = [a.elapsed_time(b) for a, b in ev]
    s1_avg_us = 1e3 * sum(s1_ms) / len(s1_ms)

    # Algorithmic bytes of one global stage-1 launch: K and V rows of every attended key
    # (4 * D bytes per key and KV head), q, and the block-table entries of the pages touched.
    ginp = dominant["inp"]
    gd = dominant["dims"]
    s1_bytes = dominant["bytes"] - gd["B"] * args.q_len * gd["Hq"] * gd["D"] * 4  # minus out
    achieved = s1_bytes / (s1_b2b_us * 1e-6) / 1e9
    plain = args.q_len == 1 and args.sink == 0 and not args.k_eq_v
    traffic = load_traffic(args.workload, dominant["plan"].num_splits) if plain else None
    trace_us = load_trace_mean_us(args.workload) if plain else None
    # Long query chunks (prefill) carry more flops per byte than the MFMA/HBM ridge: then the
    # kernel is priced against the bf16 MFMA peak instead.
    s1_flops = dominant["flops"]
    mfma_bound = s1_flops / s1_bytes > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    roofline = {
        "kernel": "stage1 global (D=%d, G=%d)" % (gd["D"], dominant["plan"].group_size),
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": PEAK_HBM_GBS,
        "unit": "GB/s",
        "frac": round(achieved / PEAK_HBM_GBS, 4),
        "traffic": traffic,
        "traffic_GB_per_s": (round(traffic / (s1_b2b_us * 1e-6) / 1e9, 1)
                             if traffic is not None else None),
        "traffic_over_algorithmic": round(traffic / s1_bytes, 4) if traffic is not None else None,
        "avg_launch_us": round(s1_b2b_us, 3),
        "avg_launch_us_source": "median over 5 batches of %d back-to-back stage-1 launches, each "
                                "batch between one HIP event pair on the launch stream" % K,
        "event_pair_per_launch_avg_us": round(s1_avg_us, 3),
        "trace_mean_us": trace_us,
        "trace_frac": (round(s1_bytes / (trace_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
                       if trace_us is not None else None),
        "trace_profile": ("profiles/stage1_global_%s_kernel_trace.txt" % args.workload
                          if trace_us is not None else None),
        "algorithmic_bytes_per_launch": s1_bytes,
        "algorithmic_flops_per_launch": s1_flops,
    }
    if mfma_bound:
        tflops = s1_flops / (s1_b2b_us * 1e-6) / 1e12
        roofline.update(bound="mfma", achieved=round(tflops, 1), peak=PEAK_BF16_TFLOPS,
                        unit="TFLOP/s", frac=round(tflops / PEAK_BF16_TFLOPS, 4),
                        hbm_GB_per_s=round(achieved, 1))

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "description": wl.description,
            "batch": B,
            "ctx_lens": [int(x) for x in ginp.ctx_lens],
            "page_size": wl.page_size,
            "layers": {L["kind"]: dict(num_q_heads=L["plan"].problem.num_q_heads,
                                       num_kv_heads=L["plan"].problem.num_kv_heads,
                                       head_dim=L["plan"].problem.head_dim,
                                       window=L["plan"].problem.window,
                                       num_splits=L["plan"].num_splits,
                                       algorithmic_bytes=L["bytes"]) for L in layers},
            "step_algorithmic_bytes": step_bytes,
            "kv_pool_copies_rotated": R,
            "clock_settle_steps": settle_steps,
            "k_eq_v": bool(args.k_eq_v),
            "q_len": args.q_len,
            "sliding_sink": args.sink,
            "append_in_step": bool(appends),
            "qk_norm_rope_in_step": bool(args.rope),
        },
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "graph_replay": (None if graph_us is None else {
            "us_per_step": round(graph_us, 2),
            "GB_per_s": round(step_bytes / (graph_us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100.0 * step_bytes / (graph_us * 1e-6) / 1e9 /
                                     PEAK_HBM_GBS, 2)}),
        "roofline": roofline,
        "cpu_baseline": None,
        "layers_detail": detail,
        "global_layer_range": range_detail,
        "extras": extras,
        "global_layer_cold_pct_of_hbm_peak": dict(
            [(args.workload, detail["global"]["pct_of_hbm_peak"])] if "global" in detail else [],
            **{k: v["pct_of_hbm_peak"] for k, v in range_detail.items()}),
        "provenance": provenance(),
    }

    if not args.no_cpu_baseline:
        import oracle
        oracle.build(force=False)
        host = [wl_mod.make_workload_layer(args.workload, L["kind"], q_len=args.q_len,
                                           sink=L["sink"]) for L in layers]
        if args.k_eq_v:
            for h in host:
                h.v_pool = h.k_pool
        Lq = args.q_len
        if args.rope:
            # The step before attention, by the oracle, once and untimed (its arithmetic is under
            # 0.1% of the attention's): rotated q and the appended keys.
            from oracle import rope as orope
            for h, L in zip(host, layers):
                ro = L["rope"]
                n = ro["new"]
                qb = orope.prepare_and_append(
                    n["q"], n["k"], None if args.k_eq_v else n["v"], h.k_pool, h.v_pool,
                    h.block_table, h.ctx_lens, ro["max_pos"], True, False, n["q_weight"],
                    n["k_weight"], None, ro["eps"], ro["theta"], h.k_pool.shape[-1], False)
                h.q = qb if Lq > 1 else qb[:, 0]

        # A bounded sample: the whole step when its flops are within budget, else the last k of
        # the L query tokens of every sequence (exactly those queries' outputs; the oracle's time
        # is proportional to the flops, so the step's time is the sample's scaled by the ratio).
        def sample_flops(k):
            return sum(wl_mod.algorithmic_flops(L["inp"].ctx_lens, L["spec"].num_q_heads,
                                                L["spec"].head_dim, L["spec"].window,
                                                sink=L["sink"], q_len=k) for L in layers)

        full_flops = sample_flops(Lq)

        def tail_queries(budget):
            return Lq if full_flops <= budget else max(1, int(Lq * budget // full_flops))

        def oracle_pass(k, **kw):
            refs = []
            for h in host:
                q4 = h.q if h.q_len > 1 else h.q[:, None]
                refs.append(oracle.decode_attn_multi(q4[:, Lq - k:], h.k_pool, h.v_pool,
                                                     h.block_table, h.ctx_lens, h.scale, h.window,
                                                     h.sink, **kw))
            return refs

        def describe(reps, k, what):
            if args.rope:
                what += "; the QK-norm + RoPE + append step run once by the oracle, untimed"
            if k == Lq:
                return "%d full %s steps (all layers), fp64 oracle, %s" % (reps, args.workload,
                                                                            what)
            return ("%d passes over the last %d of the %d query tokens of every sequence (all "
                    "layers; the step's time scaled by the flop ratio %.1f), fp64 oracle, %s" % (
                        reps, k, Lq, full_flops / sample_flops(k), what))

        k_all = tail_queries(CPU_SAMPLE_FLOPS)
        reps, t_cpu, refs = 0, 0.0, None
        while True:
            t_a = time.perf_counter()
            refs = oracle_pass(k_all)
            t_cpu += time.perf_counter() - t_a
            reps += 1
            if t_cpu >= args.cpu_seconds or reps >= 1000:
                break
        gpu_out = []
        for L in layers:
            o = L["out"].cpu().double().numpy()
            gpu_out.append(o[:, None] if Lq == 1 else o[:, Lq - k_all:])
        err = max(float(np.abs(g - r[0]).max()) for g, r in zip(gpu_out, refs))
        cos = min(float(((g * r[0]).sum(-1) / (np.linalg.norm(g, axis=-1) *
                                                np.linalg.norm(r[0], axis=-1))).min())
                  for g, r in zip(gpu_out, refs))
        cpu_step_s = t_cpu / reps * full_flops / sample_flops(k_all)
        result["cpu_baseline"] = {
            "value": round(step_bytes / cpu_step_s / 1e9, 3),
            "unit": "GB/s",
            "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": describe(reps, k_all, "%.1f s total" % t_cpu),
            "us_per_step": round(cpu_step_s * 1e6, 1),
            "cpu_model": _cpu_model(),
        }
        result["parity_vs_oracle"] = {"max_abs_err": err, "min_cos": cos,
                                      "query_tokens_checked": k_all}
        # The same oracle on one host thread, one pass (context for the all-cores figure).
        k_one = tail_queries(CPU_ONE_THREAD_FLOPS)
        t_a = time.perf_counter()
        oracle_pass(k_one, num_threads=1)
        one = (time.perf_counter() - t_a) * full_flops / sample_flops(k_one)
        result["cpu_baseline_one_thread"] = {
            "value": round(step_bytes / one / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "sample": describe(1, k_one, "%.1f s per step" % one)}

    result["kernel_code_sha256_16"] = kernel_code_hash()
    result["kernel_code_sha256_16_by_source"] = {k: kernel_code_hash(k) for k in KERNEL_FAMILIES}
    print(json.dumps(result), flush=True)
    return 0


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    sys.exit(main())
