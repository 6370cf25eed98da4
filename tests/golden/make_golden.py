"""Write oracle_tiny_cases.json: oracle outputs for tiny seeded inputs.

The pages print no worked example with numbers, so the stored values here come from the fp64 CPU
oracle alone (this script imports nothing else that computes attention). They serve as a
regression guard for later changes to the oracle.
Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from paged_gqa_kv_attn_amd.workloads import make_layer_inputs  # noqa: E402

CASES = [
    # name, ctx_lens, Hq, Hkv, D, S, window, seed, q_mult[, sink, q_len]
    ("global_g4_ragged", [1, 17, 40], 4, 1, 32, 16, 0, 1, 1.0),
    ("global_g8_two_seq", [33, 64], 8, 1, 32, 16, 0, 2, 2.0),
    ("sliding_g2_w20", [19, 45, 64], 4, 2, 32, 16, 20, 3, 1.0),
    ("sliding_g2_w33_page32", [70, 5], 4, 2, 32, 32, 33, 4, 1.0),
    ("sliding_g2_w20_sink5", [19, 45, 64], 4, 2, 32, 16, 20, 5, 1.0, 5, 1),
    ("global_g4_three_tokens", [2, 17, 40], 4, 1, 32, 16, 0, 6, 1.0, 0, 3),
    ("sliding_g2_w16_sink4_two_tokens", [1, 30, 70], 4, 2, 32, 16, 16, 7, 1.0, 4, 2),
]


def main():
    out_cases = []
    for name, ctx, hq, hkv, d, s, w, seed, qm, *extra in CASES:
        sink, q_len = extra if extra else (0, 1)
        inp = make_layer_inputs(ctx, hq, hkv, d, page_size=s, window=w, seed=seed, q_mult=qm,
                                sink=sink, q_len=q_len)
        if sink or q_len > 1:
            q4 = inp.q if q_len > 1 else inp.q[:, None]
            out, lse = oracle.decode_attn_multi(q4, inp.k_pool, inp.v_pool, inp.block_table,
                                                inp.ctx_lens, inp.scale, w, sink)
        else:
            out, lse = oracle.decode_attn(inp.q, inp.k_pool, inp.v_pool, inp.block_table,
                                          inp.ctx_lens, inp.scale, window=w)
        out_cases.append(dict(name=name, ctx_lens=ctx, Hq=hq, Hkv=hkv, D=d, S=s, window=w,
                              seed=seed, q_mult=qm, sink=sink, q_len=q_len, scale=inp.scale,
                              out=out.tolist(), lse=lse.tolist()))
    doc = {
        "source": "fp64 CPU oracle (oracle/oracle.c) on inputs from "
                  "paged_gqa_kv_attn_amd.workloads.make_layer_inputs; no printed worked example "
                  "exists on the pages, so these are oracle regression values, not page values",
        "cases": out_cases,
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_cases.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
