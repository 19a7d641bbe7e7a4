"""Write the stored expected outputs in this folder.

Every value is computed by the CPU fp64 oracle (oracle/attention.py) on inputs
drawn by the seeded generator (gqa_paged_kv_attention_amd/workloads.py); this
script calls nothing else.  The pages print no worked example of the
operation, so the fixtures pin the oracle's outputs on small cases: a CPU test
checks that the oracle still produces them, and GPU tests compare the HIP path
with the stored values without running the oracle.

Usage: python tests/golden/make_golden.py   (rewrites oracle_small_cases.json)
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from gqa_paged_kv_attention_amd import workloads as wl  # noqa: E402
from oracle import decode_ref, paged_attention_ref  # noqa: E402

# name -> generator arguments and the oracle mode.  Sources of the definitions:
# "[Performance] Use optimized kernels for MQA/GQA" (opening post: head map,
# paged cache), "[Kernel] [V1] Further optimizations to ROCm (Triton) Backend to
# better handle GQA" (mixed batch), "[Core] More-efficient cross-attention
# parallel QKV computation" (cross-attention phases).
CASES = {
    "decode_fp32": dict(mode="decode", seed=11, num_heads=4, num_kv_heads=2, head_dim=64, block_size=16,
                        seq_lens=[1, 17, 40], query_lens=[1, 1, 1], dtype=wl.F32),
    "mixed_bf16": dict(mode="causal", seed=12, num_heads=4, num_kv_heads=1, head_dim=64, block_size=16,
                       seq_lens=[5, 40, 70], query_lens=[1, 3, 5], dtype=wl.BF16),
    "cross_bf16": dict(mode="cross", seed=13, num_heads=4, num_kv_heads=2, head_dim=64, block_size=32,
                       seq_lens=[0, 9, 50], query_lens=[2, 3, 1], dtype=wl.BF16),
}


def build(case: dict) -> wl.PagedBatch:
    kw = {k: v for k, v in case.items() if k != "mode"}
    return wl.make_batch(name="golden", cross=case["mode"] == "cross", **kw)


def expected(case: dict, bt: wl.PagedBatch):
    if case["mode"] == "decode":
        return decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                          bt.scale)
    return paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                               bt.query_start_loc, bt.num_kv_heads, bt.scale, causal=case["mode"] != "cross")


def main():
    out = {"written_by": "tests/golden/make_golden.py (CPU fp64 oracle only)", "cases": {}}
    for name, case in CASES.items():
        ref = expected(case, build(case))
        out["cases"][name] = {"args": case, "shape": list(ref.shape),
                              "out": [float(f"{x:.9g}") for x in ref.reshape(-1)]}
    with open(os.path.join(HERE, "oracle_small_cases.json"), "w") as f:
        json.dump(out, f, separators=(",", ":"))
        f.write("\n")


if __name__ == "__main__":
    main()
