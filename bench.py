"""Benchmark: paged GQA decode on Llama-3.1-8B shapes (one MI355X).

One step = the whole decode hot path on one batch: write the step's new K/V
into the paged cache and run paged GQA attention with split-K partitions
merged by log-sum-exp, as one call (paged_gqa_decode_append: the cache write
fused into the balanced decode kernel).  The same step as two calls
(reshape_and_cache, then paged_gqa_decode) is reported beside it.  Workload: 64
sequences, Hq=32, Hkv=8, d=128, block 16, bf16 cache, context U{512..4096},
randomly permuted pages, seeded synthetic N(0,1) data.

Metric: effective KV GB/s = sum(seq_len) * 2 * Hkv * d * 2 bytes / step time.
Also reported: the decode kernel's roofline (HIP events on its launch
stream), the mixed chunked-prefill + decode batch's tokens/s, the GQA saving
against the same cache expanded per query head, cross-attention over a static
encoder cache, the decode per page size, the shared-prefix decode against the
plain decode, the 16 x 32k-token split-K decode, reshape_and_cache alone on
the decode step and on the mixed batch, and the CPU oracle's throughput on a
bounded sample as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--partition P]
       python bench.py --copy-calibration   (a plain 512 MiB device copy, for
       scaling the FETCH_SIZE / WRITE_SIZE counters of rocprofv3 to bytes)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix, published
METRIC = "paged GQA decode effective KV GB/s (% HBM peak); mixed-batch tokens/s"

# HBM traffic of one step call (paged_gqa_decode_append on this workload, both
# of its kernels), from two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE, KiB
# per dispatch) over `bench.py --profile-leg decode_step --profile-calls 20`, each
# scaled by what the same counter reads for the 512 MiB copy of
# `bench.py --copy-calibration`.  Valid only for the decode sources it was
# measured on (their SHA-256 below); otherwise reported as null.
DECODE_SOURCES = ["attention.hip", "decode_core.h", "gqa_common.h", "gqa_internal.h", "abi.hip"]
DECODE_TRAFFIC = {"sources_sha256": "8f59521f386ef659462c58c8f96826b7058c9cc0153742d94c275ab2f8089459", "partition_size": 0, "seed": 2, "fetch_bytes_per_call": 657209634, "write_bytes_per_call": 8565856, "hbm_bytes_per_call": 665775490, "fetch_factor": 1.9999, "write_factor": 1.0}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--partition", type=int, default=0, help="0 = library picks (balanced split)")
    ap.add_argument("--mixed-partition", type=int, default=0)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--no-gqa-comparison", action="store_true")
    ap.add_argument("--no-cross", action="store_true", help="skip the cross-attention leg")
    ap.add_argument("--no-page-sizes", action="store_true", help="skip the 16/32/64-token page comparison")
    ap.add_argument("--no-shared-prefix", action="store_true", help="skip the shared-prefix decode comparison")
    ap.add_argument("--no-long-context", action="store_true", help="skip the 16 x 32k-token split-K decode")
    ap.add_argument("--no-cache-write", action="store_true", help="skip the reshape_and_cache leg")
    ap.add_argument("--no-comparisons", action="store_true",
                    help="skip the unfused step and the plain decode call (so that a profiler sees the step only)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true", help="run a plain 512 MiB device copy and exit")
    ap.add_argument("--profile-leg", choices=sorted(PROFILE_LEGS), default=None,
                    help="run only this leg's call --profile-calls times (no timing, no JSON line): a short "
                         "program for rocprofv3 counter passes")
    ap.add_argument("--profile-calls", type=int, default=20)
    return ap.parse_args()


def decode_sources_sha256() -> str:
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gqa_paged_kv_attention_amd", "csrc")
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def copy_calibration():
    """A plain device-to-device copy of 512 MiB, repeated 5 times: it reads and
    writes exactly 512 MiB per dispatch, the yardstick for the HBM counters."""
    import torch
    n = 512 << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 5}), flush=True)


def warm_up(fn, stream, ms=30.0):
    """Run fn() for about `ms` of device time before it is timed: the clocks
    and caches settle over tens of milliseconds of a new kind of load (a
    matrix-bound call timed right after HBM-bound ones read 10-15% slow after
    only a few warm-up calls)."""
    import torch
    for _ in range(3):
        fn()
    per = event_time_ms(fn, 3, stream)
    for _ in range(int(ms / max(per, 1e-3))):
        fn()
    torch.cuda.synchronize()


def event_time_ms(fn, reps, stream):
    """Average duration of fn() over reps calls, from HIP events on `stream`."""
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def cold_times_ms(fn, reps, stream, flush):
    """fn() timed alone, rep by rep, each after a read of `flush` (1 GiB, filled
    once beforehand; more than the 256 MB Infinity Cache and the L2s) outside
    the event pair, so no input is cached from an earlier call.  The flush
    reads rather than writes: a write would leave the caches full of dirty
    lines, and fn() would pay for their write-back.  Returns p10, p50, p90 in ms."""
    import torch
    times = []
    for _ in range(reps):
        torch.amax(flush)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        fn()
        end.record(stream)
        end.synchronize()
        times.append(start.elapsed_time(end))
    p10, p50, p90 = np.percentile(times, [10, 50, 90])
    return {"p10_ms": round(float(p10), 5), "p50_ms": round(float(p50), 5), "p90_ms": round(float(p90), 5)}


def mixed_part_call(mb, idx, mq, mkc, mvc, mt, ml, dev):
    """A callable running chunked_prefill_paged_decode on the sequences `idx` of
    the mixed batch alone (their query rows, block-table rows and lengths; the
    same caches and pages), bf16 output."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    idx = np.asarray(idx, dtype=np.int64)
    ql = mb.query_lens.astype(np.int64)[idx]
    qsl = mb.query_start_loc.astype(np.int64)
    sub_qsl = np.zeros(len(idx) + 1, np.int32)
    sub_qsl[1:] = np.cumsum(ql)
    rows = np.concatenate([np.arange(qsl[i], qsl[i + 1]) for i in idx])
    sel = lambda t, ix: t[torch.from_numpy(ix).to(dev)].contiguous()
    q, tb, sl = sel(mq, rows), sel(mt, idx), sel(ml, idx)
    s_qsl = ops.to_device(sub_qsl, dev)
    T = int(sub_qsl[-1])
    max_sl = int(mb.seq_lens[idx].max())
    out = torch.empty(T, mb.num_heads, mb.head_dim, dtype=torch.bfloat16, device=dev)
    dims = ops.make_dims(num_seqs=len(idx), num_heads=mb.num_heads, key_cache=mkc, block_tables=tb, q_dtype=q.dtype,
                         out_dtype=out.dtype)
    ws = torch.zeros(max(ops.mixed_workspace_size(dims, T, max_sl, 0), 1), dtype=torch.uint8, device=dev)
    return ops.chunked_prefill_paged_decode(q, mkc, mvc, tb, sl, s_qsl, int(ql.max()), max_sl, mb.scale,
                                            partition_size=0, out=out, workspace=ws, bind=True)


def mixed_part_ms(mb, idx, mq, mkc, mvc, mt, ml, dev, stream, reps=50):
    """ms per call of mixed_part_call's callable."""
    f = mixed_part_call(mb, idx, mq, mkc, mvc, mt, ml, dev)
    warm_up(f, stream)
    return event_time_ms(f, reps, stream)


# Legs that --profile-leg can run alone (workload, call):
#   decode_step    the headline step (paged_gqa_decode_append, llama31_8b_decode)
#   mixed          chunked_prefill_paged_decode on the whole mixed batch, bf16 output
#   mixed_prefill  the mixed batch's 51 prefill chunks alone, same call
#   mixed_decode   the mixed batch's 205 decodes alone, same call
#   longctx512     16 x 32k tokens, paged_gqa_decode with 512-token partitions
#   longctx        the same with the library's split
#   mqa            paged_gqa_decode on the Llama-2-7B sweep with one kv head (Hq = 32)
PROFILE_LEGS = ("decode_step", "mixed", "mixed_prefill", "mixed_decode", "longctx512", "longctx", "mqa", "cross_chunk")


def profile_leg(name, calls, dev, stream, seed):
    """Build one leg's inputs, run its call once, then `calls` more times; print one line."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl
    up = lambda a: ops.to_device(a, dev)
    if name == "decode_step":
        bt = wl.llama31_8b_decode(seed=seed)
        q, kc, vc, nk, nv = up(bt.query), up(bt.key_cache), up(bt.value_cache), up(bt.new_key), up(bt.new_value)
        tb, sl = up(bt.block_tables), up(bt.seq_lens)
        out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
        f = lambda: ops.paged_gqa_decode_append(q, nk, nv, kc, vc, tb, sl, bt.max_seq_len, bt.scale, out=out)
    elif name.startswith("mixed"):
        mb = wl.mixed_chunked(seed=4)
        mq, mkc, mvc = up(mb.query), up(mb.key_cache), up(mb.value_cache)
        mt, ml, mqsl = up(mb.block_tables), up(mb.seq_lens), up(mb.query_start_loc)
        ops.reshape_and_cache(up(mb.new_key), up(mb.new_value), mkc, mvc, mt, ml, mqsl)
        ql = mb.query_lens.astype(np.int64)
        idx = {"mixed": np.arange(mb.num_seqs), "mixed_prefill": np.where(ql > 1)[0],
               "mixed_decode": np.where(ql == 1)[0]}[name]
        f = mixed_part_call(mb, idx, mq, mkc, mvc, mt, ml, dev)
    elif name == "cross_chunk":
        # 16 chunks of 256 decoder rows over the static encoder cache (8-wave launch)
        bt = wl.cross_attention(seed=6, query_len=256)
        q, kc, vc = up(bt.query), up(bt.key_cache), up(bt.value_cache)
        tb, el, qsl = up(bt.block_tables), up(bt.seq_lens), up(bt.query_start_loc)
        out = torch.empty(bt.num_tokens, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
        f = lambda: ops.paged_cross_attention(q, kc, vc, tb, el, qsl, bt.max_query_len, bt.max_seq_len, bt.scale,
                                              out=out)
    else:
        bt = wl.longctx_splitk(seed=5) if name.startswith("longctx") else wl.llama2_7b_sweep(1, seed=3)
        q, kc, vc, tb, sl = up(bt.query), up(bt.key_cache), up(bt.value_cache), up(bt.block_tables), up(bt.seq_lens)
        out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
        part = 512 if name == "longctx512" else 0
        f = lambda: ops.paged_gqa_decode(q, kc, vc, tb, sl, bt.max_seq_len, bt.scale, partition_size=part, out=out)
    f()
    torch.cuda.synchronize()
    for _ in range(calls):
        f()
    torch.cuda.synchronize()
    print(f"profile leg {name}: {calls} calls after one warm-up call", flush=True)


def measured_mfma_peak(dev, stream):
    """bf16 matrix-core rate this device sustains: the library's probe (8 waves
    per compute unit, 8 independent chains of v_mfma_f32_16x16x32_bf16 each),
    timed with HIP events after a warm-up.  TFLOP/s."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    groups, iters = 2 * cus, 4000
    out = torch.empty(4 * groups, dtype=torch.float32, device=dev)
    flops = ops.probe_mfma_bf16(out, groups, iters, stream)
    f = lambda: ops.probe_mfma_bf16(out, groups, iters, stream)
    warm_up(f, stream)
    ms = min(event_time_ms(f, 10, stream) for _ in range(3))
    return round(flops / (ms * 1e-3) / 1e12, 1)


def stream_copy_gbs(buf, stream, reps=20):
    """HBM bandwidth of a plain device copy here: one half of `buf` (1 GiB)
    copied into the other, 512 MiB read + 512 MiB written, GB/s of bytes moved."""
    half = buf.numel() // 2
    src, dst = buf[:half], buf[half:]
    f = lambda: dst.copy_(src)
    warm_up(f, stream, 10.0)
    return round(buf.numel() * buf.element_size() / (event_time_ms(f, reps, stream) * 1e-3) / 1e9, 1)


def cpu_baseline(bt, seconds):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same workload.

    The sample is whole passes over the batch's sequences (after the step's cache
    write), repeated until `seconds` of CPU time have been spent.
    """
    from threadpoolctl import threadpool_limits
    from oracle import cache_write_ref, decode_ref
    kc, vc = cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                             bt.query_start_loc)
    per_tok = 2 * bt.num_kv_heads * bt.head_dim * bt.kv_itemsize
    done_bytes, n_seq, t0 = 0, 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < seconds:
            for b in range(bt.num_seqs):
                decode_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale, seqs=[b])
                done_bytes += int(bt.seq_lens[b]) * per_tok
                n_seq += 1
                if time.perf_counter() - t0 >= seconds:
                    break
    el = time.perf_counter() - t0
    return {"value": round(done_bytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host_cores_available": len(os.sched_getaffinity(0)),
            "sample": f"{n_seq} sequence decodes ({n_seq / bt.num_seqs:.2f} passes over the {bt.num_seqs}-sequence "
                      f"batch), numpy fp64 with BLAS limited to 1 thread, {el:.1f} s"}


def gqa_comparison(dev, stream, reps, flush=None):
    """The GQA saving at kernel level, on the Llama-2-7B decode sweep shape (128
    sequences, Hq=32, d=128, context U{32..1024}).  The GQA batch (Hkv=8) is timed
    as it is and with its K/V expanded per query head (Hkv=32, the cache an
    MHA-style kernel reads; outputs must agree), and an MQA batch (Hkv=1) with
    the same lengths."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl

    def run(bt, kc, vc):
        q, tb, sl = ops.to_device(bt.query, dev), ops.to_device(bt.block_tables, dev), ops.to_device(bt.seq_lens, dev)
        out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
        dims = ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=kc, block_tables=tb,
                             q_dtype=q.dtype, out_dtype=out.dtype)
        ws = torch.zeros(max(ops.decode_workspace_size(dims, bt.max_seq_len, 0), 1), dtype=torch.uint8, device=dev)
        f = ops.paged_gqa_decode(q, kc, vc, tb, sl, bt.max_seq_len, bt.scale, out=out, workspace=ws, bind=True)
        warm_up(f, stream)
        ms = event_time_ms(f, reps, stream)
        cold = cold_times_ms(f, 20, stream, flush) if flush is not None else None
        return ms, out.clone(), cold

    gqa = wl.llama2_7b_sweep(8, seed=3)
    kc, vc = ops.to_device(gqa.key_cache, dev), ops.to_device(gqa.value_cache, dev)
    t_gqa, o_gqa, c_gqa = run(gqa, kc, vc)
    G = gqa.num_heads // gqa.num_kv_heads
    kce, vce = kc.repeat_interleave(G, dim=1).contiguous(), vc.repeat_interleave(G, dim=1).contiguous()
    del kc, vc
    t_exp, o_exp, c_exp = run(gqa, kce, vce)
    del kce, vce
    mqa = wl.llama2_7b_sweep(1, seed=3)
    t_mqa, _, c_mqa = run(mqa, ops.to_device(mqa.key_cache, dev), ops.to_device(mqa.value_cache, dev))
    torch.cuda.synchronize()
    tokens = int(gqa.seq_lens.sum())
    per_tok = 2 * gqa.head_dim * 2
    return {"workload": "llama2_7b_sweep (128 seqs, Hq=32, d=128, context U{32..1024}, bf16)",
            "expanded_kv_us": round(t_exp * 1e3, 2), "gqa_us": round(t_gqa * 1e3, 2), "mqa_us": round(t_mqa * 1e3, 2),
            "kv_bytes": {"expanded": tokens * per_tok * gqa.num_heads, "gqa": tokens * per_tok * gqa.num_kv_heads,
                         "mqa": tokens * per_tok},
            "expanded_over_gqa": round(t_exp / t_gqa, 3),
            # back-to-back calls above; each call alone after a cache flush here (the MQA set,
            # 34 MB, fits in the Infinity Cache when calls follow each other)
            "cold_p50_us": None if c_gqa is None else {"expanded": round(c_exp["p50_ms"] * 1e3, 2),
                                                      "gqa": round(c_gqa["p50_ms"] * 1e3, 2),
                                                      "mqa": round(c_mqa["p50_ms"] * 1e3, 2)},
            "max_abs_diff_expanded_vs_gqa": float((o_exp - o_gqa).abs().max())}


def cross_attention_leg(dev, stream, reps):
    """Cross-attention over a static encoder cache (16 sequences, Hq=32, Hkv=8,
    d=128, bf16, encoder lengths U{1024..6400}): a decode step (one decoder row
    per sequence, HBM-bound) and a chunk of 256 decoder rows per sequence
    (matrix-bound).  No cache write: the encoder cache is static."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl

    res = {"workload": "cross_attention (16 seqs, Hq=32, Hkv=8, d=128, encoder U{1024..6400}, bf16)"}
    for q_len in (1, 256):
        bt = wl.cross_attention(seed=6, query_len=q_len)
        up = lambda a: ops.to_device(a, dev)
        q, kc, vc = up(bt.query), up(bt.key_cache), up(bt.value_cache)
        tb, el, qsl = up(bt.block_tables), up(bt.seq_lens), up(bt.query_start_loc)
        out = torch.empty(bt.num_tokens, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
        dims = ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=kc, block_tables=tb,
                             q_dtype=q.dtype, out_dtype=out.dtype)
        ws = torch.zeros(max(ops.cross_workspace_size(dims, bt.num_tokens, bt.max_seq_len, 0), 1),
                         dtype=torch.uint8, device=dev)
        f = lambda: ops.paged_cross_attention(q, kc, vc, tb, el, qsl, bt.max_query_len, bt.max_seq_len, bt.scale,
                                              out=out, workspace=ws)
        warm_up(f, stream)
        ms = event_time_ms(f, reps, stream)
        enc = bt.seq_lens.astype(np.int64)
        if q_len == 1:
            gbs = bt.kv_bytes() / (ms * 1e-3) / 1e9
            res["decode_step"] = {"us": round(ms * 1e3, 2), "kv_bytes": bt.kv_bytes(), "kv_gbs": round(gbs, 1),
                                  "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        else:
            flops = 4 * bt.head_dim * bt.num_heads * int(np.sum(enc * q_len))
            res[f"chunk_{q_len}"] = {"us": round(ms * 1e3, 2), "gflop": round(flops / 1e9, 3),
                                     "tokens_per_s": round(bt.num_tokens / (ms * 1e-3), 1),
                                     "mfma_util": round(flops / (ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12), 4)}
        del q, kc, vc, out, ws
    return res


def long_context_leg(dev, stream, reps, flush=None):
    """Long-context split-K decode: 16 sequences of 32768 tokens, Hq=64, Hkv=8,
    d=128, bf16 (2.15 GB of K+V), with 512-token partitions merged by
    log-sum-exp (splitk_lse_reduce inside the call) and with the split the
    library picks (balanced workers + merge)."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl

    bt = wl.longctx_splitk(seed=5)
    up = lambda a: ops.to_device(a, dev)
    q, kc, vc, tb, sl = up(bt.query), up(bt.key_cache), up(bt.value_cache), up(bt.block_tables), up(bt.seq_lens)
    out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
    dims = ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=kc, block_tables=tb,
                         q_dtype=q.dtype, out_dtype=out.dtype)
    res = {"workload": "longctx_splitk (16 seqs x 32768 tokens, Hq=64, Hkv=8, d=128, bf16)",
           "kv_bytes": bt.kv_bytes()}
    for part in (512, 0):
        ws = torch.zeros(max(ops.decode_workspace_size(dims, bt.max_seq_len, part), 1), dtype=torch.uint8,
                         device=dev)
        f = ops.paged_gqa_decode(q, kc, vc, tb, sl, bt.max_seq_len, bt.scale, partition_size=part, out=out,
                                 workspace=ws, bind=True)
        warm_up(f, stream)
        ms = event_time_ms(f, reps, stream)
        gbs = bt.kv_bytes() / (ms * 1e-3) / 1e9
        leg = {"us": round(ms * 1e3, 2), "kv_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if flush is not None:
            leg["cold"] = cold_times_ms(f, 10, stream, flush)
        res["partition_512" if part else "library_split"] = leg
        del ws
    del q, kc, vc, out
    return res


def cache_write_leg(dev, stream, reps, seed):
    """reshape_and_cache alone: the decode step's 64 new tokens and the mixed
    batch's 8166 (prefill chunks and decodes), each token's K and V rows read
    once and written once (2 * Hkv * d * 2 bytes each way per token)."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl

    res = {}
    for name, bt in (("decode_step", wl.llama31_8b_decode(seed=seed)), ("mixed_batch", wl.mixed_chunked(seed=4))):
        up = lambda a: ops.to_device(a, dev)
        nk, nv, kc, vc = up(bt.new_key), up(bt.new_value), up(bt.key_cache), up(bt.value_cache)
        tb, sl, qsl = up(bt.block_tables), up(bt.seq_lens), up(bt.query_start_loc)
        f = ops.reshape_and_cache(nk, nv, kc, vc, tb, sl, qsl, bind=True)
        warm_up(f, stream)
        ms = event_time_ms(f, reps, stream)
        nbytes = 2 * bt.num_tokens * 2 * bt.num_kv_heads * bt.head_dim * bt.kv_itemsize   # read + written
        res[name] = {"tokens": bt.num_tokens, "us": round(ms * 1e3, 2), "bytes": nbytes,
                     "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        del nk, nv, kc, vc
    return res


def page_size_leg(dev, stream, reps, seed):
    """The decode call on the same workload (same lengths and seed) with 16-,
    32- and 64-token pages: the kernels' tiles do not depend on the page size,
    but larger pages make each (page, kv head) slab a longer contiguous read."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl

    res = {"workload": "llama31_8b_decode (64 seqs, Hq=32, Hkv=8, d=128, context U{512..4096}, bf16)",
           "call": "paged_gqa_decode, partition_size 0"}
    for bs in (16, 32, 64):
        bt = wl.llama31_8b_decode(seed=seed, block_size=bs)
        up = lambda a: ops.to_device(a, dev)
        q, kc, vc, tb, sl = up(bt.query), up(bt.key_cache), up(bt.value_cache), up(bt.block_tables), up(bt.seq_lens)
        out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
        dims = ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=kc, block_tables=tb,
                             q_dtype=q.dtype, out_dtype=out.dtype)
        ws = torch.zeros(max(ops.decode_workspace_size(dims, bt.max_seq_len, 0), 1), dtype=torch.uint8, device=dev)
        f = ops.paged_gqa_decode(q, kc, vc, tb, sl, bt.max_seq_len, bt.scale, out=out, workspace=ws, bind=True)
        warm_up(f, stream)
        ms = event_time_ms(f, reps, stream)
        res[f"bs{bs}"] = {"us": round(ms * 1e3, 2), "kv_gbs": round(bt.kv_bytes() / (ms * 1e-3) / 1e9, 1),
                          "page_slab_bytes": bs * bt.head_dim * 2}
        del q, kc, vc, out, ws
    return res


def shared_prefix_leg(dev, stream, reps):
    """Groups of sequences sharing a prompt prefix (prefix-cached pages): the
    plain decode over the aliased block tables, the shared-prefix decode, and
    the plain decode over private copies of the prefix, on the same tokens."""
    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl

    res = {"workload": "shared_prefix_decode (groups of sequences sharing a prompt, suffixes U{16..512}, "
                       "Hq=32, Hkv=8, d=128, bf16)"}
    for groups, size, prefix in ((4, 16, 2048), (4, 64, 4096)):
        bt, gs, pl = wl.shared_prefix_decode(seed=7, num_groups=groups, group_size=size, prefix_len=prefix)
        up = lambda a: ops.to_device(a, dev)
        q, kc, vc, tb, sl, dgs, dpl = (up(x) for x in (bt.query, bt.key_cache, bt.value_cache, bt.block_tables,
                                                        bt.seq_lens, gs, pl))
        out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
        dims = ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=kc, block_tables=tb,
                             q_dtype=q.dtype, out_dtype=out.dtype)
        ws = torch.zeros(max(ops.shared_prefix_workspace_size(dims, groups, size, bt.max_seq_len, 0),
                             ops.decode_workspace_size(dims, bt.max_seq_len, 0), 1), dtype=torch.uint8, device=dev)
        plain = ops.paged_gqa_decode(q, kc, vc, tb, sl, bt.max_seq_len, bt.scale, out=out, workspace=ws, bind=True)
        shared = lambda: ops.paged_gqa_decode_shared_prefix(q, kc, vc, tb, sl, dgs, dpl, size, bt.max_seq_len,
                                                            bt.scale, out=out, workspace=ws)
        times = {}
        for name, f in (("plain_aliased", plain), ("shared_prefix", shared)):
            warm_up(f, stream)
            times[name] = event_time_ms(f, reps, stream)
        o_shared = out.clone()
        plain()
        torch.cuda.synchronize()
        max_diff = float((out - o_shared).abs().max())
        # every sequence with pages of its own: a batch of the same lengths without aliasing
        bt2 = wl.make_batch(name="private", seed=7, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                            seq_lens=bt.seq_lens, query_lens=bt.query_lens, dtype=bt.dtype)
        kc2, vc2, tb2 = up(bt2.key_cache), up(bt2.value_cache), up(bt2.block_tables)
        private = ops.paged_gqa_decode(q, kc2, vc2, tb2, sl, bt.max_seq_len, bt.scale, out=out, workspace=ws, bind=True)
        warm_up(private, stream)
        times["plain_private"] = event_time_ms(private, reps, stream)
        unique = (prefix * groups + int(bt.seq_lens.sum()) - prefix * bt.num_seqs) * bt.num_kv_heads * 512
        res[f"g{groups}x{size}_p{prefix}"] = {
            "us": {k: round(v * 1e3, 2) for k, v in times.items()},
            "speedup_vs_aliased": round(times["plain_aliased"] / times["shared_prefix"], 2),
            "unique_kv_bytes": unique, "logical_kv_bytes": bt.kv_bytes(),
            "unique_gbs_shared": round(unique / (times["shared_prefix"] * 1e-3) / 1e9, 1),
            "max_abs_diff_vs_plain": max_diff}
        del q, kc, vc, kc2, vc2, out, ws
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library runs on one GPU; multi-GPU runs are not supported "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        sys.exit(2)

    import torch
    from gqa_paged_kv_attention_amd import ops
    from gqa_paged_kv_attention_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration()
        return
    ops.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.profile_leg:
        profile_leg(args.profile_leg, args.profile_calls, dev, stream, args.seed)
        return

    bt = wl.llama31_8b_decode(seed=args.seed)
    up = lambda a: ops.to_device(a, dev)
    q, kc, vc = up(bt.query), up(bt.key_cache), up(bt.value_cache)
    nk, nv = up(bt.new_key), up(bt.new_value)
    tables, lens, qsl = up(bt.block_tables), up(bt.seq_lens), up(bt.query_start_loc)
    out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device=dev)
    dims = ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=kc, block_tables=tables,
                         q_dtype=q.dtype, out_dtype=out.dtype)
    ws_bytes = ops.decode_workspace_size(dims, bt.max_seq_len, args.partition)
    ws = torch.zeros(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    # Calls bound once (arguments checked and marshalled before the timed
    # loops), so that the binding's per-call host checks do not pace the GPU.
    decode = ops.paged_gqa_decode(q, kc, vc, tables, lens, bt.max_seq_len, bt.scale, partition_size=args.partition,
                                  out=out, workspace=ws, bind=True)
    cache_write = ops.reshape_and_cache(nk, nv, kc, vc, tables, lens, qsl, bind=True)

    def step_unfused():
        cache_write()
        decode()

    step = ops.paged_gqa_decode_append(q, nk, nv, kc, vc, tables, lens, bt.max_seq_len, bt.scale,
                                       partition_size=args.partition, out=out, workspace=ws, bind=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    kv_bytes = bt.kv_bytes()
    gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: the step's call, timed with HIP events on its stream
    reps = max(20, args.steps // 2)
    call_ms = event_time_ms(step, reps, stream)
    achieved = kv_bytes / (call_ms * 1e-3) / 1e9
    traffic = None
    if DECODE_TRAFFIC is not None and DECODE_TRAFFIC["sources_sha256"] == decode_sources_sha256() \
            and args.partition == DECODE_TRAFFIC["partition_size"] and args.seed == DECODE_TRAFFIC["seed"]:
        traffic = DECODE_TRAFFIC["hbm_bytes_per_call"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "paged_gqa_decode_append call (balanced decode kernel with the cache write fused + "
                          "merge kernel)", "avg_ms": round(call_ms, 5), "bytes_per_launch": kv_bytes}
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    roofline["cold"] = dict(cold_times_ms(step, 20, stream, flush),
                            note="each call alone after a 1 GiB read (caches flushed); achieved uses back-to-back calls")
    # the same achieved rate against a plain device copy's
    copy_gbs = stream_copy_gbs(flush, stream)
    roofline["measured_copy"] = {"gbs": copy_gbs, "frac": round(achieved / copy_gbs, 4),
                                 "kernel": "torch copy_ of 512 MiB (read + write)"}
    # the same step as two calls, and the attention call alone
    unfused_ms = decode_ms = None
    if not args.no_comparisons:
        # warmed first: the copy above leaves the caches full of dirty lines
        warm_up(step_unfused, stream)
        unfused_ms = event_time_ms(step_unfused, reps, stream)
        warm_up(decode, stream)
        decode_ms = event_time_ms(decode, reps, stream)

    record = {"metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
              "config": {"workload": "llama31_8b_decode", "num_seqs": bt.num_seqs, "num_heads": bt.num_heads,
                         "num_kv_heads": bt.num_kv_heads, "head_dim": bt.head_dim, "block_size": bt.block_size,
                         "context": "U{512..4096}", "sum_seq_len": int(bt.seq_lens.sum()), "seed": args.seed,
                         "partition_size": args.partition, "kv_dtype": "bf16", "out_dtype": "fp32",
                         "step": "paged_gqa_decode_append (cache write fused into the decode)"},
              "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
              "roofline": roofline}
    if not args.no_comparisons:
        record["unfused_step"] = {"calls": "reshape_and_cache + paged_gqa_decode", "ms": round(unfused_ms, 5),
                                  "kv_gbs": round(kv_bytes / (unfused_ms * 1e-3) / 1e9, 2)}
        record["decode_call"] = {"call": "paged_gqa_decode (no cache write)", "ms": round(decode_ms, 5),
                                 "kv_gbs": round(kv_bytes / (decode_ms * 1e-3) / 1e9, 2),
                                 "hbm_frac": round(kv_bytes / (decode_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    if not args.no_mixed:
        mb = wl.mixed_chunked(seed=4)
        mq, mkc, mvc = up(mb.query), up(mb.key_cache), up(mb.value_cache)
        mnk, mnv = up(mb.new_key), up(mb.new_value)
        mt, ml, mqsl = up(mb.block_tables), up(mb.seq_lens), up(mb.query_start_loc)
        ops.reshape_and_cache(mnk, mnv, mkc, mvc, mt, ml, mqsl)
        ql = mb.query_lens.astype(np.int64)
        prior = mb.seq_lens.astype(np.int64) - ql
        flops = 4 * mb.head_dim * mb.num_heads * int(np.sum(ql * prior + ql * (ql + 1) // 2))
        rows = mb.num_tokens * mb.num_heads * mb.head_dim
        times = {}
        # bf16 output (what a serving engine consumes) and fp32 output
        for name, odt in (("bf16", torch.bfloat16), ("fp32", torch.float32)):
            mout = torch.empty(mb.num_tokens, mb.num_heads, mb.head_dim, dtype=odt, device=dev)
            mdims = ops.make_dims(num_seqs=mb.num_seqs, num_heads=mb.num_heads, key_cache=mkc, block_tables=mt,
                                  q_dtype=mq.dtype, out_dtype=mout.dtype)
            mws = torch.zeros(max(ops.mixed_workspace_size(mdims, mb.num_tokens, mb.max_seq_len,
                                                           args.mixed_partition), 1), dtype=torch.uint8, device=dev)

            mixed = ops.chunked_prefill_paged_decode(mq, mkc, mvc, mt, ml, mqsl, mb.max_query_len, mb.max_seq_len,
                                                     mb.scale, partition_size=args.mixed_partition, out=mout,
                                                     workspace=mws, bind=True)
            warm_up(mixed, stream)
            times[name] = event_time_ms(mixed, 50, stream)
            if name == "bf16":
                mixed_cold = cold_times_ms(mixed, 20, stream, flush)
        mixed_ms = times["bf16"]
        mfma_peak = measured_mfma_peak(dev, stream)
        # diagnostics: each part of the batch alone through the same entry point
        pf_idx, dec_idx = np.where(ql > 1)[0], np.where(ql == 1)[0]
        pf_flops = 4 * mb.head_dim * mb.num_heads * int(np.sum(ql[pf_idx] * prior[pf_idx] +
                                                                ql[pf_idx] * (ql[pf_idx] + 1) // 2))
        dec_kv = int(mb.seq_lens[dec_idx].astype(np.int64).sum()) * 2 * mb.num_kv_heads * mb.head_dim * mb.kv_itemsize
        pf_ms = mixed_part_ms(mb, pf_idx, mq, mkc, mvc, mt, ml, dev, stream)
        dec_ms = mixed_part_ms(mb, dec_idx, mq, mkc, mvc, mt, ml, dev, stream)
        record["mixed_batch"] = {"workload": "mixed_chunked (256 seqs, 80% decode, lognormal chunks)",
                                 "num_tokens": mb.num_tokens, "out_dtype": "bf16", "ms": round(mixed_ms, 5),
                                 "tokens_per_s": round(mb.num_tokens / (mixed_ms * 1e-3), 1),
                                 "algorithmic_gflop": round(flops / 1e9, 3),
                                 "mfma_util": round(flops / (mixed_ms * 1e-3) / (BF16_MFMA_PEAK_TFLOPS * 1e12), 4),
                                 "measured_mfma_peak_tflops": mfma_peak,
                                 "mfma_util_vs_measured_peak": round(flops / (mixed_ms * 1e-3) / (mfma_peak * 1e12), 4),
                                 "cold": dict(mixed_cold, note="each call alone after a 1 GiB read (caches flushed)"),
                                 "kv_gb": round(mb.kv_bytes() / 1e9, 4),
                                 # K/V once, queries once, outputs once: the batch's least HBM traffic
                                 "min_hbm_gb": round((mb.kv_bytes() + rows * 2 + rows * 2) / 1e9, 4),
                                 "parts_alone": {
                                     "prefill": {"seqs": int(len(pf_idx)), "ms": round(pf_ms, 5),
                                                 "gflop": round(pf_flops / 1e9, 3),
                                                 "mfma_util": round(pf_flops / (pf_ms * 1e-3) /
                                                                    (BF16_MFMA_PEAK_TFLOPS * 1e12), 4)},
                                     "decode": {"seqs": int(len(dec_idx)), "ms": round(dec_ms, 5),
                                                "kv_bytes": dec_kv,
                                                "kv_gbs": round(dec_kv / (dec_ms * 1e-3) / 1e9, 1)}},
                                 "fp32_out": {"ms": round(times["fp32"], 5),
                                              "tokens_per_s": round(mb.num_tokens / (times["fp32"] * 1e-3), 1),
                                              "min_hbm_gb": round((mb.kv_bytes() + rows * 2 + rows * 4) / 1e9, 4)}}

    if not args.no_gqa_comparison:
        record["gqa_comparison"] = gqa_comparison(dev, stream, 30, flush)

    if not args.no_cross:
        record["cross_attention"] = cross_attention_leg(dev, stream, 30)

    if not args.no_page_sizes:
        record["page_sizes"] = page_size_leg(dev, stream, 50, args.seed)

    if not args.no_shared_prefix:
        record["shared_prefix"] = shared_prefix_leg(dev, stream, 30)

    if not args.no_long_context:
        record["long_context"] = long_context_leg(dev, stream, 20, flush)

    if not args.no_cache_write:
        record["cache_write"] = cache_write_leg(dev, stream, 50, args.seed)

    if not args.no_cpu_baseline:
        record["cpu_baseline"] = cpu_baseline(bt, args.cpu_seconds)
    print(json.dumps(record), flush=True)


if __name__ == "__main__":
    main()
