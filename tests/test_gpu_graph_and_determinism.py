"""Reproducibility and HIP-graph capture of the attention calls.

Every call (the fused decode-and-append too) is bitwise deterministic (no atomics in the arithmetic; merges
run in a fixed order), so two runs on the same inputs agree bit for bit.
The library allocates nothing and never synchronises, so a serving loop can
capture its calls in a HIP graph (torch.cuda.graph on ROCm) and replay them;
each replay must equal the eager result.  Replays are interleaved with eager
work and host synchronisation.
"""
import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import ops
from gqa_paged_kv_attention_amd import workloads as wl
from tests.gpu_util import DeviceBatch, have_gpu

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def dims_of(bt, dev, out_dtype=torch.float32):
    return ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=dev.key_cache,
                         block_tables=dev.block_tables, q_dtype=dev.query.dtype, out_dtype=out_dtype)


def shared_batch():
    return wl.shared_prefix_decode(seed=21, num_groups=3, group_size=6, prefix_len=512, suffix_lo=1, suffix_hi=200)


def calls():
    """(name, batch, function(out, workspace) running the call, output shape, workspace bytes)."""
    out = []
    bt = wl.llama31_8b_decode(seed=12, num_seqs=24, ctx_lo=100, ctx_hi=3000)
    d = DeviceBatch(bt)
    for P in (0, 256):
        n = ops.decode_workspace_size(dims_of(bt, d), bt.max_seq_len, P)
        out.append((f"decode_P{P}", (bt.num_seqs, bt.num_heads, bt.head_dim), n,
                    lambda o, w, d=d, bt=bt, P=P: ops.paged_gqa_decode(
                        d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, bt.max_seq_len, bt.scale,
                        partition_size=P, out=o, workspace=w)))
    # the fused append writes each sequence's new token into its slot; a repeated
    # call writes the same bytes again, so every replay must give the same output
    for P in (0, 256):
        da = DeviceBatch(bt)
        n = ops.decode_workspace_size(dims_of(bt, da), bt.max_seq_len, P)
        out.append((f"append_P{P}", (bt.num_seqs, bt.num_heads, bt.head_dim), n,
                    lambda o, w, d=da, bt=bt, P=P: ops.paged_gqa_decode_append(
                        d.query, d.new_key, d.new_value, d.key_cache, d.value_cache, d.block_tables, d.seq_lens,
                        bt.max_seq_len, bt.scale, partition_size=P, out=o, workspace=w)))
    # MQA over a small cache: two 16-row units per kv head on one XCD, 8 waves per work-group
    qb = wl.llama2_7b_sweep(1, seed=15, num_seqs=37)
    dq = DeviceBatch(qb)
    n = ops.decode_workspace_size(dims_of(qb, dq), qb.max_seq_len, 0)
    out.append(("decode_mqa", (qb.num_seqs, qb.num_heads, qb.head_dim), n,
                lambda o, w, d=dq, bt=qb: ops.paged_gqa_decode(
                    d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, bt.max_seq_len, bt.scale,
                    out=o, workspace=w)))
    mb = wl.mixed_chunked(seed=13, num_seqs=40, token_budget=1500)
    dm = DeviceBatch(mb)
    n = ops.mixed_workspace_size(dims_of(mb, dm), mb.num_tokens, mb.max_seq_len, 0)
    out.append(("mixed", (mb.num_tokens, mb.num_heads, mb.head_dim), n,
                lambda o, w, d=dm, bt=mb: ops.chunked_prefill_paged_decode(
                    d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, d.query_start_loc,
                    bt.max_query_len, bt.max_seq_len, bt.scale, out=o, workspace=w)))
    # prefill-heavy: four 512-token chunks beside two decodes take the 8-wave launch
    hb = wl.make_batch(name="heavy", seed=16, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       seq_lens=[768, 768, 768, 768, 3000, 100], query_lens=[512, 512, 512, 512, 1, 1], dtype=wl.BF16)
    dh = DeviceBatch(hb)
    n = ops.mixed_workspace_size(dims_of(hb, dh), hb.num_tokens, hb.max_seq_len, 0)
    out.append(("mixed_8_waves", (hb.num_tokens, hb.num_heads, hb.head_dim), n,
                lambda o, w, d=dh, bt=hb: ops.chunked_prefill_paged_decode(
                    d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, d.query_start_loc,
                    bt.max_query_len, bt.max_seq_len, bt.scale, out=o, workspace=w)))
    cb = wl.cross_attention(seed=14, num_seqs=6, enc_lo=100, enc_hi=2000, query_len=40)
    dc = DeviceBatch(cb)
    n = ops.cross_workspace_size(dims_of(cb, dc), cb.num_tokens, cb.max_seq_len, 0)
    out.append(("cross", (cb.num_tokens, cb.num_heads, cb.head_dim), n,
                lambda o, w, d=dc, bt=cb: ops.paged_cross_attention(
                    d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, d.query_start_loc,
                    bt.max_query_len, bt.max_seq_len, bt.scale, out=o, workspace=w)))
    sb, gs, pl = shared_batch()
    ds = DeviceBatch(sb)
    dgs, dpl = ops.to_device(gs), ops.to_device(pl)
    n = ops.shared_prefix_workspace_size(dims_of(sb, ds), len(pl), 6, sb.max_seq_len, 0)
    out.append(("shared_prefix", (sb.num_seqs, sb.num_heads, sb.head_dim), n,
                lambda o, w, d=ds, bt=sb, gs=dgs, pl=dpl: ops.paged_gqa_decode_shared_prefix(
                    d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens, gs, pl, 6, bt.max_seq_len,
                    bt.scale, out=o, workspace=w)))
    return out


CALLS = None
N_CALLS = 9


def get_calls():
    global CALLS
    if CALLS is None:
        CALLS = calls()
        assert len(CALLS) == N_CALLS
    return CALLS


@pytest.mark.parametrize("idx", range(N_CALLS))
def test_bitwise_deterministic(idx):
    name, shape, nbytes, f = get_calls()[idx]
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    a = torch.empty(shape, device="cuda")
    b = torch.empty(shape, device="cuda")
    f(a, ws)
    ws.fill_(0x5A)                       # the workspace needs no initialisation
    f(b, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b), name


@pytest.mark.parametrize("idx", range(N_CALLS))
def test_graph_capture_replays_match_eager(idx):
    name, shape, nbytes, f = get_calls()[idx]
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    eager = torch.empty(shape, device="cuda")
    f(eager, ws)
    torch.cuda.synchronize()
    out = torch.zeros(shape, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        f(out, ws)                        # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f(out, ws)
    for rep in range(4):
        out.zero_()
        scratch = torch.randn(1 << 16, device="cuda").sum()    # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(out, eager), f"{name} replay {rep}"
