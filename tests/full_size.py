"""Oracle outputs of the full-size workloads, each computed once per test session.

The full-size GPU tests compare the WHOLE output tensor with the CPU fp64
oracle (max-abs <= 1e-2 and relative L2 <= 2e-3 over every element), in the
launch configurations the benchmark times.  Each workload's oracle output is
computed here from a freshly generated batch and memoised, so that tests which
share a workload (several splits, the fused step, bf16 output) pay for it once.
Nothing here touches the GPU.
"""
from __future__ import annotations

import functools

import numpy as np

from gqa_paged_kv_attention_amd import workloads as wl
from oracle import cache_write_ref, decode_ref, paged_attention_ref


def _after_write(bt):
    return cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                           bt.query_start_loc)


@functools.lru_cache(maxsize=None)
def llama31_decode(block_size: int = 16) -> np.ndarray:
    """64 sequences, Hq 32, Hkv 8, d 128, context U{512..4096}, seed 2: the
    decode over every cached token after the step's cache write."""
    bt = wl.llama31_8b_decode(seed=2, block_size=block_size)
    kc, vc = _after_write(bt)
    return decode_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale)


@functools.lru_cache(maxsize=None)
def llama2_sweep(hkv: int) -> np.ndarray:
    bt = wl.llama2_7b_sweep(hkv, seed=3)
    kc, vc = _after_write(bt)
    return decode_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale)


@functools.lru_cache(maxsize=None)
def mixed() -> np.ndarray:
    bt = wl.mixed_chunked(seed=4)
    kc, vc = _after_write(bt)
    return paged_attention_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.query_start_loc,
                               bt.num_kv_heads, bt.scale)


@functools.lru_cache(maxsize=None)
def longctx() -> np.ndarray:
    bt = wl.longctx_splitk(seed=5)
    kc, vc = _after_write(bt)
    return decode_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale)


@functools.lru_cache(maxsize=None)
def cross(query_len: int) -> np.ndarray:
    bt = wl.cross_attention(seed=6, query_len=query_len)
    return paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                               bt.query_start_loc, bt.num_kv_heads, bt.scale, causal=False)


@functools.lru_cache(maxsize=None)
def shared_prefix(prefix_len: int, group_size: int) -> np.ndarray:
    bt, _, _ = wl.shared_prefix_decode(seed=7, num_groups=4, group_size=group_size, prefix_len=prefix_len)
    return decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                      bt.scale)
