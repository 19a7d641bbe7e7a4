"""Seeded synthetic batches for paged GQA attention.

This module only builds inputs: sequence lengths, page tables, cache pools and
query/key/value values.  It contains none of the attention arithmetic, so the
CPU oracle and the HIP path can both consume its output without sharing any
computation.

Storage conventions (the library's cache layout, chosen for 16-byte loads):

* ``key_cache``   : ``[num_blocks, num_kv_heads, block_size, head_dim]``
* ``value_cache`` : ``[num_blocks, num_kv_heads, head_dim, block_size]``
* ``query``       : ``[num_tokens, num_heads, head_dim]`` (token-major)
* ``new_key`` / ``new_value`` : ``[num_tokens, num_kv_heads, head_dim]``
* ``block_tables``: ``[num_seqs, max_blocks_per_seq]`` int32
* ``seq_lens``    : ``[num_seqs]`` int32, cached tokens *including* this step's
* ``query_start_loc`` : ``[num_seqs + 1]`` int32 prefix sums of query lengths

Floating-point arrays are held as *storage*: ``np.float32`` for fp32 batches
and ``np.uint16`` bfloat16 bit patterns for bf16 batches.  Values are drawn as
float32 N(0,1) and rounded to nearest-even into bf16, so both sides see the
same exactly-representable numbers.

The shapes follow the workloads of the source pages: Llama-3.1-8B and
Llama-2-7B head shapes, the TensorRT-LLM latency run of "[Performance] Use
optimized kernels for MQA/GQA" (input 32 / output 992 tokens), and the ShareGPT
serving run of "[Kernel] [V1] Further optimizations to ROCm (Triton) Backend to
better handle GQA" (about 215 input and 200 output tokens per request), for
which a lognormal length mix stands in.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os
from typing import Optional, Sequence

import numpy as np

BF16 = "bf16"
F32 = "f32"


_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _chunked(n: int, fn) -> None:
    """Run fn(start, stop) over [0, n) in fixed-size chunks on a thread pool."""
    starts = range(0, n, _CHUNK)
    if len(starts) <= 1:
        for s in starts:
            fn(s, min(n, s + _CHUNK))
        return
    with cf.ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(lambda s: fn(s, min(n, s + _CHUNK)), starts))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest-even bfloat16; return uint16 bits.

    NaNs map to the quiet NaN 0x7FC0; the uint32 sum below can only wrap for
    NaN bit patterns, which are overwritten.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)

    def conv(a, b):
        u = flat[a:b].view(np.uint32)
        r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        o = r.astype(np.uint16)
        nan = np.isnan(flat[a:b])
        if nan.any():
            o[nan] = 0x7FC0
        out[a:b] = o

    _chunked(flat.size, conv)
    return out.reshape(x.shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def storage_to_f32(arr: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(arr) if arr.dtype == np.uint16 else np.asarray(arr, dtype=np.float32)


def _normal_storage(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) float32 values in storage form.

    Each 4M-element chunk draws from its own PCG64 stream spawned from one seed
    taken from ``rng``, so the values do not depend on the thread count.
    """
    n = int(np.prod(shape))
    vals = np.empty(n, dtype=np.float32)
    kids = np.random.SeedSequence(int(rng.integers(0, 2 ** 63))).spawn(max(1, -(-n // _CHUNK)))

    def fill(a, b):
        np.random.Generator(np.random.PCG64(kids[a // _CHUNK])).standard_normal(out=vals[a:b], dtype=np.float32)

    _chunked(n, fill)
    vals = vals.reshape(shape)
    if dtype == BF16:
        return f32_to_bf16_bits(vals)
    if dtype == F32:
        return vals
    raise ValueError(f"unknown dtype {dtype!r}")


def _nan_storage(dtype: str):
    return np.uint16(0x7FC0) if dtype == BF16 else np.float32("nan")


@dataclasses.dataclass
class PagedBatch:
    """One synthetic batch over a paged KV cache (host arrays)."""

    name: str
    seed: int
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    seq_lens: np.ndarray
    query_lens: np.ndarray
    query_start_loc: np.ndarray
    block_tables: np.ndarray
    num_blocks: int
    slack_pages: np.ndarray
    key_cache: np.ndarray
    value_cache: np.ndarray
    query: np.ndarray
    new_key: np.ndarray
    new_value: np.ndarray

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def kv_itemsize(self) -> int:
        return 2 if self.dtype == BF16 else 4

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one attention pass reads (valid tokens only)."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * self.kv_itemsize

    def describe(self) -> str:
        return (f"{self.name}[seed={self.seed}] B={self.num_seqs} Hq={self.num_heads} Hkv={self.num_kv_heads} "
                f"d={self.head_dim} bs={self.block_size} {self.dtype} T={self.num_tokens} "
                f"max_seq={self.max_seq_len} max_q={self.max_query_len} blocks={self.num_blocks}")


def make_batch(*, name: str, seed: int, num_heads: int, num_kv_heads: int, head_dim: int,
               block_size: int, seq_lens: Sequence[int], query_lens: Sequence[int], dtype: str,
               scale: Optional[float] = None, slack_frac: float = 0.1,
               max_blocks_per_seq: Optional[int] = None, poison_slack: bool = False,
               rng: Optional[np.random.Generator] = None, cross: bool = False) -> PagedBatch:
    """Build a batch: a seeded permutation of physical pages and N(0,1) data.

    Every page of the pool (including slack pages that no sequence owns) is
    filled with N(0,1) values; ``poison_slack`` fills the slack pages with NaN
    instead, so that an out-of-table read shows up in the output.  Block-table
    entries past a sequence's last page point at a slack page.  ``cross``
    marks a cross-attention batch: ``seq_lens`` are encoder lengths and a
    sequence may have more query rows than encoder positions.
    """
    rng = rng if rng is not None else np.random.default_rng(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    query_lens = np.asarray(query_lens, dtype=np.int32)
    if seq_lens.shape != query_lens.shape:
        raise ValueError("seq_lens and query_lens differ in length")
    if (query_lens < 0).any() or (seq_lens < 0).any():
        raise ValueError("lengths must be non-negative")
    if not cross and (query_lens > seq_lens).any():
        raise ValueError("each query length must lie in [0, seq_len]")
    B = int(seq_lens.shape[0])
    pages = (seq_lens.astype(np.int64) + block_size - 1) // block_size
    used = int(pages.sum())
    slack = max(1, int(math.ceil(slack_frac * used)))
    num_blocks = used + slack
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max(1, int(pages.max()) if B else 1)
    if B and pages.max() > max_blocks_per_seq:
        raise ValueError("max_blocks_per_seq too small")
    perm = rng.permutation(num_blocks).astype(np.int32)
    slack_pages = np.sort(perm[used:])
    block_tables = np.full((B, max_blocks_per_seq), slack_pages[0], dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(pages[b])
        block_tables[b, :n] = perm[off:off + n]
        off += n
    qsl = np.zeros(B + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(query_lens, dtype=np.int64).astype(np.int32)
    T = int(qsl[-1])

    key_cache = _normal_storage(rng, (num_blocks, num_kv_heads, block_size, head_dim), dtype)
    value_cache = _normal_storage(rng, (num_blocks, num_kv_heads, head_dim, block_size), dtype)
    query = _normal_storage(rng, (T, num_heads, head_dim), dtype)
    new_key = _normal_storage(rng, (T, num_kv_heads, head_dim), dtype)
    new_value = _normal_storage(rng, (T, num_kv_heads, head_dim), dtype)
    if poison_slack:
        key_cache[slack_pages] = _nan_storage(dtype)
        value_cache[slack_pages] = _nan_storage(dtype)
    return PagedBatch(name=name, seed=seed, dtype=dtype, num_heads=num_heads, num_kv_heads=num_kv_heads,
                      head_dim=head_dim, block_size=block_size,
                      scale=float(scale if scale is not None else 1.0 / math.sqrt(head_dim)),
                      seq_lens=seq_lens, query_lens=query_lens, query_start_loc=qsl,
                      block_tables=block_tables, num_blocks=num_blocks, slack_pages=slack_pages,
                      key_cache=key_cache, value_cache=value_cache, query=query,
                      new_key=new_key, new_value=new_value)


# --------------------------------------------------------------------------
# Named workloads
# --------------------------------------------------------------------------

def tiny_decode(seed: int = 1, **kw) -> PagedBatch:
    """4 sequences, Hq=8, Hkv=2, d=64, block 16, context U{1..256}, fp32, scale 1/8."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, 257, size=4)
    return make_batch(name="tiny_decode", seed=seed, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                      seq_lens=ctx, query_lens=np.ones(4, np.int32), dtype=F32, scale=1.0 / 8.0, rng=rng, **kw)


def llama31_8b_decode(seed: int = 2, num_seqs: int = 64, ctx_lo: int = 512, ctx_hi: int = 4096,
                      block_size: int = 16, **kw) -> PagedBatch:
    """Llama-3.1-8B decode: Hq=32, Hkv=8, d=128, block 16 (or block_size), bf16, context U{512..4096}."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=num_seqs)
    return make_batch(name="llama31_8b_decode", seed=seed, num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=block_size, seq_lens=ctx, query_lens=np.ones(num_seqs, np.int32), dtype=BF16,
                      rng=rng, **kw)


def llama2_7b_sweep(num_kv_heads: int, seed: int = 3, num_seqs: int = 128, **kw) -> PagedBatch:
    """Llama-2-7B decode: Hq=32, d=128, Hkv in {32, 8, 1}; context U{32..1024}.

    The context draw comes first from the seed, so all three head counts see the
    same lengths (32-token prompts plus up to 992 generated tokens).
    """
    rng = np.random.default_rng(seed)
    ctx = rng.integers(32, 1025, size=num_seqs)
    data_rng = np.random.default_rng([seed, num_kv_heads])
    return make_batch(name=f"llama2_7b_sweep_hkv{num_kv_heads}", seed=seed, num_heads=32,
                      num_kv_heads=num_kv_heads, head_dim=128, block_size=16, seq_lens=ctx,
                      query_lens=np.ones(num_seqs, np.int32), dtype=BF16, rng=data_rng, **kw)


def mixed_lengths(rng: np.random.Generator, num_seqs: int = 256, decode_frac: float = 0.8,
                  q_mean: float = 215.0, ctx_mean: float = 200.0, sigma: float = 1.0,
                  q_cap: int = 2048, token_budget: int = 8192):
    """Query/context lengths of a mixed chunked-prefill + decode batch.

    80% decodes (query length 1) and 20% prefill chunks whose lengths are
    lognormal with the given mean, clamped to [2, q_cap]; if the total query
    tokens exceed the budget, every chunk is scaled down by the budget ratio.
    Prior context is lognormal with mean ``ctx_mean``.  Positions are shuffled.
    """
    n_dec = int(round(decode_frac * num_seqs))
    n_pf = num_seqs - n_dec
    mu_q = math.log(q_mean) - sigma * sigma / 2
    q = np.clip(np.rint(rng.lognormal(mu_q, sigma, size=n_pf)), 2, q_cap).astype(np.int64)
    room = token_budget - n_dec
    if n_pf and q.sum() > room:
        ratio = room / q.sum()
        q = np.maximum(2, np.floor(q * ratio)).astype(np.int64)
    mu_c = math.log(ctx_mean) - sigma * sigma / 2
    prior = np.rint(rng.lognormal(mu_c, sigma, size=num_seqs)).astype(np.int64)
    qlens = np.concatenate([np.ones(n_dec, np.int64), q])
    order = rng.permutation(num_seqs)
    qlens = qlens[order]
    seq_lens = prior + qlens
    return seq_lens.astype(np.int32), qlens.astype(np.int32)


def mixed_chunked(seed: int = 4, num_seqs: int = 256, token_budget: int = 8192, **kw) -> PagedBatch:
    """Mixed chunked-prefill + decode batch on Llama-3.1-8B shapes (Hq=32, Hkv=8, d=128, bf16)."""
    rng = np.random.default_rng(seed)
    seq_lens, qlens = mixed_lengths(rng, num_seqs=num_seqs, token_budget=token_budget)
    return make_batch(name="mixed_chunked", seed=seed, num_heads=32, num_kv_heads=8, head_dim=128,
                      block_size=16, seq_lens=seq_lens, query_lens=qlens, dtype=BF16, rng=rng, **kw)


def longctx_splitk(seed: int = 5, num_seqs: int = 16, ctx: int = 32768, **kw) -> PagedBatch:
    """Long-context decode: 16 sequences of 32768 tokens, Hq=64, Hkv=8, d=128, bf16."""
    rng = np.random.default_rng(seed)
    return make_batch(name="longctx_splitk", seed=seed, num_heads=64, num_kv_heads=8, head_dim=128,
                      block_size=16, seq_lens=np.full(num_seqs, ctx, np.int32),
                      query_lens=np.ones(num_seqs, np.int32), dtype=BF16, rng=rng, **kw)


def cross_attention(seed: int = 6, num_seqs: int = 16, enc_lo: int = 1024, enc_hi: int = 6400,
                    query_len: int = 1, **kw) -> PagedBatch:
    """Cross-attention over a static encoder cache: ``query_len`` decoder rows
    per sequence against U{enc_lo..enc_hi} encoder positions; 16 sequences,
    Hq=32, Hkv=8, d=128, block 16, bf16."""
    rng = np.random.default_rng(seed)
    enc = rng.integers(enc_lo, enc_hi + 1, size=num_seqs)
    return make_batch(name=f"cross_attention_q{query_len}", seed=seed, num_heads=32, num_kv_heads=8,
                      head_dim=128, block_size=16, seq_lens=enc,
                      query_lens=np.full(num_seqs, query_len, np.int32), dtype=BF16, rng=rng, cross=True, **kw)


def shared_prefix_decode(seed: int = 7, num_groups: int = 4, group_size: int = 16, prefix_len: int = 2048,
                         suffix_lo: int = 16, suffix_hi: int = 512, num_heads: int = 32, num_kv_heads: int = 8,
                         head_dim: int = 128, block_size: int = 16, dtype: str = BF16, **kw):
    """Decode batch of `num_groups` groups of `group_size` consecutive sequences.

    The members of a group share their first `prefix_len` tokens: their block
    tables point at the first member's pages for them (as with prefix caching;
    `prefix_len` is a multiple of the page size), and each member then has
    U{suffix_lo..suffix_hi} tokens of its own.  Returns (batch, group_start
    [num_groups + 1], prefix_lens [num_groups]), both int32.
    """
    if prefix_len % block_size:
        raise ValueError("prefix_len must be a multiple of block_size")
    rng = np.random.default_rng(seed)
    B = num_groups * group_size
    suffix = rng.integers(suffix_lo, suffix_hi + 1, size=B)
    bt = make_batch(name="shared_prefix_decode", seed=seed, num_heads=num_heads, num_kv_heads=num_kv_heads,
                    head_dim=head_dim, block_size=block_size, seq_lens=prefix_len + suffix,
                    query_lens=np.ones(B, np.int32), dtype=dtype, rng=rng, **kw)
    shared_pages = prefix_len // block_size
    for g in range(num_groups):
        first = g * group_size
        bt.block_tables[first + 1:first + group_size, :shared_pages] = bt.block_tables[first, :shared_pages]
    group_start = np.arange(0, B + 1, group_size, dtype=np.int32)
    prefix_lens = np.full(num_groups, prefix_len, dtype=np.int32)
    return bt, group_start, prefix_lens


LONGCTX_PARTITION = 512
