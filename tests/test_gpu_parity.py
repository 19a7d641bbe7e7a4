"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle.

Every test compares the whole output tensor: small cases, edge cases, and the
full-size workloads in the launch configurations the benchmark times.  The bar: max-abs <= 1e-2 and relative L2 <= 2e-3
for bf16 inputs with fp32 accumulation; fp32 inputs also meet relative L2 <=
1e-5; the cache write is bit-exact.
"""
import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import ops
from gqa_paged_kv_attention_amd import workloads as wl
from oracle import cache_write_ref, decode_ref, lse_merge_ref, paged_attention_ref
from tests import full_size
from tests.gpu_util import DeviceBatch, assert_parity, have_gpu, host, poison_tails

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def oracle_after_write(bt, seqs=None, mixed=False):
    kc, vc = cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                             bt.query_start_loc)
    if mixed:
        return paged_attention_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.query_start_loc,
                                   bt.num_kv_heads, bt.scale, seqs=seqs)
    return decode_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale, seqs=seqs)


def decode_step(bt, partition_size, out_dtype=torch.float32):
    d = DeviceBatch(bt)
    d.cache_write()
    return host(d.decode(partition_size, out_dtype=out_dtype))


def mixed_step(bt, partition_size, out_dtype=torch.float32):
    d = DeviceBatch(bt)
    d.cache_write()
    return host(d.mixed(partition_size, out_dtype=out_dtype))


# --------------------------------------------------------------------------
# reshape_and_cache: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["mixed", "decode", "one_chunk", "sparse_chunks"])
def test_reshape_and_cache_bit_exact(dtype, d, kind):
    """Batches with chunks (four or more new tokens per sequence on average)
    take the grouped kernel; a decode step (token t is sequence t) and a batch
    with few short chunks among many decodes take the per-chunk kernel, the
    latter through its query_start_loc search."""
    rng = np.random.default_rng(7)
    q_lens = {"mixed": np.array([1, 5, 0, 17, 1, 33, 2]), "decode": np.ones(300, dtype=np.int64),
              "one_chunk": np.array([70]),
              "sparse_chunks": np.array([1] * 30 + [3, 0, 5, 2] + [1] * 6)}[kind]
    seq_lens = q_lens + rng.integers(0, 40, size=len(q_lens))
    bt = wl.make_batch(name="rc", seed=8, num_heads=8, num_kv_heads=4, head_dim=d, block_size=16,
                       seq_lens=seq_lens, query_lens=q_lens, dtype=dtype)
    dev = DeviceBatch(bt)
    dev.cache_write()
    torch.cuda.synchronize()
    kc, vc = cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                             bt.query_start_loc)
    assert np.array_equal(ops.to_host_storage(dev.key_cache).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(ops.to_host_storage(dev.value_cache).view(np.uint8), vc.view(np.uint8))


# --------------------------------------------------------------------------
# decode: small workloads, full oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [1, 101, 102, 103])
@pytest.mark.parametrize("partition", [0, 32, 64])
def test_tiny_decode_fp32(seed, partition):
    bt = wl.tiny_decode(seed)
    assert_parity(decode_step(bt, partition), oracle_after_write(bt), bt.dtype, bt.describe())


@pytest.mark.parametrize("partition", [0, 64, 512])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_llama31_decode_small(partition, out_dtype):
    bt = wl.llama31_8b_decode(seed=2, num_seqs=10)
    out = decode_step(bt, partition, out_dtype)
    ref = oracle_after_write(bt)
    if out_dtype == torch.bfloat16:
        # bf16 output rounding alone is ~1.7e-3 relative; check it against the
        # fp32-output kernel rounded to bf16 (at most one bf16 ulp apart)
        f32 = decode_step(bt, partition, torch.float32)
        rounded = torch.from_numpy(f32).to(torch.bfloat16).double().numpy()
        ulp = np.abs(rounded) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(out - rounded) <= ulp)
        assert np.max(np.abs(out - ref)) <= 1e-2
    else:
        assert_parity(out, ref, bt.dtype, bt.describe())


@pytest.mark.parametrize("hkv", [32, 8, 1])
def test_llama2_sweep_small(hkv):
    bt = wl.llama2_7b_sweep(hkv, seed=3, num_seqs=12)
    assert_parity(decode_step(bt, 256), oracle_after_write(bt), bt.dtype, bt.describe())


def test_longctx_small():
    bt = wl.longctx_splitk(seed=5, num_seqs=2, ctx=4000)
    assert_parity(decode_step(bt, wl.LONGCTX_PARTITION), oracle_after_write(bt), bt.dtype, bt.describe())


# --------------------------------------------------------------------------
# decode edge cases
# --------------------------------------------------------------------------

EDGE_LENS = [0, 1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 511, 512, 513]


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 4), (6, 2), (8, 2), (10, 2), (16, 2), (16, 1), (32, 2), (32, 1)])
def test_decode_edge_shapes(dtype, d, hq, hkv):
    bt = wl.make_batch(name="edge", seed=hq * 100 + hkv + d, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       block_size=16, seq_lens=EDGE_LENS, query_lens=[0 if L == 0 else 1 for L in EDGE_LENS],
                       dtype=dtype, poison_slack=True)
    poison_tails(bt)
    # zero-length sequences have no query token; give them a query row anyway (decode is one row per sequence)
    q = wl._normal_storage(np.random.default_rng(0), (len(EDGE_LENS), hq, d), dtype)
    bt.query = q
    dev = DeviceBatch(bt)
    ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, hkv, bt.scale)
    for partition in (0, 32, 96):
        out = host(dev.decode(partition))
        assert_parity(out, ref, dtype, f"{bt.describe()} P={partition}")
        assert np.all(out[0] == 0)          # empty sequence -> zero row


@pytest.mark.parametrize("d", [64, 128])
def test_decode_g32_round_robin_schedule(d):
    """bf16 with G = 32 over a page pool above 512 MiB (the library then keeps
    each kv head's 32 query heads in one unit: two row blocks per wave): the
    waves of a work-group take a partition's 32-token tiles round-robin through
    the alternating double-buffered schedule (stride 4, clamped prefetches past
    the last tile).  Every length from 1 to 300 tokens, so each wave's first and
    last tile positions, and partitions with fewer tiles than waves, all occur,
    plus one 8192-token sequence; unsplit and in 64- and 160-token partitions."""
    lens = np.concatenate([np.arange(1, 301), [8192]])
    pool_tokens = 1 << 20                    # K + V of 2^20 tokens: 512 MiB at d = 128, 256 MiB at d = 64
    slack = (pool_tokens * (128 // d) // 16 + 16) / float(sum((L + 15) // 16 for L in lens))
    bt = wl.make_batch(name="g32", seed=d + 32, num_heads=32, num_kv_heads=1, head_dim=d, block_size=16,
                       seq_lens=lens, query_lens=np.ones(len(lens), np.int64), dtype=wl.BF16, poison_slack=True,
                       slack_frac=slack)
    assert bt.num_blocks * 16 * 2 * d * 2 > (512 << 20)
    poison_tails(bt)
    dev = DeviceBatch(bt)
    ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, 1, bt.scale)
    for partition in (0, 64, 160):
        assert_parity(host(dev.decode(partition)), ref, wl.BF16, f"{bt.describe()} P={partition}")


@pytest.mark.parametrize("num_seqs", [37, 300])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_g32_split_units(d, num_seqs):
    """bf16 with G = 32 over a pool the last-level cache holds: each kv head's
    query heads run as two units of 16 rows whose work-groups are paired onto
    one XCD (a grid that is not a multiple of 16 work-groups takes the
    remainder pairing too).  37 sequences: one work-group per compute unit or
    fewer, 8 waves each; 300 sequences: 4 waves.  Unsplit and in 64-token
    partitions."""
    lens = np.arange(1, 301)[:: 300 // num_seqs][:num_seqs] if num_seqs < 300 else np.arange(1, 301)
    bt = wl.make_batch(name="g32s", seed=d + num_seqs, num_heads=32, num_kv_heads=1, head_dim=d, block_size=16,
                       seq_lens=lens, query_lens=np.ones(len(lens), np.int64), dtype=wl.BF16, poison_slack=True)
    poison_tails(bt)
    dev = DeviceBatch(bt)
    ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, 1, bt.scale)
    for partition in (0, 64):
        assert_parity(host(dev.decode(partition)), ref, wl.BF16, f"{bt.describe()} P={partition}")


def test_decode_peaky_scores_exercise_rescale():
    """Scores far from uniform (q scaled up) so the running max moves across tiles."""
    bt = wl.llama31_8b_decode(seed=9, num_seqs=6, ctx_lo=100, ctx_hi=1500)
    qf = wl.bf16_bits_to_f32(bt.query) * 4.0
    bt.query = wl.f32_to_bf16_bits(qf)
    for partition in (0, 128):
        assert_parity(decode_step(bt, partition), oracle_after_write(bt), bt.dtype, f"peaky P={partition}")


def test_decode_is_deterministic():
    bt = wl.llama31_8b_decode(seed=11, num_seqs=16)
    dev = DeviceBatch(bt)
    a = dev.decode(256).cpu()
    b = dev.decode(256).cpu()
    assert torch.equal(a, b)


def test_split_invariance():
    bt = wl.llama31_8b_decode(seed=12, num_seqs=8, ctx_lo=900, ctx_hi=2100)
    dev = DeviceBatch(bt)
    ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                     bt.scale)
    outs = [host(dev.decode(p)) for p in (0, 32, 64, 160, 512, 2048)]
    for o in outs:
        assert_parity(o, ref, bt.dtype)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-5


def test_workspace_reuse_across_shapes():
    """One workspace (never cleared) serves decodes of different shapes and split modes in turn."""
    a = wl.llama31_8b_decode(seed=13, num_seqs=9, ctx_lo=300, ctx_hi=2000)
    b = wl.llama2_7b_sweep(1, seed=14, num_seqs=40)
    c = wl.make_batch(name="c", seed=15, num_heads=16, num_kv_heads=2, head_dim=64, block_size=16,
                      seq_lens=[700, 33, 1500], query_lens=[1, 1, 1], dtype=wl.F32)
    ws = torch.full((64 << 20,), 0x7F, dtype=torch.uint8, device="cuda")
    for bt, P in ((a, 128), (b, 0), (c, 96), (a, 0), (b, 32), (c, 0), (a, 256)):
        dev = DeviceBatch(bt)
        ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                         bt.scale)
        assert_parity(host(dev.decode(P, workspace=ws)), ref, bt.dtype, f"{bt.describe()} P={P}")


# --------------------------------------------------------------------------
# split-K reduce on its own
# --------------------------------------------------------------------------

@pytest.mark.parametrize("use_qsl", [False, True])
def test_splitk_lse_reduce_random_partials(use_qsl):
    rng = np.random.default_rng(21)
    B, Hq, P, d, psize = 6, 8, 5, 128, 64
    seq_lens = np.array([0, 1, 64, 65, 200, 320], np.int32)
    O = rng.standard_normal((B, Hq, P, d)).astype(np.float32)
    lse = (rng.standard_normal((B, Hq, P)) * 3).astype(np.float32)
    nparts = np.minimum(-(-seq_lens // psize), P)
    for b in range(B):
        lse[b, :, nparts[b]:] = -np.inf        # partitions past the sequence are never read
        O[b, :, nparts[b]:] = np.nan
    lse[4, 3, 1] = -np.inf                      # an empty partition inside a sequence
    ref = np.zeros((B, Hq, d))
    for b in range(B):
        if nparts[b] > 0:
            ref[b] = lse_merge_ref(O[b, :, :nparts[b]].astype(np.float64), lse[b, :, :nparts[b]].astype(np.float64))
    qsl = None
    rows = B
    if use_qsl:
        q_lens = np.ones(B, np.int32)
        q_lens[2] = 3                            # not a decode: must be left alone
        qsl_h = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        qsl = torch.from_numpy(qsl_h).cuda()
        rows = int(qsl_h[-1])
    out = ops.splitk_lse_reduce(torch.from_numpy(O).cuda(), torch.from_numpy(lse).cuda(),
                                torch.from_numpy(seq_lens).cuda(), psize, num_kv_heads=2, max_blocks_per_seq=32,
                                query_start_loc=qsl, num_out_rows=rows)
    got = host(out)
    if use_qsl:
        for b in range(B):
            if b == 2:
                assert np.all(got[qsl_h[b]:qsl_h[b + 1]] == 0)
            else:
                np.testing.assert_allclose(got[qsl_h[b]], ref[b], rtol=0, atol=2e-6)
    else:
        np.testing.assert_allclose(got, ref, rtol=0, atol=2e-6)


# --------------------------------------------------------------------------
# mixed chunked-prefill + decode
# --------------------------------------------------------------------------

@pytest.mark.parametrize("partition", [0, 128])
def test_mixed_small(partition):
    bt = wl.mixed_chunked(seed=4, num_seqs=30, token_budget=1200)
    assert_parity(mixed_step(bt, partition), oracle_after_write(bt, mixed=True), bt.dtype, bt.describe())


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (32, 1), (12, 2), (16, 1)])
def test_mixed_edge_shapes(dtype, d, hq, hkv):
    q_lens = [2, 1, 0, 7, 33, 1, 64, 130, 5, 1, 16]
    prior = [0, 40, 3, 9, 0, 300, 17, 70, 511, 0, 16]
    seq_lens = [a + b for a, b in zip(q_lens, prior)]
    bt = wl.make_batch(name="medge", seed=hq + 7 * hkv + d, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       block_size=16, seq_lens=seq_lens, query_lens=q_lens, dtype=dtype, poison_slack=True)
    poison_tails(bt)
    dev = DeviceBatch(bt)
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, hkv, bt.scale)
    for partition in (0, 64):
        assert_parity(host(dev.mixed(partition)), ref, dtype, f"{bt.describe()} P={partition}")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.3])
def test_mixed_scale_sign(dtype, scale):
    """The softmax is of scale * q.k for any finite scale: a negative scale
    reverses which keys dominate, zero averages the visible values."""
    q_lens = [1, 40, 3, 1, 97]
    prior = [50, 0, 200, 7, 33]
    bt = wl.make_batch(name="scale", seed=41, num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                       seq_lens=[a + b for a, b in zip(q_lens, prior)], query_lens=q_lens, dtype=dtype)
    dev = DeviceBatch(bt)
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, scale)
    got = host(ops.chunked_prefill_paged_decode(dev.query, dev.key_cache, dev.value_cache, dev.block_tables,
                                                dev.seq_lens, dev.query_start_loc, bt.max_query_len, bt.max_seq_len,
                                                scale))
    assert_parity(got, ref, dtype, f"{bt.describe()} scale={scale}")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_mixed_long_decodes_split_by_library(dtype):
    """partition_size = 0 with decodes longer than the library's decode
    partition: the long decodes are split and merged, the rest are not."""
    q_lens = [1, 1, 37, 1, 1, 300]
    seq_lens = [9000, 4100, 500, 4096, 17, 800]
    bt = wl.make_batch(name="mlong", seed=61, num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                       seq_lens=seq_lens, query_lens=q_lens, dtype=dtype, poison_slack=True)
    poison_tails(bt)
    dev = DeviceBatch(bt)
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale)
    assert_parity(host(dev.mixed(0)), ref, dtype, bt.describe())


@pytest.mark.parametrize("n_short", [1, 2, 3, 4, 5, 9])
def test_mixed_decode_packs(n_short):
    """Decode partitions of at most 64 tiles run one per wave, four to a
    work-group; longer ones run on a whole work-group.  n_short short decodes
    leave the last pack with 1..4 partitions; lengths at the 64-tile boundary
    (2048 keys: packed; 2049: whole work-group) and empty and one-key decodes
    sit beside prefill chunks."""
    rng = np.random.default_rng(90 + n_short)
    short = list(rng.integers(1, 2049, size=n_short))
    short[0] = 2048
    q_lens = [1] * n_short + [1, 1, 1, 40, 3]
    seq_lens = short + [2049, 1, 5000, 300, 45]
    q_lens.append(0)
    seq_lens.append(5)
    bt = wl.make_batch(name="packs", seed=91 + n_short, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       seq_lens=seq_lens, query_lens=q_lens, dtype=wl.BF16, poison_slack=True)
    poison_tails(bt)
    dev = DeviceBatch(bt)
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale)
    for partition in (0, 512):
        assert_parity(host(dev.mixed(partition)), ref, bt.dtype, f"{bt.describe()} P={partition}")


def test_mixed_more_sequences_than_schedule_threads():
    """Over 1024 sequences the scheduling pass lets each thread write several
    sequences' units (below that, all threads write the units together)."""
    rng = np.random.default_rng(71)
    B = 1100
    q_lens = np.where(rng.random(B) < 0.85, 1, rng.integers(2, 24, size=B))
    seq_lens = q_lens + rng.integers(0, 90, size=B)
    bt = wl.make_batch(name="many", seed=72, num_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                       seq_lens=seq_lens, query_lens=q_lens, dtype=wl.BF16)
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale)
    dev = DeviceBatch(bt)
    for partition in (0, 32):
        assert_parity(host(dev.mixed(partition)), ref, bt.dtype, f"{bt.describe()} P={partition}")


def test_mixed_bf16_output_is_rounded_fp32():
    """bf16 output of the mixed call is the fp32 result rounded to bf16."""
    bt = wl.mixed_chunked(seed=4, num_seqs=24, token_budget=900)
    dev = DeviceBatch(bt)
    dev.cache_write()
    o32 = dev.mixed(0, out_dtype=torch.float32)
    o16 = dev.mixed(0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert_parity(host(o16), oracle_after_write(bt, mixed=True), bt.dtype, bt.describe() + " bf16 out")


def test_mixed_workspace_reuse_across_batches():
    """One workspace serves successive mixed calls of different shapes: each
    call's scheduling pass rewrites the unit list it reads."""
    big = wl.mixed_chunked(seed=8, num_seqs=40, token_budget=1500)
    small = wl.mixed_chunked(seed=9, num_seqs=12, token_budget=300)
    dims = lambda bt, d: ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=d.key_cache,
                                       block_tables=d.block_tables, q_dtype=d.query.dtype, out_dtype=torch.float32)
    db, dsm = DeviceBatch(big), DeviceBatch(small)
    nbytes = max(ops.mixed_workspace_size(dims(big, db), big.num_tokens, big.max_seq_len, 0),
                 ops.mixed_workspace_size(dims(small, dsm), small.num_tokens, small.max_seq_len, 0))
    ws = torch.full((nbytes,), 0x7F, dtype=torch.uint8, device="cuda")
    for bt, d in ((big, db), (small, dsm), (big, db)):
        d.cache_write()
        out = ops.chunked_prefill_paged_decode(d.query, d.key_cache, d.value_cache, d.block_tables, d.seq_lens,
                                               d.query_start_loc, bt.max_query_len, bt.max_seq_len, bt.scale,
                                               workspace=ws)
        assert_parity(host(out), oracle_after_write(bt, mixed=True), bt.dtype, bt.describe())


@pytest.mark.parametrize("mode", ["decode0", "decode512", "mixed"])
def test_prefix_shared_pages(mode):
    """Sequences whose block tables alias the pages of a shared prompt prefix
    (read-only sharing, new tokens in private pages)."""
    rng = np.random.default_rng(71)
    B, prefix_pages = 12, 64                       # 1024 shared tokens
    if mode == "mixed":
        q_lens = [1, 40, 1, 1, 130, 1, 7, 1, 1, 64, 1, 2]
    else:
        q_lens = [1] * B
    seq_lens = [prefix_pages * 16 + int(x) + q for x, q in zip(rng.integers(1, 600, size=B), q_lens)]
    bt = wl.make_batch(name="prefix", seed=72, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       seq_lens=seq_lens, query_lens=q_lens, dtype=wl.BF16)
    for b in range(1, B):
        bt.block_tables[b, :prefix_pages] = bt.block_tables[0, :prefix_pages]
    dev = DeviceBatch(bt)
    dev.cache_write()
    kc, vc = cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                             bt.query_start_loc)
    if mode == "mixed":
        ref = paged_attention_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.query_start_loc,
                                  bt.num_kv_heads, bt.scale)
        got = host(dev.mixed(0))
    else:
        ref = decode_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale)
        got = host(dev.decode(0 if mode == "decode0" else 512))
    assert_parity(got, ref, bt.dtype, f"{bt.describe()} {mode}")


def test_gqa_equals_expanded_kv_on_gpu():
    """The grouped decode equals the same decode over K/V expanded per query
    head (Hkv = Hq), the layout a GQA-unaware kernel reads."""
    bt = wl.llama2_7b_sweep(8, seed=3, num_seqs=24)
    dev = DeviceBatch(bt)
    G = bt.num_heads // bt.num_kv_heads
    grouped = host(dev.decode(0))
    kce = dev.key_cache.repeat_interleave(G, dim=1).contiguous()
    vce = dev.value_cache.repeat_interleave(G, dim=1).contiguous()
    expanded = host(ops.paged_gqa_decode(dev.query, kce, vce, dev.block_tables, dev.seq_lens, bt.max_seq_len,
                                         bt.scale))
    assert np.max(np.abs(expanded - grouped)) <= 1e-5
    ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale)
    assert_parity(grouped, ref, bt.dtype, bt.describe())


def test_prefill_chunk_invariance_on_gpu():
    """A 96-token chunk equals three sequential 32-token chunks over the same cache."""
    L, C = 400, 96
    full = wl.make_batch(name="chunk", seed=33, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                         seq_lens=[L], query_lens=[C], dtype=wl.BF16)
    dev = DeviceBatch(full)
    whole = host(dev.mixed())
    parts = []
    for c in range(3):
        qsl = torch.tensor([0, 32], dtype=torch.int32, device="cuda")
        sl = torch.tensor([L - C + 32 * (c + 1)], dtype=torch.int32, device="cuda")
        parts.append(host(ops.chunked_prefill_paged_decode(dev.query[32 * c:32 * (c + 1)].contiguous(), dev.key_cache,
                                                           dev.value_cache, dev.block_tables, sl, qsl, 32,
                                                           L - C + 32 * (c + 1), full.scale)))
    assert np.max(np.abs(np.concatenate(parts) - whole)) <= 1e-5


@pytest.mark.parametrize("v_scale", [1e-4, 1e-5])
def test_mixed_small_values(v_scale):
    """Values far below 1 (N(0, s^2) with s = 1e-4, 1e-5): the prefill rows
    convert V to fp16, where magnitudes under 2^-14 become subnormals; the
    conversion rounds to nearest, so the error stays unbiased and the whole
    output meets the bar (a CPU model of the conversion puts its share of the
    relative L2 error at 5e-5 and 1.4e-3)."""
    bt = wl.mixed_chunked(seed=41, num_seqs=24, token_budget=900)
    for arr in (bt.value_cache, bt.new_value):
        scaled = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(arr) * np.float32(v_scale))
        arr[...] = scaled
    out = mixed_step(bt, 0)
    assert_parity(out, oracle_after_write(bt, mixed=True), bt.dtype, f"{bt.describe()} V x {v_scale:g}")


def _prefill_heavy(hq, hkv, d, bs, seed):
    """Prefill chunks with ragged 256-row tiles beside decodes of every kind:
    packed short ones (up to 2048 keys), whole-work-group ones (2049 and more
    keys), a one-key decode and an empty query.  Query rows (tokens x G)
    average 1024 or more per sequence over several sequences, and their
    128-row tiles times Hkv outnumber the compute units, so the fused kernel
    runs 8-wave work-groups."""
    G = hq // hkv
    chunk = {1: 3700, 4: 1000, 8: 500, 16: 250}[G]
    q_lens = [chunk, 1, 1, 1, chunk + 37, 0, 1, chunk // 2 + 3, 1]
    prior = [0, 3000, 700, 2047, 100, 5, 2048, 1500, 0]
    bt = wl.make_batch(name="heavy", seed=seed, num_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                       seq_lens=[a + b for a, b in zip(q_lens, prior)], query_lens=q_lens, dtype=wl.BF16,
                       poison_slack=True)
    rows = bt.num_tokens * G
    assert rows >= 1024 * bt.num_seqs
    assert rows // 128 * hkv >= torch.cuda.get_device_properties(0).multi_processor_count
    poison_tails(bt)
    return bt


@pytest.mark.parametrize("bs", [16, 32, 64])
@pytest.mark.parametrize("d", [64, 128])
def test_mixed_prefill_heavy_eight_waves(d, bs):
    bt = _prefill_heavy(32, 8, d, bs, seed=d + bs)
    dev = DeviceBatch(bt)
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale)
    for partition in (0, 512):
        assert_parity(host(dev.mixed(partition)), ref, bt.dtype, f"{bt.describe()} P={partition}")


@pytest.mark.parametrize("hq,hkv", [(4, 4), (32, 4), (64, 4)])
def test_mixed_prefill_heavy_eight_waves_groups(hq, hkv):
    bt = _prefill_heavy(hq, hkv, 128, 16, seed=hq + hkv)
    dev = DeviceBatch(bt)
    dev.cache_write()
    ref = oracle_after_write(bt, mixed=True)
    o32 = dev.mixed(0, out_dtype=torch.float32)
    o16 = dev.mixed(0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert_parity(host(o32), ref, bt.dtype, bt.describe())


# --------------------------------------------------------------------------
# full-size workloads: the whole output against the oracle, in the launch
# configurations the benchmark times
# --------------------------------------------------------------------------

@pytest.mark.parametrize("partition", [0, 512])
def test_full_llama31_decode(partition):
    """partition 0: the library's split (balanced at this shape), what the benchmark times."""
    bt = wl.llama31_8b_decode(seed=2)
    assert_parity(decode_step(bt, partition), full_size.llama31_decode(), bt.dtype, bt.describe())


@pytest.mark.parametrize("partition", [0, 256])
@pytest.mark.parametrize("hkv", [32, 8, 1])
def test_full_llama2_sweep(hkv, partition):
    bt = wl.llama2_7b_sweep(hkv, seed=3)
    assert_parity(decode_step(bt, partition), full_size.llama2_sweep(hkv), bt.dtype, bt.describe())


@pytest.mark.parametrize("partition", [0, 512])
def test_full_mixed(partition):
    """partition 0: the library's decode split, what the benchmark times (with
    bf16 output there: every element the fp32 result rounded to nearest even,
    and the bf16 output itself within the bar)."""
    bt = wl.mixed_chunked(seed=4)
    d = DeviceBatch(bt)
    d.cache_write()
    o32 = d.mixed(partition)
    ref = full_size.mixed()
    assert_parity(host(o32), ref, bt.dtype, bt.describe())
    if partition == 0:
        o16 = d.mixed(partition, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(o32.to(torch.bfloat16), o16)
        assert np.max(np.abs(host(o16) - ref)) <= 1e-2


def test_full_uniform_prefill_eight_waves():
    """The 8-wave launch at full size: 16 chunks of 512 new tokens on
    3584-token prefixes (Hq = 32, Hkv = 8, d = 128, bf16).  The oracle computes
    the first and the last sequence whole (every row of their 256-row tiles,
    causal limits up to 4096 keys); the other sequences' outputs must be finite
    and, as the same computation on other data, are covered by the random
    prefill-heavy draws."""
    bt = wl.make_batch(name="uniform", seed=11, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                       seq_lens=[4096] * 16, query_lens=[512] * 16, dtype=wl.BF16)
    assert bt.num_tokens * 4 // 128 * 8 >= torch.cuda.get_device_properties(0).multi_processor_count
    got = host(DeviceBatch(bt).mixed(0))
    assert np.all(np.isfinite(got))
    seqs = [0, bt.num_seqs - 1]
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale, seqs=seqs)
    rows = np.concatenate([np.arange(bt.query_start_loc[b], bt.query_start_loc[b + 1]) for b in seqs])
    assert_parity(got[rows], ref[rows], bt.dtype, bt.describe() + " sequences 0 and 15")


@pytest.mark.parametrize("name", ["mixed", "decode"])
def test_full_cache_write_bit_exact(name):
    """reshape_and_cache at the benchmark's sizes (the mixed batch's 8166 new
    tokens through the grouped kernel, the decode step's 64 through the
    per-chunk kernel): both whole caches equal the oracle's, byte for byte."""
    bt = wl.mixed_chunked(seed=4) if name == "mixed" else wl.llama31_8b_decode(seed=2)
    dev = DeviceBatch(bt)
    dev.cache_write()
    torch.cuda.synchronize()
    kc, vc = cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                             bt.query_start_loc)
    assert np.array_equal(ops.to_host_storage(dev.key_cache).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(ops.to_host_storage(dev.value_cache).view(np.uint8), vc.view(np.uint8))


@pytest.mark.parametrize("partition", [wl.LONGCTX_PARTITION, 0])
def test_full_longctx_splitk(partition):
    """Both splits the benchmark times: 512-token partitions and the library's."""
    bt = wl.longctx_splitk(seed=5)
    assert_parity(decode_step(bt, partition), full_size.longctx(), bt.dtype, bt.describe())


def test_bound_calls_match_direct_calls():
    """A BoundCall re-issues the very call the binding makes: same outputs, bit for bit, on every re-issue."""
    bt = wl.llama31_8b_decode(seed=21, num_seqs=12, ctx_lo=200, ctx_hi=1500)
    dev = DeviceBatch(bt)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    out = torch.empty(bt.num_seqs, bt.num_heads, bt.head_dim, dtype=torch.float32, device="cuda")
    direct = ops.paged_gqa_decode(dev.query, dev.key_cache, dev.value_cache, dev.block_tables, dev.seq_lens,
                                  bt.max_seq_len, bt.scale, partition_size=64, workspace=ws).clone()
    bound = ops.paged_gqa_decode(dev.query, dev.key_cache, dev.value_cache, dev.block_tables, dev.seq_lens,
                                 bt.max_seq_len, bt.scale, partition_size=64, out=out, workspace=ws, bind=True)
    assert isinstance(bound, ops.BoundCall)
    for _ in range(3):
        out.fill_(float("nan"))
        assert bound() is out
        torch.cuda.synchronize()
        assert torch.equal(out, direct)

    # The fused step: the bound call writes the caches and the output like the direct call.
    a, b = DeviceBatch(bt), DeviceBatch(bt)
    ref = ops.paged_gqa_decode_append(a.query, a.new_key, a.new_value, a.key_cache, a.value_cache, a.block_tables,
                                      a.seq_lens, bt.max_seq_len, bt.scale)
    step = ops.paged_gqa_decode_append(b.query, b.new_key, b.new_value, b.key_cache, b.value_cache, b.block_tables,
                                       b.seq_lens, bt.max_seq_len, bt.scale, bind=True)
    got = step()
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert torch.equal(a.key_cache, b.key_cache) and torch.equal(a.value_cache, b.value_cache)

    # A failing bound call raises like the direct call.
    bad = ops.paged_gqa_decode(dev.query, dev.key_cache, dev.value_cache, dev.block_tables, dev.seq_lens,
                               bt.max_seq_len, bt.scale, partition_size=64, out=out,
                               workspace=torch.zeros(16, dtype=torch.uint8, device="cuda"), bind=True)
    with pytest.raises(ops.GqaError):
        bad()
