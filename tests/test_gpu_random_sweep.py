"""Seeded random configurations through every attention entry point, each
compared with the CPU fp64 oracle at the usual bar (max-abs <= 1e-2 and
relative L2 <= 2e-3 for bf16 inputs; fp32 inputs also relative L2 <= 1e-5).

Each case draws the head shape, head size, page size, dtype, batch and
lengths from its seed (all valid inputs), so the sweep reaches combinations
the targeted tests do not list one by one.
"""
import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import ops
from gqa_paged_kv_attention_amd import workloads as wl
from oracle import cache_write_ref, decode_ref, paged_attention_ref
from tests.gpu_util import DeviceBatch, assert_parity, have_gpu, host, poison_tails

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

HEADS = [(4, 4), (8, 2), (8, 1), (12, 4), (16, 2), (24, 3), (32, 8), (32, 1), (40, 5), (64, 2)]


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    hq, hkv = HEADS[rng.integers(len(HEADS))]
    return rng, dict(num_heads=hq, num_kv_heads=hkv, head_dim=int(rng.choice([64, 128])),
                     block_size=int(rng.choice([16, 32, 64])),
                     dtype=wl.F32 if rng.random() < 0.25 else wl.BF16)


def lengths(rng, n, hi):
    """Context lengths with some zeros, short and long ones."""
    kind = rng.integers(3, size=n)
    return np.where(kind == 0, rng.integers(0, 3, size=n),
                    np.where(kind == 1, rng.integers(1, 64, size=n), rng.integers(64, hi, size=n)))


@pytest.mark.parametrize("seed", range(48))
def test_random_decode(seed):
    rng, shape = draw(seed)
    B = int(rng.integers(1, 24))
    L = lengths(rng, B, 1500)
    bt = wl.make_batch(name="rnd_dec", seed=seed, seq_lens=L, query_lens=np.minimum(L, 1), poison_slack=True,
                       **shape)
    bt.query = wl._normal_storage(rng, (B, shape["num_heads"], shape["head_dim"]), shape["dtype"])
    poison_tails(bt)
    partition = int(rng.choice([0, 32, 96, 256]))
    got = host(DeviceBatch(bt).decode(partition))
    ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                     bt.scale)
    assert_parity(got, ref, bt.dtype, f"{bt.describe()} P={partition}")


@pytest.mark.parametrize("seed", range(32))
def test_random_decode_append(seed):
    """The fused append: caches bit-exact against the oracle's cache write of
    each sequence's new token (none for an empty sequence), output at the bar
    against the oracle's decode over them."""
    rng, shape = draw(300 + seed)
    B = int(rng.integers(1, 24))
    L = lengths(rng, B, 1500)
    bt = wl.make_batch(name="rnd_app", seed=seed, seq_lens=L, query_lens=np.minimum(L, 1), poison_slack=True,
                       **shape)
    bt.query = wl._normal_storage(rng, (B, shape["num_heads"], shape["head_dim"]), shape["dtype"])
    rows = (B, shape["num_kv_heads"], shape["head_dim"])
    nk, nv = wl._normal_storage(rng, rows, shape["dtype"]), wl._normal_storage(rng, rows, shape["dtype"])
    has = L > 0
    qsl = np.concatenate([[0], np.cumsum(has)])
    kc, vc = cache_write_ref(nk[has], nv[has], bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, qsl)
    ref = decode_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.num_kv_heads, bt.scale)
    dev = DeviceBatch(bt)
    partition = int(rng.choice([0, 0, 64, 256]))
    got = ops.paged_gqa_decode_append(dev.query, ops.to_device(nk), ops.to_device(nv), dev.key_cache, dev.value_cache,
                                      dev.block_tables, dev.seq_lens, bt.max_seq_len, bt.scale,
                                      partition_size=partition)
    torch.cuda.synchronize()
    assert np.array_equal(ops.to_host_storage(dev.key_cache).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(ops.to_host_storage(dev.value_cache).view(np.uint8), vc.view(np.uint8))
    assert_parity(host(got), ref, bt.dtype, f"{bt.describe()} P={partition}")


@pytest.mark.parametrize("seed", range(24))
@pytest.mark.parametrize("causal", [True, False])
def test_random_mixed_and_cross(seed, causal):
    rng, shape = draw(100 + seed)
    B = int(rng.integers(1, 16))
    L = lengths(rng, B, 900)
    if causal:
        q = np.where(rng.random(B) < 0.5, np.minimum(L, 1), rng.integers(0, L + 1))
    else:
        q = np.where(rng.random(B) < 0.4, 1, rng.integers(0, 200, size=B))
    bt = wl.make_batch(name="rnd_mix", seed=seed, seq_lens=L, query_lens=q, poison_slack=True, cross=not causal,
                       **shape)
    poison_tails(bt)
    dev = DeviceBatch(bt)
    partition = int(rng.choice([0, 64, 512]))
    got = host(dev.mixed(partition) if causal else dev.cross(partition))
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale, causal=causal)
    assert_parity(got, ref, bt.dtype, f"{bt.describe()} causal={causal} P={partition}")


HEAVY_HEADS = [(hq, hkv) for hq, hkv in HEADS if 2 <= hq // hkv <= 16]


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("causal", [True, False])
def test_random_prefill_heavy(seed, causal):
    """Random batches that take the fused kernel's 8-wave launch (two or more
    sequences, query rows x G averaging 1024 or more per sequence, more 128-row
    tiles x Hkv than compute units): random heads, head size, page size and
    lengths, with decodes among the chunks."""
    rng, shape = draw(500 + seed)
    hq, hkv = HEAVY_HEADS[rng.integers(len(HEAVY_HEADS))]
    shape.update(num_heads=hq, num_kv_heads=hkv, dtype=wl.BF16)
    G = hq // hkv
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    B = int(rng.integers(2, 9))
    n_dec = int(rng.integers(0, B // 2 + 1))
    rows_needed = max(1024 * B, 128 * -(-cus // hkv))
    tokens = -(-rows_needed // G) - n_dec
    n_chunk = B - n_dec
    cuts = np.sort(rng.integers(0, tokens + 1, size=n_chunk - 1))
    q_chunks = np.diff(np.concatenate([[0], cuts, [tokens]]))
    q = np.concatenate([q_chunks, np.ones(n_dec, dtype=np.int64)])
    rng.shuffle(q)
    if causal:
        L = q + rng.integers(0, 1500, size=B)
    else:
        L = rng.integers(1, 3000, size=B)
    bt = wl.make_batch(name="rnd_heavy", seed=seed, seq_lens=L, query_lens=q, poison_slack=True, cross=not causal,
                       **shape)
    rows = bt.num_tokens * G
    assert B >= 2 and rows >= 1024 * B and rows // 128 * hkv >= cus
    poison_tails(bt)
    dev = DeviceBatch(bt)
    partition = int(rng.choice([0, 512]))
    got = host(dev.mixed(partition) if causal else dev.cross(partition))
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale, causal=causal)
    assert_parity(got, ref, bt.dtype, f"{bt.describe()} causal={causal} P={partition}")


@pytest.mark.parametrize("seed", range(24))
def test_random_shared_prefix(seed):
    rng, shape = draw(200 + seed)
    bs = shape["block_size"]
    groups = []
    for _ in range(int(rng.integers(1, 5))):
        members = int(rng.integers(0, 12))
        prefix = bs * int(rng.integers(0, 1200 // bs))
        groups.append((members, prefix, [int(x) for x in rng.integers(0, 300, size=members)]))
    seq_lens, starts, prefixes = [], [0], []
    for members, prefix, suffixes in groups:
        seq_lens += [prefix + s for s in suffixes]
        starts.append(starts[-1] + members)
        prefixes.append(prefix)
    if not seq_lens:
        pytest.skip("empty draw")
    L = np.asarray(seq_lens)
    bt = wl.make_batch(name="rnd_sp", seed=seed, seq_lens=L, query_lens=np.minimum(L, 1), poison_slack=True,
                       **shape)
    # one query row per sequence, an empty one included (its output row is zero)
    bt.query = wl._normal_storage(rng, (len(L), shape["num_heads"], shape["head_dim"]), shape["dtype"])
    for g, (members, prefix, _) in enumerate(groups):
        first = starts[g]
        if members > 1 and prefix > 0:
            bt.block_tables[first + 1:first + members, :prefix // bs] = bt.block_tables[first, :prefix // bs]
    dev = DeviceBatch(bt)
    partition = int(rng.choice([0, 64, 256]))
    got = host(ops.paged_gqa_decode_shared_prefix(
        dev.query, dev.key_cache, dev.value_cache, dev.block_tables, dev.seq_lens,
        ops.to_device(np.array(starts, np.int32)), ops.to_device(np.array(prefixes, np.int32)),
        max(1, max(m for m, _, _ in groups)), bt.max_seq_len, bt.scale, partition_size=partition))
    ref = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                     bt.scale)
    assert_parity(got, ref, bt.dtype, f"{bt.describe()} groups={[(m, p) for m, p, _ in groups]} P={partition}")
