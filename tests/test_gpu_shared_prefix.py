"""GPU parity of paged_gqa_decode_shared_prefix: groups of sequences whose
block tables share their first pages (prefix caching).  The result must be
that of the plain decode of each sequence over its own pages, checked against
the CPU fp64 oracle (decode_ref) at the usual bar: max-abs <= 1e-2 and
relative L2 <= 2e-3 for bf16 inputs; fp32 caches run the plain decode and
must equal paged_gqa_decode bitwise.
"""
import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import ops
from gqa_paged_kv_attention_amd import workloads as wl
from oracle import decode_ref
from tests import full_size
from tests.gpu_util import DeviceBatch, assert_parity, have_gpu, host, poison_tails

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def grouped_batch(seed, groups, hq=32, hkv=8, d=128, bs=16, dtype=wl.BF16, poison=True):
    """groups: list of (members, prefix_len, [suffix lengths]); prefix_len a multiple of bs."""
    seq_lens, starts, prefixes = [], [0], []
    for members, prefix, suffixes in groups:
        assert len(suffixes) == members
        seq_lens += [prefix + s for s in suffixes]
        starts.append(starts[-1] + members)
        prefixes.append(prefix)
    bt = wl.make_batch(name="grouped", seed=seed, num_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs,
                       seq_lens=seq_lens, query_lens=[1] * len(seq_lens), dtype=dtype, poison_slack=poison)
    for g, (members, prefix, _) in enumerate(groups):
        first = starts[g]
        bt.block_tables[first + 1:first + members, :prefix // bs] = bt.block_tables[first, :prefix // bs]
    if poison:
        poison_tails(bt)
    return bt, np.array(starts, np.int32), np.array(prefixes, np.int32)


def run_shared(bt, starts, prefixes, partition=0, out_dtype=torch.float32, max_group_size=None):
    dev = DeviceBatch(bt)
    gs, pl = ops.to_device(starts), ops.to_device(prefixes)
    mg = int(np.max(np.diff(starts))) if len(prefixes) else 0
    out = ops.paged_gqa_decode_shared_prefix(dev.query, dev.key_cache, dev.value_cache, dev.block_tables,
                                             dev.seq_lens, gs, pl, mg if max_group_size is None else max_group_size,
                                             bt.max_seq_len, bt.scale, partition_size=partition, out_dtype=out_dtype)
    return dev, out


def oracle(bt):
    return decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                      bt.scale)


# prefixes on and off 64-key tiles and 256-key chunks, a suffix of 0 (the
# whole sequence is the prefix), groups of 1, 3 and 40 members (40 x G rows
# need several row tiles), an empty group
GROUPS = [(3, 1024, [0, 7, 300]), (1, 64, [40]), (40, 528, list(range(1, 401, 10))), (2, 0, [33, 1]),
          (0, 256, []), (5, 16, [100, 0, 64, 65, 2000])]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(32, 8), (32, 1), (8, 8), (48, 2)])
def test_shared_prefix_matches_oracle(d, hq, hkv):
    bt, starts, prefixes = grouped_batch(hq * 3 + hkv + d, GROUPS, hq=hq, hkv=hkv, d=d)
    ref = oracle(bt)
    for partition in (0, 64):
        _, out = run_shared(bt, starts, prefixes, partition)
        assert_parity(host(out), ref, bt.dtype, f"{bt.describe()} P={partition}")


@pytest.mark.parametrize("bs", [32, 64])
def test_shared_prefix_page_sizes(bs):
    groups = [(4, 1024, [0, 7, 300, 64]), (6, 64 * 3, [1, 2, 3, 500, 64, 65])]
    bt, starts, prefixes = grouped_batch(bs, groups, bs=bs)
    _, out = run_shared(bt, starts, prefixes)
    assert_parity(host(out), oracle(bt), bt.dtype, bt.describe())


def test_shared_prefix_ungrouped_sequences_and_bf16_output():
    """Sequences outside every group decode on their own; bf16 output is the
    fp32 result rounded."""
    bt, starts, prefixes = grouped_batch(5, [(4, 512, [3, 30, 300, 0]), (3, 0, [10, 1000, 64])])
    # only the first group is declared: the last three sequences are in no group
    starts, prefixes = starts[:2], prefixes[:1]
    _, o32 = run_shared(bt, starts, prefixes)
    _, o16 = run_shared(bt, starts, prefixes, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert_parity(host(o32), oracle(bt), bt.dtype, bt.describe())
    _, none = run_shared(bt, np.zeros(1, np.int32), np.zeros(0, np.int32), max_group_size=0)
    assert_parity(host(none), oracle(bt), bt.dtype, bt.describe() + " no groups")


def test_shared_prefix_fp32_runs_plain_decode():
    bt, starts, prefixes = grouped_batch(6, [(5, 256, [1, 2, 3, 4, 5])], hq=8, hkv=2, d=64, dtype=wl.F32)
    dev, out = run_shared(bt, starts, prefixes, partition=64)
    plain = dev.decode(64)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)
    assert_parity(host(out), oracle(bt), bt.dtype, bt.describe())


def test_shared_prefix_many_groups():
    """More groups than a work-group has threads (300 groups of one or two
    members, prefixes on and off 64-key tiles): the suffix units find their
    sequence's group in a later chunk of the group list."""
    rng = np.random.default_rng(31)
    groups = []
    for g in range(300):
        members = 1 + g % 2
        groups.append((members, 16 * int(rng.integers(0, 9)), [int(x) for x in rng.integers(1, 90, members)]))
    bt, starts, prefixes = grouped_batch(30, groups, hq=8, hkv=2, d=64)
    for partition in (0, 64):
        _, out = run_shared(bt, starts, prefixes, partition=partition)
        assert_parity(host(out), oracle(bt), bt.dtype, f"{bt.describe()} P={partition}")


def test_shared_prefix_workspace_reuse():
    """One workspace, two calls in a row (the second smaller): each call
    rewrites the partial counts it reads."""
    big, s1, p1 = grouped_batch(8, [(10, 1024, list(range(5, 505, 50))), (3, 256, [1, 2, 3])])
    small, s2, p2 = grouped_batch(9, [(2, 512, [10, 20])])
    dims = lambda bt, d: ops.make_dims(num_seqs=bt.num_seqs, num_heads=bt.num_heads, key_cache=d.key_cache,
                                       block_tables=d.block_tables, q_dtype=d.query.dtype, out_dtype=torch.float32)
    db, dsm = DeviceBatch(big), DeviceBatch(small)
    n = max(ops.shared_prefix_workspace_size(dims(big, db), 2, 10, big.max_seq_len, 0),
            ops.shared_prefix_workspace_size(dims(small, dsm), 1, 2, small.max_seq_len, 0))
    ws = torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")
    for bt, dev, s, p in ((big, db, s1, p1), (small, dsm, s2, p2)):
        out = ops.paged_gqa_decode_shared_prefix(dev.query, dev.key_cache, dev.value_cache, dev.block_tables,
                                                 dev.seq_lens, ops.to_device(s), ops.to_device(p),
                                                 int(np.max(np.diff(s))), bt.max_seq_len, bt.scale, workspace=ws)
        assert_parity(host(out), oracle(bt), bt.dtype, bt.describe())


@pytest.mark.parametrize("prefix_len,group_size", [(2048, 16), (4096, 64)])
def test_full_shared_prefix(prefix_len, group_size):
    """Benchmark shapes: groups sharing a long prompt; the whole output against
    the oracle's plain decode of every sequence."""
    bt, starts, prefixes = wl.shared_prefix_decode(seed=7, num_groups=4, group_size=group_size,
                                                   prefix_len=prefix_len)
    _, out = run_shared(bt, starts, prefixes)
    assert_parity(host(out), full_size.shared_prefix(prefix_len, group_size), bt.dtype, bt.describe())
