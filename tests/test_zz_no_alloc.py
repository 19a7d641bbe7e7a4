"""paged_gqa_decode_noalloc (the decode with the library's static per-device
scratch instead of a caller workspace) against paged_gqa_decode with a
workspace, through the C ABI, on two calls in a row, the second on a smaller
batch: the scratch keeps the first call's contents, and the second call must
not depend on them.  Both calls also meet the parity bar against the oracle."""
import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import ops
from gqa_paged_kv_attention_amd import workloads as wl
from oracle import decode_ref
from tests.gpu_util import DeviceBatch, assert_parity, have_gpu, host, poison_tails

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def oracle(bt):
    return decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                      bt.scale)


@pytest.mark.parametrize("partition", [0, 512])
def test_noalloc_matches_workspace_decode_twice(partition):
    big = wl.llama31_8b_decode(seed=2, num_seqs=48, ctx_lo=300, ctx_hi=3000)
    small = wl.make_batch(name="noalloc_small", seed=9, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                          seq_lens=[1, 17, 300, 0, 64, 1000, 33], query_lens=[1, 1, 1, 0, 1, 1, 1], dtype=wl.BF16,
                          poison_slack=True)
    small.query = wl._normal_storage(np.random.default_rng(3), (small.num_seqs, 32, 128), wl.BF16)
    poison_tails(small)
    for bt in (big, small):
        dev = DeviceBatch(bt)
        want = dev.decode(partition)
        got = ops.paged_gqa_decode_noalloc(dev.query, dev.key_cache, dev.value_cache, dev.block_tables,
                                           dev.seq_lens, bt.max_seq_len, bt.scale, partition_size=partition)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{bt.describe()} P={partition}"
        assert_parity(host(got), oracle(bt), bt.dtype, f"{bt.describe()} P={partition}")


def test_noalloc_rejects_a_call_beyond_its_scratch():
    """A call whose partials exceed the static scratch returns GQA_ERR_SCRATCH
    (the binding raises) and launches nothing; a fitting call afterwards works."""
    bt = wl.make_batch(name="noalloc_big", seed=4, num_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                       seq_lens=[40] * 1024, query_lens=[1] * 1024, dtype=wl.BF16)
    dev = DeviceBatch(bt)
    dims = ops.make_dims(num_seqs=bt.num_seqs, num_heads=64, key_cache=dev.key_cache,
                         block_tables=dev.block_tables, q_dtype=dev.query.dtype, out_dtype=torch.float32)
    assert ops.decode_workspace_size(dims, 8192, 32) > ops.NOALLOC_SCRATCH_BYTES
    with pytest.raises(ops.GqaError, match="GQA_ERR_SCRATCH"):
        ops.paged_gqa_decode_noalloc(dev.query, dev.key_cache, dev.value_cache, dev.block_tables, dev.seq_lens,
                                     8192, bt.scale, partition_size=32)
    got = ops.paged_gqa_decode_noalloc(dev.query, dev.key_cache, dev.value_cache, dev.block_tables, dev.seq_lens,
                                       bt.max_seq_len, bt.scale)
    assert_parity(host(got), oracle(bt), bt.dtype, bt.describe())
