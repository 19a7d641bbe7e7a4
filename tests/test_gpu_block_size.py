"""Page sizes of 16, 32 and 64 tokens.

The kernels walk keys in 32-token tiles (64-token tiles in the bf16 prefill)
of 16-token halves, each inside one page, whatever the page size.  So the
same cached tokens stored in 16-, 32- or 64-token pages give bitwise equal
results; each page size is also compared with the CPU fp64 oracle, and the
cache write is bit-exact.  Parity bar as in test_gpu_parity.py.
"""
import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import ops
from gqa_paged_kv_attention_amd import workloads as wl
from oracle import cache_write_ref, decode_ref, paged_attention_ref
from tests import full_size
from tests.gpu_util import DeviceBatch, assert_parity, have_gpu, host, poison_tails, repage

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]

BLOCK_SIZES = [32, 64]


@pytest.mark.parametrize("bs", BLOCK_SIZES)
@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kind", ["mixed", "decode"])
def test_cache_write_bit_exact(bs, dtype, d, kind):
    rng = np.random.default_rng(17)
    q_lens = {"mixed": np.array([1, 5, 0, 70, 1, 33, 2, 130]), "decode": np.ones(300, dtype=np.int64)}[kind]
    seq_lens = q_lens + rng.integers(0, 150, size=len(q_lens))
    bt = wl.make_batch(name="rc_bs", seed=18, num_heads=8, num_kv_heads=4, head_dim=d, block_size=bs,
                       seq_lens=seq_lens, query_lens=q_lens, dtype=dtype)
    dev = DeviceBatch(bt)
    dev.cache_write()
    torch.cuda.synchronize()
    kc, vc = cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                             bt.query_start_loc)
    assert np.array_equal(ops.to_host_storage(dev.key_cache).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(ops.to_host_storage(dev.value_cache).view(np.uint8), vc.view(np.uint8))


DEC_LENS = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 511, 512, 513, 1000, 3000]


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (32, 1), (16, 16)])
def test_decode_page_size_invariance(dtype, d, hq, hkv):
    base = wl.make_batch(name="dec_bs", seed=hq + hkv + d, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                         block_size=16, seq_lens=DEC_LENS, query_lens=[0 if L == 0 else 1 for L in DEC_LENS],
                         dtype=dtype, poison_slack=True)
    base.query = wl._normal_storage(np.random.default_rng(1), (len(DEC_LENS), hq, d), dtype)
    poison_tails(base)
    ref = decode_ref(base.query, base.key_cache, base.value_cache, base.block_tables, base.seq_lens, hkv, base.scale)
    for partition in (0, 64, 512):
        want = DeviceBatch(base).decode(partition)
        for bs in BLOCK_SIZES:
            bt = repage(base, bs, seed=bs)
            got = DeviceBatch(bt).decode(partition)
            torch.cuda.synchronize()
            if partition:
                assert torch.equal(got, want), f"bs={bs} P={partition}"
            else:
                # the balanced split sizes its workers by the kernel's occupancy,
                # which may differ between page sizes: equal up to rounding
                torch.testing.assert_close(got, want, rtol=1e-5, atol=1e-6)
        assert_parity(host(want), ref, dtype, f"{base.describe()} P={partition}")


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (16, 1)])
def test_mixed_page_size_invariance(dtype, d, hq, hkv):
    q_lens = [2, 1, 0, 7, 33, 1, 64, 130, 5, 1, 16, 300]
    prior = [0, 40, 3, 9, 0, 300, 17, 70, 511, 0, 16, 1000]
    base = wl.make_batch(name="mix_bs", seed=3 * hq + hkv + d, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                         block_size=16, seq_lens=[a + b for a, b in zip(q_lens, prior)], query_lens=q_lens,
                         dtype=dtype, poison_slack=True)
    poison_tails(base)
    ref = paged_attention_ref(base.query, base.key_cache, base.value_cache, base.block_tables, base.seq_lens,
                              base.query_start_loc, hkv, base.scale)
    for partition in (0, 64):
        want = DeviceBatch(base).mixed(partition)
        for bs in BLOCK_SIZES:
            got = DeviceBatch(repage(base, bs, seed=bs)).mixed(partition)
            torch.cuda.synchronize()
            assert torch.equal(got, want), f"bs={bs} P={partition}"
        assert_parity(host(want), ref, dtype, f"{base.describe()} P={partition}")


@pytest.mark.parametrize("bs", BLOCK_SIZES)
def test_cross_page_size(bs):
    base = wl.make_batch(name="cross_bs", seed=bs, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                         seq_lens=[3, 40, 0, 700, 129], query_lens=[7, 40, 2, 100, 1], dtype=wl.BF16, cross=True,
                         poison_slack=True)
    poison_tails(base)
    want = DeviceBatch(base).cross(0)
    bt = repage(base, bs, seed=bs)
    got = DeviceBatch(bt).cross(0)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    ref = paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                              bt.query_start_loc, bt.num_kv_heads, bt.scale, causal=False)
    assert_parity(host(got), ref, bt.dtype, bt.describe())


@pytest.mark.parametrize("bs", BLOCK_SIZES)
def test_full_llama31_decode_step_page_size(bs):
    """The benchmark's decode step (cache write + decode, library-picked split)
    with bs-token pages: the whole output against the oracle."""
    bt = wl.llama31_8b_decode(seed=2, block_size=bs)
    dev = DeviceBatch(bt)
    dev.cache_write()
    out = host(dev.decode(0))
    assert_parity(out, full_size.llama31_decode(bs), bt.dtype, bt.describe())
