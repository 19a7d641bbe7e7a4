"""GPU parity of paged_cross_attention: decoder rows over a static encoder
cache with no causal mask, against the CPU fp64 oracle (``causal=False``).

Same bar as the other parity tests: max-abs <= 1e-2 and relative L2 <= 2e-3
(bf16 inputs, fp32 accumulation); fp32 inputs also meet relative L2 <= 1e-5.
"""
import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import ops
from gqa_paged_kv_attention_amd import workloads as wl
from oracle import paged_attention_ref
from tests import full_size
from tests.gpu_util import DeviceBatch, assert_parity, have_gpu, host, poison_tails

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not have_gpu(), reason="needs a GPU")]


def cross_ref(bt, scale=None, seqs=None):
    return paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                               bt.query_start_loc, bt.num_kv_heads, bt.scale if scale is None else scale,
                               seqs=seqs, causal=False)


# chunks longer than, equal to and shorter than their encoder sequence, single
# rows, an empty chunk, empty encoder sequences (with rows and with one row),
# encoder lengths on and off tile and page boundaries
Q_LENS = [7, 1, 0, 40, 33, 1, 300, 130, 5, 1, 16, 3, 64]
ENC_LENS = [3, 40, 12, 40, 0, 0, 129, 700, 511, 64, 2000, 1, 64]


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (32, 1), (12, 2), (32, 8)])
def test_cross_edge_shapes(dtype, d, hq, hkv):
    bt = wl.make_batch(name="cross_edge", seed=hq + 5 * hkv + d, num_heads=hq, num_kv_heads=hkv, head_dim=d,
                       block_size=16, seq_lens=ENC_LENS, query_lens=Q_LENS, dtype=dtype, poison_slack=True,
                       cross=True)
    poison_tails(bt)
    dev = DeviceBatch(bt)
    ref = cross_ref(bt)
    for partition in (0, 64):
        got = host(dev.cross(partition))
        assert_parity(got, ref, dtype, f"{bt.describe()} P={partition}")
        for b in (4, 5):                               # empty encoder: zero rows
            q0, q1 = bt.query_start_loc[b], bt.query_start_loc[b + 1]
            assert not got[q0:q1].any()


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
@pytest.mark.parametrize("scale", [-0.2, 0.0])
def test_cross_scale_sign(dtype, scale):
    """Zero scale averages every encoder value for every row; a negative scale
    reverses which keys dominate."""
    bt = wl.make_batch(name="cross_scale", seed=77, num_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                       seq_lens=[50, 9, 300, 7], query_lens=[80, 1, 33, 2], dtype=dtype, cross=True)
    dev = DeviceBatch(bt)
    got = host(ops.paged_cross_attention(dev.query, dev.key_cache, dev.value_cache, dev.block_tables,
                                         dev.seq_lens, dev.query_start_loc, bt.max_query_len, bt.max_seq_len, scale))
    assert_parity(got, cross_ref(bt, scale=scale), dtype, f"{bt.describe()} scale={scale}")


@pytest.mark.parametrize("partition", [0, 256])
def test_cross_decode_rows_equal_paged_decode(partition):
    """A batch of single decoder rows runs the decode: the result is bitwise
    that of paged_gqa_decode on the same encoder cache, and matches the oracle."""
    bt = wl.cross_attention(seed=6, num_seqs=12, enc_lo=100, enc_hi=3000, query_len=1)
    dev = DeviceBatch(bt)
    got = dev.cross(partition)
    dec = dev.decode(partition)
    torch.cuda.synchronize()
    assert torch.equal(got, dec)
    assert_parity(host(got), cross_ref(bt), bt.dtype, bt.describe())


def test_cross_bf16_output_is_rounded_fp32():
    bt = wl.cross_attention(seed=7, num_seqs=6, enc_lo=200, enc_hi=1500, query_len=40)
    dev = DeviceBatch(bt)
    o32 = dev.cross(0, out_dtype=torch.float32)
    o16 = dev.cross(0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert_parity(host(o16), cross_ref(bt), bt.dtype, bt.describe() + " bf16 out")


def test_cross_rows_are_independent_of_position_on_gpu():
    """Reversing a chunk's rows reverses the output rows (no causal mask)."""
    bt = wl.cross_attention(seed=8, num_seqs=3, enc_lo=300, enc_hi=900, query_len=70)
    dev = DeviceBatch(bt)
    out = host(dev.cross(0))
    rows = torch.arange(bt.num_tokens, device="cuda")
    for b in range(bt.num_seqs):
        q0, q1 = int(bt.query_start_loc[b]), int(bt.query_start_loc[b + 1])
        rows[q0:q1] = torch.arange(q1 - 1, q0 - 1, -1, device="cuda")
    dev.query = dev.query[rows].contiguous()
    rev = host(dev.cross(0))
    assert_parity(rev, out[rows.cpu().numpy()], bt.dtype, bt.describe() + " reversed rows")


# --------------------------------------------------------------------------
# full-size workloads (the benchmark's shapes and launch configuration): the
# whole output against the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("query_len", [1, 256])
def test_full_cross_attention(query_len):
    bt = wl.cross_attention(seed=6, query_len=query_len)
    out = host(DeviceBatch(bt).cross(0))
    assert_parity(out, full_size.cross(query_len), bt.dtype, bt.describe())
