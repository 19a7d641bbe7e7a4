"""Shape validation of the Python binding (CPU only, no kernel launch).

Every wrapper checks the shapes of its tensors against each other before it
touches the library or the device, so a short output, a short block table or a
value cache in the key cache's layout raises ValueError instead of reaching a
kernel as a pointer.  Plain CPU tensors suffice: the checks run first.
"""
import pytest
import torch

from gqa_paged_kv_attention_amd import ops

NB, HKV, BS, D, HQ, B = 12, 2, 16, 64, 8, 3


def caches(value_layout="channel_major"):
    kc = torch.empty(NB, HKV, BS, D, dtype=torch.bfloat16)
    vc = torch.empty(NB, HKV, D, BS, dtype=torch.bfloat16) if value_layout == "channel_major" else \
        torch.empty(NB, HKV, BS, D, dtype=torch.bfloat16)
    return kc, vc


def tables(rows=B):
    return torch.zeros(rows, 4, dtype=torch.int32)


def lens(n=B):
    return torch.full((n,), 20, dtype=torch.int32)


def qsl(n=B):
    return torch.arange(n + 1, dtype=torch.int32)


def query(rows=B, hq=HQ, d=D):
    return torch.empty(rows, hq, d, dtype=torch.bfloat16)


def test_value_cache_in_key_layout_is_rejected():
    kc, vc = caches("token_major")
    with pytest.raises(ValueError, match="value_cache"):
        ops.paged_gqa_decode(query(), kc, vc, tables(), lens(), 64, 0.125)
    with pytest.raises(ValueError, match="value_cache"):
        ops.chunked_prefill_paged_decode(query(), kc, vc, tables(), lens(), qsl(), 1, 64, 0.125)


@pytest.mark.parametrize("call", ["decode", "append", "mixed", "cross", "shared"])
def test_short_output_is_rejected(call):
    kc, vc = caches()
    out = torch.empty(B - 1, HQ, D)
    with pytest.raises(ValueError, match="out"):
        if call == "decode":
            ops.paged_gqa_decode(query(), kc, vc, tables(), lens(), 64, 0.125, out=out)
        elif call == "append":
            kv = torch.empty(B, HKV, D, dtype=torch.bfloat16)
            ops.paged_gqa_decode_append(query(), kv, kv, kc, vc, tables(), lens(), 64, 0.125, out=out)
        elif call == "mixed":
            ops.chunked_prefill_paged_decode(query(), kc, vc, tables(), lens(), qsl(), 1, 64, 0.125, out=out)
        elif call == "cross":
            ops.paged_cross_attention(query(), kc, vc, tables(), lens(), qsl(), 1, 64, 0.125, out=out)
        else:
            gs, pl = torch.tensor([0, B], dtype=torch.int32), torch.tensor([16], dtype=torch.int32)
            ops.paged_gqa_decode_shared_prefix(query(), kc, vc, tables(), lens(), gs, pl, B, 64, 0.125, out=out)


def test_short_block_table_and_length_arrays_are_rejected():
    kc, vc = caches()
    with pytest.raises(ValueError, match="block_tables"):
        ops.paged_gqa_decode(query(), kc, vc, tables(B - 1), lens(), 64, 0.125)
    with pytest.raises(ValueError, match="seq_lens"):
        ops.paged_gqa_decode(query(), kc, vc, tables(), lens(B + 1), 64, 0.125)
    with pytest.raises(ValueError, match="query_start_loc"):
        ops.chunked_prefill_paged_decode(query(), kc, vc, tables(), lens(), qsl(B - 1), 1, 64, 0.125)
    # the lengths array sets the sequence count, so a short one disagrees with query_start_loc
    with pytest.raises(ValueError, match="query_start_loc"):
        ops.paged_cross_attention(query(), kc, vc, tables(), lens(B - 1), qsl(), 1, 64, 0.125)
    with pytest.raises(ValueError, match="encoder_lens"):
        ops.paged_cross_attention(query(), kc, vc, tables(), lens().view(B, 1), qsl(), 1, 64, 0.125)


def test_query_and_new_token_shapes_are_checked():
    kc, vc = caches()
    with pytest.raises(ValueError, match="query"):
        ops.paged_gqa_decode(query(d=128), kc, vc, tables(), lens(), 64, 0.125)
    with pytest.raises(ValueError, match="query"):
        ops.paged_gqa_decode(query(hq=HQ + 1), kc, vc, tables(), lens(), 64, 0.125)
    bad = torch.empty(B, HKV + 1, D, dtype=torch.bfloat16)
    good = torch.empty(B, HKV, D, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="key"):
        ops.paged_gqa_decode_append(query(), bad, good, kc, vc, tables(), lens(), 64, 0.125)
    with pytest.raises(ValueError, match="key"):
        ops.reshape_and_cache(bad, bad, kc, vc, tables(), lens(), qsl())
    with pytest.raises(ValueError, match="value"):
        ops.reshape_and_cache(good, torch.empty(B + 1, HKV, D, dtype=torch.bfloat16), kc, vc, tables(), lens(),
                              qsl())


def test_splitk_partial_shapes_are_checked():
    po = torch.empty(B, HQ, 4, D)
    with pytest.raises(ValueError, match="partial_lse"):
        ops.splitk_lse_reduce(po, torch.empty(B, HQ, 3), lens(), 32, num_kv_heads=HKV, max_blocks_per_seq=4)
    with pytest.raises(ValueError, match="seq_lens"):
        ops.splitk_lse_reduce(po, torch.empty(B, HQ, 4), lens(B - 1), 32, num_kv_heads=HKV, max_blocks_per_seq=4)
    with pytest.raises(ValueError, match="out"):
        ops.splitk_lse_reduce(po, torch.empty(B, HQ, 4), lens(), 32, num_kv_heads=HKV, max_blocks_per_seq=4,
                              out=torch.empty(B, HQ, D + 1))


def test_well_formed_cpu_tensors_pass_the_shape_checks():
    """With every shape right, the first complaint is the device check."""
    kc, vc = caches()
    with pytest.raises(ValueError, match="GPU"):
        ops.paged_gqa_decode(query(), kc, vc, tables(), lens(), 64, 0.125)
    with pytest.raises(ValueError, match="GPU"):
        ops.chunked_prefill_paged_decode(query(), kc, vc, tables(), lens(), qsl(), 1, 64, 0.125)
