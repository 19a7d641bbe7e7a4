"""Host-side checks of the C ABI: the library loads without a GPU, exports every
function include/gqa_paged.h declares, and rejects bad scalar arguments with
status codes before touching the device."""
import ctypes
import os

import pytest

from gqa_paged_kv_attention_amd import ops

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    # GQA_TEST_LIB: another build of the same sources (tests/test_abi_sanitized.py runs this
    # module against the library with its host code built under AddressSanitizer and UBSan)
    return ops.load_library(os.environ.get("GQA_TEST_LIB", ops.LIB_PATH))


def dims(**kw):
    base = dict(num_seqs=4, num_heads=32, num_kv_heads=8, head_dim=128, block_size=16, num_blocks=100,
                max_blocks_per_seq=16, q_dtype=ops.GQA_BF16, kv_dtype=ops.GQA_BF16, out_dtype=ops.GQA_F32)
    base.update(kw)
    return ops.Dims(*[base[f] for f, _ in ops.Dims._fields_])


FAKE = ctypes.c_void_p(0x1000)    # never dereferenced: every call below fails validation first


def test_every_declared_symbol_is_exported(lib):
    names = ops.declared_functions()
    assert {"reshape_and_cache", "paged_gqa_decode", "paged_gqa_decode_append", "splitk_lse_reduce",
            "chunked_prefill_paged_decode",
            "paged_gqa_decode_workspace_size", "chunked_prefill_paged_decode_workspace_size",
            "paged_cross_attention", "paged_cross_attention_workspace_size",
            "paged_gqa_decode_shared_prefix", "paged_gqa_decode_shared_prefix_workspace_size",
            "gqa_status_string", "gqa_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert lib.gqa_status_string(0) == b"ok"
    assert lib.gqa_status_string(3) == b"workspace missing or too small"
    assert lib.gqa_status_string(99) == b"unknown status"
    assert lib.gqa_version() >= 100


def decode(lib, d, max_seq_len=256, partition=0, ws=None, wsb=0, ptr=FAKE, scale=0.1):
    return lib.paged_gqa_decode(ptr, ptr, ptr, ptr, ptr, ptr, max_seq_len, d, scale, partition, ws, wsb, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(num_kv_heads=7), INVALID),
    (dict(num_heads=0), INVALID),
    (dict(head_dim=96), UNSUPPORTED),
    (dict(block_size=8), UNSUPPORTED),
    (dict(block_size=48), UNSUPPORTED),
    (dict(block_size=128), UNSUPPORTED),
    (dict(q_dtype=ops.GQA_F32), UNSUPPORTED),
    (dict(out_dtype=7), INVALID),
    (dict(num_heads=64, num_kv_heads=1), UNSUPPORTED),       # group of 64 > 32
])
def test_decode_rejects_bad_dims(lib, kw, expect):
    assert decode(lib, dims(**kw)) == expect


@pytest.mark.parametrize("bs", [16, 32, 64])
def test_page_sizes_accepted(lib, bs):
    # past the dims check, a missing workspace is reported
    assert decode(lib, dims(block_size=bs, max_blocks_per_seq=4096 // bs), max_seq_len=4096, partition=512) == \
        WORKSPACE


def test_library_partition_pick_for_large_groups(lib):
    """With partition_size 0 and G = 32 over K/V beyond twice the 256 MB last-level cache, a
    batch of fewer (sequence, kv head) units than the device's 256 compute units is cut into
    partitions of at least 512 tokens (about two work-groups per compute unit).  Smaller K/V
    runs the 16-row units unsplit, and so does a batch that fills the device."""
    al = lambda x: (x + 255) // 256 * 256
    # 128 units, 16k tokens, a 1 GiB pool: four 4096-token partitions per sequence
    big = dims(num_seqs=128, num_kv_heads=1, max_blocks_per_seq=1024, num_blocks=131072)
    rows = 128 * 32 * 4
    assert lib.paged_gqa_decode_workspace_size(big, 16384, 0) == al(rows * 128 * 4) + al(rows * 4)
    # 4 units of up to 512k tokens: 128 partitions of 4096 tokens per sequence
    few = dims(num_seqs=4, num_kv_heads=1, max_blocks_per_seq=32768, num_blocks=131072)
    rows = 4 * 32 * 128
    assert lib.paged_gqa_decode_workspace_size(few, 524288, 0) == al(rows * 128 * 4) + al(rows * 4)
    # 4 units of 16k tokens (33.5 MB of K/V): no partitions
    assert lib.paged_gqa_decode_workspace_size(few, 16384, 0) == 0
    # the same batches over a small pool (K/V the cache holds): no partitions
    assert lib.paged_gqa_decode_workspace_size(dims(num_seqs=128, num_kv_heads=1, max_blocks_per_seq=1024), 16384, 0) == 0
    # 256 units fill the device: one partition per sequence
    g2 = dims(num_seqs=128, num_kv_heads=2, num_heads=64, max_blocks_per_seq=1024, num_blocks=131072)
    assert lib.paged_gqa_decode_workspace_size(g2, 16384, 0) == 0
    # an explicit partition size is kept
    rows = 128 * 32 * 4
    mqa = dims(num_seqs=128, num_kv_heads=1, max_blocks_per_seq=64)
    assert lib.paged_gqa_decode_workspace_size(mqa, 1024, 256) == al(rows * 128 * 4) + al(rows * 4)


def test_decode_rejects_null_pointer_and_bad_partition(lib):
    assert decode(lib, dims(), ptr=None) == INVALID
    assert decode(lib, dims(), partition=48) == INVALID        # not a multiple of 32
    assert decode(lib, dims(), partition=-32) == INVALID
    assert decode(lib, dims(), max_seq_len=-1) == INVALID
    assert decode(lib, dims(), scale=float("nan")) == INVALID


def test_workspace_size_and_check(lib):
    d = dims()
    # no split: nothing needed
    assert lib.paged_gqa_decode_workspace_size(d, 256, 256) == 0
    assert lib.paged_gqa_decode_workspace_size(d, 200, 1024) == 0
    # fixed split: partials for 8 partitions of every (sequence, query head)
    n = lib.paged_gqa_decode_workspace_size(d, 4096, 512)
    rows = 4 * 32 * 8
    assert n >= rows * 128 * 4 + rows * 4 and n % 256 == 0
    assert decode(lib, d, max_seq_len=4096, partition=512) == WORKSPACE
    assert decode(lib, d, max_seq_len=4096, partition=512, ws=FAKE, wsb=n - 1) == WORKSPACE
    f32 = dims(q_dtype=ops.GQA_F32, kv_dtype=ops.GQA_F32)
    assert lib.chunked_prefill_paged_decode_workspace_size(f32, 100, 4096, 512) == \
        lib.paged_gqa_decode_workspace_size(f32, 4096, 512)
    # balanced split: prefix table plus two segment slots per worker (at least one work-group's worth)
    s = lib.paged_gqa_decode_workspace_size(d, 4096, 0)
    assert s >= 4 * 2 * 4 * (128 + 1) * 4 and s % 256 == 0
    assert decode(lib, d, max_seq_len=4096, partition=0) == WORKSPACE
    assert decode(lib, d, max_seq_len=4096, partition=0, ws=FAKE, wsb=256) == WORKSPACE


def append(lib, d, key=FAKE, value=FAKE, ptr=FAKE, max_seq_len=256, partition=0, ws=None, wsb=0, scale=0.1):
    return lib.paged_gqa_decode_append(ptr, ptr, key, value, ptr, ptr, ptr, ptr, max_seq_len, d, scale, partition,
                                       ws, wsb, None)


def test_decode_append_validation(lib):
    """The fused append checks what paged_gqa_decode checks, plus its key and
    value rows; it takes paged_gqa_decode's workspace."""
    assert append(lib, dims(), key=None) == INVALID
    assert append(lib, dims(), value=None) == INVALID
    assert append(lib, dims(), partition=48) == INVALID
    assert append(lib, dims(), scale=float("inf")) == INVALID
    assert append(lib, dims(head_dim=96)) == UNSUPPORTED
    assert append(lib, dims(num_seqs=0), key=None, value=None, ptr=None) == OK
    assert append(lib, dims(), max_seq_len=4096, partition=512) == WORKSPACE
    assert append(lib, dims(), max_seq_len=4096, partition=0, ws=FAKE, wsb=256) == WORKSPACE


def test_empty_batches_return_ok_without_launch(lib):
    assert decode(lib, dims(num_seqs=0), ptr=None) == OK
    assert lib.reshape_and_cache(None, None, None, None, None, None, None, 0, dims(), None) == OK
    assert lib.chunked_prefill_paged_decode(None, None, None, None, None, None, None, 0, 0, 0, dims(), 0.1, 0,
                                            None, 0, None) == OK


def test_mixed_and_reduce_validation(lib):
    d = dims()
    assert lib.chunked_prefill_paged_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 20, 10, d, 0.1, 0,
                                            None, 0, None) == INVALID        # max_query_len > max_seq_len
    assert lib.chunked_prefill_paged_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 10, 5, 10, d, 0.1, 0,
                                            None, 0, None) == INVALID        # no query_start_loc
    assert lib.reshape_and_cache(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -1, d, None) == INVALID
    assert lib.splitk_lse_reduce(FAKE, FAKE, FAKE, FAKE, None, d, 0, 512, 1, None) == INVALID
    assert lib.splitk_lse_reduce(FAKE, FAKE, FAKE, FAKE, None, d, 4, 0, 1, None) == INVALID


def test_mixed_bf16_workspace(lib):
    """bf16 mixed batches need the scheduled unit list (64 bytes per unit, at
    least num_tokens * G / 128 prefill row tiles plus one unit per decode), a
    count, and partials only when decodes are split; a batch of decodes only
    runs the decode, so the decode's workspace fits as well."""
    d = dims()                                     # 4 seqs, G = 4, bf16
    n = lib.chunked_prefill_paged_decode_workspace_size(d, 1000, 256, 0)
    assert n % 256 == 0 and n >= (1000 * 4 // 128 + 4) * 64 + 4
    assert n >= lib.paged_gqa_decode_workspace_size(d, 256, 0)
    # a split adds the partials of 16 partitions per (sequence, query head)
    split = lib.chunked_prefill_paged_decode_workspace_size(d, 1000, 8192, 512)
    assert split >= (1000 * 4 // 128 + 4 * 17) * 64 + 4 * 32 * 16 * 128 * 4
    assert split >= lib.paged_gqa_decode_workspace_size(d, 8192, 512)
    call = lambda ws, wsb: lib.chunked_prefill_paged_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1000, 100, 256,
                                                            d, 0.1, 0, ws, wsb, None)
    assert call(None, 0) == WORKSPACE
    assert call(FAKE, n - 1) == WORKSPACE
    assert lib.chunked_prefill_paged_decode_workspace_size(d, -1, 256, 0) == 0


def cross(lib, d, num_tokens=10, max_query_len=20, max_encoder_len=10, ws=None, wsb=0, ptr=FAKE, qsl=FAKE):
    return lib.paged_cross_attention(ptr, ptr, ptr, ptr, ptr, ptr, qsl, num_tokens, max_query_len, max_encoder_len,
                                     d, 0.1, 0, ws, wsb, None)


def test_cross_attention_validation(lib):
    d = dims()
    # a chunk may be longer than the encoder sequence: past validation, the
    # missing workspace is reported (the causal call rejects the same lengths)
    assert cross(lib, d) == WORKSPACE
    assert lib.chunked_prefill_paged_decode(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 10, 20, 10, d, 0.1, 0,
                                            None, 0, None) == INVALID
    assert cross(lib, d, qsl=None) == INVALID
    assert cross(lib, d, ptr=None) == INVALID
    assert cross(lib, d, max_query_len=-1) == INVALID
    assert cross(lib, dims(head_dim=96)) == UNSUPPORTED
    assert cross(lib, dims(num_seqs=0), ptr=None, qsl=None) == OK
    n = lib.paged_cross_attention_workspace_size(d, 1000, 6400, 0)
    assert n == lib.chunked_prefill_paged_decode_workspace_size(d, 1000, 6400, 0)
    assert cross(lib, d, num_tokens=1000, max_query_len=100, max_encoder_len=6400, ws=FAKE, wsb=n - 1) == WORKSPACE


def shared(lib, d, num_groups=2, max_group_size=4, max_seq_len=4096, partition=0, ws=None, wsb=0, ptr=FAKE, gptr=FAKE):
    return lib.paged_gqa_decode_shared_prefix(ptr, ptr, ptr, ptr, ptr, ptr, gptr, gptr, num_groups, max_group_size,
                                              max_seq_len, d, 0.1, partition, ws, wsb, None)


def test_shared_prefix_validation(lib):
    d = dims()                                     # 4 sequences
    n = lib.paged_gqa_decode_shared_prefix_workspace_size(d, 2, 4, 4096, 0)
    # partials for at least 2 prefix chunks (of <= 2048 keys) + 1 suffix partition per (sequence, head)
    assert n >= 4 * 32 * 3 * (128 + 1) * 4 and n % 256 == 0
    # a fixed partition size sets the suffix slots: 4096 / 256 = 16 of them
    assert lib.paged_gqa_decode_shared_prefix_workspace_size(d, 2, 4, 4096, 256) >= 4 * 32 * 17 * (128 + 1) * 4
    assert shared(lib, d) == WORKSPACE
    assert shared(lib, d, ws=FAKE, wsb=n - 1) == WORKSPACE
    assert shared(lib, d, max_group_size=5) == INVALID          # larger than the batch
    assert shared(lib, d, partition=48) == INVALID
    assert shared(lib, d, num_groups=-1) == INVALID
    assert shared(lib, d, gptr=None) == INVALID
    assert shared(lib, d, ptr=None) == INVALID
    assert shared(lib, dims(num_seqs=0), num_groups=0, max_group_size=0, ptr=None, gptr=None) == OK
    assert lib.paged_gqa_decode_shared_prefix_workspace_size(d, 2, 5, 4096, 0) == 0
    f32 = dims(q_dtype=ops.GQA_F32, kv_dtype=ops.GQA_F32)
    assert lib.paged_gqa_decode_shared_prefix_workspace_size(f32, 2, 4, 4096, 512) == \
        lib.paged_gqa_decode_workspace_size(f32, 4096, 512)


def test_noalloc_rejects_calls_beyond_its_scratch(lib):
    """paged_gqa_decode_noalloc checks the call's scratch need against its fixed
    static buffer on the host, before any device call: 4096 sequences x 64
    heads in 8 partitions need 1 GiB of partials."""
    assert lib.gqa_status_string(5) == b"call needs more scratch than the library's static buffer holds"
    big = dims(num_seqs=4096, num_heads=64, num_kv_heads=8, max_blocks_per_seq=256)
    assert lib.paged_gqa_decode_workspace_size(big, 4096, 512) > ops.NOALLOC_SCRATCH_BYTES
    assert lib.paged_gqa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, big, 0.1, 512, None) == 5
    # argument errors come first, as in paged_gqa_decode
    assert lib.paged_gqa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4096, dims(num_kv_heads=7), 0.1, 0,
                                        None) == INVALID
    assert lib.paged_gqa_decode_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 256, dims(), 0.1, 48, None) == INVALID
    # no sequences: nothing to do, nothing looked up
    assert lib.paged_gqa_decode_noalloc(None, None, None, None, None, None, 0, dims(num_seqs=0), 0.1, 0, None) == OK


def test_mfma_probe_rejects_bad_arguments(lib):
    flops = ctypes.c_longlong(0)
    assert lib.gqa_probe_mfma_bf16(None, 4, 10, ctypes.byref(flops), None) == INVALID
    assert lib.gqa_probe_mfma_bf16(FAKE, 0, 10, ctypes.byref(flops), None) == INVALID
    assert lib.gqa_probe_mfma_bf16(FAKE, 4, 0, ctypes.byref(flops), None) == INVALID
