"""Pins for the CPU fp64 oracle, each independent of the oracle's own code.

Each test checks the oracle against something fixed outside it: a pure-Python
brute force, the GQA == expanded-MHA equivalence of "[Performance] Use optimized
kernels for MQA/GQA" (opening post, item 1), closed forms, invariances, or a
library routine (torch SDPA in float64 on the CPU).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from gqa_paged_kv_attention_amd import workloads as wl
from oracle import (cache_write_ref, decode_partials_ref, decode_ref, gather_sequence, lse_merge_ref,
                    paged_attention_ref)


# --------------------------------------------------------------------------
# helpers (test-side only)
# --------------------------------------------------------------------------

def small_batch(seed, seq_lens, query_lens, Hq=4, Hkv=2, d=8, bs=4, dtype=wl.F32, **kw):
    return wl.make_batch(name="t", seed=seed, num_heads=Hq, num_kv_heads=Hkv, head_dim=d, block_size=bs,
                         seq_lens=seq_lens, query_lens=query_lens, dtype=dtype, **kw)


def f(arr):
    return wl.storage_to_f32(arr).astype(np.float64)


def run_ref(bt, **kw):
    return paged_attention_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                               bt.query_start_loc, bt.num_kv_heads, bt.scale, **kw)


def bruteforce(bt, causal=True):
    """Pure-Python loops: per token, per head, per key, with math.exp.  A row
    with no visible key stays zero."""
    Hq, Hkv, d, bs = bt.num_heads, bt.num_kv_heads, bt.head_dim, bt.block_size
    G = Hq // Hkv
    Kc, Vc, Q = f(bt.key_cache), f(bt.value_cache), f(bt.query)
    out = np.zeros((bt.num_tokens, Hq, d))
    for b in range(bt.num_seqs):
        L = int(bt.seq_lens[b])
        q0, q1 = int(bt.query_start_loc[b]), int(bt.query_start_loc[b + 1])
        for j in range(q1 - q0):
            last_visible = L - (q1 - q0) + j if causal else L - 1
            if last_visible < 0:
                continue
            for h in range(Hq):
                kv = h // G
                scores = []
                for t in range(last_visible + 1):
                    page = int(bt.block_tables[b][t // bs])
                    slot = t % bs
                    s = 0.0
                    for c in range(d):
                        s += float(Q[q0 + j, h, c]) * float(Kc[page, kv, slot, c])
                    scores.append(bt.scale * s)
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                for c in range(d):
                    acc = 0.0
                    for t in range(last_visible + 1):
                        page = int(bt.block_tables[b][t // bs])
                        acc += ws[t] * float(Vc[page, kv, c, t % bs])
                    out[q0 + j, h, c] = acc / tot
    return out


def poison_tails(bt):
    """NaN into every slot past the end of each sequence's last page (test-side)."""
    nan = np.uint16(0x7FC0) if bt.dtype == wl.BF16 else np.float32("nan")
    for b in range(bt.num_seqs):
        L = int(bt.seq_lens[b])
        n = -(-L // bt.block_size)
        if n == 0:
            continue
        used = L - (n - 1) * bt.block_size
        page = bt.block_tables[b][n - 1]
        bt.key_cache[page, :, used:, :] = nan
        bt.value_cache[page, :, :, used:] = nan


# --------------------------------------------------------------------------
# brute force
# --------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_mixed(seed):
    rng = np.random.default_rng(100 + seed)
    B = 3
    q_lens = rng.integers(1, 6, size=B)
    seq_lens = q_lens + rng.integers(0, 30, size=B)
    bt = small_batch(seed, seq_lens, q_lens, Hq=6, Hkv=2, d=5, bs=4)
    ref = run_ref(bt)
    bf = bruteforce(bt)
    assert np.max(np.abs(ref - bf)) <= 1e-12


def test_bruteforce_bf16_mqa():
    bt = small_batch(7, [9, 17, 1], [1, 3, 1], Hq=4, Hkv=1, d=8, bs=4, dtype=wl.BF16)
    assert np.max(np.abs(run_ref(bt) - bruteforce(bt))) <= 1e-12


# --------------------------------------------------------------------------
# cross-attention (no causal mask) over a static encoder cache
# --------------------------------------------------------------------------

def cross_batch(seed, enc_lens, q_lens, **kw):
    return small_batch(seed, enc_lens, q_lens, cross=True, **kw)


@pytest.mark.parametrize("seed", [0, 1])
def test_cross_bruteforce(seed):
    # chunks longer than, equal to and shorter than the encoder sequence, a
    # single-row decode, an empty encoder and an empty chunk
    bt = cross_batch(40 + seed, [9, 5, 23, 0, 14], [12, 5, 3, 2, 0], Hq=6, Hkv=2, d=5, bs=4)
    ref = run_ref(bt, causal=False)
    assert np.max(np.abs(ref - bruteforce(bt, causal=False))) <= 1e-12
    q0, q1 = bt.query_start_loc[3], bt.query_start_loc[4]
    assert not ref[q0:q1].any()                    # empty encoder: zero rows


def test_cross_bruteforce_bf16_mqa():
    bt = cross_batch(42, [7, 17], [9, 1], Hq=4, Hkv=1, d=8, bs=4, dtype=wl.BF16)
    assert np.max(np.abs(run_ref(bt, causal=False) - bruteforce(bt, causal=False))) <= 1e-12


def test_cross_equals_unmasked_sdpa():
    """Library cross-check: torch SDPA in float64 without a mask, K/V expanded per query head."""
    bt = cross_batch(43, [21, 40, 3], [30, 1, 6], Hq=8, Hkv=2, d=16, bs=8, dtype=wl.BF16)
    G = bt.num_heads // bt.num_kv_heads
    Q = torch.from_numpy(f(bt.query))
    want = torch.zeros(bt.num_tokens, bt.num_heads, bt.head_dim, dtype=torch.float64)
    for b in range(bt.num_seqs):
        L = int(bt.seq_lens[b])
        q0, q1 = int(bt.query_start_loc[b]), int(bt.query_start_loc[b + 1])
        kv = [gather_sequence(bt.key_cache, bt.value_cache, bt.block_tables[b], L, h) for h in range(2)]
        K = torch.stack([torch.from_numpy(k) for k, _ in kv]).repeat_interleave(G, dim=0)
        V = torch.stack([torch.from_numpy(v) for _, v in kv]).repeat_interleave(G, dim=0)
        q = Q[q0:q1].transpose(0, 1).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=bt.scale)
        want[q0:q1] = o.transpose(0, 1)
    assert np.max(np.abs(run_ref(bt, causal=False) - want.numpy())) <= 1e-10


def test_cross_zero_scale_gives_mean_of_all_encoder_values():
    """Every row (not a causal prefix) averages all encoder positions."""
    bt = cross_batch(44, [11, 6], [4, 9], Hq=4, Hkv=2, d=4, bs=4)
    bt.scale = 0.0
    out = run_ref(bt, causal=False)
    Vc = f(bt.value_cache)
    for b in range(2):
        L = int(bt.seq_lens[b])
        q0, q1 = int(bt.query_start_loc[b]), int(bt.query_start_loc[b + 1])
        for h in range(4):
            vals = [Vc[bt.block_tables[b][t // 4], h // 2, :, t % 4] for t in range(L)]
            np.testing.assert_allclose(out[q0:q1, h], np.broadcast_to(np.mean(vals, axis=0), (q1 - q0, 4)),
                                       rtol=0, atol=1e-13)


def test_cross_rows_are_independent_of_position():
    """Reversing a chunk's query rows reverses its output rows; each row equals
    the decode of that row alone."""
    bt = cross_batch(45, [19], [7], Hq=4, Hkv=2, d=8, bs=4)
    out = run_ref(bt, causal=False)
    rev = cross_batch(45, [19], [7], Hq=4, Hkv=2, d=8, bs=4)
    rev.query = bt.query[::-1].copy()
    np.testing.assert_array_equal(run_ref(rev, causal=False), out[::-1])
    for j in range(7):
        one = decode_ref(bt.query[j:j + 1], bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens,
                         bt.num_kv_heads, bt.scale)
        np.testing.assert_allclose(out[j], one[0], rtol=0, atol=1e-13)
    # the causal reading differs on every row but the last
    causal = run_ref(bt)
    assert all(not np.allclose(out[j], causal[j]) for j in range(6))
    np.testing.assert_allclose(out[6], causal[6], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# head map: GQA == MHA on K/V expanded per query head
# --------------------------------------------------------------------------

def expand_caches(bt):
    """Repeat each kv head G times next to itself: [.., Hkv, ..] -> [.., Hkv*G, ..].

    This is the expand of the page's snippet (new group axis inserted after the
    kv-head axis) followed by a flatten of (kv, group) into one head axis.
    """
    G = bt.num_heads // bt.num_kv_heads
    kc = np.repeat(bt.key_cache, G, axis=1)
    vc = np.repeat(bt.value_cache, G, axis=1)
    return kc, vc


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 1), (6, 3), (4, 4)])
def test_gqa_equals_expanded_mha(Hq, Hkv):
    bt = small_batch(11, [13, 40, 7], [1, 5, 7], Hq=Hq, Hkv=Hkv, d=8, bs=4)
    gqa = run_ref(bt)
    kc, vc = expand_caches(bt)
    mha = paged_attention_ref(bt.query, kc, vc, bt.block_tables, bt.seq_lens, bt.query_start_loc, Hq, bt.scale)
    assert np.max(np.abs(gqa - mha)) <= 1e-12


def test_per_kv_head_constant_value_pins_head_map():
    Hq, Hkv = 8, 4
    bt = small_batch(12, [10, 23], [1, 4], Hq=Hq, Hkv=Hkv, d=4, bs=4)
    consts = np.array([1.0, 2.0, 3.0, 4.0], np.float32)
    for kv in range(Hkv):
        bt.value_cache[:, kv] = consts[kv]
    out = run_ref(bt)
    G = Hq // Hkv
    for h in range(Hq):
        # h // G, not h % Hkv: heads 0,1 -> 1.0; 2,3 -> 2.0; ...
        np.testing.assert_allclose(out[:, h, :], consts[h // G], rtol=0, atol=1e-14)
    assert not np.allclose(out[:, 1, :], consts[1 % Hkv])


# --------------------------------------------------------------------------
# paging: paged == contiguous (library cross-check) and permutation invariance
# --------------------------------------------------------------------------

def sdpa_reference(bt):
    """torch SDPA in float64 on the CPU, with K/V expanded per query head and an explicit mask."""
    G = bt.num_heads // bt.num_kv_heads
    out = torch.zeros(bt.num_tokens, bt.num_heads, bt.head_dim, dtype=torch.float64)
    Q = torch.from_numpy(f(bt.query))
    for b in range(bt.num_seqs):
        L = int(bt.seq_lens[b])
        q0, q1 = int(bt.query_start_loc[b]), int(bt.query_start_loc[b + 1])
        if q1 == q0:
            continue
        Ks, Vs = [], []
        for kv in range(bt.num_kv_heads):
            K, V = gather_sequence(bt.key_cache, bt.value_cache, bt.block_tables[b], L, kv)
            Ks.append(torch.from_numpy(K))
            Vs.append(torch.from_numpy(V))
        K = torch.stack(Ks).repeat_interleave(G, dim=0)          # [Hq, L, d]
        V = torch.stack(Vs).repeat_interleave(G, dim=0)
        q = Q[q0:q1].transpose(0, 1).contiguous()                  # [Hq, q_len, d]
        qlen = q1 - q0
        mask = torch.arange(L)[None, :] <= (L - qlen + torch.arange(qlen))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, attn_mask=mask, scale=bt.scale)
        out[q0:q1] = o.transpose(0, 1)
    return out.numpy()


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_paged_equals_contiguous_sdpa(dtype):
    rng = np.random.default_rng(5)
    q_lens = np.array([1, 1, 7, 16, 3])
    seq_lens = q_lens + rng.integers(0, 50, size=5)
    bt = small_batch(21, seq_lens, q_lens, Hq=8, Hkv=2, d=16, bs=8, dtype=dtype)
    assert np.max(np.abs(run_ref(bt) - sdpa_reference(bt))) <= 1e-10


def test_page_permutation_invariance():
    bt = small_batch(22, [37, 5, 64], [3, 1, 2], Hq=4, Hkv=2, d=8, bs=4)
    ref = run_ref(bt)
    perm = np.random.default_rng(0).permutation(bt.num_blocks)
    kc = np.empty_like(bt.key_cache)
    vc = np.empty_like(bt.value_cache)
    kc[perm] = bt.key_cache
    vc[perm] = bt.value_cache
    bt2 = small_batch(22, [37, 5, 64], [3, 1, 2], Hq=4, Hkv=2, d=8, bs=4)
    bt2.key_cache, bt2.value_cache = kc, vc
    bt2.block_tables = perm[bt.block_tables].astype(np.int32)
    assert np.array_equal(run_ref(bt2), ref)


def test_prefix_shared_pages_equal_duplicated_pages():
    """Block tables may alias physical pages (a shared prompt prefix): the result
    equals that of the same batch with the shared pages copied into private
    ones."""
    seq_lens, q_lens = [37, 29, 44], [3, 1, 2]
    bt = small_batch(24, seq_lens, q_lens, Hq=4, Hkv=2, d=8, bs=4)
    shared = 5                                     # first 5 pages (20 tokens) of sequence 0
    aliased = small_batch(24, seq_lens, q_lens, Hq=4, Hkv=2, d=8, bs=4)
    for b in (1, 2):
        aliased.block_tables[b, :shared] = aliased.block_tables[0, :shared]
    # duplicated: copy sequence 0's prefix pages into each sequence's own pages
    dup = small_batch(24, seq_lens, q_lens, Hq=4, Hkv=2, d=8, bs=4)
    for b in (1, 2):
        own = dup.block_tables[b, :shared]
        src = dup.block_tables[0, :shared]
        dup.key_cache[own] = dup.key_cache[src]
        dup.value_cache[own] = dup.value_cache[src]
    assert np.array_equal(run_ref(aliased), run_ref(dup))
    assert not np.array_equal(run_ref(aliased), run_ref(bt))      # the prefix really changed


def test_nan_poison_outside_sequences_is_ignored():
    seq_lens, q_lens = [13, 6, 32], [2, 1, 5]
    clean = small_batch(23, seq_lens, q_lens, bs=8)
    dirty = small_batch(23, seq_lens, q_lens, bs=8, poison_slack=True)
    poison_tails(dirty)
    a, b = run_ref(clean), run_ref(dirty)
    assert np.isfinite(b).all()
    assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# softmax closed forms
# --------------------------------------------------------------------------

def test_constant_value_gives_constant():
    bt = small_batch(31, [20, 9], [4, 1])
    bt.value_cache[:] = np.float32(2.5)
    assert np.allclose(run_ref(bt), 2.5, atol=1e-14, rtol=0)


def test_single_token_gives_its_value():
    bt = small_batch(32, [1, 1, 1], [1, 1, 1])
    out = run_ref(bt)
    for b in range(3):
        page = bt.block_tables[b][0]
        for h in range(bt.num_heads):
            np.testing.assert_array_equal(out[b, h], f(bt.value_cache)[page, h // 2, :, 0])


@pytest.mark.parametrize("zero", ["query", "scale"])
def test_uniform_weights_give_mean_of_visible_values(zero):
    bt = small_batch(33, [11, 30], [1, 6], Hq=4, Hkv=2, d=4, bs=4)
    if zero == "query":
        bt.query[:] = 0
    else:
        bt.scale = 0.0
    out = run_ref(bt)
    Vc = f(bt.value_cache)
    G = 2
    for b in range(2):
        L = int(bt.seq_lens[b])
        q0, q1 = int(bt.query_start_loc[b]), int(bt.query_start_loc[b + 1])
        for j in range(q1 - q0):
            n_vis = L - (q1 - q0) + j + 1            # bottom-right causal alignment
            for h in range(4):
                vals = [Vc[bt.block_tables[b][t // 4], h // G, :, t % 4] for t in range(n_vis)]
                np.testing.assert_allclose(out[q0 + j, h], np.mean(vals, axis=0), rtol=0, atol=1e-13)


def test_log_integer_keys_give_rational_weights():
    """Closed form: with q = e_c and k_t[c] = ln w_t, softmax weights are w_t / sum w."""
    Hq, Hkv, d, bs = 4, 2, 4, 2
    bt = small_batch(34, [5], [1], Hq=Hq, Hkv=Hkv, d=d, bs=bs)
    bt.scale = 1.0
    w = np.array([[[1, 2, 3, 4], [2, 1, 1, 5], [3, 3, 2, 1], [1, 4, 4, 2], [5, 1, 2, 3]],
                  [[2, 2, 1, 1], [1, 3, 2, 2], [4, 1, 5, 1], [1, 1, 1, 6], [3, 2, 1, 1]]])   # [kv, t, c]
    vals = np.arange(2 * 5 * d).reshape(2, 5, d) % 7 - 3                                    # [kv, t, c]
    for kv in range(Hkv):
        for t in range(5):
            page = bt.block_tables[0][t // bs]
            bt.key_cache[page, kv, t % bs, :] = np.log(w[kv, t]).astype(np.float32)
            bt.value_cache[page, kv, :, t % bs] = vals[kv, t]
    bt.query[:] = 0
    for h in range(Hq):
        bt.query[0, h, h] = 1.0                      # head h selects key component h
    out = run_ref(bt)
    for h in range(Hq):
        kv = h // (Hq // Hkv)
        num = [sum(Fraction(int(w[kv, t, h])) * int(vals[kv, t, c]) for t in range(5)) for c in range(d)]
        den = sum(Fraction(int(w[kv, t, h])) for t in range(5))
        expect = np.array([float(x / den) for x in num])
        # keys are float32-rounded logs, so weights match the rationals to ~1e-7
        np.testing.assert_allclose(out[0, h], expect, rtol=0, atol=2e-6)


def test_weights_sum_to_one_and_respect_mask():
    bt = small_batch(35, [12, 19], [4, 1])
    _, W = run_ref(bt, return_weights=True)
    for b, Wb in W.items():
        np.testing.assert_allclose(Wb.sum(-1), 1.0, rtol=0, atol=1e-14)
        q_len = int(bt.query_lens[b])
        L = int(bt.seq_lens[b])
        for j in range(q_len):
            assert np.all(Wb[j, :, L - q_len + j + 1:] == 0)
            assert np.all(Wb[j, :, :L - q_len + j + 1] > 0)


# --------------------------------------------------------------------------
# chunking / decode consistency
# --------------------------------------------------------------------------

def test_chunk_invariance():
    """One chunk of 12 tokens vs. three chunks of 4 (later chunks see the cache grow)."""
    L = 30
    full = small_batch(41, [L], [12])
    whole = run_ref(full)
    outs = []
    for c in range(3):
        qsl = np.array([0, 4], np.int32)
        q = full.query[c * 4:(c + 1) * 4]
        seq = np.array([L - 12 + 4 * (c + 1)], np.int32)
        outs.append(paged_attention_ref(q, full.key_cache, full.value_cache, full.block_tables, seq, qsl,
                                        full.num_kv_heads, full.scale))
    np.testing.assert_allclose(np.concatenate(outs), whole, rtol=0, atol=1e-13)


def test_single_token_chunk_equals_decode():
    bt = small_batch(42, [17, 3, 40], [1, 1, 1])
    a = run_ref(bt)
    b = decode_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, bt.num_kv_heads,
                   bt.scale)
    assert np.array_equal(a, b)


def test_decode_empty_sequence_is_zero():
    bt = small_batch(43, [0, 5], [0, 1])
    q = np.concatenate([np.zeros((1, 4, 8), np.float32), bt.query])
    out = decode_ref(q, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, 2, bt.scale)
    assert np.all(out[0] == 0)
    assert np.any(out[1] != 0)


# --------------------------------------------------------------------------
# split-K
# --------------------------------------------------------------------------

@pytest.mark.parametrize("P", [4, 8, 12, 64])
def test_split_merge_equals_unsplit(P):
    bt = small_batch(51, [1, 17, 33, 64, 0], [1, 1, 1, 1, 0], Hq=8, Hkv=2, d=8, bs=4)
    q = np.concatenate([bt.query[:4], np.zeros((1, 8, 8), np.float32)])
    full = decode_ref(q, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, 2, bt.scale)
    nparts = -(-64 // P)
    O, lse = decode_partials_ref(q, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, 2, bt.scale, P,
                                 nparts)
    merged = lse_merge_ref(O, lse)
    np.testing.assert_allclose(merged, full, rtol=0, atol=1e-13)
    assert np.all(merged[4] == 0)


def test_merge_closed_form_and_degenerate_cases():
    O = np.array([[[1.0, 2.0], [5.0, -1.0], [7.0, 7.0]]])              # [1, P=3, d=2]
    lse = np.array([[math.log(3.0), math.log(1.0), -np.inf]])
    np.testing.assert_allclose(lse_merge_ref(O, lse), [[(3 * 1 + 5) / 4, (3 * 2 - 1) / 4]], rtol=0, atol=1e-15)
    # a single non-empty partition comes back unchanged
    np.testing.assert_array_equal(lse_merge_ref(O[:, :1], lse[:, :1]), O[:, 0])
    # partition order does not matter
    np.testing.assert_allclose(lse_merge_ref(O[:, ::-1], lse[:, ::-1]), lse_merge_ref(O, lse), rtol=0, atol=1e-15)
    # all partitions empty -> zero, never NaN
    assert np.all(lse_merge_ref(O, np.full((1, 3), -np.inf)) == 0)


def test_partition_lse_is_log_partition_function():
    """lse_p equals log(sum exp(scale*q.k)) over the partition's keys (scale 0: log of its size)."""
    bt = small_batch(52, [10], [1], Hq=2, Hkv=1, d=4, bs=4)
    bt.scale = 0.0
    O, lse = decode_partials_ref(bt.query, bt.key_cache, bt.value_cache, bt.block_tables, bt.seq_lens, 1, 0.0, 4, 3)
    np.testing.assert_allclose(lse[0, 0], [math.log(4), math.log(4), math.log(2)], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# cache write
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_cache_write_round_trip(dtype):
    bt = small_batch(61, [9, 4, 23, 1], [3, 4, 1, 1], Hq=4, Hkv=2, d=8, bs=4, dtype=dtype)
    kc, vc = cache_write_ref(bt.new_key, bt.new_value, bt.key_cache, bt.value_cache, bt.block_tables,
                             bt.seq_lens, bt.query_start_loc)
    for b in range(bt.num_seqs):
        L = int(bt.seq_lens[b])
        q0, q1 = int(bt.query_start_loc[b]), int(bt.query_start_loc[b + 1])
        for kv in range(2):
            K, V = gather_sequence(kc, vc, bt.block_tables[b], L, kv)
            np.testing.assert_array_equal(K[L - (q1 - q0):], f(bt.new_key)[q0:q1, kv])
            np.testing.assert_array_equal(V[L - (q1 - q0):], f(bt.new_value)[q0:q1, kv])
            K0, V0 = gather_sequence(bt.key_cache, bt.value_cache, bt.block_tables[b], L, kv)
            np.testing.assert_array_equal(K[:L - (q1 - q0)], K0[:L - (q1 - q0)])
    # on a zero-filled cache, exactly the written elements become nonzero
    kz, vz = cache_write_ref(bt.new_key, bt.new_value, np.zeros_like(bt.key_cache), np.zeros_like(bt.value_cache),
                             bt.block_tables, bt.seq_lens, bt.query_start_loc)
    changed = (kz != 0).sum() + (vz != 0).sum()
    assert changed == 2 * bt.num_tokens * bt.num_kv_heads * bt.head_dim


# --------------------------------------------------------------------------
# generator sanity
# --------------------------------------------------------------------------

def test_generator_is_deterministic_and_tables_are_permutations():
    a, b = wl.tiny_decode(1), wl.tiny_decode(1)
    np.testing.assert_array_equal(a.key_cache, b.key_cache)
    np.testing.assert_array_equal(a.block_tables, b.block_tables)
    owned = np.concatenate([a.block_tables[i][:-(-int(a.seq_lens[i]) // 16)] for i in range(a.num_seqs)])
    assert len(set(owned.tolist())) == len(owned)
    assert set(owned.tolist()) | set(a.slack_pages.tolist()) == set(range(a.num_blocks))


def test_mixed_generator_shape():
    rng = np.random.default_rng(4)
    seq_lens, q = wl.mixed_lengths(rng)
    assert len(q) == 256 and (q == 1).sum() == 205
    assert q.sum() <= 8192 and q[q > 1].min() >= 2 and q.max() <= 2048
    assert (seq_lens >= q).all()


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.0 - 2 ** -7 - 2 ** -9, 3.0e38], np.float32)
    bits = wl.f32_to_bf16_bits(x)
    back = wl.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back[:3], [1.0, 1.0, 1.0 + 2 ** -6])
    assert back[3] == -2.0 - 2 ** -6
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
