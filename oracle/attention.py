"""CPU fp64 oracle for GQA/MQA attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module; the library never calls it, and it shares
no code with the HIP path (it imports numpy only).

What it computes, written as the plain definition (slow, vectorised per
(sequence, kv head) with numpy, everything in float64):

* Query head ``h`` reads kv head ``h // G`` with ``G = num_heads // num_kv_heads``.
  "[Performance] Use optimized kernels for MQA/GQA" (vLLM issue #1880), opening
  post, item 1: keys and values of shape ``[T, num_kv_heads, head]`` are expanded
  with a new group axis *after* the kv-head axis, so after flattening, the query
  heads of one group are contiguous and share one kv head.
* Keys and values live in fixed-size pages addressed through a per-sequence
  block table (same post, item 2: a paged KV cache read by the decode kernel).
  Token ``t`` of sequence ``b`` sits in page ``block_tables[b][t // bs]`` at
  slot ``t % bs``.  Layouts: key ``[num_blocks, Hkv, bs, d]``, value
  ``[num_blocks, Hkv, d, bs]``.
* ``out = softmax(scale * q K^T) V`` over the visible keys.
* Mixed batches ("[Kernel] [V1] Further optimizations to ROCm (Triton) Backend
  to better handle GQA", vLLM PR #14431, the review thread on
  ``chunked_prefill_paged_decode``): sequences with one query token are decodes,
  longer ones are prefill chunks.  Readings where the pages are silent: a chunk
  of ``q_len`` new tokens is the *last* ``q_len`` tokens of the sequence (the
  cache already holds them), and new token ``j`` sees key positions
  ``t <= seq_len - q_len + j`` (causal, bottom-right aligned).
* Cross-attention over a static encoder cache ("[Core] More-efficient
  cross-attention parallel QKV computation", vLLM PR #7448, opening post: the
  decoder supplies the queries, the encoder output supplies keys and values,
  and after prefill only queries are new).  Reading where the page is silent:
  no causal mask, so every query row of sequence ``b`` sees all
  ``seq_lens[b]`` encoder positions, a chunk may be longer than the encoder
  sequence, and an empty encoder sequence gives zero rows (``causal=False``).
* Split-K: partition ``p`` of a decode covers keys ``[p*P, min((p+1)*P, L))`` and
  yields the normalised partial output and its natural-log log-sum-exp; merging
  partials weighted by ``exp(lse_p - logsumexp(lse))`` gives the unsplit result.

Parity of every function here is pinned by CPU tests (brute force, the GQA ==
expanded-MHA equivalence, closed forms, library cross-checks); see tests/.
"""
from __future__ import annotations

import numpy as np


def _to_f64(arr: np.ndarray) -> np.ndarray:
    """Storage (float array, or uint16 bfloat16 bit patterns) -> float64, exactly."""
    arr = np.asarray(arr)
    if arr.dtype == np.uint16:
        return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return arr.astype(np.float64)


def gather_sequence(key_cache, value_cache, block_table_row, n_tokens: int, kv_head: int):
    """Read tokens ``0..n_tokens-1`` of one sequence and one kv head through its block table.

    Returns ``(K, V)`` as float64 ``[n_tokens, d]`` arrays.
    """
    bs = key_cache.shape[2]
    n_pages = -(-n_tokens // bs)
    pages = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    k = _to_f64(key_cache[pages, kv_head])                    # [n_pages, bs, d]
    v = _to_f64(value_cache[pages, kv_head])                  # [n_pages, d, bs]
    d = k.shape[-1]
    K = k.reshape(n_pages * bs, d)[:n_tokens]
    V = np.transpose(v, (0, 2, 1)).reshape(n_pages * bs, d)[:n_tokens]
    return K, V


def _softmax_rows(S: np.ndarray) -> np.ndarray:
    """Row softmax in float64; rows that are all -inf give all-zero weights."""
    m = S.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S - m)
    den = E.sum(axis=-1, keepdims=True)
    return np.where(den > 0, E / np.where(den > 0, den, 1.0), 0.0)


def paged_attention_ref(query, key_cache, value_cache, block_tables, seq_lens, query_start_loc,
                        num_kv_heads: int, scale: float, seqs=None, return_weights: bool = False,
                        causal: bool = True):
    """Attention of a mixed batch (prefill chunks and decodes) over the paged cache.

    ``query``: ``[T, Hq, d]``.  Returns ``out [T, Hq, d]`` float64 (rows of
    sequences not listed in ``seqs`` stay zero).  With ``return_weights`` also
    returns ``{b: W}``, the softmax weights of sequence ``b`` shaped
    ``[q_len, Hq, seq_len]``.  ``causal=False`` is cross-attention: every row
    sees all ``seq_len`` keys.
    """
    Q = _to_f64(query)
    T, Hq, d = Q.shape
    if Hq % num_kv_heads:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    G = Hq // num_kv_heads
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    out = np.zeros((T, Hq, d), dtype=np.float64)
    weights = {}
    seqs = range(len(seq_lens)) if seqs is None else seqs
    for b in seqs:
        L = int(seq_lens[b])
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        q_len = q1 - q0
        if q_len == 0:
            continue
        if causal:
            if q_len > L:
                raise ValueError(f"sequence {b}: query length {q_len} exceeds seq_len {L}")
            # key t is visible to new token j iff t <= (L - q_len) + j
            visible = np.arange(L)[None, :] <= (L - q_len + np.arange(q_len))[:, None]   # [q_len, L]
        else:
            visible = np.ones((q_len, L), dtype=bool)
        if return_weights:
            W_b = np.zeros((q_len, Hq, L))
        if L == 0:
            # no visible key: the rows stay zero
            if return_weights:
                weights[b] = W_b
            continue
        for kv in range(num_kv_heads):
            K, V = gather_sequence(key_cache, value_cache, block_tables[b], L, kv)
            Qg = Q[q0:q1, kv * G:(kv + 1) * G, :]                                     # [q_len, G, d]
            S = scale * np.matmul(Qg, K.T)                                            # [q_len, G, L]
            S = np.where(visible[:, None, :], S, -np.inf)
            W = _softmax_rows(S)
            out[q0:q1, kv * G:(kv + 1) * G, :] = np.matmul(W, V)
            if return_weights:
                W_b[:, kv * G:(kv + 1) * G, :] = W
        if return_weights:
            weights[b] = W_b
    if return_weights:
        return out, weights
    return out


def decode_ref(query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads: int, scale: float,
               seqs=None):
    """Decode: one query token per sequence (``query [B, Hq, d]``) attending to all
    ``seq_lens[b]`` cached tokens.  ``seq_len == 0`` gives a zero row."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    Q = _to_f64(query)
    out = np.zeros(Q.shape, dtype=np.float64)
    live = [b for b in (range(B) if seqs is None else seqs) if seq_lens[b] > 0]
    if not live:
        return out
    qsl = np.arange(B + 1, dtype=np.int64)
    # a decode is a chunk of length one whose token is the sequence's last
    res = paged_attention_ref(Q, key_cache, value_cache, block_tables, seq_lens, qsl, num_kv_heads, scale,
                              seqs=live)
    out[live] = res[live]
    return out


def decode_partials_ref(query, key_cache, value_cache, block_tables, seq_lens, num_kv_heads: int,
                        scale: float, partition_size: int, num_partitions: int):
    """Split-K partials of a decode.

    Partition ``p`` covers keys ``[p*P, min((p+1)*P, L))``.  Returns
    ``(O [B, Hq, num_partitions, d], lse [B, Hq, num_partitions])`` with ``O`` the
    partition's normalised output and ``lse`` the natural log of its softmax
    denominator (including the max shift).  Empty partitions give ``O = 0`` and
    ``lse = -inf``.
    """
    Q = _to_f64(query)
    B, Hq, d = Q.shape
    G = Hq // num_kv_heads
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    O = np.zeros((B, Hq, num_partitions, d))
    lse = np.full((B, Hq, num_partitions), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        for kv in range(num_kv_heads):
            K, V = gather_sequence(key_cache, value_cache, block_tables[b], L, kv)
            Qg = Q[b, kv * G:(kv + 1) * G, :]                                           # [G, d]
            for p in range(num_partitions):
                lo, hi = p * partition_size, min((p + 1) * partition_size, L)
                if hi <= lo:
                    continue
                S = scale * (Qg @ K[lo:hi].T)                                           # [G, n]
                m = S.max(axis=-1, keepdims=True)
                E = np.exp(S - m)
                den = E.sum(axis=-1, keepdims=True)
                O[b, kv * G:(kv + 1) * G, p, :] = (E / den) @ V[lo:hi]
                lse[b, kv * G:(kv + 1) * G, p] = (m + np.log(den))[:, 0]
    return O, lse


def lse_merge_ref(partial_out, partial_lse):
    """Merge split-K partials: ``out = sum_p exp(lse_p - LSE) * O_p`` with
    ``LSE = log sum_p exp(lse_p)``.  Inputs ``[..., P, d]`` and ``[..., P]``;
    rows whose partials are all empty (``lse = -inf``) give zero."""
    O = np.asarray(partial_out, dtype=np.float64)
    lse = np.asarray(partial_lse, dtype=np.float64)
    m = lse.max(axis=-1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse - m_safe)                      # exp(-inf) = 0 for empty partitions
    den = w.sum(axis=-1, keepdims=True)
    w = np.where(den > 0, w / np.where(den > 0, den, 1.0), 0.0)
    return np.einsum("...p,...pd->...d", w, O)


def cache_write_ref(new_key, new_value, key_cache, value_cache, block_tables, seq_lens, query_start_loc):
    """Write this step's keys/values into the paged caches; returns new cache arrays.

    New token ``j`` of sequence ``b`` (row ``query_start_loc[b] + j`` of
    ``new_key [T, Hkv, d]``) is at position ``seq_lens[b] - q_len + j``, i.e. page
    ``block_tables[b][pos // bs]``, slot ``pos % bs``.  The copy is bit-exact
    (it moves storage, whatever its dtype).
    """
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    bs = kc.shape[2]
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    for b in range(len(seq_lens)):
        q0, q1 = int(qsl[b]), int(qsl[b + 1])
        first = int(seq_lens[b]) - (q1 - q0)
        for j in range(q1 - q0):
            pos = first + j
            page = int(block_tables[b][pos // bs])
            slot = pos % bs
            kc[page, :, slot, :] = new_key[q0 + j]
            vc[page, :, :, slot] = new_value[q0 + j]
    return kc, vc
