/*
 * gqa_paged.h - GQA/MQA-aware attention over a paged KV cache, MI355X (gfx950).
 *
 * C ABI of libgqa_paged.so.  Every pointer argument named *_cache, query, key,
 * value, out, block_tables, seq_lens, query_start_loc, partial_* and workspace
 * is a DEVICE pointer owned by the caller; `stream` is a hipStream_t cast to
 * void* (NULL = the null stream).  Calls only enqueue work on `stream` and
 * return without synchronising; the library allocates nothing, frees nothing
 * and keeps no state between calls (it is re-entrant; two calls that share a
 * workspace must not overlap).
 *
 * The operation follows three pages:
 *  - "[Performance] Use optimized kernels for MQA/GQA" (vLLM issue #1880),
 *    opening post: several query heads share one kv head, and attention should
 *    read the KV cache once per kv head instead of expanding K/V per query head
 *    (item 1, the expand of keys/values with a group axis after the kv-head
 *    axis); the decode reads a paged KV cache (item 2).
 *  - "[Kernel] [V1] Further optimizations to ROCm (Triton) Backend to better
 *    handle GQA" (vLLM PR #14431), TLDR and review thread: one op,
 *    chunked_prefill_paged_decode, serves a batch that mixes prefill chunks and
 *    single-token decodes over the same paged cache; the prefill part skips the
 *    decodes and a second kernel handles them.
 *
 * Semantics, for sequence b, query head h, G = num_heads / num_kv_heads:
 *   kv   = h / G                              (heads of a group are contiguous)
 *   q_len = query_start_loc[b+1] - query_start_loc[b]   (decode: 1)
 *   new token j (row query_start_loc[b] + j) sits at position seq_lens[b]-q_len+j
 *   and sees keys t <= seq_lens[b] - q_len + j   (causal, bottom-right aligned)
 *   K_b[t] = key_cache  [block_tables[b][t / bs]][kv][t % bs][:]
 *   V_b[t] = value_cache[block_tables[b][t / bs]][kv][:][t % bs]
 *   out[row][h] = sum_t softmax_t(scale * q.K_b[t]) * V_b[t]
 *
 * Layouts (all contiguous, row-major):
 *   query, out      [num_tokens, num_heads, head_dim]
 *   key, value      [num_tokens, num_kv_heads, head_dim]    (this step's new tokens)
 *   key_cache       [num_blocks, num_kv_heads, block_size, head_dim]
 *   value_cache     [num_blocks, num_kv_heads, head_dim, block_size]
 *   block_tables    [num_seqs, max_blocks_per_seq] int32
 *   seq_lens        [num_seqs] int32, tokens in the cache INCLUDING this step's
 *   query_start_loc [num_seqs + 1] int32, prefix sums of query lengths, [0] = 0
 *
 * The value page is stored head_dim-major (tokens of a page contiguous per
 * channel) so that the P.V matrix-core operand is a plain 16-byte load; the key
 * page is token-major for the same reason on the Q.K^T side.  Pages of 16, 32
 * or 64 tokens are supported by every call; the kernels' key tiles do not
 * depend on the page size ("[Performance] Use optimized kernels for MQA/GQA",
 * thread: a paged kernel that required the page size to equal its key tile),
 * and the same tokens give the same results in any of them.
 *
 * Device-data preconditions (not checked on the host; the kernels clamp so that
 * a violation gives a wrong result, never an out-of-bounds access):
 *   0 <= seq_lens[b] <= max_seq_len <= max_blocks_per_seq * block_size,
 *   0 <= block_tables[b][i] < num_blocks for i < ceil(seq_lens[b] / block_size),
 *   query_start_loc non-decreasing, query_start_loc[num_seqs] == num_tokens,
 *   q_len <= seq_lens[b].
 *
 * Errors: every call returns a gqa_status.  Host-side validation looks at the
 * scalar arguments only; no exception crosses the ABI.
 */
#ifndef GQA_PAGED_H_
#define GQA_PAGED_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, num_heads % num_kv_heads != 0, ... */
  GQA_ERR_UNSUPPORTED = 2,   /* head_dim, block_size, group size or dtype combination not built */
  GQA_ERR_WORKSPACE = 3,     /* workspace pointer null or smaller than *_workspace_size() */
  GQA_ERR_LAUNCH = 4,        /* the HIP runtime reported an error at launch (or no device) */
  GQA_ERR_SCRATCH = 5        /* paged_gqa_decode_noalloc: the call needs more than GQA_NOALLOC_SCRATCH_BYTES */
} gqa_status;

typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;

typedef struct {
  int32_t num_seqs;            /* B */
  int32_t num_heads;           /* Hq */
  int32_t num_kv_heads;        /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;            /* d: 64 or 128 */
  int32_t block_size;          /* tokens per page: 16, 32 or 64 */
  int32_t num_blocks;          /* pages in each cache */
  int32_t max_blocks_per_seq;  /* row stride of block_tables */
  int32_t q_dtype;             /* a gqa_dtype: query (and key/value of reshape_and_cache) */
  int32_t kv_dtype;            /* a gqa_dtype: caches; must equal q_dtype */
  int32_t out_dtype;           /* a gqa_dtype: output; accumulation is always fp32 */
} gqa_dims;

/* Human-readable name of a status code (static storage). */
const char* gqa_status_string(int32_t status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t gqa_version(void);

/*
 * gqa_probe_mfma_bf16: a measurement probe, not part of the attention path.
 * Enqueues `groups` work-groups of 4 waves, each wave issuing `iters` rounds
 * of 8 independent v_mfma_f32_16x16x32_bf16 products, and writes one float per
 * wave to out[groups * 4] (device).  *flops (host) receives the launch's
 * multiply-add flops (2 per multiply-add), so that flops / elapsed time is the
 * bf16 matrix rate this device sustains.  GQA_ERR_INVALID_ARG for a null
 * pointer or non-positive sizes.
 */
int32_t gqa_probe_mfma_bf16(float* out, int32_t groups, int32_t iters, long long* flops, void* stream);

/*
 * reshape_and_cache: copy this step's keys and values into the paged caches.
 * New token j of sequence b (row query_start_loc[b] + j of key/value) goes to
 * position pos = seq_lens[b] - q_len + j, i.e. page block_tables[b][pos / bs],
 * slot pos % bs.  A bit-exact copy in the cache dtype (kv_dtype; key/value are
 * in kv_dtype too).  Slots not written are left untouched.  num_tokens may be 0
 * (no launch).  When the batch has more new tokens than sequences (prefill
 * chunks), each 16-position run of a value page's channel row is rewritten
 * whole around the new tokens (its other slots with the values they hold), so
 * a page that receives one sequence's new tokens must not receive another
 * sequence's in the same call (a paged allocator never does that).
 * ("[Performance] Use optimized kernels for MQA/GQA", opening post: incoming
 * keys/values are [tokens, num_kv_heads, head]; item 2: the decode reads them
 * back from a paged cache.)
 */
int32_t reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          const int32_t* query_start_loc, int32_t num_tokens, gqa_dims dims,
                          void* stream);

/*
 * paged_gqa_decode: one query token per sequence (query/out are [num_seqs,
 * num_heads, head_dim]) attending to all seq_lens[b] cached tokens.  Each
 * (sequence, kv head) pair reads its K/V pages once for all G query heads of
 * the group ("[Performance] Use optimized kernels for MQA/GQA", opening post,
 * item 2).
 *
 * partition_size == 0 (recommended): the library picks the split.  When the
 * batch has fewer (sequence, kv head) units than twice the device's resident
 * work-groups and G <= 16, it uses a balanced split: the (sequence, kv head,
 * 32-token tile) work items of the whole batch are divided into equal
 * contiguous ranges, one per resident wave, so every wave streams the same
 * number of K/V bytes whatever the mix of context lengths; a (sequence, kv
 * head) whose keys fall in one range is finished by that wave, one cut by
 * range boundaries is merged by log-sum-exp in a second, small kernel, in a
 * fixed order (results are reproducible on a given device).  Otherwise (many
 * units, G > 16, num_seqs > 7935, or more than 2^31 tiles) each (sequence,
 * kv head) is one work-group's job, with no split.
 *
 * partition_size > 0: fixed split-K.  Each sequence of L tokens is split into
 * ceil(L / partition_size) partitions of nearly equal length (whole 32-token
 * tiles; partition_size must be a multiple of 32), each processed by one
 * work-group; partials are merged by log-sum-exp in partition order by a
 * second kernel.  partition_size >= max_seq_len means no split.
 *
 * The result does not depend on the split beyond fp32 rounding.  max_seq_len
 * (host) bounds seq_lens and sizes the grid without a device sync.
 * seq_lens[b] == 0 gives a zero output row.
 *
 * Workspace (device, >= paged_gqa_decode_workspace_size bytes, 256-byte
 * aligned; may be NULL when that size is 0): scratch for the split partials;
 * its contents need no initialisation and are meaningless between calls.  For
 * the balanced split the size depends on the current device's compute-unit
 * count and occupancy; a smaller (but non-zero) workspace is accepted and uses
 * fewer waves.
 */
size_t paged_gqa_decode_workspace_size(gqa_dims dims, int32_t max_seq_len, int32_t partition_size);
int32_t paged_gqa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, int32_t max_seq_len,
                         gqa_dims dims, float scale, int32_t partition_size, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * paged_gqa_decode_noalloc: paged_gqa_decode without a workspace argument, for
 * callers that cannot allocate device memory around the call (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  The
 * split partials and metadata live in a static device array of
 * GQA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; the call allocates nothing and calls no allocating
 * routine.  Same arguments, kernels and results as paged_gqa_decode with a
 * workspace of that size.
 *
 * Returns GQA_ERR_SCRATCH, before any launch, when
 * paged_gqa_decode_workspace_size(dims, max_seq_len, partition_size) exceeds
 * GQA_NOALLOC_SCRATCH_BYTES.  The array's device address is looked up once per
 * device, at the first call on that device (GQA_ERR_LAUNCH if that fails).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or host threads) race on it and must be serialised by
 * the caller.  No kernel needs the array cleared: each call writes what it
 * reads.
 */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int32_t paged_gqa_decode_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, const int32_t* seq_lens, int32_t max_seq_len,
                                 gqa_dims dims, float scale, int32_t partition_size, void* stream);

/*
 * paged_gqa_decode_append: one decode step with the cache write fused in.
 * key/value [num_seqs, num_kv_heads, head_dim] (kv_dtype, device) hold each
 * sequence's new token, at position seq_lens[b] - 1 (seq_lens counts it).
 * The call writes it into the caches exactly as reshape_and_cache with
 * query_start_loc = [0, 1, ..., num_seqs] does, and returns the attention of
 * paged_gqa_decode over all seq_lens[b] tokens, the new one included ("[Performance]
 * Use optimized kernels for MQA/GQA", opening post, item 2: the step's keys and
 * values go into the paged cache that the decode then reads).
 *
 * Same dims, dtypes, page sizes, partition_size meaning and workspace
 * (paged_gqa_decode_workspace_size) as paged_gqa_decode.  With the balanced
 * split it is the same two launches as paged_gqa_decode and no more: the
 * decode kernel reads keys [0, seq_lens[b] - 1) from the pages, and the merge
 * kernel adds the new token's term from key/value and stores key/value into
 * the pages.  The other decompositions run the cache write, then the decode.
 * Precondition of the balanced path (as in any paged allocator): the page
 * that receives a sequence's new token holds no other sequence's new token.
 * The caches end bit-identical to reshape_and_cache's; the output agrees with
 * reshape_and_cache followed by paged_gqa_decode up to fp32 rounding.  seq_lens[b] == 0: nothing is written
 * and the output row is zero.  Errors as paged_gqa_decode, plus
 * GQA_ERR_INVALID_ARG for a null key or value.
 */
int32_t paged_gqa_decode_append(void* out, const void* query, const void* key, const void* value,
                                void* key_cache, void* value_cache, const int32_t* block_tables,
                                const int32_t* seq_lens, int32_t max_seq_len, gqa_dims dims, float scale,
                                int32_t partition_size, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * splitk_lse_reduce: merge per-partition decode results.
 *   partial_out [num_seqs, num_heads, max_partitions, head_dim] fp32: the
 *                partition's normalised output;
 *   partial_lse [num_seqs, num_heads, max_partitions] fp32: natural-log
 *                log-sum-exp of the partition's scaled scores (-inf if empty).
 * Sequence b has n_b = ceil(seq_lens[b] / partition_size) partitions (clamped
 * to max_partitions); out[row][h] = sum_{p<n_b} exp(lse_p - LSE) * O_p with
 * LSE = log sum_p exp(lse_p); zero if every partition is empty.
 * row = b, or query_start_loc[b] when query_start_loc is non-NULL, in which
 * case only sequences with exactly one query token are written.
 * Sequences with n_b <= 1 are skipped when skip_single != 0, merged
 * otherwise.  (paged_gqa_decode merges its own partials in-kernel; this entry
 * point serves partials produced elsewhere, e.g. one per device of a
 * sequence-sharded decode.)
 */
int32_t splitk_lse_reduce(void* out, const float* partial_out, const float* partial_lse,
                          const int32_t* seq_lens, const int32_t* query_start_loc, gqa_dims dims,
                          int32_t max_partitions, int32_t partition_size, int32_t skip_single,
                          void* stream);

/*
 * chunked_prefill_paged_decode: attention for a mixed batch of prefill chunks
 * (q_len > 1, causal within the chunk, bottom-right aligned against the cached
 * prefix) and decodes (q_len == 1), all over the same paged cache ("[Kernel]
 * [V1] Further optimizations to ROCm (Triton) Backend to better handle GQA",
 * review thread: the prefill kernel skips single-token sequences, which a
 * decode kernel handles alongside it).  query/out are [num_tokens, num_heads,
 * head_dim]; max_query_len and max_seq_len are host-side bounds (sequences
 * whose q_len exceeds max_query_len are not computed).  Sequences with
 * q_len 0 produce no rows.
 *
 * bf16: a one-work-group scheduling pass lists the work units (prefill row
 * tiles of 128 (token, head) rows and decode partitions) in decreasing order
 * of cost, and one fused kernel runs them, so decodes proceed alongside the
 * prefill tiles; a merge kernel follows when decodes are split.  Decodes are
 * split into partitions of partition_size tokens (merged by log-sum-exp in
 * partition order); partition_size == 0 lets the library pick (partitions of
 * 4096 tokens, i.e. no split unless max_seq_len > 4096).  Prefill rows compute
 * P.V on fp16 matrix cores (P rounded to fp16, V converted from bf16 to
 * fp16 rounding to nearest): preconditions |V| < 65504 (larger values
 * overflow) and V not so small that fp16's subnormal spacing 2^-24 matters
 * (for V ~ N(0, s^2) the parity bar holds down to s of about 1e-5).
 * fp32: a prefill kernel, then the decode of paged_gqa_decode (same meaning of
 * partition_size).  Either dtype: a batch whose max_query_len is 1 (decodes
 * only) runs the decode of paged_gqa_decode alone.  bf16 batches with 2^20 or more work units (num_tokens * G /
 * 128 + num_seqs * (1 + decode partitions)) return GQA_ERR_UNSUPPORTED.
 *
 * Workspace (device, >= chunked_prefill_paged_decode_workspace_size bytes for
 * the same dims, num_tokens, max_seq_len and partition_size; 256-byte
 * aligned; no initialisation needed): the unit list and split partials.
 */
size_t chunked_prefill_paged_decode_workspace_size(gqa_dims dims, int32_t num_tokens, int32_t max_seq_len,
                                                   int32_t partition_size);
int32_t chunked_prefill_paged_decode(void* out, const void* query, const void* key_cache,
                                     const void* value_cache, const int32_t* block_tables,
                                     const int32_t* seq_lens, const int32_t* query_start_loc,
                                     int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                                     gqa_dims dims, float scale, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_cross_attention: attention of decoder rows over a static encoder
 * cache ("[Core] More-efficient cross-attention parallel QKV computation",
 * opening post: the queries come from the decoder, the keys and values from
 * the encoder output, and after the prefill only queries are new, so the
 * encoder cache is written once and never appended to).  Same arguments,
 * layouts, workspace and precision as chunked_prefill_paged_decode, with
 * encoder_lens in place of seq_lens and no causal mask: every query row of
 * sequence b sees all encoder_lens[b] positions.  A sequence may have more
 * query rows than encoder positions (max_query_len may exceed
 * max_encoder_len); an empty encoder sequence gives zero rows.  A batch
 * whose max_query_len is 1 runs the decode of paged_gqa_decode.
 *
 * Workspace: >= paged_cross_attention_workspace_size bytes for the same dims,
 * num_tokens, max_encoder_len and partition_size.
 */
size_t paged_cross_attention_workspace_size(gqa_dims dims, int32_t num_tokens, int32_t max_encoder_len,
                                            int32_t partition_size);
int32_t paged_cross_attention(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, const int32_t* encoder_lens,
                              const int32_t* query_start_loc, int32_t num_tokens, int32_t max_query_len,
                              int32_t max_encoder_len, gqa_dims dims, float scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_gqa_decode_shared_prefix: the decode of paged_gqa_decode for a batch
 * whose sequences share prompt prefixes, reading each shared page once per
 * group instead of once per sequence.  With automatic prefix caching the
 * block tables of such sequences point at the same physical pages ("[Kernel]
 * [V1] Further optimizations to ROCm (Triton) Backend to better handle GQA",
 * benchmark discussion: prefix caching changes the measured results).
 *
 * Groups are ranges of consecutive sequences: group g is sequences
 * [group_start[g], group_start[g + 1]) (group_start non-decreasing, within
 * [0, num_seqs]); its members hold the same first prefix_lens[g] tokens, read
 * through the block table of the group's first member.  Sequences in no group
 * are decoded on their own.  The result is that of paged_gqa_decode on the
 * same arguments (each sequence attends to its own seq_lens[b] tokens).
 * Preconditions (device data, unchecked; a violation gives wrong rows, never
 * an out-of-bounds access): prefix_lens[g] <= seq_lens of every member, group
 * sizes <= max_group_size, seq_lens <= max_seq_len.
 *
 * bf16: the shared part of a group (its prefix rounded down to 64 keys) is
 * attended by all members together: their query rows (member x head) form
 * matrix-core tiles against each shared K/V tile, in chunks of 512 to 2048
 * keys.  Each member's remaining keys run the decode in partitions of
 * partition_size tokens (0: the library picks, at least 256).  The partials
 * of both are merged by log-sum-exp.  The prefix tiles compute P.V on fp16
 * matrix cores as chunked_prefill_paged_decode does (same preconditions on
 * the magnitude of V).  fp32: runs paged_gqa_decode (no sharing), with the same
 * meaning of partition_size.
 *
 * Workspace (device, >= paged_gqa_decode_shared_prefix_workspace_size bytes
 * for the same dims, num_groups, max_group_size, max_seq_len and
 * partition_size; no initialisation needed): the partials and their counts.
 */
size_t paged_gqa_decode_shared_prefix_workspace_size(gqa_dims dims, int32_t num_groups, int32_t max_group_size,
                                                    int32_t max_seq_len, int32_t partition_size);
int32_t paged_gqa_decode_shared_prefix(void* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       const int32_t* seq_lens, const int32_t* group_start,
                                       const int32_t* prefix_lens, int32_t num_groups, int32_t max_group_size,
                                       int32_t max_seq_len, gqa_dims dims, float scale, int32_t partition_size,
                                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif  /* GQA_PAGED_H_ */
