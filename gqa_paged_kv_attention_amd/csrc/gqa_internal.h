// Host-side launch interface between the C ABI (abi.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Launch kernel k with its arguments (passed by value) and return the status
// of this launch alone.  hipLaunchKernel reports its own result, so an error
// left pending by the caller's earlier HIP calls is neither read as this
// launch's nor cleared.
template <class... P, class... A>
inline hipError_t launch_kernel(void (*k)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, const A&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "one value per kernel parameter");
  void* args[] = {const_cast<void*>(static_cast<const void*>(&a))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(k), grid, block, args, lds, s);
}

// Fixed-partition decode (one work-group per (partition, kv head, sequence)).
struct DecodeArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;   // nullptr: query row = sequence index
  float* partial_out;               // [B, Hq, max_partitions, D]
  float* partial_lse;               // [B, Hq, max_partitions]
  int num_heads;
  int num_kv_heads;
  int group;                        // num_heads / num_kv_heads
  int num_blocks;
  int max_blocks_per_seq;
  int num_tokens;
  int partition_size;               // tokens per partition, multiple of 32
  int max_partitions;
  float scale_log2;                 // scale * log2(e)
  // 1, or 2 when each kv head's query heads run as two units of `group` rows:
  // num_kv_heads and the kv index then count those units, and the cache's kv
  // head is kv / kv_split of num_kv_heads / kv_split.
  int kv_split = 1;
  // waves per work-group of the one-work-group-per-partition decode (G <= 16):
  // 4, or 8 when the grid holds at most one work-group per compute unit, so
  // that each wave walks half as many tiles one after another
  int waves = 4;
};

// Balanced ("stream") decode: persistent waves, each owning an equal slice of
// the list of (sequence, kv head, 32-token tile) work items.
constexpr int kMaxStreamSeqs = 7935;    // prefix and length tables fit 62 KiB of LDS
constexpr int kStreamWorkersPerGroup = 4;
struct StreamArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;   // nullptr: pure decode
  const void* new_key;              // [B, Hkv, D] or nullptr: the step's new token of each sequence,
  const void* new_value;            // written into the pages and attended from here (fused append)
  int* tile_prefix;                 // [B + 1]: prefix of tiles * Hkv (work-group 0 writes it)
  int4* unit_meta;                  // [B * Hkv]: {first worker, last worker, first slot, out row}
  float* seg_out;                   // [num_workers, 2, G, D]: cut segments, normalised
  float* seg_lse;                   // [num_workers, 2, G]
  float* unit_out;                  // [B, Hq, D]: fused append, a whole unit's normalised output
  float* unit_lse;                  // [B, Hq]: and its natural-log log-sum-exp
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;
  int num_blocks;
  int max_blocks_per_seq;
  int num_tokens;
  int num_workers;                  // 4 per work-group
  int block_size;                   // tokens per page
  float scale_log2;
};

// Balanced decode in fixed partitions: persistent waves walk contiguous runs
// of whole partitions (balanced by tiles) and write one partial per partition
// into d.partial_out / d.partial_lse ([B, Hq, max_partitions, D] and
// [B, Hq, max_partitions]); a sequence of one partition writes d.out.
struct StreamPartArgs {
  DecodeArgs d;
  int num_seqs;
  int num_workers;                  // 4 per work-group
};

struct PrefillArgs {
  void* out;
  const void* query;
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int group;
  int num_blocks;
  int max_blocks_per_seq;
  int num_tokens;
  float scale_log2;
  int causal;                       // 1: bottom-right causal; 0: every row sees all seq_len keys
};

struct ReduceArgs {
  void* out;
  const float* partial_out;
  const float* partial_lse;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;
  int num_heads;
  int num_kv_heads;
  int group;
  int max_blocks_per_seq;
  int block_size;                   // tokens per page
  int max_partitions;
  int partition_size;
  int num_tokens;
  int skip_single;
};

struct CacheWriteArgs {
  const void* key;
  const void* value;
  void* key_cache;
  void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;   // nullptr: token b is sequence b's single new token
  int num_seqs;
  int num_tokens;
  int num_kv_heads;
  int num_blocks;
  int max_blocks_per_seq;
};

// kv_f32 / out_f32 select fp32 (true) or bf16 (false) storage; block_size is
// the page size in tokens (16, 32 or 64).
// stream_kv: bf16 K/V loads with the non-temporal hint (for batches whose K/V
// is far larger than the last-level cache).
hipError_t launch_decode(const DecodeArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32, int num_seqs,
                         bool stream_kv, hipStream_t stream);
// Workers (4 per work-group) that fill the device at full occupancy.
int stream_workers(int head_dim, int block_size, bool kv_f32, bool out_f32, int group, int num_seqs);
hipError_t launch_stream_decode(const StreamArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32,
                                bool stream_kv, hipStream_t stream);
hipError_t launch_stream_reduce(const StreamArgs& a, int head_dim, bool kv_f32, bool out_f32, hipStream_t stream);
// Resident waves of the partitioned balanced decode, and its launch (a.num_workers / 4 work-groups).
int partition_workers(int head_dim, int block_size, bool kv_f32, bool out_f32, int num_seqs);
hipError_t launch_stream_partition(const StreamPartArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32,
                                   bool stream_kv, hipStream_t stream);
// Rows per prefill work-group (depends only on the build).
int prefill_rows_per_group();
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32,
                          int grid_groups, hipStream_t stream);
// Mixed batch, bf16: the scheduling pass writes the work units, ordered by
// decreasing cost; the fused kernel runs unit i / Hkv for kv head i % Hkv.
// Rows of a prefill unit for a launch of `waves` waves per work-group (4 or 8;
// 32 rows per wave):
int prefill_lds_rows_per_group(int waves = 4);
// Decode partitions per pack record: one per wave of a 4-wave work-group (an
// 8-wave work-group of the fused kernel runs them on its first four waves).
constexpr int kPackSlots = 4;
// A scheduled unit, four 16-byte slots, read by its work-group together with
// the unit count.
//  - Prefill row tile rt of sequence b: s[0] = {b, rt, q0, q1} (the sequence's
//    query_start_loc[b], [b + 1]), s[1] = {seq_len, 0, 0, 0}, s[2], s[3] =
//    block_tables[b][min(j, pages - 1)] for j = 0..7: the pages of the first
//    two 64-key tiles, so that the unit's first K/V loads wait on no other
//    load than the record's.
//  - Decode partition p of sequence b run by the whole work-group (a long
//    partition): s[0] = {b, -1 - p, row, seq_len} (row: the sequence's query
//    row), s[1].x = kUnitWholeGroup.
//  - Up to four short decode partitions, one per wave: s[w] = {b, -1 - p, row,
//    seq_len} for wave w, s[w].x = kUnitEmpty for a wave without one.
struct MixedUnit {
  int4 s[4];
};
constexpr int kUnitEmpty = -1;
constexpr int kUnitWholeGroup = -2;
// Decode partitions of more 32-token tiles than this are run by a whole
// work-group (its waves take the tiles round-robin); shorter ones by one wave.
constexpr int kWaveDecodeMaxTiles = 64;
struct ScheduleArgs {
  const int32_t* seq_lens;
  const int32_t* block_tables;
  const int32_t* query_start_loc;
  MixedUnit* units;                 // [unit_capacity]
  int* unit_count;
  int unit_capacity;
  int num_seqs;
  int num_tokens;
  int max_query_len;
  int group;
  int rows_per_group;
  int max_blocks_per_seq;
  int block_size;                   // tokens per page
  int partition_size;               // decode partitions (tokens, multiple of 32)
  int max_partitions;
  int causal;                       // as PrefillArgs::causal
};
struct MixedArgs {
  PrefillArgs prefill;
  DecodeArgs decode;
  const MixedUnit* units;
  const int* unit_count;
};
// Shared-prefix decode, bf16: groups of consecutive sequences whose first
// prefix_lens[g] tokens are the same.  Prefix units (group, row tile, key
// chunk, kv head) run the prefill role over the group's queries against the
// shared keys [chunk * PC, ...) of the first member's block table; suffix
// units (sequence, partition, kv head) run the decode over the sequence's
// remaining keys.  Both write partials, merged per (sequence, head).
struct SharedPrefixArgs {
  PrefillArgs prefill;              // query rows = sequences, causal = 0
  DecodeArgs decode;                // suffix partitions of partition_size tokens
  const int32_t* group_start;       // [num_groups + 1]
  const int32_t* prefix_lens;       // [num_groups]
  float* part_out;                  // [B, Hq, slots, D]
  float* part_lse;                  // [B, Hq, slots]
  int2* seq_meta;                   // [B]: {prefix chunks, suffix partitions}
  int num_seqs;
  int num_groups;
  int row_tiles;                    // row tiles of the largest group
  int prefix_chunks;                // MC: chunk slots [0, MC)
  int chunk_tokens;                 // PC, a multiple of 64
  int slots;                        // MC + suffix partitions
};
hipError_t launch_shared_prefix(const SharedPrefixArgs& a, int head_dim, int block_size, bool out_f32,
                                hipStream_t stream);

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t stream);
hipError_t launch_mixed(const MixedArgs& a, int head_dim, int block_size, bool out_f32, int grid_groups, int waves,
                        hipStream_t stream);
hipError_t launch_reduce(const ReduceArgs& a, int head_dim, bool out_f32, int num_seqs, hipStream_t stream);
hipError_t launch_cache_write(const CacheWriteArgs& a, int head_dim, int block_size, bool kv_f32,
                              hipStream_t stream);
// Measurement probe: `groups` work-groups of 4 waves issue bf16 matrix-core
// products for `iters` rounds; mfma_probe_flops gives the flops of one launch.
hipError_t launch_mfma_probe(float* out, int groups, int iters, hipStream_t stream);
long long mfma_probe_flops(int groups, int iters);

}  // namespace gqa
