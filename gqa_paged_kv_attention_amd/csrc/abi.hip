// C ABI of libgqa_paged.so: host-side validation of scalar arguments, grid
// sizing and kernel dispatch.  No allocation, no synchronisation, no state.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>

#include "gqa_paged.h"
#include "gqa_internal.h"

namespace {

constexpr int kTileTokens = 32;
constexpr int kMaxGroup = 32;
constexpr int kMaxSeqLen = 1 << 28;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int check_dims(const gqa_dims& d) {
  if (d.num_seqs < 0 || d.num_heads <= 0 || d.num_kv_heads <= 0 || d.head_dim <= 0 || d.block_size <= 0 ||
      d.num_blocks <= 0 || d.max_blocks_per_seq <= 0)
    return GQA_ERR_INVALID_ARG;
  if (d.num_heads % d.num_kv_heads != 0) return GQA_ERR_INVALID_ARG;
  if (d.q_dtype != GQA_F32 && d.q_dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  if (d.kv_dtype != GQA_F32 && d.kv_dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  if (d.out_dtype != GQA_F32 && d.out_dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  if (d.head_dim != 64 && d.head_dim != 128) return GQA_ERR_UNSUPPORTED;
  if (d.block_size != 16 && d.block_size != 32 && d.block_size != 64) return GQA_ERR_UNSUPPORTED;
  if (d.q_dtype != d.kv_dtype) return GQA_ERR_UNSUPPORTED;
  if ((long long)d.max_blocks_per_seq * d.block_size > kMaxSeqLen) return GQA_ERR_UNSUPPORTED;
  if (d.num_seqs > 65535) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

// Effective partitioning: tokens per partition and number of partitions.
bool partitioning(int32_t max_seq_len, int32_t partition_size, int* psize, int* nparts) {
  if (max_seq_len < 0 || max_seq_len > kMaxSeqLen || partition_size < 0) return false;
  if (partition_size > 0 && partition_size % kTileTokens != 0) return false;
  if (partition_size == 0 || partition_size >= max_seq_len) {
    const int p = max_seq_len <= 0 ? kTileTokens : (max_seq_len + kTileTokens - 1) / kTileTokens * kTileTokens;
    *psize = partition_size > 0 ? (p > partition_size ? p : partition_size) : p;
    *nparts = 1;
  } else {
    *psize = partition_size;
    *nparts = (max_seq_len + partition_size - 1) / partition_size;
  }
  return true;
}

// Fixed-partition workspace: [partial_out][partial_lse]; nothing when every
// sequence fits one partition.
size_t partial_bytes(const gqa_dims& d, int nparts) {
  if (nparts <= 1) return 0;
  const size_t rows = (size_t)d.num_seqs * d.num_heads * nparts;
  return align_up(rows * d.head_dim * sizeof(float)) + align_up(rows * sizeof(float));
}

int status_from(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_ERR_LAUNCH; }

int device_workers(const gqa_dims& d);

// partition_size == 0 picks the decomposition: the balanced (stream) decode,
// or one work-group per (sequence, kv head) unit.  The balanced decode pays a
// merge kernel, the partials of the units it cuts (G x D fp32 each) and a
// start per segment; one work-group per unit pays for the longest unit, whose
// four waves walk max_seq_len / 128 tiles each while shorter units' work-groups
// sit idle.  So the balanced decode runs when the batch has few units (at most
// an eighth of the device's resident work-groups) or when the longest sequence
// is long enough for that imbalance to outweigh the split's costs, a length
// that grows with G (more partial bytes per cut): max_seq_len > 768 G.
// Measured (bf16, d = 128, lengths uniform in the ranges; balanced / one
// work-group per unit, us):
//   64 seqs x 8 kv heads, 512..4096 tokens, G = 4: 106 / 128 -> balanced
//   16 x 8, 1024..8192, G = 4: 56 / 84;  16 x 8, 512..4096, G = 4: 34 / 40
//   2 kv heads x 16 seqs, 2048..4096, G = 16: 32 / 39
//   128 x 2, 32..1024, G = 16: 28 / 17 -> one per unit
//   32 x 8, 512..1024, G = 4: 26 / 19;  32 x 8, 1024..2048, G = 4: 40 / 34
//   32 x 8, 2048..4096, G = 8: 85 / 76;  16 x 8, 1024..2048, G = 8: 28 / 25
//   64 x 8, 512..1024, G = 4: 40 / 34;  64 x 2, 1024..2048, G = 16: 31 / 26
// G > 16 never takes it (a cut segment's partial weighs as much as a tile).
// The stream kernel also needs the batch to fit its LDS table and the tile
// count to fit in 32 bits.
bool use_stream(const gqa_dims& d, int32_t partition_size, int32_t max_seq_len) {
  if (partition_size != 0 || d.num_seqs == 0 || d.num_seqs > gqa::kMaxStreamSeqs) return false;
  const int G = d.num_heads / d.num_kv_heads;
  if (G > 16) return false;
  const long long tiles_per_seq = ((long long)d.max_blocks_per_seq * d.block_size + kTileTokens - 1) / kTileTokens;
  if ((long long)d.num_seqs * d.num_kv_heads * tiles_per_seq >= (1LL << 31) - 1) return false;
  const long long resident_groups = device_workers(d) / gqa::kStreamWorkersPerGroup;
  const long long units = (long long)d.num_seqs * d.num_kv_heads;
  if (units >= 2 * resident_groups) return false;
  return 8 * units <= resident_groups || (long long)max_seq_len > 768LL * G;
}

// Compute units of the current device (cached per device; 256 without one).
int device_cus() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
  cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// The partition size the library picks (partition_size == 0) when the
// balanced decode does not run: one partition per sequence, except for G > 16
// over K/V beyond the last-level cache (smaller K/V runs each kv head's query
// heads as two 16-row units instead, see run_decode) when the batch has fewer
// (sequence, kv head) units than the device has compute units.  Then
// sequences are cut into partitions of at least kMinPickedPartition tokens,
// enough of them for about two work-groups per compute unit: with G = 32 a
// partition's partial (32 rows x D fp32) is as large as the K and V of 32
// tokens, and shorter partitions lost (MQA, 128 sequences of U{32..1024}
// tokens, before the 16-row units: 23.6 us with one partition per sequence,
// 20.6 us at 512 tokens, 26.8 us at 256, 38.6 us at 128; with the 16-row
// units, 16.8 us unsplit and 21.4 us at 512 tokens).
constexpr int kMinPickedPartition = 512;
bool stream_kv(const gqa_dims& d, int32_t max_seq_len);
int32_t picked_partition(const gqa_dims& d, int32_t max_seq_len, int32_t partition_size) {
  if (partition_size != 0 || d.num_seqs == 0 || d.num_heads / d.num_kv_heads <= 16) return partition_size;
  if (!stream_kv(d, max_seq_len)) return 0;
  const long long units = (long long)d.num_seqs * d.num_kv_heads;
  const long long cus = device_cus();
  if (units >= cus) return 0;
  const long long want = (2 * cus + units - 1) / units;                // partitions per sequence
  const long long p = std::max<long long>(kMinPickedPartition, (max_seq_len + want - 1) / want);
  const long long psize = (p + kTileTokens - 1) / kTileTokens * kTileTokens;
  return psize < max_seq_len ? (int32_t)psize : 0;
}

// Cache policy of the decode's K/V loads: the non-temporal hint when the
// K/V the call can read, min(num_seqs x max_seq_len, the whole page pool)
// tokens, exceeds twice the 256 MB last-level cache of the device, so that
// the stream of pages that will not be reused before they are evicted does
// not evict what is; plain loads below that, which leave a batch that fits
// in that cache for the next call on the same batch to find there.  The
// bound overestimates what is read (up to 2x for lengths spread evenly up to
// max_seq_len), hence twice the cache.
constexpr double kStreamKvBytes = 512.0 * (1 << 20);
bool stream_kv(const gqa_dims& d, int32_t max_seq_len) {
  const double per_token = 2.0 * d.num_kv_heads * d.head_dim * (d.kv_dtype == GQA_F32 ? 4 : 2);
  const double upper = (double)d.num_seqs * std::max(max_seq_len, 0) * per_token;
  const double pool = (double)d.num_blocks * d.block_size * per_token;
  return std::min(upper, pool) > kStreamKvBytes;
}

// Fixed partitions (partition_size > 0) with G <= 16 run the partitioned
// balanced decode: persistent waves walk whole partitions back to back, their
// load pipeline running across partition boundaries, instead of one
// work-group per partition.  Same partials, same workspace, same reduce.
// The kernel's LDS (a 32-row partial buffer per wave plus the per-sequence
// tables) leaves room for two work-groups per compute unit up to
// kMaxPartitionedSeqs sequences; buffered partial rows are int indices.
constexpr int kMaxPartitionedSeqs = 1536;
bool use_stream_partitioned(const gqa_dims& d, int32_t partition_size, int nparts) {
  if (partition_size <= 0 || nparts <= 1 || d.num_seqs == 0 || d.num_seqs > kMaxPartitionedSeqs) return false;
  if (d.num_heads / d.num_kv_heads > 16) return false;
  if ((long long)d.num_seqs * d.num_heads * nparts >= (1LL << 31) - 1) return false;
  const long long tiles_per_seq = ((long long)d.max_blocks_per_seq * d.block_size + kTileTokens - 1) / kTileTokens;
  return (long long)d.num_seqs * d.num_kv_heads * tiles_per_seq < (1LL << 31) - 1;
}

// Balanced-decode workspace: [tile prefix, B + 1 ints][unit metadata, B * Hkv int4]
// [segment outputs][segment lse][whole-unit outputs, B * Hq * D][whole-unit lse, B * Hq]
// (the last two serve the fused append).
size_t stream_bytes(const gqa_dims& d, int workers) {
  const int G = d.num_heads / d.num_kv_heads;
  const size_t segs = (size_t)workers * 2 * G;
  const size_t rows = (size_t)d.num_seqs * d.num_heads;
  return align_up((size_t)(d.num_seqs + 1) * sizeof(int)) +
         align_up((size_t)d.num_seqs * d.num_kv_heads * 4 * sizeof(int)) + align_up(segs * d.head_dim * sizeof(float)) +
         align_up(segs * sizeof(float)) + align_up(rows * d.head_dim * sizeof(float)) + align_up(rows * sizeof(float));
}

int device_workers(const gqa_dims& d) {
  return gqa::stream_workers(d.head_dim, d.block_size, d.kv_dtype == GQA_F32, d.out_dtype == GQA_F32,
                             d.num_heads / d.num_kv_heads, d.num_seqs);
}

size_t decode_workspace(const gqa_dims& d, int32_t max_seq_len, int32_t partition_size) {
  if (use_stream(d, partition_size, max_seq_len)) return stream_bytes(d, device_workers(d));
  int psize = 0, nparts = 0;
  if (!partitioning(max_seq_len, picked_partition(d, max_seq_len, partition_size), &psize, &nparts)) return 0;
  return partial_bytes(d, nparts);
}

// Mixed call, bf16: decode partitions of partition_size tokens, or of
// kMixedDecodePartition when the library picks.
constexpr int kMixedDecodePartition = 4096;

bool mixed_decode_split(int32_t max_seq_len, int32_t partition_size, int* psize, int* nparts) {
  return partitioning(max_seq_len, partition_size > 0 ? partition_size : kMixedDecodePartition, psize, nparts);
}

// Upper bound on scheduled units: prefill row tiles (at most one partial tile
// per sequence beyond num_tokens * G / rows) plus decode partitions.  The
// scheduling pass places units exactly for lists below kMaxMixedUnits.
constexpr long long kMaxMixedUnits = 1LL << 20;
long long mixed_unit_capacity(const gqa_dims& d, int32_t num_tokens, int nparts) {
  const long long G = d.num_heads / d.num_kv_heads;
  const long long rows = gqa::prefill_lds_rows_per_group();
  return ((long long)num_tokens * G + rows - 1) / rows + (long long)d.num_seqs * (1 + nparts);
}

// Mixed-call workspace, bf16: [units, MixedUnit][unit count][decode partials],
// or the decode's workspace if larger (a batch of decodes only runs the decode).
size_t mixed_bytes(const gqa_dims& d, int32_t num_tokens, int32_t max_seq_len, int32_t partition_size) {
  const size_t dec = decode_workspace(d, max_seq_len, partition_size);
  if (d.kv_dtype == GQA_F32) return dec;
  int psize = 0, nparts = 0;
  if (num_tokens < 0 || !mixed_decode_split(max_seq_len, partition_size, &psize, &nparts)) return 0;
  const long long cap = mixed_unit_capacity(d, num_tokens, nparts);
  const size_t fused =
      align_up((size_t)cap * sizeof(gqa::MixedUnit)) + align_up(sizeof(int)) + partial_bytes(d, nparts);
  return std::max(fused, dec);
}

// Decode launch shared by paged_gqa_decode and the decode half of the mixed call.
// new_key / new_value (decode only, query_start_loc null): a fused append of
// each sequence's new token at position seq_lens[b] - 1 (the balanced decode
// does it in its own launch; the other decompositions run the cache write
// first).
int run_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
               const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start_loc,
               int32_t num_tokens, int32_t max_seq_len, const gqa_dims& dims, float scale, int32_t partition_size,
               void* workspace, size_t workspace_bytes, hipStream_t stream, const void* new_key = nullptr,
               const void* new_value = nullptr) {
  int psize = 0, nparts = 0;
  if (!partitioning(max_seq_len, partition_size, &psize, &nparts)) return GQA_ERR_INVALID_ARG;
  const bool kv_f32 = dims.kv_dtype == GQA_F32, out_f32 = dims.out_dtype == GQA_F32;
  const float scale_log2 = scale * 1.4426950408889634f;

  if (use_stream(dims, partition_size, max_seq_len)) {
    if (workspace == nullptr) return GQA_ERR_WORKSPACE;
    // as many workers as the device holds at once, fewer if the workspace is smaller
    int workers = device_workers(dims);
    while (workers > gqa::kStreamWorkersPerGroup && stream_bytes(dims, workers) > workspace_bytes)
      workers -= gqa::kStreamWorkersPerGroup;
    if (stream_bytes(dims, workers) > workspace_bytes) return GQA_ERR_WORKSPACE;
    const int G = dims.num_heads / dims.num_kv_heads;
    char* ws = reinterpret_cast<char*>(workspace);
    const size_t segs = (size_t)workers * 2 * G;
    gqa::StreamArgs a;
    a.out = out;
    a.query = query;
    a.key_cache = key_cache;
    a.value_cache = value_cache;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.query_start_loc = query_start_loc;
    a.new_key = new_key;
    a.new_value = new_value;
    a.tile_prefix = reinterpret_cast<int*>(ws);
    ws += align_up((size_t)(dims.num_seqs + 1) * sizeof(int));
    a.unit_meta = reinterpret_cast<int4*>(ws);
    ws += align_up((size_t)dims.num_seqs * dims.num_kv_heads * 4 * sizeof(int));
    a.seg_out = reinterpret_cast<float*>(ws);
    ws += align_up(segs * dims.head_dim * sizeof(float));
    a.seg_lse = reinterpret_cast<float*>(ws);
    ws += align_up(segs * sizeof(float));
    a.unit_out = reinterpret_cast<float*>(ws);
    ws += align_up((size_t)dims.num_seqs * dims.num_heads * dims.head_dim * sizeof(float));
    a.unit_lse = reinterpret_cast<float*>(ws);
    a.num_seqs = dims.num_seqs;
    a.num_heads = dims.num_heads;
    a.num_kv_heads = dims.num_kv_heads;
    a.group = G;
    a.num_blocks = dims.num_blocks;
    a.max_blocks_per_seq = dims.max_blocks_per_seq;
    a.num_tokens = num_tokens;
    a.num_workers = workers;
    a.block_size = dims.block_size;
    a.scale_log2 = scale_log2;
    hipError_t e = gqa::launch_stream_decode(a, dims.head_dim, dims.block_size, kv_f32, out_f32,
                                             stream_kv(dims, max_seq_len), stream);
    if (e != hipSuccess) return GQA_ERR_LAUNCH;
    return status_from(gqa::launch_stream_reduce(a, dims.head_dim, kv_f32, out_f32, stream));
  }

  if (!partitioning(max_seq_len, picked_partition(dims, max_seq_len, partition_size), &psize, &nparts))
    return GQA_ERR_INVALID_ARG;
  const size_t need = partial_bytes(dims, nparts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GQA_ERR_WORKSPACE;
  if (dims.num_seqs == 0) return GQA_OK;
  if (new_key) {
    gqa::CacheWriteArgs w;
    w.key = new_key;
    w.value = new_value;
    w.key_cache = const_cast<void*>(key_cache);
    w.value_cache = const_cast<void*>(value_cache);
    w.block_tables = block_tables;
    w.seq_lens = seq_lens;
    w.query_start_loc = nullptr;          // token b is sequence b's new token
    w.num_seqs = dims.num_seqs;
    w.num_tokens = dims.num_seqs;
    w.num_kv_heads = dims.num_kv_heads;
    w.num_blocks = dims.num_blocks;
    w.max_blocks_per_seq = dims.max_blocks_per_seq;
    if (gqa::launch_cache_write(w, dims.head_dim, dims.block_size, dims.kv_dtype == GQA_F32, stream) != hipSuccess)
      return GQA_ERR_LAUNCH;
  }
  gqa::DecodeArgs a;
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  const size_t rows = (size_t)dims.num_seqs * dims.num_heads * nparts;
  char* ws = reinterpret_cast<char*>(workspace);
  a.partial_out = need ? reinterpret_cast<float*>(ws) : nullptr;
  a.partial_lse = need ? reinterpret_cast<float*>(ws + align_up(rows * dims.head_dim * sizeof(float))) : nullptr;
  a.num_heads = dims.num_heads;
  a.num_kv_heads = dims.num_kv_heads;
  a.group = dims.num_heads / dims.num_kv_heads;
  a.num_blocks = dims.num_blocks;
  a.max_blocks_per_seq = dims.max_blocks_per_seq;
  a.num_tokens = num_tokens;
  a.partition_size = psize;
  a.max_partitions = nparts;
  a.scale_log2 = scale_log2;
  hipError_t e;
  if (use_stream_partitioned(dims, partition_size, nparts)) {
    gqa::StreamPartArgs sp;
    sp.d = a;
    sp.num_seqs = dims.num_seqs;
    sp.num_workers = gqa::partition_workers(dims.head_dim, dims.block_size, kv_f32, out_f32, dims.num_seqs);
    e = gqa::launch_stream_partition(sp, dims.head_dim, dims.block_size, kv_f32, out_f32, stream_kv(dims, max_seq_len),
                                     stream);
  } else {
    // G = 32 over K/V that the last-level cache holds: each kv head's query heads run as two
    // units of 16 rows (the 16-row kernel, twice the work-groups); the second unit to read a
    // page finds it in the cache.
    const bool skv = stream_kv(dims, max_seq_len);
    if (a.group > 16 && !skv) {
      a.kv_split = 2;
      a.group /= 2;
      a.num_kv_heads *= 2;
    }
    // at most one work-group per compute unit and at most 1024 keys per
    // work-group: 8 waves, each walking half as many tiles
    if ((long long)nparts * a.num_kv_heads * dims.num_seqs <= device_cus() && std::min(psize, max_seq_len) <= 1024)
      a.waves = 8;
    e = gqa::launch_decode(a, dims.head_dim, dims.block_size, kv_f32, out_f32, dims.num_seqs, skv, stream);
  }
  if (e != hipSuccess || nparts <= 1) return status_from(e);
  gqa::ReduceArgs r;
  r.out = out;
  r.partial_out = a.partial_out;
  r.partial_lse = a.partial_lse;
  r.seq_lens = seq_lens;
  r.query_start_loc = query_start_loc;
  r.num_heads = dims.num_heads;
  r.num_kv_heads = dims.num_kv_heads;
  r.group = a.group;
  r.max_blocks_per_seq = dims.max_blocks_per_seq;
  r.block_size = dims.block_size;
  r.max_partitions = nparts;
  r.partition_size = psize;
  r.num_tokens = num_tokens;
  r.skip_single = 1;
  return status_from(gqa::launch_reduce(r, dims.head_dim, out_f32, dims.num_seqs, stream));
}

// Mixed batch of prefill chunks and decodes; `causal` false is cross-attention
// (every row sees all seq_len keys, and a chunk may be longer than seq_len).
int run_mixed(void* out, const void* query, const void* key_cache, const void* value_cache,
              const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start_loc,
              int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, const gqa_dims& dims, float scale,
              int32_t partition_size, void* workspace, size_t workspace_bytes, hipStream_t s, bool causal) {
  int st = check_dims(dims);
  if (st != GQA_OK) return st;
  if (dims.num_heads / dims.num_kv_heads > kMaxGroup) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || num_tokens < 0 || max_query_len < 0) return GQA_ERR_INVALID_ARG;
  if (causal && max_query_len > max_seq_len) return GQA_ERR_INVALID_ARG;
  if (dims.num_seqs == 0 || num_tokens == 0) {
    int ps = 0, np = 0;
    return partitioning(max_seq_len, partition_size, &ps, &np) ? GQA_OK : GQA_ERR_INVALID_ARG;
  }
  if (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens || !query_start_loc)
    return GQA_ERR_INVALID_ARG;
  // decodes only: the decode launch (one query row sees every key either way)
  if (max_query_len <= 1)
    return run_decode(out, query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, num_tokens,
                      max_seq_len, dims, scale, partition_size, workspace, workspace_bytes, s);
  const bool kv_f32 = dims.kv_dtype == GQA_F32, out_f32 = dims.out_dtype == GQA_F32;
  const int G = dims.num_heads / dims.num_kv_heads;
  const float scale_log2 = scale * 1.4426950408889634f;

  gqa::PrefillArgs p;
  p.out = out;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.query_start_loc = query_start_loc;
  p.num_seqs = dims.num_seqs;
  p.num_heads = dims.num_heads;
  p.num_kv_heads = dims.num_kv_heads;
  p.group = G;
  p.num_blocks = dims.num_blocks;
  p.max_blocks_per_seq = dims.max_blocks_per_seq;
  p.num_tokens = num_tokens;
  p.scale_log2 = scale_log2;
  p.causal = causal ? 1 : 0;

  if (!kv_f32) {
    // scheduling pass + fused prefill/decode kernel (+ merge of split decodes)
    int psize = 0, nparts = 0;
    if (!mixed_decode_split(max_seq_len, partition_size, &psize, &nparts)) return GQA_ERR_INVALID_ARG;
    const long long cap = mixed_unit_capacity(dims, num_tokens, nparts);
    if (cap >= kMaxMixedUnits || cap * dims.num_kv_heads > 0x7fffffffLL) return GQA_ERR_UNSUPPORTED;
    const size_t need = mixed_bytes(dims, num_tokens, max_seq_len, partition_size);
    if (workspace == nullptr || workspace_bytes < need) return GQA_ERR_WORKSPACE;
    char* ws = reinterpret_cast<char*>(workspace);
    gqa::MixedUnit* units = reinterpret_cast<gqa::MixedUnit*>(ws);
    ws += align_up((size_t)cap * sizeof(gqa::MixedUnit));
    int* count = reinterpret_cast<int*>(ws);
    ws += align_up(sizeof(int));
    const size_t rows = (size_t)dims.num_seqs * dims.num_heads * nparts;

    gqa::ScheduleArgs sa;
    sa.seq_lens = seq_lens;
    sa.block_tables = block_tables;
    sa.query_start_loc = query_start_loc;
    sa.units = units;
    sa.unit_count = count;
    sa.unit_capacity = (int)cap;
    sa.num_seqs = dims.num_seqs;
    sa.num_tokens = num_tokens;
    sa.max_query_len = max_query_len;
    sa.group = G;
    // Prefill-heavy batches (on average 1024 or more query rows, tokens x G,
    // per sequence) run 8-wave work-groups with 256-row prefill tiles: each
    // K/V tile is staged once for twice the rows (16 x 512 new tokens on
    // 3584-token prefixes: 7% faster; cross-attention, 16 chunks of 256 rows
    // over 1024..6400 encoder tokens: 1-6%; 2 to 8 chunks of 256..1024 tokens:
    // 5-9%).  Shorter chunks lose more to the coarser row tiles than they gain
    // (51 chunks of 624 rows each on average: 102 -> 115 us), and so do a
    // single sequence (one 2048-token chunk: 4%; the 8-wave tiles of one chunk
    // differ in cost along the diagonal, and one tile per compute unit leaves
    // nothing to even them out) and a batch of fewer 4-wave tiles than compute
    // units (one 300-token chunk: 12%).
    const long long qrows = (long long)num_tokens * G;
    const int waves = (G <= 16 && dims.num_seqs >= 2 && qrows >= 1024LL * dims.num_seqs &&
                       qrows / gqa::prefill_lds_rows_per_group(4) * dims.num_kv_heads >= device_cus())
                          ? 8
                          : 4;
    sa.rows_per_group = gqa::prefill_lds_rows_per_group(waves);
    sa.max_blocks_per_seq = dims.max_blocks_per_seq;
    sa.block_size = dims.block_size;
    sa.partition_size = psize;
    sa.max_partitions = nparts;
    sa.causal = causal ? 1 : 0;
    if (gqa::launch_schedule(sa, s) != hipSuccess) return GQA_ERR_LAUNCH;

    gqa::MixedArgs ma;
    ma.prefill = p;
    gqa::DecodeArgs& d = ma.decode;
    d.out = out;
    d.query = query;
    d.key_cache = key_cache;
    d.value_cache = value_cache;
    d.block_tables = block_tables;
    d.seq_lens = seq_lens;
    d.query_start_loc = query_start_loc;
    d.partial_out = nparts > 1 ? reinterpret_cast<float*>(ws) : nullptr;
    d.partial_lse = nparts > 1 ? reinterpret_cast<float*>(ws + align_up(rows * dims.head_dim * sizeof(float))) : nullptr;
    d.num_heads = dims.num_heads;
    d.num_kv_heads = dims.num_kv_heads;
    d.group = G;
    d.num_blocks = dims.num_blocks;
    d.max_blocks_per_seq = dims.max_blocks_per_seq;
    d.num_tokens = num_tokens;
    d.partition_size = psize;
    d.max_partitions = nparts;
    d.scale_log2 = scale_log2;
    ma.units = units;
    ma.unit_count = count;
    hipError_t e =
        gqa::launch_mixed(ma, dims.head_dim, dims.block_size, out_f32, (int)(cap * dims.num_kv_heads), waves, s);
    if (e != hipSuccess || nparts <= 1) return status_from(e);
    gqa::ReduceArgs r;
    r.out = out;
    r.partial_out = d.partial_out;
    r.partial_lse = d.partial_lse;
    r.seq_lens = seq_lens;
    r.query_start_loc = query_start_loc;
    r.num_heads = dims.num_heads;
    r.num_kv_heads = dims.num_kv_heads;
    r.group = G;
    r.max_blocks_per_seq = dims.max_blocks_per_seq;
    r.block_size = dims.block_size;
    r.max_partitions = nparts;
    r.partition_size = psize;
    r.num_tokens = num_tokens;
    r.skip_single = 1;
    return status_from(gqa::launch_reduce(r, dims.head_dim, out_f32, dims.num_seqs, s));
  }

  // fp32: prefill kernel, then the decode of paged_gqa_decode
  {
    int ps = 0, np = 0;
    if (!partitioning(max_seq_len, partition_size, &ps, &np)) return GQA_ERR_INVALID_ARG;
    if (!partitioning(max_seq_len, picked_partition(dims, max_seq_len, partition_size), &ps, &np))
      return GQA_ERR_INVALID_ARG;
    if (use_stream(dims, partition_size, max_seq_len)) {
      if (workspace == nullptr || workspace_bytes < stream_bytes(dims, gqa::kStreamWorkersPerGroup))
        return GQA_ERR_WORKSPACE;
    } else {
      const size_t need = partial_bytes(dims, np);
      if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GQA_ERR_WORKSPACE;
    }
  }
  if (max_query_len > 1) {
    const long long rpg = gqa::prefill_rows_per_group();
    // Upper bound on row tiles: every prefill sequence wastes at most one partial tile.
    const long long prefill_seqs = std::min<long long>(dims.num_seqs, num_tokens / 2);
    const long long tiles = ((long long)num_tokens * G + rpg - 1) / rpg + prefill_seqs;
    const long long groups = tiles * dims.num_kv_heads;
    if (groups > 0x7fffffffLL) return GQA_ERR_UNSUPPORTED;
    hipError_t e = gqa::launch_prefill(p, dims.head_dim, dims.block_size, true, out_f32, (int)groups, s);
    if (e != hipSuccess) return GQA_ERR_LAUNCH;
  }
  return run_decode(out, query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, num_tokens,
                    max_seq_len, dims, scale, partition_size, workspace, workspace_bytes, s);
}

// Shared-prefix decode (bf16).  Prefix chunks of 512..2048 keys (whole 64-key
// tiles) over num_groups x row tiles x Hkv, cut to give about three prefix
// work-groups per four compute units: the matrix-bound prefix units then hold
// under half of the resident work-group slots, and the HBM-bound suffix
// decodes run beside them from the start (4 groups x 64 sequences, 4096-token
// prefix: 108.8 us with about two prefix work-groups per compute unit, which
// filled every slot before any suffix started; 89.4 us at three per four;
// 89.2 us at one per two, which slowed the 4 x 16, 2048-token batch from 27.2
// to 29.6 us).  Suffix partitions of partition_size tokens or, when the
// library picks, of at least 256 tokens, cut to give about kSharedUnits
// work-groups over num_seqs x Hkv.  max_seq_len bounds both the prefixes and
// the suffixes.
constexpr long long kSharedUnits = 512;

struct SharedPrefixPlan {
  int row_tiles, chunk_tokens, prefix_chunks, suffix_parts, suffix_psize, slots;
  size_t out_bytes, lse_bytes, meta_bytes;
  long long groups;
};

int round_up(long long x, int m) { return (int)((x + m - 1) / m * m); }

bool shared_prefix_plan(const gqa_dims& d, int32_t num_groups, int32_t max_group_size, int32_t max_seq_len,
                        int32_t partition_size, SharedPrefixPlan* pl) {
  if (num_groups < 0 || max_group_size < 0 || max_group_size > d.num_seqs) return false;
  if (max_seq_len < 0 || max_seq_len > kMaxSeqLen || partition_size < 0 || partition_size % kTileTokens) return false;
  const int G = d.num_heads / d.num_kv_heads;
  const long long len = std::max(1, max_seq_len);
  pl->row_tiles = (int)(((long long)max_group_size * G + gqa::prefill_lds_rows_per_group() - 1) /
                        gqa::prefill_lds_rows_per_group());
  const long long chunk_units = std::max(1LL, (long long)num_groups * pl->row_tiles * d.num_kv_heads);
  const long long prefix_goal = std::max(1LL, (long long)device_cus() * 3 / 4);
  const long long chunks_goal = std::max(1LL, (prefix_goal + chunk_units - 1) / chunk_units);
  pl->chunk_tokens = std::min(2048, std::max(512, round_up((len + chunks_goal - 1) / chunks_goal, 64)));
  pl->prefix_chunks = (int)((len + pl->chunk_tokens - 1) / pl->chunk_tokens);
  if (partition_size > 0) {
    pl->suffix_psize = partition_size;
  } else {
    const long long seq_units = std::max(1LL, (long long)d.num_seqs * d.num_kv_heads);
    const long long parts_goal = std::max(1LL, (kSharedUnits + seq_units - 1) / seq_units);
    pl->suffix_psize = std::max(256, round_up((len + parts_goal - 1) / parts_goal, kTileTokens));
  }
  pl->suffix_parts = (int)((len + pl->suffix_psize - 1) / pl->suffix_psize);
  pl->slots = pl->prefix_chunks + pl->suffix_parts;
  const size_t rows = (size_t)d.num_seqs * d.num_heads * pl->slots;
  pl->out_bytes = align_up(rows * d.head_dim * sizeof(float));
  pl->lse_bytes = align_up(rows * sizeof(float));
  pl->meta_bytes = align_up((size_t)d.num_seqs * 2 * sizeof(int));
  pl->groups = (long long)num_groups * pl->row_tiles * pl->prefix_chunks * d.num_kv_heads +
               (long long)d.num_seqs * pl->suffix_parts * d.num_kv_heads;
  return true;
}

// Scratch of paged_gqa_decode_noalloc: one array per device, held until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol); it uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept here.
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;

// Device address of this device's scratch array, or nullptr if the runtime
// cannot give one.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" {

const char* gqa_status_string(int32_t status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_LAUNCH: return "kernel launch failed";
    case GQA_ERR_SCRATCH: return "call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

int32_t gqa_version(void) { return 101; }

int32_t gqa_probe_mfma_bf16(float* out, int32_t groups, int32_t iters, long long* flops, void* stream) {
  if (!out || !flops || groups <= 0 || iters <= 0) return GQA_ERR_INVALID_ARG;
  *flops = gqa::mfma_probe_flops(groups, iters);
  return status_from(gqa::launch_mfma_probe(out, groups, iters, reinterpret_cast<hipStream_t>(stream)));
}

int32_t reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int32_t* block_tables, const int32_t* seq_lens, const int32_t* query_start_loc,
                          int32_t num_tokens, gqa_dims dims, void* stream) {
  int st = check_dims(dims);
  if (st != GQA_OK) return st;
  if (num_tokens < 0) return GQA_ERR_INVALID_ARG;
  if (num_tokens == 0 || dims.num_seqs == 0) return GQA_OK;
  if (!key || !value || !key_cache || !value_cache || !block_tables || !seq_lens || !query_start_loc)
    return GQA_ERR_INVALID_ARG;
  gqa::CacheWriteArgs a;
  a.key = key;
  a.value = value;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = dims.num_seqs;
  a.num_tokens = num_tokens;
  a.num_kv_heads = dims.num_kv_heads;
  a.num_blocks = dims.num_blocks;
  a.max_blocks_per_seq = dims.max_blocks_per_seq;
  return status_from(gqa::launch_cache_write(a, dims.head_dim, dims.block_size, dims.kv_dtype == GQA_F32,
                                             reinterpret_cast<hipStream_t>(stream)));
}

size_t paged_gqa_decode_workspace_size(gqa_dims dims, int32_t max_seq_len, int32_t partition_size) {
  if (check_dims(dims) != GQA_OK) return 0;
  return decode_workspace(dims, max_seq_len, partition_size);
}

int32_t paged_gqa_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                         const int32_t* block_tables, const int32_t* seq_lens, int32_t max_seq_len, gqa_dims dims,
                         float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int st = check_dims(dims);
  if (st != GQA_OK) return st;
  if (dims.num_heads / dims.num_kv_heads > kMaxGroup) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (dims.num_seqs > 0 && (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens))
    return GQA_ERR_INVALID_ARG;
  return run_decode(out, query, key_cache, value_cache, block_tables, seq_lens, nullptr, dims.num_seqs,
                    max_seq_len, dims, scale, partition_size, workspace, workspace_bytes,
                    reinterpret_cast<hipStream_t>(stream));
}

int32_t paged_gqa_decode_noalloc(void* out, const void* query, const void* key_cache, const void* value_cache,
                                 const int32_t* block_tables, const int32_t* seq_lens, int32_t max_seq_len,
                                 gqa_dims dims, float scale, int32_t partition_size, void* stream) {
  int st = check_dims(dims);
  if (st != GQA_OK) return st;
  if (dims.num_heads / dims.num_kv_heads > kMaxGroup) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (dims.num_seqs > 0 && (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens))
    return GQA_ERR_INVALID_ARG;
  int psize = 0, nparts = 0;
  if (!partitioning(max_seq_len, partition_size, &psize, &nparts)) return GQA_ERR_INVALID_ARG;
  if (decode_workspace(dims, max_seq_len, partition_size) > GQA_NOALLOC_SCRATCH_BYTES) return GQA_ERR_SCRATCH;
  if (dims.num_seqs == 0) return GQA_OK;
  void* ws = device_scratch();
  if (ws == nullptr) return GQA_ERR_LAUNCH;
  return run_decode(out, query, key_cache, value_cache, block_tables, seq_lens, nullptr, dims.num_seqs,
                    max_seq_len, dims, scale, partition_size, ws, GQA_NOALLOC_SCRATCH_BYTES,
                    reinterpret_cast<hipStream_t>(stream));
}

int32_t paged_gqa_decode_append(void* out, const void* query, const void* key, const void* value, void* key_cache,
                                void* value_cache, const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t max_seq_len, gqa_dims dims, float scale, int32_t partition_size,
                                void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims);
  if (st != GQA_OK) return st;
  if (dims.num_heads / dims.num_kv_heads > kMaxGroup) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  if (dims.num_seqs > 0 &&
      (!out || !query || !key || !value || !key_cache || !value_cache || !block_tables || !seq_lens))
    return GQA_ERR_INVALID_ARG;
  return run_decode(out, query, key_cache, value_cache, block_tables, seq_lens, nullptr, dims.num_seqs,
                    max_seq_len, dims, scale, partition_size, workspace, workspace_bytes,
                    reinterpret_cast<hipStream_t>(stream), key, value);
}

int32_t splitk_lse_reduce(void* out, const float* partial_out, const float* partial_lse, const int32_t* seq_lens,
                          const int32_t* query_start_loc, gqa_dims dims, int32_t max_partitions,
                          int32_t partition_size, int32_t skip_single, void* stream) {
  int st = check_dims(dims);
  if (st != GQA_OK) return st;
  if (max_partitions <= 0 || partition_size <= 0) return GQA_ERR_INVALID_ARG;
  if (dims.num_heads / dims.num_kv_heads > kMaxGroup) return GQA_ERR_UNSUPPORTED;
  if (dims.num_seqs == 0) return GQA_OK;
  if (!out || !partial_out || !partial_lse || !seq_lens) return GQA_ERR_INVALID_ARG;
  gqa::ReduceArgs r;
  r.out = out;
  r.partial_out = partial_out;
  r.partial_lse = partial_lse;
  r.seq_lens = seq_lens;
  r.query_start_loc = query_start_loc;
  r.num_heads = dims.num_heads;
  r.num_kv_heads = dims.num_kv_heads;
  r.group = dims.num_heads / dims.num_kv_heads;
  r.max_blocks_per_seq = dims.max_blocks_per_seq;
  r.block_size = dims.block_size;
  r.max_partitions = max_partitions;
  r.partition_size = partition_size;
  r.num_tokens = query_start_loc ? 0x7fffffff : dims.num_seqs;
  r.skip_single = skip_single;
  return status_from(gqa::launch_reduce(r, dims.head_dim, dims.out_dtype == GQA_F32, dims.num_seqs,
                                        reinterpret_cast<hipStream_t>(stream)));
}

size_t chunked_prefill_paged_decode_workspace_size(gqa_dims dims, int32_t num_tokens, int32_t max_seq_len,
                                                   int32_t partition_size) {
  if (check_dims(dims) != GQA_OK) return 0;
  return mixed_bytes(dims, num_tokens, max_seq_len, partition_size);
}

int32_t chunked_prefill_paged_decode(void* out, const void* query, const void* key_cache, const void* value_cache,
                                     const int32_t* block_tables, const int32_t* seq_lens,
                                     const int32_t* query_start_loc, int32_t num_tokens, int32_t max_query_len,
                                     int32_t max_seq_len, gqa_dims dims, float scale, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return run_mixed(out, query, key_cache, value_cache, block_tables, seq_lens, query_start_loc, num_tokens,
                   max_query_len, max_seq_len, dims, scale, partition_size, workspace, workspace_bytes,
                   reinterpret_cast<hipStream_t>(stream), true);
}

size_t paged_cross_attention_workspace_size(gqa_dims dims, int32_t num_tokens, int32_t max_encoder_len,
                                            int32_t partition_size) {
  if (check_dims(dims) != GQA_OK) return 0;
  return mixed_bytes(dims, num_tokens, max_encoder_len, partition_size);
}

int32_t paged_cross_attention(void* out, const void* query, const void* key_cache, const void* value_cache,
                              const int32_t* block_tables, const int32_t* encoder_lens,
                              const int32_t* query_start_loc, int32_t num_tokens, int32_t max_query_len,
                              int32_t max_encoder_len, gqa_dims dims, float scale, int32_t partition_size,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return run_mixed(out, query, key_cache, value_cache, block_tables, encoder_lens, query_start_loc, num_tokens,
                   max_query_len, max_encoder_len, dims, scale, partition_size, workspace, workspace_bytes,
                   reinterpret_cast<hipStream_t>(stream), false);
}

size_t paged_gqa_decode_shared_prefix_workspace_size(gqa_dims dims, int32_t num_groups, int32_t max_group_size,
                                                    int32_t max_seq_len, int32_t partition_size) {
  if (check_dims(dims) != GQA_OK) return 0;
  if (dims.kv_dtype == GQA_F32) return decode_workspace(dims, max_seq_len, partition_size);
  SharedPrefixPlan pl;
  if (!shared_prefix_plan(dims, num_groups, max_group_size, max_seq_len, partition_size, &pl)) return 0;
  return pl.out_bytes + pl.lse_bytes + pl.meta_bytes;
}

int32_t paged_gqa_decode_shared_prefix(void* out, const void* query, const void* key_cache, const void* value_cache,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       const int32_t* group_start, const int32_t* prefix_lens, int32_t num_groups,
                                       int32_t max_group_size, int32_t max_seq_len, gqa_dims dims, float scale,
                                       int32_t partition_size, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  int st = check_dims(dims);
  if (st != GQA_OK) return st;
  if (dims.num_heads / dims.num_kv_heads > kMaxGroup) return GQA_ERR_UNSUPPORTED;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dims.kv_dtype == GQA_F32) {
    // fp32 caches: the plain decode (each sequence reads its own pages)
    if (dims.num_seqs > 0 && (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens))
      return GQA_ERR_INVALID_ARG;
    return run_decode(out, query, key_cache, value_cache, block_tables, seq_lens, nullptr, dims.num_seqs,
                      max_seq_len, dims, scale, partition_size, workspace, workspace_bytes, s);
  }
  SharedPrefixPlan pl;
  if (!shared_prefix_plan(dims, num_groups, max_group_size, max_seq_len, partition_size, &pl))
    return GQA_ERR_INVALID_ARG;
  if (dims.num_seqs == 0) return GQA_OK;
  if (!out || !query || !key_cache || !value_cache || !block_tables || !seq_lens) return GQA_ERR_INVALID_ARG;
  if (num_groups > 0 && (!group_start || !prefix_lens)) return GQA_ERR_INVALID_ARG;
  if (pl.groups >= 0x7fffffffLL) return GQA_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < pl.out_bytes + pl.lse_bytes + pl.meta_bytes) return GQA_ERR_WORKSPACE;
  const int G = dims.num_heads / dims.num_kv_heads;
  const float scale_log2 = scale * 1.4426950408889634f;
  char* ws = reinterpret_cast<char*>(workspace);

  gqa::SharedPrefixArgs a;
  gqa::PrefillArgs& p = a.prefill;
  p.out = out;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.query_start_loc = nullptr;
  p.num_seqs = dims.num_seqs;
  p.num_heads = dims.num_heads;
  p.num_kv_heads = dims.num_kv_heads;
  p.group = G;
  p.num_blocks = dims.num_blocks;
  p.max_blocks_per_seq = dims.max_blocks_per_seq;
  p.num_tokens = dims.num_seqs;
  p.scale_log2 = scale_log2;
  p.causal = 0;
  gqa::DecodeArgs& d = a.decode;
  d.out = out;
  d.query = query;
  d.key_cache = key_cache;
  d.value_cache = value_cache;
  d.block_tables = block_tables;
  d.seq_lens = seq_lens;
  d.query_start_loc = nullptr;
  d.partial_out = nullptr;
  d.partial_lse = nullptr;
  d.num_heads = dims.num_heads;
  d.num_kv_heads = dims.num_kv_heads;
  d.group = G;
  d.num_blocks = dims.num_blocks;
  d.max_blocks_per_seq = dims.max_blocks_per_seq;
  d.num_tokens = dims.num_seqs;
  d.partition_size = pl.suffix_psize;
  d.max_partitions = pl.suffix_parts;
  d.scale_log2 = scale_log2;
  a.group_start = group_start;
  a.prefix_lens = prefix_lens;
  a.part_out = reinterpret_cast<float*>(ws);
  a.part_lse = reinterpret_cast<float*>(ws + pl.out_bytes);
  a.seq_meta = reinterpret_cast<int2*>(ws + pl.out_bytes + pl.lse_bytes);
  a.num_seqs = dims.num_seqs;
  a.num_groups = num_groups;
  a.row_tiles = pl.row_tiles;
  a.prefix_chunks = pl.prefix_chunks;
  a.chunk_tokens = pl.chunk_tokens;
  a.slots = pl.slots;
  return status_from(gqa::launch_shared_prefix(a, dims.head_dim, dims.block_size, dims.out_dtype == GQA_F32, s));
}

}  // extern "C"
