// Paged GQA attention kernels for gfx950: decode (fixed split-K partitions or
// a balanced persistent split) and the fp32 chunked prefill.  The G heads (and
// for prefill, the chunk's new tokens times G) form the 16-wide column block of
// the matrix-core products described in gqa_common.h; the per-wave tile
// pipeline is in decode_core.h.
#include <map>
#include <mutex>
#include <tuple>

#include "decode_core.h"
#include "work_map.h"

namespace gqa {

namespace {

// Fixed-partition decode: grid (max_partitions, Hkv, B), W waves per work-group.
template <class Tile, int D, int NT, class OutT, int W>
__global__ __launch_bounds__(W * kWave) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<Tile, D, NT>())))
void decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) float lds[DecodeMergeLds<D, NT, W>::kFloats];
  int p = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  if (a.kv_split == 2) {
    // The two units of a kv head (kv = 2 k and 2 k + 1) read the same pages:
    // paired_unit gives them ids 8 apart (one XCD, one L2), so that the second
    // finds the pages the first one fetched.  u enumerates (p, k, b), p fastest.
    int u, half;
    paired_unit(p + gridDim.x * (kv + gridDim.y * b), gridDim.x * gridDim.y * gridDim.z, &u, &half);
    const int hk = gridDim.y / 2;
    p = u % gridDim.x;
    kv = 2 * (u / gridDim.x % hk) + half;
    b = u / gridDim.x / hk;
  }
  decode_partition<Tile, D, NT, OutT, W>(a, p, kv, b, lds);
}

// ---------------------------------------------------------------------------
// Balanced decode.  Work items are 32-token tiles; sequence b contributes
// Hkv units of ceil(L_b / 32) tiles each (none if it is not a decode), laid
// out sequence-major, then kv head, then tile.  With T items and W workers
// (waves), worker w owns items [floor(T w / W), floor(T (w+1) / W)): every wave
// streams the same number of tiles whatever the length mix, and it runs
// through consecutive units without a work-group barrier.  A unit that lies
// inside one worker's range is written to `out` directly; a unit cut by range
// boundaries leaves one normalised partial per worker (slot 0 if it is the
// worker's first segment, else slot 1), merged by stream_reduce_kernel.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int worker_of(long long t, long long T, int W) {
  return (int)(((t + 1) * W - 1) / T);
}

__device__ __forceinline__ bool stream_is_decode(const StreamArgs& a, int b, int* row) {
  if (!a.query_start_loc) {
    *row = b;
    return true;
  }
  const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
  *row = q0;
  return q1 - q0 == 1 && q1 <= a.num_tokens && q0 >= 0;
}

__device__ __forceinline__ float load1f(const float* p) { return *p; }
__device__ __forceinline__ float load1f(const uint16_t* p) { return bf16_bits_to_float(*p); }

// Fused append (paged_gqa_decode_append), new token of sequence b at position
// L - 1 = seq_lens[b] - 1: the decode reads keys [0, L - 1) from the pages and
// masks that slot; the merge kernel folds the token in from new_key /
// new_value and then stores it into its page slot, as reshape_and_cache would.
// True when sequence b (seq_lens[b] = seq_len, L = seq_len clamped to its
// block-table row) takes that path.
__device__ __forceinline__ bool append_folds(const StreamArgs& a, int seq_len, int L) {
  return a.new_key != nullptr && L > 0 && L == seq_len;
}

template <class Tile, int D, int NT, class OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<Tile, D, NT>())))
void stream_decode_kernel(StreamArgs a) {
  extern __shared__ int s_pref[];          // [B + 1] exclusive prefix of tiles * Hkv, then s_len
  __shared__ int s_scan[kWaves];
  const int B = a.num_seqs, G = a.group;
  int* s_len = s_pref + B + 1;             // [B]: keys each decode reads from the pages
  const int lane = lane_id();
  const int n = lane & 15, q = lane >> 4;
  OutT* out = reinterpret_cast<OutT*>(a.out);

  // ---- prefix of per-sequence work, in chunks of kThreads sequences ----
  int running = 0;
  for (int c0 = 0; c0 < B; c0 += kThreads) {
    const int b = c0 + threadIdx.x;
    int v = 0;
    if (b < B) {
      int row;
      const bool dec = stream_is_decode(a, b, &row);
      const int sl = a.seq_lens[b];
      const int L = dec ? clamp_len(sl, a.max_blocks_per_seq, Tile::kBS) : 0;
      v = (L + kTile - 1) / kTile * a.num_kv_heads;
      // fused append: the pages supply keys [0, L - 1); the merge kernel adds the new token
      s_len[b] = append_folds(a, sl, L) ? L - 1 : L;
      if (dec && L == 0 && (b % gridDim.x) == (int)blockIdx.x) {
        // an empty decode sequence has a zero output row
        for (int i = 0; i < a.num_heads * D; ++i) store1(out + (size_t)row * a.num_heads * D + i, 0.f);
      }
    }
    // inclusive scan within the wave (lane shuffles), then across the four
    // wave totals: two barriers per chunk
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    const int w = wave_id();
    if (lane == kWave - 1) s_scan[w] = x;
    __syncthreads();
    int base = running;
    for (int i = 0; i < w; ++i) base += s_scan[i];
    if (b < B) s_pref[b + 1] = base + x;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) running += s_scan[i];
    __syncthreads();
  }
  if (threadIdx.x == 0) s_pref[0] = 0;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= B; i += kThreads) a.tile_prefix[i] = s_pref[i];

  const long long T = s_pref[B];
  const int W = a.num_workers;
  // merge metadata of units blockIdx.x, blockIdx.x + gridDim.x, ...: the workers
  // that hold the unit's first and last tiles, the slot of its first segment,
  // and its output row (first worker == last worker: nothing to merge)
  for (int u = blockIdx.x * kThreads + threadIdx.x; u < B * a.num_kv_heads; u += gridDim.x * kThreads) {
    const int b = u / a.num_kv_heads, kv = u % a.num_kv_heads;
    const int nt = (s_pref[b + 1] - s_pref[b]) / a.num_kv_heads;
    int4 m = make_int4(0, 0, 0, -1);
    if (nt > 0) {
      const long long u0 = s_pref[b] + (long long)kv * nt;
      int row;
      stream_is_decode(a, b, &row);
      m = make_int4(worker_of(u0, T, W), worker_of(u0 + nt - 1, T, W), (T * worker_of(u0, T, W) / W == u0) ? 0 : 1,
                    row);
    }
    a.unit_meta[u] = m;
  }
  const int w = blockIdx.x * kWaves + wave_id();
  const long long lo = T * w / W, hi = T * (w + 1) / W;
  long long t = lo;
  bool first = true;
  while (t < hi) {
    // sequence owning item t: the largest b with s_pref[b] <= t
    int bl = 0, bh = B;
    while (bh - bl > 1) {
      const int mid = (bl + bh) >> 1;
      if (s_pref[mid] <= t) bl = mid; else bh = mid;
    }
    const int b = uniform(bl);
    const int nt = (s_pref[b + 1] - s_pref[b]) / a.num_kv_heads;
    const int off = (int)(t - s_pref[b]);
    const int kv = off / nt;
    const int tile_begin = off % nt;
    const long long unit0 = s_pref[b] + (long long)kv * nt;
    const int tile_end = (int)min((long long)nt, hi - unit0);
    int row;
    stream_is_decode(a, b, &row);
    const int Lp = s_len[b];                 // from the prefix pass: no dependent load before the page ids

    typename Tile::Q qf[NT];
    load_group_query<Tile, D, NT>(qf, a.query, row, a.num_heads, kv, G, lane);
    WaveState<Tile, NT> st;
    st.reset();
    run_tiles<Tile, D, NT>(st, qf, a.key_cache, a.value_cache, a.block_tables + (size_t)b * a.max_blocks_per_seq,
                           a.num_blocks, a.num_kv_heads, kv, Lp, Lp - 1, tile_begin, tile_end, 1, a.scale_log2, lane);

    const bool whole = tile_begin == 0 && tile_end == nt;
    const int slot = first ? 0 : 1;
#pragma unroll
    for (int nt_ = 0; nt_ < NT; ++nt_) {
      const int g = nt_ * 16 + n;
      const float lr = row_sum4(st.l[nt_]);
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      if (g < G) {
        if (whole && a.new_key) {
          // fused append: every unit goes through the merge kernel
          const size_t r = (size_t)b * a.num_heads + kv * G + g;
          float* dst = a.unit_out + r * D + 4 * q;
#pragma unroll
          for (int dt = 0; dt < Tile::DT; ++dt) store4(dst + dt * 16, st.o[nt_][dt] * inv);
          if (q == 0) a.unit_lse[r] = lr > 0.f ? (st.m[nt_] + __log2f(lr)) * kLn2 : -INFINITY;
        } else if (whole) {
          OutT* dst = out + ((size_t)row * a.num_heads + kv * G + g) * D + 4 * q;
#pragma unroll
          for (int dt = 0; dt < Tile::DT; ++dt) store4(dst + dt * 16, st.o[nt_][dt] * inv);
        } else {
          const size_t seg = ((size_t)w * 2 + slot) * G + g;
          float* dst = a.seg_out + seg * D + 4 * q;
#pragma unroll
          for (int dt = 0; dt < Tile::DT; ++dt) store4(dst + dt * 16, st.o[nt_][dt] * inv);
          if (q == 0) a.seg_lse[seg] = lr > 0.f ? (st.m[nt_] + __log2f(lr)) * kLn2 : -INFINITY;
        }
      }
    }
    t = unit0 + tile_end;
    first = false;
  }
}

// Merge the cut units of the balanced decode: grid (units, G), one thread per
// output channel.  The work-group reads its unit's metadata and, if the unit's
// tiles span several workers, combines their segments in worker order
// (reproducible), folding kMergeBatch segments at a time with independent loads
// and an online log-sum-exp: two memory round trips in all.  In a fused append
// every unit comes here (a whole unit as its one fp32 partial), and the new
// token is one more term: log-weight scale * q.k_new, value v_new, loaded
// beside the partials.
constexpr int kMergeBatch = 8;

// Fused append, the work-group of (unit b * Hkv + kv, row 0) in the merge
// kernel: the new token into its page slot (a missing page leaves it
// unwritten), thread d taking channel d.  The key row is token-major, so the
// threads' elements are one contiguous store.  In the channel-major value page
// the token's elements lie one per channel row; each thread rewrites the whole
// 32-byte sector around its element (the slot patched in registers) instead of
// storing the element alone, which memory serves as a partial-sector write.
// No kernel of the call reads the slot, and the sector's other tokens are the
// sequence's own, which nothing writes while it appends.
template <int D, class T>
__device__ __forceinline__ void append_store(const StreamArgs& a, int b, int kv, int d) {
  const int pos = a.seq_lens[b] - 1;
  const int page = a.block_tables[(size_t)b * a.max_blocks_per_seq + pos / a.block_size];
  if ((unsigned)page >= (unsigned)a.num_blocks) return;
  const int slot = pos % a.block_size;
  const T* kn = reinterpret_cast<const T*>(a.new_key) + ((size_t)b * a.num_kv_heads + kv) * D;
  const T* vn = reinterpret_cast<const T*>(a.new_value) + ((size_t)b * a.num_kv_heads + kv) * D;
  const size_t pbase = ((size_t)page * a.num_kv_heads + kv) * (size_t)a.block_size * D;
  T* kcache = const_cast<T*>(reinterpret_cast<const T*>(a.key_cache)) + pbase;
  T* vcache = const_cast<T*>(reinterpret_cast<const T*>(a.value_cache)) + pbase;
  kcache[(size_t)slot * D + d] = kn[d];
  constexpr int EPS = 32 / sizeof(T);                  // elements per 32-byte sector
  T* sec = vcache + (size_t)d * a.block_size + (slot & ~(EPS - 1));
  const uint4 lo = ld16(sec), hi = ld16(sec + EPS / 2);
  uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  // patch element slot mod EPS (selects on the eight 32-bit words, no indexed array)
  const int k = slot & (EPS - 1);
  uint32_t bits, mask;
  int word;
  if constexpr (sizeof(T) == 2) {
    word = k >> 1;
    const int sh = (k & 1) * 16;
    bits = (uint32_t)*reinterpret_cast<const uint16_t*>(vn + d) << sh;
    mask = 0xFFFFu << sh;
  } else {
    word = k;
    bits = *reinterpret_cast<const uint32_t*>(vn + d);
    mask = 0xFFFFFFFFu;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = (j == word) ? ((w[j] & ~mask) | bits) : w[j];
  *reinterpret_cast<uint4*>(sec) = make_uint4(w[0], w[1], w[2], w[3]);
  *reinterpret_cast<uint4*>(sec + EPS / 2) = make_uint4(w[4], w[5], w[6], w[7]);
}

template <int D, class OutT, class InT>
__global__ __launch_bounds__(D) void stream_reduce_kernel(StreamArgs a) {
  __shared__ float s_dot[D / kWave];
  const int u = blockIdx.x, g = blockIdx.y, d = threadIdx.x;
  const int4 m = a.unit_meta[u];
  const long long T = a.tile_prefix[a.num_seqs];
  const int w0 = m.x, w1 = m.y, slot0 = m.z, row = m.w;
  if (row < 0 || (w1 <= w0 && !a.new_key)) return;     // no keys, or written by the decode kernel
  const int b = u / a.num_kv_heads, kv = u % a.num_kv_heads;
  const int G = a.group, W = a.num_workers;
  const size_t r = (size_t)b * a.num_heads + kv * G + g;
  float qk = 0.f, vn = 0.f;
  bool fold = false;
  if (a.new_key) {
    // loaded beside the partials (valid addresses whether or not the sequence folds)
    const int sl = a.seq_lens[b];
    fold = append_folds(a, sl, clamp_len(sl, a.max_blocks_per_seq, a.block_size));
    qk = load1f(reinterpret_cast<const InT*>(a.query) + ((size_t)row * a.num_heads + kv * G + g) * D + d) *
         load1f(reinterpret_cast<const InT*>(a.new_key) + ((size_t)b * a.num_kv_heads + kv) * D + d);
    vn = load1f(reinterpret_cast<const InT*>(a.new_value) + ((size_t)b * a.num_kv_heads + kv) * D + d);
  }
  float M = -INFINITY, den = 0.f, acc = 0.f;
  if (w1 <= w0) {
    // a whole unit of a fused append: its normalised output and log-sum-exp
    M = a.unit_lse[r];
    den = M == -INFINITY ? 0.f : 1.f;
    acc = M == -INFINITY ? 0.f : a.unit_out[r * D + d];
  } else {
    for (int wb = w0; wb <= w1; wb += kMergeBatch) {
      float lv[kMergeBatch], ov[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const int w = wb + k;
        // workers past the unit, or with an empty range, hold no segment; every
        // range holds at least floor(T / W) items, so only T < W needs the
        // (64-bit, slow) division
        const bool has = w <= w1 && (T >= W || T * w / W != T * (w + 1) / W);
        const size_t seg = ((size_t)w * 2 + (w == w0 ? slot0 : 0)) * G + g;
        lv[k] = has ? a.seg_lse[seg] : -INFINITY;
        ov[k] = has ? a.seg_out[seg * D + d] : 0.f;
      }
      float bm = -INFINITY;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, lv[k]);
      const float nm = fmaxf(M, bm);
      const float nu = (nm == -INFINITY) ? 0.f : nm;
      const float rr = fast_exp2((M - nu) * kLog2e);
      den *= rr;
      acc *= rr;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const float wgt = fast_exp2((lv[k] - nu) * kLog2e);
        den += wgt;
        acc += wgt == 0.f ? 0.f : wgt * ov[k];
      }
      M = nm;
    }
  }
  if (fold) {
    // scale * q.k_new over the D threads: within each wave, then across waves
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) qk += __shfl_xor(qk, off);
    if (D > kWave) {
      if ((d & (kWave - 1)) == 0) s_dot[d / kWave] = qk;
      __syncthreads();
      qk = 0.f;
#pragma unroll
      for (int i = 0; i < D / kWave; ++i) qk += s_dot[i];
    }
    const float sn = qk * a.scale_log2 * kLn2;         // natural-log weight of the new token
    const float nm = fmaxf(M, sn);
    const float rr = fast_exp2((M - nm) * kLog2e);     // 0 while M = -inf
    const float wn = fast_exp2((sn - nm) * kLog2e);
    den = den * rr + wn;
    acc = acc * rr + wn * vn;
  }
  OutT* out = reinterpret_cast<OutT*>(a.out);
  store1(out + ((size_t)row * a.num_heads + kv * G + g) * D + d, den > 0.f ? acc / den : 0.f);
  if (fold && g == 0) append_store<D, InT>(a, b, kv, d);
}

// ---------------------------------------------------------------------------
// Balanced decode in fixed partitions (partition_size > 0, G <= 16).  Each
// decode unit (sequence, kv head) of nt 32-token tiles is split into
// np = ceil(nt / PT) partitions of nearly equal length (PT = partition_size /
// 32; the split decode_partition_at uses).  Units are laid out as in the
// balanced decode; worker (wave) w owns the partitions that start in
// [snap(T w / W), snap(T (w + 1) / W)), snap moving a tile position forward to
// the next partition start, so every partition belongs to exactly one worker
// and the tiles are balanced up to one partition per worker.  A wave walks its
// partitions' tiles as one stream: the paired load pipeline runs across
// partition boundaries.  When a partition is complete the wave puts its
// normalised output and log-sum-exp into an LDS buffer (kPartRows rows per
// wave) and resets its softmax state; the buffer goes to the split-K partials
// in global memory when it is full and when the wave has walked its range.
// Partials stored as each partition ended, inside the HBM read stream, cost 40
// us on 16 x 32k tokens (409 against 369 us without them); written in bursts
// at the end, with the non-temporal hint, they overlap the other waves' last
// reads (409 -> 389 us, and 384 us with the hint).  A sequence of one
// partition writes `out` directly.  splitk_reduce_kernel merges the partials.
// ---------------------------------------------------------------------------

constexpr int kPartRows = 32;           // rows of partials a wave buffers in LDS

// First tile of partition p of a unit of nt tiles in np partitions.
__device__ __forceinline__ int part_first_tile(int p, int nt, int np) {
  const int per = nt / np, extra = nt % np;
  return p * per + min(p, extra);
}

// Index of the first partition that starts at or after tile offset off (np
// when off is past the last start); the first `extra` partitions hold per + 1
// tiles, the others per (per >= 1 since np <= nt).
__device__ __forceinline__ int part_at_or_after(int off, int nt, int np) {
  const int per = nt / np, extra = nt % np;
  const int big = extra * (per + 1);
  if (off <= big) return (off + per) / (per + 1);
  return extra + (off - big + per - 1) / per;
}

// Largest b in [0, B) with s_pref[b] <= t (s_pref non-decreasing, s_pref[0] = 0 <= t).
__device__ __forceinline__ int seq_of_item(const int* s_pref, int B, long long t) {
  int bl = 0, bh = B;
  while (bh - bl > 1) {
    const int mid = (bl + bh) >> 1;
    if (s_pref[mid] <= t) bl = mid; else bh = mid;
  }
  return bl;
}

template <class Tile, int D, class OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<Tile, D, 1>())))
void stream_partition_kernel(StreamPartArgs sp) {
  // partial buffer: per wave kPartRows rows of D floats, their lse, and the
  // target row (index into the [B * Hq, max_partitions] partial rows) of
  // each buffered partition
  __shared__ __attribute__((aligned(16))) float s_part[kWaves][kPartRows][D];
  __shared__ float s_plse[kWaves][kPartRows];
  __shared__ int s_ptgt[kWaves][kPartRows];
  extern __shared__ int s_pref[];          // [B + 1] exclusive prefix of tiles * Hkv, then s_len [B]
  __shared__ int s_scan[kWaves];
  const DecodeArgs& a = sp.d;
  const int B = sp.num_seqs, G = a.group, Hkv = a.num_kv_heads;
  int* s_len = s_pref + B + 1;
  const int lane = lane_id();
  const int n = lane & 15, q = lane >> 4;
  OutT* out = reinterpret_cast<OutT*>(a.out);
  const int PT = a.partition_size / kTile;

  // ---- prefix of per-sequence tiles x Hkv, in chunks of kThreads sequences ----
  int running = 0;
  for (int c0 = 0; c0 < B; c0 += kThreads) {
    const int b = c0 + threadIdx.x;
    int v = 0;
    if (b < B) {
      int row = b;
      bool dec = true;
      if (a.query_start_loc) {
        const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
        row = q0;
        dec = q1 - q0 == 1 && q1 <= a.num_tokens && q0 >= 0;
      }
      const int L = dec ? min(clamp_len(a.seq_lens[b], a.max_blocks_per_seq, Tile::kBS),
                              a.max_partitions * a.partition_size)
                        : 0;
      v = (L + kTile - 1) / kTile * Hkv;
      s_len[b] = L;
      if (dec && L == 0 && (b % gridDim.x) == (int)blockIdx.x)
        for (int i = 0; i < a.num_heads * D; ++i) store1(out + (size_t)row * a.num_heads * D + i, 0.f);
    }
    int x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    const int wv = wave_id();
    if (lane == kWave - 1) s_scan[wv] = x;
    __syncthreads();
    int base = running;
    for (int i = 0; i < wv; ++i) base += s_scan[i];
    if (b < B) s_pref[b + 1] = base + x;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) running += s_scan[i];
    __syncthreads();
  }
  if (threadIdx.x == 0) s_pref[0] = 0;
  __syncthreads();

  const long long T = s_pref[B];
  const int W = sp.num_workers;
  // next partition start at or after item position t (T at the end)
  auto snap = [&](long long t) -> long long {
    if (t >= T) return T;
    const int b = seq_of_item(s_pref, B, t);
    const int nt = (s_pref[b + 1] - s_pref[b]) / Hkv;
    const int in_seq = (int)(t - s_pref[b]);
    const int kv = in_seq / nt, off = in_seq % nt;
    const int np = (nt + PT - 1) / PT;
    return s_pref[b] + (long long)kv * nt + part_first_tile(part_at_or_after(off, nt, np), nt, np);
  };
  const int w = blockIdx.x * kWaves + wave_id();
  const long long start = snap(T * w / W), end = snap(T * (w + 1) / W);
  const int wv = wave_id();
  const int per_buf = kPartRows / G;       // partitions the wave's buffer holds (G <= 16 <= kPartRows)
  int nbuf = 0;
  // write the wave's buffered partitions to the partials: two rows of D
  // floats per 16-byte store instruction, then the lse values
  auto drain = [&]() {
    for (int i = lane; i < nbuf * G * (D / 4); i += kWave) {
      const int r = i / (D / 4), c = 4 * (i % (D / 4));
      const int j = r / G, g = r % G;
      const size_t row = (size_t)s_ptgt[wv][j] + (size_t)g * a.max_partitions;
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t*>(&s_part[wv][r][c]),
                                  reinterpret_cast<f32x4_t*>(a.partial_out + row * D + c));
    }
    for (int r = lane; r < nbuf * G; r += kWave)
      a.partial_lse[(size_t)s_ptgt[wv][r / G] + (size_t)(r % G) * a.max_partitions] = s_plse[wv][r];
    nbuf = 0;
  };
  long long t = start;
  while (t < end) {
    const int b = uniform(seq_of_item(s_pref, B, t));
    const int nt = (s_pref[b + 1] - s_pref[b]) / Hkv;
    const int in_seq = (int)(t - s_pref[b]);
    const int kv = in_seq / nt, tile_begin = in_seq % nt;
    const long long unit0 = s_pref[b] + (long long)kv * nt;
    const int tile_end = (int)min((long long)nt, end - unit0);
    const int np = (nt + PT - 1) / PT;
    const int L = s_len[b];
    const int row = a.query_start_loc ? a.query_start_loc[b] : b;

    typename Tile::Q qf[1];
    load_group_query<Tile, D, 1>(qf, a.query, row, a.num_heads, kv, G, lane);
    WaveState<Tile, 1> st;
    st.reset();
    const size_t head0 = (size_t)b * a.num_heads + kv * G;
    int p = part_at_or_after(tile_begin, nt, np);          // tile_begin is a partition start
    int p_end = part_first_tile(p + 1, nt, np);
    // write partition p's partial, reset the state, move on to partition p + 1
    auto flush = [&]() {
      const int g = n;
      const float lr = row_sum4(st.l[0]);
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      if (np == 1) {
        if (g < G) {
          OutT* dst = out + ((size_t)row * a.num_heads + kv * G + g) * D + 4 * q;
#pragma unroll
          for (int dt = 0; dt < Tile::DT; ++dt) store4(dst + dt * 16, st.o[0][dt] * inv);
        }
      } else {
        if (nbuf == per_buf) drain();
        if (g < G) {
          const int r = nbuf * G + g;
#pragma unroll
          for (int dt = 0; dt < Tile::DT; ++dt) {
            const f32x4_t v = st.o[0][dt] * inv;
            *reinterpret_cast<float4*>(&s_part[wv][r][dt * 16 + 4 * q]) = make_float4(v[0], v[1], v[2], v[3]);
          }
          if (q == 0) s_plse[wv][r] = lr > 0.f ? (st.m[0] + __log2f(lr)) * kLn2 : -INFINITY;
        }
        if (lane == 0) s_ptgt[wv][nbuf] = (int)(head0 * a.max_partitions + p);
        ++nbuf;
      }
      st.reset();
      ++p;
      p_end = part_first_tile(p + 1, nt, np);
    };
    auto before = [&](int tile) {
      if (tile == p_end) flush();                          // partition p ended with tile - 1
    };
    run_tiles<Tile, D, 1>(st, qf, a.key_cache, a.value_cache, a.block_tables + (size_t)b * a.max_blocks_per_seq,
                          a.num_blocks, Hkv, kv, L, L - 1, tile_begin, tile_end, 1, a.scale_log2, lane, before);
    flush();                                               // the range ends with a partition's last tile
    t = unit0 + tile_end;
  }
  drain();
}

template <int NTW>
struct PrefillShape {
  static constexpr int kRowsPerWave = NTW * 16;
  static constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
};

constexpr int kPrefillNTW = 2;

template <class Tile, int D, int NTW, class OutT>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  typedef typename Tile::elem_t elem_t;
  constexpr int RWG = PrefillShape<NTW>::kRowsPerGroup;
  const int G = a.group;
  const int kv = blockIdx.x % a.num_kv_heads;
  const int tile = blockIdx.x / a.num_kv_heads;

  __shared__ int s_scan[kThreads];          // one entry per thread: locate_prefill_tile scans over them
  __shared__ int s_found[2];
  static_assert(sizeof(s_scan) / sizeof(s_scan[0]) == kThreads, "the tile locator indexes s_scan by thread");
  int local = 0;
  const int b = locate_prefill_tile(a.query_start_loc, a.num_seqs, G, RWG, tile, s_scan, s_found, &local);
  if (b < 0) return;
  const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
  const int q_len = q1 - q0;
  if (q1 > a.num_tokens || q0 < 0) return;
  const int L = clamp_len(a.seq_lens[b], a.max_blocks_per_seq, Tile::kBS);
  const int prior = L - q_len;
  if (a.causal && prior < 0) return;
  // last key visible to new token j (causal), or every key (cross-attention)
  auto last_key = [&](int j) { return a.causal ? prior + j : L - 1; };
  const int rows_total = q_len * G;
  const int n_row_tiles = (rows_total + RWG - 1) / RWG;
  // heaviest row tile (most keys) of the sequence first
  const int rt = n_row_tiles - 1 - local;

  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15, q = lane >> 4;
  const int r0 = rt * RWG + w * (NTW * 16);
  if (r0 >= rows_total) return;          // no barriers below

  typename Tile::Q qf[NTW];
  int lim[NTW];
  int tok[NTW], head[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = r0 + nt * 16 + n;
    const bool valid = r < rows_total;
    const int j = r / G, g = r % G;
    lim[nt] = valid ? last_key(j) : -1;
    tok[nt] = valid ? q0 + j : -1;
    head[nt] = kv * G + g;
    const elem_t* qrow = valid ? reinterpret_cast<const elem_t*>(a.query) + ((size_t)tok[nt] * a.num_heads + head[nt]) * D
                               : nullptr;
    Tile::load_q(qf[nt], qrow, lane);
  }
  const int lim_lo = last_key(r0 / G);                                   // first row of the wave
  const int lim_hi = last_key(min(q_len - 1, (r0 + NTW * 16 - 1) / G));  // last row of the wave
  const int n_tiles = (lim_hi + 1 + kTile - 1) / kTile;                  // 0 when no key is visible
  const int npages = (L + Tile::kBS - 1) / Tile::kBS;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;

  float m[NTW], l[NTW];
  f32x4_t o[NTW][Tile::DT];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < Tile::DT; ++dt) o[nt][dt] = zero4();
  }

  for (int it = 0; it < n_tiles; ++it) {
    const int tb = it * kTile;
    TilePages<Tile, D> pg;
    pg.fetch(bt, it, npages, a.num_blocks);
    typename Tile::K kf;
    typename Tile::V vf;
    load_tile<Tile, D>(kf, vf, pg, a.key_cache, a.value_cache, a.num_kv_heads, kv, lane);
    const bool masked = tb + kTile - 1 > lim_lo;
    if (tb + kTile > L) Tile::mask_v(vf, tb, L, lane);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      float s[8];
      Tile::qk(s, kf, qf[nt]);
      softmax_pv<Tile>(s, m[nt], l[nt], o[nt], vf, a.scale_log2, masked, tb, lim[nt], q);
    }
  }

  OutT* out = reinterpret_cast<OutT*>(a.out);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float lr = row_sum4(l[nt]);
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    if (tok[nt] >= 0) {
      OutT* dst = out + ((size_t)tok[nt] * a.num_heads + head[nt]) * D + 4 * q;
#pragma unroll
      for (int dt = 0; dt < Tile::DT; ++dt) store4(dst + dt * 16, o[nt][dt] * inv);
    }
  }
}

template <class Tile, int D, class OutT>
hipError_t decode_dispatch_nt(const DecodeArgs& a, int num_seqs, hipStream_t stream) {
  dim3 grid(a.max_partitions, a.num_kv_heads, num_seqs);
  if (a.group > 16) return launch_kernel(decode_kernel<Tile, D, 2, OutT, kWaves>, grid, dim3(kThreads), 0, stream, a);
  if (a.waves == 2 * kWaves)
    return launch_kernel(decode_kernel<Tile, D, 1, OutT, 2 * kWaves>, grid, dim3(2 * kThreads), 0, stream, a);
  return launch_kernel(decode_kernel<Tile, D, 1, OutT, kWaves>, grid, dim3(kThreads), 0, stream, a);
}

// Call f(Tile type tag, head dim tag) for the cache dtype, head_dim and page
// size; bf16 tiles with non-temporal K/V loads when `stream_kv`.
template <class F>
auto with_tile(int D, int block_size, bool kv_f32, bool stream_kv, F f) {
  return with_block_size(block_size, [&](auto bs) {
    constexpr int BS = decltype(bs)::value;
    if (kv_f32)
      return D == 64 ? f(TileF32<64, BS>{}, std::integral_constant<int, 64>{})
                     : f(TileF32<128, BS>{}, std::integral_constant<int, 128>{});
    if (stream_kv)
      return D == 64 ? f(TileBF16<64, BS, true>{}, std::integral_constant<int, 64>{})
                     : f(TileBF16<128, BS, true>{}, std::integral_constant<int, 128>{});
    return D == 64 ? f(TileBF16<64, BS, false>{}, std::integral_constant<int, 64>{})
                   : f(TileBF16<128, BS, false>{}, std::integral_constant<int, 128>{});
  });
}

// Resolve the stream-decode instantiation for (D, page size, dtype, out dtype,
// group) and hand it to `f`.
template <class F>
auto with_stream_kernel(int D, int block_size, bool kv_f32, bool out_f32, int group, bool stream_kv, F f) {
  typedef void (*K)(StreamArgs);
  K k = with_tile(D, block_size, kv_f32, stream_kv, [&](auto tile, auto dd) {
    typedef decltype(tile) Tile;
    constexpr int DD = decltype(dd)::value;
    if (group <= 16)
      return out_f32 ? (K)stream_decode_kernel<Tile, DD, 1, float> : (K)stream_decode_kernel<Tile, DD, 1, uint16_t>;
    return out_f32 ? (K)stream_decode_kernel<Tile, DD, 2, float> : (K)stream_decode_kernel<Tile, DD, 2, uint16_t>;
  });
  return f(k);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32, int num_seqs,
                         bool stream_kv, hipStream_t stream) {
  return with_tile(head_dim, block_size, kv_f32, stream_kv, [&](auto tile, auto dd) {
    typedef decltype(tile) Tile;
    constexpr int DD = decltype(dd)::value;
    return out_f32 ? decode_dispatch_nt<Tile, DD, float>(a, num_seqs, stream)
                   : decode_dispatch_nt<Tile, DD, uint16_t>(a, num_seqs, stream);
  });
}

int prefill_rows_per_group() { return PrefillShape<kPrefillNTW>::kRowsPerGroup; }

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32,
                          int grid_groups, hipStream_t stream) {
  // chunks re-read their keys across row tiles: plain loads
  return with_tile(head_dim, block_size, kv_f32, false, [&](auto tile, auto dd) {
    typedef decltype(tile) Tile;
    constexpr int DD = decltype(dd)::value;
    if (out_f32)
      return launch_kernel(prefill_kernel<Tile, DD, kPrefillNTW, float>, dim3(grid_groups), dim3(kThreads), 0,
                           stream, a);
    return launch_kernel(prefill_kernel<Tile, DD, kPrefillNTW, uint16_t>, dim3(grid_groups), dim3(kThreads), 0,
                         stream, a);
  });
}

// Resident waves of a persistent decode kernel: compute units x resident
// work-groups per compute unit x 4 waves.  The compute-unit count and the
// kernel's occupancy are queried once per (device, kernel, 1 KiB step of its
// dynamic LDS) and cached: workspace queries and decode calls then make no
// runtime query beyond hipGetDevice.  The occupancy is taken at the top of the
// LDS step, so it never exceeds what the launch's actual LDS allows.
int resident_workers(const void* kernel, size_t lds_bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  const size_t lds_step = (lds_bytes + 1023) / 1024;
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  const auto key = std::make_tuple(dev, kernel, lds_step);
  {
    std::lock_guard<std::mutex> lock(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int cus = 256, per_cu = 2;
  if (dev >= 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kThreads, lds_step * 1024) == hipSuccess &&
        blocks > 0)
      per_cu = blocks;
  }
  const int workers = cus * per_cu * kWaves;
  std::lock_guard<std::mutex> lock(mu);
  cache[key] = workers;
  return workers;
}

// Both cache-policy instantiations of a kernel use the same registers and LDS
// (they differ only in the hint bits of the loads), so the counts come from
// the streaming one.
int stream_workers(int head_dim, int block_size, bool kv_f32, bool out_f32, int group, int num_seqs) {
  void (*kernel)(StreamArgs) = with_stream_kernel(head_dim, block_size, kv_f32, out_f32, group, true,
                                                  [](void (*k)(StreamArgs)) { return k; });
  return resident_workers(reinterpret_cast<const void*>(kernel), (size_t)(2 * num_seqs + 1) * sizeof(int));
}

// The partitioned balanced decode's instantiation for (D, page size, dtype, out dtype).
void (*partition_kernel(int head_dim, int block_size, bool kv_f32, bool out_f32, bool stream_kv))(StreamPartArgs) {
  typedef void (*K)(StreamPartArgs);
  return with_tile(head_dim, block_size, kv_f32, stream_kv, [&](auto tile, auto dd) {
    typedef decltype(tile) Tile;
    constexpr int DD = decltype(dd)::value;
    return out_f32 ? (K)stream_partition_kernel<Tile, DD, float> : (K)stream_partition_kernel<Tile, DD, uint16_t>;
  });
}

int partition_workers(int head_dim, int block_size, bool kv_f32, bool out_f32, int num_seqs) {
  return resident_workers(reinterpret_cast<const void*>(partition_kernel(head_dim, block_size, kv_f32, out_f32, true)),
                          (size_t)(2 * num_seqs + 1) * sizeof(int));
}

hipError_t launch_stream_partition(const StreamPartArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32,
                                   bool stream_kv, hipStream_t stream) {
  const size_t lds = (size_t)(2 * a.num_seqs + 1) * sizeof(int);
  return launch_kernel(partition_kernel(head_dim, block_size, kv_f32, out_f32, stream_kv), dim3(a.num_workers / kWaves),
                       dim3(kThreads), lds, stream, a);
}

hipError_t launch_stream_decode(const StreamArgs& a, int head_dim, int block_size, bool kv_f32, bool out_f32,
                                bool stream_kv, hipStream_t stream) {
  const size_t lds = (size_t)(2 * a.num_seqs + 1) * sizeof(int);
  const dim3 grid(a.num_workers / kWaves), block(kThreads);
  return with_stream_kernel(head_dim, block_size, kv_f32, out_f32, a.group, stream_kv, [&](void (*k)(StreamArgs)) {
    return launch_kernel(k, grid, block, lds, stream, a);
  });
}

template <class InT>
hipError_t reduce_dispatch(const StreamArgs& a, int head_dim, bool out_f32, hipStream_t stream) {
  const dim3 grid(a.num_kv_heads * a.num_seqs, a.group);
  if (head_dim == 64)
    return out_f32 ? launch_kernel(stream_reduce_kernel<64, float, InT>, grid, dim3(64), 0, stream, a)
                   : launch_kernel(stream_reduce_kernel<64, uint16_t, InT>, grid, dim3(64), 0, stream, a);
  return out_f32 ? launch_kernel(stream_reduce_kernel<128, float, InT>, grid, dim3(128), 0, stream, a)
                 : launch_kernel(stream_reduce_kernel<128, uint16_t, InT>, grid, dim3(128), 0, stream, a);
}

hipError_t launch_stream_reduce(const StreamArgs& a, int head_dim, bool kv_f32, bool out_f32, hipStream_t stream) {
  return kv_f32 ? reduce_dispatch<float>(a, head_dim, out_f32, stream)
                : reduce_dispatch<uint16_t>(a, head_dim, out_f32, stream);
}

}  // namespace gqa
