// Decode building blocks shared by the decode kernels and the fused
// mixed-batch kernel: per-wave tile pipeline (page lookup, K/V loads, Q.K^T,
// online softmax, P.V) and the fixed-partition decode of one (sequence, kv
// head) by a 4-wave work-group.
//
// Every work item reads each (sequence, kv head) K/V page once and shares it
// across the G query heads of the group, as "[Performance] Use optimized
// kernels for MQA/GQA" (vLLM issue #1880, opening post) asks of a GQA-aware
// kernel, instead of expanding K/V per query head.
#pragma once

#include "gqa_common.h"
#include "gqa_internal.h"
#include "tile_schedule.h"

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// Base of page `page`, kv head kv, in a cache of BS-token pages.
template <class T, int BS>
__device__ __forceinline__ const T* page_ptr(const void* cache, int page, int num_kv_heads, int kv, int D) {
  return reinterpret_cast<const T*>(cache) + ((size_t)page * num_kv_heads + kv) * (size_t)(BS * D);
}

// One online-softmax + P.V step for a 16-row block.  `s` holds the block's 8
// raw scores of this lane (tile-relative tokens Tile::token_offset(q, idx));
// `lim` is the last visible key position of this lane's row (inclusive) and is
// applied only when `masked`.
template <class Tile>
__device__ __forceinline__ void softmax_pv(float s[8], float& m, float& l, f32x4_t* o, const typename Tile::V& vf,
                                           float scale_log2, bool masked, int tile_base, int lim, int q) {
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x = s[i] * scale_log2;
    if (masked) x = (tile_base + Tile::token_offset(q, i) <= lim) ? x : -INFINITY;
    s[i] = x;
    mx = fmaxf(mx, x);
  }
  mx = row_max4(mx);
  const float m_new = fmaxf(m, mx);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = fast_exp2(m - m_use);
  float rs = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s[i] = fast_exp2(s[i] - m_use);
    rs += s[i];
  }
  l = l * alpha + rs;
  m = m_new;
#pragma unroll
  for (int dt = 0; dt < Tile::DT; ++dt) o[dt] *= alpha;
  Tile::pv(o, vf, s);
}

// Running softmax state of one wave for NT blocks of 16 rows.
template <class Tile, int NT>
struct WaveState {
  float m[NT], l[NT];
  f32x4_t o[NT][Tile::DT];
  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m[nt] = -INFINITY;
      l[nt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < Tile::DT; ++dt) o[nt][dt] = zero4();
    }
  }
};

// Decode rows of one (sequence, kv head) for this wave: G heads in NT blocks.
template <class Tile, int D, int NT>
__device__ __forceinline__ void load_group_query(typename Tile::Q qf[NT], const void* query, int row, int num_heads,
                                                 int kv, int G, int lane) {
  typedef typename Tile::elem_t elem_t;
  const int n = lane & 15;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int g = nt * 16 + n;
    const elem_t* qrow =
        (g < G) ? reinterpret_cast<const elem_t*>(query) + ((size_t)row * num_heads + kv * G + g) * D : nullptr;
    Tile::load_q(qf[nt], qrow, lane);
  }
}

// Pages of tile `it`: with 16-token pages the two halves are pages 2 it and
// 2 it + 1 (the second clamped to the last page); with 32- or 64-token pages
// both halves sit in page 32 it / BS, from token (32 it) mod BS on.
template <class Tile, int D>
struct TilePages {
  static constexpr int BS = Tile::kBS;
  int pA, pB;
  int off;                                  // in-page token of the tile's first key (BS > 16)
  __device__ __forceinline__ void fetch(const int32_t* bt, int it, int npages, int num_blocks) {
    if constexpr (BS == kHalf) {
      pA = page_at(bt, 2 * it, num_blocks);
      pB = page_at(bt, min(2 * it + 1, npages - 1), num_blocks);
      off = 0;
    } else {
      pA = pB = page_at(bt, it * kTile / BS, num_blocks);
      off = it * kTile % BS;
    }
  }
};

template <class Tile, int D>
__device__ __forceinline__ void load_tile(typename Tile::K& kf, typename Tile::V& vf, const TilePages<Tile, D>& pg,
                                          const void* kc, const void* vc, int num_kv_heads, int kv, int lane) {
  typedef typename Tile::elem_t elem_t;
  constexpr int BS = Tile::kBS;
  const elem_t* kA = page_ptr<elem_t, BS>(kc, pg.pA, num_kv_heads, kv, D);
  const elem_t* vA = page_ptr<elem_t, BS>(vc, pg.pA, num_kv_heads, kv, D);
  if constexpr (BS == kHalf) {
    Tile::load_k(kf, kA, page_ptr<elem_t, BS>(kc, pg.pB, num_kv_heads, kv, D), lane);
    Tile::load_v(vf, vA, page_ptr<elem_t, BS>(vc, pg.pB, num_kv_heads, kv, D), lane);
  } else {
    kA += pg.off * D;
    vA += pg.off;
    Tile::load_k(kf, kA, kA + kHalf * D, lane);
    Tile::load_v(vf, vA, vA + kHalf, lane);
  }
}

template <class Tile, int NT>
__device__ __forceinline__ void compute_tile(WaveState<Tile, NT>& st, const typename Tile::Q qf[NT],
                                             const typename Tile::K& kf, typename Tile::V& vf, int tb, int L, int lim,
                                             float scale_log2, int lane) {
  const int q = lane >> 4;
  const bool masked = tb + kTile - 1 > lim;
  if (tb + kTile > L) Tile::mask_v(vf, tb, L, lane);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float s[8];
    Tile::qk(s, kf, qf[nt]);
    softmax_pv<Tile>(s, st.m[nt], st.l[nt], st.o[nt], vf, scale_log2, masked, tb, lim, q);
  }
}

// Walk tiles it0, it0+step, ... < it1 of one (sequence, kv head); tile i covers
// keys [32 i, 32 i + 32).  Keys past `lim` are masked; values of tokens at or
// past L are zeroed so that whatever sits in the pool beyond the sequence
// (including NaN) cannot reach the output.
//
// The visiting order is tile_schedule's (tile_schedule.h, checked on the host
// for every range a work-group produces).  Pipelined tiles use two register
// sets (A, B): a wave that walks consecutive tiles (step 1) loads them in
// pairs, then computes both, so it has 64 tokens of K and V in flight at once
// (with 64-token pages the pair is one page and the two halves of every value
// line are requested together; one tile at a time, L2 evicted most lines
// before the second half was asked for: +34% HBM reads).  Otherwise (tiles
// shared round-robin by the waves of a work-group) the sets alternate: the
// loads of the next tile are issued before the current tile is computed.
// Prefetches past the last tile repeat it (its re-read hits in cache), which
// keeps the load count per round fixed and lets the compiler wait on just the
// tile about to be computed.  Register and page-set indices are literals at
// every call of the callbacks, so the selects below fold away.  `before(tile)`
// runs just before each tile is computed, in tile order, after that tile's
// loads were issued: the partitioned decode writes the previous partition's
// partial there, so that the next wait on a load does not also wait for those
// stores (loads and stores complete in order on one counter).
struct NoBefore {
  __device__ __forceinline__ void operator()(int) const {}
};

template <class Tile, int D, int NT, class Before = NoBefore>
__device__ __forceinline__ void run_tiles(WaveState<Tile, NT>& st, const typename Tile::Q qf[NT], const void* kc,
                                          const void* vc, const int32_t* bt, int num_blocks, int num_kv_heads, int kv,
                                          int L, int lim, int it0, int it1, int step, float scale_log2, int lane,
                                          Before before = Before()) {
  if (it0 >= it1) return;
  // at least one page: a fused append walks the tile of its only key with L = 0
  const int npages = max(1, (L + Tile::kBS - 1) / Tile::kBS);
  typename Tile::K kA, kB;
  typename Tile::V vA, vB;
  TilePages<Tile, D> pa, pb;
  auto fetch = [&](int p, int tile) __attribute__((always_inline)) {
    (p == 0 ? pa : pb).fetch(bt, tile, npages, num_blocks);
  };
  auto load = [&](int r, int p) __attribute__((always_inline)) {
    load_tile<Tile, D>(r == 0 ? kA : kB, r == 0 ? vA : vB, p == 0 ? pa : pb, kc, vc, num_kv_heads, kv, lane);
  };
  auto compute = [&](int r, int tile) __attribute__((always_inline)) {
    before(tile);
    compute_tile<Tile, NT>(st, qf, r == 0 ? kA : kB, r == 0 ? vA : vB, tile * kTile, L, lim, scale_log2, lane);
  };
  tile_schedule(it0, it1, step, Tile::kPipelined ? kPaired : kSingle, fetch, load, compute);
}

// Clamp a sequence length into what the block table can address.
__device__ __forceinline__ int clamp_len(int L, int max_blocks_per_seq, int block_size) {
  return max(0, min(L, max_blocks_per_seq * block_size));
}

// ---------------------------------------------------------------------------
// Fixed-partition decode: grid (max_partitions, Hkv, B), W waves (4, or 8 when
// the grid holds at most one work-group per compute unit).  Sequence b is
// split into n = ceil(L / partition_size) partitions of nearly equal length
// (whole 32-token tiles); the work-group owns partition p of one (sequence, kv
// head), its waves share the partition's tiles and merge through LDS.  With
// n == 1 the work-group writes `out`; otherwise it writes the partition's
// normalised output and log-sum-exp for the split-K reduce kernel.
// ---------------------------------------------------------------------------
// Waves per SIMD the decode kernels are compiled for: two when a double-buffered
// K/V tile (2 x 2 x 32 tokens x D x elem bytes per wave) fits next to one row
// block's state, else one.
template <class Tile, int D, int NT>
constexpr int decode_waves_per_simd() {
  return (NT == 1 && (sizeof(typename Tile::elem_t) * D <= 256 || !Tile::kPipelined)) ? 2 : 1;
}

// LDS the merge of the W waves needs (floats): per wave, R row maxima, R row
// sums and an R x (D + 4) output block.
template <int D, int NT, int W = kWaves>
struct DecodeMergeLds {
  static constexpr int R = NT * 16;
  static constexpr int kFloats = W * R * (2 + D + 4);
};

// Where a unit that covers part of a row's keys writes: each row's
// normalised partial output and its natural-log log-sum-exp, in slot `slot`
// (plus the unit's partition index, for decode partitions) of `slots` per
// (row, head).
struct UnitOut {
  float* part_out = nullptr;               // [rows, Hq, slots, D]
  float* part_lse = nullptr;               // [rows, Hq, slots]
  int slot = 0, slots = 1;
};

// Partition p of (sequence b, kv head kv), run by the W waves of a work-group,
// for query row `row` and seq_lens[b] = seq_len; `lds` holds
// DecodeMergeLds<D, NT, W>::kFloats floats.  Partitions cover keys [k_begin, L)
// (k_begin a multiple of 32).  With `uo`, every partition writes a partial to
// uo's slots; otherwise a single partition writes `out` and several write
// a.partial_out / a.partial_lse.
template <class Tile, int D, int NT, class OutT, int W = kWaves>
__device__ __forceinline__ void decode_partition_at(const DecodeArgs& a, int p, int kv, int b, int row, int seq_len,
                                                    float* lds, int k_begin = 0, const UnitOut* uo = nullptr) {
  constexpr int R = NT * 16;            // padded rows of the group
  const int G = a.group;
  constexpr int kT = W * kWave;    // threads of the work-group
  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15, q = lane >> 4;

  typename Tile::Q qf[NT];
  load_group_query<Tile, D, NT>(qf, a.query, row, a.num_heads, kv, G, lane);

  const int L = min(clamp_len(seq_len, a.max_blocks_per_seq, Tile::kBS), k_begin + a.max_partitions * a.partition_size);
  const int nparts = L > k_begin ? (L - k_begin + a.partition_size - 1) / a.partition_size : 0;
  OutT* out = reinterpret_cast<OutT*>(a.out);

  if (nparts == 0) {
    if (p == 0 && !uo)
      for (int i = threadIdx.x; i < G * D / 4; i += kT)
        store4(out + ((size_t)row * a.num_heads + kv * G) * D + 4 * i, zero4());
    return;
  }
  if (p >= nparts) return;

  // equal split of the range's tiles over its partitions (each gets >= 1 tile)
  const int tiles_all = (L - k_begin + kTile - 1) / kTile;
  const int per = tiles_all / nparts, extra = tiles_all % nparts;
  const int tile0 = k_begin / kTile + p * per + min(p, extra);
  const int n_tiles = per + (p < extra ? 1 : 0);
  const int t1 = min((tile0 + n_tiles) * kTile, L);

  WaveState<Tile, NT> st;
  st.reset();
  if constexpr (NT == 1) {
    // each wave a contiguous share (1 / W) of the partition's tiles, walked in pairs
    // (two tiles per round trip); measured faster than round-robin tiles for
    // G <= 16 (Llama-3.1-8B shapes at 512-token partitions 148.8 -> 141.3 us)
    const int wper = n_tiles / W, wextra = n_tiles % W;
    const int wb = tile0 + w * wper + min(w, wextra);
    const int we = wb + wper + (w < wextra ? 1 : 0);
    run_tiles<Tile, D, NT>(st, qf, a.key_cache, a.value_cache, a.block_tables + (size_t)b * a.max_blocks_per_seq,
                           a.num_blocks, a.num_kv_heads / a.kv_split, kv / a.kv_split, L, t1 - 1, wb, we, 1,
                           a.scale_log2, lane);
  } else {
    // two row blocks per wave (G > 16): tiles round-robin over the waves, which
    // was faster there (MQA, G = 32: 19.4 vs 20.5 us)
    run_tiles<Tile, D, NT>(st, qf, a.key_cache, a.value_cache, a.block_tables + (size_t)b * a.max_blocks_per_seq,
                           a.num_blocks, a.num_kv_heads / a.kv_split, kv / a.kv_split, L, t1 - 1, tile0 + w,
                           tile0 + n_tiles, W, a.scale_log2, lane);
  }

  // ---- merge the W waves ----
  float (*sm_m)[R] = reinterpret_cast<float (*)[R]>(lds);
  float (*sm_l)[R] = reinterpret_cast<float (*)[R]>(lds + W * R);
  float (*sm_o)[R][D + 4] = reinterpret_cast<float (*)[R][D + 4]>(lds + 2 * W * R);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lr = row_sum4(st.l[nt]);
    if (q == 0) {
      sm_m[w][nt * 16 + n] = st.m[nt];
      sm_l[w][nt * 16 + n] = lr;
    }
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int r = nt * 16 + n;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; ++v) M = fmaxf(M, sm_m[v][r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) Ls += sm_l[v][r] * fast_exp2(sm_m[v][r] - Mu);
    const float f = (Ls > 0.f) ? fast_exp2(st.m[nt] - Mu) / Ls : 0.f;
    if (r < G) {
#pragma unroll
      for (int dt = 0; dt < Tile::DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) sm_o[w][r][dt * 16 + 4 * q + j] = st.o[nt][dt][j] * f;
    }
  }
  __syncthreads();

  const size_t head0 = (size_t)b * a.num_heads + kv * G;
  // partial slot of row r: [(head0 + r) * stride + slot]
  const bool partial = uo || nparts > 1;
  float* part_out = uo ? uo->part_out : a.partial_out;
  float* part_lse = uo ? uo->part_lse : a.partial_lse;
  const int stride = uo ? uo->slots : a.max_partitions;
  const int slot = uo ? uo->slot + p : p;
  // four channels per thread: 16-byte LDS reads (rows of D + 4 floats stay
  // 16-byte aligned), 16-byte fp32 or 8-byte bf16 stores
  for (int i = threadIdx.x; i < G * D / 4; i += kT) {
    const int r = 4 * i / D, d = 4 * i % D;
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(&sm_o[0][r][d]);
#pragma unroll
    for (int u = 1; u < W; ++u) v += *reinterpret_cast<const f32x4_t*>(&sm_o[u][r][d]);
    if (!partial)
      store4(out + ((size_t)row * a.num_heads + kv * G + r) * D + d, v);
    else
      store4(part_out + ((head0 + r) * stride + slot) * D + d, v);
  }
  if (partial && threadIdx.x < G) {
    const int r = threadIdx.x;
    float M = -INFINITY;
    for (int v = 0; v < W; ++v) M = fmaxf(M, sm_m[v][r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
    for (int v = 0; v < W; ++v) Ls += sm_l[v][r] * fast_exp2(sm_m[v][r] - Mu);
    part_lse[(head0 + r) * stride + slot] = (Ls > 0.f) ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
  }
}

// Partition p of (sequence b, kv head kv) run by this wave alone, for query
// row `row` and seq_lens[b] = seq_len: the same split into partitions as
// decode_partition_at, its tiles walked in pairs by the wave's own pipeline,
// and no merge between waves.  It writes `out` when the sequence has one
// partition, else the partition's normalised partial and log-sum-exp.
template <class Tile, int D, int NT, class OutT>
__device__ __forceinline__ void decode_wave_partition(const DecodeArgs& a, int p, int kv, int b, int row,
                                                      int seq_len) {
  const int G = a.group;
  const int lane = lane_id();
  const int n = lane & 15, q = lane >> 4;
  OutT* out = reinterpret_cast<OutT*>(a.out);
  const int L = min(clamp_len(seq_len, a.max_blocks_per_seq, Tile::kBS), a.max_partitions * a.partition_size);
  const int nparts = L > 0 ? (L + a.partition_size - 1) / a.partition_size : 0;
  if (nparts == 0) {
    if (p == 0)
      for (int i = lane; i < G * D / 4; i += kWave)
        store4(out + ((size_t)row * a.num_heads + kv * G) * D + 4 * i, zero4());
    return;
  }
  if (p >= nparts) return;
  const int tiles_all = (L + kTile - 1) / kTile;
  const int per = tiles_all / nparts, extra = tiles_all % nparts;
  const int tile0 = p * per + min(p, extra);
  const int n_tiles = per + (p < extra ? 1 : 0);
  const int t1 = min((tile0 + n_tiles) * kTile, L);

  typename Tile::Q qf[NT];
  load_group_query<Tile, D, NT>(qf, a.query, row, a.num_heads, kv, G, lane);
  WaveState<Tile, NT> st;
  st.reset();
  run_tiles<Tile, D, NT>(st, qf, a.key_cache, a.value_cache, a.block_tables + (size_t)b * a.max_blocks_per_seq,
                         a.num_blocks, a.num_kv_heads / a.kv_split, kv / a.kv_split, L, t1 - 1, tile0, tile0 + n_tiles,
                         1, a.scale_log2, lane);

  const size_t head0 = (size_t)b * a.num_heads + kv * G;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int g = nt * 16 + n;
    const float lr = row_sum4(st.l[nt]);
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    if (g >= G) continue;
    if (nparts == 1) {
      OutT* dst = out + ((size_t)row * a.num_heads + kv * G + g) * D + 4 * q;
#pragma unroll
      for (int dt = 0; dt < Tile::DT; ++dt) store4(dst + dt * 16, st.o[nt][dt] * inv);
    } else {
      float* dst = a.partial_out + ((head0 + g) * a.max_partitions + p) * D + 4 * q;
#pragma unroll
      for (int dt = 0; dt < Tile::DT; ++dt) store4(dst + dt * 16, st.o[nt][dt] * inv);
      if (q == 0)
        a.partial_lse[(head0 + g) * a.max_partitions + p] = lr > 0.f ? (st.m[nt] + __log2f(lr)) * kLn2 : -INFINITY;
    }
  }
}

// As decode_partition_at, reading the query row (sequence b's only new token
// when query_start_loc is given, else row b) and seq_lens[b] itself.
template <class Tile, int D, int NT, class OutT, int W = kWaves>
__device__ __forceinline__ void decode_partition(const DecodeArgs& a, int p, int kv, int b, float* lds) {
  int row = b;
  if (a.query_start_loc) {
    const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
    if (q1 - q0 != 1 || q1 > a.num_tokens || q0 < 0) return;
    row = q0;
  }
  decode_partition_at<Tile, D, NT, OutT, W>(a, p, kv, b, row, a.seq_lens[b], lds);
}

}  // namespace

}  // namespace gqa
