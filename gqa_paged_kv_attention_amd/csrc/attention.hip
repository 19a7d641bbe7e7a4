// Paged GQA attention kernels for gfx950: decode (fixed split-K partitions or
// a balanced persistent split) and chunked prefill.
//
// All kernels read each (sequence, kv head) K/V page once per work item and
// share it across the G query heads of the group, as "[Performance] Use
// optimized kernels for MQA/GQA" (vLLM issue #1880, opening post) asks of a
// GQA-aware kernel, instead of expanding K/V per query head.  The G heads (and
// for prefill, the chunk's new tokens times G) form the 16-wide column block of
// the matrix-core products described in gqa_common.h.
#include "gqa_common.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

template <class T>
__device__ __forceinline__ const T* page_ptr(const void* cache, int page, int num_kv_heads, int kv, int D) {
  return reinterpret_cast<const T*>(cache) + ((size_t)page * num_kv_heads + kv) * (size_t)(kPage * D);
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

// Walk tiles it0, it0+step, ... < it1 of one (sequence, kv head); tile i covers
// keys [32 i, 32 i + 32).  Keys past `lim` are masked; values of tokens at or
// past L are zeroed so that whatever sits in the pool beyond the sequence
// (including NaN) cannot reach the output.
//
// Software pipelining: two register sets (A, B) alternate, and the loads of
// the next tile are issued before the current tile is computed, so a wave
// always has a tile in flight.  The prefetch is unconditional (its tile index
// is clamped to the last tile, whose re-read hits in cache), which keeps the
// load count per iteration fixed and lets the compiler wait on just the
// current tile's loads.
template <class Tile, int D>
struct TilePages {
  int pA, pB;
  __device__ __forceinline__ void fetch(const int32_t* bt, int it, int npages, int num_blocks) {
    const int pg = it * (kTile / kPage);
    pA = page_at(bt, pg, num_blocks);
    pB = page_at(bt, min(pg + 1, npages - 1), num_blocks);
  }
};

template <class Tile, int D>
__device__ __forceinline__ void load_tile(typename Tile::K& kf, typename Tile::V& vf, const TilePages<Tile, D>& pg,
                                          const void* kc, const void* vc, int num_kv_heads, int kv, int lane) {
  typedef typename Tile::elem_t elem_t;
  Tile::load_k(kf, page_ptr<elem_t>(kc, pg.pA, num_kv_heads, kv, D), page_ptr<elem_t>(kc, pg.pB, num_kv_heads, kv, D),
               lane);
  Tile::load_v(vf, page_ptr<elem_t>(vc, pg.pA, num_kv_heads, kv, D), page_ptr<elem_t>(vc, pg.pB, num_kv_heads, kv, D),
               lane);
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

template <class Tile, int D, int NT>
__device__ __forceinline__ void run_tiles(WaveState<Tile, NT>& st, const typename Tile::Q qf[NT], const void* kc,
                                          const void* vc, const int32_t* bt, int num_blocks, int num_kv_heads, int kv,
                                          int L, int lim, int it0, int it1, int step, float scale_log2, int lane) {
  if (it0 >= it1) return;
  const int npages = (L + kPage - 1) / kPage;
  if constexpr (!Tile::kPipelined) {
    for (int it = it0; it < it1; it += step) {
      typename Tile::K kf;
      typename Tile::V vf;
      TilePages<Tile, D> pg;
      pg.fetch(bt, it, npages, num_blocks);
      load_tile<Tile, D>(kf, vf, pg, kc, vc, num_kv_heads, kv, lane);
      compute_tile<Tile, NT>(st, qf, kf, vf, it * kTile, L, lim, scale_log2, lane);
    }
    return;
  }
  const int last = it0 + (it1 - 1 - it0) / step * step;     // last tile this wave visits
  typename Tile::K kA, kB;
  typename Tile::V vA, vB;
  TilePages<Tile, D> pg;
  pg.fetch(bt, it0, npages, num_blocks);
  load_tile<Tile, D>(kA, vA, pg, kc, vc, num_kv_heads, kv, lane);
  pg.fetch(bt, min(it0 + step, last), npages, num_blocks);
  for (int it = it0;; it += 2 * step) {
    // B <- tile it + step (clamped), then compute A = tile it
    load_tile<Tile, D>(kB, vB, pg, kc, vc, num_kv_heads, kv, lane);
    pg.fetch(bt, min(it + 2 * step, last), npages, num_blocks);
    compute_tile<Tile, NT>(st, qf, kA, vA, it * kTile, L, lim, scale_log2, lane);
    if (it + step > last) break;
    // A <- tile it + 2 step (clamped), then compute B = tile it + step
    load_tile<Tile, D>(kA, vA, pg, kc, vc, num_kv_heads, kv, lane);
    pg.fetch(bt, min(it + 3 * step, last), npages, num_blocks);
    compute_tile<Tile, NT>(st, qf, kB, vB, (it + step) * kTile, L, lim, scale_log2, lane);
    if (it + 2 * step > last) break;
  }
}

// Clamp a sequence length into what the block table can address.
__device__ __forceinline__ int clamp_len(int L, int max_blocks_per_seq) {
  return max(0, min(L, max_blocks_per_seq * kPage));
}

// ---------------------------------------------------------------------------
// Fixed-partition decode: grid (max_partitions, Hkv, B), 4 waves.  Sequence b
// is split into n = ceil(L / partition_size) partitions of nearly equal length
// (whole 32-token tiles); the work-group owns partition p of one (sequence, kv
// head), its waves take the partition's tiles round-robin and merge through
// LDS.  With n == 1 the work-group writes `out`; otherwise it writes the
// partition's normalised output and log-sum-exp for the split-K reduce kernel.
// ---------------------------------------------------------------------------
// Waves per SIMD the decode kernels are compiled for: two when a double-buffered
// K/V tile (2 x 2 x 32 tokens x D x elem bytes per wave) fits next to one row
// block's state, else one.
template <class Tile, int D, int NT>
constexpr int decode_waves_per_simd() {
  return (NT == 1 && (sizeof(typename Tile::elem_t) * D <= 256 || !Tile::kPipelined)) ? 2 : 1;
}

template <class Tile, int D, int NT, class OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<Tile, D, NT>())))
void decode_kernel(DecodeArgs a) {
  constexpr int R = NT * 16;            // padded rows of the group
  const int p = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15, q = lane >> 4;

  int row = b;
  if (a.query_start_loc) {
    const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
    if (q1 - q0 != 1 || q1 > a.num_tokens || q0 < 0) return;
    row = q0;
  }
  typename Tile::Q qf[NT];
  load_group_query<Tile, D, NT>(qf, a.query, row, a.num_heads, kv, G, lane);

  const int L = min(clamp_len(a.seq_lens[b], a.max_blocks_per_seq), a.max_partitions * a.partition_size);
  const int nparts = (L + a.partition_size - 1) / a.partition_size;
  OutT* out = reinterpret_cast<OutT*>(a.out);

  if (L == 0) {
    if (p == 0)
      for (int i = threadIdx.x; i < G * D; i += kThreads)
        store1(out + ((size_t)row * a.num_heads + kv * G) * D + i, 0.f);
    return;
  }
  if (p >= nparts) return;

  // equal split of the sequence's tiles over its partitions (each gets >= 1 tile)
  const int tiles_all = (L + kTile - 1) / kTile;
  const int per = tiles_all / nparts, extra = tiles_all % nparts;
  const int tile0 = p * per + min(p, extra);
  const int n_tiles = per + (p < extra ? 1 : 0);
  const int t1 = min((tile0 + n_tiles) * kTile, L);

  WaveState<Tile, NT> st;
  st.reset();
  run_tiles<Tile, D, NT>(st, qf, a.key_cache, a.value_cache, a.block_tables + (size_t)b * a.max_blocks_per_seq,
                         a.num_blocks, a.num_kv_heads, kv, L, t1 - 1, tile0 + w, tile0 + n_tiles, kWaves,
                         a.scale_log2, lane);

  // ---- merge the four waves ----
  __shared__ float sm_m[kWaves][R];
  __shared__ float sm_l[kWaves][R];
  __shared__ float sm_o[kWaves][R][D + 4];
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
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm_m[v][r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) Ls += sm_l[v][r] * fast_exp2(sm_m[v][r] - Mu);
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
  for (int i = threadIdx.x; i < G * D; i += kThreads) {
    const int r = i / D, d = i % D;
    const float v = sm_o[0][r][d] + sm_o[1][r][d] + sm_o[2][r][d] + sm_o[3][r][d];
    if (nparts == 1)
      store1(out + ((size_t)row * a.num_heads + kv * G + r) * D + d, v);
    else
      a.partial_out[((head0 + r) * a.max_partitions + p) * D + d] = v;
  }
  if (nparts > 1 && threadIdx.x < G) {
    const int r = threadIdx.x;
    float M = -INFINITY;
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm_m[v][r]);
    const float Mu = (M == -INFINITY) ? 0.f : M;
    float Ls = 0.f;
    for (int v = 0; v < kWaves; ++v) Ls += sm_l[v][r] * fast_exp2(sm_m[v][r] - Mu);
    a.partial_lse[(head0 + r) * a.max_partitions + p] = (Ls > 0.f) ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
  }
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

template <class Tile, int D, int NT, class OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd<Tile, D, NT>())))
void stream_decode_kernel(StreamArgs a) {
  extern __shared__ int s_pref[];          // [B + 1] exclusive prefix of tiles * Hkv
  __shared__ int s_scan[kThreads];
  const int B = a.num_seqs, G = a.group;
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
      const int L = dec ? clamp_len(a.seq_lens[b], a.max_blocks_per_seq) : 0;
      v = (L + kTile - 1) / kTile * a.num_kv_heads;
      if (dec && L == 0 && (b % gridDim.x) == (int)blockIdx.x) {
        // an empty decode sequence has a zero output row
        for (int i = 0; i < a.num_heads * D; ++i) store1(out + (size_t)row * a.num_heads * D + i, 0.f);
      }
    }
    s_scan[threadIdx.x] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int add = (threadIdx.x >= off) ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += add;
      __syncthreads();
    }
    if (b < B) s_pref[b + 1] = running + s_scan[threadIdx.x];
    running += s_scan[kThreads - 1];
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
    const int L = clamp_len(a.seq_lens[b], a.max_blocks_per_seq);

    typename Tile::Q qf[NT];
    load_group_query<Tile, D, NT>(qf, a.query, row, a.num_heads, kv, G, lane);
    WaveState<Tile, NT> st;
    st.reset();
    run_tiles<Tile, D, NT>(st, qf, a.key_cache, a.value_cache, a.block_tables + (size_t)b * a.max_blocks_per_seq,
                           a.num_blocks, a.num_kv_heads, kv, L, L - 1, tile_begin, tile_end, 1, a.scale_log2, lane);

    const bool whole = tile_begin == 0 && tile_end == nt;
    const int slot = first ? 0 : 1;
#pragma unroll
    for (int nt_ = 0; nt_ < NT; ++nt_) {
      const int g = nt_ * 16 + n;
      const float lr = row_sum4(st.l[nt_]);
      const float inv = lr > 0.f ? 1.f / lr : 0.f;
      if (g < G) {
        if (whole) {
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
// and an online log-sum-exp: two memory round trips in all.
constexpr int kMergeBatch = 8;

template <int D, class OutT>
__global__ __launch_bounds__(D) void stream_reduce_kernel(StreamArgs a) {
  const int u = blockIdx.x, g = blockIdx.y, d = threadIdx.x;
  const int4 m = a.unit_meta[u];
  const long long T = a.tile_prefix[a.num_seqs];
  const int w0 = m.x, w1 = m.y, slot0 = m.z, row = m.w;
  if (w1 <= w0) return;
  const int kv = u % a.num_kv_heads;
  const int G = a.group, W = a.num_workers;
  float M = -INFINITY, den = 0.f, acc = 0.f;
  for (int wb = w0; wb <= w1; wb += kMergeBatch) {
    float lv[kMergeBatch], ov[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int w = wb + k;
      // workers past the unit, or with an empty range (T < W), hold no segment
      const bool has = w <= w1 && T * w / W != T * (w + 1) / W;
      const size_t seg = ((size_t)w * 2 + (w == w0 ? slot0 : 0)) * G + g;
      lv[k] = has ? a.seg_lse[seg] : -INFINITY;
      ov[k] = has ? a.seg_out[seg * D + d] : 0.f;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) bm = fmaxf(bm, lv[k]);
    const float nm = fmaxf(M, bm);
    const float nu = (nm == -INFINITY) ? 0.f : nm;
    const float r = fast_exp2((M - nu) * kLog2e);
    den *= r;
    acc *= r;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float wgt = fast_exp2((lv[k] - nu) * kLog2e);
      den += wgt;
      acc += wgt == 0.f ? 0.f : wgt * ov[k];
    }
    M = nm;
  }
  OutT* out = reinterpret_cast<OutT*>(a.out);
  store1(out + ((size_t)row * a.num_heads + kv * G + g) * D + d, den > 0.f ? acc / den : 0.f);
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

  __shared__ int s_scan[kThreads];
  __shared__ int s_found[2];
  int local = 0;
  const int b = locate_prefill_tile(a.query_start_loc, a.num_seqs, G, RWG, tile, s_scan, s_found, &local);
  if (b < 0) return;
  const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
  const int q_len = q1 - q0;
  if (q1 > a.num_tokens || q0 < 0) return;
  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_blocks_per_seq * kPage));
  const int prior = L - q_len;
  if (prior < 0) return;
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
    lim[nt] = valid ? prior + j : -1;
    tok[nt] = valid ? q0 + j : -1;
    head[nt] = kv * G + g;
    const elem_t* qrow = valid ? reinterpret_cast<const elem_t*>(a.query) + ((size_t)tok[nt] * a.num_heads + head[nt]) * D
                               : nullptr;
    Tile::load_q(qf[nt], qrow, lane);
  }
  const int lim_lo = prior + r0 / G;                                   // first row of the wave
  const int lim_hi = prior + min(q_len - 1, (r0 + NTW * 16 - 1) / G);  // last row of the wave
  const int n_tiles = (lim_hi + 1 + kTile - 1) / kTile;
  const int npages = (L + kPage - 1) / kPage;
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
    const int pg = tb / kPage;
    const int pA = page_at(bt, pg, a.num_blocks);
    const int pB = page_at(bt, min(pg + 1, npages - 1), a.num_blocks);
    typename Tile::K kf;
    typename Tile::V vf;
    Tile::load_k(kf, page_ptr<elem_t>(a.key_cache, pA, a.num_kv_heads, kv, D),
                 page_ptr<elem_t>(a.key_cache, pB, a.num_kv_heads, kv, D), lane);
    Tile::load_v(vf, page_ptr<elem_t>(a.value_cache, pA, a.num_kv_heads, kv, D),
                 page_ptr<elem_t>(a.value_cache, pB, a.num_kv_heads, kv, D), lane);
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
  if (a.group <= 16)
    hipLaunchKernelGGL((decode_kernel<Tile, D, 1, OutT>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_kernel<Tile, D, 2, OutT>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <class OutT>
hipError_t decode_dispatch_out(const DecodeArgs& a, int D, bool kv_f32, int num_seqs, hipStream_t s) {
  if (kv_f32) {
    return D == 64 ? decode_dispatch_nt<TileF32<64>, 64, OutT>(a, num_seqs, s)
                   : decode_dispatch_nt<TileF32<128>, 128, OutT>(a, num_seqs, s);
  }
  return D == 64 ? decode_dispatch_nt<TileBF16<64>, 64, OutT>(a, num_seqs, s)
                 : decode_dispatch_nt<TileBF16<128>, 128, OutT>(a, num_seqs, s);
}

// Resolve the stream-decode instantiation for (D, dtype, out dtype, group) and
// hand it to `f`.
template <class F>
auto with_stream_kernel(int D, bool kv_f32, bool out_f32, int group, F f) {
  typedef void (*K)(StreamArgs);
  K k;
#define GQA_PICK(TILE, DD, NT)                                                                     \
  k = out_f32 ? (K)stream_decode_kernel<TILE<DD>, DD, NT, float>                                  \
              : (K)stream_decode_kernel<TILE<DD>, DD, NT, uint16_t>
  if (kv_f32) {
    if (D == 64) { if (group <= 16) GQA_PICK(TileF32, 64, 1); else GQA_PICK(TileF32, 64, 2); }
    else { if (group <= 16) GQA_PICK(TileF32, 128, 1); else GQA_PICK(TileF32, 128, 2); }
  } else {
    if (D == 64) { if (group <= 16) GQA_PICK(TileBF16, 64, 1); else GQA_PICK(TileBF16, 64, 2); }
    else { if (group <= 16) GQA_PICK(TileBF16, 128, 1); else GQA_PICK(TileBF16, 128, 2); }
  }
#undef GQA_PICK
  return f(k);
}

template <class OutT>
hipError_t prefill_dispatch_out(const PrefillArgs& a, int D, bool kv_f32, int groups, hipStream_t s) {
  dim3 grid(groups), block(kThreads);
  if (kv_f32) {
    if (D == 64)
      hipLaunchKernelGGL((prefill_kernel<TileF32<64>, 64, kPrefillNTW, OutT>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((prefill_kernel<TileF32<128>, 128, kPrefillNTW, OutT>), grid, block, 0, s, a);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((prefill_kernel<TileBF16<64>, 64, kPrefillNTW, OutT>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((prefill_kernel<TileBF16<128>, 128, kPrefillNTW, OutT>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool kv_f32, bool out_f32, int num_seqs,
                         hipStream_t stream) {
  return out_f32 ? decode_dispatch_out<float>(a, head_dim, kv_f32, num_seqs, stream)
                 : decode_dispatch_out<uint16_t>(a, head_dim, kv_f32, num_seqs, stream);
}

int prefill_rows_per_group() { return PrefillShape<kPrefillNTW>::kRowsPerGroup; }

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, bool kv_f32, bool out_f32, int grid_groups,
                          hipStream_t stream) {
  return out_f32 ? prefill_dispatch_out<float>(a, head_dim, kv_f32, grid_groups, stream)
                 : prefill_dispatch_out<uint16_t>(a, head_dim, kv_f32, grid_groups, stream);
}

int stream_workers(int head_dim, bool kv_f32, bool out_f32, int group, int num_seqs) {
  int dev = 0, cus = 256, per_cu = 2;
  if (hipGetDevice(&dev) == hipSuccess) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    const size_t lds = (size_t)(num_seqs + 1) * sizeof(int);
    with_stream_kernel(head_dim, kv_f32, out_f32, group, [&](void (*k)(StreamArgs)) {
      int blocks = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, reinterpret_cast<const void*>(k), kThreads, lds) ==
              hipSuccess && blocks > 0)
        per_cu = blocks;
      return 0;
    });
  }
  (void)hipGetLastError();
  return cus * per_cu * kWaves;
}

hipError_t launch_stream_decode(const StreamArgs& a, int head_dim, bool kv_f32, bool out_f32, hipStream_t stream) {
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
  const dim3 grid(a.num_workers / kWaves), block(kThreads);
  return with_stream_kernel(head_dim, kv_f32, out_f32, a.group, [&](void (*k)(StreamArgs)) {
    hipLaunchKernelGGL(k, grid, block, lds, stream, a);
    return hipGetLastError();
  });
}

hipError_t launch_stream_reduce(const StreamArgs& a, int head_dim, bool out_f32, hipStream_t stream) {
  const dim3 grid(a.num_kv_heads * a.num_seqs, a.group);
  if (head_dim == 64) {
    if (out_f32) hipLaunchKernelGGL((stream_reduce_kernel<64, float>), grid, dim3(64), 0, stream, a);
    else hipLaunchKernelGGL((stream_reduce_kernel<64, uint16_t>), grid, dim3(64), 0, stream, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((stream_reduce_kernel<128, float>), grid, dim3(128), 0, stream, a);
    else hipLaunchKernelGGL((stream_reduce_kernel<128, uint16_t>), grid, dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace gqa
