// Paged GQA attention kernels for gfx950: decode (split-K) and chunked prefill.
//
// Both kernels read each (sequence, kv head) K/V page once per work item and
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

// ---------------------------------------------------------------------------
// Decode: grid (max_partitions, Hkv, B), 4 waves.  The work-group owns keys
// [p*P, min((p+1)*P, L)) of one (sequence, kv head); its waves take the
// partition's 32-token tiles round-robin and merge through LDS at the end.
// A sequence with a single partition writes `out`; otherwise the work-group
// writes its normalised partial output and log-sum-exp for the reduce kernel.
// ---------------------------------------------------------------------------
template <class Tile, int D, int NT, class OutT>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  typedef typename Tile::elem_t elem_t;
  constexpr int R = NT * 16;            // padded rows of the group
  const int p = blockIdx.x, kv = blockIdx.y, b = blockIdx.z;
  const int G = a.group;

  int row = b;
  if (a.query_start_loc) {
    const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
    if (q1 - q0 != 1 || q1 > a.num_tokens || q0 < 0) return;
    row = q0;
  }
  int L = a.seq_lens[b];
  L = max(0, min(L, min(a.max_blocks_per_seq * kPage, a.max_partitions * a.partition_size)));
  const int nparts = (L + a.partition_size - 1) / a.partition_size;
  OutT* out = reinterpret_cast<OutT*>(a.out);

  if (L == 0) {
    if (p == 0)
      for (int i = threadIdx.x; i < G * D; i += kThreads)
        store1(out + ((size_t)row * a.num_heads + kv * G) * D + i, 0.f);
    return;
  }
  if (p >= nparts) return;

  const int t0 = p * a.partition_size;
  const int t1 = min(t0 + a.partition_size, L);
  const int n_tiles = (t1 - t0 + kTile - 1) / kTile;
  const int npages = (L + kPage - 1) / kPage;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;

  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15, q = lane >> 4;

  typename Tile::Q qf[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int g = nt * 16 + n;
    const elem_t* qrow = (g < G) ? reinterpret_cast<const elem_t*>(a.query) +
                                       ((size_t)row * a.num_heads + kv * G + g) * D
                                 : nullptr;
    Tile::load_q(qf[nt], qrow, lane);
  }

  float m[NT], l[NT];
  f32x4_t o[NT][Tile::DT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -INFINITY;
    l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < Tile::DT; ++dt) o[nt][dt] = zero4();
  }

  for (int it = w; it < n_tiles; it += kWaves) {
    const int tb = t0 + it * kTile;
    const int pg = tb / kPage;
    const int pA = page_at(bt, pg, a.num_blocks);
    const int pB = page_at(bt, min(pg + 1, npages - 1), a.num_blocks);
    typename Tile::K kf;
    typename Tile::V vf;
    Tile::load_k(kf, page_ptr<elem_t>(a.key_cache, pA, a.num_kv_heads, kv, D),
                 page_ptr<elem_t>(a.key_cache, pB, a.num_kv_heads, kv, D), lane);
    Tile::load_v(vf, page_ptr<elem_t>(a.value_cache, pA, a.num_kv_heads, kv, D),
                 page_ptr<elem_t>(a.value_cache, pB, a.num_kv_heads, kv, D), lane);
    const bool masked = tb + kTile > t1;
    if (tb + kTile > L) Tile::mask_v(vf, tb, L, lane);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float s[8];
      Tile::qk(s, kf, qf[nt]);
      softmax_pv<Tile>(s, m[nt], l[nt], o[nt], vf, a.scale_log2, masked, tb, t1 - 1, q);
    }
  }

  // ---- merge the four waves ----
  __shared__ float sm_m[kWaves][R];
  __shared__ float sm_l[kWaves][R];
  __shared__ float sm_o[kWaves][R][D + 4];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float lr = row_sum4(l[nt]);
    if (q == 0) {
      sm_m[w][nt * 16 + n] = m[nt];
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
    const float f = (Ls > 0.f) ? fast_exp2(m[nt] - Mu) / Ls : 0.f;
    if (r < G) {
#pragma unroll
      for (int dt = 0; dt < Tile::DT; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) sm_o[w][r][dt * 16 + 4 * q + j] = o[nt][dt][j] * f;
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
// Prefill (chunked): one work-group per (row tile, kv head) of the sequences
// with more than one query token.  Rows of a sequence are (token j, head g)
// pairs packed r = j * G + g, so one 16-row block covers 16/G new tokens of a
// GQA group and the key tile it multiplies is loaded once for all of them.
// Each wave owns NTW blocks of rows and walks the keys from 0 to its last
// row's causal limit seq_len - q_len + j.
// ---------------------------------------------------------------------------
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

  // Locate (sequence, row tile) for this work-group: scan the per-sequence
  // tile counts in chunks of kThreads sequences.
  __shared__ int s_scan[kThreads];
  __shared__ int s_found[2];
  if (threadIdx.x == 0) s_found[0] = -1;
  int base = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += kThreads) {
    const int bb = c0 + threadIdx.x;
    int cnt = 0;
    if (bb < a.num_seqs) {
      const int ql = a.query_start_loc[bb + 1] - a.query_start_loc[bb];
      cnt = (ql > 1) ? (ql * G + RWG - 1) / RWG : 0;
    }
    s_scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int add = (threadIdx.x >= off) ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += add;
      __syncthreads();
    }
    const int total = s_scan[kThreads - 1];
    if (tile < base + total) {
      const int incl = base + s_scan[threadIdx.x];
      if (cnt > 0 && tile < incl && tile >= incl - cnt) {
        s_found[0] = bb;
        s_found[1] = tile - (incl - cnt);
      }
      __syncthreads();
      break;
    }
    base += total;
    __syncthreads();
  }
  __syncthreads();
  const int b = s_found[0];
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
  const int rt = n_row_tiles - 1 - s_found[1];

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

}  // namespace gqa
