// Mixed chunked-prefill + decode batch over the paged cache, bf16: a
// scheduling pass and one fused kernel.
//
// The mixed batch of "[Kernel] [V1] Further optimizations to ROCm (Triton)
// Backend to better handle GQA" (vLLM PR #14431, review thread on
// chunked_prefill_paged_decode) holds sequences with more than one new token
// (prefill chunks: each new token attends causally to the cached prefix and to
// the chunk's earlier tokens, bottom-right aligned) and sequences with one new
// token (decodes), which the thread runs as a prefill kernel plus a decode
// kernel launched alongside it.  Here both kinds of work are units of one
// launch, ordered by a scheduling pass (below).
//
// Prefill units:
// GQA packing: the rows of a (sequence, kv head) are the pairs (new token j,
// query head g of the group), r = j * G + g, so the G heads that share a kv
// head share every K/V tile that is loaded ("[Performance] Use optimized
// kernels for MQA/GQA", opening post: GQA should cut KV reads and let the dot
// products run on matrix cores).  A work-group owns 4 waves x NTW blocks of 16
// rows; the four waves load each 32-key tile once, cooperatively, into LDS
// (double-buffered, the next tile's global loads in flight while the current
// one is consumed) and each wave multiplies it against its own rows:
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (bf16 in, fp32 out),
//   O^T += V^T P^T on v_mfma_f32_16x16x32_f16 with P rounded to fp16 (11-bit
//   significand, relative error 2^-12) and V converted bf16 -> fp16 when the
//   tile is written to LDS (exact for |v| in fp16's range; larger magnitudes
//   saturate at 65504, a precondition of this path).
// The softmax denominator is the same product with V replaced by ones, so it
// sums exactly the rounded P that weighs V and costs no VALU additions.
#include "decode_core.h"

namespace gqa {

namespace {

constexpr float kLazyRescale = 8.f;      // log2 growth of a row max before O is rescaled

template <int D, int NTW>
struct PrefillLds {
  static constexpr int kRowsPerWave = NTW * 16;
  static constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
  static constexpr int KC = D / 32;                 // 16-byte chunks of a row per Q.K^T product
  static constexpr int DT = D / 16;                 // 16-channel output blocks
  static constexpr int KROW = D + 8;                // LDS row stride of the key tile (elements)
  static constexpr int VROW = kTile + 8;            // LDS row stride of the value tile (elements)
  static constexpr int KCH = kTile * D / 8 / kThreads;   // 16-byte key chunks per thread per tile
  static constexpr int VCH = 2 * D * 2 / kThreads;       // 16-byte value chunks per thread per tile
};

// LDS row of key token t.  A 128-bit LDS read is served 8 lanes at a time over
// 32 four-byte banks, so with a 272-byte row stride row r lands in 16-byte bank
// group r mod 8.  Lanes 0-7 of a Q.K^T product read tokens {0-3, 8-11} (+4, +16
// for lanes 8-15): flipping bit 2 of tokens whose bit 3 is set sends those runs
// to distinct groups.
__device__ __forceinline__ int key_row(int t) { return t ^ ((t >> 1) & 4); }

// max without the NaN canonicalisation fmaxf implies (operands are never NaN
// here: masked scores are -inf, not NaN)
__device__ __forceinline__ float max2(float a, float b) { return a > b ? a : b; }

// This thread's share of a tile: for each 16-byte chunk, the page it comes from
// (0 = first page of the tile, 1 = second), its element offset inside that
// page, and its element offset in the LDS tile.
template <int D, int NTW>
struct TileCopyPlan {
  typedef PrefillLds<D, NTW> S;
  // k_page / v_page are wave-uniform: 16 tokens of keys (or 16 tokens of one
  // page's values) are a multiple of a wave's 64 chunks for D = 64 and 128
  int k_page[S::KCH], k_src[S::KCH], k_dst[S::KCH];
  int v_page[S::VCH], v_src[S::VCH], v_dst[S::VCH], v_tok[S::VCH];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < S::KCH; ++i) {
      const int ci = threadIdx.x + i * kThreads;
      const int token = ci / (D / 8), col = ci % (D / 8);
      k_page[i] = uniform(token / kPage);
      k_src[i] = (token % kPage) * D + col * 8;
      k_dst[i] = key_row(token) * S::KROW + col * 8;
    }
#pragma unroll
    for (int i = 0; i < S::VCH; ++i) {
      const int ci = threadIdx.x + i * kThreads;
      const int h = ci / (2 * D), rem = ci % (2 * D);
      const int d = rem / 2, e = rem % 2;
      v_page[i] = uniform(h);
      v_src[i] = d * kPage + 8 * e;
      v_dst[i] = d * S::VROW + 16 * h + 8 * e;
      v_tok[i] = 16 * h + 8 * e;                     // first token (in the tile) of this 8-token run
    }
  }
};

template <int D, int NTW>
__device__ __forceinline__ void load_tile_regs(uint4* kreg, uint4* vreg, const TileCopyPlan<D, NTW>& plan,
                                               const uint16_t* kA, const uint16_t* kB, const uint16_t* vA,
                                               const uint16_t* vB) {
  typedef PrefillLds<D, NTW> S;
#pragma unroll
  for (int i = 0; i < S::KCH; ++i) kreg[i] = ld16((plan.k_page[i] ? kB : kA) + plan.k_src[i]);
#pragma unroll
  for (int i = 0; i < S::VCH; ++i) vreg[i] = ld16((plan.v_page[i] ? vB : vA) + plan.v_src[i]);
}

// Registers -> LDS; values are converted to fp16, and with `tail` set those of
// tokens at or past L become 0.
template <int D, int NTW>
__device__ __forceinline__ void store_tile_lds(uint16_t* sK, uint16_t* sV, const uint4* kreg, const uint4* vreg,
                                               const TileCopyPlan<D, NTW>& plan, int tile_base, int L, bool tail) {
  typedef PrefillLds<D, NTW> S;
#pragma unroll
  for (int i = 0; i < S::KCH; ++i) *reinterpret_cast<uint4*>(sK + plan.k_dst[i]) = kreg[i];
#pragma unroll
  for (int i = 0; i < S::VCH; ++i) {
    uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
    if (tail) {
      const int t0 = tile_base + plan.v_tok[i];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[k] &= (t0 + 2 * k < L ? 0xFFFFu : 0u) | (t0 + 2 * k + 1 < L ? 0xFFFF0000u : 0u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = bf16x2_to_f16x2(w[k]);
    *reinterpret_cast<uint4*>(sV + plan.v_dst[i]) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Row tile rt (rows [rt * R, rt * R + R) of the r = j * G + g order, R =
// kRowsPerGroup) of sequence b against kv head kv.  sK / sV: two LDS buffers
// each of kTile * KROW and D * VROW elements.
template <int D, int NTW, class OutT>
__device__ __forceinline__ void prefill_unit(const PrefillArgs& a, int b, int rt, int kv, uint16_t* sK, uint16_t* sV) {
  typedef PrefillLds<D, NTW> S;
  constexpr int KBUF = kTile * S::KROW, VBUF = D * S::VROW;
  const int G = a.group;
  const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
  const int q_len = q1 - q0;
  if (q1 > a.num_tokens || q0 < 0) return;
  const int L = max(0, min(a.seq_lens[b], a.max_blocks_per_seq * kPage));
  const int prior = L - q_len;
  if (prior < 0) return;
  const int rows_total = q_len * G;

  const int lane = lane_id(), w = wave_id();
  const int n = lane & 15, q = lane >> 4;
  const int r0 = rt * S::kRowsPerGroup + w * S::kRowsPerWave;
  const bool wave_rows = r0 < rows_total;

  // Scores are scaled after their max is taken, which needs a positive scale:
  // a negative one flips the query's sign (exact in bf16) and |scale| is used;
  // a zero scale (every visible score 0) zeroes the query and uses 1, so that
  // masked scores stay -inf instead of -inf * 0.
  const bool zero_scale = a.scale_log2 == 0.f;
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  const uint32_t qkeep = zero_scale ? 0u : 0xFFFFFFFFu;
  const float sl2 = zero_scale ? 1.f : __builtin_fabsf(a.scale_log2);
  uint4 qf[NTW][S::KC];
  int lim[NTW], tok[NTW], head[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const int r = r0 + nt * 16 + n;
    const bool valid = r < rows_total;
    const int j = r / G, g = r % G;
    lim[nt] = valid ? prior + j : -1;
    tok[nt] = valid ? q0 + j : -1;
    head[nt] = kv * G + g;
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.query) + ((size_t)(valid ? tok[nt] : 0) * a.num_heads + head[nt]) * D;
#pragma unroll
    for (int c = 0; c < S::KC; ++c) {
      uint4 x = valid ? ld16(qrow + 32 * c + 8 * q) : make_uint4(0, 0, 0, 0);
      x.x = (x.x ^ qsign) & qkeep;
      x.y = (x.y ^ qsign) & qkeep;
      x.z = (x.z ^ qsign) & qkeep;
      x.w = (x.w ^ qsign) & qkeep;
      qf[nt][c] = x;
    }
  }
  const int lim_lo = prior + r0 / G;
  const int lim_hi = wave_rows ? prior + min(q_len - 1, (r0 + S::kRowsPerWave - 1) / G) : -1;
  const int group_hi = prior + min(q_len - 1, (rt * S::kRowsPerGroup + S::kRowsPerGroup - 1) / G);
  const int n_tiles = group_hi / kTile + 1;
  const int npages = (L + kPage - 1) / kPage;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.key_cache) + (size_t)kv * (kPage * D);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.value_cache) + (size_t)kv * (kPage * D);
  const size_t page_stride = (size_t)a.num_kv_heads * (kPage * D);

  TileCopyPlan<D, NTW> plan;
  plan.init();
  // Raw block-table entries of tile t (clamped to the last tile).  They are
  // loaded one iteration before they are used, so that waiting for them never
  // waits for the K/V loads issued just before.
  auto fetch_pages = [&](int t, int& rawA, int& rawB) {
    const int pg = min(t, n_tiles - 1) * 2;
    rawA = bt[pg];
    rawB = bt[min(pg + 1, npages - 1)];
  };
  auto page_id = [&](int raw) { return uniform((unsigned)raw < (unsigned)a.num_blocks ? raw : 0); };
  auto issue = [&](int pA, int pB, uint4* kr, uint4* vr) {
    load_tile_regs<D, NTW>(kr, vr, plan, kc + pA * page_stride, kc + pB * page_stride, vc + pA * page_stride,
                           vc + pB * page_stride);
  };

  float m[NTW], mu[NTW];
  f32x4_t o[NTW][S::DT], ol[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    m[nt] = -INFINITY;
    mu[nt] = 0.f;
    ol[nt] = zero4();
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) o[nt][dt] = zero4();
  }

  uint4 kreg[S::KCH], vreg[S::VCH];
  int rawA, rawB;
  fetch_pages(0, rawA, rawB);
  issue(page_id(rawA), page_id(rawB), kreg, vreg);
  store_tile_lds<D, NTW>(sK, sV, kreg, vreg, plan, 0, L, kTile > L);
  fetch_pages(1, rawA, rawB);
  __syncthreads();

  // LDS offsets of this lane's key rows (products s = 0, 1; token fed to row m
  // as in TileBF16) and value rows
  const int kslot = ((n < 8) ? 0 : kPage) + (n & 3) + 8 * ((n >> 2) & 1);
  const int koff0 = key_row(kslot) * S::KROW + 8 * q, koff1 = key_row(kslot + 4) * S::KROW + 8 * q;
  const int voff = n * S::VROW + 8 * q;
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);   // fp16 1.0 x 8
  const float pinf = opaque(INFINITY);

  // One tile against this wave's rows; `masked` applies the causal limit per
  // score (tiles wholly below the diagonal skip it).
  auto compute = [&](const uint16_t* K, const uint16_t* V, int tb, bool masked) {
    f32x4_t acc[NTW][2];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[nt][0] = acc[nt][1] = zero4();
#pragma unroll
    for (int c = 0; c < S::KC; ++c) {
      const uint4 k0 = *reinterpret_cast<const uint4*>(K + koff0 + 32 * c);
      const uint4 k1 = *reinterpret_cast<const uint4*>(K + koff1 + 32 * c);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        acc[nt][0] = mfma_bf16(k0, qf[nt][c], acc[nt][0]);
        acc[nt][1] = mfma_bf16(k1, qf[nt][c], acc[nt][1]);
      }
    }
    uint4 pf[NTW];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      float sc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sc[i] = i < 4 ? acc[nt][0][i] : acc[nt][1][i - 4];
      if (masked) {
#pragma unroll
        for (int i = 0; i < 8; ++i) sc[i] = (tb + 8 * q + i <= lim[nt]) ? sc[i] : -INFINITY;
      }
      const float mx = fmax_nn(fmax_nn(fmax_nn(sc[0], sc[1], pinf), fmax_nn(sc[2], sc[3], pinf), pinf),
                               fmax_nn(fmax_nn(sc[4], sc[5], pinf), fmax_nn(sc[6], sc[7], pinf), pinf), pinf);
      // Running max in log2 units, raised (and O rescaled) only when some row's
      // max grows by more than kLazyRescale, so P stays <= 2^kLazyRescale.  A
      // lane's own max decides whether any row needs it; only then is the row
      // max taken across the row's four lanes.
      if (__any(mx * sl2 > m[nt] + kLazyRescale)) {
        const float m_new = fmax_nn(m[nt], row_max4(mx) * sl2, pinf);
        const float mu_new = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m[nt] - mu_new);     // 0 while m = -inf (O and l are 0)
        ol[nt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) o[nt][dt] *= alpha;
        m[nt] = m_new;
        mu[nt] = mu_new;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) sc[i] = fast_exp2(__builtin_fmaf(sc[i], sl2, -mu[nt]));
      pf[nt] = make_uint4(f32x2_to_f16x2(sc[0], sc[1]), f32x2_to_f16x2(sc[2], sc[3]), f32x2_to_f16x2(sc[4], sc[5]),
                          f32x2_to_f16x2(sc[6], sc[7]));
      ol[nt] = mfma_f16(ones, pf[nt], ol[nt]);
    }
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
      const uint4 vf = *reinterpret_cast<const uint4*>(V + voff + 16 * dt * S::VROW);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) o[nt][dt] = mfma_f16(vf, pf[nt], o[nt][dt]);
    }
  };

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int tb = it * kTile;
    const bool more = it + 1 < n_tiles;
    // tile it + 1: global loads in flight while tile it is computed; the
    // block-table entries of tile it + 2 follow them
    const int pA = page_id(rawA), pB = page_id(rawB);
    if (more) issue(pA, pB, kreg, vreg);
    fetch_pages(it + 2, rawA, rawB);
    if (tb <= lim_hi) compute(sK + buf * KBUF, sV + buf * VBUF, tb, tb + kTile - 1 > lim_lo);
    if (more)
      store_tile_lds<D, NTW>(sK + (buf ^ 1) * KBUF, sV + (buf ^ 1) * VBUF, kreg, vreg, plan, tb + kTile, L,
                             tb + 2 * kTile > L);
    __syncthreads();
  }

  if (!wave_rows) return;
  OutT* out = reinterpret_cast<OutT*>(a.out);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    // every element of ol is the row sum of the rounded P of this lane's row
    const float lr = ol[nt][0];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    if (tok[nt] >= 0) {
      OutT* dst = out + ((size_t)tok[nt] * a.num_heads + head[nt]) * D + 4 * q;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) store4(dst + dt * 16, o[nt][dt] * inv);
    }
  }
}

constexpr int kLdsNTW = 2;

// ---------------------------------------------------------------------------
// Scheduling pass.  The mixed batch splits into work units, each run by one
// work-group per kv head: a prefill row tile of a sequence with q_len > 1, or
// a decode partition of a sequence with q_len = 1.  Their costs differ by
// orders of magnitude (a row tile near the end of a long chunk reads the whole
// prefix; most decodes read a few pages), and work-groups are dispatched in
// index order, so the list is ordered by decreasing cost (longest processing
// time first): the long units start first and the short ones fill in behind
// them.  Cost, in tile steps of a work-group: a prefill row tile takes one step
// per 32-key tile up to its last row's causal limit; a decode partition's
// tiles are shared by the 4 waves.  One work-group of 1024 threads counts the
// units per cost bucket in LDS, scans, and scatters (order within a bucket is
// arbitrary; each unit's result does not depend on it).
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kCostBuckets = 4096;

__device__ __forceinline__ int unit_cost_bucket(int c) { return min(c, kCostBuckets - 1); }

template <class F>
__device__ __forceinline__ void for_each_unit(const ScheduleArgs& a, int b, F&& emit) {
  const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
  const int q_len = q1 - q0;
  if (q1 > a.num_tokens || q0 < 0 || q_len <= 0 || q_len > a.max_query_len) return;
  const int L = max(0, min(a.seq_lens[b], a.max_blocks_per_seq * kPage));
  if (q_len == 1) {
    const int Lp = min(L, a.max_partitions * a.partition_size);
    const int nparts = max(1, (Lp + a.partition_size - 1) / a.partition_size);
    const int tiles_all = (Lp + kTile - 1) / kTile;
    const int per = tiles_all / nparts, extra = tiles_all % nparts;
    for (int p = 0; p < nparts; ++p) {
      const int t = per + (p < extra ? 1 : 0);
      emit(b, -1 - p, (t + 3) / 4);
    }
    return;
  }
  const int prior = L - q_len;
  if (prior < 0) return;
  const int G = a.group, R = a.rows_per_group;
  const int n_rt = (q_len * G + R - 1) / R;
  for (int rt = n_rt - 1; rt >= 0; --rt) {
    const int hi = prior + min(q_len - 1, (rt * R + R - 1) / G);
    emit(b, rt, hi / kTile + 1);
  }
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(ScheduleArgs a) {
  __shared__ int hist[kCostBuckets];
  __shared__ int part[kSchedThreads];
  for (int i = threadIdx.x; i < kCostBuckets; i += kSchedThreads) hist[i] = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < a.num_seqs; b += kSchedThreads)
    for_each_unit(a, b, [&](int, int, int c) { atomicAdd(&hist[unit_cost_bucket(c)], 1); });
  __syncthreads();
  // exclusive scan in decreasing cost: start[c] = number of units costlier than c
  constexpr int PER = kCostBuckets / kSchedThreads;
  const int top = kCostBuckets - 1 - PER * threadIdx.x;       // this thread's buckets: top, top-1, ...
  int local[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    local[i] = hist[top - i];
    sum += local[i];
  }
  part[threadIdx.x] = sum;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int add = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  const int total = part[kSchedThreads - 1];
  int run = part[threadIdx.x] - sum;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    hist[top - i] = run;
    run += local[i];
  }
  __syncthreads();
  for (int b = threadIdx.x; b < a.num_seqs; b += kSchedThreads)
    for_each_unit(a, b, [&](int bb, int code, int c) {
      const int pos = atomicAdd(&hist[unit_cost_bucket(c)], 1);
      if (pos < a.unit_capacity) a.units[pos] = make_int2(bb, code);
    });
  if (threadIdx.x == 0) *a.unit_count = min(total, a.unit_capacity);
}

// ---------------------------------------------------------------------------
// Mixed batch: work-group i runs unit i / Hkv of the scheduled list for kv
// head i % Hkv, as a prefill row tile (K/V tiles shared through LDS) or as a
// decode partition (per-wave tile pipeline, waves merged through LDS).  The
// decode units ride along the prefill ones in one launch: HBM-bound decodes
// and matrix-bound prefill tiles then share the device instead of running one
// after the other.
// ---------------------------------------------------------------------------
template <int D, int NT>
struct MixedLds {
  typedef PrefillLds<D, kLdsNTW> S;
  static constexpr int kPrefillBytes = 2 * (kTile * S::KROW + D * S::VROW) * 2;
  static constexpr int kDecodeBytes = DecodeMergeLds<D, NT>::kFloats * 4;
  static constexpr int kBytes = kPrefillBytes > kDecodeBytes ? kPrefillBytes : kDecodeBytes;
};

template <int D, int NT, class OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1)))
void mixed_kernel(MixedArgs a) {
  typedef PrefillLds<D, kLdsNTW> S;
  __shared__ __attribute__((aligned(16))) char lds[MixedLds<D, NT>::kBytes];
  const int Hkv = a.prefill.num_kv_heads;
  const int slot = blockIdx.x / Hkv, kv = blockIdx.x % Hkv;
  if (slot >= *a.unit_count) return;
  const int2 u = a.units[slot];
  if (u.y >= 0) {
    uint16_t* sK = reinterpret_cast<uint16_t*>(lds);
    prefill_unit<D, kLdsNTW, OutT>(a.prefill, u.x, u.y, kv, sK, sK + 2 * kTile * S::KROW);
  } else {
    decode_partition<TileBF16<D>, D, NT, OutT>(a.decode, -1 - u.y, kv, u.x, reinterpret_cast<float*>(lds));
  }
}

template <int D, class OutT>
hipError_t mixed_dispatch(const MixedArgs& a, int groups, hipStream_t s) {
  if (a.prefill.group <= 16)
    hipLaunchKernelGGL((mixed_kernel<D, 1, OutT>), dim3(groups), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((mixed_kernel<D, 2, OutT>), dim3(groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int prefill_lds_rows_per_group() { return PrefillLds<128, kLdsNTW>::kRowsPerGroup; }

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mixed(const MixedArgs& a, int head_dim, bool out_f32, int grid_groups, hipStream_t stream) {
  if (head_dim == 64)
    return out_f32 ? mixed_dispatch<64, float>(a, grid_groups, stream) : mixed_dispatch<64, uint16_t>(a, grid_groups, stream);
  return out_f32 ? mixed_dispatch<128, float>(a, grid_groups, stream) : mixed_dispatch<128, uint16_t>(a, grid_groups, stream);
}

}  // namespace gqa
