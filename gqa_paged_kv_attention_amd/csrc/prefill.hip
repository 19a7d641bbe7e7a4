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
constexpr int kKeyTile = 64;             // keys per iteration
constexpr int kTileBlocks = kKeyTile / kHalf;   // 16-token blocks per tile, each inside one page

template <int D, int NTW>
struct PrefillLds {
  static constexpr int kRowsPerWave = NTW * 16;
  static constexpr int kRowsPerGroup = kWaves * kRowsPerWave;
  static constexpr int KC = D / 32;                 // 16-byte chunks of a row per Q.K^T product
  static constexpr int DT = D / 16;                 // 16-channel output blocks
  static constexpr int KROW = D + 16;               // LDS row stride of the key tile (elements)
  static constexpr int VROW = kKeyTile + 16;        // LDS row stride of the value tile (elements)
  static constexpr int KBUF = kKeyTile * KROW;      // one key buffer (elements)
  static constexpr int VBUF = D * VROW;             // one value buffer (elements)
  static constexpr int kBytes = 2 * (KBUF + VBUF) * 2;
  static constexpr int CH = kKeyTile * D / 8 / kThreads;   // 16-byte chunks per thread per tile, K and V each
  // chunk i of a thread comes from 16-token block i * PI + (thread / (kThreads / PI)) of the tile
  static constexpr int PI = 128 / D;
};

// LDS banking (gfx950, measured): a 128-bit access is served 32 lanes at a
// time by 128 four-byte banks, so the 32 lanes' 16-byte slots must differ mod
// 512 bytes.  Key rows are D + 16 elements apart (an even number of slots whose
// half is odd: 18 for D = 128, 10 for D = 64), so rows that differ mod 16 land
// on distinct even slots and the two 16-byte chunks of a 32-lane group fill the
// odd ones.  Lanes 0-15 of a Q.K^T product read tokens {0-3, 8-11, 16-19,
// 24-27} (+4 for the second product, +32 for the second half of the tile):
// moving bit 4 of the token onto bit 2 makes them distinct mod 16.  Value rows
// (channels) are kKeyTile + 16 elements apart (10 slots): 16 consecutive
// channels land on distinct even slots as well.
__device__ __forceinline__ int key_row(int t) { return t ^ ((t >> 2) & 4); }

// This thread's share of a tile: for each 16-byte chunk of keys and of values,
// its element offset from the first token of its 16-token block (key rows D
// elements apart, value channels BS apart) and in the LDS tile.  The chunk's
// block is wave-uniform: i * PI + pw.
template <int D, int NTW, int BS>
struct TileCopyPlan {
  typedef PrefillLds<D, NTW> S;
  int k_src[S::CH], k_dst[S::CH];
  int v_src[S::CH], v_dst[S::CH], v_tok[S::CH];
  int pw;                                           // wave-uniform block offset of chunk 0
  __device__ __forceinline__ void init() {
    pw = S::PI == 1 ? 0 : uniform(threadIdx.x / (kThreads / S::PI));
#pragma unroll
    for (int i = 0; i < S::CH; ++i) {
      const int ci = threadIdx.x + i * kThreads;
      const int token = ci / (D / 8), col = ci % (D / 8);        // token / 16: block of chunk i
      k_src[i] = (token % kHalf) * D + col * 8;
      k_dst[i] = key_row(token) * S::KROW + col * 8;
      const int h = ci / (2 * D), rem = ci % (2 * D);            // h: block of chunk i
      const int d = rem / 2, e = rem % 2;
      v_src[i] = d * BS + 8 * e;
      v_dst[i] = d * S::VROW + 16 * h + 8 * e;
      v_tok[i] = 16 * h + 8 * e;                     // first token (in the tile) of this 8-token run
    }
  }
  // base pointer of chunk i (constant indices only, so TilePtrs stays in registers)
  template <class P>
  __device__ __forceinline__ P block_of(int i, const P* blocks) const {
    if (S::PI == 1) return blocks[i];
    return pw ? blocks[i * S::PI + 1] : blocks[i * S::PI];
  }
};

// First-token pointers (K row, channel-0 value; this kv head) of the four
// 16-token blocks of a tile.
struct TilePtrs {
  const uint16_t* k[kTileBlocks];
  const uint16_t* v[kTileBlocks];
};

template <int D, int NTW, int BS>
__device__ __forceinline__ void load_tile_regs(uint4* kreg, uint4* vreg, const TileCopyPlan<D, NTW, BS>& plan,
                                               const TilePtrs& tp) {
  typedef PrefillLds<D, NTW> S;
#pragma unroll
  for (int i = 0; i < S::CH; ++i) {
    kreg[i] = ld16(plan.block_of(i, tp.k) + plan.k_src[i]);
    vreg[i] = ld16(plan.block_of(i, tp.v) + plan.v_src[i]);
  }
}

// Registers -> LDS; values are converted to fp16, and with `tail` set those of
// tokens at or past L become 0.
template <int D, int NTW, int BS>
__device__ __forceinline__ void store_tile_lds(uint16_t* sK, uint16_t* sV, const uint4* kreg, const uint4* vreg,
                                               const TileCopyPlan<D, NTW, BS>& plan, int tile_base, int L, bool tail) {
  typedef PrefillLds<D, NTW> S;
#pragma unroll
  for (int i = 0; i < S::CH; ++i) *reinterpret_cast<uint4*>(sK + plan.k_dst[i]) = kreg[i];
  uint32_t w[S::CH][4];
#pragma unroll
  for (int i = 0; i < S::CH; ++i) {
    w[i][0] = vreg[i].x;
    w[i][1] = vreg[i].y;
    w[i][2] = vreg[i].z;
    w[i][3] = vreg[i].w;
  }
  if (tail) {
#pragma unroll
    for (int i = 0; i < S::CH; ++i) {
      const int t0 = tile_base + plan.v_tok[i];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        w[i][k] &= (t0 + 2 * k < L ? 0xFFFFu : 0u) | (t0 + 2 * k + 1 < L ? 0xFFFF0000u : 0u);
    }
  }
#pragma unroll
  for (int i = 0; i < S::CH; ++i)
    *reinterpret_cast<uint4*>(sV + plan.v_dst[i]) =
        make_uint4(bf16x2_to_f16x2(w[i][0]), bf16x2_to_f16x2(w[i][1]), bf16x2_to_f16x2(w[i][2]),
                   bf16x2_to_f16x2(w[i][3]));
}

// Row tile rt (rows [rt * R, rt * R + R) of the r = j * G + g order, R =
// kRowsPerGroup) of sequence b (new tokens [q0, q1), seq_lens[b] = seq_len)
// against kv head kv.  Causal: token j sees keys up to seq_len - q_len + j;
// otherwise (cross-attention) every row sees all seq_len keys, and q_len may
// exceed seq_len.  Pages hold BS tokens.  sK / sV: two LDS buffers of KBUF
// and VBUF elements each.
template <int D, int NTW, int BS, class OutT>
__device__ __forceinline__ void prefill_unit(const PrefillArgs& a, int b, int rt, int q0, int q1, int seq_len, int kv,
                                             uint16_t* sK, uint16_t* sV) {
  typedef PrefillLds<D, NTW> S;
  const int G = a.group;
  const int q_len = q1 - q0;
  if (q1 > a.num_tokens || q0 < 0) return;
  const int L = clamp_len(seq_len, a.max_blocks_per_seq, BS);
  const int prior = L - q_len;
  if (a.causal && prior < 0) return;
  const int rows_total = q_len * G;
  // last key visible to new token j
  auto last_key = [&](int j) { return a.causal ? prior + j : L - 1; };

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
    lim[nt] = valid ? last_key(j) : -1;
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
  const int lim_lo = last_key(r0 / G);
  const int lim_hi = wave_rows ? last_key(min(q_len - 1, (r0 + S::kRowsPerWave - 1) / G)) : -1;
  const int group_hi = last_key(min(q_len - 1, (rt * S::kRowsPerGroup + S::kRowsPerGroup - 1) / G));
  // no tile when no key is visible (an empty encoder sequence): zero rows
  const int n_tiles = group_hi < 0 ? 0 : group_hi / kKeyTile + 1;
  const int npages = (L + BS - 1) / BS;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const char* kc = reinterpret_cast<const char*>(a.key_cache) + (size_t)kv * (BS * D * 2);
  const char* vc = reinterpret_cast<const char*>(a.value_cache) + (size_t)kv * (BS * D * 2);
  const uint32_t page_bytes = (uint32_t)a.num_kv_heads * (BS * D * 2);
  constexpr int kEntries = kKeyTile / BS;           // block-table entries per tile: 4, 2 or 1

  TileCopyPlan<D, NTW, BS> plan;
  plan.init();
  // Raw block-table entries of tile t (clamped to the last tile and page).
  // They are loaded one iteration before they are used, so that waiting for
  // them never waits for the K/V loads issued just before.
  auto fetch_pages = [&](int t, int* raw) {
    const int pg = min(t, n_tiles - 1) * kEntries;
#pragma unroll
    for (int j = 0; j < kEntries; ++j) raw[j] = bt[min(pg + j, npages - 1)];
  };
  // 16-token block j of the tile: entry j * 16 / BS, from token j * 16 mod BS of that page
  auto issue = [&](const int* raw, uint4* kr, uint4* vr) {
    TilePtrs tp;
#pragma unroll
    for (int j = 0; j < kTileBlocks; ++j) {
      const int e = j * kHalf / BS, slot = j * kHalf % BS;
      const uint32_t pid = (uint32_t)uniform((unsigned)raw[e] < (unsigned)a.num_blocks ? raw[e] : 0);
      const size_t off = (size_t)pid * page_bytes;
      tp.k[j] = reinterpret_cast<const uint16_t*>(kc + off) + slot * D;
      tp.v[j] = reinterpret_cast<const uint16_t*>(vc + off) + slot;
    }
    load_tile_regs<D, NTW, BS>(kr, vr, plan, tp);
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

  // Pipeline: tile t is loaded into registers during iteration t - 2, written
  // to LDS buffer t & 1 at the top of iteration t - 1 and consumed in
  // iteration t, so each load has a whole iteration to arrive.
  uint4 kreg[S::CH], vreg[S::CH];
  int raw[kEntries];
  if (n_tiles > 0) {                     // uniform over the work-group
    fetch_pages(0, raw);
    issue(raw, kreg, vreg);
    fetch_pages(1, raw);
    store_tile_lds<D, NTW, BS>(sK, sV, kreg, vreg, plan, 0, L, kKeyTile > L);
    if (n_tiles > 1) issue(raw, kreg, vreg);
    fetch_pages(2, raw);
    __syncthreads();
  }

  // LDS offsets of this lane's key rows (32-key half 0, products s = 0, 1;
  // token fed to row m as in TileBF16; half 1 is 32 rows further) and value
  // rows
  const int kslot = ((n < 8) ? 0 : kHalf) + (n & 3) + 8 * ((n >> 2) & 1);
  const int koff0 = key_row(kslot) * S::KROW + 8 * q, koff1 = key_row(kslot + 4) * S::KROW + 8 * q;
  const int voff = n * S::VROW + 8 * q;
  const uint4 ones = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);   // fp16 1.0 x 8
  const float pinf = opaque(INFINITY);

  // One 64-key tile against this wave's rows; `masked` applies the causal
  // limit per score (tiles wholly below the diagonal skip it).  Scores of
  // half hf, product s sit at keys 32 hf + 8 q + 4 s + i (i = 0..3).
  auto compute = [&](const uint16_t* K, const uint16_t* V, int tb, bool masked) {
    f32x4_t acc[NTW][4];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int x = 0; x < 4; ++x) acc[nt][x] = zero4();
#pragma unroll
    for (int c = 0; c < S::KC; ++c) {
      uint4 kf[4];
#pragma unroll
      for (int x = 0; x < 4; ++x)
        kf[x] = *reinterpret_cast<const uint4*>(K + (x >> 1) * 32 * S::KROW + ((x & 1) ? koff1 : koff0) + 32 * c);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[nt][x] = mfma_bf16(kf[x], qf[nt][c], acc[nt][x]);
    }
    float sc[NTW][16], mx[NTW];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[nt][i] = acc[nt][i >> 2][i & 3];
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sc[nt][i] = (tb + 32 * (i >> 3) + 8 * q + (i & 7) <= lim[nt]) ? sc[nt][i] : -INFINITY;
      }
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) t8[i] = fmax_nn(sc[nt][2 * i], sc[nt][2 * i + 1], pinf);
#pragma unroll
      for (int i = 0; i < 4; ++i) t8[i] = fmax_nn(t8[2 * i], t8[2 * i + 1], pinf);
      mx[nt] = fmax_nn(fmax_nn(t8[0], t8[1], pinf), fmax_nn(t8[2], t8[3], pinf), pinf);
      grow |= mx[nt] * sl2 > m[nt] + kLazyRescale;
    }
    // Running max in log2 units, raised (and O rescaled) only when some row's
    // max grows by more than kLazyRescale, so P stays <= 2^kLazyRescale.  A
    // lane's own max decides whether any row needs it; only then is the row
    // max taken across the row's four lanes.
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const float m_new = fmax_nn(m[nt], row_max4(mx[nt]) * sl2, pinf);
        if (m_new > m[nt] + kLazyRescale) {
          const float mu_new = m_new;
          const float alpha = fast_exp2(m[nt] - mu_new);   // 0 while m = -inf (O and l are 0)
          ol[nt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < S::DT; ++dt) o[nt][dt] *= alpha;
          m[nt] = m_new;
          mu[nt] = mu_new;
        }
      }
    }
    uint4 pf[NTW][2];
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[nt][i] = fast_exp2(__builtin_fmaf(sc[nt][i], sl2, -mu[nt]));
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float* x = sc[nt] + 8 * hf;
        pf[nt][hf] = make_uint4(f32x2_to_f16x2(x[0], x[1]), f32x2_to_f16x2(x[2], x[3]), f32x2_to_f16x2(x[4], x[5]),
                                f32x2_to_f16x2(x[6], x[7]));
        ol[nt] = mfma_f16(ones, pf[nt][hf], ol[nt]);
      }
    }
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
      const uint4 v0 = *reinterpret_cast<const uint4*>(V + voff + 16 * dt * S::VROW);
      const uint4 v1 = *reinterpret_cast<const uint4*>(V + voff + 16 * dt * S::VROW + 32);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        o[nt][dt] = mfma_f16(v0, pf[nt][0], o[nt][dt]);
        o[nt][dt] = mfma_f16(v1, pf[nt][1], o[nt][dt]);
      }
    }
  };

  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    const int tb = it * kKeyTile;
    // tile it + 1 (loaded during the previous iteration) -> the other buffer,
    // which every wave finished reading before the last barrier; then the
    // loads of tile it + 2, and the block-table entries of tile it + 3
    if (it + 1 < n_tiles)
      store_tile_lds<D, NTW, BS>(sK + (buf ^ 1) * S::KBUF, sV + (buf ^ 1) * S::VBUF, kreg, vreg, plan, tb + kKeyTile, L,
                             tb + 2 * kKeyTile > L);
    if (it + 2 < n_tiles) issue(raw, kreg, vreg);
    fetch_pages(it + 3, raw);
    if (tb <= lim_hi) compute(sK + buf * S::KBUF, sV + buf * S::VBUF, tb, tb + kKeyTile - 1 > lim_lo);
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
// index order, so sequences are listed by decreasing cost of their costliest
// unit (longest processing time first): the long units start first and the
// short ones fill in behind them.  Prefill and decode units form two such
// lists, merged in proportion to their lengths, so that the HBM-bound decodes
// run beside the matrix-bound prefill tiles all through the launch rather
// than after them.  A sequence's units stay contiguous, heaviest
// first: its row tiles then run at the same time and stream the same K/V
// pages, which they mostly find in L2 instead of each fetching the prefix from
// HBM (work-group i goes to XCD i mod 8, so with Hkv a multiple of 8 all work-
// groups of one kv head share an XCD and its L2).  Cost,
// in tile steps of a work-group: a prefill row tile takes one step per 32-key
// tile up to its last row's causal limit; a decode partition's tiles are
// shared by the 4 waves.  One work-group of 1024 threads counts the units per
// cost bucket and list in LDS, scans, and reserves a range per sequence (the
// order of sequences within a bucket is arbitrary; each unit's result does not
// depend on it).
// ---------------------------------------------------------------------------
constexpr int kSchedThreads = 1024;
constexpr int kCostBuckets = 2048;

__device__ __forceinline__ int unit_cost_bucket(int c) { return min(c, kCostBuckets - 1); }

// Units of sequence b and the cost of its costliest unit, without walking
// them: the last row tile reaches furthest, and the first decode partition
// holds the extra tile of an uneven split.  Both are 0 for a sequence that
// produces no work.
struct SeqInfo {
  int q0, q1, seq_len;
};

__device__ __forceinline__ bool seq_summary(const ScheduleArgs& a, int b, int* units, int* cost, SeqInfo* info) {
  *units = 0;
  *cost = 0;
  const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
  const int sl = a.seq_lens[b];
  *info = SeqInfo{q0, q1, sl};
  const int q_len = q1 - q0;
  if (q1 > a.num_tokens || q0 < 0 || q_len <= 0 || q_len > a.max_query_len) return false;
  const int L = clamp_len(sl, a.max_blocks_per_seq, a.block_size);
  if (q_len == 1) {
    const int Lp = min(L, a.max_partitions * a.partition_size);
    const int nparts = max(1, (Lp + a.partition_size - 1) / a.partition_size);
    const int tiles_all = (Lp + kTile - 1) / kTile;
    const int first = tiles_all / nparts + (tiles_all % nparts ? 1 : 0);
    *units = nparts;
    *cost = (first + 3) / 4;
    return true;
  }
  const int prior = L - q_len;
  if (a.causal && prior < 0) return false;
  *units = (q_len * a.group + a.rows_per_group - 1) / a.rows_per_group;
  // tiles up to the last row's last visible key (all L keys without the mask)
  *cost = (a.causal ? prior + q_len - 1 : max(L - 1, 0)) / kTile + 1;
  return false;
}

// Exclusive prefix sum of one value per thread over the work-group (wave
// scans, then a scan of the 16 wave totals); *total gets the sum of all.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (w == 0) {
    int t = lane < kSchedThreads / 64 ? wsum[lane] : 0;
#pragma unroll
    for (int off = 1; off < kSchedThreads / 64; off <<= 1) {
      const int y = __shfl_up(t, off);
      if (lane >= off) t += y;
    }
    if (lane < kSchedThreads / 64) wsum[lane] = t;
  }
  __syncthreads();
  *total = wsum[kSchedThreads / 64 - 1];
  const int base = w ? wsum[w - 1] : 0;
  __syncthreads();
  return base + x - v;
}

// Positions in the merged list of elements r, r + 1, ... of one list when the
// prefill and decode lists (n_self and n_other elements) are interleaved in
// proportion: element i of the prefill list sits at key (2i + 1) n_decode,
// element j of the decode list at (2j + 1) n_prefill, prefill first on ties.
// The count of other-list elements before element r is a quotient of
// num(r) = (2r + 1) n_other - n_self by den = 2 n_self (ceiling for prefill,
// floor + 1 for decode, clamped to [0, n_other]); it is kept as an exact
// quotient and remainder and stepped by 2 n_other per element.
struct MergeCursor {
  long long q;                  // floor(num / den)
  int rem, den, step_q, step_r, n_other, r;
  bool decode;
  __device__ __forceinline__ MergeCursor(int r0, int n_self, int n_oth, bool is_decode) {
    den = 2 * n_self;
    n_other = n_oth;
    r = r0;
    decode = is_decode;
    const long long num = (2LL * r0 + 1) * n_oth - n_self;
    // floor division of a possibly negative 64-bit value by a positive int
    q = num >= 0 ? num / den : -((-num + den - 1) / den);
    rem = (int)(num - q * den);
    step_q = (2 * n_oth) / den;
    step_r = (2 * n_oth) % den;
  }
  __device__ __forceinline__ int position() const {
    long long before = decode ? (q >= 0 ? q + 1 : 0) : (q + (rem > 0 ? 1 : 0));
    before = before < 0 ? 0 : (before > n_other ? n_other : before);
    return r + (int)before;
  }
  __device__ __forceinline__ void next() {
    ++r;
    q += step_q;
    rem += step_r;
    if (rem >= den) {
      rem -= den;
      ++q;
    }
  }
};

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(ScheduleArgs a) {
  __shared__ int hist[2][kCostBuckets];      // [prefill, decode][cost bucket]
  __shared__ int wsum[kSchedThreads / 64];
  for (int i = threadIdx.x; i < 2 * kCostBuckets; i += kSchedThreads) hist[i / kCostBuckets][i % kCostBuckets] = 0;
  __syncthreads();
  // the summary of this thread's first sequence is kept for the second pass
  int nu0 = 0, cmax0 = 0;
  bool dec0 = false;
  SeqInfo info0{0, 0, 0};
  for (int b = threadIdx.x; b < a.num_seqs; b += kSchedThreads) {
    int nu, cmax;
    SeqInfo info;
    const bool dec = seq_summary(a, b, &nu, &cmax, &info);
    if (b == threadIdx.x) {
      nu0 = nu;
      cmax0 = cmax;
      dec0 = dec;
      info0 = info;
    }
    if (nu) atomicAdd(&hist[dec][unit_cost_bucket(cmax)], nu);
  }
  __syncthreads();
  // exclusive scans in decreasing cost: start[c] = units of that list costlier than c
  constexpr int PER = kCostBuckets / kSchedThreads;
  const int top = kCostBuckets - 1 - PER * threadIdx.x;       // this thread's buckets: top, top-1, ...
  int n_list[2];
#pragma unroll
  for (int l = 0; l < 2; ++l) {
    int local[PER], sum = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      local[i] = hist[l][top - i];
      sum += local[i];
    }
    int run = block_exclusive_scan(sum, &n_list[l], wsum);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      hist[l][top - i] = run;
      run += local[i];
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < a.num_seqs; b += kSchedThreads) {
    int nu = nu0, cmax = cmax0;
    bool dec = dec0;
    SeqInfo info = info0;
    if (b != threadIdx.x) dec = seq_summary(a, b, &nu, &cmax, &info);
    if (!nu) continue;
    // a contiguous range of its list; units heaviest first (the last row tile
    // reaches furthest; decode partitions are in order)
    MergeCursor cur(atomicAdd(&hist[dec][unit_cost_bucket(cmax)], nu), n_list[dec], n_list[!dec], dec);
    for (int k = 0; k < nu; ++k, cur.next()) {
      const int pos = cur.position();
      if (pos < a.unit_capacity) {
        a.units[pos].a = make_int4(b, dec ? -1 - k : nu - 1 - k, info.q0, info.q1);
        a.units[pos].b = make_int4(info.seq_len, 0, 0, 0);
      }
    }
  }
  if (threadIdx.x == 0) *a.unit_count = min(n_list[0] + n_list[1], a.unit_capacity);
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
  static constexpr int kPrefillBytes = S::kBytes;
  static constexpr int kDecodeBytes = DecodeMergeLds<D, NT>::kFloats * 4;
  static constexpr int kBytes = kPrefillBytes > kDecodeBytes ? kPrefillBytes : kDecodeBytes;
};

template <int D, int NT, int BS, class OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1)))
void mixed_kernel(MixedArgs a) {
  typedef PrefillLds<D, kLdsNTW> S;
  __shared__ __attribute__((aligned(16))) char lds[MixedLds<D, NT>::kBytes];
  const int Hkv = a.prefill.num_kv_heads;
  const int slot = blockIdx.x / Hkv, kv = blockIdx.x % Hkv;
  // the record is read together with the count (slot < the list's capacity)
  const int count = *a.unit_count;
  const int4 u = a.units[slot].a;
  const int seq_len = a.units[slot].b.x;
  if (slot >= count) return;
  if (u.y >= 0) {
    uint16_t* sK = reinterpret_cast<uint16_t*>(lds);
    prefill_unit<D, kLdsNTW, BS, OutT>(a.prefill, u.x, u.y, u.z, u.w, seq_len, kv, sK, sK + 2 * S::KBUF);
  } else {
    decode_partition_at<TileBF16<D, BS>, D, NT, OutT>(a.decode, -1 - u.y, kv, u.x, u.z, seq_len,
                                                      reinterpret_cast<float*>(lds));
  }
}

template <int D, int BS, class OutT>
hipError_t mixed_dispatch(const MixedArgs& a, int groups, hipStream_t s) {
  if (a.prefill.group <= 16)
    hipLaunchKernelGGL((mixed_kernel<D, 1, BS, OutT>), dim3(groups), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((mixed_kernel<D, 2, BS, OutT>), dim3(groups), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int prefill_lds_rows_per_group() { return PrefillLds<128, kLdsNTW>::kRowsPerGroup; }

hipError_t launch_schedule(const ScheduleArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_mixed(const MixedArgs& a, int head_dim, int block_size, bool out_f32, int grid_groups,
                        hipStream_t stream) {
  return with_block_size(block_size, [&](auto bs) {
    constexpr int BS = decltype(bs)::value;
    if (head_dim == 64)
      return out_f32 ? mixed_dispatch<64, BS, float>(a, grid_groups, stream)
                     : mixed_dispatch<64, BS, uint16_t>(a, grid_groups, stream);
    return out_f32 ? mixed_dispatch<128, BS, float>(a, grid_groups, stream)
                   : mixed_dispatch<128, BS, uint16_t>(a, grid_groups, stream);
  });
}

}  // namespace gqa
