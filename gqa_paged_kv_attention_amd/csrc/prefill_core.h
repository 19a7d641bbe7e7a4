// Prefill role shared by the mixed-batch kernel and the shared-prefix decode:
// one row tile of packed (token, query head) rows against a range of keys of
// one kv head, bf16 caches, K/V tiles shared by the work-group through LDS.
//
// GQA packing: the rows of a (sequence, kv head) are the pairs (new token j,
// query head g of the group), r = j * G + g, so the G heads that share a kv
// head share every K/V tile that is loaded ("[Performance] Use optimized
// kernels for MQA/GQA", opening post: GQA should cut KV reads and let the dot
// products run on matrix cores).  A work-group owns W waves (4, or 8 in the
// launch for prefill-heavy batches) x NTW blocks of 16 rows; the waves load
// each 64-key tile once, cooperatively, into LDS
// (double-buffered, the next tile's global loads in flight while the current
// one is consumed) and each wave multiplies it against its own rows:
//   S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (bf16 in, fp32 out),
//   O^T += V^T P^T on v_mfma_f32_16x16x32_f16 with P rounded to fp16 (11-bit
//   significand, relative error 2^-12) and V converted bf16 -> fp16, rounding
//   to nearest, when the tile is written to LDS: exact for |v| in
//   [2^-14, 65504]; smaller magnitudes keep an absolute error of at most 2^-25
//   (unbiased), larger ones overflow.  Preconditions of this path: |V| < 65504,
//   and V not so small that 2^-25 matters (an N(0, s^2) V meets the parity bar
//   down to s of about 1e-5).
// The softmax denominator is the same product with V replaced by ones, so it
// sums exactly the rounded P that weighs V and costs no VALU additions.
#pragma once

#include "decode_core.h"

namespace gqa {

namespace {

constexpr float kLazyRescale = 8.f;      // log2 growth of a row max before O is rescaled
constexpr int kKeyTile = 64;             // keys per iteration
constexpr int kTileBlocks = kKeyTile / kHalf;   // 16-token blocks per tile, each inside one page

template <int D, int NTW, int W = kWaves>
struct PrefillLds {
  static constexpr int kT = W * kWave;               // threads of the work-group
  static constexpr int kRowsPerWave = NTW * 16;
  static constexpr int kRowsPerGroup = W * kRowsPerWave;
  static constexpr int KC = D / 32;                 // 16-byte chunks of a row per Q.K^T product
  static constexpr int DT = D / 16;                 // 16-channel output blocks
  static constexpr int KROW = D + 16;               // LDS row stride of the key tile (elements)
  static constexpr int VROW = kKeyTile + 16;        // LDS row stride of the value tile (elements)
  static constexpr int KBUF = kKeyTile * KROW;      // one key buffer (elements)
  static constexpr int VBUF = D * VROW;             // one value buffer (elements)
  static constexpr int kBytes = 2 * (KBUF + VBUF) * 2;
  static constexpr int CH = kKeyTile * D / 8 / kT;   // 16-byte chunks per thread per tile, K and V each
  // chunk i of a thread comes from 16-token block i * PI + (thread / (kT / PI)) of the tile
  static constexpr int PI = kT / (2 * D);
  static_assert(PI == 1 || PI == 2 || PI == 4, "a copy chunk spans 1, 2 or 4 blocks");
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
template <int D, int NTW, int BS, int W = kWaves>
struct TileCopyPlan {
  typedef PrefillLds<D, NTW, W> S;
  int k_src[S::CH], k_dst[S::CH];
  int v_src[S::CH], v_dst[S::CH], v_tok[S::CH];
  int pw;                                           // wave-uniform block offset of chunk 0
  __device__ __forceinline__ void init() {
    pw = S::PI == 1 ? 0 : uniform(threadIdx.x / (S::kT / S::PI));
#pragma unroll
    for (int i = 0; i < S::CH; ++i) {
      const int ci = threadIdx.x + i * S::kT;
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
    if (S::PI == 2) return pw ? blocks[i * S::PI + 1] : blocks[i * S::PI];
    const P lo = (pw & 1) ? blocks[i * S::PI + 1] : blocks[i * S::PI];
    const P hi = (pw & 1) ? blocks[i * S::PI + 3] : blocks[i * S::PI + 2];
    return (pw & 2) ? hi : lo;
  }
};

// First-token pointers (K row, channel-0 value; this kv head) of the four
// 16-token blocks of a tile.
struct TilePtrs {
  const uint16_t* k[kTileBlocks];
  const uint16_t* v[kTileBlocks];
};

template <int D, int NTW, int BS, int W = kWaves>
__device__ __forceinline__ void load_tile_regs(uint4* kreg, uint4* vreg, const TileCopyPlan<D, NTW, BS, W>& plan,
                                               const TilePtrs& tp) {
  typedef PrefillLds<D, NTW, W> S;
#pragma unroll
  for (int i = 0; i < S::CH; ++i) {
    kreg[i] = ld16(plan.block_of(i, tp.k) + plan.k_src[i]);
    vreg[i] = ld16(plan.block_of(i, tp.v) + plan.v_src[i]);
  }
}

// Registers -> LDS; values are converted to fp16, and with `tail` set those of
// tokens at or past L become 0.
template <int D, int NTW, int BS, int W = kWaves>
__device__ __forceinline__ void store_tile_lds(uint16_t* sK, uint16_t* sV, const uint4* kreg, const uint4* vreg,
                                               const TileCopyPlan<D, NTW, BS, W>& plan, int tile_base, int L, bool tail) {
  typedef PrefillLds<D, NTW, W> S;
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
  // Only a sequence's last tile is partial; `tail` is uniform over the
  // work-group, and the branch keeps the masking off every other tile (as a
  // select it cost about a quarter of the loop's vector instructions).
  if (__builtin_expect(tail, 0)) {
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
// exceed seq_len.  Keys before 64 * t_begin are skipped (a split over keys).
// Pages hold BS tokens.  sK / sV: two LDS buffers of KBUF and VBUF elements
// each.  `first_pages`, when given (t_begin = 0 only), holds
// block_tables[b][min(j, pages - 1)] for j = 0..7, the entries of tiles 0 and
// 1, already loaded with the unit.
template <int D, int NTW, int BS, class OutT, int W = kWaves>
__device__ __forceinline__ void prefill_unit(const PrefillArgs& a, int b, int rt, int q0, int q1, int seq_len, int kv,
                                             uint16_t* sK, uint16_t* sV, int t_begin = 0,
                                             const UnitOut& uo = UnitOut(), const int* first_pages = nullptr) {
  typedef PrefillLds<D, NTW, W> S;
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

  TileCopyPlan<D, NTW, BS, W> plan;
  plan.init();
  // Raw block-table entries of tile t (clamped to the last tile and page).
  // They are loaded one iteration before they are used, with scalar loads
  // (the entries are uniform over the work-group), so that waiting for them
  // never waits for K/V loads in the vector memory path.
  auto fetch_pages = [&](int t, int* raw) {
    const int pg = min(t, n_tiles - 1) * kEntries;
#pragma unroll
    for (int j = 0; j < kEntries; ++j) raw[j] = scalar_entry(bt, min(pg + j, npages - 1));
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
    load_tile_regs<D, NTW, BS, W>(kr, vr, plan, tp);
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
  if (n_tiles > t_begin) {               // uniform over the work-group
    if (first_pages) {
      // tile 0's entries and, when there is a tile 1, its entries (the same
      // values fetch_pages(1) reads)
      issue(first_pages, kreg, vreg);
#pragma unroll
      for (int j = 0; j < kEntries; ++j) raw[j] = first_pages[kEntries + j];
    } else {
      fetch_pages(t_begin, raw);
      issue(raw, kreg, vreg);
      fetch_pages(t_begin + 1, raw);
    }
    store_tile_lds<D, NTW, BS, W>(sK, sV, kreg, vreg, plan, t_begin * kKeyTile, L, (t_begin + 1) * kKeyTile > L);
    if (n_tiles > t_begin + 1) issue(raw, kreg, vreg);
    fetch_pages(t_begin + 2, raw);
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

  for (int it = t_begin; it < n_tiles; ++it) {
    const int buf = (it - t_begin) & 1;
    const int tb = it * kKeyTile;
    // tile it from its buffer; then tile it + 1 (loaded during the previous
    // iteration) -> the other buffer, which every wave finished reading
    // before the last barrier; then the loads of tile it + 2 and the block-
    // table entries of tile it + 3.  Computing first lets the first tile of
    // a unit start while the second is still arriving.
    if (tb <= lim_hi) compute(sK + buf * S::KBUF, sV + buf * S::VBUF, tb, tb + kKeyTile - 1 > lim_lo);
    if (it + 1 < n_tiles)
      store_tile_lds<D, NTW, BS, W>(sK + (buf ^ 1) * S::KBUF, sV + (buf ^ 1) * S::VBUF, kreg, vreg, plan,
                                    tb + kKeyTile, L, tb + 2 * kKeyTile > L);
    if (it + 2 < n_tiles) issue(raw, kreg, vreg);
    fetch_pages(it + 3, raw);
    __syncthreads();
  }

  if (!wave_rows) return;
  OutT* out = reinterpret_cast<OutT*>(a.out);
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    // every element of ol is the row sum of the rounded P of this lane's row
    const float lr = ol[nt][0];
    const float inv = lr > 0.f ? 1.f / lr : 0.f;
    if (tok[nt] < 0) continue;
    const size_t rh = (size_t)tok[nt] * a.num_heads + head[nt];
    if (uo.part_out) {
      // P = 2^(s * sl2 - mu): the row's log2 partition function is mu + log2(l)
      float* dst = uo.part_out + (rh * uo.slots + uo.slot) * D + 4 * q;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) store4(dst + dt * 16, o[nt][dt] * inv);
      if (q == 0) uo.part_lse[rh * uo.slots + uo.slot] = lr > 0.f ? (mu[nt] + __log2f(lr)) * kLn2 : -INFINITY;
    } else {
      OutT* dst = out + rh * D + 4 * q;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) store4(dst + dt * 16, o[nt][dt] * inv);
    }
  }
}

constexpr int kLdsNTW = 2;

// LDS of a work-group that runs either a prefill unit or a decode partition.
template <int D, int NT, int W = kWaves>
struct MixedLds {
  typedef PrefillLds<D, kLdsNTW, W> S;
  static constexpr int kPrefillBytes = S::kBytes;
  static constexpr int kDecodeBytes = DecodeMergeLds<D, NT, W>::kFloats * 4;
  static constexpr int kBytes = kPrefillBytes > kDecodeBytes ? kPrefillBytes : kDecodeBytes;
};

}  // namespace

}  // namespace gqa
