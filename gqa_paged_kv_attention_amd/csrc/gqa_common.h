// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4).
//
// Matrix-core formulation.  For a tile of key tokens and a block of 16 query
// rows (a GQA group's heads, or (token, head) pairs of a prefill chunk):
//
//   S^T[t][r] = sum_d K[t][d] * Q[r][d]          A = K tile,  B = Q^T
//   O^T[d][r] += sum_t V^T[d][t] * P^T[t][r]     A = V^T tile, B = P^T
//
// With the key page stored token-major ([bs][d]) and the value page stored
// channel-major ([d][bs]), every A operand is a contiguous 16-byte load per
// lane, and the score fragment that the first product leaves in a lane is
// exactly the P^T fragment the second product needs from that lane, so the
// softmax runs in registers with no LDS round trip.
//
// Operand layouts of the 16x16 MFMAs used here (wave64, lane l, n = l % 16,
// q = l / 16):
//   A[m][k]: lane l holds row m = n and a run of k indices owned by group q
//   B[k][c]: lane l holds column c = n and the same run of k indices
//   D[m][c]: lane l holds column c = n, rows m = 4q + j (j = 0..3)
// Because the contraction index k only has to agree between A and B, the
// kernels are free to choose which memory element feeds which k slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gqa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kTile = 32;        // key tokens per tile (two 16-token halves)
constexpr int kHalf = 16;        // tokens per half tile; pages hold 16, 32 or 64 tokens
constexpr float kLog2e = 1.4426950408889634f;

// Host dispatch: call f(std::integral_constant<int, BS>) for a page size of
// 16, 32 or 64 tokens (the only sizes the library is built for).
template <class F>
auto with_block_size(int block_size, F f) {
  if (block_size == 64) return f(std::integral_constant<int, 64>{});
  if (block_size == 32) return f(std::integral_constant<int, 32>{});
  return f(std::integral_constant<int, 16>{});
}
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// bf16 (as 16-bit pattern) from float, round to nearest even (hardware convert).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ f32x4_t mfma_bf16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4_t mfma_f16(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                 0, 0, 0);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two bf16 (packed in a word) -> two fp16 (packed), round to nearest even (one
// v_cvt_pk_f16_f32).  Exact for magnitudes in [2^-14, 65504] (a bf16
// significand fits fp16's); smaller ones become fp16 subnormals (absolute
// error <= 2^-25, unbiased), larger ones overflow to infinity.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                          (f32x2_t{__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u)}),
                                          f16x2_t));
}

// Two fp32 -> two fp16 (packed), round to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), f16x2_t));
}

// A value the optimiser cannot see through (the empty asm emits nothing).
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// max(a, b) for non-NaN operands as one v_med3_f32(a, b, pinf), pinf = +inf
// made opaque: with a literal +inf the optimiser turns it back into fmaxf,
// which quiets NaNs first (an extra v_max_f32 per operand whose origin it
// cannot trace).
__device__ __forceinline__ float fmax_nn(float a, float b, float pinf) { return __builtin_amdgcn_fmed3f(a, b, pinf); }

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte load with the non-temporal hint, for K/V pages that a call reads
// once: the lines stream through instead of displacing others in L2 and the
// Infinity Cache.  On the Llama-3.1-8B decode batch (633 MB of K/V) the
// decode call went from 125.8 to 111.9 us with it; on 16 x 32k tokens from
// 373 to 340 us.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ float4 ld16f_stream(const float* p) {
  const f32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum across the four lane groups that share a row (lanes n, n+16,
// n+32, n+48).  v_permlane16_swap(x, x) returns, in its two results, x of this
// lane and of lane ^ 16 (in some order); v_permlane32_swap likewise for lane ^
// 32.  Both are VALU operations, so the reduction stays off the LDS pipe.
__device__ __forceinline__ float row_max4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float x0 = __uint_as_float(a[0]), x1 = __uint_as_float(a[1]);
  x = x0 > x1 ? x0 : x1;
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y0 = __uint_as_float(b[0]), y1 = __uint_as_float(b[1]);
  return y0 > y1 ? y0 : y1;
}

__device__ __forceinline__ float row_sum4(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Entry idx of a wave-uniform int32 row (a block-table row: every lane of a
// wave walks the same tile), read with a scalar load through the constant
// address space.  A vector load would queue in the compute unit's vector
// memory path behind the K/V loads of the other waves there, and the next
// tile's K/V loads cannot be issued before it returns (at the decode's start
// that wait was 5-20 us per wave).  The tables are not written while a kernel
// runs.
__device__ __forceinline__ int scalar_entry(const int32_t* row_ptr, int idx) {
  typedef const __attribute__((address_space(4))) int32_t* const_row;
  const uint64_t row = reinterpret_cast<uint64_t>(row_ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)row);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(row >> 32));
  return reinterpret_cast<const_row>(((uint64_t)hi << 32) | lo)[__builtin_amdgcn_readfirstlane(idx)];
}

// Page id through the block table, clamped into the pool so that a corrupt
// entry can give a wrong answer but never an out-of-bounds read.
__device__ __forceinline__ int page_at(const int32_t* bt_row, int idx, int num_blocks) {
  const int p = scalar_entry(bt_row, idx);
  return (unsigned)p < (unsigned)num_blocks ? p : 0;
}

// ---------------------------------------------------------------------------
// Tile operations, specialised by cache dtype and page size BS.  A "tile" is
// 32 key tokens of one kv head in two 16-token halves (A = tokens 0..15, B =
// tokens 16..31).  Each half lies inside one page: with 16-token pages the
// halves are two pages, with 32- or 64-token pages they are consecutive runs
// of one page, so the tile does not depend on the page size.  The loads take
// the address of each half's first token: key rows are D elements apart in
// any page, value channels BS elements apart.  Each lane ends a Q.K^T product
// holding 8 scores per 16-row block, indexed idx = 0..7; token_offset(q, idx)
// gives their key offsets inside the tile.
// ---------------------------------------------------------------------------

// bf16 caches: v_mfma_f32_16x16x32_bf16.
//  - Q.K^T: two products per 16-row block, each over 16 tokens.  Product s
//    feeds row m of A with token (m < 8 ? half A : half B), offset
//    (m & 3) + 8 * ((m >> 2) & 1) + 4 * s, and k slots 8q..8q+7 of chunk kk with
//    channels 32 kk + 8q .. +7.  Lane group q then holds tokens 8q + idx.
//  - P.V: one product per 16 channels over the whole 32-token tile; lane group
//    q supplies k slots 8q..8q+7 = tokens 8q .. 8q+7 (half q >= 2 ? B : A,
//    offsets 8 (q & 1) ..), a contiguous 16-byte run of the channel-major page.
//  - P is fed as a hi/lo pair of bf16 (p = hi + lo to ~2^-16 relative), so the
//    P.V product keeps fp32-grade weights.
//  - Stream: K/V loads carry the non-temporal hint (read once, do not keep
//    them in L2 / the last-level cache).  The host picks it per call from the
//    batch's K/V footprint: for a batch far larger than the last-level cache
//    the hint keeps the stream from evicting what is reused (Llama-3.1-8B
//    decode batch, 634 MB: 123 -> 111 us); a batch that fits is read again
//    from that cache by the next call on it, which the hint would forgo
//    (Llama-2-7B sweep with Hkv = 8, 273 MB: 48 us plain, 57 us with it).
template <int D, int BS, bool Stream = false>
struct TileBF16 {
  static constexpr int kBS = BS;
  // Value loads stream only when one 128-byte line of a channel does not hold
  // both tiles of a pair (64-token pages): the second tile's half of the line
  // must still be in L2 when it is asked for (with the hint, 64-token pages
  // went from 129 to 152 us on the Llama-3.1-8B decode batch).  Key loads
  // stream only with 64-token pages: with 16- and 32-token pages the hint on
  // the values alone is faster (Llama-3.1-8B decode step 114.6-114.9 ->
  // 109.8-110.5 us, its attention call 110.5-111.0 -> 107.5-107.7 us, the
  // Llama-2-7B sweep expanded to 32 kv heads 191.3-191.4 -> 182.1-182.7 us;
  // 64-token pages 125.2-125.6 -> 128.4-128.9 us, so they keep it).
  static constexpr bool kStreamK = Stream && BS * 2 > 64;
  static constexpr bool kStreamV = Stream && BS * 2 <= 64;
  static constexpr bool kPipelined = true;  // double-buffered tile loop
  static constexpr int KC = D / 32;   // 16-byte chunks per lane per Q.K^T product
  static constexpr int DT = D / 16;   // 16-channel blocks of the output
  struct K { uint4 v[2][KC]; };
  struct V { uint4 v[DT]; };
  struct Q { uint4 v[KC]; };
  typedef uint16_t elem_t;

  __device__ __forceinline__ static int token_offset(int q, int idx) { return 8 * q + idx; }
  __device__ __forceinline__ static int v_token_offset(int q, int e) { return 8 * q + e; }

  // kA/kB: key row of the first token of half A / B (rows D elements apart).
  __device__ __forceinline__ static void load_k(K& k, const elem_t* kA, const elem_t* kB, int lane) {
    const int m = lane & 15, q = lane >> 4;
    const elem_t* pg = (m < 8) ? kA : kB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int slot = (m & 3) + 8 * ((m >> 2) & 1) + 4 * s;
      const elem_t* row = pg + slot * D + 8 * q;
#pragma unroll
      for (int c = 0; c < KC; ++c) k.v[s][c] = kStreamK ? ld16_stream(row + 32 * c) : ld16(row + 32 * c);
    }
  }

  // vA/vB: channel-0 value of the first token of half A / B (channels BS
  // elements apart, [D][BS] pages).
  __device__ __forceinline__ static void load_v(V& v, const elem_t* vA, const elem_t* vB, int lane) {
    const int n = lane & 15, q = lane >> 4;
    const elem_t* pg = (q < 2) ? vA : vB;
    const elem_t* base = pg + n * BS + 8 * (q & 1);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) v.v[dt] = kStreamV ? ld16_stream(base + dt * 16 * BS) : ld16(base + dt * 16 * BS);
  }

  // row: query row base ([D] elements) or nullptr for a padding row.
  __device__ __forceinline__ static void load_q(Q& qf, const elem_t* row, int lane) {
    const int q = lane >> 4;
#pragma unroll
    for (int c = 0; c < KC; ++c) qf.v[c] = row ? ld16(row + 32 * c + 8 * q) : make_uint4(0, 0, 0, 0);
  }

  __device__ __forceinline__ static void qk(float s[8], const K& k, const Q& qf) {
    f32x4_t acc0 = zero4(), acc1 = zero4();
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      acc0 = mfma_bf16(k.v[0][c], qf.v[c], acc0);
      acc1 = mfma_bf16(k.v[1][c], qf.v[c], acc1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) { s[j] = acc0[j]; s[4 + j] = acc1[j]; }
  }

  // Zero value elements of tokens at or past `end` (offsets relative to the tile).
  __device__ __forceinline__ static void mask_v(V& v, int tile_base, int end, int lane) {
    const int q = lane >> 4;
    const int first = tile_base + 8 * q;
    uint32_t keep[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (first + 2 * w) < end ? 0xFFFFu : 0u;
      const uint32_t hi = (first + 2 * w + 1) < end ? 0xFFFF0000u : 0u;
      keep[w] = lo | hi;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      v.v[dt].x &= keep[0];
      v.v[dt].y &= keep[1];
      v.v[dt].z &= keep[2];
      v.v[dt].w &= keep[3];
    }
  }

  __device__ __forceinline__ static void pv(f32x4_t o[DT], const V& v, const float p[8]) {
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint16_t h0 = float_to_bf16_bits(p[2 * w]);
      const uint16_t h1 = float_to_bf16_bits(p[2 * w + 1]);
      const uint16_t l0 = float_to_bf16_bits(p[2 * w] - bf16_bits_to_float(h0));
      const uint16_t l1 = float_to_bf16_bits(p[2 * w + 1] - bf16_bits_to_float(h1));
      hi[w] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lo[w] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    const uint4 phi = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    const uint4 plo = make_uint4(lo[0], lo[1], lo[2], lo[3]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      o[dt] = mfma_bf16(v.v[dt], phi, o[dt]);
      o[dt] = mfma_bf16(v.v[dt], plo, o[dt]);
    }
  }
};

// fp32 caches: v_mfma_f32_16x16x4_f32 (exact fp32 products).
//  - Q.K^T: per half s, A row m = token m of the half; a 16-byte load gives
//    channels 16c + 4q .. +3, consumed by four products (k slot q <-> channel
//    16c+4q+i).  Lane group q then holds tokens 16 s + 4q + j.
//  - P.V: per half s and channel block, a 16-byte load of the channel-major
//    page gives tokens 4q .. 4q+3 of the half, consumed by four products (k
//    slot q <-> token 4q + i), whose B operand is the lane's own score for that
//    token.
template <int D, int BS>
struct TileF32 {
  static constexpr int kBS = BS;
  // Single-buffered tile loop.  Two fp32 register sets take the decode kernels
  // past 256 VGPRs (one wave per SIMD): on 32 sequences of 512..4096 tokens,
  // G = 4, the double-buffered loop took 119 us against 107 (d = 128) and 58
  // against 55 (d = 64).  (An earlier form of the double-buffered loop gave
  // wrong fp32 d = 64 results with a 4-tile stride; the current one, whose
  // visiting order is checked on the host, passes every GPU test and equals
  // the single-buffered loop bit for bit.)
  static constexpr bool kPipelined = false;
  static constexpr int KC = D / 16;
  static constexpr int DT = D / 16;
  struct K { float4 v[2][KC]; };
  struct V { float4 v[2][DT]; };
  struct Q { float4 v[KC]; };
  typedef float elem_t;

  __device__ __forceinline__ static int token_offset(int q, int idx) {
    return 16 * (idx >> 2) + 4 * q + (idx & 3);
  }

  __device__ __forceinline__ static void load_k(K& k, const elem_t* kA, const elem_t* kB, int lane) {
    const int m = lane & 15, q = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const elem_t* row = (s ? kB : kA) + m * D + 4 * q;
#pragma unroll
      for (int c = 0; c < KC; ++c) k.v[s][c] = ld16f_stream(row + 16 * c);
    }
  }

  __device__ __forceinline__ static void load_v(V& v, const elem_t* vA, const elem_t* vB, int lane) {
    const int n = lane & 15, q = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const elem_t* base = (s ? vB : vA) + n * BS + 4 * q;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        v.v[s][dt] = BS * 4 <= 64 ? ld16f_stream(base + dt * 16 * BS) : *reinterpret_cast<const float4*>(base + dt * 16 * BS);
    }
  }

  __device__ __forceinline__ static void load_q(Q& qf, const elem_t* row, int lane) {
    const int q = lane >> 4;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      qf.v[c] = row ? *reinterpret_cast<const float4*>(row + 16 * c + 4 * q) : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  __device__ __forceinline__ static void qk(float s[8], const K& k, const Q& qf) {
    f32x4_t acc0 = zero4(), acc1 = zero4();
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      acc0 = mfma_f32(k.v[0][c].x, qf.v[c].x, acc0);
      acc0 = mfma_f32(k.v[0][c].y, qf.v[c].y, acc0);
      acc0 = mfma_f32(k.v[0][c].z, qf.v[c].z, acc0);
      acc0 = mfma_f32(k.v[0][c].w, qf.v[c].w, acc0);
      acc1 = mfma_f32(k.v[1][c].x, qf.v[c].x, acc1);
      acc1 = mfma_f32(k.v[1][c].y, qf.v[c].y, acc1);
      acc1 = mfma_f32(k.v[1][c].z, qf.v[c].z, acc1);
      acc1 = mfma_f32(k.v[1][c].w, qf.v[c].w, acc1);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) { s[j] = acc0[j]; s[4 + j] = acc1[j]; }
  }

  __device__ __forceinline__ static void mask_v(V& v, int tile_base, int end, int lane) {
    const int q = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int first = tile_base + 16 * s + 4 * q;
      const bool k0 = first < end, k1 = first + 1 < end, k2 = first + 2 < end, k3 = first + 3 < end;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        float4& x = v.v[s][dt];
        x.x = k0 ? x.x : 0.f;
        x.y = k1 ? x.y : 0.f;
        x.z = k2 ? x.z : 0.f;
        x.w = k3 ? x.w : 0.f;
      }
    }
  }

  __device__ __forceinline__ static void pv(f32x4_t o[DT], const V& v, const float p[8]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        o[dt] = mfma_f32(v.v[s][dt].x, p[4 * s + 0], o[dt]);
        o[dt] = mfma_f32(v.v[s][dt].y, p[4 * s + 1], o[dt]);
        o[dt] = mfma_f32(v.v[s][dt].z, p[4 * s + 2], o[dt]);
        o[dt] = mfma_f32(v.v[s][dt].w, p[4 * s + 3], o[dt]);
      }
    }
  }
};

// Locate this work-group's (sequence, row tile) among the row tiles of the
// sequences with more than one query token (ceil(q_len * G / rows_per_group)
// tiles each, in sequence order): a block-wide scan of the tile counts, in
// chunks of NTHR sequences, one entry of s_scan per thread.  The work-group
// must have exactly NTHR threads (the caller's launch bound), so that every
// thread's entry exists.  Returns the sequence (or -1 past the last tile) and
// the tile's index within it.
template <int NTHR>
__device__ __forceinline__ int locate_prefill_tile(const int32_t* qsl, int num_seqs, int G, int rows_per_group,
                                                   int tile, int (&s_scan)[NTHR], int* s_found, int* local_tile) {
  constexpr int nthr = NTHR;
  if (threadIdx.x == 0) s_found[0] = -1;
  int base = 0;
  for (int c0 = 0; c0 < num_seqs; c0 += nthr) {
    const int bb = c0 + threadIdx.x;
    int cnt = 0;
    if (bb < num_seqs) {
      const int ql = qsl[bb + 1] - qsl[bb];
      cnt = (ql > 1) ? (ql * G + rows_per_group - 1) / rows_per_group : 0;
    }
    s_scan[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < nthr; off <<= 1) {
      const int add = (threadIdx.x >= off) ? s_scan[threadIdx.x - off] : 0;
      __syncthreads();
      s_scan[threadIdx.x] += add;
      __syncthreads();
    }
    const int total = s_scan[nthr - 1];
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
  *local_tile = s_found[1];
  return s_found[0];
}

// Store 4 consecutive output channels (fp32 values) as fp32 or bf16.
__device__ __forceinline__ void store4(float* dst, f32x4_t x) {
  *reinterpret_cast<float4*>(dst) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store4(uint16_t* dst, f32x4_t x) {
  const uint32_t a = (uint32_t)float_to_bf16_bits(x[0]) | ((uint32_t)float_to_bf16_bits(x[1]) << 16);
  const uint32_t b = (uint32_t)float_to_bf16_bits(x[2]) | ((uint32_t)float_to_bf16_bits(x[3]) << 16);
  *reinterpret_cast<uint2*>(dst) = make_uint2(a, b);
}
__device__ __forceinline__ void store1(float* dst, float x) { *dst = x; }
__device__ __forceinline__ void store1(uint16_t* dst, float x) { *dst = float_to_bf16_bits(x); }

}  // namespace gqa
