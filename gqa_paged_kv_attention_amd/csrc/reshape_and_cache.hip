// reshape_and_cache: write this step's keys/values into the paged caches.
//
// Incoming key/value rows are [tokens, num_kv_heads, head_dim] ("[Performance]
// Use optimized kernels for MQA/GQA", opening post, item 1).  New token j of
// sequence b is the sequence's position seq_lens[b] - q_len + j; it lands in
// page block_tables[b][pos / bs] at slot pos % bs.  Keys go to the token-major
// key page ([bs][d]); values to the channel-major value page ([d][bs]).  The
// copy moves bit patterns, so it is exact for any storage dtype.  Pages hold
// bs = 16, 32 or 64 tokens.
#include "gqa_common.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kThreads = 256;
constexpr int kLdsSeqs = 4095;          // query_start_loc staged in LDS up to this many sequences

// One thread per (token, kv head, 16-byte chunk of the head): VEC elements.
// The thread first guesses that token tok is the single new token of sequence
// tok (a decode step): query_start_loc[tok], query_start_loc[tok + 1] and
// seq_lens[tok] are loaded together with the source row, and only when the
// guess fails does it search query_start_loc (staged in LDS by the work-group
// when the batch is small enough, else in memory).  The work-group-wide
// staging therefore sits behind a uniform branch that decode steps skip.
template <int D, int BS, class T>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(CacheWriteArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CH = D / VEC;
  __shared__ int s_qsl[kLdsSeqs + 1];
  const long long gid = (long long)blockIdx.x * kThreads + threadIdx.x;
  const long long per_tok = (long long)a.num_kv_heads * CH;
  const bool active = gid < (long long)a.num_tokens * per_tok;
  const int tok = active ? (int)(gid / per_tok) : 0;
  const int rem = active ? (int)(gid % per_tok) : 0;
  const int kv = rem / CH, c = rem % CH;
  // the source row does not depend on the sequence: start its loads early
  const size_t src = ((size_t)tok * a.num_kv_heads + kv) * D + c * VEC;
  uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
  if (active) {
    kx = ld16(reinterpret_cast<const T*>(a.key) + src);
    vx = ld16(reinterpret_cast<const T*>(a.value) + src);
  }
  const int guess = min(tok, a.num_seqs - 1);
  // without query_start_loc, token t is sequence t's single new token
  int q0 = a.query_start_loc ? a.query_start_loc[guess] : guess;
  int q1 = a.query_start_loc ? a.query_start_loc[guess + 1] : guess + 1;
  int len = a.seq_lens[guess];
  int b = guess;
  const bool hit = q0 <= tok && tok < q1;
  if (a.query_start_loc && __syncthreads_and(hit || !active) == 0) {
    // some token of the work-group is not in its guessed sequence: search
    const bool staged = a.num_seqs <= kLdsSeqs;
    if (staged)
      for (int i = threadIdx.x; i <= a.num_seqs; i += kThreads) s_qsl[i] = a.query_start_loc[i];
    __syncthreads();
    if (active && !hit) {
      // sequence owning this token: last b with query_start_loc[b] <= tok
      int lo = 0, hi = a.num_seqs;           // invariant: qsl[lo] <= tok < qsl[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        const int v = staged ? s_qsl[mid] : a.query_start_loc[mid];
        if (v <= tok) lo = mid; else hi = mid;
      }
      b = lo;
      q0 = staged ? s_qsl[b] : a.query_start_loc[b];
      q1 = staged ? s_qsl[b + 1] : a.query_start_loc[b + 1];
      len = a.seq_lens[b];
    }
  }
  if (!active) return;
  if (tok < q0 || tok >= q1) return;
  const int pos = len - (q1 - q0) + (tok - q0);
  if (pos < 0 || pos >= a.max_blocks_per_seq * BS) return;
  const int page = a.block_tables[(size_t)b * a.max_blocks_per_seq + pos / BS];
  if ((unsigned)page >= (unsigned)a.num_blocks) return;
  const int slot = pos % BS;

  const size_t pbase = ((size_t)page * a.num_kv_heads + kv) * (size_t)(BS * D);
  *reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.key_cache) + pbase + (size_t)slot * D + c * VEC) = kx;
  T vals[VEC];
  __builtin_memcpy(vals, &vx, 16);
  T* vdst = reinterpret_cast<T*>(a.value_cache) + pbase + (size_t)(c * VEC) * BS + slot;
#pragma unroll
  for (int e = 0; e < VEC; ++e) vdst[(size_t)e * BS] = vals[e];
}

// Batches with prefill chunks: one work-group per 16-position group of a
// sequence's new positions, for every kv head.  A sequence's new positions
// [seq_len - q_len, seq_len) are cut at multiples of 16; each group lies in one
// page (pages hold 16, 32 or 64 tokens).  Key rows are token-major: the group's
// rows are copied as 16-byte chunks.  In the channel-major value page the
// group's values of channel d are one 32-byte (bf16) or 64-byte (fp32) run, so
// the work-group stages the group's value rows in LDS and writes each run whole
// from there, the lanes of one run side by side in one store instruction; the
// run is read first when the group is partial (the other slots keep what they
// hold).  Writing one element per store instead leaves partial sectors, which
// memory completes with a read (0.6 TB/s on a batch of 8k new tokens).  Kv
// heads go through LDS kCwPassBytes at a time.  Precondition (as in any paged
// allocator): a page receiving one sequence's new tokens receives no other
// sequence's.  The work-group finds its sequence by a scan of the per-sequence
// group counts, kThreads sequences at a time.
constexpr int kGroup = 16;
constexpr int kGroupMaxSeqs = 1024;
constexpr int kCwPassBytes = 32768;      // value rows staged per pass (before padding)

template <int D, int BS, class T>
__global__ __launch_bounds__(kThreads) void cache_write_group_kernel(CacheWriteArgs a) {
  constexpr int E = 16 / (int)sizeof(T);              // elements per 16-byte chunk
  constexpr int CPR = D / E;                          // chunks per row (one token, one kv head)
  constexpr int RUN = kGroup / E;                     // chunks per value run
  constexpr int KVP = kCwPassBytes / (kGroup * D * (int)sizeof(T));   // kv heads per pass
  // LDS row stride (elements): one 16-byte chunk of padding, so that the rows
  // the lanes of one run read (8 apart) fall on different banks
  constexpr int ROW = D + E;
  static_assert(KVP >= 1 && RUN >= 1, "pass and run sizes");
  __shared__ __attribute__((aligned(16))) T s_v[KVP * kGroup * ROW];
  __shared__ int s_tot[kThreads / 64];
  __shared__ int s_found[5];                 // sequence, group index, q0, first new position, seq_len
  const int g = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_found[0] = -1;
  __syncthreads();
  int base = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += kThreads) {
    const int b = c0 + threadIdx.x;
    int cnt = 0, q0 = 0, p0 = 0, L = 0;
    if (b < a.num_seqs) {
      q0 = a.query_start_loc[b];
      const int q1 = a.query_start_loc[b + 1];
      L = a.seq_lens[b];
      p0 = L - (q1 - q0);
      if (q1 > q0 && q1 <= a.num_tokens && q0 >= 0 && p0 >= 0) cnt = (L - 1) / kGroup - p0 / kGroup + 1;
    }
    int x = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_tot[w] = x;
    __syncthreads();
    int incl = base + x, total = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) {
      incl += i < w ? s_tot[i] : 0;
      total += s_tot[i];
    }
    if (cnt > 0 && g >= incl - cnt && g < incl) {
      s_found[0] = b;
      s_found[1] = g - (incl - cnt);
      s_found[2] = q0;
      s_found[3] = p0;
      s_found[4] = L;
    }
    base += total;
    __syncthreads();
    if (s_found[0] >= 0) break;                // uniform (read after the barrier)
  }
  const int b = s_found[0];
  if (b < 0) return;
  const int q0 = s_found[2], p0 = s_found[3], L = s_found[4];
  const int P = (p0 / kGroup + s_found[1]) * kGroup;    // first position of the group
  const int cap = a.max_blocks_per_seq * BS;
  const int lo = max(P, p0), hi = min(min(P + kGroup, L), cap);
  if (lo >= hi) return;
  const int page = a.block_tables[(size_t)b * a.max_blocks_per_seq + P / BS];
  if ((unsigned)page >= (unsigned)a.num_blocks) return;
  const int Hkv = a.num_kv_heads;
  const int slot0 = P % BS;
  const bool partial = lo > P || hi < P + kGroup;
  const T* key = reinterpret_cast<const T*>(a.key);
  const T* value = reinterpret_cast<const T*>(a.value);
  for (int kv0 = 0; kv0 < Hkv; kv0 += KVP) {
    const int nkv = min(KVP, Hkv - kv0);
    // key rows to their page rows, value rows to LDS: chunk i = (kv, row j, chunk c)
    for (int i = threadIdx.x; i < nkv * kGroup * CPR; i += kThreads) {
      const int c = i % CPR, j = (i / CPR) % kGroup, kvl = i / (CPR * kGroup);
      const int pos = P + j;
      if (pos < lo || pos >= hi) continue;
      const size_t src = ((size_t)(q0 + pos - p0) * Hkv + kv0 + kvl) * D + c * E;
      const uint4 kx = ld16(key + src), vx = ld16(value + src);
      const size_t pbase = ((size_t)page * Hkv + kv0 + kvl) * (size_t)(BS * D);
      *reinterpret_cast<uint4*>(reinterpret_cast<T*>(a.key_cache) + pbase + (size_t)(slot0 + j) * D + c * E) = kx;
      *reinterpret_cast<uint4*>(s_v + (kvl * kGroup + j) * ROW + c * E) = vx;
    }
    __syncthreads();
    // value runs: output chunk i = (kv, channel d, chunk q of the run), q fastest
    for (int i = threadIdx.x; i < nkv * D * RUN; i += kThreads) {
      const int qq = i % RUN, d = (i / RUN) % D, kvl = i / (RUN * D);
      const size_t pbase = ((size_t)page * Hkv + kv0 + kvl) * (size_t)(BS * D);
      T* dst = reinterpret_cast<T*>(a.value_cache) + pbase + (size_t)d * BS + slot0 + qq * E;
      T vals[E];
      if (partial) *reinterpret_cast<uint4*>(vals) = ld16(dst);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = qq * E + e, pos = P + j;
        if (pos >= lo && pos < hi) vals[e] = s_v[(kvl * kGroup + j) * ROW + d];
      }
      *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(vals);
    }
    __syncthreads();                           // s_v is refilled by the next pass
  }
}

template <class T>
hipError_t dispatch(const CacheWriteArgs& a, int D, int block_size, hipStream_t s) {
  // A decode step, or few new tokens per sequence, or so many sequences that
  // each work-group's scan of them would cost more than the stores it saves:
  // one thread per 16-byte chunk, two dependent loads.  Prefill chunks (on
  // average four or more new tokens per sequence, up to 1024 sequences): the
  // grouped kernel.
  if (!a.query_start_loc || (long long)a.num_tokens < 4LL * a.num_seqs || a.num_seqs > kGroupMaxSeqs) {
    const long long total = (long long)a.num_tokens * a.num_kv_heads * (D * (long long)sizeof(T) / 16);
    const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
    return with_block_size(block_size, [&](auto bs) {
      constexpr int BS = decltype(bs)::value;
      if (D == 64) return launch_kernel(cache_write_kernel<64, BS, T>, dim3(blocks), dim3(kThreads), 0, s, a);
      return launch_kernel(cache_write_kernel<128, BS, T>, dim3(blocks), dim3(kThreads), 0, s, a);
    });
  }
  // groups: each sequence's new positions touch at most q_len / 16 + 2 of them
  const long long groups = (long long)a.num_tokens / kGroup + 2LL * a.num_seqs + 1;
  if (groups > 0x7fffffffLL) return hipErrorInvalidValue;
  return with_block_size(block_size, [&](auto bs) {
    constexpr int BS = decltype(bs)::value;
    const dim3 grid((unsigned)groups);
    if (D == 64) return launch_kernel(cache_write_group_kernel<64, BS, T>, grid, dim3(kThreads), 0, s, a);
    return launch_kernel(cache_write_group_kernel<128, BS, T>, grid, dim3(kThreads), 0, s, a);
  });
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, int head_dim, int block_size, bool kv_f32,
                              hipStream_t stream) {
  return kv_f32 ? dispatch<float>(a, head_dim, block_size, stream)
                : dispatch<uint16_t>(a, head_dim, block_size, stream);
}

}  // namespace gqa
