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

template <class T>
hipError_t dispatch(const CacheWriteArgs& a, int D, int block_size, hipStream_t s) {
  const long long total = (long long)a.num_tokens * a.num_kv_heads * (D * (long long)sizeof(T) / 16);
  const unsigned blocks = (unsigned)((total + kThreads - 1) / kThreads);
  return with_block_size(block_size, [&](auto bs) {
    constexpr int BS = decltype(bs)::value;
    if (D == 64)
      hipLaunchKernelGGL((cache_write_kernel<64, BS, T>), dim3(blocks), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((cache_write_kernel<128, BS, T>), dim3(blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  });
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteArgs& a, int head_dim, int block_size, bool kv_f32,
                              hipStream_t stream) {
  return kv_f32 ? dispatch<float>(a, head_dim, block_size, stream)
                : dispatch<uint16_t>(a, head_dim, block_size, stream);
}

}  // namespace gqa
