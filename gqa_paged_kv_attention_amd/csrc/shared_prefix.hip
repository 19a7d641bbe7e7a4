// Decode over a batch whose sequences share prompt prefixes, bf16.
//
// With automatic prefix caching, sequences that start with the same prompt
// have block tables that point at the same physical pages for that prompt
// ("[Kernel] [V1] Further optimizations to ROCm (Triton) Backend to better
// handle GQA", benchmark discussion: prefix caching changes the measured
// results, so the server is restarted between runs).  A plain decode still
// streams the shared pages once per sequence.  Here the sequences of a group
// are attended to the shared part together: their query rows (G heads of each
// member per kv head) form the rows of prefill-role units that read each
// shared K/V tile once for the whole group and multiply it on the matrix
// cores.  Each member's remaining keys are decoded on their own.  Every unit
// leaves a normalised partial and its log-sum-exp; a merge kernel combines
// them per (sequence, head), which gives the same softmax as one pass over
// all keys (the split-K identity).
//
// The shared part of group g is its prefix rounded down to whole 64-key
// tiles, S = 64 floor(prefix_lens[g] / 64); keys [S, seq_len) of each member
// belong to its own decode.  Shared keys are read through the block table of
// the group's first member.
#include "prefill_core.h"

namespace gqa {

namespace {

// Shared part of a group with this prefix length (keys): whole 64-key tiles,
// within what a block table addresses and the prefix chunk slots hold.
template <int BS>
__device__ __forceinline__ int shared_keys(const SharedPrefixArgs& a, int prefix_len) {
  const int cap = min(a.prefill.max_blocks_per_seq * BS, a.prefix_chunks * a.chunk_tokens);
  return max(0, min(prefix_len, cap)) / kKeyTile * kKeyTile;
}

// Work-group i runs unit i / Hkv for kv head i % Hkv: the prefix units
// (num_groups x row_tiles x prefix_chunks, matrix-bound and the longest) come
// first, then the suffix units (B x suffix partitions).  Spreading the prefix
// units through the launch, in proportion to the suffix units, was measured
// slower: the last prefix units then start late and set the end of the launch.
template <int D, int NT, int BS, class OutT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1)))
void shared_prefix_kernel(SharedPrefixArgs a) {
  typedef PrefillLds<D, kLdsNTW> S;
  __shared__ __attribute__((aligned(16))) char lds[MixedLds<D, NT>::kBytes];
  __shared__ int s_group;
  const int Hkv = a.prefill.num_kv_heads, G = a.prefill.group;
  const int kv = blockIdx.x % Hkv;
  const long long n_prefix = (long long)a.num_groups * a.row_tiles * a.prefix_chunks;
  const long long unit = blockIdx.x / Hkv;
  if (unit < n_prefix) {
    const int u = (int)unit;
    const int c = u % a.prefix_chunks;
    const int rt = (u / a.prefix_chunks) % a.row_tiles;
    const int g = u / (a.prefix_chunks * a.row_tiles);
    const int g0 = a.group_start[g], g1 = a.group_start[g + 1];
    const int shared = shared_keys<BS>(a, a.prefix_lens[g]);
    if (g0 < 0 || g1 > a.num_seqs || g1 <= g0) return;
    if (c * a.chunk_tokens >= shared || rt * S::kRowsPerGroup >= (g1 - g0) * G) return;
    const int k1 = min((c + 1) * a.chunk_tokens, shared);
    UnitOut uo;
    uo.part_out = a.part_out;
    uo.part_lse = a.part_lse;
    uo.slot = c;
    uo.slots = a.slots;
    uint16_t* sK = reinterpret_cast<uint16_t*>(lds);
    // the group's decode queries are rows g0 .. g1 - 1: a chunk of g1 - g0
    // rows against keys [c * PC, k1) of the first member, no causal mask
    prefill_unit<D, kLdsNTW, BS, OutT>(a.prefill, g0, rt, g0, g1, k1, kv, sK, sK + 2 * S::KBUF,
                                       c * a.chunk_tokens / kKeyTile, uo);
    return;
  }
  const int u = (int)(unit - n_prefix);
  const int nparts = a.decode.max_partitions;
  const int p = u % nparts, b = u / nparts;
  const int L = clamp_len(a.decode.seq_lens[b], a.decode.max_blocks_per_seq, BS);
  // group of sequence b: the one whose [group_start[t], group_start[t + 1]) holds b
  // (chunks of kThreads groups; every thread reads the result into a register
  // before the barrier that lets any thread write the next chunk's, so all
  // threads leave the loop after the same chunk)
  if (threadIdx.x == 0) s_group = -1;
  __syncthreads();
  int g = -1;
  for (int t0 = 0; t0 < a.num_groups; t0 += kThreads) {
    const int t = t0 + threadIdx.x;
    if (t < a.num_groups && a.group_start[t] <= b && b < a.group_start[t + 1]) s_group = t;
    __syncthreads();
    g = s_group;
    __syncthreads();
    if (g >= 0) break;
  }
  const int shared = g >= 0 ? shared_keys<BS>(a, a.prefix_lens[g]) : 0;
  const int rest = min(L, shared + nparts * a.decode.partition_size) - shared;
  const int n_sp = rest > 0 ? (rest + a.decode.partition_size - 1) / a.decode.partition_size : 0;
  if (p == 0 && kv == 0 && threadIdx.x == 0)
    a.seq_meta[b] = make_int2((shared + a.chunk_tokens - 1) / a.chunk_tokens, n_sp);
  if (p >= n_sp) return;                 // before the query loads: most slots of short suffixes are empty
  UnitOut uo;
  uo.part_out = a.part_out;
  uo.part_lse = a.part_lse;
  uo.slot = a.prefix_chunks;
  uo.slots = a.slots;
  decode_partition_at<TileBF16<D, BS>, D, NT, OutT>(a.decode, p, kv, b, b, L, reinterpret_cast<float*>(lds), shared,
                                                    &uo);
}

// grid (Hq, B), one thread per channel: merge the prefix chunks [0, n_pc) and
// the suffix partitions [MC, MC + n_sp) of (sequence, head) in slot order.
constexpr int kMergeUnroll = 8;

template <int D, class OutT>
__global__ __launch_bounds__(D) void shared_prefix_merge_kernel(SharedPrefixArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int2 meta = a.seq_meta[b];
  const int n = meta.x + meta.y;
  const size_t hb = (size_t)b * a.prefill.num_heads + h;
  const float* lse = a.part_lse + hb * a.slots;
  const float* po = a.part_out + hb * a.slots * D + d;
  float M = -INFINITY, den = 0.f, acc = 0.f;
  for (int i = 0; i < n; i += kMergeUnroll) {
    float lv[kMergeUnroll], ov[kMergeUnroll];
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) {
      const int j = i + k;
      const int s = j < meta.x ? j : a.prefix_chunks + (j - meta.x);
      lv[k] = j < n ? lse[s] : -INFINITY;
      ov[k] = j < n ? po[(size_t)s * D] : 0.f;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) bm = fmaxf(bm, lv[k]);
    const float nm = fmaxf(M, bm);
    const float nu = (nm == -INFINITY) ? 0.f : nm;
    const float r = fast_exp2((M - nu) * kLog2e);
    den *= r;
    acc *= r;
#pragma unroll
    for (int k = 0; k < kMergeUnroll; ++k) {
      const float w = fast_exp2((lv[k] - nu) * kLog2e);
      den += w;
      acc += w == 0.f ? 0.f : w * ov[k];
    }
    M = nm;
  }
  OutT* out = reinterpret_cast<OutT*>(a.prefill.out);
  store1(out + hb * D + d, den > 0.f ? acc / den : 0.f);
}

template <int D, int BS, class OutT>
hipError_t dispatch(const SharedPrefixArgs& a, hipStream_t s) {
  const long long groups = (long long)a.num_groups * a.row_tiles * a.prefix_chunks * a.prefill.num_kv_heads +
                           (long long)a.num_seqs * a.decode.max_partitions * a.prefill.num_kv_heads;
  if (groups > 0) {
    const hipError_t e =
        a.prefill.group <= 16
            ? launch_kernel(shared_prefix_kernel<D, 1, BS, OutT>, dim3((unsigned)groups), dim3(kThreads), 0, s, a)
            : launch_kernel(shared_prefix_kernel<D, 2, BS, OutT>, dim3((unsigned)groups), dim3(kThreads), 0, s, a);
    if (e != hipSuccess) return e;
  }
  return launch_kernel(shared_prefix_merge_kernel<D, OutT>, dim3(a.prefill.num_heads, a.num_seqs), dim3(D), 0, s, a);
}

}  // namespace

hipError_t launch_shared_prefix(const SharedPrefixArgs& a, int head_dim, int block_size, bool out_f32,
                                hipStream_t stream) {
  return with_block_size(block_size, [&](auto bs) {
    constexpr int BS = decltype(bs)::value;
    if (head_dim == 64)
      return out_f32 ? dispatch<64, BS, float>(a, stream) : dispatch<64, BS, uint16_t>(a, stream);
    return out_f32 ? dispatch<128, BS, float>(a, stream) : dispatch<128, BS, uint16_t>(a, stream);
  });
}

}  // namespace gqa
