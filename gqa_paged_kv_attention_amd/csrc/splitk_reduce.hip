// Log-sum-exp merge of split-K decode partials.
//
// Partition p of a sequence left O_p (its normalised output) and lse_p (natural
// log of its softmax denominator, max shift included).  The unsplit result is
// sum_p exp(lse_p - LSE) O_p with LSE = log sum_p exp(lse_p): exact in real
// arithmetic, so the split is a pure performance choice.  Summation runs over
// p in increasing order, so the result is bitwise reproducible.
#include "gqa_common.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kUnroll = 16;

// grid (Hq, B), one thread per output channel; partitions are folded kUnroll
// at a time with independent loads and an online log-sum-exp.
template <int D, class OutT>
__global__ __launch_bounds__(D) void splitk_reduce_kernel(ReduceArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  int row = b;
  if (a.query_start_loc) {
    const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
    if (q1 - q0 != 1 || q1 > a.num_tokens || q0 < 0) return;
    row = q0;
  }
  const int L = max(0, min(a.seq_lens[b], a.max_blocks_per_seq * a.block_size));
  const int n = min((L + a.partition_size - 1) / a.partition_size, a.max_partitions);
  if (a.skip_single && n <= 1) return;
  const size_t hb = (size_t)b * a.num_heads + h;
  const float* lse = a.partial_lse + hb * a.max_partitions;
  const float* po = a.partial_out + hb * a.max_partitions * D + d;
  float M = -INFINITY, den = 0.f, acc = 0.f;
  for (int p = 0; p < n; p += kUnroll) {
    float lv[kUnroll], ov[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      lv[u] = p + u < n ? lse[p + u] : -INFINITY;
      ov[u] = p + u < n ? po[(size_t)(p + u) * D] : 0.f;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) bm = fmaxf(bm, lv[u]);
    const float nm = fmaxf(M, bm);
    const float nu = (nm == -INFINITY) ? 0.f : nm;
    const float r = fast_exp2((M - nu) * kLog2e);
    den *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float w = fast_exp2((lv[u] - nu) * kLog2e);
      den += w;
      acc += w == 0.f ? 0.f : w * ov[u];
    }
    M = nm;
  }
  OutT* out = reinterpret_cast<OutT*>(a.out);
  store1(out + ((size_t)row * a.num_heads + h) * D + d, den > 0.f ? acc / den : 0.f);
}

template <class OutT>
hipError_t dispatch(const ReduceArgs& a, int D, int num_seqs, hipStream_t s) {
  dim3 grid(a.num_heads, num_seqs);
  if (D == 64) return launch_kernel(splitk_reduce_kernel<64, OutT>, grid, dim3(64), 0, s, a);
  return launch_kernel(splitk_reduce_kernel<128, OutT>, grid, dim3(128), 0, s, a);
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, bool out_f32, int num_seqs, hipStream_t stream) {
  return out_f32 ? dispatch<float>(a, head_dim, num_seqs, stream) : dispatch<uint16_t>(a, head_dim, num_seqs, stream);
}

}  // namespace gqa
