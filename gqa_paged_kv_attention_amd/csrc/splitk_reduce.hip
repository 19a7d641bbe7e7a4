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

// grid (Hq, B), one wave; lane handles channels lane, lane + 64, ...
template <int D, class OutT>
__global__ __launch_bounds__(kWave) void splitk_reduce_kernel(ReduceArgs a) {
  const int h = blockIdx.x, b = blockIdx.y;
  int row = b;
  if (a.query_start_loc) {
    const int q0 = a.query_start_loc[b], q1 = a.query_start_loc[b + 1];
    if (q1 - q0 != 1 || q1 > a.num_tokens || q0 < 0) return;
    row = q0;
  }
  int L = a.seq_lens[b];
  L = max(0, min(L, a.max_blocks_per_seq * kPage));
  const int n = min((L + a.partition_size - 1) / a.partition_size, a.max_partitions);
  if (a.skip_single && n <= 1) return;

  const size_t hb = (size_t)b * a.num_heads + h;
  const float* lse = a.partial_lse + hb * a.max_partitions;
  const float* po = a.partial_out + hb * a.max_partitions * D;
  OutT* out = reinterpret_cast<OutT*>(a.out) + ((size_t)row * a.num_heads + h) * D;

  float M = -INFINITY;
  for (int p = 0; p < n; ++p) M = fmaxf(M, lse[p]);
  if (M == -INFINITY) {
    for (int d = threadIdx.x; d < D; d += kWave) store1(out + d, 0.f);
    return;
  }
  float den = 0.f;
  for (int p = 0; p < n; ++p) den += fast_exp2((lse[p] - M) * kLog2e);
  const float inv = 1.f / den;
  for (int d = threadIdx.x; d < D; d += kWave) {
    float acc = 0.f;
    for (int p = 0; p < n; ++p) {
      const float w = fast_exp2((lse[p] - M) * kLog2e);
      if (w != 0.f) acc += w * po[(size_t)p * D + d];
    }
    store1(out + d, acc * inv);
  }
}

template <class OutT>
hipError_t dispatch(const ReduceArgs& a, int D, int num_seqs, hipStream_t s) {
  dim3 grid(a.num_heads, num_seqs);
  if (D == 64)
    hipLaunchKernelGGL((splitk_reduce_kernel<64, OutT>), grid, dim3(kWave), 0, s, a);
  else
    hipLaunchKernelGGL((splitk_reduce_kernel<128, OutT>), grid, dim3(kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs& a, int head_dim, bool out_f32, int num_seqs, hipStream_t stream) {
  return out_f32 ? dispatch<float>(a, head_dim, num_seqs, stream) : dispatch<uint16_t>(a, head_dim, num_seqs, stream);
}

}  // namespace gqa
