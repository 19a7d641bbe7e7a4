// Measurement probe (not part of the attention path): the bf16 matrix-core
// issue rate this device sustains, against which the prefill's matrix
// utilisation is read beside the published peak.
//
// Every wave runs kChains independent accumulation chains of
// v_mfma_f32_16x16x32_bf16 (16 x 16 x 32 multiply-adds each, 16384 flops) for
// `iters` rounds: independent chains keep the matrix pipe issuing back to back
// instead of waiting on a dependent result.  The accumulators are summed into
// `out` (one float per wave) so that nothing is optimised away.
#include "gqa_common.h"
#include "gqa_internal.h"

namespace gqa {

namespace {

constexpr int kProbeChains = 8;
constexpr int kProbeWaves = 4;

// Eight chains with distinct operands and starting values, so that no two
// compute the same thing.
__global__ __launch_bounds__(kProbeWaves * kWave) void mfma_rate_kernel(float* out, int iters) {
  const int lane = lane_id();
  const uint4 a = make_uint4(0x3F803F80u ^ lane, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);   // bf16 ~1.0
  uint4 b[kProbeChains];
  f32x4_t c[kProbeChains];
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k) {
    b[k] = make_uint4(0x3C003C00u + k, 0x3C003C00u, 0x3C003C00u ^ (k << 16), 0x3C003C00u);
    c[k] = f32x4_t{(float)k, 0.f, 0.f, (float)lane};
  }
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kProbeChains; ++k) {
      c[k] = mfma_bf16(a, b[k], c[k]);
    }
  }
  f32x4_t s4 = c[0];
#pragma unroll
  for (int k = 1; k < kProbeChains; ++k) s4 += c[k];
  if (lane == 0) out[blockIdx.x * kProbeWaves + threadIdx.x / kWave] = s4[0] + s4[1] + s4[2] + s4[3];
}

}  // namespace

hipError_t launch_mfma_probe(float* out, int groups, int iters, hipStream_t stream) {
  return launch_kernel(mfma_rate_kernel, dim3(groups), dim3(kProbeWaves * kWave), 0, stream, out, iters);
}

long long mfma_probe_flops(int groups, int iters) {
  return (long long)groups * kProbeWaves * iters * kProbeChains * 16LL * 16 * 32 * 2;
}

}  // namespace gqa
