// MFMA throughput probe for gfx950: back-to-back v_mfma_f32_32x32x16_{bf16}
// on register-resident operands, the ceiling the attention kernels' matrix
// work is compared with.  The dense peak in AMD's specification assumes the
// 2.4 GHz shader clock; under sustained MFMA load the clock is set by the
// power limit and depends on how many operand bits toggle, so the probe runs
// on operands the caller fills (random values for a realistic ceiling,
// constants for the clock-limited upper bound).
//
// Each wavefront cycles four A and four B fragments through four independent
// accumulators (so no product waits for the previous one) and finally stores
// its accumulators with vector stores so nothing is optimised away.
#include "attn_common.hpp"
#include "../../include/attn_probe.h"

namespace {

using namespace attn;

constexpr int PROBE_THREADS = 256;

__global__ void __launch_bounds__(PROBE_THREADS) mfma_probe_kernel(const uint16_t* operands, float* out,
                                                                    int iters) {
  const int gtid = blockIdx.x * PROBE_THREADS + threadIdx.x;
  frag8_t a[4], b[4];
  const uint16_t* src = operands + (size_t)gtid * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = *(const frag8_t*)(src + 8 * i);
    b[i] = *(const frag8_t*)(src + 32 + 8 * i);
  }
  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (f32x16_t){};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = mfma32(Bf16Tag{}, a[(i + r) & 3], b[i], acc[i]);
  }
  f32x16_t s = acc[0] + acc[1] + acc[2] + acc[3];
  float* dst = out + (size_t)gtid * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) *(f32x4_t*)(dst + 4 * i) = (f32x4_t){s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
}

}  // namespace

extern "C" {

int attn_probe_mfma(const void* operands, float* out, int workgroups, int iters, void* stream) {
  if (!operands || !out) return 1;
  if (workgroups < 1 || iters < 1 || workgroups > (1 << 20)) return 2;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(PROBE_THREADS), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(operands), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

double attn_probe_mfma_flops(int workgroups, int iters) {
  // 16 products of 32 x 32 x 16 per wavefront and iteration, 4 wavefronts per workgroup
  return (double)workgroups * 4 * (double)iters * 16 * 2.0 * 32 * 32 * 16;
}

}  // extern "C"
