// Throughput probes for gfx950 (the ceilings the attention kernels are
// compared with), starting with back-to-back v_mfma_f32_32x32x16_{bf16}
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

// v_exp_f32 throughput: eight independent chains x <- 2^(-x) per lane (x
// stays in (0.5, 1)), so every instruction is one exponential.
__global__ void __launch_bounds__(PROBE_THREADS) exp_probe_kernel(const float* in, float* out, int iters) {
  const int gtid = blockIdx.x * PROBE_THREADS + threadIdx.x;
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = 0.5f + 0.4f * fabsf(in[(size_t)gtid * 8 + i]) / (1.0f + fabsf(in[(size_t)gtid * 8 + i]));
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(-x[i]);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i];
  out[gtid] = s;
}

// LDS read bandwidth: each thread issues blocks of eight 16-byte reads
// (ds_read_b128, consecutive lanes on consecutive 16-byte chunks, so no bank
// conflicts) and waits for them inside the same asm block; one XOR per read
// keeps every result live.  Wavefront 0 of workgroup 0 also records the
// shader-clock and 100 MHz counters around its loop (clock = ratio).
__global__ void __launch_bounds__(PROBE_THREADS) lds_probe_kernel(float* out, unsigned long long* clk, int iters) {
  __shared__ __attribute__((aligned(16))) uint32_t buf[8192];  // 32 KiB
  const int tid = threadIdx.x;
  for (int i = tid; i < 8192; i += PROBE_THREADS) buf[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  const uint32_t addr = (uint32_t)(tid * 16);  // byte offset; reads span [0, 32 KiB)
  u32x4_t r0, r1, r2, r3, r4, r5, r6, r7;
  uint32_t acc = 0;
  const unsigned long long c0 = __builtin_amdgcn_s_memtime(), t0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:4096\n\t"
        "ds_read_b128 %2, %8 offset:8192\n\t"
        "ds_read_b128 %3, %8 offset:12288\n\t"
        "ds_read_b128 %4, %8 offset:16384\n\t"
        "ds_read_b128 %5, %8 offset:20480\n\t"
        "ds_read_b128 %6, %8 offset:24576\n\t"
        "ds_read_b128 %7, %8 offset:28672\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3), "=v"(r4), "=v"(r5), "=v"(r6), "=v"(r7)
        : "v"(addr)
        : "memory");
    acc ^= r0[it & 3] ^ r1[(it + 1) & 3] ^ r2[(it + 2) & 3] ^ r3[(it + 3) & 3] ^ r4[it & 3] ^ r5[(it + 1) & 3] ^
           r6[(it + 2) & 3] ^ r7[(it + 3) & 3];
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime(), t1 = __builtin_amdgcn_s_memrealtime();
  out[blockIdx.x * PROBE_THREADS + tid] = __builtin_bit_cast(float, acc);
  if (blockIdx.x == 0 && tid == 0) {
    clk[0] = c1 - c0;
    clk[1] = t1 - t0;
  }
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

int attn_probe_exp(const float* in, float* out, int workgroups, int iters, void* stream) {
  if (!in || !out) return 1;
  if (workgroups < 1 || iters < 1 || workgroups > (1 << 20)) return 2;
  hipLaunchKernelGGL(exp_probe_kernel, dim3(workgroups), dim3(PROBE_THREADS), 0, static_cast<hipStream_t>(stream),
                     in, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int attn_probe_lds(float* out, unsigned long long* clk, int workgroups, int iters, void* stream) {
  if (!out || !clk) return 1;
  if (workgroups < 1 || iters < 1 || workgroups > (1 << 20)) return 2;
  hipLaunchKernelGGL(lds_probe_kernel, dim3(workgroups), dim3(PROBE_THREADS), 0, static_cast<hipStream_t>(stream),
                     out, clk, iters);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

double attn_probe_mfma_flops(int workgroups, int iters) {
  // 16 products of 32 x 32 x 16 per wavefront and iteration, 4 wavefronts per workgroup
  return (double)workgroups * 4 * (double)iters * 16 * 2.0 * 32 * 32 * 16;
}

}  // extern "C"
