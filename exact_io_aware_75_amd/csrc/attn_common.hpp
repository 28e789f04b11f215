// Shared device helpers for the gfx950 attention kernels: vector types, MFMA
// wrappers for bf16/fp16, conversions and the workgroup -> work-item mapping.
//
// MFMA operand layouts used throughout (v_mfma_f32_32x32x16_{bf16,f16}, a
// 64-lane wavefront, h = lane / 32):
//   A (32 x 16, row m, col k): lane holds m = lane % 32, k = 8h .. 8h + 7
//   B (16 x 32, row k, col n): lane holds n = lane % 32, k = 8h .. 8h + 7
//   C (32 x 32 fp32):          lane holds n = lane % 32 and rows
//                              m = 8 (r / 4) + 4h + r % 4 for r = 0..15
// Because the reduction index k may be permuted freely (as long as A and B
// agree), the C registers r = 8s .. 8s + 7 of an accumulator whose rows are
// the reduction index of a following product are directly that product's B
// operand for k-step s, with slot t <-> row 16s + 8 (t / 4) + 4h + t % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

struct Bf16Tag {};
struct F16Tag {};

// 8 packed 16-bit elements (one MFMA operand register quad).
typedef s16x8_t frag8_t;

__device__ __forceinline__ f32x16_t mfma32(Bf16Tag, frag8_t a, frag8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(F16Tag, frag8_t a, frag8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                 __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

// Round two fp32 values to nearest-even 16-bit floats, packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack2(Bf16Tag, float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint32_t pack2(F16Tag, float lo, float hi) {
  f16x2_t p = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// acc + lo + hi of a packed pair (sums exactly the rounded values the MFMA uses).
__device__ __forceinline__ float add_pair(Bf16Tag, uint32_t pair, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), one, acc, false);
}
__device__ __forceinline__ float add_pair(F16Tag, uint32_t pair, float acc) {
  const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pair), one, acc, false);
}

__device__ __forceinline__ float to_float(Bf16Tag, uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}
__device__ __forceinline__ float to_float(F16Tag, uint16_t x) {
  return (float)__builtin_bit_cast(_Float16, x);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte chunks addressed by lanes
// 4j + i / 4, for j = 0..3.
__device__ __forceinline__ s16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
}

__device__ __forceinline__ float wave_xor32(float x) {
  return __shfl_xor(x, 32, 64);
}

// Block-sparse attention: compacts the indices i in [first, last) whose mask
// entry p[i * stride] is nonzero, in increasing order, into list[] (LDS), and
// returns their count (wave-uniform).  Run by one whole wavefront; the
// workgroup synchronises before other wavefronts read the list.
__device__ __forceinline__ int compact_mask(const uint8_t* p, int stride, int first, int last,
                                            uint16_t* list, int lane) {
  int cnt = 0;
  for (int base = first; base < last; base += 64) {
    const int i = base + lane;
    const bool on = i < last && p[(size_t)i * stride] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
    if (on) {
      const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      list[cnt + pos] = (uint16_t)i;
    }
    cnt += __builtin_popcountll(bal);
  }
  return cnt;
}

// floor(a / b) for b > 0 and any sign of a (causal bounds with an offset).
__device__ __forceinline__ int floor_div(int a, int b) { return a >= 0 ? a / b : -((b - 1 - a) / b); }

// Wave-uniform read of an LDS list entry (kept in a scalar register).
__device__ __forceinline__ int lds_uniform(const uint16_t* list, int i) {
  return __builtin_amdgcn_readfirstlane((int)list[i]);
}

// The workgroup's index along x, reversed in the reversed-order test mode.
__device__ __forceinline__ int grid_x(int reverse) {
  return reverse ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
}

// Dynamic LDS bytes that keep one workgroup of `kernel` per CU in the
// one-workgroup-per-CU test mode (its static LDS plus this exceed half of
// the CU's 160 KiB); 0 otherwise.
inline size_t one_wg_lds_pad(const void* kernel, int on) {
  if (!on) return 0;
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, kernel) != hipSuccess) return 0;
  const size_t half = 80 * 1024;
  return attr.sharedSizeBytes > half ? 0 : half + 256 - attr.sharedSizeBytes;
}

// Block index remap so that consecutive logical work items run on the same
// XCD (the hardware dispatches workgroup i to XCD i % 8).  `total` must be a
// multiple of 8 for the remap to be a bijection; otherwise identity.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  if ((total & 7) != 0) return bid;
  return (bid & 7) * (total >> 3) + (bid >> 3);
}

}  // namespace attn
