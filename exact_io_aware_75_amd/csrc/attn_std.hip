// Standard (materialising) attention on gfx950: the baseline the IO-aware
// method is measured against.  The FlashAttention-1 news page ("FlashAttention"
// section) and the FlashAttention-2 review ("Введение") describe it: the score
// matrix S = scale * Q K^T and the probabilities P = softmax(S) are written to
// HBM in full, read back for O = P V, and the backward pass reads the stored P
// again.  Its HBM traffic grows with N^2, which is what the tiled kernels
// avoid; this path exists to measure that difference on the same device with
// the same inputs.
//
// Passes (each a separate launch, every intermediate in HBM):
//   forward   S = scale Q K^T (fp32)  ->  P = softmax(S) row-wise (16-bit),
//             LSE                     ->  O = P V
//   backward  dV = P^T dO  ->  dP = dO V^T (fp32, over S)  ->
//             dS = P * (dP - rowsum(P * dP)) (16-bit)  ->  dQ = scale dS K,
//             dK = scale dS^T Q
// with the causal mask applied in the softmax (masked P entries are stored as
// zeros, so every product runs over the full N x N matrices, as standard
// attention does).
//
// The products run on one MFMA tile kernel: 128 x 128 output tiles, four
// wavefronts of 64 x 64, k staged through LDS 32 at a time, fp32
// accumulation with v_mfma_f32_32x32x16.  An operand stored with its
// reduction index contiguous (Q, K, dO as rows, P and dS as rows) is read
// with 64-bit LDS reads; one stored the other way round (V and K as the B
// operand of P V and dS K; P, dS, dO and Q as operands of the P^T / dS^T
// products) with ds_read_b64_tr_b16, so nothing is transposed in memory.
// Within each 16-wide k-step both forms hold reduction indices
// 4h .. 4h+3 and 8+4h .. 8+4h+3 (h = lane / 32), so A and B agree.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn {

namespace {

constexpr int GT = 128;   // output tile edge (rows of C and columns of C)
constexpr int GK = 32;    // reduction indices per LDS stage
constexpr int LDK = 36;   // pitch (elements) of a reduction-contiguous tile [128][GK]: 18 banks per row
constexpr int LDX = 160;  // pitch of an index-contiguous tile [GK][128]: 16 banks per row
constexpr int GTHREADS = 256;

__device__ __forceinline__ uint16_t to_bits(Bf16Tag, float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ uint16_t to_bits(F16Tag, float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

// Keep the first `nvalid` (0..8) 16-bit elements of a 16-byte chunk, zero the rest.
__device__ __forceinline__ u32x4_t keep_first(u32x4_t v, int nvalid) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t m = (2 * w < nvalid ? 0x0000FFFFu : 0u) | (2 * w + 1 < nvalid ? 0xFFFF0000u : 0u);
    v[w] &= m;
  }
  return v;
}

// One operand of the tile product.  TRANS = false: element (x, k) at
// p[x * ld + k] (reduction index contiguous); TRANS = true: at p[k * ld + x].
// x < xext is the operand's own index (rows of C for A, columns for B); the
// head of stage s of output head ho is (ho * hmul + s) / hdiv.
template <bool TRANS>
__device__ __forceinline__ void load_stage(const StdOperand& op, int b, int head, int x0, int k0, int K,
                                           int tid, u32x4_t* r) {
  const uint16_t* base = op.p + (size_t)b * op.bstride + (size_t)head * op.hstride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + GTHREADS * i;
    int x, k, nvalid;
    if (!TRANS) {  // [128 x][32 k]: 4 chunks per row
      x = x0 + (c >> 2);
      k = k0 + 8 * (c & 3);
      nvalid = (x < op.xext) ? min(8, K - k) : 0;
    } else {       // [32 k][128 x]: 16 chunks per row
      k = k0 + (c >> 4);
      x = x0 + 8 * (c & 15);
      nvalid = (k < K) ? min(8, op.xext - x) : 0;
    }
    if (nvalid > 0) {
      const uint16_t* src = TRANS ? base + (size_t)k * op.ld + x : base + (size_t)x * op.ld + k;
      u32x4_t v = *(const u32x4_t*)src;
      r[i] = nvalid < 8 ? keep_first(v, nvalid) : v;
    } else {
      r[i] = (u32x4_t){0u, 0u, 0u, 0u};
    }
  }
}

template <bool TRANS>
__device__ __forceinline__ void store_stage(uint16_t* L, int tid, const u32x4_t* r) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + GTHREADS * i;
    if (!TRANS) {  // 72-byte rows: two 8-byte writes
      uint16_t* dst = L + (c >> 2) * LDK + 8 * (c & 3);
      *(u32x2_t*)dst = (u32x2_t){r[i][0], r[i][1]};
      *(u32x2_t*)(dst + 4) = (u32x2_t){r[i][2], r[i][3]};
    } else {
      *(u32x4_t*)(L + (c >> 4) * LDX + 8 * (c & 15)) = r[i];
    }
  }
}

// MFMA operand fragment of 32-index block xb, k-step s (16 reduction indices).
template <bool TRANS>
__device__ __forceinline__ frag8_t read_frag(const uint16_t* L, int xb, int s, int lane) {
  const int h = lane >> 5;
  s16x4_t lo, hi;
  if (!TRANS) {
    const uint16_t* p = L + (32 * xb + (lane & 31)) * LDK + 16 * s + 4 * h;
    lo = *(const s16x4_t*)p;
    hi = *(const s16x4_t*)(p + 8);
  } else {
    const int grp = lane >> 4, gi = lane & 15;
    const uint16_t* p = L + (16 * s + 4 * h + (gi >> 2)) * LDX + 32 * xb + 16 * (grp & 1) + 4 * (gi & 3);
    lo = lds_read_tr(p);
    hi = lds_read_tr(p + 8 * LDX);
  }
  return (frag8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// C[b, ho] (M x Nn) = alpha * sum_s A_s B_s^T over K, where A_s is operand
// a at head (ho * a.hmul + s) / a.hdiv and likewise for b.
template <typename Tag, bool AT, bool BT, bool OUT_F32>
__global__ void __launch_bounds__(GTHREADS) std_gemm_kernel(StdGemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t la[AT ? GK * LDX : GT * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t lb[BT ? GK * LDX : GT * LDK];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * GT;
  const int m0 = blockIdx.y * GT;
  const int bz = blockIdx.z;
  const int b = bz / g.Hout;
  const int ho = bz - b * g.Hout;
  const int nkt = (g.K + GK - 1) / GK;
  const int total = g.nsum * nkt;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = (f32x16_t){};

  u32x4_t ra[2], rb[2];
  auto fetch = [&](int t) __attribute__((always_inline)) {
    const int s = t / nkt;
    const int k0 = (t - s * nkt) * GK;
    load_stage<AT>(g.a, b, (ho * g.a.hmul + s) / g.a.hdiv, m0, k0, g.K, tid, ra);
    load_stage<BT>(g.b, b, (ho * g.b.hmul + s) / g.b.hdiv, n0, k0, g.K, tid, rb);
  };
  if (total > 0) fetch(0);
  for (int t = 0; t < total; ++t) {
    __syncthreads();  // every wavefront is done with the previous stage
    store_stage<AT>(la, tid, ra);
    store_stage<BT>(lb, tid, rb);
    __syncthreads();
    if (t + 1 < total) fetch(t + 1);  // in flight during this stage's products
#pragma unroll
    for (int s = 0; s < GK / 16; ++s) {
      frag8_t fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = read_frag<AT>(la, 2 * wm + i, s, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = read_frag<BT>(lb, 2 * wn + j, s, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(Tag{}, fa[i], fb[j], acc[i][j]);
    }
  }

  // C fragment: lane holds column n = lane % 32 and rows 8 (r / 4) + 4 h + r % 4.
  const int h = lane >> 5;
  const size_t cbase = (size_t)b * g.c_bstride + (size_t)ho * g.c_hstride;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + 32 * (2 * wn + j) + (lane & 31);
      if (n >= g.Nn) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * (2 * wm + i) + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m >= g.M) continue;
        const float val = g.alpha * acc[i][j][r];
        const size_t off = cbase + (size_t)m * g.c_ld + n;
        if (OUT_F32) ((float*)g.c)[off] = val;
        else ((uint16_t*)g.c)[off] = to_bits(Tag{}, val);
      }
    }
}

// Sum / max over the 256 threads of a workgroup (every thread gets the result).
template <bool MAX>
__device__ __forceinline__ float block_reduce(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float y = __shfl_xor(x, o, 64);
    x = MAX ? fmaxf(x, y) : x + y;
  }
  const int wave = threadIdx.x >> 6;
  __syncthreads();  // red[] free from any previous use
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < GTHREADS / 64; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// The row kernels read each row from HBM once when it fits in registers:
// CAP floats per thread (row pitch ldn <= 256 CAP), chunk t of thread tid at
// column 4 tid + 1024 t.  CAP = 0 streams the row once per pass instead.
__device__ __forceinline__ float pe_of(Bf16Tag, u32x2_t w, int e) { return to_float(Bf16Tag{}, (uint16_t)(w[e >> 1] >> (16 * (e & 1)))); }
__device__ __forceinline__ float pe_of(F16Tag, u32x2_t w, int e) { return to_float(F16Tag{}, (uint16_t)(w[e >> 1] >> (16 * (e & 1)))); }

template <typename Tag>
__device__ __forceinline__ u32x2_t pack4(const float* x) {
  return (u32x2_t){(uint32_t)to_bits(Tag{}, x[0]) | ((uint32_t)to_bits(Tag{}, x[1]) << 16),
                   (uint32_t)to_bits(Tag{}, x[2]) | ((uint32_t)to_bits(Tag{}, x[3]) << 16)};
}

// One workgroup per (batch, head, query row i): P[i, :] = softmax of the
// allowed entries of S[i, :] (keys j < N, and j <= i when causal), stored in
// the 16-bit type with zeros elsewhere (up to the row pitch), and
// LSE[i] = max + ln(sum).
template <typename Tag, int CAP>
__global__ void __launch_bounds__(GTHREADS) std_softmax_kernel(StdRowArgs a) {
  __shared__ float red[GTHREADS / 64];
  constexpr int NC = CAP > 0 ? CAP / 4 : 1;
  const int row = blockIdx.x;  // (b * Hq + h) * N + i
  const int i = row % a.N;
  const int nvis = a.causal ? min(i + 1, a.N) : a.N;
  const float* s = a.s + (size_t)row * a.ldn;
  uint16_t* p = a.p + (size_t)row * a.ldn;
  const int tid = threadIdx.x;

  f32x4_t c[NC];
  float m = -INFINITY;
  if constexpr (CAP > 0) {
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int j = 4 * tid + 4 * GTHREADS * t;
      c[t] = j < nvis ? *(const f32x4_t*)(s + j) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) m = (j + e < nvis) ? fmaxf(m, c[t][e]) : m;
    }
  } else {
    for (int j = 4 * tid; j < nvis; j += 4 * GTHREADS) {
      const f32x4_t v = *(const f32x4_t*)(s + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) m = (j + e < nvis) ? fmaxf(m, v[e]) : m;
    }
  }
  m = block_reduce<true>(m, red);
  float l = 0.f;
  if constexpr (CAP > 0) {
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int j = 4 * tid + 4 * GTHREADS * t;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[t][e] = (j + e < nvis) ? fast_exp2((c[t][e] - m) * LOG2E) : 0.f;
        l += c[t][e];
      }
    }
  } else {
    for (int j = 4 * tid; j < nvis; j += 4 * GTHREADS) {
      const f32x4_t v = *(const f32x4_t*)(s + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) l += (j + e < nvis) ? fast_exp2((v[e] - m) * LOG2E) : 0.f;
    }
  }
  l = block_reduce<false>(l, red);
  const float inv = 1.0f / l;
  if constexpr (CAP > 0) {
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int j = 4 * tid + 4 * GTHREADS * t;
      if (j < a.ldn) {
        const float pe[4] = {c[t][0] * inv, c[t][1] * inv, c[t][2] * inv, c[t][3] * inv};
        *(u32x2_t*)(p + j) = pack4<Tag>(pe);
      }
    }
  } else {
    for (int j = 4 * tid; j < a.ldn; j += 4 * GTHREADS) {
      float pe[4] = {0.f, 0.f, 0.f, 0.f};
      if (j < nvis) {
        const f32x4_t v = *(const f32x4_t*)(s + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[e] = (j + e < nvis) ? fast_exp2((v[e] - m) * LOG2E) * inv : 0.f;
      }
      *(u32x2_t*)(p + j) = pack4<Tag>(pe);
    }
  }
  if (tid == 0) a.lse[row] = m + fast_log2(l) * LN2;
}

// One workgroup per (batch, head, query row i): D = sum_j P[i, j] dP[i, j]
// over the keys j < N, then dS[i, j] = P[i, j] (dP[i, j] - D) in the 16-bit
// type, zeros past N.
template <typename Tag, int CAP>
__global__ void __launch_bounds__(GTHREADS) std_softmax_bwd_kernel(StdRowArgs a) {
  __shared__ float red[GTHREADS / 64];
  constexpr int NC = CAP > 0 ? CAP / 4 : 1;
  const int row = blockIdx.x;
  const float* dp = a.s + (size_t)row * a.ldn;
  const uint16_t* p = a.p + (size_t)row * a.ldn;
  uint16_t* ds = a.ds + (size_t)row * a.ldn;
  const int tid = threadIdx.x;
  f32x4_t cdp[NC];
  u32x2_t cp[NC];
  float dsum = 0.f;
  if constexpr (CAP > 0) {
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int j = 4 * tid + 4 * GTHREADS * t;
      const bool in = j < a.N;
      cdp[t] = in ? *(const f32x4_t*)(dp + j) : (f32x4_t){0.f, 0.f, 0.f, 0.f};
      cp[t] = in ? *(const u32x2_t*)(p + j) : (u32x2_t){0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum += (j + e < a.N) ? pe_of(Tag{}, cp[t], e) * cdp[t][e] : 0.f;
    }
  } else {
    for (int j = 4 * tid; j < a.N; j += 4 * GTHREADS) {
      const f32x4_t v = *(const f32x4_t*)(dp + j);
      const u32x2_t w = *(const u32x2_t*)(p + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) dsum += (j + e < a.N) ? pe_of(Tag{}, w, e) * v[e] : 0.f;
    }
  }
  const float D = block_reduce<false>(dsum, red);
  if constexpr (CAP > 0) {
#pragma unroll
    for (int t = 0; t < NC; ++t) {
      const int j = 4 * tid + 4 * GTHREADS * t;
      if (j < a.ldn) {
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (j + e < a.N) ? pe_of(Tag{}, cp[t], e) * (cdp[t][e] - D) : 0.f;
        *(u32x2_t*)(ds + j) = pack4<Tag>(o);
      }
    }
  } else {
    for (int j = 4 * tid; j < a.ldn; j += 4 * GTHREADS) {
      float o[4] = {0.f, 0.f, 0.f, 0.f};
      if (j < a.N) {
        const f32x4_t v = *(const f32x4_t*)(dp + j);
        const u32x2_t w = *(const u32x2_t*)(p + j);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (j + e < a.N) ? pe_of(Tag{}, w, e) * (v[e] - D) : 0.f;
      }
      *(u32x2_t*)(ds + j) = pack4<Tag>(o);
    }
  }
}

// Launch a row kernel with the register capacity that holds a row of pitch ldn.
template <typename Tag, int CAP>
hipError_t launch_rows(bool fwd, const StdRowArgs& r, int rows, hipStream_t st) {
  if (fwd) hipLaunchKernelGGL((std_softmax_kernel<Tag, CAP>), dim3(rows), dim3(GTHREADS), 0, st, r);
  else hipLaunchKernelGGL((std_softmax_bwd_kernel<Tag, CAP>), dim3(rows), dim3(GTHREADS), 0, st, r);
  return hipGetLastError();
}

template <typename Tag>
hipError_t row_pass(bool fwd, const StdRowArgs& r, int rows, hipStream_t st) {
  if (r.ldn <= 4 * GTHREADS) return launch_rows<Tag, 4>(fwd, r, rows, st);
  if (r.ldn <= 16 * GTHREADS) return launch_rows<Tag, 16>(fwd, r, rows, st);
  if (r.ldn <= 64 * GTHREADS) return launch_rows<Tag, 64>(fwd, r, rows, st);
  return launch_rows<Tag, 0>(fwd, r, rows, st);
}

template <typename Tag, bool AT, bool BT, bool OUT_F32>
hipError_t gemm(const StdGemmArgs& g, int B, hipStream_t st) {
  const dim3 grid((g.Nn + GT - 1) / GT, (g.M + GT - 1) / GT, B * g.Hout);
  hipLaunchKernelGGL((std_gemm_kernel<Tag, AT, BT, OUT_F32>), grid, dim3(GTHREADS), 0, st, g);
  return hipGetLastError();
}

StdOperand operand(const void* p, long long bstride, long long hstride, int ld, int hmul, int hdiv, int xext) {
  StdOperand o;
  o.p = (const uint16_t*)p;
  o.bstride = bstride;
  o.hstride = hstride;
  o.ld = ld;
  o.hmul = hmul;
  o.hdiv = hdiv;
  o.xext = xext;
  return o;
}

StdGemmArgs product(const StdOperand& a, const StdOperand& b, void* c, long long c_bstride,
                    long long c_hstride, int c_ld, int K, int Hout, int nsum, float alpha) {
  StdGemmArgs g;
  g.a = a;
  g.b = b;
  g.c = c;
  g.c_bstride = c_bstride;
  g.c_hstride = c_hstride;
  g.c_ld = c_ld;
  g.M = a.xext;
  g.Nn = b.xext;
  g.K = K;
  g.Hout = Hout;
  g.nsum = nsum;
  g.alpha = alpha;
  return g;
}

template <typename Tag>
hipError_t std_fwd(const StdArgs& a, hipStream_t st) {
  const int N = a.N, d = a.d, grp = a.Hq / a.Hkv;
  const long long qb = (long long)N * a.Hq * d, kb = (long long)N * a.Hkv * d;
  const long long mh = (long long)N * a.ldn, mb = (long long)a.Hq * mh;  // N x N matrices
  // S = scale Q K^T (fp32)
  hipError_t e = gemm<Tag, false, false, true>(
      product(operand(a.q, qb, d, a.Hq * d, 1, 1, N), operand(a.k, kb, d, a.Hkv * d, 1, grp, N),
              a.s, mb, mh, a.ldn, d, a.Hq, 1, a.scale), a.B, st);
  if (e != hipSuccess) return e;
  StdRowArgs r{a.s, a.p, a.ds, a.lse, N, a.ldn, a.causal};
  if ((e = row_pass<Tag>(true, r, a.B * a.Hq * N, st)) != hipSuccess) return e;
  // O = P V: V is the B operand with its key (reduction) index as rows
  return gemm<Tag, false, true, false>(
      product(operand(a.p, mb, mh, a.ldn, 1, 1, N), operand(a.v, kb, d, a.Hkv * d, 1, grp, d),
              a.o, qb, d, a.Hq * d, N, a.Hq, 1, 1.0f), a.B, st);
}

template <typename Tag>
hipError_t std_bwd(const StdArgs& a, hipStream_t st) {
  const int N = a.N, d = a.d, grp = a.Hq / a.Hkv;
  const long long qb = (long long)N * a.Hq * d, kb = (long long)N * a.Hkv * d;
  const long long mh = (long long)N * a.ldn, mb = (long long)a.Hq * mh;
  hipError_t e;
  // dV = P^T dO, summed over the query heads of each K/V head
  e = gemm<Tag, true, true, false>(
      product(operand(a.p, mb, mh, a.ldn, grp, 1, N), operand(a.dout, qb, d, a.Hq * d, grp, 1, d),
              a.dv, kb, d, a.Hkv * d, N, a.Hkv, grp, 1.0f), a.B, st);
  if (e != hipSuccess) return e;
  // dP = dO V^T (fp32, over the score buffer)
  e = gemm<Tag, false, false, true>(
      product(operand(a.dout, qb, d, a.Hq * d, 1, 1, N), operand(a.v, kb, d, a.Hkv * d, 1, grp, N),
              a.s, mb, mh, a.ldn, d, a.Hq, 1, 1.0f), a.B, st);
  if (e != hipSuccess) return e;
  StdRowArgs r{a.s, a.p, a.ds, a.lse, N, a.ldn, a.causal};
  if ((e = row_pass<Tag>(false, r, a.B * a.Hq * N, st)) != hipSuccess) return e;
  // dQ = scale dS K
  e = gemm<Tag, false, true, false>(
      product(operand(a.ds, mb, mh, a.ldn, 1, 1, N), operand(a.k, kb, d, a.Hkv * d, 1, grp, d),
              a.dq, qb, d, a.Hq * d, N, a.Hq, 1, a.scale), a.B, st);
  if (e != hipSuccess) return e;
  // dK = scale dS^T Q, summed over the query heads of each K/V head
  return gemm<Tag, true, true, false>(
      product(operand(a.ds, mb, mh, a.ldn, grp, 1, N), operand(a.q, qb, d, a.Hq * d, grp, 1, d),
              a.dk, kb, d, a.Hkv * d, N, a.Hkv, grp, a.scale), a.B, st);
}

}  // namespace

hipError_t launch_std_fwd(const StdArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? std_fwd<Bf16Tag>(a, st) : std_fwd<F16Tag>(a, st);
}

hipError_t launch_std_bwd(const StdArgs& a, bool bf16, hipStream_t st) {
  return bf16 ? std_bwd<Bf16Tag>(a, st) : std_bwd<F16Tag>(a, st);
}

}  // namespace attn
