// Backward pass of exact attention on gfx950: dQ, dK, dV of L = sum(O * dO),
// recomputing the probabilities tile by tile from Q, K and the saved LSE
// instead of storing them (FlashAttention-2 announcement, "具体实现" section;
// FlashAttention-1 news page, "FlashAttention" section: recomputation in the
// backward pass).  The textbook gradient it evaluates:
//     P  = exp(scale * Q K^T - LSE)          (causal: 0 above the diagonal)
//     dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D)
//     dK = scale * dS^T Q,  dQ = scale * dS K
//
// Three launches on the caller's stream:
//  1. bwd_pre:  D = rowsum(dO * O) per query row (fp32) and dQacc = 0.
//  2. bwd_main: one workgroup per (batch, K/V head, block of keys) -- parallel
//     over the key (column) dimension, as the pages describe for the backward
//     pass (FlashAttention-2 review, "Параллелизм").  Each 64-lane wavefront
//     owns 32 keys; dK and dV stay in registers for the whole loop over the
//     query heads of the GQA group and the query tiles (causal: only tiles
//     at or below the diagonal).  dQ partials go to an fp32 accumulator with
//     atomic adds.
//  3. bwd_dq:   dQ = scale * dQacc rounded to the input dtype.
//
// CDNA4 mapping (v_mfma_f32_32x32x16, 64-lane wavefronts).  Scores are formed
// as S = Q K^T with the key index on the lane, so P and dS come out of the
// accumulators already laid out as the B operands of dV^T += dO^T P and
// dK^T += Q^T dS; dO^T and Q^T are read from the row-major LDS tiles with
// ds_read_b64_tr_b16.  dS is staged once through LDS (as 16-bit values) for
// dQ = dS K, whose K operand is again a transposed LDS read.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn {

namespace {

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O), dQacc = 0
// ---------------------------------------------------------------------------
template <typename Tag, int D>
__global__ void __launch_bounds__(256) attn_bwd_pre_kernel(BwdArgs a) {
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int ROWS = 256 / CPR;       // rows per workgroup
  const int tid = threadIdx.x;
  const int rloc = tid / CPR;
  const int c = tid - rloc * CPR;
  const long long row = (long long)blockIdx.x * ROWS + rloc;  // over B * N * Hq rows
  const long long nrows = (long long)a.B * a.N * a.Hq;
  float acc = 0.f;
  if (row < nrows) {
    const uint16_t* o = (const uint16_t*)a.o + row * D + 8 * c;
    const uint16_t* d = (const uint16_t*)a.dout + row * D + 8 * c;
    const u32x4_t ov = *(const u32x4_t*)o;
    const u32x4_t dv = *(const u32x4_t*)d;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc += to_float(Tag{}, (uint16_t)(ov[i] & 0xffff)) * to_float(Tag{}, (uint16_t)(dv[i] & 0xffff));
      acc += to_float(Tag{}, (uint16_t)(ov[i] >> 16)) * to_float(Tag{}, (uint16_t)(dv[i] >> 16));
    }
    f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    float* q = a.dq_acc + row * D + 8 * c;
    *(f32x4_t*)q = z;
    *(f32x4_t*)(q + 4) = z;
  }
  // reduce over the CPR lanes of the row (CPR is a power of two <= 32)
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < nrows && c == 0) {
    // row = (b * N + n) * Hq + h  ->  delta[b][h][n]
    const long long bn = row / a.Hq;
    const int h = (int)(row - bn * a.Hq);
    const long long b = bn / a.N;
    const int n = (int)(bn - b * a.N);
    a.delta[((size_t)b * a.Hq + h) * a.N + n] = acc;
  }
}

// ---------------------------------------------------------------------------
// 2. main kernel
// ---------------------------------------------------------------------------
template <int D> struct BwdCfg;
template <> struct BwdCfg<64> {
  static constexpr int NW = 4, BM = 64;
  static constexpr bool KV_REGS = true;
};
template <> struct BwdCfg<128> {
  static constexpr int NW = 4, BM = 64;
  static constexpr bool KV_REGS = true;
};
template <> struct BwdCfg<256> {
  static constexpr int NW = 2, BM = 32;
  static constexpr bool KV_REGS = false;
};

template <typename Tag, int D, bool CAUSAL>
__global__ void __launch_bounds__(BwdCfg<D>::NW * 64)
attn_bwd_main_kernel(BwdArgs a) {
  constexpr int NW = BwdCfg<D>::NW;
  constexpr int NT = NW * 64;
  constexpr int BN = NW * 32;            // keys per workgroup
  constexpr int BM = BwdCfg<D>::BM;      // query rows per tile
  constexpr bool KV_REGS = BwdCfg<D>::KV_REGS;
  constexpr int QSTR = D + 16;           // Q / dO tile row stride (elements): tr reads
  constexpr int KSTR = D + 16;           // K block row stride: tr reads (and b128 reads)
  constexpr int SSTR = BN + 8;           // dS tile row stride: b128 reads
  constexpr int NKK = D / 16;            // k-steps over d
  constexpr int NQB = BM / 32;           // 32-query blocks per tile
  constexpr int NDB = D / 32;            // 32-wide d blocks
  constexpr int NKS = BM / 16;           // k-steps over queries (dV, dK)
  constexpr int CPR = D / 8;
  constexpr int TCPT = BM * CPR / NT;    // Q (and dO) tile chunks per thread
  constexpr int KCPT = BN * CPR / NT;    // K (and V) block chunks per thread
  constexpr int DQ_BLOCKS = NQB * NDB / NW;  // 32x32 dQ blocks per wavefront
  static_assert(TCPT >= 1 && BM * CPR % NT == 0 && KCPT >= 1 && DQ_BLOCKS >= 1 &&
                NQB * NDB % NW == 0, "tile/thread mismatch");

  constexpr int QT = BM * QSTR;          // one Q (or dO) tile
  constexpr int ST = BM * SSTR;          // one dS tile
  constexpr int KB = BN * KSTR;          // the K (or V) block
  // LDS: [Q,dO] x 2 buffers | dS x 2 buffers | K block | V block (if not in regs) | lse2, delta x 2
  constexpr int LDS_ELEMS = 4 * QT + 2 * ST + KB + (KV_REGS ? 0 : KB);
  __shared__ __attribute__((aligned(16))) uint16_t smem[LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) float s_lse[2][BM];
  __shared__ __attribute__((aligned(16))) float s_del[2][BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;
  const int gi = lane & 15;

  // ---- which (batch, kv head, key block) this workgroup owns ----
  const int nkb = (a.N + BN - 1) / BN;
  const int total = nkb * a.Hkv * a.B;
  const int Lw = xcd_remap(blockIdx.x, total);
  const int bg = Lw / nkb;
  const int kb = Lw - bg * nkb;
  const int b = bg / a.Hkv;
  const int g = bg - b * a.Hkv;
  const int k0 = kb * BN;                // first key of the block
  const int kw0 = k0 + wave * 32;        // first key of this wavefront
  const int mykey = kw0 + l32;           // this lane's key (C-layout column)

  const size_t q_row = (size_t)a.Hq * D;
  const size_t kv_row = (size_t)a.Hkv * D;
  const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)b * a.N * a.Hkv + g) * D;
  const uint16_t* vbase = (const uint16_t*)a.v + ((size_t)b * a.N * a.Hkv + g) * D;

  uint16_t* const s_k = smem + 4 * QT + 2 * ST;
  uint16_t* const s_v = s_k + KB;  // used only when !KV_REGS

  // ---- stage the K (and V) block in LDS; zeros past the sequence end ----
#pragma unroll
  for (int i = 0; i < KCPT; ++i) {
    const int cidx = tid + i * NT;
    const int r = cidx / CPR;
    const int col = (cidx - r * CPR) * 8;
    const int key = k0 + r;
    u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
    if (key < a.N) {
      kx = *(const u32x4_t*)(kbase + (size_t)key * kv_row + col);
      if (!KV_REGS) vx = *(const u32x4_t*)(vbase + (size_t)key * kv_row + col);
    }
    *(u32x4_t*)(s_k + r * KSTR + col) = kx;
    if (!KV_REGS) *(u32x4_t*)(s_v + r * KSTR + col) = vx;
  }
  // K / V fragments as B operands (lane = key, 8 consecutive d per k-step)
  frag8_t kf[KV_REGS ? NKK : 1], vf[KV_REGS ? NKK : 1];
  if (KV_REGS) {
    const bool ok = mykey < a.N;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (ok) {
        kx = *(const u32x4_t*)(kbase + (size_t)mykey * kv_row + 16 * kk + 8 * half);
        vx = *(const u32x4_t*)(vbase + (size_t)mykey * kv_row + 16 * kk + 8 * half);
      }
      kf[KV_REGS ? kk : 0] = __builtin_bit_cast(frag8_t, kx);
      vf[KV_REGS ? kk : 0] = __builtin_bit_cast(frag8_t, vx);
    }
  }
  auto kfrag = [&](int kk) -> frag8_t {
    if (KV_REGS) return kf[KV_REGS ? kk : 0];
    return *(const frag8_t*)(s_k + (wave * 32 + l32) * KSTR + 16 * kk + 8 * half);
  };
  auto vfrag = [&](int kk) -> frag8_t {
    if (KV_REGS) return vf[KV_REGS ? kk : 0];
    return *(const frag8_t*)(s_v + (wave * 32 + l32) * KSTR + 16 * kk + 8 * half);
  };

  f32x16_t dk_acc[NDB], dv_acc[NDB];  // dK^T, dV^T: lane = key, rows = d
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk_acc[i] = (f32x16_t){};
    dv_acc[i] = (f32x16_t){};
  }

  const int nqt = (a.N + BM - 1) / BM;
  const int qt0 = CAUSAL ? (k0 / BM) : 0;   // first query tile with a row >= k0
  const int tiles_per_head = nqt - qt0;
  const int ntiles = tiles_per_head * a.group;
  const float c = a.scale_log2;             // scale * log2(e), signed

  // global -> register staging of the next (head, query tile)
  u32x4_t qreg[TCPT], oreg[TCPT];
  float lreg = 0.f, dreg = 0.f;
  auto tile_coords = [&](int t, int& h, int& q0) {
    const int hh = t / tiles_per_head;
    h = g * a.group + hh;
    q0 = (qt0 + (t - hh * tiles_per_head)) * BM;
  };
  auto load_tile = [&](int t) {
    int h, q0;
    tile_coords(t, h, q0);
    const uint16_t* qb = (const uint16_t*)a.q + ((size_t)b * a.N * a.Hq + h) * D;
    const uint16_t* db = (const uint16_t*)a.dout + ((size_t)b * a.N * a.Hq + h) * D;
#pragma unroll
    for (int i = 0; i < TCPT; ++i) {
      const int cidx = tid + i * NT;
      const int r = cidx / CPR;
      const int col = (cidx - r * CPR) * 8;
      const int qr = q0 + r;
      u32x4_t qx = {0u, 0u, 0u, 0u}, dx = {0u, 0u, 0u, 0u};
      if (qr < a.N) {
        qx = *(const u32x4_t*)(qb + (size_t)qr * q_row + col);
        dx = *(const u32x4_t*)(db + (size_t)qr * q_row + col);
      }
      qreg[i] = qx;
      oreg[i] = dx;
    }
    if (tid < BM) {
      const int qr = q0 + tid;
      const size_t li = ((size_t)b * a.Hq + h) * a.N + qr;
      // rows past the end get LSE = +inf, so their probabilities are 0
      lreg = qr < a.N ? a.lse[li] * 1.4426950408889634f : INFINITY;
      dreg = qr < a.N ? a.delta[li] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* sq = smem + buf * 2 * QT;
    uint16_t* sd = sq + QT;
#pragma unroll
    for (int i = 0; i < TCPT; ++i) {
      const int cidx = tid + i * NT;
      const int r = cidx / CPR;
      const int col = (cidx - r * CPR) * 8;
      *(u32x4_t*)(sq + r * QSTR + col) = qreg[i];
      *(u32x4_t*)(sd + r * QSTR + col) = oreg[i];
    }
    if (tid < BM) {
      s_lse[buf][tid] = lreg;
      s_del[buf][tid] = dreg;
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    int h, q0;
    tile_coords(t, h, q0);
    const uint16_t* sq = smem + buf * 2 * QT;
    const uint16_t* sd = sq + QT;
    uint16_t* sds = smem + 4 * QT + buf * ST;
    const bool need_mask = CAUSAL && q0 < kw0 + 31;

    // transposed-read base for A = Q^T / dO^T (lane = d, 8 query slots per k-step)
    const int tr_off = (4 * half + (gi >> 2)) * QSTR + 16 * (grp & 1) + 4 * (gi & 3);

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 queries x this wavefront's 32 keys
      f32x16_t s = {}, dp = {};
      const uint16_t* qrow = sq + (32 * qb + l32) * QSTR + 8 * half;
      const uint16_t* drow = sd + (32 * qb + l32) * QSTR + 8 * half;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = mfma32(Tag{}, *(const frag8_t*)(qrow + 16 * kk), kfrag(kk), s);
        dp = mfma32(Tag{}, *(const frag8_t*)(drow + 16 * kk), vfrag(kk), dp);
      }
      // P = 2^(S c - LSE log2 e), dS = P (dP - D); rows = queries 8(r/4) + 4h + r%4
      const float* lsep = &s_lse[buf][32 * qb + 4 * half];
      const float* delp = &s_del[buf][32 * qb + 4 * half];
      uint32_t pw[8], dsw[8];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4_t l4 = *(const f32x4_t*)(lsep + 8 * r4);
        const f32x4_t d4 = *(const f32x4_t*)(delp + 8 * r4);
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          float pv = fast_exp2(s[r] * c - l4[e]);
          if (need_mask) {
            const int qi = q0 + 32 * qb + 8 * r4 + 4 * half + e;
            if (mykey > qi) pv = 0.f;
          }
          p[e] = pv;
          ds[e] = pv * (dp[r] - d4[e]);
        }
        pw[2 * r4] = pack2(Tag{}, p[0], p[1]);
        pw[2 * r4 + 1] = pack2(Tag{}, p[2], p[3]);
        dsw[2 * r4] = pack2(Tag{}, ds[0], ds[1]);
        dsw[2 * r4 + 1] = pack2(Tag{}, ds[2], ds[3]);
      }
      // dS -> LDS as [query][key] for dQ = dS K (rows 8(r/4) + 4h + e, column = key)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = 32 * qb + 8 * r4 + 4 * half + e;
          const uint32_t w = dsw[2 * r4 + (e >> 1)];
          sds[qi * SSTR + wave * 32 + l32] = (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffff));
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS  (k-steps over this block's 32 queries)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const u32x4_t pv4 = {pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]};
        const u32x4_t dv4 = {dsw[4 * ks], dsw[4 * ks + 1], dsw[4 * ks + 2], dsw[4 * ks + 3]};
        const frag8_t pfrag = __builtin_bit_cast(frag8_t, pv4);
        const frag8_t dsfrag = __builtin_bit_cast(frag8_t, dv4);
        const int rowoff = (32 * qb + 16 * ks) * QSTR + tr_off;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* pd = sd + rowoff + 32 * db;
          const uint16_t* pq = sq + rowoff + 32 * db;
          const frag8_t dof = __builtin_shufflevector(lds_read_tr(pd), lds_read_tr(pd + 8 * QSTR),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
          const frag8_t qtf = __builtin_shufflevector(lds_read_tr(pq), lds_read_tr(pq + 8 * QSTR),
                                                      0, 1, 2, 3, 4, 5, 6, 7);
          dv_acc[db] = mfma32(Tag{}, dof, pfrag, dv_acc[db]);
          dk_acc[db] = mfma32(Tag{}, qtf, dsfrag, dk_acc[db]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();  // dS tile complete (and the next Q/dO tile staged)

    // dQacc[q0 .. q0+BM) += dS K over this block's BN keys
    float* dqb = a.dq_acc + ((size_t)b * a.N * a.Hq + h) * D;
#pragma unroll
    for (int blk = 0; blk < DQ_BLOCKS; ++blk) {
      const int id = wave * DQ_BLOCKS + blk;
      const int qb = id / NDB;
      const int db = id - qb * NDB;
      f32x16_t acc = {};
      const uint16_t* arow = sds + (32 * qb + l32) * SSTR + 8 * half;
      // B = K[key][d]: lane = d, keys 16s + 8h + 4a + j via transposed reads
      const uint16_t* kb_rd = s_k + (8 * half + (gi >> 2)) * KSTR + 32 * db + 16 * (grp & 1) + 4 * (gi & 3);
#pragma unroll
      for (int ks = 0; ks < BN / 16; ++ks) {
        const frag8_t af = *(const frag8_t*)(arow + 16 * ks);
        const uint16_t* p = kb_rd + 16 * ks * KSTR;
        const frag8_t bf = __builtin_shufflevector(lds_read_tr(p), lds_read_tr(p + 4 * KSTR),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
        acc = mfma32(Tag{}, af, bf, acc);
      }
      // C: lane = d column (32 db + l32), rows = queries 32 qb + 8(r/4) + 4h + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + 32 * qb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (qi < a.N) atomicAdd(dqb + (size_t)qi * q_row + 32 * db + l32, acc[r]);
      }
    }
  }

  // ---- epilogue: dK = scale * dK_acc, dV = dV_acc; lane = key, rows = d ----
  if (mykey < a.N) {
    uint16_t* dkp = (uint16_t*)a.dk + ((size_t)b * a.N * a.Hkv + g) * D + (size_t)mykey * kv_row;
    uint16_t* dvp = (uint16_t*)a.dv + ((size_t)b * a.N * a.Hkv + g) * D + (size_t)mykey * kv_row;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * half;
        const u32x2_t wk = {pack2(Tag{}, dk_acc[db][4 * q4] * a.scale, dk_acc[db][4 * q4 + 1] * a.scale),
                            pack2(Tag{}, dk_acc[db][4 * q4 + 2] * a.scale, dk_acc[db][4 * q4 + 3] * a.scale)};
        const u32x2_t wv = {pack2(Tag{}, dv_acc[db][4 * q4], dv_acc[db][4 * q4 + 1]),
                            pack2(Tag{}, dv_acc[db][4 * q4 + 2], dv_acc[db][4 * q4 + 3])};
        *(u32x2_t*)(dkp + d0) = wk;
        *(u32x2_t*)(dvp + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ = scale * dQacc -> input dtype
// ---------------------------------------------------------------------------
template <typename Tag>
__global__ void __launch_bounds__(256) attn_bwd_dq_kernel(BwdArgs a, long long nchunks) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // 8-element chunk index
  if (i >= nchunks) return;
  const f32x4_t x0 = *(const f32x4_t*)(a.dq_acc + 8 * i);
  const f32x4_t x1 = *(const f32x4_t*)(a.dq_acc + 8 * i + 4);
  const float s = a.scale;
  const u32x4_t w = {pack2(Tag{}, x0[0] * s, x0[1] * s), pack2(Tag{}, x0[2] * s, x0[3] * s),
                     pack2(Tag{}, x1[0] * s, x1[1] * s), pack2(Tag{}, x1[2] * s, x1[3] * s)};
  *(u32x4_t*)((uint16_t*)a.dq + 8 * i) = w;
}

}  // namespace

template <typename Tag, int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, int stages, hipStream_t stream) {
  const long long rows = (long long)a.B * a.N * a.Hq;
  if (stages & 1) {
    constexpr int ROWS = 256 / (D / 8);
    const long long grid = (rows + ROWS - 1) / ROWS;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_bwd_pre_kernel<Tag, D>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 2) {
    constexpr int BN = BwdCfg<D>::NW * 32;
    const long long grid = (long long)((a.N + BN - 1) / BN) * a.Hkv * a.B;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_bwd_main_kernel<Tag, D, CAUSAL>), dim3((unsigned)grid),
                       dim3(BwdCfg<D>::NW * 64), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 4) {
    const long long nchunks = rows * D / 8;
    const long long grid = (nchunks + 255) / 256;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<Tag>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                       nchunks);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a, bool bf16, int d, bool causal, int stages,
                      hipStream_t stream) {
#define ATTN_BWD_CASE(TAG, DD)                                                     \
  if (d == DD) return causal ? launch_bwd_t<TAG, DD, true>(a, stages, stream)     \
                             : launch_bwd_t<TAG, DD, false>(a, stages, stream);
  if (bf16) {
    ATTN_BWD_CASE(Bf16Tag, 64)
    ATTN_BWD_CASE(Bf16Tag, 128)
    ATTN_BWD_CASE(Bf16Tag, 256)
  } else {
    ATTN_BWD_CASE(F16Tag, 64)
    ATTN_BWD_CASE(F16Tag, 128)
    ATTN_BWD_CASE(F16Tag, 256)
  }
#undef ATTN_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
