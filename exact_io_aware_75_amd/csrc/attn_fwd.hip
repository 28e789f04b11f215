// Forward pass of exact attention on gfx950: O = softmax(scale * Q K^T) V and
// LSE = per-row natural log-sum-exp, without materialising the N x N scores.
//
// Method (the pages' FlashAttention-2 design, re-laid for CDNA4):
//  * Tiling: K/V blocks are staged from HBM into on-chip memory and the block
//    result is folded into the output (FlashAttention-2 announcement, "具体实现"
//    section; FlashAttention-1 news page, "FlashAttention" section).
//  * Parallel over sequence length: one workgroup per (batch, query head,
//    block of BM query rows), so the grid fills 256 CUs even for small
//    batch * heads (announcement, "具体实现"; review, "Параллелизм").
//  * Work split inside a workgroup: each 64-lane wavefront owns 32 query rows
//    and all wavefronts share the K/V tiles, so wavefronts never exchange
//    partial outputs (announcement, "具体实现": Q split across warps, K/V
//    shared).
//  * Online softmax with the rescale deferred: the running max only moves
//    (and the accumulator is only rescaled) when a tile raises a row's max by
//    more than 2^8 in the exp2 domain, and the single division by the row sum
//    happens once in the epilogue -- fewer non-matmul operations without
//    changing the output (announcement, "具体实现": the softmax trick
//    rewritten to cut rescaling, bounds checks and causal masking).
//  * Causal: key tiles wholly above the diagonal are never visited; only
//    tiles that cross the diagonal or the ragged end of the sequence run the
//    element mask (review, "Алгоритм вычисления").
//
// CDNA4 mapping.  Scores are formed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16: the accumulator then holds one query per lane and 16
// keys per register block, so row max / row sum are in-lane except one
// exchange between lanes l and l ^ 32, and the probabilities are already the
// B operand of O^T += V^T P^T.  V^T comes from the row-major V tile through
// ds_read_b64_tr_b16.  Q stays in registers for the whole loop; K/V tiles are
// double-buffered in LDS and the next tile's global loads are in flight while
// the current one is consumed.  exp is v_exp_f32 (2^x) with log2(e) folded
// into the score scale.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn {

namespace {

constexpr int FWD_BM = 128;     // query rows per workgroup
constexpr int FWD_WAVES = 4;    // 32 query rows per wavefront
constexpr int FWD_THREADS = FWD_WAVES * 64;
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units: rescale only if the max grows > 2^8

template <int D> struct FwdTile;
template <> struct FwdTile<64> { static constexpr int BN = 128; };
template <> struct FwdTile<128> { static constexpr int BN = 64; };
template <> struct FwdTile<256> { static constexpr int BN = 32; };

template <typename Tag, int D, bool CAUSAL>
__global__ void __launch_bounds__(FWD_THREADS)
attn_fwd_kernel(FwdArgs a) {
  constexpr int BN = FwdTile<D>::BN;
  constexpr int KSTR = D + 8;    // K tile row stride (elements): 16 B pad
  constexpr int VSTR = D + 16;   // V tile row stride (elements): 32 B pad
  constexpr int KT = BN * KSTR;
  constexpr int VT = BN * VSTR;
  constexpr int CPR = D / 8;                         // 16-byte chunks per row
  constexpr int CPT = BN * CPR / FWD_THREADS;        // chunks per thread per tensor
  constexpr int NKK = D / 16;                        // MFMA k-steps over d
  constexpr int NSB = BN / 32;                       // 32-key sub-blocks per tile
  constexpr int NDB = D / 32;                        // 32-wide d blocks of O
  constexpr int NKS = BN / 16;                       // k-steps over keys in P V
  static_assert(CPT >= 1 && BN * CPR % FWD_THREADS == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KT + VT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- which (batch, head, row block) this workgroup owns ----
  const int nblk = (a.N + FWD_BM - 1) / FWD_BM;
  const int total = nblk * a.Hq * a.B;
  const int L = xcd_remap(blockIdx.x, total);
  const int bh = L / nblk;
  const int rb = nblk - 1 - (L - bh * nblk);  // heaviest (causal) row blocks first
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / a.group;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v;
  const size_t q_row = (size_t)a.Hq * D;   // elements between consecutive query rows
  const size_t kv_row = (size_t)a.Hkv * D;
  const uint16_t* qbase = qp + ((size_t)b * a.N * a.Hq + h) * D;
  const uint16_t* kbase = kp + ((size_t)b * a.N * a.Hkv + g) * D;
  const uint16_t* vbase = vp + ((size_t)b * a.N * a.Hkv + g) * D;

  const int row0 = rb * FWD_BM;                 // first query row of the workgroup
  const int wrow0 = row0 + wave * 32;           // first query row of this wavefront
  const int qrow = wrow0 + l32;                 // this lane's query row
  const bool qvalid = qrow < a.N;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop ----
  frag8_t qf[NKK];
  {
    const uint16_t* src = qbase + (size_t)qrow * q_row + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4_t x = {0u, 0u, 0u, 0u};
      if (qvalid) x = *(const u32x4_t*)(src + 16 * kk);
      // a negative scale is folded into Q's sign so the score scale is >= 0
      if (a.neg_scale) x ^= (u32x4_t){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[kk] = __builtin_bit_cast(frag8_t, x);
    }
  }
  const float c = a.scale_log2;  // |scale| * log2(e)

  // ---- key tiles this workgroup visits ----
  const int ntiles_all = (a.N + BN - 1) / BN;
  int ntiles = ntiles_all;
  if (CAUSAL) {
    const int last_row = min(row0 + FWD_BM, a.N) - 1;
    ntiles = min(ntiles_all, last_row / BN + 1);
  }

  // global -> register staging of one K/V tile (zeros past the sequence end)
  u32x4_t kreg[CPT], vreg[CPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cidx = tid + i * FWD_THREADS;
      const int r = cidx / CPR;
      const int col = (cidx - r * CPR) * 8;
      const int key = j * BN + r;
      u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (key < a.N) {
        kx = *(const u32x4_t*)(kbase + (size_t)key * kv_row + col);
        vx = *(const u32x4_t*)(vbase + (size_t)key * kv_row + col);
      }
      kreg[i] = kx;
      vreg[i] = vx;
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * (KT + VT);
    uint16_t* vs = ks + KT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cidx = tid + i * FWD_THREADS;
      const int r = cidx / CPR;
      const int col = (cidx - r * CPR) * 8;
      *(u32x4_t*)(ks + r * KSTR + col) = kreg[i];
      *(u32x4_t*)(vs + r * VSTR + col) = vreg[i];
    }
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = (f32x16_t){};
  float m_ref = -INFINITY;  // running max (exp2 domain) the accumulator is scaled to
  float lsum = 0.f;         // this lane's partial row sum (keys of its half)

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    const int kbase_j = j * BN;
    const bool wave_active = !CAUSAL || kbase_j <= wrow0 + 31;
    if (wave_active) {
      const uint16_t* ks = smem + buf * (KT + VT);
      const uint16_t* vs = ks + KT;
      // S^T = K Q^T for this wavefront's 32 queries
      f32x16_t s[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        f32x16_t acc = {};
        const uint16_t* krow = ks + (32 * sb + l32) * KSTR + 8 * half;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          frag8_t kf = *(const frag8_t*)(krow + 16 * kk);
          acc = mfma32(Tag{}, kf, qf[kk], acc);
        }
        s[sb] = acc;
      }
      // element mask only on tiles that cross the diagonal or the sequence end
      const bool need_mask = (kbase_j + BN > a.N) || (CAUSAL && kbase_j + BN - 1 > wrow0);
      float mx = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase_j + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
            const bool ok = key < a.N && (!CAUSAL || key <= qrow);
            mx = fmaxf(mx, ok ? s[sb][r] : -INFINITY);
          }
      } else {
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[sb][r]);
      }
      mx = fmaxf(mx, wave_xor32(mx));
      const float mxs = mx * c;  // NaN only if the row is fully masked and c == 0
      // deferred rescale: move the reference max only when it grows by > 2^8
      const bool grow = mxs > m_ref + RESCALE_THRESHOLD;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = fmaxf(m_ref, mxs);
        const float alpha = fast_exp2(m_ref - m_new);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m_ref = m_new;
      }
      // P = 2^(s*c - m_ref), rounded to 16 bits: the B operand of O^T += V^T P^T
      frag8_t pf[NKS];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = 8 * hh + 2 * t;
            float p0 = fast_exp2(s[sb][r] * c - m_ref);
            float p1 = fast_exp2(s[sb][r + 1] * c - m_ref);
            if (need_mask) {
              const int key0 = kbase_j + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
              if (!(key0 < a.N && (!CAUSAL || key0 <= qrow))) p0 = 0.f;
              if (!(key0 + 1 < a.N && (!CAUSAL || key0 + 1 <= qrow))) p1 = 0.f;
            }
            w[t] = pack2(Tag{}, p0, p1);
            lsum += p0 + p1;  // fp32 row sum: LSE must not carry 16-bit rounding
          }
          u32x4_t wv = {w[0], w[1], w[2], w[3]};
          pf[2 * sb + hh] = __builtin_bit_cast(frag8_t, wv);
        }
      }
      // O^T += V^T P^T : A operand V^T via transposed LDS reads
      const int grp = lane >> 4;         // 16-lane group
      const int gi = lane & 15;
      const uint16_t* vrd = vs + (4 * half + (gi >> 2)) * VSTR + 16 * (grp & 1) + 4 * (gi & 3);
#pragma unroll
      for (int ksb = 0; ksb < NKS; ++ksb) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint16_t* p = vrd + (16 * ksb) * VSTR + 32 * db;
          s16x4_t lo = lds_read_tr(p);
          s16x4_t hi = lds_read_tr(p + 8 * VSTR);
          frag8_t vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = mfma32(Tag{}, vf, pf[ksb], oacc[db]);
        }
      }
    }
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: one division per row, LSE in natural log ----
  const float ltot = lsum + wave_xor32(lsum);
  if (qvalid) {
    const float inv = 1.0f / ltot;
    uint16_t* orow = (uint16_t*)a.o + ((size_t)b * a.N * a.Hq + h) * D + (size_t)qrow * q_row;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * half;
        u32x2_t w = {pack2(Tag{}, oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv),
                     pack2(Tag{}, oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv)};
        *(u32x2_t*)(orow + d0) = w;
      }
    if (half == 0) {
      const float lse2 = m_ref + log2f(ltot);
      a.lse[((size_t)b * a.Hq + h) * a.N + qrow] = lse2 * 0.69314718055994530942f;
    }
  }
}

}  // namespace

template <typename Tag, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int nblk = (a.N + FWD_BM - 1) / FWD_BM;
  const long long total = (long long)nblk * a.Hq * a.B;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_kernel<Tag, D, CAUSAL>), dim3((unsigned)total), dim3(FWD_THREADS),
                     0, stream, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, bool bf16, int d, bool causal, hipStream_t stream) {
#define ATTN_FWD_CASE(TAG, DD)                                                     \
  if (d == DD) return causal ? launch_fwd_t<TAG, DD, true>(a, stream)             \
                             : launch_fwd_t<TAG, DD, false>(a, stream);
  if (bf16) {
    ATTN_FWD_CASE(Bf16Tag, 64)
    ATTN_FWD_CASE(Bf16Tag, 128)
    ATTN_FWD_CASE(Bf16Tag, 256)
  } else {
    ATTN_FWD_CASE(F16Tag, 64)
    ATTN_FWD_CASE(F16Tag, 128)
    ATTN_FWD_CASE(F16Tag, 256)
  }
#undef ATTN_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace attn
