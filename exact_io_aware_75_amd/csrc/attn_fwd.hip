// Forward pass of exact attention on gfx950: O = softmax(scale * Q K^T) V and
// LSE = per-row natural log-sum-exp, without materialising the N x N scores.
//
// Method (the pages' FlashAttention-2 design, re-laid for CDNA4):
//  * Tiling: K/V blocks are staged from HBM into on-chip memory and the block
//    result is folded into the output (FlashAttention-2 announcement, "具体实现"
//    section; FlashAttention-1 news page, "FlashAttention" section).
//  * Parallel over sequence length: one workgroup per (batch, query head,
//    block of 128 query rows), so the grid fills 256 CUs even for small
//    batch * heads (announcement, "具体实现"; review, "Параллелизм").
//  * Work split inside a workgroup: each 64-lane wavefront owns 32 query rows
//    and all wavefronts share the K/V tiles, so wavefronts never exchange
//    partial outputs (announcement, "具体实现": Q split across warps, K/V
//    shared).
//  * Online softmax with the rescale deferred: the reference max only moves
//    (and the accumulator is only rescaled) when a tile raises a row's max by
//    more than 2^8 in the exp2 domain, and the single division by the row sum
//    happens once in the epilogue -- fewer non-matmul operations without
//    changing the output (announcement, "具体实现": the softmax trick
//    rewritten to cut rescaling, bounds checks and causal masking).
//  * Causal: key tiles wholly above the diagonal are never visited, and only
//    tiles that cross the diagonal or the ragged end of the sequence run the
//    element mask; the steady-state loop carries no mask code at all (review,
//    "Алгоритм вычисления").
//
// CDNA4 mapping.
//  * Occupancy: two workgroups of four wavefronts per CU (two wavefronts per
//    SIMD, <= 256 registers each), so one wavefront's softmax (VALU) runs
//    while the other's matrix products (MFMA) run on the same SIMD.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: the
//    accumulator holds one query per lane and 16 keys per register block, so
//    the row max / row sum are in-lane except one v_permlane32_swap between
//    lanes l and l ^ 32, and the probabilities are already the B operand of
//    O^T += V^T P^T.  V^T comes from the row-major V tile through
//    ds_read_b64_tr_b16.  Q stays in registers for the whole loop.
//  * K/V tiles go HBM -> LDS by global_load_lds_dwordx4 (no register staging),
//    double-buffered: the next tile's loads are in flight while the current
//    one is consumed.  The LDS tiles are unpadded and XOR-swizzled in 16-byte
//    chunks so that both the 128-bit K reads and the transposed V reads are
//    free of bank conflicts.
//  * exp is v_exp_f32 (2^x) with log2(e) folded into the score scale.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn {

namespace {

constexpr int FWD_BM = 128;     // query rows per workgroup
constexpr int FWD_WAVES = 4;    // 32 query rows per wavefront
constexpr int FWD_THREADS = FWD_WAVES * 64;
constexpr float RESCALE_THRESHOLD = 8.0f;  // log2 units: rescale only if the max grows > 2^8

// Key-tile height per head dimension: every K or V tile is 16 KiB.
template <int D> struct FwdTile { static constexpr int BN = 8192 / D; };

// 16-byte-chunk swizzles of the LDS tiles (row r, logical chunk c is stored at
// chunk c ^ swz(r)); LDS has 64 four-byte banks, i.e. 16 chunk-wide bank groups.
// K: a 128-bit read serves 16 lanes per cycle, here 16 consecutive rows at one
// logical chunk, so the 16 rows must land in 16 different bank groups.
// V: a transposed 64-bit read serves 32 lanes per cycle, here 4 consecutive
// rows x 4 adjacent chunks, so each of the 4 rows must own 4 bank groups.
template <int D> __device__ __forceinline__ int swz_k(int r) {
  return D == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int D> __device__ __forceinline__ int swz_v(int r) {
  return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;

// Wavefronts per SIMD the register budget is cut for: two for d <= 128; at
// d = 256 the resident Q (64 registers) and O^T (128) leave too little for two.
template <int D> struct FwdOcc { static constexpr int WAVES_PER_SIMD = D <= 128 ? 2 : 1; };

template <typename Tag, int D, bool CAUSAL>
__global__ void __launch_bounds__(FWD_THREADS, FwdOcc<D>::WAVES_PER_SIMD)
attn_fwd_kernel(FwdArgs a) {
  constexpr int BN = FwdTile<D>::BN;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int TILE = BN * D;          // elements per K or V tile (8192)
  constexpr int LPT = TILE / 8 / FWD_THREADS;  // 16-byte loads per thread per tensor (4)
  constexpr int NKK = D / 16;           // MFMA k-steps over d
  constexpr int NSB = BN / 32;          // 32-key sub-blocks per tile
  constexpr int NDB = D / 32;           // 32-wide d blocks of O
  constexpr int NKS = BN / 16;          // k-steps over keys in P V
  static_assert(TILE == 8192 && LPT == 4, "tile shape");

  // Two LDS buffers of [K tile, V tile], as separate objects so the compiler can
  // tell that the loads in flight into one never alias reads of the other.
  __shared__ __attribute__((aligned(1024))) uint16_t smem0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t smem1[2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
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

  const size_t q_row = (size_t)a.Hq * D;   // elements between consecutive query rows
  const size_t kv_row = (size_t)a.Hkv * D;
  const uint16_t* qbase = (const uint16_t*)a.q + ((size_t)b * a.N * a.Hq + h) * D;
  const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)b * a.N * a.Hkv + g) * D;
  const uint16_t* vbase = (const uint16_t*)a.v + ((size_t)b * a.N * a.Hkv + g) * D;

  const int row0 = rb * FWD_BM;                 // first query row of the workgroup
  const int wrow0 = row0 + wave * 32;           // first query row of this wavefront
  const int qrow = wrow0 + l32;                 // this lane's query row
  const bool qvalid = qrow < a.N;

  // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole loop ----
  frag8_t qf[NKK];
  {
    const uint16_t* src = qbase + (size_t)min(qrow, a.N - 1) * q_row + 8 * half;
    const uint32_t flip = a.neg_scale ? 0x80008000u : 0u;  // a negative scale flips Q's sign
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4_t x = *(const u32x4_t*)(src + 16 * kk);
      x ^= (u32x4_t){flip, flip, flip, flip};
      qf[kk] = __builtin_bit_cast(frag8_t, x);
    }
  }
  const float c = a.scale_log2;  // |scale| * log2(e)

  // ---- key tiles: the workgroup's trip count and this wavefront's share ----
  const int ntiles_all = (a.N + BN - 1) / BN;
  int ntiles = ntiles_all;   // tiles the workgroup streams through LDS
  int nwave = ntiles_all;    // tiles this wavefront computes
  int nfull = a.N / BN;      // leading tiles that need no element mask
  if (CAUSAL) {
    ntiles = min(ntiles_all, (min(row0 + FWD_BM, a.N) - 1) / BN + 1);
    nwave = min(ntiles_all, (wrow0 + 31) / BN + 1);
    nfull = min(nfull, (wrow0 + 1) / BN);
  }

  // ---- HBM -> LDS tile loads: thread (wave, lane) fills chunk (4 i + wave) * 64 + lane ----
  // of each tile for i = 0..3; its source row and logical chunk follow from the swizzle.
  // Source offsets are 32-bit byte offsets from the tile's first row (the host
  // bounds N * H * d below 2^31 elements), so each load is a scalar base plus
  // one vector offset.  Rows past the end of the sequence are redirected to
  // the last row: any finite values do, since they are masked.
  uint32_t ld_koff[LPT], ld_voff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int q = (i * FWD_WAVES + wave) * 64 + lane;
    const int r = q / CPR;
    const int p = q % CPR;
    ld_koff[i] = (uint32_t)(2 * (r * (int)kv_row + (p ^ swz_k<D>(r)) * 8));
    ld_voff[i] = (uint32_t)(2 * (r * (int)kv_row + (p ^ swz_v<D>(r)) * 8));
  }
  auto load_tile = [&](int j, uint16_t* kt) {
    uint16_t* vt = kt + TILE;
    const size_t tile_off = (size_t)j * BN * kv_row;
    const char* ksrc = (const char*)(kbase + tile_off);
    const char* vsrc = (const char*)(vbase + tile_off);
    if (j * BN + BN <= a.N) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int dst = (i * FWD_WAVES + wave) * 64 * 8;  // wave-uniform LDS element offset
        __builtin_amdgcn_global_load_lds((gptr_t)(ksrc + ld_koff[i]), (lptr_t)(kt + dst), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gptr_t)(vsrc + ld_voff[i]), (lptr_t)(vt + dst), 16, 0, 0);
      }
    } else {  // the tile runs past the sequence end
      const int last = a.N - 1 - j * BN;  // last valid row of the tile
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int r = ((i * FWD_WAVES + wave) * 64 + lane) / CPR;
        const uint32_t back = (uint32_t)(2 * max(0, r - last) * (int)kv_row);
        const int dst = (i * FWD_WAVES + wave) * 64 * 8;
        __builtin_amdgcn_global_load_lds((gptr_t)(ksrc + (ld_koff[i] - back)), (lptr_t)(kt + dst), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((gptr_t)(vsrc + (ld_voff[i] - back)), (lptr_t)(vt + dst), 16, 0, 0);
      }
    }
  };

  // ---- per-lane LDS read offsets (elements, within one tile) ----
  // K (A operand of S^T): row 32 sb + l32, logical chunk 2 kk + half.
  int k_rd[NKK];
  {
    const int x = swz_k<D>(l32) ^ half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) k_rd[kk] = l32 * D + ((2 * kk) ^ x) * 8;
  }
  // V^T (A operand of O^T += V^T P^T) by transposed reads: row 16 ks + 8 hi + 4 half + gi / 4,
  // element 32 db + 16 (grp & 1) + 4 (gi & 3), i.e. logical chunk 4 db + cl.
  int v_rd[NDB];
  {
    const int grp = lane >> 4;
    const int gi = lane & 15;
    const int r = 4 * half + (gi >> 2);
    const int cl = 2 * (grp & 1) + ((gi & 3) >> 1);
    const int x = swz_v<D>(r) ^ cl;
#pragma unroll
    for (int db = 0; db < NDB; ++db) v_rd[db] = r * D + ((4 * db) ^ x) * 8 + 4 * (gi & 1);
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = (f32x16_t){};
  float m_ref = -INFINITY;  // running max (exp2 domain) the accumulator is scaled to
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // this lane's partial row sums (keys of its half)

  auto do_tile = [&](int j, const uint16_t* ks, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const uint16_t* vs = ks + TILE;
    const int key0 = j * BN;
    // S^T = K Q^T for this wavefront's 32 queries.  The NSB accumulator chains
    // advance together one k-step at a time, and the K fragments are read
    // PF k-steps ahead, so no product waits on its own LDS read.
    f32x16_t s[NSB];
    {
      constexpr int PF = 2;
      frag8_t kf[PF + 1][NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) s[sb] = (f32x16_t){};
#pragma unroll
      for (int kk = 0; kk < PF && kk < NKK; ++kk)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) kf[kk][sb] = *(const frag8_t*)(ks + 32 * sb * D + k_rd[kk]);
      __builtin_amdgcn_sched_group_barrier(0x100, PF * NSB, 0);  // DS reads
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + PF < NKK) {
#pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
            kf[(kk + PF) % (PF + 1)][sb] = *(const frag8_t*)(ks + 32 * sb * D + k_rd[kk + PF]);
        }
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) s[sb] = mfma32(Tag{}, kf[kk % (PF + 1)][sb], qf[kk], s[sb]);
        if (kk + PF < NKK) __builtin_amdgcn_sched_group_barrier(0x100, NSB, 0);  // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, NSB, 0);                     // MFMA
      }
    }
    if (MASK) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool ok = key < a.N && (!CAUSAL || key <= qrow);
          s[sb][r] = ok ? s[sb][r] : -INFINITY;
        }
    }
    // row max: four independent v_max3 chains, then one exchange between the halves
    float mx4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        mx4[(r >> 1) & 3] = fmaxf(mx4[(r >> 1) & 3], fmaxf(s[sb][r], s[sb][r + 1]));
    float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                       __builtin_bit_cast(uint32_t, mx), false, false);
      mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
    }
    const float mxs = mx * c;
    // deferred rescale: move the reference max only when it grows by > 2^8
    if (__builtin_amdgcn_ballot_w64(mxs > m_ref + RESCALE_THRESHOLD) != 0) {
      const float m_new = fmaxf(m_ref, mxs);
      const float alpha = fast_exp2(m_ref - m_new);
#pragma unroll
      for (int t = 0; t < 4; ++t) lsum[t] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_ref = m_new;
    }
    // P = 2^(s*c - m_ref), rounded to 16 bits: the B operand of O^T += V^T P^T
    const float nm = -m_ref;
    frag8_t pf[NKS];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 8 * hh + 2 * t;
          float p0 = fast_exp2(__builtin_fmaf(s[sb][r], c, nm));
          float p1 = fast_exp2(__builtin_fmaf(s[sb][r + 1], c, nm));
          if (MASK) {  // exp2(-inf * 0) would be NaN when scale == 0
            p0 = s[sb][r] == -INFINITY ? 0.f : p0;
            p1 = s[sb][r + 1] == -INFINITY ? 0.f : p1;
          }
          w[t] = pack2(Tag{}, p0, p1);
          lsum[t] += p0 + p1;  // fp32 row sum: LSE must not carry 16-bit rounding
        }
        u32x4_t wv = {w[0], w[1], w[2], w[3]};
        pf[2 * sb + hh] = __builtin_bit_cast(frag8_t, wv);
      }
    }
    // O^T += V^T P^T : A operand V^T via transposed LDS reads
#pragma unroll
    for (int ksb = 0; ksb < NKS; ++ksb) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint16_t* p = vs + 16 * ksb * D + v_rd[db];
        s16x4_t lo = lds_read_tr(p);
        s16x4_t hi = lds_read_tr(p + 8 * D);
        frag8_t vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = mfma32(Tag{}, vf, pf[ksb], oacc[db]);
      }
    }
  };

  uint16_t* const buf0 = smem0;
  uint16_t* const buf1 = smem1;
  load_tile(0, buf0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // One barrier per tile: every wavefront passes exactly `ntiles` barriers,
  // whichever loop it spends them in.  Tile j lives in buffer j & 1; the
  // steady-state loop takes tiles in pairs so both buffer offsets are constants.
  auto step = [&](int j, uint16_t* cur, uint16_t* nxt, auto mask_tag) {
    if (j + 1 < ntiles) load_tile(j + 1, nxt);
    do_tile(j, cur, mask_tag);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  int j = 0;
  for (; j + 1 < nfull; j += 2) {  // steady state: no element mask
    step(j, buf0, buf1, std::false_type{});
    step(j + 1, buf1, buf0, std::false_type{});
  }
  if (j < nfull) {
    step(j, buf0, buf1, std::false_type{});
    ++j;
  }
  for (; j < ntiles; ++j) {  // diagonal / ragged tiles, then tiles only other wavefronts need
    uint16_t* cur = (j & 1) ? buf1 : buf0;
    uint16_t* nxt = (j & 1) ? buf0 : buf1;
    if (j + 1 < ntiles) load_tile(j + 1, nxt);
    if (j < nwave) do_tile(j, cur, std::true_type{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // ---- epilogue: one division per row, LSE in natural log ----
  float ltot;
  {
    const float ls = (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, ls),
                                                     __builtin_bit_cast(uint32_t, ls), false, false);
    ltot = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
  }
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
