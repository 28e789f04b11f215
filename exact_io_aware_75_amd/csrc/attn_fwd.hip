// Forward pass of exact attention on gfx950: O = softmax(scale * Q K^T) V and
// LSE = per-row natural log-sum-exp, without materialising the N x N scores.
//
// Method (the pages' FlashAttention-2 design, re-laid for CDNA4):
//  * Tiling: K/V blocks are staged from HBM into on-chip memory and the block
//    result is folded into the output (FlashAttention-2 announcement, "具体实现"
//    section; FlashAttention-1 news page, "FlashAttention" section).
//  * Parallel over sequence length: one workgroup per (batch, query head,
//    block of 256 query rows; 128 at d = 256, causal at d = 64, over short
//    key sequences, block-sparse and split-KV), so the grid fills 256 CUs
//    even for small batch * heads (announcement, "具体实现"; review,
//    "Параллелизм").
//  * Work split inside a workgroup: each 64-lane wavefront owns 32 query rows
//    and all wavefronts share the K/V tiles, so wavefronts never exchange
//    partial outputs (announcement, "具体实现": Q split across warps, K/V
//    shared).
//  * Online softmax with the rescale deferred: the reference max only moves
//    (and the accumulator is only rescaled) when it must -- at d <= 128 when
//    a tile's probabilities, formed against it, would sum past 2^16 in a
//    lane; at d = 256 when a tile raises a row's max by more than 2^8 in the
//    exp2 domain -- and the single division by the row sum happens once in
//    the epilogue: fewer non-matmul operations without changing the output
//    (announcement, "具体实现": the softmax trick rewritten to cut rescaling,
//    bounds checks and causal masking).
//  * Causal: key tiles wholly above the diagonal are never visited, and only
//    tiles that cross the diagonal or the ragged end of the sequence run the
//    element mask; the steady-state loop carries no mask code at all (review,
//    "Алгоритм вычисления").
//
// CDNA4 mapping.
//  * Occupancy: two wavefronts per SIMD (<= 256 registers each) at d <= 128:
//    one workgroup of eight wavefronts per CU, so a K/V tile staged in LDS
//    serves 256 query rows, or two workgroups of four (causal at d = 64, short
//    key sequences; three over short key sequences at d = 64, non-causal).
//    At d = 256 one wavefront per SIMD.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16: the
//    accumulator holds one query per lane and 16 keys per register block, so
//    the row max / row sum are in-lane except one v_permlane32_swap between
//    lanes l and l ^ 32, and the probabilities are already the B operand of
//    O^T += V^T P^T.  V^T comes from the row-major V tile through
//    ds_read_b64_tr_b16.  Q stays in registers for the whole loop.
//  * Software pipeline inside each wavefront: while the matrix cores form
//    the scores of key tile j + 1, the VALU forms the probabilities of tile j
//    (d <= 128: all of them; d = 256: its row max and the first half, the
//    second half under the first half of tile j's P V products).  A
//    single wavefront's VALU work thus issues in the shadow of its own MFMAs
//    instead of waiting for the other wavefront on the SIMD.  Only each
//    wavefront's last tile runs unpipelined (and, at the ragged end of a
//    non-causal sequence, the tiles after the last two whole ones).
//  * K/V tiles go HBM -> LDS by buffer_load_dwordx4 ... lds (no register
//    staging) through a buffer resource whose record count ends at the last
//    key: rows past the end of the sequence arrive as zeros, with no clamp
//    or branch.  K and V are double-buffered separately, K one tile ahead of
//    V, so iteration j reads K_{j+1} and V_j while K_{j+2} and V_{j+1} are in
//    flight.  The LDS tiles are unpadded and XOR-swizzled in 16-byte chunks
//    so that both the 128-bit K reads and the transposed V reads are free of
//    bank conflicts.
//  * exp is v_exp_f32 (2^x) with log2(e) folded into the score scale.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn {

namespace {

// Wavefronts per workgroup (32 query rows each).  Dense d <= 128: eight,
// one workgroup per CU at two wavefronts per SIMD, so each K/V tile is staged
// once per 256 query rows -- except over short key sequences (the SHORT
// instantiation, which the host picks up to NarrowKeys keys; causal, SHORT
// pairs row blocks instead, FwdPaired), where each workgroup's loop is short
// next to its fixed prologue and epilogue: there two workgroups of four per
// CU, one in its loop while the other loads or stores, win over staging each
// tile for more rows.  Causal d = 64: four, since the wavefronts of a
// diagonal block have unequal trip counts and wait for the longest at every
// barrier (eight: 3% slower at 4096 rows); at d = 128 the halved staging
// outweighs that from 4096 rows on (+2.5-3% at 8192-65536, even at 4096).  d = 256: four (one wavefront per
// SIMD).  Block-sparse: four, so that a workgroup's 128 rows are one row of
// the block mask.  Split-KV: four, since it serves short query sequences,
// where 256-row blocks would be mostly past the end.
template <int D, bool CAUSAL, bool SPARSE = false, bool SPLIT = false, bool SHORT = false> struct FwdWG {
  static constexpr int WAVES = (D <= 128 && !SPARSE && !SPLIT && !SHORT && (!CAUSAL || D == 128)) ? 8 : 4;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int BM = WAVES * 32;
};
// Dense causal launches at d <= 128 over short sequences (at most
// PAIRED_MAX_BLOCKS row blocks; the SHORT instantiation) pair row blocks of
// complementary weight in one workgroup.  Longer sequences keep the
// weight-major order, which measured 0.5-1% faster there.
template <bool CAUSAL, bool SPARSE, bool SPLIT, bool SHORT> struct FwdPaired {
  static constexpr bool value = CAUSAL && !SPARSE && !SPLIT && SHORT;
};
constexpr int PAIRED_MAX_BLOCKS = 16;
// Key count up to which the non-causal dense forward runs four-wavefront
// workgroups (the crossover measured on MI355X lies between 2048 and 4096 keys
// at d = 128; at d = 64, with three wavefronts per SIMD, they were still 4.4%
// faster at 16384, the longest measured).
template <int D> struct NarrowKeys { static constexpr int MAX = D == 64 ? 16384 : 2048; };
// Reference max of the online softmax.  d <= 128: it moves (and the
// accumulators are rescaled) only when a lane's partial row sum over a tile
// exceeds PSUM_LIMIT.  d = 256: when a tile's row max exceeds it by more than
// RESCALE_THRESHOLD (log2 units).
constexpr float PSUM_LIMIT = 65536.0f;
constexpr float RESCALE_THRESHOLD = 8.0f;

// Key-tile height per head dimension: 64 keys at d <= 128 (8 KiB K or V tiles
// at d = 64, 16 KiB at d = 128), 32 at d = 256 (16 KiB).  At d = 64, 128-key
// tiles would double the score registers of the pipeline (two tiles' worth
// live at once), which left no room for the row-max-free softmax and cost
// 4-10% there.  The paired short causal kernel and the causal kernels at
// d = 64 (SMALL; the block-sparse one too, so that an all-ones mask steps
// through the keys as the dense kernel does) take 32-key tiles: their passes
// end on the diagonal, where the finer tiles waste less (paired: d = 128
// +2-7% at 512-2048 rows, d = 64 +7-15%; long causal d = 64: +1-5% at
// 4096-16384 rows, with 132 instead of 179 registers).  So does split-KV,
// whose short query blocks stream long key runs (+12% on 128 queries x
// 65536 keys; its 12-byte spill is gone).  Elsewhere 32-key tiles were 1-5%
// slower (block-sparse d = 128: 4-5%).
template <int D, bool SMALL = false> struct FwdTile {
  static constexpr int BN = D == 256 || SMALL ? 32 : 64;
};

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
// The four-wavefront non-causal kernel at d = 64 fits three (168 registers,
// with K fragments read one k-step ahead): +3-10% over two at N <= 16384.
template <int D, bool CAUSAL, bool SPARSE, bool SPLIT, bool SHORT> struct FwdOcc {
  static constexpr int WAVES_PER_SIMD = (D == 64 && SHORT && !CAUSAL) ? 3 : D <= 128 ? 2 : 1;
  static constexpr int MIN_WG_PER_CU =
      WAVES_PER_SIMD * 4 / FwdWG<D, CAUSAL, SPARSE, SPLIT, SHORT>::WAVES;  // launch-bounds form
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// How far ahead the LDS operand reads run: K fragments in k-steps of the score
// product (three at d = 256, whose 16 k-steps per tile leave more room; one in
// the three-wavefront-per-SIMD kernel), V^T fragments in products of P V.
template <int D> struct FwdPrefetch {
  static constexpr int K = D == 256 ? 3 : 2;
  static constexpr int V = 2;
};

template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool SPLIT, bool SHORT>
__global__ void __launch_bounds__((FwdWG<D, CAUSAL, SPARSE, SPLIT, SHORT>::THREADS),
                                  (FwdOcc<D, CAUSAL, SPARSE, SPLIT, SHORT>::MIN_WG_PER_CU))
attn_fwd_kernel(FwdArgs a) {
  constexpr int BN = FwdTile<D, FwdPaired<CAUSAL, SPARSE, SPLIT, SHORT>::value || (D == 64 && CAUSAL) || SPLIT>::BN;
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int TILE = BN * D;          // elements per K or V tile
  using WG = FwdWG<D, CAUSAL, SPARSE, SPLIT, SHORT>;
  constexpr int FWD_WAVES = WG::WAVES;
  constexpr int FWD_BM = WG::BM;
  constexpr int LPT = TILE / 8 / WG::THREADS;  // 16-byte loads per thread per tensor
  constexpr int NKK = D / 16;           // MFMA k-steps over d
  constexpr int NSB = BN / 32;          // 32-key sub-blocks per tile
  constexpr int NDB = D / 32;           // 32-wide d blocks of O
  constexpr int NKS = BN / 16;          // k-steps over keys in P V
  static_assert(LPT * 8 * WG::THREADS == TILE, "tile shape");
  constexpr int TPB = SPARSE_BLOCK / BN;  // key tiles per block of the mask
  static_assert(!SPARSE || FWD_BM == SPARSE_BLOCK, "one workgroup per row of the block mask");
  constexpr bool PAIRED = FwdPaired<CAUSAL, SPARSE, SPLIT, SHORT>::value;

  // K and V tiles are double-buffered separately: iteration j reads K_{j+1}
  // and V_j while K_{j+2} and V_{j+1} stream in.  Four separate objects, so
  // the compiler can tell the loads in flight never alias the reads.
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[TILE];
  // block-sparse: the key blocks this row block computes, in increasing order
  __shared__ uint16_t blist[SPARSE ? SPARSE_MAX_NB : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: keep it scalar
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- which (batch, head, row block) this workgroup owns ----
  const int nblk = (a.N + FWD_BM - 1) / FWD_BM;
  const int bid = grid_x(a.lt.reverse);
  int bh, rb_first, rb_second = -1;
  if constexpr (PAIRED) {
    // Short causal sequences (d = 128, the SHORT instantiation): each
    // workgroup takes row block nblk - 1 - p and then its complement p (none
    // when they coincide), nblk + 1 blocks of keys in all, so every
    // workgroup has the same work.  Consecutive work items are the pairs of one (batch, head)
    // on one XCD (xcd_remap), which run side by side and stream the same K/V
    // prefix through that XCD's L2.
    const int npair = (nblk + 1) / 2;
    const int L = xcd_remap(bid, npair * a.Hq * a.B);
    bh = L / npair;
    const int p = L - bh * npair;
    rb_first = nblk - 1 - p;
    rb_second = p != rb_first ? p : -1;
  } else if constexpr (CAUSAL && !SPARSE) {
    // Causal row blocks differ in work.  Weight-major order: the heaviest
    // row block of every (batch, head) first, then the next heaviest, ...
    // Consecutive work items go to consecutive XCDs (the hardware's round
    // robin), so every XCD gets an equal share of each weight and, when
    // B * Hq is a multiple of 8, every row block of a fixed set of heads.
    // Within a weight class the XCD of item i is i % 8 (B * Hq a multiple of
    // 8); XCD x takes the contiguous range of (batch, head) pairs
    // [x B Hq / 8, (x + 1) B Hq / 8), so the query heads of a GQA group and
    // the heads of one batch share K/V in one L2.
    const int BH = a.Hq * a.B;
    const int r = bid / BH;
    const int i = bid - r * BH;
    bh = (BH & 7) == 0 ? (i & 7) * (BH >> 3) + (i >> 3) : i;
    rb_first = nblk - 1 - r;
  } else {
    const int L = xcd_remap(bid, nblk * a.Hq * a.B);
    bh = L / nblk;
    rb_first = nblk - 1 - (L - bh * nblk);
  }
  // one row block, or (paired) two in turn; the LDS tiles are free between
  // them, every loop step ending with a barrier
  const int npass = PAIRED && rb_second >= 0 ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int rb = pass == 0 ? rb_first : rb_second;
    const int b = bh / a.Hq;
    const int h = bh - b * a.Hq;
    const int g = h / a.group;

    const size_t q_row = (size_t)a.Hq * D;   // elements between consecutive query rows
    const size_t kv_row = (size_t)a.Hkv * D;
    const uint16_t* qbase = (const uint16_t*)a.q + ((size_t)b * a.N * a.Hq + h) * D;
    // Split-KV: this workgroup's keys are [key_base, key_base + nk) of the
    // sequence; seen from them, the causal offset moves by -key_base.
    const int key_base = SPLIT ? (int)blockIdx.y * a.split_len : 0;
    const int nk = SPLIT ? max(0, min(a.split_len, a.Nk - key_base)) : a.Nk;
    const int coff = a.coff - key_base;
    const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)b * a.Nk * a.Hkv + g) * D + (size_t)key_base * kv_row;
    const uint16_t* vbase = (const uint16_t*)a.v + ((size_t)b * a.Nk * a.Hkv + g) * D + (size_t)key_base * kv_row;

    const int row0 = rb * FWD_BM;                 // first query row of the workgroup
    const int wrow0 = row0 + wave * 32;           // first query row of this wavefront
    const int qrow = wrow0 + l32;                 // this lane's query row
    const bool qvalid = qrow < a.N;
    // split-KV partials of this row
    float* const opart = SPLIT ? a.opart + ((((size_t)blockIdx.y * a.B + b) * a.N + qrow) * a.Hq + h) * D : nullptr;
    float* const lsepart = SPLIT ? a.lsepart + (((size_t)blockIdx.y * a.B + b) * a.Hq + h) * a.N + qrow : nullptr;
    // O = 0 and LSE = -inf for the rows of a workgroup that sees no key at all
    auto write_empty = [&]() __attribute__((always_inline)) {
      if (SPLIT) {
        if (qvalid) {
  #pragma unroll
          for (int i = 0; i < D / 8; ++i) *(f32x4_t*)(opart + 8 * i + 4 * half) = (f32x4_t){0.f, 0.f, 0.f, 0.f};
          if (half == 0) *lsepart = -INFINITY;
        }
        return;
      }
      if (qvalid) {
        uint16_t* orow = (uint16_t*)a.o + ((size_t)b * a.N * a.Hq + h) * D + (size_t)qrow * q_row;
  #pragma unroll
        for (int i = 0; i < D / 16; ++i) *(u32x4_t*)(orow + 16 * i + 8 * half) = (u32x4_t){0u, 0u, 0u, 0u};
        if (half == 0) a.lse[((size_t)b * a.Hq + h) * a.N + qrow] = -INFINITY;
      }
    };

    // ---- block-sparse: list the allowed key blocks of row block rb ----
    // (causal: blocks past the diagonal are dropped whatever the mask says)
    int nlist = 0;
    if constexpr (SPARSE) {
      if (wave == 0) {
        const uint8_t* mrow = a.sp.bmask + (size_t)g * a.sp.mask_hstride + (size_t)rb * a.sp.nb;
        const int cnt = compact_mask(mrow, 1, 0, CAUSAL ? rb + 1 : a.sp.nb, blist, lane);
        if (lane == 0) bcount = cnt;
      }
      __syncthreads();
      nlist = __builtin_amdgcn_readfirstlane(bcount);
      if (nlist == 0) {  // no allowed key in any row of the block
        write_empty();
        continue;
      }
    }
    // key tile computed in loop step j: j itself, or (block-sparse) tile
    // j % TPB of the (j / TPB)-th listed block
    auto ktile = [&](int j) __attribute__((always_inline)) {
      if constexpr (SPARSE) return lds_uniform(blist, j / TPB) * TPB + j % TPB;
      else return j;
    };

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
    // (causal: query i sees keys j <= i + coff)
    const int ntiles_all = (nk + BN - 1) / BN;
    int ntiles = ntiles_all;   // tiles the workgroup streams through LDS
    int nwave = ntiles_all;    // tiles this wavefront computes
    int nfull = nk / BN;       // leading tiles that need no element mask
    if (CAUSAL) {
      ntiles = max(0, min(ntiles_all, floor_div(min(row0 + FWD_BM, a.N) - 1 + coff, BN) + 1));
      nwave = max(0, min(ntiles, floor_div(wrow0 + 31 + coff, BN) + 1));
      nfull = max(0, min(min(nfull, ntiles), floor_div(wrow0 + 1 + coff, BN)));
    }
    if ((CAUSAL || SPLIT) && ntiles == 0) {  // an offset or an empty split: no key for any row
      write_empty();
      continue;
    }
    if constexpr (SPARSE) {
      // The counts above are bounds on the key tile index.  Every listed block
      // but the last lies wholly below each of them (only the last can be the
      // diagonal or the ragged end), so each becomes a count of loop steps.
      const int last = lds_uniform(blist, nlist - 1);
      auto steps_below = [&](int bound) { return (nlist - 1) * TPB + min(max(bound - last * TPB, 0), TPB); };
      ntiles = steps_below(ntiles);
      nwave = steps_below(nwave);
      nfull = steps_below(nfull);
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
    // One tile as a raw buffer resource (stride 0, dword 3 = 0x00020000) whose
    // record count ends at the sequence end: the per-lane offset is range-
    // checked, so rows past the end read as zeros (finite, and masked out).
    auto load_one = [&](int j, const uint16_t* base, const uint32_t* off, uint16_t* dstt) {
      const uint16_t* src = base + (size_t)j * BN * kv_row;
      // bytes from the tile's first row to the sequence end: < 2^32, as the host
      // bounds N * H * d below 2^31 elements
      const uint32_t nrec = (uint32_t)(nk - j * BN) * (uint32_t)kv_row * 2u;
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, (int)nrec, 0x00020000);
  #pragma unroll
      for (int i = 0; i < LPT; ++i) {
        const int dst = (i * FWD_WAVES + wave) * 64 * 8;  // wave-uniform LDS element offset
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)(dstt + dst), 16, off[i], 0, 0, 0);
      }
    };
    auto load_k = [&](int j, uint16_t* dstt) { load_one(ktile(j), kbase, ld_koff, dstt); };
    auto load_v = [&](int j, uint16_t* dstt) { load_one(ktile(j), vbase, ld_voff, dstt); };

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

    // S^T = K Q^T for one tile into s[], the K fragments read PFK k-steps ahead.
    // hook(kk) places independent VALU work after k-step kk's products, so that
    // it issues while they run.
    auto scores = [&](const uint16_t* ks, f32x16_t* s, auto&& hook) __attribute__((always_inline)) {
      constexpr int PFK = FwdOcc<D, CAUSAL, SPARSE, SPLIT, SHORT>::WAVES_PER_SIMD == 3 ? 1 : FwdPrefetch<D>::K;
      constexpr int PF = PFK < NKK ? PFK : NKK;
      frag8_t kf[PF + 1][NSB];
  #pragma unroll
      for (int sb = 0; sb < NSB; ++sb) s[sb] = (f32x16_t){};
  #pragma unroll
      for (int kk = 0; kk < PF; ++kk)
  #pragma unroll
        for (int sb = 0; sb < NSB; ++sb) kf[kk][sb] = *(const frag8_t*)(ks + 32 * sb * D + k_rd[kk]);
      static_for<0, NKK>([&](auto kkc) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
        if constexpr (kk + PF < NKK) {
  #pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
            kf[(kk + PF) % (PF + 1)][sb] = *(const frag8_t*)(ks + 32 * sb * D + k_rd[kk + PF]);
        }
  #pragma unroll
        for (int sb = 0; sb < NSB; ++sb) s[sb] = mfma32(Tag{}, kf[kk % (PF + 1)][sb], qf[kk], s[sb]);
        hook(kkc);
      });
    };

    // Softmax of the current tile's scores, formed in the shadow of the next
    // tile's score products.  Two forms, by head dimension:
    //  * d <= 128 (MAX_FREE): no per-tile row max.  All of the tile's
    //    probabilities are formed against the running reference max m_ref; if
    //    every lane's partial row sums stay <= PSUM_LIMIT, every probability
    //    does (no overflow, full relative precision) and the tile goes on to
    //    P V.  Only a tile that exceeds it (or is infinite: a row's first tile,
    //    m_ref = -inf, unless the prologue set it) takes the rare path that
    //    moves m_ref to the tile's max, rescales what is accumulated and forms
    //    the probabilities again.
    //  * d = 256: the row max is formed over the first half of the next
    //    tile's k-steps, the first half of P over the second half, and the rest
    //    of P under the first P V products; m_ref moves only when the tile
    //    raises it by more than 2^8 (RESCALE_THRESHOLD).  (At 32 keys per
    //    tile this split measured 1.6% faster than the MAX_FREE form.)
    constexpr bool MAX_FREE = D <= 128;
    struct SoftState {
      float mx4[4];      // row-max form: partial maxima
      float nm;          // -(reference max the tile's P is formed against)
      float m_new;       // row-max form: the reference max after this tile
      bool need;         // row-max form, wave-uniform: the reference max moves
      float tsum[4];     // this tile's partial row sums
      uint32_t w[NKS][4];
    };
    constexpr int PAIRS = NKS * 4;  // probability pairs per tile

    auto row_max_part = [&](const f32x16_t* s, SoftState& st, int e0, int e1) __attribute__((always_inline)) {
  #pragma unroll
      for (int e = e0; e < e1; e += 2) {  // four max3 chains, two new scores per step
        const int sb = e / 16, r = e % 16;
        const int a = (e >> 1) & 3;
        st.mx4[a] = e < 8 ? fmaxf(s[sb][r], s[sb][r + 1]) : fmaxf(fmaxf(st.mx4[a], s[sb][r]), s[sb][r + 1]);
      }
    };
    // the tile's scaled row max (the two halves of a row meet across lanes l, l ^ 32)
    auto row_max_scaled = [&](float mx) __attribute__((always_inline)) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, mx),
                                                       __builtin_bit_cast(uint32_t, mx), false, false);
      mx = fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
      // Causal, a row can have no allowed key in a tile (mx = -inf; with scale
      // 0, -inf * 0 would be NaN, so the select keeps -inf).  Without a mask
      // every tile gives every row a key.
      return (CAUSAL && mx == -INFINITY) ? -INFINITY : mx * c;
    };
    auto row_max_end = [&](SoftState& st) __attribute__((always_inline)) {
      const float mxs = row_max_scaled(fmaxf(fmaxf(fmaxf(st.mx4[0], st.mx4[1]), st.mx4[2]), st.mx4[3]));
      // deferred rescale: move the reference max only when it grows by > 2^8
      st.need = __builtin_amdgcn_ballot_w64(mxs > m_ref + RESCALE_THRESHOLD) != 0;
      st.m_new = st.need ? fmaxf(m_ref, mxs) : m_ref;
      // a row with no key so far keeps m_new = -inf; its probabilities are
      // all masked, shifted by 0 rather than +inf
      st.nm = (CAUSAL && st.m_new == -INFINITY) ? 0.f : -st.m_new;
    };
    // probability pairs [p0, p1) of the tile, pair index = 4 * key-k-step + t
    auto probs = [&](const f32x16_t* s, SoftState& st, int p0, int p1, auto mask_tag) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
  #pragma unroll
      for (int pp = p0; pp < p1; ++pp) {
        const int f = pp / 4, t = pp % 4;
        const int sb = f / 2, r = 8 * (f % 2) + 2 * t;
        float e0 = fast_exp2(__builtin_fmaf(s[sb][r], c, st.nm));
        float e1 = fast_exp2(__builtin_fmaf(s[sb][r + 1], c, st.nm));
        if (MASK) {  // masked scores are -inf: -inf * c + nm is NaN at scale 0 (or nm = +inf)
          e0 = s[sb][r] == -INFINITY ? 0.f : e0;
          e1 = s[sb][r + 1] == -INFINITY ? 0.f : e1;
        }
        st.w[f][t] = pack2(Tag{}, e0, e1);
        // fp32 row sums (LSE must not carry 16-bit rounding); the first pair
        // of each slot starts them
        if (pp < 4) st.tsum[t] = e0 + e1;
        else st.tsum[t] += e0 + e1;
        asm volatile("" : "+v"(st.w[f][t]), "+v"(st.tsum[t]));  // formed here, not sunk to its use
      }
    };
    // max-free form, wave-uniform: some lane's partial row sums exceed PSUM_LIMIT
    auto over_limit = [&](const SoftState& st) __attribute__((always_inline)) {
      const float m = fmaxf(fmaxf(fmaxf(st.tsum[0], st.tsum[1]), st.tsum[2]), st.tsum[3]);
      return __builtin_amdgcn_ballot_w64(m > PSUM_LIMIT) != 0;
    };
    // rescale what is accumulated by exp2(m_ref - m_new) and move m_ref (rare)
    auto move_ref = [&](float m_new) __attribute__((always_inline)) {
      // a lane whose row has seen no key yet keeps m_new = -inf: its factor is
      // 1 (the accumulators are still zero), not exp2(-inf + inf) = NaN
      const float alpha = (CAUSAL && m_new == -INFINITY) ? 1.f : fast_exp2(m_ref - m_new);
  #pragma unroll
      for (int t = 0; t < 4; ++t) lsum[t] *= alpha;
  #pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_ref = m_new;
    };
    auto apply_mask = [&](f32x16_t* s, int j) __attribute__((always_inline)) {
      const int key0 = ktile(j) * BN;
  #pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * sb + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool ok = key < nk && (!CAUSAL || key <= qrow + coff);
          s[sb][r] = ok ? s[sb][r] : -INFINITY;
        }
    };
    // O^T += V^T P^T; V^T fragments read PFV products ahead.  Row-max form:
    // the second half of P formed in the shadow of the first half's products.
    auto pv = [&](const uint16_t* vs, const f32x16_t* s, SoftState& st, auto mask_tag) __attribute__((always_inline)) {
      constexpr int NF = NKS * NDB;
      constexpr int PFV = FwdPrefetch<D>::V;
      constexpr int PAIRS2 = (NKS / 2) * 4;        // pairs still to form (row-max form)
      constexpr int NM2 = (NKS / 2) * NDB;         // products they may hide under
      frag8_t vf[PFV + 1];
      auto rd = [&](int f) __attribute__((always_inline)) {
        const uint16_t* p = vs + 16 * (f / NDB) * D + v_rd[f % NDB];
        s16x4_t lo = lds_read_tr(p);
        s16x4_t hi = lds_read_tr(p + 8 * D);
        return (frag8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
  #pragma unroll
      for (int f = 0; f < PFV; ++f) vf[f] = rd(f);
      static_for<0, NF>([&](auto fc) __attribute__((always_inline)) {
        constexpr int f = decltype(fc)::value;
        if constexpr (f + PFV < NF) vf[(f + PFV) % (PFV + 1)] = rd(f + PFV);
        constexpr int ks = f / NDB, db = f % NDB;
        if constexpr (!MAX_FREE && f < NM2) {  // pairs [PAIRS2 f / NM2, PAIRS2 (f + 1) / NM2) of the second half
          constexpr int q0 = PAIRS2 * f / NM2, q1 = PAIRS2 * (f + 1) / NM2;
          probs(s, st, (NKS / 2) * 4 + q0, (NKS / 2) * 4 + q1, mask_tag);
        }
        const u32x4_t wv = {st.w[ks][0], st.w[ks][1], st.w[ks][2], st.w[ks][3]};
        oacc[db] = mfma32(Tag{}, vf[f % (PFV + 1)], __builtin_bit_cast(frag8_t, wv), oacc[db]);
      });
      if constexpr (!MAX_FREE) {
  #pragma unroll
        for (int t = 0; t < 4; ++t) lsum[t] += st.tsum[t];
      }
    };

    // One pipelined step: softmax and P V of tile j (scores in s_cur) with the
    // next tile's scores formed in between.  HAS_NEXT false: no next scores.
    auto step = [&](int j, const uint16_t* knext, const uint16_t* vcur, f32x16_t* s_cur, f32x16_t* s_next,
                    auto mask_tag, auto next_tag) __attribute__((always_inline)) {
      constexpr bool HAS_NEXT = decltype(next_tag)::value;
      SoftState st;
      if constexpr (MAX_FREE) st.nm = -m_ref;
      if (decltype(mask_tag)::value) apply_mask(s_cur, j);
      constexpr int H = NKK / 2 > 0 ? NKK / 2 : 1;   // row-max form: k-steps for the row max
      constexpr int NE = NSB * 16;                   // score elements per lane
      constexpr int PAIRS1 = (NKS / 2) * 4;          // row-max form: pairs in the first half
      constexpr int H2 = NKK - H;                    // k-steps for them
      auto hook = [&](auto kkc) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
        if constexpr (MAX_FREE) {
          probs(s_cur, st, PAIRS * kk / NKK, PAIRS * (kk + 1) / NKK, mask_tag);
        } else if constexpr (kk < H) {
          row_max_part(s_cur, st, NE * kk / H, NE * (kk + 1) / H);
          if constexpr (kk == H - 1) row_max_end(st);
        } else {
          constexpr int i = kk - H;
          probs(s_cur, st, PAIRS1 * i / H2, PAIRS1 * (i + 1) / H2, mask_tag);
        }
      };
      if constexpr (HAS_NEXT) {
        // the next tile's products (this tile's softmax interleaved) issue at
        // raised priority, ahead of the other wavefront on the SIMD
        __builtin_amdgcn_s_setprio(1);
        scores(knext, s_next, hook);
        __builtin_amdgcn_s_setprio(0);
      } else {
        static_for<0, NKK>(hook);
      }
      if constexpr (MAX_FREE) {
        if (over_limit(st)) {  // rare: move m_ref to the tile's max and form P again
          float mx = -INFINITY;
  #pragma unroll
          for (int sb = 0; sb < NSB; ++sb)
  #pragma unroll
            for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s_cur[sb][r], s_cur[sb][r + 1]));
          move_ref(fmaxf(m_ref, row_max_scaled(mx)));
          st.nm = -m_ref;
          probs(s_cur, st, 0, PAIRS, mask_tag);
        }
  #pragma unroll
        for (int t = 0; t < 4; ++t) lsum[t] += st.tsum[t];
      } else {
        if (st.need) move_ref(st.m_new);
      }
      pv(vcur, s_cur, st, mask_tag);
    };

    f32x16_t sA[NSB], sB[NSB];
    uint16_t* const kb0 = k0s;
    uint16_t* const kb1 = k1s;
    uint16_t* const vb0 = v0s;
    uint16_t* const vb1 = v1s;

    // prologue: K_0, V_0, K_1 resident; scores of tile 0
    load_k(0, kb0);
    load_v(0, vb0);
    if (1 < ntiles) load_k(1, kb1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    scores(kb0, sA, [](auto) {});
    if constexpr (MAX_FREE) {
      // the reference max starts at tile 0's row max when every row of the
      // wavefront sees all of tile 0; otherwise the first check moves it
      if (nfull > 0) {
        float mx = -INFINITY;
  #pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
  #pragma unroll
          for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(sA[sb][r], sA[sb][r + 1]));
        m_ref = row_max_scaled(mx);
      }
    }
    __syncthreads();  // every wavefront is done with K_0 before K_2 replaces it

    // Iteration j: loads K_{j+2} -> K buffer j & 1 and V_{j+1} -> V buffer
    // (j + 1) & 1, reads K_{j+1} and V_j, one barrier at its end.  Every
    // wavefront passes exactly `ntiles` of these barriers.
    auto iter_loads = [&](int j, uint16_t* kdst, uint16_t* vdst) __attribute__((always_inline)) {
      if (j + 2 < ntiles) load_k(j + 2, kdst);
      if (j + 1 < ntiles) load_v(j + 1, vdst);
    };
    auto iter_end = [&]() __attribute__((always_inline)) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    int j = 0;
    // steady state: tiles j, j + 1 and j + 2 unmasked (tile j + 2's scores
    // are formed here)
    for (; j + 2 < nfull; j += 2) {
      iter_loads(j, kb0, vb1);
      step(j, kb1, vb0, sA, sB, std::false_type{}, std::true_type{});
      iter_end();
      iter_loads(j + 1, kb1, vb0);
      step(j + 1, kb0, vb1, sB, sA, std::false_type{}, std::true_type{});
      iter_end();
    }
    if constexpr (CAUSAL) {
      // the tiles up to this wavefront's last one (the diagonal and the ragged
      // end among them), pipelined like the steady state with the element mask
      // on; j is even here, so the buffers alternate as above
      for (; j + 2 < nwave; j += 2) {
        iter_loads(j, kb0, vb1);
        step(j, kb1, vb0, sA, sB, std::true_type{}, std::true_type{});
        iter_end();
        iter_loads(j + 1, kb1, vb0);
        step(j + 1, kb0, vb1, sB, sA, std::true_type{}, std::true_type{});
        iter_end();
      }
      // two tiles left (the loop above leaves at most two): the first
      // pipelined, the last's scores in sB
      if (j + 1 < nwave) {
        iter_loads(j, kb0, vb1);
        step(j, kb1, vb0, sA, sB, std::true_type{}, std::true_type{});
        iter_end();
        iter_loads(j + 1, kb1, vb0);
        step(j + 1, kb0, vb1, sB, sA, std::true_type{}, std::false_type{});
        iter_end();
        j += 2;
      }
    }
    if constexpr (!CAUSAL && !SPLIT && !SPARSE) {
      // non-causal, two tiles left after the steady state: the first
      // (unmasked) still forms the last tile's scores under its softmax; only
      // the last (masked where the sequence ends in it) runs unpipelined.
      // (Block-sparse and split-KV leave them to the loop below: this block
      // spills registers in the block-sparse kernel.)
      if (j + 2 == ntiles && j < nfull) {
        iter_loads(j, kb0, vb1);
        step(j, kb1, vb0, sA, sB, std::false_type{}, std::true_type{});
        iter_end();
        iter_loads(j + 1, kb1, vb0);
        step(j + 1, kb0, vb1, sB, sA, std::true_type{}, std::false_type{});
        iter_end();
        j += 2;
      }
    }
    // remaining tiles: the ragged ones, the last unmasked ones, and tiles only
    // other wavefronts need (causal: at most this wavefront's last tile is
    // computed here).  Not overlapped: the next tile's scores are formed after
    // this one's P V, in the same registers.
    for (; j < ntiles; ++j) {
      uint16_t* kcur = (j & 1) ? kb1 : kb0;   // K buffer j & 1 receives K_{j+2}
      uint16_t* knext = (j & 1) ? kb0 : kb1;
      uint16_t* vcur = (j & 1) ? vb1 : vb0;
      uint16_t* vnext = (j & 1) ? vb0 : vb1;
      iter_loads(j, kcur, vnext);
      if (j < nwave) {
        step(j, knext, vcur, sA, sB, std::true_type{}, std::false_type{});
        if (j + 1 < nwave) scores(knext, sA, [](auto) {});
      }
      iter_end();
    }

    // ---- epilogue: one division per row, LSE in natural log ----
    float ltot;
    {
      const float ls = (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, ls),
                                                       __builtin_bit_cast(uint32_t, ls), false, false);
      ltot = __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
    }
    // A row with no allowed key (causal, qrow + coff < 0) gets O = 0 and
    // LSE = -inf; the test is on integers (its sum is 0).
    const bool empty = CAUSAL && qrow + coff < 0;
    if (SPLIT) {  // fp32 partials, each normalised by its own sum
      if (qvalid) {
        const float inv = empty ? 0.f : 1.0f / ltot;
  #pragma unroll
        for (int db = 0; db < NDB; ++db)
  #pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4_t w = {oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv, oacc[db][4 * q4 + 2] * inv,
                         oacc[db][4 * q4 + 3] * inv};
            if (empty) w = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            *(f32x4_t*)(opart + 32 * db + 8 * q4 + 4 * half) = w;
          }
        if (half == 0) *lsepart = empty ? -INFINITY : (m_ref + log2f(ltot)) * 0.69314718055994530942f;
      }
      continue;
    }
    if (qvalid) {
      const float inv = empty ? 0.f : 1.0f / ltot;
      uint16_t* orow = (uint16_t*)a.o + ((size_t)b * a.N * a.Hq + h) * D + (size_t)qrow * q_row;
  #pragma unroll
      for (int db = 0; db < NDB; ++db)
  #pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d0 = 32 * db + 8 * q4 + 4 * half;
          u32x2_t w = {pack2(Tag{}, oacc[db][4 * q4 + 0] * inv, oacc[db][4 * q4 + 1] * inv),
                       pack2(Tag{}, oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv)};
          if (empty) w = (u32x2_t){0u, 0u};
          *(u32x2_t*)(orow + d0) = w;
        }
      if (half == 0) {
        const float lse2 = m_ref + log2f(ltot);
        a.lse[((size_t)b * a.Hq + h) * a.N + qrow] = empty ? -INFINITY : lse2 * 0.69314718055994530942f;
      }
    }
  }  // pass
}

// Split-KV merge: for each query row, LSE = ln sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s over the splits' fp32 partials (the exact
// combination of softmax over disjoint key sets); rows no split saw get
// O = 0, LSE = -inf.  One thread per 8 elements of a row; HBM-bound.
template <typename Tag, int D>
__global__ void __launch_bounds__(256) attn_fwd_merge_kernel(FwdArgs a) {
  constexpr int CPR = D / 8;       // 8-element chunks per row
  constexpr int ROWS = 256 / CPR;  // rows per workgroup
  const int tid = threadIdx.x;
  const int rloc = tid / CPR;
  const int c = tid - rloc * CPR;
  const long long row = (long long)blockIdx.x * ROWS + rloc;  // (b * N + n) * Hq + h
  const long long nrows = (long long)a.B * a.N * a.Hq;
  if (row >= nrows) return;
  const long long bn = row / a.Hq;
  const int h = (int)(row - bn * a.Hq);
  const long long b = bn / a.N;
  const int n = (int)(bn - b * a.N);
  const size_t lstride = (size_t)a.B * a.Hq * a.N;          // between the splits' LSE arrays
  const float* lp = a.lsepart + ((size_t)b * a.Hq + h) * a.N + n;
  float m = -INFINITY;
  for (int s = 0; s < a.splits; ++s) m = fmaxf(m, lp[s * lstride]);
  f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  const bool any = m > -INFINITY;
  if (any) {
    const float* op = a.opart + (size_t)row * D + 8 * c;
    for (int s = 0; s < a.splits; ++s) {
      const float w = fast_exp2((lp[s * lstride] - m) * 1.4426950408889634f);  // 0 for an empty split
      const f32x4_t* src = (const f32x4_t*)(op + (size_t)s * nrows * D);
      acc0 += w * src[0];
      acc1 += w * src[1];
      wsum += w;
    }
  }
  const float inv = any ? 1.0f / wsum : 0.f;
  const u32x4_t out = {pack2(Tag{}, acc0[0] * inv, acc0[1] * inv), pack2(Tag{}, acc0[2] * inv, acc0[3] * inv),
                       pack2(Tag{}, acc1[0] * inv, acc1[1] * inv), pack2(Tag{}, acc1[2] * inv, acc1[3] * inv)};
  *(u32x4_t*)((uint16_t*)a.o + (size_t)row * D + 8 * c) = out;
  if (c == 0) a.lse[((size_t)b * a.Hq + h) * a.N + n] = any ? m + logf(wsum) : -INFINITY;
}

}  // namespace

SplitWorkspace split_workspace_layout(int B, int N, int Hq, int d, int splits) {
  auto align256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  SplitWorkspace w;
  w.opart_off = 0;
  w.lsepart_off = align256((size_t)splits * B * N * Hq * d * sizeof(float));
  w.total = w.lsepart_off + align256((size_t)splits * B * Hq * N * sizeof(float));
  return w;
}

template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool SPLIT, bool SHORT = false>
hipError_t launch_fwd_s(const FwdArgs& a, hipStream_t stream) {
  using WG = FwdWG<D, CAUSAL, SPARSE, SPLIT, SHORT>;
  const int nblk = (a.N + WG::BM - 1) / WG::BM;
  constexpr bool PAIRED = FwdPaired<CAUSAL, SPARSE, SPLIT, SHORT>::value;
  const long long total = (long long)(PAIRED ? (nblk + 1) / 2 : nblk) * a.Hq * a.B;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (SPARSE && (a.sp.bmask == nullptr || a.sp.nb != nblk || a.sp.nb > SPARSE_MAX_NB || a.Nk != a.N || a.coff != 0))
    return hipErrorInvalidValue;
  if (SPLIT && (a.splits < 1 || a.splits > 65535 || a.split_len < 1 || a.split_len % SPARSE_BLOCK != 0 ||
                a.opart == nullptr || a.lsepart == nullptr))
    return hipErrorInvalidValue;
  const void* kfn = reinterpret_cast<const void*>(&attn_fwd_kernel<Tag, D, CAUSAL, SPARSE, SPLIT, SHORT>);
  hipLaunchKernelGGL((attn_fwd_kernel<Tag, D, CAUSAL, SPARSE, SPLIT, SHORT>), dim3((unsigned)total, SPLIT ? a.splits : 1),
                     dim3(WG::THREADS), one_wg_lds_pad(kfn, a.lt.one_wg_per_cu), stream, a);
  hipError_t e = hipGetLastError();
  if (!SPLIT || e != hipSuccess) return e;
  constexpr int ROWS = 256 / (D / 8);
  const long long grid = ((long long)a.B * a.N * a.Hq + ROWS - 1) / ROWS;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((attn_fwd_merge_kernel<Tag, D>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename Tag, int D, bool CAUSAL>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  if (a.sp.bmask) return launch_fwd_s<Tag, D, CAUSAL, true, false>(a, stream);
  if (a.splits > 1 || a.opart) return launch_fwd_s<Tag, D, CAUSAL, false, true>(a, stream);
  if constexpr (!CAUSAL && D <= 128) {
    if (a.Nk <= NarrowKeys<D>::MAX) return launch_fwd_s<Tag, D, false, false, false, true>(a, stream);
  }
  if constexpr (CAUSAL && D <= 128) {
    if ((a.N + 127) / 128 <= PAIRED_MAX_BLOCKS) return launch_fwd_s<Tag, D, true, false, false, true>(a, stream);
  }
  return launch_fwd_s<Tag, D, CAUSAL, false, false>(a, stream);
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
