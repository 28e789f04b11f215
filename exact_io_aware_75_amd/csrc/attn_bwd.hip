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
//  1. bwd_pre:  D = rowsum(dO * O) per query row (fp32).
//  2. bwd_dkdv: one workgroup per (batch, K/V head, block of 128 keys) --
//     parallel over the key (column) dimension, as the pages describe for
//     the backward pass (FlashAttention-2 review, "Параллелизм").  Each
//     wavefront owns 32 keys; dK and dV stay in registers through the loop
//     over the query heads of the GQA group and the query tiles (causal: only
//     tiles at or below the diagonal).  Products: S, dP, dV, dK.
//  3. bwd_dq:   one workgroup per (batch, query head, block of 256 queries,
//     128 when causal or at d = 256) --
//     parallel over rows like the forward pass.  Each wavefront owns 32
//     queries and recomputes S and dP for them, then dQ += dS K.  Products:
//     S, dP, dQ.
//
// Splitting dQ off costs two extra products (seven instead of five) but
// replaces the fp32 atomic accumulation of dQ partials, which on this 8-XCD
// part run past the per-XCD L2 (4+ GB of memory-side atomics per launch at
// N = 4k), and the cross-wavefront staging of dS; the result is also
// deterministic.
//
// CDNA4 mapping (v_mfma_f32_32x32x16, 64-lane wavefronts, two wavefronts per
// SIMD for d <= 128).  Tiles move HBM -> LDS by DMA (buffer_load_dwordx4 ...
// lds for dK/dV, global_load_lds_dwordx4 for dQ) into unpadded tiles
// swizzled in 16-byte chunks; the swizzle is free of bank
// conflicts both for 128-bit row reads (16 rows x one chunk per cycle) and
// for ds_read_b64_tr_b16 transposed reads (4 rows x 4 chunks per cycle),
// because every tile here is read both ways.
//  * dK/dV: S = Q K^T and dP = dO V^T with the key on the lane, so P and dS
//    are directly the B operands of dV^T += dO^T P and dK^T += Q^T dS; dO^T
//    and Q^T are transposed reads of the Q / dO tiles.  The operand
//    fragments of every product are read one k-step (S, dP) or two products
//    (dV, dK) ahead of their use, so a product rarely waits on LDS latency.
//  * dQ: S^T = K Q^T and dP^T = V dO^T with the query on the lane (LSE and D
//    are per lane), so dS^T is directly the B operand of dQ^T += K^T dS^T;
//    K^T is a transposed read of the K tile.  Operand fragments are read one
//    k-step (S^T, dP^T) or two products (dQ^T) ahead, as in dK/dV.
#include "attn_common.hpp"
#include "attn_kernels.hpp"

namespace attn {

namespace {

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

typedef __attribute__((address_space(1))) const void* gptr_t;
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lptr_t;

// 16-byte-chunk swizzle (row r, logical chunk c stored at chunk c ^ swz(r));
// 64 four-byte banks = 16 chunk-wide bank groups.  A 128-bit read serves 16
// lanes per cycle (here 16 consecutive rows at one logical chunk: swz must
// be a bijection on 16 consecutive rows, taking the 8-chunk rows of d = 64
// into account); a transposed read serves 32 lanes per cycle (4 consecutive
// rows x 4 adjacent chunks: the 4 rows must differ in bits 2-3 of swz).
template <int D> __device__ __forceinline__ int swz(int r) {
  return D == 64 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3) : 4 * (r & 3) + ((r >> 2) & 3);
}

// Workgroup barrier that waits for this wavefront's LDS reads only; HBM ->
// LDS loads are waited for explicitly before the barrier that precedes their
// first reader.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// HBM -> LDS load of a tile of R rows x D columns (16-bit) with the swizzle,
// shared by the W wavefronts of a workgroup.  Thread (wave, lane) fills chunks
// (W i + wave) * 64 + lane; when the tile has fewer chunks than threads, the
// wavefronts past its end load nothing.
//
// Two forms.  The buffer form (buffer_load_dwordx4 ... lds; the dK/dV pass)
// leaves the LDS wait counter usable: the compiler counts global_load_lds as
// an LDS access that may complete out of order and so waits for every
// outstanding LDS read (lgkmcnt(0)) before each product while a tile load is
// in flight, which serialised the dK/dV products on LDS latency (11% of its
// time).  The dQ pass, whose products wait less on LDS, measured within a
// few percent either way and keeps the global form (GLOBAL_DMA).  Rows at or past `valid` read row valid - 1 instead
// (any finite values do: they are masked or never stored).
// One 16-byte-per-lane HBM -> LDS load through a raw buffer resource
// (stride 0, dword 3 = 0x00020000) of nrec bytes from base: lanes whose offset
// is past the record count write zeros.  (A free function: with the resource
// built inside a member of a class template, this compiler silently dropped
// the host-side launch stubs of some kernel instantiations.)
__device__ __forceinline__ void buffer_lds16(const void* base, uint32_t nrec, uint32_t voff, uint16_t* dst) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)nrec, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lptr_t)dst, 16, voff, 0, 0, 0);
}

template <int D, int R, int W = 4, bool GLOBAL_DMA = false>
struct TileDma {
  static constexpr int CPR = D / 8;
  static constexpr int CHUNKS = R * CPR;
  static constexpr int LPT = (CHUNKS + 64 * W - 1) / (64 * W);
  static_assert(CHUNKS % 64 == 0, "tile/thread mismatch");
  uint32_t off[LPT];  // byte offset of each chunk's source within the tile
  int wave, lane;
  // chunk index of load i of this thread; wave-uniform test for existence
  __device__ __forceinline__ bool has(int i) const { return (i * W + wave) * 64 < CHUNKS; }
  __device__ __forceinline__ void init(int gstride, int wave_, int lane_) {
    wave = wave_;
    lane = lane_;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int q = (i * W + wave) * 64 + lane;
      const int r = q / CPR;
      const int p = q % CPR;
      off[i] = (uint32_t)(2 * (r * gstride + (p ^ swz<D>(r)) * 8));
    }
  }
  // src: first row of the tile; valid: rows of the tile that exist.  Rows at
  // or past `valid` read as zeros (buffer form: the record count ends there)
  // or as row valid - 1 (global form); any finite values do, since their
  // probabilities are masked to 0.
  __device__ __forceinline__ void load(const uint16_t* src, int valid, int gstride, uint16_t* dst) const {
    if (GLOBAL_DMA) {
      const char* s = (const char*)src;
      if (valid >= R) {
#pragma unroll
        for (int i = 0; i < LPT; ++i)
          if (has(i))
            __builtin_amdgcn_global_load_lds((gptr_t)(s + off[i]), (lptr_t)(dst + (i * W + wave) * 512), 16, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
          if (!has(i)) continue;
          const int r = ((i * W + wave) * 64 + lane) / CPR;
          const uint32_t back = (uint32_t)(2 * max(0, r - (valid - 1)) * gstride);
          __builtin_amdgcn_global_load_lds((gptr_t)(s + (off[i] - back)), (lptr_t)(dst + (i * W + wave) * 512), 16, 0, 0);
        }
      }
      return;
    }
    const uint32_t nrec = (uint32_t)(valid < R ? valid : R) * (uint32_t)gstride * 2u;
#pragma unroll
    for (int i = 0; i < LPT; ++i)
      if (has(i)) buffer_lds16(src, nrec, off[i], dst + (i * W + wave) * 512);
  }
};

// Per-lane LDS element offsets for reading operand fragments out of a
// swizzled tile whose row stride is D elements.
template <int D>
struct FragRd {
  // Per-lane base element offsets.  The swizzled chunk bits of every offset
  // lie below the row bits, so the offset of k-step kk (or d block db) is the
  // base XOR a constant: one v_xor per read instead of a shift, XOR and add.
  // 128-bit row reads: row = 32-aligned base + l32, logical chunk 2 kk + half.
  int row_b;
  // transposed reads: rows 16 ks + {0, 8} + 4 half + gi / 4, elements
  // 32 db + 16 (grp & 1) + 4 (gi & 3).
  int tr_lo, tr_hi;
  __device__ __forceinline__ void init(int lane) {
    const int half = lane >> 5, l32 = lane & 31, grp = lane >> 4, gi = lane & 15;
    row_b = l32 * D + ((swz<D>(l32) ^ half) << 3);
    const int r = 4 * half + (gi >> 2);
    const int cl = 2 * (grp & 1) + ((gi & 3) >> 1);
    tr_lo = r * D + 4 * (gi & 1) + ((swz<D>(r) ^ cl) << 3);
    tr_hi = (r + 8) * D + 4 * (gi & 1) + ((swz<D>(r + 8) ^ cl) << 3);
  }
  // Hide the offsets from loop-invariant code motion (which would otherwise
  // keep one copy of every address per LDS buffer live across the loop).
  __device__ __forceinline__ void pin() { asm volatile("" : "+v"(row_b), "+v"(tr_lo), "+v"(tr_hi)); }
  // fragment of rows [32 rb, 32 rb + 32), k-step kk (16 columns)
  __device__ __forceinline__ frag8_t row(const uint16_t* t, int rb, int kk) const {
    return *(const frag8_t*)(t + 32 * rb * D + (row_b ^ (16 * kk)));
  }
  // transposed fragment: reduction rows [16 ks, 16 ks + 16), columns [32 db, 32 db + 32)
  __device__ __forceinline__ frag8_t tr(const uint16_t* t, int ks, int db) const {
    const uint16_t* base = t + 16 * ks * D;
    const s16x4_t lo = lds_read_tr(base + (tr_lo ^ (32 * db)));
    const s16x4_t hi = lds_read_tr(base + (tr_hi ^ (32 * db)));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// ---------------------------------------------------------------------------
// 1. D = rowsum(dO * O)
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

// Registers are budgeted for two wavefronts per SIMD up to d = 128.
template <int D> struct BwdOcc { static constexpr int WAVES_PER_SIMD = D <= 128 ? 2 : 1; };

// Wavefronts per workgroup (32 keys or 32 queries each).  The non-causal dQ
// pass at d <= 128 runs eight (one workgroup per CU at two wavefronts per
// SIMD), so each staged K/V tile serves 256 queries: 5-8% faster than four.
// Causal dQ keeps four (the wavefronts of a diagonal block have unequal trip
// counts) except at d = 128 from DQ_WIDE_ROWS query rows on (the WIDE
// instantiation: +1-2% there, up to 9% slower over short sequences), and
// dK/dV keeps four, where eight measured 3% slower non-causal and 14% slower
// causal (a 256-key block computes more masked diagonal tiles).
// Block-sparse dQ keeps four too, so that a workgroup's 128 queries are one
// row of the block mask (as a dK/dV workgroup's 128 keys are one column).
template <int D, bool CAUSAL> struct DkdvWG { static constexpr int WAVES = 4; };
template <int D, bool CAUSAL, bool SPARSE = false, bool WIDE = false> struct DqWG {
  static constexpr int WAVES = (D <= 128 && !SPARSE && (!CAUSAL || WIDE)) ? 8 : 4;
};
constexpr int DQ_WIDE_ROWS = 8192;
template <int D, int W> struct BwdBounds {
  static constexpr int THREADS = 64 * W;
  static constexpr int MIN_WG = BwdOcc<D>::WAVES_PER_SIMD * 4 / W;
};

// ---------------------------------------------------------------------------
// 2. dK, dV: one workgroup per (batch, K/V head, 128 keys)
// ---------------------------------------------------------------------------
constexpr int KV_BM = 32;   // query rows per tile
constexpr int BWD_PFT = 2;  // transposed fragments read ahead in dV/dK

template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool PAIRED = false>
__global__ void __launch_bounds__((BwdBounds<D, DkdvWG<D, CAUSAL>::WAVES>::THREADS),
                                  (BwdBounds<D, DkdvWG<D, CAUSAL>::WAVES>::MIN_WG))
attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int W = DkdvWG<D, CAUSAL>::WAVES;
  constexpr int KV_BN = 32 * W;  // keys per workgroup
  constexpr int TQ = KV_BM * D;   // elements of one Q (or dO) tile
  constexpr int NKK = D / 16;     // k-steps over d
  constexpr int NDB = D / 32;     // 32-wide d blocks
  // V stays in LDS at d >= 128 (its B-operand fragments would not fit in
  // registers next to the dK/dV accumulators); at d = 64 it is in registers.
  constexpr bool V_LDS = D >= 128;
  constexpr bool FOLD_D = D <= 128;  // -D as the dP accumulator's initial value
  static_assert(!SPARSE || KV_BN == SPARSE_BLOCK, "one workgroup per column of the block mask");

  __shared__ __attribute__((aligned(1024))) uint16_t q0s[TQ];
  __shared__ __attribute__((aligned(1024))) uint16_t q1s[TQ];
  __shared__ __attribute__((aligned(1024))) uint16_t o0s[TQ];
  __shared__ __attribute__((aligned(1024))) uint16_t o1s[TQ];
  __shared__ __attribute__((aligned(1024))) uint16_t vblk[V_LDS ? KV_BN * D : 8];
  __shared__ __attribute__((aligned(16))) float lse0[KV_BM], lse1[KV_BM], del0[KV_BM], del1[KV_BM];
  // block-sparse: the query blocks this key block meets, in increasing order
  __shared__ uint16_t blist[SPARSE ? SPARSE_MAX_NB : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- which (batch, kv head, head split, key block) this workgroup owns ----
  // (consecutive work items: consecutive key blocks of one head split, which
  // stream the same query tiles)
  // (d = 256 never splits: its registers are already full)
  const int hs = D <= 128 ? a.hsplit : 1;
  const int nkb = (a.Nk + KV_BN - 1) / KV_BN;
  const int bid = grid_x(a.lt.reverse);
  int bgs, kb_first, kb_second = -1;
  if constexpr (PAIRED) {
    // Short causal sequences (at most PAIRED_MAX_BLOCKS key blocks): each
    // workgroup takes key block p (the heavier) and then nkb - 1 - p, so all
    // have the same work; the pairs of one (batch, kv head, head split) are
    // consecutive work items on one XCD, which stream the same Q/dO tiles
    // through its L2 at the same time.
    const int npair = (nkb + 1) / 2;
    const int L = xcd_remap(bid, npair * a.Hkv * a.B * hs);
    bgs = L / npair;
    kb_first = L - bgs * npair;
    kb_second = nkb - 1 - kb_first != kb_first ? nkb - 1 - kb_first : -1;
  } else if constexpr (CAUSAL && !SPARSE) {
    // Causal key blocks differ in work (the first sees every query):
    // weight-major order with consecutive work items on consecutive XCDs,
    // as in the causal forward pass.
    const int G = a.Hkv * a.B * hs;
    kb_first = bid / G;
    bgs = bid - kb_first * G;
  } else {
    const int Lw = xcd_remap(bid, nkb * a.Hkv * a.B * hs);
    bgs = Lw / nkb;
    kb_first = Lw - bgs * nkb;
  }
  // one key block, or (paired) two in turn; the LDS buffers are free between
  // them, every loop step ending with a barrier
  auto body = [&](const int kb) __attribute__((always_inline)) {
    const int bg = bgs / hs;
    const int split = bgs - bg * hs;
    const int gs = a.group / hs;  // query heads of the group this workgroup covers
    const int b = bg / a.Hkv;
    const int g = bg - b * a.Hkv;
    const int k0 = kb * KV_BN;           // first key of the block
    const int kw0 = k0 + wave * 32;      // first key of this wavefront
    const int mykey = kw0 + l32;         // this lane's key (C-layout column)

    const int q_row = a.Hq * D;
    const int kv_row = a.Hkv * D;
    const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)b * a.Nk * a.Hkv + g) * D;
    const uint16_t* vbase = (const uint16_t*)a.v + ((size_t)b * a.Nk * a.Hkv + g) * D;

    // K (and V if in registers) as B operands: lane = key, 8 consecutive d per k-step
    frag8_t kf[NKK], vf[V_LDS ? 1 : NKK];
    {
      const uint16_t* kr = kbase + (size_t)min(mykey, a.Nk - 1) * kv_row + 8 * half;
      const uint16_t* vr = vbase + (size_t)min(mykey, a.Nk - 1) * kv_row + 8 * half;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        kf[kk] = *(const frag8_t*)(kr + 16 * kk);
        if (!V_LDS) vf[V_LDS ? 0 : kk] = *(const frag8_t*)(vr + 16 * kk);
      }
    }
    FragRd<D> fr;
    fr.init(lane);
    if (V_LDS) {  // the V block, [key][d], swizzled; read as B operand (lane = key)
      TileDma<D, KV_BN, W> vdma;
      vdma.init(kv_row, wave, lane);
      vdma.load(vbase + (size_t)k0 * kv_row, a.Nk - k0, kv_row, vblk);
    }

    f32x16_t dk_acc[NDB], dv_acc[NDB];  // dK^T, dV^T: lane = key, rows = d
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
      dk_acc[i] = (f32x16_t){};
      dv_acc[i] = (f32x16_t){};
    }

    // query tiles: every head of the GQA group x tiles of KV_BM rows
    // (causal: only tiles with a row i that sees key k0, i + coff >= k0)
    const int nqt = (a.N + KV_BM - 1) / KV_BM;
    const int qt0 = CAUSAL ? min(nqt, max(0, floor_div(k0 - a.coff, KV_BM))) : 0;
    int tiles_per_head = nqt - qt0;
    // Block-sparse: the query tiles of the listed query blocks (causal: from
    // the diagonal block on), KV_BM rows at a time; only the last block of the
    // sequence can be ragged, and it can only be the last listed.
    int nlist = 0;
    if constexpr (SPARSE) {
      if (wave == 0) {
        const uint8_t* mcol = a.sp.bmask + (size_t)g * a.sp.mask_hstride + kb;
        const int cnt = compact_mask(mcol, a.sp.nb, CAUSAL ? kb : 0, a.sp.nb, blist, lane);
        if (lane == 0) bcount = cnt;
      }
      __syncthreads();
      nlist = __builtin_amdgcn_readfirstlane(bcount);
      constexpr int QPB = SPARSE_BLOCK / KV_BM;  // query tiles per block
      tiles_per_head = nlist * QPB;
      if (nlist > 0 && lds_uniform(blist, nlist - 1) == a.sp.nb - 1)
        tiles_per_head -= QPB - (a.N - (a.sp.nb - 1) * SPARSE_BLOCK + KV_BM - 1) / KV_BM;
    }
    const int ntiles = tiles_per_head * gs;
    const float c = a.scale_log2;  // scale * log2(e), signed

    TileDma<D, KV_BM, W> qdma;
    qdma.init(q_row, wave, lane);
    // Tile coordinates advance incrementally: query rows within a head, then
    // the next head of the group.
    const int qfirst = qt0 * KV_BM, qend = nqt * KV_BM;
    int li = 0;  // block-sparse: list entry of the next tile to load
    auto advance = [&](int& h, int& q0) {
      q0 += KV_BM;
      if constexpr (SPARSE) {
        const int blk = q0 - KV_BM - (q0 - KV_BM) % SPARSE_BLOCK;  // first row of the tile's block
        if (q0 >= min(blk + SPARSE_BLOCK, a.N)) {
          if (++li == nlist) {
            li = 0;
            ++h;
          }
          q0 = lds_uniform(blist, li) * SPARSE_BLOCK;
        }
      } else if (q0 >= qend) {
        q0 = qfirst;
        ++h;
      }
    };
    // Q and dO tiles by DMA.  LSE and D of the tile's rows are loaded raw into
    // a register by threads 0 .. 2 KV_BM - 1 (LSE by the first KV_BM, D by the
    // rest) and only converted and stored to LDS at the end of the step, so
    // nothing waits for the load before the tile's products.
    float lsd_raw = 0.f;
    bool lsd_valid = false;
    auto load = [&](int h, int q0, uint16_t* qs, uint16_t* os) {
      if (tid < 2 * KV_BM) {
        const int qr = q0 + (tid & (KV_BM - 1));
        const size_t li = ((size_t)b * a.Hq + h) * a.N + min(qr, a.N - 1);
        const float* src = tid < KV_BM ? a.lse : a.delta;
        lsd_raw = src[li];
        lsd_valid = qr < a.N;
      }
      const size_t rowbase = ((size_t)b * a.N + q0) * a.Hq + h;
      qdma.load((const uint16_t*)a.q + rowbase * D, a.N - q0, q_row, qs);
      qdma.load((const uint16_t*)a.dout + rowbase * D, a.N - q0, q_row, os);
    };
    auto store_lsd = [&](float* ls, float* ds) {
      // LSE in log2 units; rows past the end get +inf, so their probabilities
      // are 0.  D is stored negated where it initialises the dP accumulator.
      if (tid < KV_BM) ls[tid] = lsd_valid ? lsd_raw * 1.4426950408889634f : INFINITY;
      else if (tid < 2 * KV_BM) ds[tid - KV_BM] = FOLD_D ? -lsd_raw : lsd_raw;
    };

    // Causal: one tile body serves all tiles (a second full body spills); only
    // the formation of P and dS takes the element mask, and at d >= 128 only
    // on the tiles that cross the wavefront's diagonal.
    auto tile = [&](int q0, const uint16_t* qs, const uint16_t* os, const float* ls, const float* dls)
        __attribute__((always_inline)) {
      // S = Q K^T and dP = dO V^T for 32 queries x this wavefront's 32 keys;
      // the Q, dO (and V) fragments of k-step kk + 1 are read while k-step kk's
      // two products run
      // At d <= 128 dP starts from -D (C rows = queries 8 (r / 4) + 4 half +
      // r % 4, four consecutive rows per 128-bit read), so the products leave
      // dP - D; at d = 256 (registers too tight) D is subtracted afterwards.
      f32x16_t s = {}, dp = {};
      if (FOLD_D) {
        const f32x4_t n0 = *(const f32x4_t*)(dls + 4 * half), n1 = *(const f32x4_t*)(dls + 8 + 4 * half);
        const f32x4_t n2 = *(const f32x4_t*)(dls + 16 + 4 * half), n3 = *(const f32x4_t*)(dls + 24 + 4 * half);
        const f32x8_t lo = __builtin_shufflevector(n0, n1, 0, 1, 2, 3, 4, 5, 6, 7);
        const f32x8_t hi = __builtin_shufflevector(n2, n3, 0, 1, 2, 3, 4, 5, 6, 7);
        dp = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      }
      {
        frag8_t qa[2], oa[2], va[2];
        auto rd = [&](int kk, int i) __attribute__((always_inline)) {
          qa[i] = fr.row(qs, 0, kk);
          oa[i] = fr.row(os, 0, kk);
          if (V_LDS) va[i] = fr.row(vblk, wave, kk);
        };
        rd(0, 0);
        // Issue priority: while a wavefront runs a block of products it issues
        // ahead of the other wavefront on its SIMD, which meanwhile runs its
        // exponentials; the matrix pipe then sees fewer gaps (3-4% on this pass).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if (kk + 1 < NKK) rd(kk + 1, (kk + 1) & 1);
          s = mfma32(Tag{}, qa[kk & 1], kf[kk], s);
          const frag8_t vv = V_LDS ? va[kk & 1] : vf[V_LDS ? 0 : kk];
          dp = mfma32(Tag{}, oa[kk & 1], vv, dp);
          if (kk + 1 < NKK) __builtin_amdgcn_sched_group_barrier(0x100, V_LDS ? 3 : 2, 0);  // DS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                                // MFMA
        }
        __builtin_amdgcn_s_setprio(0);
      }
      // P = 2^(S c - LSE2), dS = P (dP - D)
      const int klim = mykey - a.coff - q0 - 4 * half;
      u32x4_t pq[2], dsq[2];  // packed P and dS, already the B-operand register tuples
      auto form = [&](auto mask_tag) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4_t l4 = *(const f32x4_t*)(ls + 8 * r4 + 4 * half);
          f32x4_t d4 = {};
          if (!FOLD_D) d4 = *(const f32x4_t*)(dls + 8 * r4 + 4 * half);
          float p[4], dsv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            float pv = fast_exp2(__builtin_fmaf(s[r], c, -l4[e]));
            if (MASK) pv = (8 * r4 + e) < klim ? 0.f : pv;  // query < key
            p[e] = pv;
            dsv[e] = pv * (FOLD_D ? dp[r] : dp[r] - d4[e]);
          }
          pq[r4 >> 1][2 * (r4 & 1)] = pack2(Tag{}, p[0], p[1]);
          pq[r4 >> 1][2 * (r4 & 1) + 1] = pack2(Tag{}, p[2], p[3]);
          dsq[r4 >> 1][2 * (r4 & 1)] = pack2(Tag{}, dsv[0], dsv[1]);
          dsq[r4 >> 1][2 * (r4 & 1) + 1] = pack2(Tag{}, dsv[2], dsv[3]);
        }
      };
      // causal: only the tiles that cross this wavefront's diagonal (some lane
      // has a query before its key) take the element mask -- at d >= 128; at
      // d = 64 the second form would cost the three wavefronts per SIMD
      if constexpr (CAUSAL && D >= 128) {
        if (__builtin_amdgcn_ballot_w64(klim > 0) != 0) form(std::true_type{});
        else form(std::false_type{});
      } else {
        form(std::bool_constant<CAUSAL>{});
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the tile's 32 queries (two
      // k-steps); the transposed fragments are read PFT products ahead
      {
        constexpr int NF = 2 * 2 * NDB;  // products, in (ks, db, dV/dK) order
        constexpr int PFT = BWD_PFT;
        frag8_t ta[PFT + 1];
        auto rd = [&](int f) __attribute__((always_inline)) {
          const int ks = f / (2 * NDB), db = (f / 2) % NDB;
          return fr.tr((f & 1) ? qs : os, ks, db);
        };
#pragma unroll
        for (int f = 0; f < PFT; ++f) ta[f] = rd(f);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + PFT < NF) ta[(f + PFT) % (PFT + 1)] = rd(f + PFT);
          const int ks = f / (2 * NDB), db = (f / 2) % NDB;
          if (f & 1)
            dk_acc[db] = mfma32(Tag{}, ta[f % (PFT + 1)], __builtin_bit_cast(frag8_t, dsq[ks]), dk_acc[db]);
          else
            dv_acc[db] = mfma32(Tag{}, ta[f % (PFT + 1)], __builtin_bit_cast(frag8_t, pq[ks]), dv_acc[db]);
          if (f + PFT < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
        }
        __builtin_amdgcn_s_setprio(0);
      }
    };

    // Tile t lives in buffer t & 1; one barrier per tile, the same number for
    // every wavefront.
    int lh = g * a.group + split * gs, lq = qfirst;  // coordinates of the next tile to load
    if constexpr (SPARSE) lq = nlist > 0 ? lds_uniform(blist, 0) * SPARSE_BLOCK : 0;
    if (ntiles > 0) {
      load(lh, lq, q0s, o0s);
      store_lsd(lse0, del0);
    }
    int cq = lq;  // first query row of the tile being computed
    if (!SPARSE || ntiles > 0) advance(lh, lq);  // (an empty list has no entry to advance to)
    wait_loads();
    __syncthreads();
    auto step = [&](int t, int buf) __attribute__((always_inline)) {
      if (t + 1 < ntiles) {
        if (buf) load(lh, lq, q0s, o0s);
        else load(lh, lq, q1s, o1s);
      }
      fr.pin();
      if (buf) tile(cq, q1s, o1s, lse1, del1);
      else tile(cq, q0s, o0s, lse0, del0);
      cq = lq;
      advance(lh, lq);
      if (t + 1 < ntiles) {
        if (buf) store_lsd(lse0, del0);
        else store_lsd(lse1, del1);
      }
      wait_loads();
      __syncthreads();
    };
    int t = 0;
    for (; t + 1 < ntiles; t += 2) {
      step(t, 0);
      step(t + 1, 1);
    }
    if (t < ntiles) step(t, 0);

    // ---- epilogue: dK = scale * dK_acc, dV = dV_acc; lane = key, rows = d ----
    if (hs > 1) {  // fp32 partials of this head split, summed by the reduce kernel
      if (mykey < a.Nk) {
        const size_t per = (size_t)a.B * a.Nk * a.Hkv * D;
        float* pk = a.dkv_part + (size_t)split * 2 * per + (((size_t)b * a.Nk + mykey) * a.Hkv + g) * D;
        float* pv = pk + per;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int d0 = 32 * db + 8 * q4 + 4 * half;
            *(f32x4_t*)(pk + d0) = (f32x4_t){dk_acc[db][4 * q4], dk_acc[db][4 * q4 + 1], dk_acc[db][4 * q4 + 2],
                                             dk_acc[db][4 * q4 + 3]};
            *(f32x4_t*)(pv + d0) = (f32x4_t){dv_acc[db][4 * q4], dv_acc[db][4 * q4 + 1], dv_acc[db][4 * q4 + 2],
                                             dv_acc[db][4 * q4 + 3]};
          }
      }
    } else if (mykey < a.Nk) {
      uint16_t* dkp = (uint16_t*)a.dk + ((size_t)b * a.Nk * a.Hkv + g) * D + (size_t)mykey * kv_row;
      uint16_t* dvp = (uint16_t*)a.dv + ((size_t)b * a.Nk * a.Hkv + g) * D + (size_t)mykey * kv_row;
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
  };
  body(kb_first);
  if constexpr (PAIRED) {
    if (kb_second >= 0) body(kb_second);
  }
}

// ---------------------------------------------------------------------------
// 3. dQ: one workgroup per (batch, query head, 128 queries)
// ---------------------------------------------------------------------------
// Keys per K / V tile of the dQ kernel: 128 at d = 64, 32 at d = 128 and 256.
// (64 keys at d = 128 would make Q, dO and dQ^T plus one tile's S^T / dP^T
// overflow the 256 registers of two wavefronts per SIMD; measured on MI355X,
// 32-key tiles run the d = 128 dQ pass 18% faster.)
template <int D> struct DqTile { static constexpr int BN = D == 64 ? 128 : 32; };

template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool WIDE = false>
__global__ void __launch_bounds__((BwdBounds<D, DqWG<D, CAUSAL, SPARSE, WIDE>::WAVES>::THREADS),
                                  (BwdBounds<D, DqWG<D, CAUSAL, SPARSE, WIDE>::WAVES>::MIN_WG))
attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int W = DqWG<D, CAUSAL, SPARSE, WIDE>::WAVES;
  constexpr int DQ_BM = 32 * W;  // queries per workgroup
  constexpr int BN = DqTile<D>::BN;  // keys per tile
  constexpr int TILE = BN * D;
  constexpr int NKK = D / 16;
  constexpr int NSB = BN / 32;   // 32-key sub-blocks per tile
  constexpr int NDB = D / 32;
  constexpr int NKS = BN / 16;   // k-steps over keys in dQ^T += K^T dS^T
  constexpr int TPB = SPARSE_BLOCK / BN;  // key tiles per block of the mask
  static_assert(!SPARSE || DQ_BM == SPARSE_BLOCK, "one workgroup per row of the block mask");

  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[TILE];
  // block-sparse: the key blocks this row block computes, in increasing order
  __shared__ uint16_t blist[SPARSE ? SPARSE_MAX_NB : 1];
  __shared__ int bcount;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // ---- which (batch, head, row block) this workgroup owns; heaviest first ----
  const int nblk = (a.N + DQ_BM - 1) / DQ_BM;
  const int bid = grid_x(a.lt.reverse);
  int bh, rb;
  if constexpr (CAUSAL && !SPARSE) {
    // weight-major, consecutive work items on consecutive XCDs (as in the
    // causal forward pass)
    const int BH = a.Hq * a.B;
    const int r = bid / BH;
    const int i = bid - r * BH;
    bh = (BH & 7) == 0 ? (i & 7) * (BH >> 3) + (i >> 3) : i;  // contiguous heads per XCD
    rb = nblk - 1 - r;
  } else {
    const int L = xcd_remap(bid, nblk * a.Hq * a.B);
    bh = L / nblk;
    rb = nblk - 1 - (L - bh * nblk);
  }
  const int b = bh / a.Hq;
  const int h = bh - b * a.Hq;
  const int g = h / a.group;

  const int q_row = a.Hq * D;
  const int kv_row = a.Hkv * D;
  const int row0 = rb * DQ_BM;
  const int wrow0 = row0 + wave * 32;
  const int qrow = wrow0 + l32;
  const int qsafe = min(qrow, a.N - 1);

  // ---- block-sparse: list the allowed key blocks of row block rb ----
  int nlist = 0;
  if constexpr (SPARSE) {
    if (wave == 0) {
      const uint8_t* mrow = a.sp.bmask + (size_t)g * a.sp.mask_hstride + (size_t)rb * a.sp.nb;
      const int cnt = compact_mask(mrow, 1, 0, CAUSAL ? rb + 1 : a.sp.nb, blist, lane);
      if (lane == 0) bcount = cnt;
    }
    __syncthreads();
    nlist = __builtin_amdgcn_readfirstlane(bcount);
    if (nlist == 0) {  // no allowed key in any row of the block: dQ = 0
      if (qrow < a.N) {
        uint16_t* dqr = (uint16_t*)a.dq + (((size_t)b * a.N + qrow) * a.Hq + h) * D;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) *(u32x4_t*)(dqr + 16 * i + 8 * half) = (u32x4_t){0u, 0u, 0u, 0u};
      }
      return;
    }
  }
  // key tile of loop step j: j itself, or (block-sparse) tile j % TPB of the
  // (j / TPB)-th listed block
  auto ktile = [&](int j) __attribute__((always_inline)) {
    if constexpr (SPARSE) return lds_uniform(blist, j / TPB) * TPB + j % TPB;
    else return j;
  };

  // Q and dO as B operands (lane = query, 8 consecutive d per k-step)
  frag8_t qf[NKK], of[NKK];
  {
    const size_t ro = ((size_t)b * a.N + qsafe) * a.Hq + h;
    const uint16_t* qr = (const uint16_t*)a.q + ro * D + 8 * half;
    const uint16_t* orr = (const uint16_t*)a.dout + ro * D + 8 * half;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      qf[kk] = *(const frag8_t*)(qr + 16 * kk);
      of[kk] = *(const frag8_t*)(orr + 16 * kk);
    }
  }
  const size_t li = ((size_t)b * a.Hq + h) * a.N + qsafe;
  const float lse2 = a.lse[li] * 1.4426950408889634f;
  // dP^T starts from -D (the same for every key of this lane's query), so
  // the products leave dP - D; the first product reads it and writes other
  // registers, so it is never copied
  const float nd = -a.delta[li];
  const f32x16_t negd = {nd, nd, nd, nd, nd, nd, nd, nd, nd, nd, nd, nd, nd, nd, nd, nd};
  const float c = a.scale_log2;  // scale * log2(e), signed

  const uint16_t* kbase = (const uint16_t*)a.k + ((size_t)b * a.Nk * a.Hkv + g) * D;
  const uint16_t* vbase = (const uint16_t*)a.v + ((size_t)b * a.Nk * a.Hkv + g) * D;
  TileDma<D, BN, W, true> dma;
  dma.init(kv_row, wave, lane);
  FragRd<D> fr;
  fr.init(lane);

  // (causal: query i sees keys j <= i + coff)
  const int ntiles_all = (a.Nk + BN - 1) / BN;
  int ntiles = ntiles_all, nwave = ntiles_all, nfull = a.Nk / BN;
  if (CAUSAL) {
    ntiles = max(0, min(ntiles_all, floor_div(min(row0 + DQ_BM, a.N) - 1 + a.coff, BN) + 1));
    nwave = max(0, min(ntiles, floor_div(wrow0 + 31 + a.coff, BN) + 1));
    nfull = max(0, min(min(nfull, ntiles), floor_div(wrow0 + 1 + a.coff, BN)));
    if (ntiles == 0) {  // an offset can leave every row of the block without a key: dQ = 0
      if (qrow < a.N) {
        uint16_t* dqr = (uint16_t*)a.dq + (((size_t)b * a.N + qrow) * a.Hq + h) * D;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) *(u32x4_t*)(dqr + 16 * i + 8 * half) = (u32x4_t){0u, 0u, 0u, 0u};
      }
      return;
    }
  }
  if constexpr (SPARSE) {
    // bounds on the key tile index -> counts of loop steps (every listed
    // block but the last lies wholly below each bound)
    const int last = lds_uniform(blist, nlist - 1);
    auto steps_below = [&](int bound) { return (nlist - 1) * TPB + min(max(bound - last * TPB, 0), TPB); };
    ntiles = steps_below(ntiles);
    nwave = steps_below(nwave);
    nfull = steps_below(nfull);
  }

  f32x16_t dq_acc[NDB];  // dQ^T: lane = query, rows = d
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq_acc[i] = (f32x16_t){};

  auto load = [&](int j, uint16_t* ks, uint16_t* vs) {
    const int kt = ktile(j);
    const size_t off = (size_t)kt * BN * kv_row;
    dma.load(kbase + off, a.Nk - kt * BN, kv_row, ks);
    dma.load(vbase + off, a.Nk - kt * BN, kv_row, vs);
  };

  // Several 32-key sub-blocks per tile (d = 64): software-pipelined, the
  // S^T / dP^T products of sub-block sb + 1 issuing while the dS of sub-block
  // sb forms, then sub-block sb's dQ products.
  auto tile_pipe = [&](int j, const uint16_t* ks, const uint16_t* vs, auto mask_tag)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int key0 = MASK ? ktile(j) * BN : 0;
    int lim = 0;
    if (MASK) {
      lim = a.Nk - 1 - key0 - 4 * half;
      if (CAUSAL) lim = min(lim, qrow + a.coff - key0 - 4 * half);
    }
    f32x16_t sx[2], dpx[2];
    // S^T, dP^T - D of sub-block sb into s, dp; hook(kk) after k-step kk
    auto prod_a = [&](auto sbc, f32x16_t& s, f32x16_t& dp, auto&& hook) __attribute__((always_inline)) {
      constexpr int sb = decltype(sbc)::value;
      s = (f32x16_t){};
      dp = negd;
      frag8_t ka[2], va[2];
      ka[0] = fr.row(ks, sb, 0);
      va[0] = fr.row(vs, sb, 0);
      static_for<0, NKK>([&](auto kkc) __attribute__((always_inline)) {
        constexpr int kk = decltype(kkc)::value;
        if constexpr (kk + 1 < NKK) {
          ka[(kk + 1) & 1] = fr.row(ks, sb, kk + 1);
          va[(kk + 1) & 1] = fr.row(vs, sb, kk + 1);
        }
        s = mfma32(Tag{}, ka[kk & 1], qf[kk], s);
        dp = mfma32(Tag{}, va[kk & 1], of[kk], dp);
        hook(kkc);
      });
    };
    // dS pair t (elements r = 8 (t / 4) + 2 (t % 4), r + 1) of sub-block sb
    auto ds_pair = [&](auto sbc, const f32x16_t& s, const f32x16_t& dp, int t, uint32_t* w)
        __attribute__((always_inline)) {
      constexpr int sb = decltype(sbc)::value;
      const int r = 8 * (t >> 2) + 2 * (t & 3);
      float p0 = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
      float p1 = fast_exp2(__builtin_fmaf(s[r + 1], c, -lse2));
      if (MASK) {
        p0 = (32 * sb + 8 * (r >> 2) + (r & 3)) <= lim ? p0 : 0.f;
        p1 = (32 * sb + 8 * ((r + 1) >> 2) + ((r + 1) & 3)) <= lim ? p1 : 0.f;
      }
      w[t] = pack2(Tag{}, p0 * dp[r], p1 * dp[r + 1]);
      asm volatile("" : "+v"(w[t]));  // formed here, under the products
    };
    auto prod_c = [&](auto sbc, const frag8_t* dsf) __attribute__((always_inline)) {
      constexpr int sb = decltype(sbc)::value;
      constexpr int NF = 2 * NDB;
      constexpr int PFT = 2;
      frag8_t ta[PFT + 1];
#pragma unroll
      for (int f = 0; f < PFT; ++f) ta[f] = fr.tr(ks, 2 * sb + f / NDB, f % NDB);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + PFT < NF) ta[(f + PFT) % (PFT + 1)] = fr.tr(ks, 2 * sb + (f + PFT) / NDB, (f + PFT) % NDB);
        dq_acc[f % NDB] = mfma32(Tag{}, ta[f % (PFT + 1)], dsf[f / NDB], dq_acc[f % NDB]);
      }
    };
    prod_a(std::integral_constant<int, 0>{}, sx[0], dpx[0], [](auto) {});
    static_for<0, NSB>([&](auto sbc) __attribute__((always_inline)) {
      constexpr int sb = decltype(sbc)::value;
      uint32_t w[8];
      if constexpr (sb + 1 < NSB) {
        constexpr int PER = 8 / NKK;  // dS pairs per k-step of the next products
        prod_a(std::integral_constant<int, sb + 1>{}, sx[(sb + 1) & 1], dpx[(sb + 1) & 1],
               [&](auto kkc) __attribute__((always_inline)) {
                 constexpr int kk = decltype(kkc)::value;
#pragma unroll
                 for (int t = PER * kk; t < PER * (kk + 1); ++t) ds_pair(sbc, sx[sb & 1], dpx[sb & 1], t, w);
               });
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) ds_pair(sbc, sx[sb & 1], dpx[sb & 1], t, w);
      }
      const frag8_t dsf[2] = {__builtin_bit_cast(frag8_t, (u32x4_t){w[0], w[1], w[2], w[3]}),
                              __builtin_bit_cast(frag8_t, (u32x4_t){w[4], w[5], w[6], w[7]})};
      prod_c(sbc, dsf);
    });
  };

  auto tile = [&](int j, const uint16_t* ks, const uint16_t* vs, auto mask_tag)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // Per 32-key sub-block: S^T = K Q^T and dP^T - D = V dO^T - D for this
    // wavefront's 32 queries, then dS^T = P^T (dP^T - D) with
    // P^T = 2^(S^T c - LSE2); rows = keys 32 sb + 8 (r / 4) + 4 half + r % 4.
    const int key0 = MASK ? ktile(j) * BN : 0;
    int lim = 0;
    if (MASK) {
      lim = a.Nk - 1 - key0 - 4 * half;
      if (CAUSAL) lim = min(lim, qrow + a.coff - key0 - 4 * half);
    }
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      frag8_t dsf[2];
      f32x16_t s = {}, dp = negd;
      {  // K and V fragments of k-step kk + 1 are read while k-step kk's products run
        frag8_t ka[2], va[2];
        ka[0] = fr.row(ks, sb, 0);
        va[0] = fr.row(vs, sb, 0);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          if (kk + 1 < NKK) {
            ka[(kk + 1) & 1] = fr.row(ks, sb, kk + 1);
            va[(kk + 1) & 1] = fr.row(vs, sb, kk + 1);
          }
          s = mfma32(Tag{}, ka[kk & 1], qf[kk], s);
          dp = mfma32(Tag{}, va[kk & 1], of[kk], dp);
          if (kk + 1 < NKK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                    // MFMA
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 8 * hh + 2 * t;
          float p0 = fast_exp2(__builtin_fmaf(s[r], c, -lse2));
          float p1 = fast_exp2(__builtin_fmaf(s[r + 1], c, -lse2));
          if (MASK) {
            p0 = (32 * sb + 8 * (r >> 2) + (r & 3)) <= lim ? p0 : 0.f;
            p1 = (32 * sb + 8 * ((r + 1) >> 2) + ((r + 1) & 3)) <= lim ? p1 : 0.f;
          }
          w[t] = pack2(Tag{}, p0 * dp[r], p1 * dp[r + 1]);
        }
        const u32x4_t wv = {w[0], w[1], w[2], w[3]};
        dsf[hh] = __builtin_bit_cast(frag8_t, wv);
      }
      // dQ^T += K^T dS^T over the sub-block's 32 keys: A operand K^T via
      // transposed reads of the K tile, two products ahead
      {
        constexpr int NF = 2 * NDB;
        constexpr int PFT = 2;
        frag8_t ta[PFT + 1];
#pragma unroll
        for (int f = 0; f < PFT; ++f) ta[f] = fr.tr(ks, 2 * sb + f / NDB, f % NDB);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (f + PFT < NF) ta[(f + PFT) % (PFT + 1)] = fr.tr(ks, 2 * sb + (f + PFT) / NDB, (f + PFT) % NDB);
          dq_acc[f % NDB] = mfma32(Tag{}, ta[f % (PFT + 1)], dsf[f / NDB], dq_acc[f % NDB]);
          if (f + PFT < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    // MFMA
        }
      }
    }
  };

  load(0, k0s, v0s);
  wait_loads();
  barrier_lds();
  auto step = [&](int j, int buf, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    fr.pin();
    if (j + 1 < ntiles) {
      if (buf) load(j + 1, k0s, v0s);
      else load(j + 1, k1s, v1s);
    }
    if (!MASK || j < nwave) {
      if constexpr (NSB > 1) {
        if (buf) tile_pipe(j, k1s, v1s, mask_tag);
        else tile_pipe(j, k0s, v0s, mask_tag);
      } else {
        if (buf) tile(j, k1s, v1s, mask_tag);
        else tile(j, k0s, v0s, mask_tag);
      }
    }
    wait_loads();
    barrier_lds();
  };
  // one barrier per tile for every wavefront; steady state in pairs so both
  // buffers are compile-time objects
  int j = 0;
  for (; j + 1 < nfull; j += 2) {
    step(j, 0, std::false_type{});
    step(j + 1, 1, std::false_type{});
  }
  if (j < nfull) {
    step(j, 0, std::false_type{});
    ++j;
  }
  for (; j < ntiles; ++j) step(j, j & 1, std::true_type{});

  // ---- epilogue: dQ = scale * dQ^T acc; lane = query, rows = d ----
  if (qrow < a.N) {
    uint16_t* dqr = (uint16_t*)a.dq + (((size_t)b * a.N + qrow) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * half;
        const u32x2_t w = {pack2(Tag{}, dq_acc[db][4 * q4] * a.scale, dq_acc[db][4 * q4 + 1] * a.scale),
                           pack2(Tag{}, dq_acc[db][4 * q4 + 2] * a.scale, dq_acc[db][4 * q4 + 3] * a.scale)};
        *(u32x2_t*)(dqr + d0) = w;
      }
  }
}

}  // namespace

// dK = scale * sum of the head splits' partials, dV = sum, in split order
// (deterministic); four elements per thread of the [B, Nk, Hkv, d] outputs.
template <typename Tag, int D>
__global__ void __launch_bounds__(256) attn_bwd_dkv_reduce_kernel(BwdArgs a) {
  const size_t per = (size_t)a.B * a.Nk * a.Hkv * D;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= per) return;
  f32x4_t sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.hsplit; ++s) {
    const float* p = a.dkv_part + (size_t)s * 2 * per + i;
    sk += *(const f32x4_t*)p;
    sv += *(const f32x4_t*)(p + per);
  }
  *(u32x2_t*)((uint16_t*)a.dk + i) = (u32x2_t){pack2(Tag{}, sk[0] * a.scale, sk[1] * a.scale),
                                               pack2(Tag{}, sk[2] * a.scale, sk[3] * a.scale)};
  *(u32x2_t*)((uint16_t*)a.dv + i) = (u32x2_t){pack2(Tag{}, sv[0], sv[1]), pack2(Tag{}, sv[2], sv[3])};
}

template <typename Tag, int D, bool CAUSAL, bool SPARSE, bool WIDE>
hipError_t launch_dq(const BwdArgs& a, hipStream_t stream) {
  constexpr int W = DqWG<D, CAUSAL, SPARSE, WIDE>::WAVES;
  const long long grid = (long long)((a.N + 32 * W - 1) / (32 * W)) * a.Hq * a.B;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const void* kfn = reinterpret_cast<const void*>(&attn_bwd_dq_kernel<Tag, D, CAUSAL, SPARSE, WIDE>);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<Tag, D, CAUSAL, SPARSE, WIDE>), dim3((unsigned)grid), dim3(64 * W),
                     one_wg_lds_pad(kfn, a.lt.one_wg_per_cu), stream, a);
  return hipGetLastError();
}

// Dense causal dK/dV over short key sequences (at most PAIRED_MAX_BLOCKS blocks
// of 128 keys) at d = 128: key blocks of complementary weight share a
// workgroup (+3-16% on the backward at 512-2048 keys; at d = 64 the paired
// kernel needs more registers than three wavefronts per SIMD allow and was
// 3-8% slower).
constexpr int PAIRED_MAX_BLOCKS = 16;

template <typename Tag, int D, bool CAUSAL, bool SPARSE>
hipError_t launch_bwd_t(const BwdArgs& a, int stages, hipStream_t stream) {
  if (SPARSE && (a.sp.bmask == nullptr || a.sp.nb != (a.N + SPARSE_BLOCK - 1) / SPARSE_BLOCK ||
                 a.sp.nb > SPARSE_MAX_NB || a.Nk != a.N || a.coff != 0))
    return hipErrorInvalidValue;
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
    constexpr int W = DkdvWG<D, CAUSAL>::WAVES;
    if (a.hsplit < 1 || a.group % a.hsplit != 0 ||
        (a.hsplit > 1 && (SPARSE || D > 128 || a.dkv_part == nullptr)))
      return hipErrorInvalidValue;
    const long long nkb = (a.Nk + 32 * W - 1) / (32 * W);
    const long long grid = nkb * a.Hkv * a.B * a.hsplit;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    bool paired = false;
    if constexpr (CAUSAL && !SPARSE && D == 128) {
      if (nkb <= PAIRED_MAX_BLOCKS) {
        paired = true;
        const void* kfn = reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<Tag, D, true, false, true>);
        hipLaunchKernelGGL((attn_bwd_dkdv_kernel<Tag, D, true, false, true>),
                           dim3((unsigned)((nkb + 1) / 2 * a.Hkv * a.B * a.hsplit)), dim3(64 * W),
                           one_wg_lds_pad(kfn, a.lt.one_wg_per_cu), stream, a);
      }
    }
    if (!paired) {
      const void* kfn = reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<Tag, D, CAUSAL, SPARSE>);
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<Tag, D, CAUSAL, SPARSE>), dim3((unsigned)grid), dim3(64 * W),
                         one_wg_lds_pad(kfn, a.lt.one_wg_per_cu), stream, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.hsplit > 1) {
      const long long n4 = ((long long)a.B * a.Nk * a.Hkv * D) / 4;
      const long long rg = (n4 + 255) / 256;
      if (rg > 0x7fffffffLL) return hipErrorInvalidConfiguration;
      hipLaunchKernelGGL((attn_bwd_dkv_reduce_kernel<Tag, D>), dim3((unsigned)rg), dim3(256), 0, stream, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (stages & 4) {
    if constexpr (CAUSAL && !SPARSE && D == 128) {
      if (a.N >= DQ_WIDE_ROWS) return launch_dq<Tag, D, CAUSAL, SPARSE, true>(a, stream);
    }
    return launch_dq<Tag, D, CAUSAL, SPARSE, false>(a, stream);
  }
  return hipSuccess;
}

hipError_t launch_bwd(const BwdArgs& a, bool bf16, int d, bool causal, int stages,
                      hipStream_t stream) {
#define ATTN_BWD_CASE(TAG, DD)                                                            \
  if (d == DD) {                                                                          \
    if (a.sp.bmask)                                                                       \
      return causal ? launch_bwd_t<TAG, DD, true, true>(a, stages, stream)                \
                    : launch_bwd_t<TAG, DD, false, true>(a, stages, stream);              \
    return causal ? launch_bwd_t<TAG, DD, true, false>(a, stages, stream)                 \
                  : launch_bwd_t<TAG, DD, false, false>(a, stages, stream);               \
  }
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
