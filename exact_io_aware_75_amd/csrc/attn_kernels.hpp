// Internal interface between the C-ABI host layer (attn_api.cpp) and the HIP
// kernels.  Argument structs are passed by value to the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Block-sparse attention: the mask has one entry per (query block, key block)
// pair of SPARSE_BLOCK x SPARSE_BLOCK; the kernels keep the allowed blocks of
// one row (or column) of the mask as a list in LDS, so nb <= SPARSE_MAX_NB.
constexpr int SPARSE_BLOCK = 128;
constexpr int SPARSE_MAX_NB = 2048;

// Optional block mask shared by the forward and backward argument structs.
struct SparseArgs {
  const uint8_t* bmask;  // null: dense; else uint8 [mask heads][nb][nb], nonzero = computed
  int nb;                // ceil(N / SPARSE_BLOCK)
  int mask_hstride;      // entries between the masks of consecutive K/V heads (0: one mask)
};

// Launch-order test modes (the race checks): the kernels' results must not
// depend on the order or the concurrency in which workgroups run.
struct LaunchTest {
  int reverse;        // 1: workgroup x takes the work item of gridDim.x - 1 - x
  int one_wg_per_cu;  // 1: dynamic LDS padding keeps every CU to one workgroup
};

struct FwdArgs {
  const void* q;  // [B, N, Hq, d]
  const void* k;  // [B, Nk, Hkv, d]
  const void* v;  // [B, Nk, Hkv, d]
  void* o;        // [B, N, Hq, d]
  float* lse;     // [B, Hq, N]
  int B, N, Hq, Hkv;
  int Nk;            // keys (K/V rows per sequence); N is the number of queries
  int coff;          // causal: query i sees key j iff j <= i + coff (clamped to [-N, Nk])
  // split-KV: workgroup (x, y) covers keys [y split_len, (y + 1) split_len)
  // and writes fp32 partials that a merge kernel combines into o and lse
  int splits;        // 1: no split
  int split_len;     // keys per split, a multiple of 128
  float* opart;      // [splits, B, N, Hq, d] fp32: each split's O, normalised by its own sum
  float* lsepart;    // [splits, B, Hq, N] fp32: each split's natural-log LSE (-inf: no key)
  int group;         // Hq / Hkv
  int neg_scale;     // 1 if scale < 0 (folded into Q's sign)
  float scale_log2;  // |scale| * log2(e)
  SparseArgs sp;
  LaunchTest lt;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;  // [B, Hq, N]
  void* dq;
  void* dk;
  void* dv;
  float* delta;      // workspace: [B, Hq, N] fp32, rowsum(dO * O)
  int B, N, Hq, Hkv;
  int Nk;            // keys; N is the number of queries
  int coff;          // causal offset, as in FwdArgs
  int group;
  float scale;       // signed softmax scale
  float scale_log2;  // scale * log2(e)
  SparseArgs sp;
  // dK/dV pass over small grids: the query heads of each GQA group are split
  // over `hsplit` workgroups per key block, which write fp32 partials
  // [hsplit][2 (dK, dV)][B][Nk][Hkv][d] to dkv_part; a reduce kernel sums them
  // (in split order) into dk, dv.  hsplit = 1: dk, dv written directly.
  int hsplit;
  float* dkv_part;
  LaunchTest lt;
};

// Workspace layout of the backward pass (offsets in bytes, 256-byte aligned).
struct BwdWorkspace {
  size_t delta_off, delta_bytes;
  int hsplit;                   // head split of the dK/dV pass (1: none)
  size_t part_off, part_bytes;  // fp32 dK/dV partials when hsplit > 1
  size_t total;
};
// Head split of the dK/dV pass: 1 unless the pass would have fewer than 512
// workgroups (B * Hkv * ceil(Nk / 128)), a group has several query heads and
// d <= 128; then the smallest divisor of the group that gives >= 1024 (or
// the group).
int bwd_head_split(int B, int Nk, int Hkv, int group, int d);
// with_split = false: the layout without the partials (rectangular and
// block-sparse calls, which run unsplit).
BwdWorkspace bwd_workspace_layout(int B, int N, int Hq, int Hkv, int d, bool with_split = true);

hipError_t launch_fwd(const FwdArgs& a, bool bf16, int d, bool causal, hipStream_t stream);
// Split-KV layout of the forward workspace (offsets in bytes, 256-byte aligned).
struct SplitWorkspace {
  size_t opart_off, lsepart_off, total;
};
SplitWorkspace split_workspace_layout(int B, int N, int Hq, int d, int splits);
// stage_mask: bit 0 = D preprocess, bit 1 = dK/dV kernel, bit 2 = dQ kernel
hipError_t launch_bwd(const BwdArgs& a, bool bf16, int d, bool causal, int stage_mask,
                      hipStream_t stream);

// ---- standard (materialising) attention ----
// One operand of the standard path's tile product (16-bit elements).
struct StdOperand {
  const uint16_t* p;
  long long bstride, hstride;  // elements between batches / heads
  int ld;                      // elements between consecutive stored rows
  int hmul, hdiv;              // head of stage s for output head ho: (ho * hmul + s) / hdiv
  int xext;                    // extent of the operand's own (non-reduction) index
};
struct StdGemmArgs {
  StdOperand a, b;
  void* c;                     // fp32 or 16-bit output
  long long c_bstride, c_hstride;
  int c_ld;
  int M, Nn, K;                // C is M x Nn, reduction length K per stage
  int Hout, nsum;              // output heads; stages summed per output head
  float alpha;
};
struct StdRowArgs {
  float* s;        // S or dP rows, fp32, pitch ldn
  uint16_t* p;     // P rows
  uint16_t* ds;    // dS rows
  float* lse;      // [B, Hq, N]
  int N, ldn, causal;
};
struct StdArgs {
  const void *q, *k, *v, *dout;
  void *o, *dq, *dk, *dv;
  float* lse;
  float* s;        // [B, Hq, N, ldn] fp32: S, later dP
  uint16_t* p;     // [B, Hq, N, ldn]: P
  uint16_t* ds;    // [B, Hq, N, ldn]: dS
  int B, N, Hq, Hkv, d, ldn, causal;
  float scale;
};
// Workspace layout of the standard path (offsets in bytes, 256-byte aligned).
struct StdWorkspace {
  int ldn;
  size_t s_off, p_off, ds_off, total;
};
StdWorkspace std_workspace_layout(int B, int N, int Hq);
hipError_t launch_std_fwd(const StdArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_std_bwd(const StdArgs& a, bool bf16, hipStream_t stream);

}  // namespace attn
