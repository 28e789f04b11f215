// C-ABI layer of libattn.so (declared in include/attn.h): argument
// validation, device check, workspace layout and dispatch to the kernels.
// No device memory is allocated here; every launch goes on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "../../include/attn.h"
#include "attn_kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
std::atomic<int> g_arch_ok[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int B, int N, int Hq, int Hkv, int d) {
  if (B < 1 || N < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 256) return ATTN_ERR_HEADDIM;
  // Element offsets inside one (batch, head) slice and the row-block grid stay
  // in int range.  Each product is formed only once its factors are known to
  // keep it below 2^63 (all sizes are positive ints here).
  const long long nh = (long long)N * Hq;   // < 2^62
  if (nh >= (1LL << 31) / d) return ATTN_ERR_TOO_LARGE;  // N * Hq * d >= 2^31 (d divides 2^31)
  const long long bh = (long long)B * Hq;   // < 2^62
  if (bh >= (1LL << 31) || bh * ((N - 1) / 128 + 1) >= (1LL << 31)) return ATTN_ERR_TOO_LARGE;
  return ATTN_OK;
}

int check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    int known = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (known == 1) return ATTN_OK;
    if (known == 2) return ATTN_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? ATTN_OK : ATTN_ERR_DEVICE;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ATTN_DEBUG=1 in the environment (read once per process): every call waits
// for its stream and reports an execution error of its kernels as
// ATTN_ERR_HIP, instead of leaving it to a later call.  For debugging only:
// it serialises the caller's stream.
bool debug_sync() {
  static const bool on = [] {
    const char* v = std::getenv("ATTN_DEBUG");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

// ATTN_LAUNCH_TEST in the environment, read on every call (a testing aid
// for the race checks): "reverse" runs each kernel's workgroups in reversed
// work-item order, "one_wg_per_cu" pads their LDS so that each CU holds one
// workgroup at a time.  Results must not change.
attn::LaunchTest launch_test() {
  attn::LaunchTest lt = {0, 0};
  const char* v = std::getenv("ATTN_LAUNCH_TEST");
  if (v != nullptr) {
    lt.reverse = std::strcmp(v, "reverse") == 0;
    lt.one_wg_per_cu = std::strcmp(v, "one_wg_per_cu") == 0;
  }
  return lt;
}

// Result of a call's launches: a launch error, or under ATTN_DEBUG an
// execution error found by synchronising the stream.
int finish(hipError_t e, void* stream) {
  if (e == hipSuccess && debug_sync()) {
    e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

// Block-mask arguments of the block-sparse entry points.
int check_mask(const unsigned char* block_mask, int mask_heads, int N, int Hkv, attn::SparseArgs* sp) {
  if (!block_mask) return ATTN_ERR_NULLPTR;
  if (mask_heads != 1 && mask_heads != Hkv) return ATTN_ERR_SHAPE;
  if (N > ATTN_SPARSE_MAX_N) return ATTN_ERR_TOO_LARGE;
  static_assert(ATTN_SPARSE_BLOCK == attn::SPARSE_BLOCK &&
                    ATTN_SPARSE_MAX_N == attn::SPARSE_BLOCK * attn::SPARSE_MAX_NB,
                "header constants match the kernels");
  sp->bmask = reinterpret_cast<const uint8_t*>(block_mask);
  sp->nb = (N + ATTN_SPARSE_BLOCK - 1) / ATTN_SPARSE_BLOCK;
  sp->mask_hstride = mask_heads == 1 ? 0 : sp->nb * sp->nb;
  return ATTN_OK;
}

const attn::SparseArgs kDense = {nullptr, 0, 0};

}  // namespace

namespace attn {

int bwd_head_split(int B, int Nk, int Hkv, int group, int d) {
  const long long base = (long long)((Nk + 127) / 128) * Hkv * B;  // dK/dV workgroups unsplit
  if (group <= 1 || base >= 512 || d > 128) return 1;
  for (int s = 2; s < group; ++s)
    if (group % s == 0 && base * s >= 1024) return s;
  return group;
}

BwdWorkspace bwd_workspace_layout(int B, int N, int Hq, int Hkv, int d, bool with_split) {
  BwdWorkspace w;
  w.delta_off = 0;
  w.delta_bytes = (size_t)B * Hq * N * sizeof(float);
  w.hsplit = with_split ? bwd_head_split(B, N, Hkv, Hq / Hkv, d) : 1;
  w.part_off = align256(w.delta_off + w.delta_bytes);
  w.part_bytes = w.hsplit > 1 ? (size_t)w.hsplit * 2 * B * N * Hkv * d * sizeof(float) : 0;
  w.total = align256(w.part_off + w.part_bytes);
  return w;
}

}  // namespace attn

namespace {

// Causal offsets beyond [-Nq, Nk] mean the same as these bounds (no row, or
// every key, visible); clamping keeps row + offset far from int overflow.
int clamp_offset(long long off, int Nq, int Nk) {
  return (int)(off < -(long long)Nq ? -(long long)Nq : (off > Nk ? Nk : off));
}

int fwd_common(const void* q, const void* k, const void* v, void* o, float* lse,
               const unsigned char* block_mask, int mask_heads, int B, int N, int Nk, int Hq,
               int Hkv, int d, int dtype, int causal, long long causal_offset, float scale,
               void* stream, int splits = 1, void* workspace = nullptr, size_t workspace_bytes = 0) {
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULLPTR;
  int st = check_shape(B, N, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  st = check_shape(B, Nk, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return ATTN_ERR_ALIGN;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  attn::SparseArgs sp = kDense;
  if (block_mask || mask_heads) {
    st = check_mask(block_mask, mask_heads, N, Hkv, &sp);
    if (st != ATTN_OK) return st;
  }
  st = check_device();
  if (st != ATTN_OK) return st;

  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.neg_scale = scale < 0.f ? 1 : 0;
  a.scale_log2 = std::fabs(scale) * 1.4426950408889634f;
  a.sp = sp;
  a.Nk = Nk;
  a.coff = clamp_offset(causal_offset, N, Nk);
  a.lt = launch_test();
  a.splits = 1;
  a.split_len = 0;
  a.opart = nullptr;
  a.lsepart = nullptr;
  if (workspace) {  // split-KV: keys in `splits` runs of a multiple of 128
    const attn::SplitWorkspace w = attn::split_workspace_layout(B, N, Hq, d, splits);
    const int per = (Nk + splits - 1) / splits;
    a.splits = splits;
    a.split_len = (per + 127) / 128 * 128;
    a.opart = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.opart_off);
    a.lsepart = reinterpret_cast<float*>(static_cast<char*>(workspace) + w.lsepart_off);
  }
  return finish(attn::launch_fwd(a, dtype == ATTN_DTYPE_BF16, d, causal != 0, static_cast<hipStream_t>(stream)),
                stream);
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int N,
             int Hq, int Hkv, int d, int dtype, int causal, float scale, void* stream) {
  return fwd_common(q, k, v, o, lse, nullptr, 0, B, N, N, Hq, Hkv, d, dtype, causal, 0, scale, stream);
}

int attn_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Nq,
                  int Nk, int Hq, int Hkv, int d, int dtype, int causal, long long causal_offset,
                  float scale, void* stream) {
  return fwd_common(q, k, v, o, lse, nullptr, 0, B, Nq, Nk, Hq, Hkv, d, dtype, causal, causal_offset,
                    scale, stream);
}

size_t attn_fwd_splitkv_workspace_bytes(int B, int Nq, int Hq, int d, int num_splits) {
  if (check_shape(B, Nq, Hq, 1, d) != ATTN_OK || num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return 0;
  return attn::split_workspace_layout(B, Nq, Hq, d, num_splits).total;
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                     size_t workspace_bytes, int B, int Nq, int Nk, int Hq, int Hkv, int d, int dtype,
                     int causal, long long causal_offset, float scale, int num_splits, void* stream) {
  if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS) return ATTN_ERR_SHAPE;
  const size_t need = attn_fwd_splitkv_workspace_bytes(B, Nq, Hq, d, num_splits);
  if (!workspace || need == 0 || workspace_bytes < need) {
    // shape errors take precedence over a workspace error
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULLPTR;
    int st = check_shape(B, Nq, Hq, Hkv, d);
    if (st == ATTN_OK) st = check_shape(B, Nk, Hq, Hkv, d);
    return st != ATTN_OK ? st : ATTN_ERR_WORKSPACE;
  }
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  return fwd_common(q, k, v, o, lse, nullptr, 0, B, Nq, Nk, Hq, Hkv, d, dtype, causal, causal_offset,
                    scale, stream, num_splits, workspace, workspace_bytes);
}

int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                         const unsigned char* block_mask, int mask_heads, int B, int N, int Hq,
                         int Hkv, int d, int dtype, int causal, float scale, void* stream) {
  if (!block_mask) return ATTN_ERR_NULLPTR;
  return fwd_common(q, k, v, o, lse, block_mask, mask_heads, B, N, N, Hq, Hkv, d, dtype, causal, 0,
                    scale, stream);
}

size_t attn_bwd_workspace_bytes(int B, int N, int Hq, int Hkv, int d) {
  if (check_shape(B, N, Hq, Hkv, d) != ATTN_OK) return 0;
  return attn::bwd_workspace_layout(B, N, Hq, Hkv, d).total;
}

}  // extern "C"

namespace {

int bwd_common(int stages, const unsigned char* block_mask, int mask_heads, int Nk,
               long long causal_offset, const void* q, const void* k, const void* v, const void* o,
               const void* dout, const float* lse, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype, int causal,
               float scale, void* stream, bool allow_split = true) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULLPTR;
  int st = check_shape(B, N, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  st = check_shape(B, Nk, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return ATTN_ERR_ALIGN;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  // the dK/dV head split serves the square dense pass only
  const bool split_ok = allow_split && block_mask == nullptr && mask_heads == 0 && Nk == N;
  const attn::BwdWorkspace ws = attn::bwd_workspace_layout(B, N, Hq, Hkv, d, split_ok);
  if (!workspace || workspace_bytes < ws.total) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  attn::SparseArgs sp = kDense;
  if (block_mask || mask_heads) {
    st = check_mask(block_mask, mask_heads, N, Hkv, &sp);
    if (st != ATTN_OK) return st;
  }
  st = check_device();
  if (st != ATTN_OK) return st;

  attn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.delta_off);
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.group = Hq / Hkv;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.sp = sp;
  a.Nk = Nk;
  a.coff = clamp_offset(causal_offset, N, Nk);
  a.lt = launch_test();
  a.hsplit = ws.hsplit;
  a.dkv_part = ws.hsplit > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + ws.part_off) : nullptr;
  return finish(attn::launch_bwd(a, dtype == ATTN_DTYPE_BF16, d, causal != 0, stages,
                                 static_cast<hipStream_t>(stream)),
                stream);
}

}  // namespace

extern "C" {

#define ATTN_BWD_ARGS                                                                       \
  const void *q, const void *k, const void *v, const void *o, const void *dout,             \
      const float *lse, void *dq, void *dk, void *dv, void *workspace,                      \
      size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype, int causal,  \
      float scale, void *stream
#define ATTN_BWD_PASS                                                                       \
  q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, N, Hq, Hkv, d, dtype,   \
      causal, scale, stream

int attn_bwd(ATTN_BWD_ARGS) { return bwd_common(7, nullptr, 0, N, 0, ATTN_BWD_PASS); }
int attn_bwd_preprocess(ATTN_BWD_ARGS) { return bwd_common(1, nullptr, 0, N, 0, ATTN_BWD_PASS); }
int attn_bwd_dkdv(ATTN_BWD_ARGS) { return bwd_common(2, nullptr, 0, N, 0, ATTN_BWD_PASS); }
int attn_bwd_dq(ATTN_BWD_ARGS) { return bwd_common(4, nullptr, 0, N, 0, ATTN_BWD_PASS); }

int attn_bwd_rect(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, int B, int Nq, int Nk, int Hq, int Hkv, int d, int dtype,
                  int causal, long long causal_offset, float scale, void* stream) {
  return bwd_common(7, nullptr, 0, Nk, causal_offset, q, k, v, o, dout, lse, dq, dk, dv, workspace,
                    workspace_bytes, B, Nq, Hq, Hkv, d, dtype, causal, scale, stream);
}

int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, const unsigned char* block_mask,
                         int mask_heads, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype,
                         int causal, float scale, void* stream) {
  if (!block_mask) return ATTN_ERR_NULLPTR;
  return bwd_common(7, block_mask, mask_heads, N, 0, ATTN_BWD_PASS);
}

#undef ATTN_BWD_ARGS
#undef ATTN_BWD_PASS

}  // extern "C"

// ---- backward with no device allocation: a static scratch array ----

namespace {

constexpr size_t kNoAllocScratch = ATTN_NOALLOC_SCRATCH_BYTES;
// The backward's scratch for callers that cannot allocate: D and, where they
// fit beside it, the fp32 dK/dV partials of a split GQA group.  Each device
// the library runs on holds its own copy until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol); it uses the device address from scratch_address().
static __device__ __align__(256) unsigned char scratch[kNoAllocScratch];

std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, looked up once
// per device (with that device current) and kept.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = (int)e;
    return ATTN_ERR_DEVICE;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        g_last_hip_error = (int)e;
        return ATTN_ERR_HIP;
      }
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                                int N, int Hq, int Hkv, int d, int dtype, int causal, float scale,
                                void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_ERR_NULLPTR;
  int st = check_shape(B, N, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  // the GQA head split only where its partials fit beside D
  const bool split = attn::bwd_workspace_layout(B, N, Hq, Hkv, d, true).total <= kNoAllocScratch;
  if (!split && attn::bwd_workspace_layout(B, N, Hq, Hkv, d, false).total > kNoAllocScratch)
    return ATTN_ERR_SCRATCH;
  st = check_device();
  if (st != ATTN_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != ATTN_OK) return st;
  return bwd_common(7, nullptr, 0, N, 0, q, k, v, o, dout, lse, dq, dk, dv, ws, kNoAllocScratch, B, N, Hq,
                    Hkv, d, dtype, causal, scale, stream, split);
}

// ---- standard (materialising) attention ----

namespace attn {

StdWorkspace std_workspace_layout(int B, int N, int Hq) {
  StdWorkspace w;
  w.ldn = (N + 63) / 64 * 64;
  const size_t elems = (size_t)B * Hq * N * w.ldn;
  w.s_off = 0;
  w.p_off = align256(w.s_off + elems * sizeof(float));
  w.ds_off = align256(w.p_off + elems * sizeof(uint16_t));
  w.total = align256(w.ds_off + elems * sizeof(uint16_t));
  return w;
}

}  // namespace attn

namespace {

// Launch limits of the standard path: one row workgroup per (batch, head,
// query row) in grid x, one (batch, head) per grid z of the tile products.
int check_std_grid(int B, int N, int Hq) {
  const long long bh = (long long)B * Hq;  // < 2^62; then bh * N < 2^24 * 2^31
  if (bh > 65535 || bh * N >= (1LL << 24)) return ATTN_ERR_TOO_LARGE;
  return ATTN_OK;
}

int std_common(bool fwd, const void* q, const void* k, const void* v, const void* dout, void* o,
               float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
               int N, int Hq, int Hkv, int d, int dtype, int causal, float scale, void* stream) {
  if (!q || !k || !v) return ATTN_ERR_NULLPTR;
  if (fwd ? (!o || !lse) : (!dout || !dq || !dk || !dv)) return ATTN_ERR_NULLPTR;
  int st = check_shape(B, N, Hq, Hkv, d);
  if (st != ATTN_OK) return st;
  st = check_std_grid(B, N, Hq);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_DTYPE_FP16 && dtype != ATTN_DTYPE_BF16) return ATTN_ERR_DTYPE;
  const void* ptrs[] = {q, k, v, fwd ? (const void*)o : dout, fwd ? (const void*)lse : dq,
                        fwd ? nullptr : dk, fwd ? nullptr : dv};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return ATTN_ERR_ALIGN;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  const attn::StdWorkspace ws = attn::std_workspace_layout(B, N, Hq);
  if (!workspace || workspace_bytes < ws.total) return ATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
  st = check_device();
  if (st != ATTN_OK) return st;

  attn::StdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.o = o;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.lse = lse;
  char* w = static_cast<char*>(workspace);
  a.s = reinterpret_cast<float*>(w + ws.s_off);
  a.p = reinterpret_cast<uint16_t*>(w + ws.p_off);
  a.ds = reinterpret_cast<uint16_t*>(w + ws.ds_off);
  a.B = B;
  a.N = N;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.d = d;
  a.ldn = ws.ldn;
  a.causal = causal != 0;
  a.scale = scale;
  const bool bf16 = dtype == ATTN_DTYPE_BF16;
  return finish(fwd ? attn::launch_std_fwd(a, bf16, static_cast<hipStream_t>(stream))
                    : attn::launch_std_bwd(a, bf16, static_cast<hipStream_t>(stream)),
                stream);
}

}  // namespace

extern "C" {

size_t attn_standard_workspace_bytes(int B, int N, int Hq, int Hkv, int d) {
  if (check_shape(B, N, Hq, Hkv, d) != ATTN_OK || check_std_grid(B, N, Hq) != ATTN_OK) return 0;
  return attn::std_workspace_layout(B, N, Hq).total;
}

int attn_fwd_standard(const void* q, const void* k, const void* v, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype, int causal,
                      float scale, void* stream) {
  return std_common(true, q, k, v, nullptr, o, lse, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                    B, N, Hq, Hkv, d, dtype, causal, scale, stream);
}

int attn_bwd_standard(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, int B, int N, int Hq, int Hkv,
                      int d, int dtype, int causal, float scale, void* stream) {
  return std_common(false, q, k, v, dout, nullptr, nullptr, dq, dk, dv, workspace, workspace_bytes, B, N,
                    Hq, Hkv, d, dtype, causal, scale, stream);
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULLPTR: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (B, N, Hq, Hkv must be >= 1 and Hq a multiple of Hkv)";
    case ATTN_ERR_HEADDIM: return "unsupported head dimension (expected 64, 128 or 256)";
    case ATTN_ERR_DTYPE: return "unsupported dtype (expected ATTN_DTYPE_FP16 or ATTN_DTYPE_BF16)";
    case ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_WORKSPACE: return "workspace is NULL or too small";
    case ATTN_ERR_DEVICE: return "no current HIP device, or it is not gfx950";
    case ATTN_ERR_HIP: return "a HIP launch failed";
    case ATTN_ERR_TOO_LARGE: return "sizes exceed the supported index range";
    case ATTN_ERR_SCRATCH:
      return "sizes need more device scratch than attn_bwd_noalloc holds (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

const char* attn_version(void) { return "libattn 0.1.0 (gfx950)"; }

}  // extern "C"
