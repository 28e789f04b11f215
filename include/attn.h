/*
 * attn.h -- C ABI of libattn.so: exact, IO-aware tiled attention (forward and
 * backward) for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  Exact scaled-dot-product attention, the same result as
 * standard attention up to rounding (FlashAttention-2 review, "Введение"
 * section: the tiled algorithm is mathematically equivalent to attention up to
 * numerical precision).  For query head h and its K/V head g = h / (Hq/Hkv):
 *
 *     S = scale * Q K^T,   P = softmax(S) row-wise,   O = P V,
 *     LSE[i] = ln sum_j exp(S[i, j])          (natural log, per query row)
 *
 * with keys j > i excluded when `causal` is set.  The N x N matrices S and P
 * never reach device memory: the forward pass streams K/V tiles through LDS
 * and keeps an online softmax in registers (tiling from HBM into on-chip
 * memory: FlashAttention-2 announcement, "具体实现" section; FlashAttention-1
 * news page, "FlashAttention" section).  The backward pass recomputes P tile
 * by tile from Q, K, V and LSE instead of storing it (same sections), and
 * produces dQ, dK, dV of L = sum(O * dO).  MQA/GQA (Hkv < Hq) and head
 * dimensions up to 256 follow the same announcement's "具体实现" section.
 *
 * Tensor layout.  All tensors are dense, row-major, device-resident:
 *     q, o, dout, dq : [B, N, Hq,  d]     (d innermost)
 *     k, v, dk, dv   : [B, N, Hkv, d]
 *     lse            : [B, Hq, N] float32
 * q, k, v, o, dout, dq, dk, dv share one element type (`dtype`).  Every
 * pointer must be 16-byte aligned.  Consecutive query heads share a K/V head
 * (query head h reads K/V head h / (Hq / Hkv)).  Supported head dimensions are
 * d = 64, 128 and 256; any N >= 1 is accepted (partial tiles are masked).
 *
 * Ownership and ordering.  All buffers are owned by the caller.  The library
 * never allocates or frees device memory and keeps no state besides a
 * per-device property cache, a thread-local last-HIP-error code and the
 * static device scratch of attn_bwd_noalloc (a fixed array in the library's
 * code object, present on every device the library runs on).  Work is
 * enqueued on `stream` (a hipStream_t; NULL means the legacy default stream)
 * and calls return without synchronising; the caller keeps every buffer alive
 * until the stream has finished.  Outputs must not alias inputs.  Calls that
 * share a backward workspace must be ordered on one stream.
 *
 * Errors.  Each entry point returns an attn_status_t.  Arguments are
 * validated before anything is launched; on any error nothing is written.
 * A failed launch returns ATTN_ERR_HIP and attn_last_hip_error() gives the
 * hipError_t of the failing call on this thread.  With the environment
 * variable ATTN_DEBUG set (to anything but "" or "0") when the library first
 * checks it, every call also waits for its stream and returns ATTN_ERR_HIP if
 * its kernels failed: a debugging aid that makes calls synchronous.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_DTYPE_FP16 = 0, /* IEEE binary16 */
  ATTN_DTYPE_BF16 = 1  /* bfloat16 */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULLPTR = 1,   /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,     /* B, N, Hq, Hkv < 1, or Hq not a multiple of Hkv */
  ATTN_ERR_HEADDIM = 3,   /* d not in {64, 128, 256} */
  ATTN_ERR_DTYPE = 4,     /* dtype not an attn_dtype_t */
  ATTN_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned */
  ATTN_ERR_SCALE = 6,     /* scale is NaN or infinite */
  ATTN_ERR_WORKSPACE = 7, /* workspace NULL or smaller than attn_bwd_workspace_bytes() */
  ATTN_ERR_DEVICE = 8,    /* no current HIP device, or it is not gfx950 */
  ATTN_ERR_HIP = 9,       /* a HIP launch failed; see attn_last_hip_error() */
  ATTN_ERR_TOO_LARGE = 10, /* a tensor has 2^31 or more elements per (batch, head) slice,
                              or the launch grid would exceed the device limits */
  ATTN_ERR_SCRATCH = 11    /* attn_bwd_noalloc: the sizes need more scratch than its static
                              array holds (ATTN_NOALLOC_SCRATCH_BYTES) */
} attn_status_t;

/*
 * Forward pass.  Writes o = softmax(scale * q k^T [causal mask]) v and the
 * per-row natural-log log-sum-exp `lse` (saved for the backward pass's
 * recomputation).  Accumulation is fp32; o is rounded to nearest-even into
 * `dtype`.
 *
 *   q [B,N,Hq,d], k/v [B,N,Hkv,d]   inputs, dtype
 *   o [B,N,Hq,d]                    output, dtype
 *   lse [B,Hq,N]                    output, float32
 *   causal                          nonzero: query i attends keys j <= i only
 *   scale                           multiplies q k^T (typically 1/sqrt(d)); 0 is legal
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int N, int Hq, int Hkv, int d, int dtype, int causal, float scale,
             void* stream);

/*
 * Bytes of device workspace attn_bwd needs for these sizes: the per-row
 * D = rowsum(dO * O) in float32, B * Hq * N values, plus alignment.  When
 * the dK/dV pass would have few workgroups -- B * Hkv * ceil(N / 128) < 512,
 * Hq > Hkv and d <= 128 (MQA/GQA with a small batch) -- the query heads of
 * each group are split over `s` workgroups per key block (s the smallest
 * divisor of Hq / Hkv with B * Hkv * ceil(N / 128) * s >= 1024, else
 * Hq / Hkv) and the workspace also holds their float32 partial dK and dV,
 * s * 2 * B * N * Hkv * d values, which are summed in a fixed order (the
 * result stays deterministic).  Either way the size is O(N).  Returns 0 if
 * the sizes are invalid.
 */
size_t attn_bwd_workspace_bytes(int B, int N, int Hq, int Hkv, int d);

/*
 * Backward pass.  Given the forward inputs, its outputs o and lse (from an
 * attn_fwd call with the same causal flag and scale) and the upstream gradient
 * dout, writes dq, dk, dv of L = sum(o * dout).  Scores and probabilities are
 * recomputed tile by tile from lse (FlashAttention-1 news page, section
 * "FlashAttention"; FlashAttention-2 announcement, section "具体实现"): dk and
 * dv in a pass parallel over key/value column blocks, dq in a pass parallel
 * over query row blocks.  dk/dv of a K/V head sum the contributions of every
 * query head in its group.  `workspace` (device memory, 16-byte aligned, at
 * least attn_bwd_workspace_bytes() bytes) is scratch: its contents on entry
 * are ignored and on exit undefined.  No atomics are used: results are
 * bitwise deterministic.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype,
             int causal, float scale, void* stream);

/*
 * attn_bwd without a workspace argument and without any device allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments (minus the workspace), result and validation as attn_bwd; its
 * scratch -- D, and the float32 dK/dV partials of a split GQA group when they
 * fit beside it (otherwise the group runs unsplit, the same result up to the
 * order of float32 sums) -- lives in a static device array of
 * ATTN_NOALLOC_SCRATCH_BYTES that every device the library runs on holds
 * until the process ends.  Sizes whose D (4 * B * Hq * N bytes, plus
 * alignment) does not fit return ATTN_ERR_SCRATCH before anything is
 * launched.  No hipMalloc, hipFree or allocating library routine is called
 * (the array's device address is looked up once per device, on the first
 * call there).  All calls on one device share the array and nothing in it
 * needs to start at zero (each call writes every value it reads): calls that
 * overlap on one device -- on different streams or from different threads --
 * race, and must be ordered by the caller.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES 67108864 /* 64 MiB */

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int B, int N, int Hq, int Hkv,
                     int d, int dtype, int causal, float scale, void* stream);

/*
 * The three stages attn_bwd runs, exposed so a caller can schedule or time
 * them separately.  Same arguments and validation as attn_bwd; they must be
 * enqueued in this order on one stream with the same workspace (the last two
 * may also be swapped), and together they are exactly attn_bwd:
 *   attn_bwd_preprocess   D = rowsum(dout * o) per query row into the
 *                         workspace;
 *   attn_bwd_dkdv         recomputation over key/value column blocks: dk and
 *                         dv written;
 *   attn_bwd_dq           recomputation over query row blocks: dq written.
 */
int attn_bwd_preprocess(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        void* workspace, size_t workspace_bytes, int B, int N, int Hq, int Hkv,
                        int d, int dtype, int causal, float scale, void* stream);
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype,
                  int causal, float scale, void* stream);
int attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype,
                int causal, float scale, void* stream);

/*
 * Rectangular attention: Nq queries against Nk keys, the shape one device
 * computes when the sequence is split across devices (the pages parallelise
 * over the sequence: FlashAttention-2 announcement, section "具体实现";
 * FlashAttention-2 review, section "Параллелизм").  q, o, dout, dq are
 * [B, Nq, Hq, d], k, v, dk, dv are [B, Nk, Hkv, d], lse is [B, Hq, Nq]; with
 * `causal` set, query i attends key j only if
 *     j <= i + causal_offset
 * (causal_offset = Nk - Nq aligns the last query with the last key; for a
 * block of keys that starts at position p of the sequence and queries that
 * start at position r, causal_offset = r - p).  Rows with no allowed key get
 * o = 0, lse = -inf and dq = 0.  Partial results over disjoint key blocks
 * combine exactly: lse = ln sum_p exp(lse_p), o = sum_p exp(lse_p - lse) o_p.
 * Everything else is that of attn_fwd / attn_bwd; the backward workspace is
 * attn_bwd_workspace_bytes(B, Nq, Hq, Hkv, d), and attn_fwd_rect(..., Nq = Nk
 * = N, causal_offset = 0) is attn_fwd.  Offsets outside [-Nq, Nk] act as
 * these bounds.
 */
int attn_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Nq, int Nk, int Hq, int Hkv, int d, int dtype, int causal,
                  long long causal_offset, float scale, void* stream);

int attn_bwd_rect(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, int B, int Nq, int Nk, int Hq, int Hkv, int d,
                  int dtype, int causal, long long causal_offset, float scale, void* stream);

/*
 * Split-KV forward: attn_fwd_rect with the keys cut into `num_splits` runs
 * (each a multiple of 128 keys, ceil(Nk / num_splits) rounded up; trailing
 * runs may be empty) that separate workgroups process in parallel, then
 * merged exactly, LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s,
 * from fp32 partials in `workspace`.  For shapes with few query rows per
 * (batch, head) -- short Nq, small B * Hq -- where one workgroup per 128 or
 * 256 query rows leaves most of the GPU idle (the pages parallelise over the
 * sequence for this reason: FlashAttention-2 announcement, section "具体实现").
 * Arguments as attn_fwd_rect, plus:
 *   num_splits       1 .. ATTN_MAX_SPLITS
 *   workspace        device memory, 16-byte aligned, at least
 *                    attn_fwd_splitkv_workspace_bytes(B, Nq, Hq, d,
 *                    num_splits) bytes (fp32 partial O and LSE of every
 *                    split); contents on entry ignored, on exit undefined
 * Calls sharing a workspace must be ordered on one stream.
 */
#define ATTN_MAX_SPLITS 256

size_t attn_fwd_splitkv_workspace_bytes(int B, int Nq, int Hq, int d, int num_splits);

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, int B, int Nq, int Nk, int Hq,
                     int Hkv, int d, int dtype, int causal, long long causal_offset, float scale,
                     int num_splits, void* stream);

/*
 * Block-sparse attention.  The FlashAttention-1 news page benchmarks a
 * block-sparse variant of the method beside the dense one (its paragraph on
 * runtime and memory against the A100 baselines); the pages do not define
 * it, and this library reads it as follows.  The key/query positions are cut
 * into blocks of ATTN_SPARSE_BLOCK, nb = ceil(N / ATTN_SPARSE_BLOCK) per
 * sequence, and a block mask says which (query block, key block) pairs are
 * computed: query i may attend key j only if
 *     block_mask[m][i / ATTN_SPARSE_BLOCK][j / ATTN_SPARSE_BLOCK] != 0
 * (and j <= i when `causal`, which still drops every block past the
 * diagonal).  Pairs whose entry is zero are never loaded or computed.
 *
 *   block_mask   device memory, uint8 [mask_heads, nb, nb], row-major
 *                (query block major), read-only, any alignment; it must
 *                stay unchanged until the stream has run the call
 *   mask_heads   1: one mask for every batch and head; Hkv: query head h
 *                uses mask m = h / (Hq / Hkv), the one of its K/V head, so
 *                all query heads of a GQA group share a pattern
 *
 * A query row with no allowed key gets o = 0 and lse = -inf, and in the
 * backward pass dq = 0 with no contribution to dk or dv.  Everything else
 * (layouts, dtypes, scale, ownership, asynchrony, error behaviour) is that of
 * attn_fwd / attn_bwd; additionally block_mask NULL gives ATTN_ERR_NULLPTR, a
 * mask_heads other than 1 or Hkv ATTN_ERR_SHAPE, and N > ATTN_SPARSE_MAX_N
 * ATTN_ERR_TOO_LARGE.  attn_bwd_blocksparse takes the same workspace as
 * attn_bwd and must be given the lse of attn_fwd_blocksparse with the same
 * mask, causal flag and scale.
 */
#define ATTN_SPARSE_BLOCK 128
#define ATTN_SPARSE_MAX_N 262144

int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                         const unsigned char* block_mask, int mask_heads, int B, int N, int Hq,
                         int Hkv, int d, int dtype, int causal, float scale, void* stream);

int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, const unsigned char* block_mask,
                         int mask_heads, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, int B, int N, int Hq, int Hkv, int d, int dtype,
                         int causal, float scale, void* stream);

/*
 * Standard (materialising) attention: the baseline the pages measure the
 * IO-aware method against (FlashAttention-1 news page, "FlashAttention"
 * section: standard attention writes the N x N attention matrix to HBM and
 * reads it back; FlashAttention-2 review, "Введение").  Same result, tensor
 * layouts, dtypes, scale and causal semantics and error behaviour as
 * attn_fwd / attn_bwd (attn_bwd_standard takes no o or lse: it reads the
 * stored P instead), but every intermediate goes through device memory, in
 * separate launches:
 *
 *   attn_fwd_standard   S = scale q k^T  (float32, full N x N per head)
 *                       P = softmax(S) row-wise with the causal mask applied
 *                           (masked entries stored as 0), rounded to dtype;
 *                           lse = per-row natural-log log-sum-exp
 *                       o = P v
 *   attn_bwd_standard   dv = P^T dout,  dP = dout v^T  (float32, over S),
 *                       dS = P * (dP - rowsum(P * dP))  (rounded to dtype),
 *                       dq = scale dS k,  dk = scale dS^T q
 *                       (dk / dv of a K/V head sum the heads of its group)
 *
 * `workspace` (device memory, 16-byte aligned, at least
 * attn_standard_workspace_bytes() bytes) holds the materialised matrices,
 * each [B, Hq, N, ldn] row-major with row pitch ldn = N rounded up to a
 * multiple of 64:
 *     byte 0                                S, then dP    float32
 *     p_off  = 4 * E rounded up to 256      P             dtype
 *     ds_off = p_off + 2 * E, rounded up    dS            dtype
 * with E = B * Hq * N * ldn, i.e. O(N^2) memory, against O(N) for attn_bwd's
 * workspace.  attn_bwd_standard reads the P that attn_fwd_standard left in
 * the same workspace (standard attention keeps P for the backward pass), so
 * the two calls must use one workspace, be ordered on one stream and use the
 * same inputs, causal flag and scale.  Limits: B * Hq * N < 2^24 and
 * B * Hq <= 65535 (ATTN_ERR_TOO_LARGE otherwise).
 */
size_t attn_standard_workspace_bytes(int B, int N, int Hq, int Hkv, int d);

int attn_fwd_standard(const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int B, int N, int Hq, int Hkv,
                      int d, int dtype, int causal, float scale, void* stream);

int attn_bwd_standard(const void* q, const void* k, const void* v, const void* dout, void* dq,
                      void* dk, void* dv, void* workspace, size_t workspace_bytes, int B, int N,
                      int Hq, int Hkv, int d, int dtype, int causal, float scale, void* stream);

/* Static, human-readable description of a status code. */
const char* attn_strerror(int status);

/* hipError_t of the last failed HIP call made by this library on this thread
 * (0 if none). */
int attn_last_hip_error(void);

/* Library version string. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
