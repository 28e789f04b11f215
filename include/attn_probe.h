/*
 * attn_probe.h -- C ABI of libattn_probe.so, the throughput probes the
 * benchmark uses as measured ceilings for the attention kernels' matrix
 * work (MFMA), exponentials and LDS reads on MI355X (gfx950).  Not part of
 * the attention library.
 *
 * The dense bf16 peak in AMD's specification (2516.6 TFLOP/s = 256 CUs x
 * 4096 FLOP/clock x 2.4 GHz) assumes the full shader clock.  Under sustained
 * matrix work the clock follows the power limit, which depends on the data,
 * so the probe measures what the part sustains on back-to-back
 * v_mfma_f32_32x32x16_bf16 with the operands the caller supplies.
 */
#ifndef ATTN_PROBE_H_
#define ATTN_PROBE_H_

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueue `workgroups` workgroups of four wavefronts; each wavefront runs
 * `iters` x 16 products of 32 x 32 x 16 on four A and four B fragments read
 * once from `operands` and keeps the results in registers until one final
 * store.
 *   operands   device memory, bf16, 16-byte aligned, workgroups * 256 * 64
 *              elements (32 A and 32 B values per thread), read-only
 *   out        device memory, float32, 16-byte aligned, workgroups * 256 * 16
 *              elements: the summed accumulators (only to keep the work live)
 *   stream     hipStream_t (NULL: the legacy default stream); asynchronous
 * Returns 0 on success, 1 for a NULL pointer, 2 for workgroups outside
 * [1, 2^20] or iters < 1, 3 if the launch failed.  Caller owns all memory.
 */
int attn_probe_mfma(const void* operands, float* out, int workgroups, int iters, void* stream);

/* Matrix FLOPs one attn_probe_mfma call performs (2 per multiply-add). */
double attn_probe_mfma_flops(int workgroups, int iters);

/*
 * v_exp_f32 throughput: `workgroups` x 256 threads each run `iters` x 8
 * exponentials (eight independent chains).  in: workgroups * 256 * 8 floats
 * (seed values), out: workgroups * 256 floats (results, only to keep the work
 * live); device memory, 4-byte aligned.  Status codes as attn_probe_mfma.
 */
int attn_probe_exp(const float* in, float* out, int workgroups, int iters, void* stream);

/*
 * LDS read bandwidth: `workgroups` x 256 threads each read `iters` x 8 x 16
 * bytes from LDS with conflict-free ds_read_b128.  out: workgroups * 256
 * floats (results, only to keep the work live); clk: 2 values written by
 * workgroup 0, the shader-clock and the 100 MHz real-time counter deltas over
 * its loop (their ratio times 100 MHz is the shader clock).  Device memory;
 * status codes as attn_probe_mfma.
 */
int attn_probe_lds(float* out, unsigned long long* clk, int workgroups, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PROBE_H_ */
