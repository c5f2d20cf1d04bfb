/*
 * moe_probe.h -- C ABI of libmoe_probe.so: microbenchmarks that measure what
 * one MI355X (gfx950) reaches on the two resources bounding the MoE layer,
 * HBM streaming and bf16 MFMA issue.  They give measured ceilings to report
 * beside the datasheet peaks (HBM3E 8 TB/s; dense bf16 MFMA 256 CUs x
 * 2.4 GHz x 4096 flop/clk = 2516.6 TFLOP/s).  They are measurement tools,
 * not part of the layer; the layer's entry points are in moe_ffn.h.
 *
 * Conventions: pointers are DEVICE pointers owned by the caller; calls are
 * asynchronous on `stream` (hipStream_t, NULL = default stream) and return
 * 0 on success, 1 on a rejected argument or a failed launch (nothing is
 * enqueued for a rejected argument).  Time them with events on that stream.
 */
#ifndef MOE_PROBE_H
#define MOE_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) from `src` (16-byte aligned) with 16-byte
 * loads spread over `blocks` blocks of 256 threads; block b writes the XOR of
 * what it read to sink[b] (sink holds `blocks` words).  Bytes moved: bytes. */
int moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream);

/* Copy `bytes` (a multiple of 16) from src to dst (both 16-byte aligned, not
 * overlapping) with 16-byte loads and stores over `blocks` blocks of 256
 * threads.  Bytes moved: 2 * bytes. */
int moe_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);

/* `blocks` blocks of 8 waves, each wave issuing `iters` rounds of eight
 * independent v_mfma_f32_32x32x16_bf16 on register operands; wave w of block
 * b writes the sum of its accumulators to sink[8 b + w] (sink holds 8 *
 * blocks floats).  Flops: moe_probe_mfma_flops(blocks, iters). */
int moe_probe_mfma(float* sink, int blocks, int iters, void* stream);
double moe_probe_mfma_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PROBE_H */
