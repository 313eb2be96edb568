/*
 * libqlinear_ceiling -- measured ceilings of one MI355X (gfx950) for the
 * benchmark: the weight-quantized linear layer of the "fp8_gemv" page is
 * bound by reading its weight at decode ("WHY it wins at decode") and by the
 * matrix cores at large M ("Matmul2dFp8", "int8_matmul"); these kernels
 * measure what a plain read-only stream and back-to-back matrix-core
 * instructions reach on the chip, so that the layer's kernels can be put
 * against an attainable figure as well as the published peaks.  Not part of
 * libqlinear; used by bench.py only.
 *
 * Pointers are device pointers on the current device; `stream` is a
 * hipStream_t (NULL = null stream).  Calls only enqueue.  Return 0 on
 * success, 1 for an invalid argument (nothing launched), 4 when the launch
 * failed.
 */
#ifndef QLINEAR_CEILING_H
#define QLINEAR_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads every byte of buf[0, bytes) once with 16-byte non-temporal loads:
 * each wave takes a contiguous span of span_kib KiB (4, 8 or 16; one load
 * instruction per KiB, all in flight at once) and the `blocks` blocks of 256
 * threads stride over the spans.  buf 16-byte aligned, bytes a positive
 * multiple of 16; sink: 4 bytes of device memory, written only if the XOR
 * of the data equals a fixed key (in practice never).
 */
int qlinear_ceiling_stream_read(const void* buf, int64_t bytes, int span_kib, int64_t blocks, void* sink,
                                void* stream);

/*
 * The same read through the DMA unit straight into LDS (global_load_lds,
 * 16 bytes per lane, non-temporal), the path the LDS-staged kernels use:
 * each wave keeps one span of span_kib KiB (4, 8 or 16) in flight and
 * waits for it before issuing the next.  Arguments as
 * qlinear_ceiling_stream_read.
 */
int qlinear_ceiling_stream_dma(const void* buf, int64_t bytes, int span_kib, int64_t blocks, void* sink,
                               void* stream);

/*
 * Re-reads of a small buffer (about 2 MiB: resident in every XCD's L2 after
 * the first pass), to measure what the L2s deliver to the CUs: each of the
 * `blocks` x 4 waves reads `iters` spans of 8 KiB (span (wave + 7919 i) mod
 * the buffer's spans), through the DMA unit into LDS (dma != 0, one span in
 * flight per wave) or into registers.  bytes >= 8 KiB; the bytes read are
 * blocks x 4 x iters x 8 KiB.
 */
int qlinear_ceiling_reread(const void* buf, int64_t bytes, int dma, int64_t blocks, int iters, void* sink,
                           void* stream);

/*
 * `blocks` blocks of 4 waves, each wave running `iters` rounds of four
 * independent back-to-back matrix-core instructions on register operands:
 * dtype 0 = v_mfma_f32_32x32x16_bf16, 1 = v_mfma_i32_32x32x32_i8,
 * 2 = v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit scales).  sink:
 * 1 KiB of device memory, written only on an impossible sum.
 */
int qlinear_ceiling_mfma(int dtype, int64_t blocks, int iters, void* sink, void* stream);

/* Floating-point (or integer) operations of one wave's round of
 * qlinear_ceiling_mfma for `dtype` (0 for an unknown dtype). */
int64_t qlinear_ceiling_mfma_ops_per_wave_round(int dtype);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_CEILING_H */
