/*
 * mla_peaks.h - achievable-peak microbenchmarks of libmla_peaks.so (MI355X, gfx950).
 *
 * Measurement support for the benchmark: the attention path never calls these.
 * They give same-run denominators for roofline fractions beside the spec-sheet
 * peaks (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).  Each enqueues one kernel on
 * `stream` (a hipStream_t passed as void*, NULL = the null stream) and returns 0,
 * -1 for a rejected argument (nothing enqueued) or -4 for a launch failure.  All
 * pointers are device pointers.  `sink` is a small device buffer (4 bytes per
 * workgroup) that the kernels write only on a value their data never produces; it
 * keeps the compiler from dropping the loads and MFMAs.
 */
#ifndef MLA_PEAKS_H_
#define MLA_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every 16-byte chunk of buf[0, bytes) once with plain vector loads (grid-
 * stride, four loads in flight per lane).  buf 16-byte aligned, bytes >= 16. */
int mla_peak_stream_read(const void* buf, size_t bytes, void* sink, int workgroups,
                         void* stream);

/* The split-KV kernel's load path alone: each of `workgroups` workgroups (four waves,
 * one per compute unit by its LDS use) streams its own contiguous range of 36,864-byte
 * blocks into a four-slot LDS ring with 16-byte direct global->LDS copies, three
 * blocks issued ahead of the one waited for.  It reads the first
 * mla_peak_dma_stream_bytes(bytes, workgroups) bytes of buf. */
int mla_peak_dma_stream(const void* buf, size_t bytes, void* sink, int workgroups,
                        void* stream);
size_t mla_peak_dma_stream_bytes(size_t bytes, int workgroups);

/* `iters` iterations of four independent v_mfma_f32_32x32x16_bf16 accumulation
 * chains per wave, four waves per workgroup; mla_peak_mfma_bf16_flops gives the
 * flops of such a launch (32,768 per MFMA). */
int mla_peak_mfma_bf16(int iters, void* sink, int workgroups, void* stream);
double mla_peak_mfma_bf16_flops(int iters, int workgroups);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PEAKS_H_ */
