/*
 * coda_probe.h - measurement support of libcoda.so: a kernel that keeps every
 * compute unit's matrix cores busy with independent bf16 MFMAs and nothing
 * else, so that a benchmark can state the shader clock and the dense bf16
 * rate this device actually sustains under a matrix-core load.  The fused
 * GEMM-epilogue kernels are judged against the published peak (256 compute
 * units x 2.4 GHz x 4096 FLOP per clock); this probe gives the clock that
 * peak assumes, as measured, beside it.  It is not part of the computation.
 *
 * Conventions are those of coda.h (caller-owned device pointers, no
 * allocation or synchronisation, launch on `stream`, coda_status return).
 */
#ifndef CODA_PROBE_H_
#define CODA_PROBE_H_

#include "coda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Launches `blocks` workgroups of four waves; each workgroup holds more than
 * half of a compute unit's LDS, so at most one runs per compute unit.  Every
 * wave issues iters x 8 independent v_mfma_f32_32x32x16_bf16 (8 accumulator
 * chains), i.e. blocks * 4 * iters * 8 * 32768 FLOP in total.  Wave 0 of
 * workgroup b writes, as unsigned 64-bit counts, out[2b] = s_memtime ticks
 * (shader clock) and out[2b + 1] = s_memrealtime ticks (the constant
 * reference clock) elapsed over its MFMA loop.  out: device, 2 * blocks
 * entries.  Needs 1 <= blocks <= 65536, 1 <= iters <= 1000000. */
coda_status coda_probe_mfma(int blocks, int iters, unsigned long long* out, hipStream_t stream);

/* Tile timeline (observability).  Only the timeline build of the library
 * (libcoda_timeline.so, compiled with CODA_TIMELINE=1; its kernels are those
 * of libcoda.so plus four clock reads and stores per wave and tile) records
 * anything; libcoda.so returns CODA_ERR_UNSUPPORTED.
 *
 * coda_timeline_set installs `buf` (device, 8-byte aligned, waves x
 * coda_timeline_words() unsigned 64-bit words, caller-owned) for every later
 * GEMM launch of the process until it is called again; buf = NULL with
 * waves = 0 uninstalls.  A launch writes the record of wave w of dispatched
 * workgroup b at index 4 b + w if that is below `waves` (later records are
 * dropped), overwriting what an earlier launch left there:
 *   words 0-3  constant reference clock (s_memrealtime, 100 MHz) at the tile
 *              start, the k-loop start (operand prologue done), the k-loop
 *              end and the epilogue end (its stores issued);
 *   words 4-7  the shader clock (s_memtime) at the same points;
 *   word 8     the tile's token width (256, or 128 for split tiles);
 *   word 9     its k-tile count;
 *   words 10, 11  the HW_ID and XCC_ID registers of the wave (which XCD,
 *              shader engine and compute unit ran it).
 * Errors: CODA_ERR_SHAPE (waves < 0, or buf NULL with waves > 0),
 * CODA_ERR_ALIGN.  Launches read the installation under a lock; records of
 * launches that overlap on the device mix. */
coda_status coda_timeline_set(unsigned long long* buf, int waves);
int coda_timeline_words(void);

#ifdef __cplusplus
}
#endif

#endif /* CODA_PROBE_H_ */
