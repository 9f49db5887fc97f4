/*
 * splat_peaks.h - C ABI of libsplat_peaks, measurement kernels that give the
 * rasterizer's roofline its peaks as measured on the machine at hand, next to
 * the datasheet's. Not part of the rasterizer's path; for the benchmark and
 * for anyone timing the library on their own hardware.
 *
 * Every pointer is caller-owned DEVICE memory; work is enqueued on `stream`
 * (0 = the null stream) and nothing blocks. Returns 0 on success, -1 for an
 * invalid argument (nothing enqueued), -2 when the launch or a query fails.
 */
#ifndef SPLAT_PEAKS_H
#define SPLAT_PEAKS_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Full-chip fp32 FMA loop: `blocks` workgroups of 256 threads, each lane
 * running splat_peaks_fma_per_iter() independent FMA chains for `iters` steps
 * (single-issue, no packed math). clk [2 * blocks] u64 receives, per
 * workgroup, the shader-clock cycles and the wall-clock ticks its first wave
 * measured around the loop (cycles / ticks x wall clock rate = the sustained
 * shader clock); sink [blocks * 256] fp32 receives the chains' sums. */
int splat_peaks_valu(unsigned long long *clk, float *sink, int blocks, int iters, hipStream_t stream);

/* The same loop with fp64 FMAs (clk and sink as above, sink holding the sums
 * rounded to fp32). */
int splat_peaks_valu64(unsigned long long *clk, float *sink, int blocks, int iters, hipStream_t stream);

/* dst = src, `bytes` (a multiple of 16) through `blocks` workgroups of 256
 * threads with 16-byte loads and stores: the HBM bandwidth of a plain copy
 * (2 x bytes moved). src and dst must not overlap. */
int splat_peaks_copy(const void *src, void *dst, size_t bytes, int blocks, hipStream_t stream);

/* Broadcast LDS reads: `blocks` workgroups of 256 threads, each lane reading
 * `iters` x splat_peaks_lds_bytes_per_iter() bytes with 16-byte reads, the four
 * 16-lane groups of a wave on four different slots per read (the compositors'
 * pattern). sink [blocks * 256] u32 receives a checksum per lane. */
int splat_peaks_lds(unsigned *sink, int blocks, int iters, hipStream_t stream);

/* Frequency of the wall clock that splat_peaks_valu reads, in kHz (HOST out). */
int splat_peaks_wall_clock_khz(int device, int *khz);

/* Bytes each lane reads per iteration of splat_peaks_lds. */
int splat_peaks_lds_bytes_per_iter(void);

/* FMAs each lane issues per iteration of splat_peaks_valu. */
int splat_peaks_fma_per_iter(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLAT_PEAKS_H */
