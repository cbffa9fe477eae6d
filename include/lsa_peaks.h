/*
 * lsa_peaks.h -- microbenchmarks of the MI355X ceilings the path's kernels are
 * measured against, on the machine that runs them: the pages report each kernel
 * step as a share of the chip's peak compute and memory bandwidth from a profiler
 * run ("Latent Sparse Attention (LSA)", App. F.1 "Measurements"), and these give the
 * reachable side of those peaks.  Measurement only; no part of the method uses them.
 *
 * Every call enqueues one kernel on `stream` (a hipStream_t as void*) and returns at
 * once: the caller times it with events on that stream.  `sink` is caller-owned
 * device memory of lsa_peak_sink_ints(n_blocks) int32 (one value per thread, so the
 * compiler cannot drop the work).  Returns 0, -1 for an invalid argument (nothing
 * launched) or -4 if the launch failed.
 */
#ifndef LSA_PEAKS_H
#define LSA_PEAKS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LSA_PEAK_MFMA_I8 = 0, LSA_PEAK_MFMA_BF16 = 1 };

/* int32 entries `sink` needs for a launch of n_blocks workgroups (256 threads each). */
int32_t lsa_peak_sink_ints(int32_t n_blocks);

/* Matrix-core issue rate: n_blocks workgroups of 4 waves, each wave running `iters`
   steps of 4 independent MFMAs -- kind LSA_PEAK_MFMA_I8: v_mfma_i32_16x16x64_i8
   (32768 int8 ops each), LSA_PEAK_MFMA_BF16: v_mfma_f32_16x16x32_bf16 (16384 flops
   each).  Work = n_blocks * 4 * iters * 4 * (ops per MFMA). */
int lsa_peak_mfma(int32_t kind, int64_t iters, int32_t n_blocks, int32_t* sink, void* stream);

/* Streaming read of `bytes` (a multiple of 16, 16-byte aligned) of device memory,
   each byte once: workgroup x reads one contiguous span of about bytes / n_blocks
   with coalesced 16-byte non-temporal loads, eight in flight per thread. */
int lsa_peak_read(const void* src, int64_t bytes, int32_t n_blocks, int32_t* sink, void* stream);

/* Random gather of 256-byte rows: rows[idx[e]] for e < n_idx (indices clamped into
   [0, n_rows)), 16 lanes per row; 256 * n_idx bytes read.  `rows` is n_rows * 256
   bytes, 16-byte aligned. */
int lsa_peak_gather(const void* rows, int64_t n_rows, const int32_t* idx, int64_t n_idx, int32_t n_blocks,
                    int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LSA_PEAKS_H */
