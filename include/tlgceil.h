/* Hardware-ceiling probes for the benchmark (libtlgceil.so).
 *
 * Not part of the GEMM path: these kernels measure what the GPU can reach
 * beside its datasheet peaks, the way "Optimizing a GPT-2-class transformer
 * on a GPU" (Act V) and "One multiply, one RTX 5090, eight kernels" ("Where
 * the time goes", "What was not measured") time an empty kernel and
 * loads-only / math-only variants.  Every function enqueues one kernel on
 * `stream` (a hipStream_t, NULL for the default stream) and returns 0, -1 for
 * an invalid argument (nothing launched) or -6 when the launch fails.
 * Pointers are device pointers owned by the caller.
 */
#ifndef TLGCEIL_H
#define TLGCEIL_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Empty kernel over `grid` (> 0) workgroups of 64 threads; `flag` is one int
 * the kernel never writes in practice. */
int tlg_ceil_empty(int grid, int* flag, void* stream);

/* Read `bytes` bytes starting at `p`: 16-byte aligned, `bytes` a non-zero
 * multiple of 128 KiB.  One workgroup of 8 waves per 128 KiB; every load of a
 * wave covers 1 KiB of consecutive bytes.  `sink` holds 512 floats and is
 * written only for a data pattern that does not occur in practice. */
int tlg_ceil_read(const void* p, size_t bytes, float* sink, void* stream);

/* On-chip read rate: `p` (16-byte aligned) holds 24 MiB; 256 workgroups of 8
 * waves each re-read their own 96 KiB block `reps` (> 0) times, the whole
 * block in flight per pass, so after the first pass the data comes from each
 * XCD's L2 (3 MiB per XCD): 24 MiB per pass in all.  `sink` holds 512 floats,
 * written like `tlg_ceil_read`'s. */
int tlg_ceil_read_l2(const void* p, int reps, float* sink, void* stream);

/* MFMA issue rate: `grid` (> 0) workgroups of 4 waves, each wave issuing
 * 16·`iters` (> 0) independent MFMAs with no memory traffic: 32x32x16 bf16
 * (32768 flop each) when `bf16` is non-zero, else 32x32x2 fp32 (4096 flop
 * each).  `sink` holds 256 floats, written like `tlg_ceil_read`'s. */
int tlg_ceil_mfma(int bf16, int grid, int iters, float* sink, void* stream);

/* tlg_ceil_mfma, and the core clock it ran at: `stamps` is NULL or holds
 * 4·`grid` counters; thread 0 of workgroup g writes stamps[4g .. 4g+3] = the
 * shader-clock counter (s_memtime) before and after its MFMA loop, then the
 * constant-rate counter (s_memrealtime) before and after.  The clock is
 * (s1 - s0) / (r1 - r0) times the constant rate. */
int tlg_ceil_mfma_clock(int bf16, int grid, int iters, float* sink, unsigned long long* stamps, void* stream);

/* Rate of the constant-rate counter of the current device in kHz (the HIP
 * wall-clock rate attribute); 0 on success, -6 if the runtime refuses. */
int tlg_ceil_wall_clock_khz(int* khz);

#ifdef __cplusplus
}
#endif

#endif /* TLGCEIL_H */
