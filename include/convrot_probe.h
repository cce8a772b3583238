/*
 * convrot_probe.h -- hardware measurement probes of libconvrot_probe.so.
 *
 * These are not part of the linear layer's interface (include/convrot.h).
 * They measure what the roofline fractions of the layer's kernels are
 * compared against on the running GPU: the int8 matrix-core rate on random
 * operands with no memory traffic, the shader clock under that load, and
 * the bandwidth of a plain streaming copy and of a plain streaming read.
 * Same conventions as convrot.h: device pointers, asynchronous on `stream`,
 * host-side validation before any launch, 0 on success.
 */
#ifndef CONVROT_PROBE_H
#define CONVROT_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Threads per workgroup of the probe (8 wavefronts, two per SIMD). */
#define CONVROT_PROBE_THREADS 512
/* Independent accumulator chains per wavefront and loop iteration. */
#define CONVROT_PROBE_CHAINS 8
/* int8 operations of one v_mfma_i32_16x16x64_i8: 2 * 16 * 16 * 64. */
#define CONVROT_PROBE_OPS_PER_MFMA 32768

/* MFMA-only int8 loop: `grid` workgroups of CONVROT_PROBE_THREADS threads
 * (one per CU when grid equals the CU count), each wavefront running
 * `iters` iterations of CONVROT_PROBE_CHAINS independent
 * v_mfma_i32_16x16x64_i8, alternating between two operand sets that each
 * lane reads from `operands` (random bytes, 64 per thread:
 * grid * CONVROT_PROBE_THREADS * 64 bytes, 16-byte aligned), so the
 * operands toggle as in a GEMM on random codes.  Total int8 operations:
 * grid * 8 * iters * CONVROT_PROBE_CHAINS * CONVROT_PROBE_OPS_PER_MFMA.
 * Each workgroup's first wavefront writes four uint64 to stamps[4 b ..]:
 * the shader-clock counter (s_memtime) and the constant 100 MHz counter
 * (s_memrealtime) before and after its loop, so the clock of that CU over
 * the loop is (t1 - t0) / ((r1 - r0) / 100 MHz).  `sink` (grid * 512
 * int32) receives the accumulators only when `flag` == 0x5eed (never in
 * use; it keeps the products live).  Returns 0, or 1 on a bad argument, 2
 * when the launch fails. */
int convrot_probe_mfma_i8(const void* operands, int grid, int iters, uint64_t* stamps, int32_t* sink, int flag,
                          void* stream);

/* Streaming device copy of `bytes` bytes (a multiple of 16; src and dst
 * 16-byte aligned, not overlapping) by `grid` workgroups of 256 threads,
 * each thread moving four 16-byte chunks per round with nontemporal loads
 * and stores: the bandwidth a plain streaming kernel reaches (read + write
 * bytes per second).  Returns 0, 1 on a bad argument, 2 when the launch
 * fails. */
int convrot_probe_copy(const void* src, void* dst, int64_t bytes, int grid, void* stream);

/* Streaming read of `bytes` bytes (a multiple of 16; src 16-byte aligned)
 * by `grid` workgroups of 256 threads, with the copy's access pattern and no
 * stores: the bandwidth and per-launch fixed cost a read-dominated kernel
 * (weight streaming at small M) is bounded by.  `sink` (grid * 256 int32)
 * is written only when `flag` == 0x5eed (never in use; it keeps the loads
 * live).  Returns 0, 1 on a bad argument, 2 when the launch fails. */
int convrot_probe_read(const void* src, int64_t bytes, int grid, int32_t* sink, int flag, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVROT_PROBE_H */
