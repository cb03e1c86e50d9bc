/*
 * pq2_probe.h -- measurement probes for AMD Instinct MI355X (gfx950), built
 * as libpq2_probe.so beside the PQ2_0 library. They are not part of the
 * PQ2_0 computation: they measure the practical ceilings the PQ2_0 kernels
 * are compared with (the page "Making a ternary reasoning model fast in
 * vLLM -- from CUDA to Triton and Gluon", section "Measure at the clock
 * speeds used in serving", judges kernels at the clock they actually run
 * at; the page "Chasing llama.cpp at batch one", section "Checkpoint: faster
 * through specialisation", frames results against the weight-bandwidth
 * bound).
 *
 * Every call validates its arguments on the host, only enqueues one kernel
 * on the given stream (NULL = the null stream), never allocates or
 * synchronises, and returns 0, or -1 for invalid arguments, or the
 * hipError_t of a rejected launch. Buffers are caller-owned device memory.
 */
#ifndef PQ2_PROBE_H
#define PQ2_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read: `blocks` blocks of 256 threads read the `bytes` bytes at
 * src once, with 16-byte loads (consecutive lanes on consecutive 16-byte
 * pieces; a grid-stride loop whose rounds issue up to eight loads per
 * thread before using any), and fold them into one word per thread. Nothing is written unless a block's
 * folded value equals a fixed constant, so the write traffic is at most one
 * word per block into sink (uint32 [blocks]).
 *   src: 16-byte aligned; bytes: a positive multiple of 16;
 *   blocks: 1 .. 2^20; sink: 4-byte aligned.
 */
int pq2_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks,
                          void *hip_stream);

/*
 * int8 matrix-core loop: `blocks` blocks of 4 waves; every wave issues
 * `iters` rounds of eight independent v_mfma_i32_16x16x64_i8 chains (no
 * memory traffic in the loop). Integer ops = 2 * 16 * 16 * 64 per
 * instruction, i.e. blocks * 4 * iters * 8 * 32768. As for the streaming
 * read, at most one word per block is written to sink (int32 [blocks]).
 *   iters: 1 .. 2^24; blocks: 1 .. 2^20.
 */
int pq2_probe_mfma_i8(int32_t *sink, int iters, int blocks, void *hip_stream);

/*
 * The instruction mix of an exact float32 per-group epilogue on int8 MFMA
 * results (the PQ2_0 float epilogue of the page "Making a ternary reasoning
 * model fast in vLLM", section "One token at a time: plain Triton is
 * enough": y += s * ws * dot per group): per 16 x 16 output tile and
 * 128-deep group, two v_mfma_i32_16x16x64_i8 (dependent), one
 * v_mfma_f32_4x4x1_16b_f32 (the scale products as outer products) and, per
 * output element of a lane, one int32 -> float32 conversion and one FMA;
 * eight tiles per wave, no memory traffic in the loop. `blocks` blocks of 4
 * waves run `iters` rounds; the int8 ops counted are those of the two int8
 * MFMAs: blocks * 4 * iters * 8 * 2 * 32768. At most one word per block is
 * written to sink (int32 [blocks]).
 *   iters: 1 .. 2^24; blocks: 1 .. 2^20.
 */
int pq2_probe_epilogue_mix(int32_t *sink, int iters, int blocks, void *hip_stream);

/*
 * Shader clock: one wave spins until the constant-rate wall clock counter
 * (wall_clock64, rate hipDeviceAttributeWallClockRate kHz) has advanced by
 * spin_ticks, and writes out[0] = shader clock cycles (clock64) and
 * out[1] = wall clock ticks over the spin; the shader clock in MHz is
 * out[0] / out[1] * (wall clock rate in MHz).
 *   out: uint64 [2], 8-byte aligned; spin_ticks: 1 .. 2^28.
 */
int pq2_probe_clock(uint64_t *out, uint64_t spin_ticks, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ2_PROBE_H */
