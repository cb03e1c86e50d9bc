// probe.hip -- the measurement probes of include/pq2_probe.h (gfx950): a
// streaming read, an int8 matrix-core loop, the instruction mix of an exact
// float32 per-group epilogue, and a shader-clock reading. They share nothing
// with the PQ2_0 kernels.
#include "../../include/pq2_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 8;               // 16-byte loads in flight per thread
constexpr uint32_t kNever = 0x9E3779B9u; // folded value that triggers the one store

// Grid-stride streaming read. Lane i of a wave reads the 16 bytes after
// lane i - 1, so each load instruction covers 1 KB of contiguous memory.
// Each round issues all of a thread's kUnroll loads (those past the end
// masked off) before it uses any of them, so a thread never waits for one
// load before issuing the next.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4 *__restrict__ src,
                                                               int64_t n16,
                                                               uint32_t *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
         i += kUnroll * stride) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            v[u] = make_uint4(0, 0, 0, 0);
            if (i + u * stride < n16) v[u] = src[i + u * stride];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == kNever) sink[blockIdx.x] = acc;
}

// Eight independent accumulation chains per wave; operands vary per lane so
// nothing folds at compile time.
__global__ __launch_bounds__(kThreads) void mfma_i8_kernel(int32_t *__restrict__ sink,
                                                           int iters) {
    const int l = (int)threadIdx.x;
    const v4i a = {l, l * 3 + 1, l ^ 0x55, 7 - l};
    const v4i b = {l * 5, l + 9, l ^ 0x33, 11 - l};
    v4i c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = v4i{j, 0, 0, 0};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) s ^= c[j].x ^ c[j].y ^ c[j].z ^ c[j].w;
    if ((uint32_t)s == kNever) sink[blockIdx.x] = s;
}

// Per 16 x 16 output tile and 128-deep group: two v_mfma_i32_16x16x64_i8 (a
// dependent pair, as a group's dot is), one v_mfma_f32_4x4x1_16b_f32 (sixteen
// 4 x 4 outer products of two per-lane floats, i.e. a scale product per
// output laid out like the int8 results), and per output element of a lane
// one int32 -> float32 conversion and one FMA that reads the conversion and
// the scale product. Eight tiles per wave with chains of their own; every
// value carries from one round to the next, so nothing is hoisted or folded.
__global__ __launch_bounds__(kThreads) void epilogue_mix_kernel(int32_t *__restrict__ sink,
                                                                int iters) {
    const int l = (int)threadIdx.x;
    const v4i a0 = {l, l * 3 + 1, l ^ 0x55, 7 - l};
    const v4i a1 = {l ^ 0x0f, l + 2, 5 * l, 3 - l};
    const v4i b0 = {l * 5, l + 9, l ^ 0x33, 11 - l};
    const v4i b1 = {l ^ 0x71, 2 * l + 1, l - 4, 13 ^ l};
    const float wf = 1e-3f * (float)((l & 7) + 1);
    const float sf = 1e-3f * (float)((l >> 3) + 1);
    v4i c[8];
    v4f sp[8];
    float acc[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        c[j] = v4i{j, 0, 0, 0};
        sp[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][i] = 0.0f;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, c[j], 0, 0, 0);
            c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, c[j], 0, 0, 0);
            sp[j] = __builtin_amdgcn_mfma_f32_4x4x1f32(wf, sf, sp[j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[j][i] = fmaf((float)c[j][i], sp[j][i], acc[j][i]);
        }
    }
    float f = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) f += acc[j][i];
    if (__builtin_bit_cast(uint32_t, f) == kNever) sink[blockIdx.x] = 1;
}

// One wave: shader clock cycles against wall clock ticks over a spin.
__global__ __launch_bounds__(64) void clock_kernel(uint64_t *__restrict__ out,
                                                   uint64_t spin_ticks) {
    const uint64_t w0 = wall_clock64();
    const uint64_t c0 = clock64();
    uint64_t w = w0;
    while (w - w0 < spin_ticks) w = wall_clock64();
    const uint64_t c1 = clock64();
    if (threadIdx.x == 0) {
        out[0] = c1 - c0;
        out[1] = w - w0;
    }
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int status(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

}  // namespace

extern "C" {

int pq2_probe_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks,
                          void *hip_stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || blocks < 1 || blocks > (1 << 20) ||
        !aligned(src, 16) || !aligned(sink, 4))
        return -1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), static_cast<const uint4 *>(src),
                       (int64_t)(bytes / 16), sink);
    return status(hipGetLastError());
}

int pq2_probe_mfma_i8(int32_t *sink, int iters, int blocks, void *hip_stream) {
    if (!sink || iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > (1 << 20) ||
        !aligned(sink, 4))
        return -1;
    hipLaunchKernelGGL(mfma_i8_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), sink, iters);
    return status(hipGetLastError());
}

int pq2_probe_epilogue_mix(int32_t *sink, int iters, int blocks, void *hip_stream) {
    if (!sink || iters < 1 || iters > (1 << 24) || blocks < 1 || blocks > (1 << 20) ||
        !aligned(sink, 4))
        return -1;
    hipLaunchKernelGGL(epilogue_mix_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                       static_cast<hipStream_t>(hip_stream), sink, iters);
    return status(hipGetLastError());
}

int pq2_probe_clock(uint64_t *out, uint64_t spin_ticks, void *hip_stream) {
    if (!out || spin_ticks < 1 || spin_ticks > (1ull << 28) || !aligned(out, 8)) return -1;
    hipLaunchKernelGGL(clock_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(hip_stream),
                       out, spin_ticks);
    return status(hipGetLastError());
}

}  // extern "C"
