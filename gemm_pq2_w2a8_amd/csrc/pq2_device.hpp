// pq2_device.hpp -- device-side helpers shared by the PQ2_0 kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pq2 {

constexpr int kGroup = 128;           // weights per scale group
constexpr int kWave = 64;             // CDNA wavefront width

typedef int v4i __attribute__((ext_vector_type(4)));

// Low 2 bits of every byte: one plane of four 2-bit codes.
constexpr uint32_t kPlaneMask = 0x03030303u;
// Bits 2..3 of every byte: the next plane left in place, i.e. 4 * code.
constexpr uint32_t kPlaneMaskX4 = 0x0C0C0C0Cu;

// v_dot4_i32_i8: acc + sum of four signed byte products.
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int acc) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, acc, false);
}

// Value of the neighbouring lane (lane ^ 1) through a DPP quad permute.
__device__ __forceinline__ int dpp_xor1(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
}

// Sum over aligned segments of `width` lanes (width a power of two <= 64);
// every lane of a segment receives the segment's sum. Fixed butterfly order.
template <int WIDTH>
__device__ __forceinline__ float segment_sum(float v) {
#pragma unroll
    for (int off = 1; off < WIDTH; off <<= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// IEEE binary16 bit pattern -> float32 (exact; v_cvt_f32_f16).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// The four 2-bit planes of a code word as four int8x4 words (plane s holds
// the codes at bits 2s..2s+1 of each byte, moved down to bits 0..1).
__device__ __forceinline__ v4i planes_of(uint32_t w) {
    v4i p;
    p.x = (int)(w & kPlaneMask);
    p.y = (int)((w >> 2) & kPlaneMask);
    p.z = (int)((w >> 4) & kPlaneMask);
    p.w = (int)((w >> 6) & kPlaneMask);
    return p;
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace pq2
