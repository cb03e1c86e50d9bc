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

// IEEE binary16 bit pattern -> float32 (exact; v_cvt_f32_f16).
__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// float32 -> bfloat16 bits, rounded to nearest, ties to even (infinities and
// NaN stay infinities and NaN).
__device__ __forceinline__ uint16_t bf16_rne(float v) {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// Output element i: float32 into y, or bfloat16 into y16 when that is given.
__device__ __forceinline__ void store_y(float *y, uint16_t *y16, int64_t i, float v) {
    if (y16)
        y16[i] = bf16_rne(v);
    else
        y[i] = v;
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

// Lane exchange patterns within aligned 32-lane segments, all symmetric (so a
// max or sum over the segment is the same value on every lane): DPP quad
// permutes (lane ^ 1, lane ^ 2), DPP row half-mirror (lane i <-> 7 - i in 8
// lanes) and row mirror (i <-> 15 - i in 16 lanes) stay in the VALU; the
// exchange across the two 16-lane rows is one ds_swizzle (lane ^ 16).
__device__ __forceinline__ int dpp_xor2(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ int dpp_half_mirror(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
}
__device__ __forceinline__ int dpp_mirror(int v) {
    return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
}
__device__ __forceinline__ int swizzle_xor16(int v) {
    return __builtin_amdgcn_ds_swizzle(v, 0x401F);   // and 0x1F, or 0, xor 0x10
}
// Value of lane i of this lane's quad.
template <int I>
__device__ __forceinline__ int dpp_quad_bcast(int v) {
    return __builtin_amdgcn_update_dpp(0, v, I * 0x55, 0xF, 0xF, false);
}

// Sum over aligned segments of `width` lanes (width a power of two <= 64);
// every lane of a segment receives the segment's sum, bit for bit the same
// on every lane (each step adds two lanes' values, and the partner adds the
// same two). Steps: quad permutes (lane ^ 1, lane ^ 2), row half-mirror and
// row mirror in the VALU, then one ds_swizzle across 16-lane rows and, for a
// whole wave, one lane shuffle across the halves.
template <int WIDTH>
__device__ __forceinline__ float segment_sum(float v) {
    static_assert(WIDTH >= 1 && WIDTH <= 64 && (WIDTH & (WIDTH - 1)) == 0, "segment width");
    auto add = [](float a, int b) __attribute__((always_inline)) {
        return a + __builtin_bit_cast(float, b);
    };
    if (WIDTH >= 2) v = add(v, dpp_xor1(__builtin_bit_cast(int, v)));
    if (WIDTH >= 4) v = add(v, dpp_xor2(__builtin_bit_cast(int, v)));
    if (WIDTH >= 8) v = add(v, dpp_half_mirror(__builtin_bit_cast(int, v)));
    if (WIDTH >= 16) v = add(v, dpp_mirror(__builtin_bit_cast(int, v)));
    if (WIDTH >= 32) v = add(v, swizzle_xor16(__builtin_bit_cast(int, v)));
    if (WIDTH >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

// Per-element steps of the int8 quantiser, shared by every kernel that
// quantises activations so that all of them give identical q: the tiny-scale
// test, the fast rounding of x / s through rc = v_rcp_f32(s) with the flag
// that says it equals the IEEE quotient's rounding, and the final clamp.
// s = amax / 127 is the IEEE float32 quotient (the library is built with
// correctly rounded division and float32 denormals) and q = clamp(rne(fl32(x
// / s)), -127, 127) the IEEE result as well, through an exact shortcut:
//   with rc = v_rcp_f32(s) (relative error <= 2^-23) and y = fl32(x * rc),
//   |y - x/s| <= 127.5 * (2^-23 + 2^-24) < 2^-15.4 and |fl32(x/s) - x/s|
//   <= 2^-18 (|x / s| <= 127.5), so y and fl32(x/s) are within 2^-15 of each
//   other; when y is farther than 2^-13 from every half-integer both round
//   to the same integer and neither is a tie. Otherwise (about 2e-4 of
//   random inputs), and for scales below 2^-100 (whose reciprocal may
//   overflow), the IEEE division decides (a wave-uniform branch, taken only
//   when some lane needs it). s == 0 gives q = 0.
__device__ __forceinline__ bool quant_tiny(float scale) { return scale < 0x1p-100f; }

__device__ __forceinline__ float quant_round_fast(float x, float rc, bool tiny, bool &ok) {
    const float y = x * rc;
    const float ry = rintf(y);
    ok = !tiny && fabsf(fabsf(y - ry) - 0.5f) > 0x1p-13f;
    return ry;
}

__device__ __forceinline__ int quant_clamp(float qf, float scale) {
    return scale == 0.0f ? 0 : (int)fminf(fmaxf(qf, -127.0f), 127.0f);
}

// Per-128-group int8 quantisation of activations in plane order, in two lane
// layouts with the same element arithmetic (the quant_* helpers; amax and
// sum(q) are exact in any order), so every kernel gives identical q, s, t.
// 32 lanes per group: lane b holds x[4b .. 4b+3] (plane position b, planes
// 0..3), amax and the sum of q reduce over the 32 lanes, and a 4x4 byte
// transpose inside each quad (lanes 4j..4j+3: quad broadcasts and byte
// permutes) leaves lane 4j+p holding the plane word (p, j): the group's
// bytes 32p + 4j .. 32p + 4j + 3. NR groups per 32-lane slot are processed
// stage by stage. Each lane's chain is short (one float4), which suits
// launches of few groups, where latency rather than issue decides.
template <int NR>
__device__ __forceinline__ void quantize_groups32(const float4 (&v)[NR], int lane32,
                                                  uint32_t (&word)[NR], float (&scale)[NR],
                                                  int (&sum)[NR]) {
    float a[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
        a[r] = fmaxf(fmaxf(fabsf(v[r].x), fabsf(v[r].y)), fmaxf(fabsf(v[r].z), fabsf(v[r].w)));
#define PQ2_SEG_MAX_STEP(EXCH)                                                            \
    _Pragma("unroll") for (int r = 0; r < NR; ++r)                                      \
        a[r] = fmaxf(a[r], __builtin_bit_cast(float, EXCH(__builtin_bit_cast(int, a[r]))));
    PQ2_SEG_MAX_STEP(dpp_xor1)
    PQ2_SEG_MAX_STEP(dpp_xor2)
    PQ2_SEG_MAX_STEP(dpp_half_mirror)
    PQ2_SEG_MAX_STEP(dpp_mirror)
    PQ2_SEG_MAX_STEP(swizzle_xor16)
#undef PQ2_SEG_MAX_STEP
    float rc[NR];
    bool slow = false;
    float qf[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        scale[r] = a[r] / 127.0f;                   // IEEE division
        rc[r] = __builtin_amdgcn_rcpf(scale[r]);
        const bool tiny = quant_tiny(scale[r]);     // includes s == 0
        const float xs[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bool ok;
            qf[r][e] = quant_round_fast(xs[e], rc[r], tiny, ok);
            slow |= !ok && scale[r] != 0.0f;
        }
    }
    if (__any(slow)) {                              // rare: the IEEE division decides
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const bool tiny = quant_tiny(scale[r]);
            const float xs[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bool ok;
                quant_round_fast(xs[e], rc[r], tiny, ok);
                if (!ok && scale[r] != 0.0f) qf[r][e] = rintf(xs[e] / scale[r]);
            }
        }
    }
    int u[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        int q[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = quant_clamp(qf[r][e], scale[r]);
        sum[r] = q[0] + q[1] + q[2] + q[3];
        // byte p of u = q of column 4*lane32 + p, i.e. plane p, position lane32
        u[r] = (int)((uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                     ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24));
    }
#define PQ2_SEG_SUM_STEP(EXCH) _Pragma("unroll") for (int r = 0; r < NR; ++r) sum[r] += EXCH(sum[r]);
    PQ2_SEG_SUM_STEP(dpp_xor1)
    PQ2_SEG_SUM_STEP(dpp_xor2)
    PQ2_SEG_SUM_STEP(dpp_half_mirror)
    PQ2_SEG_SUM_STEP(dpp_mirror)
    PQ2_SEG_SUM_STEP(swizzle_xor16)
#undef PQ2_SEG_SUM_STEP
    // byte i of the word = byte p of quad lane i's u (v_perm: selector bytes
    // 0-3 pick the second operand's bytes, 4-7 the first's, 0x0C gives zero)
    const uint32_t p = (uint32_t)(lane32 & 3);
    const uint32_t sel = p | ((4u + p) << 8) | 0x0C0C0000u;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const uint32_t o0 = (uint32_t)dpp_quad_bcast<0>(u[r]), o1 = (uint32_t)dpp_quad_bcast<1>(u[r]);
        const uint32_t o2 = (uint32_t)dpp_quad_bcast<2>(u[r]), o3 = (uint32_t)dpp_quad_bcast<3>(u[r]);
        const uint32_t t01 = __builtin_amdgcn_perm(o1, o0, sel);
        const uint32_t t23 = __builtin_amdgcn_perm(o3, o2, sel);
        word[r] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    }
}

// 8 lanes per group (aligned 8-lane segments): lane j of a segment holds
// activations 16j .. 16j + 15 of the group as
// v[i] = x[16j + 4i .. 16j + 4i + 3], i.e. plane positions b = 4j + i with
// planes 0..3 in .x .y .z .w. Plane p's bytes 32p + 4j .. 32p + 4j + 3 are
// then this lane's own q at positions 4j .. 4j + 3, so word[p] is the plane
// word (p, j) with no byte transpose; amax and sum(q) reduce over the 8 lanes
// (quad permutes and the row half-mirror). Against 32 lanes per group the
// per-group work -- the reductions, the division -- is four times rarer per
// activation, which pays where the quantisation's issue is the cost (the
// fused decode GEMV: 5.74 -> 5.02 us; the quantiser at 4096 x 5120: 20.3 ->
// 16.7 us).
__device__ __forceinline__ void quantize_groups8(const float4 (&v)[4], uint32_t (&word)[4],
                                                 float &scale, int &sum) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        a = fmaxf(a, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
    a = fmaxf(a, __builtin_bit_cast(float, dpp_xor1(__builtin_bit_cast(int, a))));
    a = fmaxf(a, __builtin_bit_cast(float, dpp_xor2(__builtin_bit_cast(int, a))));
    a = fmaxf(a, __builtin_bit_cast(float, dpp_half_mirror(__builtin_bit_cast(int, a))));
    scale = a / 127.0f;                             // IEEE division
    const float rc = __builtin_amdgcn_rcpf(scale);
    const bool tiny = quant_tiny(scale);            // includes s == 0
    float qf[4][4];                                 // [position i][plane p]
    bool slow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float xs[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            bool ok;
            qf[i][p] = quant_round_fast(xs[p], rc, tiny, ok);
            slow |= !ok && scale != 0.0f;
        }
    }
    if (__any(slow)) {                              // rare: the IEEE division decides
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float xs[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                bool ok;
                quant_round_fast(xs[p], rc, tiny, ok);
                if (!ok && scale != 0.0f) qf[i][p] = rintf(xs[p] / scale);
            }
        }
    }
    int t = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) w |= ((uint32_t)quant_clamp(qf[i][p], scale) & 0xffu) << (8 * i);
        word[p] = w;
        t = dot4(w, 0x01010101u, t);
    }
    t += dpp_xor1(t);
    t += dpp_xor2(t);
    t += dpp_half_mirror(t);
    sum = t;
}

// Buffer resource over [base, base + bytes) (bytes clamped to 32 bits; every
// offset used is in range by construction, the hardware range check is a
// second guard: loads beyond the range return zero). Word 3 selects 32-bit
// raw data, as for all gfx9 buffers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int n = bytes >= 0xffffffffLL ? (int)0xffffffffu : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

__device__ __forceinline__ v4i mfma16x16x64(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---- buffer -> LDS copies (gfx950: 16 bytes per lane) and their waits

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kCopyOob = 0x7ffffff0;         // buffer offset past every range: no memory access

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// One 16-byte buffer -> LDS copy per lane: lane i writes bytes
// [16 i, 16 i + 16) after lds (wave-uniform); offsets past the range write
// zeros and read no memory. Counted by vmcnt like a load. (A non-template
// function: the builtin is device-only, and a template kernel calling it
// directly gets no host-side launch stub.)
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, void *lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, voff, 0, 0, 0);
}

// The same copy from voff + soff, soff wave-uniform (an SGPR operand). A lane
// whose voff is kCopyOob stays out of range whatever soff is; in-range lanes
// must keep voff + soff inside the resource.
__device__ __forceinline__ void copy16_to_lds_at(__amdgpu_buffer_rsrc_t r, void *lds, int voff,
                                                 int soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, voff, soff, 0, 0);
}

// Block barrier after this wave's LDS accesses have completed. Without the
// release fence of __syncthreads, which would also wait for every buffer ->
// LDS copy in flight; the copies a step needs are waited for explicitly.
__device__ __forceinline__ void ring_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0); vmcnt and expcnt at their maxima
    asm volatile("s_barrier" ::: "memory");
}

}  // namespace pq2
