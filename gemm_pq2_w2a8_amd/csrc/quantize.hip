// quantize.hip -- K1: per-128-group int8 activation quantisation fused with the
// plane-order permutation.
//
// Per (row m, group g): amax = max|x|, s = amax / 127, q = clamp(rne(x / s),
// -127, 127), t = sum q; q is written in plane order (byte 32*s + b of the
// group holds the activation of weight 4*b + s). The buffers are those the
// page "Making a ternary reasoning model fast in vLLM" lists for its
// quantiser (section "Prompt processing: check configuration and launch
// costs"); the plane layout is from its section "One token at a time".
//
// Mapping: 32 lanes per group, lane b loads x[4b .. 4b+3] as one float4 (the
// 512-byte group is read fully coalesced). amax and t are butterfly
// reductions over the 32 lanes. Lane b then holds the four plane bytes of
// column b; a 4x4 byte transpose between lanes 4j..4j+3 gives lane 4j+s the
// 32-bit plane word (s, j), written to byte 32*s + 4*j of the group.
//
// HBM-bound: 4 bytes read and 1 + 8/128 bytes written per element.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kGroupsPerBlock = kQuantThreads / 32;

__device__ __forceinline__ int quantize_one(float x, float sc) {
    if (sc == 0.0f) return 0;
    float r = rintf(x / sc);          // IEEE division, round half to even
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__global__ __launch_bounds__(kQuantThreads) void quantize_plane_kernel(
    const float *__restrict__ x, int8_t *__restrict__ q, float *__restrict__ s,
    int32_t *__restrict__ t, int64_t MG, int64_t G, int64_t K) {
    const int lane32 = threadIdx.x & 31;
    const int64_t grp = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 5);
    const bool valid = grp < MG;
    const int64_t gg = valid ? grp : MG - 1;   // keep every lane in the shuffles
    const int64_t m = gg / G;
    const int64_t g = gg - m * G;
    const int64_t base = m * K + g * kGroup;

    const float4 v = *reinterpret_cast<const float4 *>(x + base + 4 * lane32);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
    for (int off = 16; off; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 32));
    const float sc = a / 127.0f;

    const int q0 = quantize_one(v.x, sc);
    const int q1 = quantize_one(v.y, sc);
    const int q2 = quantize_one(v.z, sc);
    const int q3 = quantize_one(v.w, sc);
    int sum = q0 + q1 + q2 + q3;
#pragma unroll
    for (int off = 16; off; off >>= 1) sum += __shfl_xor(sum, off, 32);

    // byte s of u = q of column 4*lane32 + s, i.e. plane s, position lane32
    const uint32_t u = (uint32_t)(q0 & 0xff) | ((uint32_t)(q1 & 0xff) << 8) |
                       ((uint32_t)(q2 & 0xff) << 16) | ((uint32_t)(q3 & 0xff) << 24);
    const int j = lane32 >> 2;        // output word j of plane sp
    const int sp = lane32 & 3;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t other = (uint32_t)__shfl((int)u, 4 * j + i, 32);
        word |= ((other >> (8 * sp)) & 0xffu) << (8 * i);
    }
    if (valid) {
        *reinterpret_cast<uint32_t *>(q + base + 32 * sp + 4 * j) = word;
        if (lane32 == 0) {
            s[gg] = sc;
            t[gg] = sum;
        }
    }
}

}  // namespace

hipError_t launch_quantize(const float *x, int8_t *q, float *s, int32_t *t, int64_t M,
                           int64_t K, hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t MG = M * G;
    const int64_t blocks = (MG + kGroupsPerBlock - 1) / kGroupsPerBlock;
    hipLaunchKernelGGL(quantize_plane_kernel, dim3((unsigned)blocks), dim3(kQuantThreads), 0,
                       stream, x, q, s, t, MG, G, K);
    return hipGetLastError();
}

}  // namespace pq2
