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
// 512-byte group is read fully coalesced); quantize_groups32 (shared with the
// fused GEMV) reduces amax and t over the 32 lanes and leaves lane 4j+s with
// the 32-bit plane word (s, j), written to byte 32*s + 4*j of the group.
//
// HBM-bound: 4 bytes read and 1 + 8/128 bytes written per element.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

constexpr int kQuantThreads = 256;
constexpr int kGroupsPerBlock = kQuantThreads / 32;

// Four activations of one lane as float32: float32 input as is; bfloat16 and
// binary16 input (FMT 1, 2) widened exactly, so the quantisation is that of
// the float32 values they represent.
template <int FMT>
__device__ __forceinline__ float4 load4(const void *x, int64_t i) {
    if constexpr (FMT == 0) {
        return *reinterpret_cast<const float4 *>(static_cast<const float *>(x) + i);
    } else {
        const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(x) + i);
        const uint32_t h[4] = {w.x & 0xffffu, w.x >> 16, w.y & 0xffffu, w.y >> 16};
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (FMT == 1)
                f[e] = __builtin_bit_cast(float, h[e] << 16);
            else
                f[e] = (float)__builtin_bit_cast(_Float16, (uint16_t)h[e]);
        }
        return make_float4(f[0], f[1], f[2], f[3]);
    }
}

template <int FMT>
__global__ __launch_bounds__(kQuantThreads) void quantize_plane_kernel(
    const void *__restrict__ x, int8_t *__restrict__ q, float *__restrict__ s,
    int32_t *__restrict__ t, int64_t MG, int64_t G, int64_t K) {
    const int lane32 = threadIdx.x & 31;
    const int64_t grp = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 5);
    const bool valid = grp < MG;
    const int64_t gg = valid ? grp : MG - 1;   // keep every lane in the shuffles
    const int64_t m = gg / G;
    const int64_t g = gg - m * G;
    const int64_t base = m * K + g * kGroup;

    const float4 v[1] = {load4<FMT>(x, base + 4 * lane32)};
    uint32_t word[1];
    float sc[1];
    int sum[1];
    quantize_groups32<1>(v, lane32, word, sc, sum);
    const int j = lane32 >> 2;        // output word j of plane sp
    const int sp = lane32 & 3;
    if (valid) {
        *reinterpret_cast<uint32_t *>(q + base + 32 * sp + 4 * j) = word[0];
        if (lane32 == 0) {
            s[gg] = sc[0];
            t[gg] = sum[0];
        }
    }
}

}  // namespace

hipError_t launch_quantize(const void *x, int format, int8_t *q, float *s, int32_t *t,
                           int64_t M, int64_t K, hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t MG = M * G;
    const int64_t blocks = (MG + kGroupsPerBlock - 1) / kGroupsPerBlock;
    if (format == 1)
        hipLaunchKernelGGL(quantize_plane_kernel<1>, dim3((unsigned)blocks), dim3(kQuantThreads),
                           0, stream, x, q, s, t, MG, G, K);
    else if (format == 2)
        hipLaunchKernelGGL(quantize_plane_kernel<2>, dim3((unsigned)blocks), dim3(kQuantThreads),
                           0, stream, x, q, s, t, MG, G, K);
    else
        hipLaunchKernelGGL(quantize_plane_kernel<0>, dim3((unsigned)blocks), dim3(kQuantThreads),
                           0, stream, x, q, s, t, MG, G, K);
    return hipGetLastError();
}

}  // namespace pq2
