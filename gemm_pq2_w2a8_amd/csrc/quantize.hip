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
// Mapping: 32 lanes per group (lane b loads x[4b .. 4b+3]; quantize_groups32
// leaves lane 4j+p with the plane word (p, j)) for launches of few groups, 8
// lanes per group (lane j loads x[16j .. 16j+15]; quantize_groups8, shared
// with the fused GEMV, leaves lane j with the four plane words (p, j)) for
// many. Each plane word goes to bytes 32*p + 4*j of its group.
//
// HBM-bound: 4 bytes read and 1 + 8/128 bytes written per element.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

constexpr int kQuantThreads = 256;

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

// LANES = 32 or 8 lanes per group (quantize_groups32 / quantize_groups8).
template <int FMT, int LANES>
__global__ __launch_bounds__(kQuantThreads) void quantize_plane_kernel(
    const void *__restrict__ x, int8_t *__restrict__ q, float *__restrict__ s,
    int32_t *__restrict__ t, int64_t MG, int64_t G, int64_t K) {
    constexpr int kGroupsPerBlock = kQuantThreads / LANES;
    const int lane = threadIdx.x & (LANES - 1);
    const int64_t grp = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x / LANES);
    const bool valid = grp < MG;
    const int64_t gg = valid ? grp : MG - 1;   // keep every lane in the lane exchanges
    const int64_t m = gg / G;
    const int64_t g = gg - m * G;
    const int64_t base = m * K + g * kGroup;

    if constexpr (LANES == 32) {
        const float4 v[1] = {load4<FMT>(x, base + 4 * lane)};
        uint32_t word[1];
        float sc[1];
        int sum[1];
        quantize_groups32<1>(v, lane, word, sc, sum);
        if (valid) {
            // plane word (lane & 3, lane >> 2): bytes 32 (lane & 3) + 4 (lane >> 2)
            *reinterpret_cast<uint32_t *>(q + base + 32 * (lane & 3) + 4 * (lane >> 2)) = word[0];
            if (lane == 0) {
                s[gg] = sc[0];
                t[gg] = sum[0];
            }
        }
    } else {
        float4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = load4<FMT>(x, base + 16 * lane + 4 * i);
        uint32_t word[4];
        float sc;
        int sum;
        quantize_groups8(v, word, sc, sum);
        if (valid) {
            // plane p, positions 4 lane .. 4 lane + 3: bytes 32 p + 4 lane
#pragma unroll
            for (int p = 0; p < 4; ++p)
                *reinterpret_cast<uint32_t *>(q + base + 32 * p + 4 * lane) = word[p];
            if (lane == 0) {
                s[gg] = sc;
                t[gg] = sum;
            }
        }
    }
}

// Lanes per group (MI355X, us per launch, x resident): 32 while a launch has
// few groups, where each lane's short chain decides (K = 5120: M = 1 1.96
// against 2.40 with 8 lanes, M = 128 2.46 against 2.80, M = 256 (10240
// groups) 2.99 against 3.29), 8 from 16384 groups on, where the per-group work
// is the cost (M = 512 (20480 groups) 3.87 against 4.35; M = 4096 16.7
// against 20.3).
constexpr int64_t kQuant8MinGroups = 16384;

template <int FMT>
void launch_fmt(const void *x, int8_t *q, float *s, int32_t *t, int64_t MG, int64_t G, int64_t K,
                hipStream_t stream) {
    if (MG >= kQuant8MinGroups) {
        const int64_t blocks = (MG + kQuantThreads / 8 - 1) / (kQuantThreads / 8);
        hipLaunchKernelGGL((quantize_plane_kernel<FMT, 8>), dim3((unsigned)blocks),
                           dim3(kQuantThreads), 0, stream, x, q, s, t, MG, G, K);
    } else {
        const int64_t blocks = (MG + kQuantThreads / 32 - 1) / (kQuantThreads / 32);
        hipLaunchKernelGGL((quantize_plane_kernel<FMT, 32>), dim3((unsigned)blocks),
                           dim3(kQuantThreads), 0, stream, x, q, s, t, MG, G, K);
    }
}

}  // namespace

hipError_t launch_quantize(const void *x, int format, int8_t *q, float *s, int32_t *t,
                           int64_t M, int64_t K, hipStream_t stream) {
    const int64_t G = K / kGroup;
    const int64_t MG = M * G;
    if (format == 1)
        launch_fmt<1>(x, q, s, t, MG, G, K, stream);
    else if (format == 2)
        launch_fmt<2>(x, q, s, t, MG, G, K, stream);
    else
        launch_fmt<0>(x, q, s, t, MG, G, K, stream);
    return hipGetLastError();
}

}  // namespace pq2
