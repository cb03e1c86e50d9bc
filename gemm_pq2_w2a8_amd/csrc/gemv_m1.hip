// gemv_m1.hip -- K2: the M = 1 PQ2_0 GEMV on v_dot4.
//
// Algorithm (page "Making a ternary reasoning model fast in vLLM", section
// "One token at a time: plain Triton is enough"): activations are in plane
// order, so plane s of a 32-bit code word -- the 2-bit fields at bits 2s of
// its four bytes -- lines up with four consecutive activation bytes and one
// int8 dot4 consumes them with no decode step; the -1 offset of the ternary
// code is one subtraction of sum(q) per 128-weight group; the group dot is
// then scaled by s[g] * ws[n][g] in float32 and summed over groups.
//
// gfx950 mapping:
//  * A "chunk" is 16 bytes of one row = 4 code words = half a group. A wave
//    splits into RL = 64/CL row slots of CL lanes; lane cs of a slot handles
//    chunks cs, cs+CL, cs+2CL, ... of RP rows. CL = gcd(K/64, 64), so every
//    lane is busy on every iteration and each load instruction covers RL
//    contiguous segments of CL*16 bytes (coalesced HBM streaming).
//  * The 16 plane-order q words of a chunk are loaded once per iteration and
//    reused for the RP rows; q is K bytes and stays in cache.
//  * Planes 0 and 2 are masked to bits 0..1 (after one shift by 4 for plane
//    2); planes 1 and 3 are masked in place at bits 2..3, which is 4 * code.
//    They go to a second accumulator that is divided by 4 (exactly) before
//    the two are added: five bit operations and four v_dot4 per code word.
//  * The even lane of a chunk pair seeds its accumulator with -t[g]; the two
//    half-group sums meet through a DPP lane swap, giving the exact group dot
//    on both lanes. The even lane applies the float32 epilogue.
//  * Rows are reduced over their CL lanes with a fixed butterfly at the end.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;

template <int LOG_CL, int RP, bool DOTS>
__global__ __launch_bounds__(kGemvThreads) void gemv_m1_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    int32_t *__restrict__ d, int64_t N, int64_t K) {
    constexpr int CL = 1 << LOG_CL;
    constexpr int RL = kWave / CL;
    constexpr int ROWS_PER_WAVE = RL * RP;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int cs = lane & (CL - 1);
    const int rs = lane >> LOG_CL;
    const int h = cs & 1;                       // half of the group this lane holds
    const int64_t G = K / kGroup;
    const int64_t row_bytes = K / 4;
    const int64_t iters = (K / 64) / CL;
    const int64_t row0 = ((int64_t)blockIdx.x * kGemvWaves + wave) * ROWS_PER_WAVE + rs;

    const uint8_t *rowp[RP];
    int64_t rowc[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int64_t row = row0 + (int64_t)r * RL;
        rowc[r] = row < N ? row : N - 1;
        rowp[r] = codes + rowc[r] * row_bytes;
    }

    float facc[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) facc[r] = 0.0f;

    for (int64_t it = 0; it < iters; ++it) {
        const int64_t c = cs + (int64_t)CL * it;
        const int64_t g = c >> 1;
        // plane-order activations of this half group: plane p at +32p bytes
        const uint4 *qp = reinterpret_cast<const uint4 *>(q + kGroup * g + 16 * h);
        const uint4 q0 = qp[0], q1 = qp[2], q2 = qp[4], q3 = qp[6];
        const int tg = t[g];
        float sg = 0.0f;
        if (!DOTS) sg = s[g];

        uint4 w[RP];
        uint16_t wsv[RP];
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            w[r] = reinterpret_cast<const uint4 *>(rowp[r])[c];
            if (!DOTS) wsv[r] = ws[rowc[r] * G + g];
        }
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            int da = h ? 0 : -tg;   // planes 0 and 2, and the -sum(q) offset
            int db = 0;             // planes 1 and 3, in place: 4 * (their dot)
            const uint32_t wr[4] = {w[r].x, w[r].y, w[r].z, w[r].w};
            const uint32_t p0[4] = {q0.x, q0.y, q0.z, q0.w};
            const uint32_t p1[4] = {q1.x, q1.y, q1.z, q1.w};
            const uint32_t p2[4] = {q2.x, q2.y, q2.z, q2.w};
            const uint32_t p3[4] = {q3.x, q3.y, q3.z, q3.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const uint32_t wd = wr[jj];
                const uint32_t hi = wd >> 4;
                da = dot4(wd & kPlaneMask, p0[jj], da);
                db = dot4(wd & kPlaneMaskX4, p1[jj], db);
                da = dot4(hi & kPlaneMask, p2[jj], da);
                db = dot4(hi & kPlaneMaskX4, p3[jj], db);
            }
            const int half_dot = da + (db >> 2);          // db is a multiple of 4
            const int dot = half_dot + dpp_xor1(half_dot);  // exact group dot
            if (DOTS) {
                const int64_t row = row0 + (int64_t)r * RL;
                if (!h && row < N) d[row * G + g] = dot;
            } else {
                const float coef = h ? 0.0f : sg * half_bits_to_float(wsv[r]);
                facc[r] = fmaf((float)dot, coef, facc[r]);
            }
        }
    }

    if (!DOTS) {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const float v = segment_sum<CL>(facc[r]);
            const int64_t row = row0 + (int64_t)r * RL;
            if (cs == 0 && row < N) y[row] = v;
        }
    }
}

template <int LOG_CL, int RP>
hipError_t launch_cfg(const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t N, int64_t K, hipStream_t stream) {
    constexpr int rows_per_block = kGemvWaves * (kWave >> LOG_CL) * RP;
    const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
    if (out.d) {
        hipLaunchKernelGGL((gemv_m1_kernel<LOG_CL, RP, true>), dim3((unsigned)blocks),
                           dim3(kGemvThreads), 0, stream, q, nullptr, t, codes, nullptr,
                           nullptr, out.d, N, K);
    } else {
        hipLaunchKernelGGL((gemv_m1_kernel<LOG_CL, RP, false>), dim3((unsigned)blocks),
                           dim3(kGemvThreads), 0, stream, q, out.s, t, codes, out.ws, out.y,
                           nullptr, N, K);
    }
    return hipGetLastError();
}

template <int LOG_CL>
hipError_t launch_rp(const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, int64_t N, int64_t K, hipStream_t stream) {
    // Two rows per lane once the grid has enough waves to keep every CU busy.
    const int64_t waves_rp1 = (N + (kWave >> LOG_CL) - 1) / (kWave >> LOG_CL);
    if (waves_rp1 >= 4096) return launch_cfg<LOG_CL, 2>(q, t, codes, out, N, K, stream);
    return launch_cfg<LOG_CL, 1>(q, t, codes, out, N, K, stream);
}

}  // namespace

hipError_t launch_gemv_m1(const int8_t *q, const int32_t *t, const uint8_t *codes,
                          const GemmOut &out, int64_t N, int64_t K, hipStream_t stream) {
    // chunk lanes per row: the largest power of two <= 64 dividing K/64
    const int64_t chunks = K / 64;
    int64_t cl = chunks & -chunks;
    if (cl > 64) cl = 64;
    switch (cl) {
        case 2: return launch_rp<1>(q, t, codes, out, N, K, stream);
        case 4: return launch_rp<2>(q, t, codes, out, N, K, stream);
        case 8: return launch_rp<3>(q, t, codes, out, N, K, stream);
        case 16: return launch_rp<4>(q, t, codes, out, N, K, stream);
        case 32: return launch_rp<5>(q, t, codes, out, N, K, stream);
        default: return launch_rp<6>(q, t, codes, out, N, K, stream);
    }
}

}  // namespace pq2
