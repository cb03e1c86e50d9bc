// small_mfma.hip -- K3: PQ2_0 product for 2..16 token rows on int8 MFMA.
//
// Plane dot products become arithmetic-bound from about three tokens (page
// "Making a ternary reasoning model fast in vLLM", section "One token at a
// time", last paragraph); the small-batch path instead places code bytes
// directly in the matrix-instruction operand registers and extracts each
// plane with a shift and a mask (section "Small batches: make the register
// layout explicit"), and loads every weight once for all token rows.
//
// gfx950 mapping (v_mfma_i32_16x16x64_i8, tokens padded to 16):
//  * A block owns a tile of 16 weight rows and all tokens; its NW waves split
//    the K groups between them and their float partials are summed through
//    LDS in wave order (a fixed order, so results are deterministic).
//  * Per group a lane (row/token r = lane%16, lane group lg = lane/16) loads
//    code words 2lg and 2lg+1 of row r (8 bytes) and the matching plane-order
//    activations of token r: for each plane p the 8 bytes at 32p + 8lg.
//    The A operand of MFMA h (h = 0, 1) is the four planes of code word
//    2lg+h; the B operand is the four activation words that pair with those
//    planes. The k order inside the instruction is the same function of
//    (lane group, register, byte) for A and B, so any such order is exact.
//  * The accumulator is seeded with -t[m][g], so two MFMAs give the exact
//    group dot D[n][m]; lane (lg, m) then holds rows 4lg..4lg+3 of token m and
//    applies acc += D * (s[m][g] * ws[n][g]).
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

template <int NW, bool DOTS>
__global__ __launch_bounds__(NW * kWave) void small_mfma_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    int32_t *__restrict__ d, int64_t M, int64_t N, int64_t K) {
    __shared__ float partial[DOTS ? 1 : NW][kWave][4];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15;          // A row within the tile, and B token
    const int lg = lane >> 4;         // lane group: k slice and output rows
    const int64_t G = K / kGroup;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t arow = (n0 + r < N) ? n0 + r : N - 1;
    const bool mvalid = r < M;
    const int64_t mc = mvalid ? r : M - 1;
    const int64_t g_begin = (G * wave) / NW;
    const int64_t g_end = (G * (wave + 1)) / NW;

    const uint8_t *ap = codes + arow * (K / 4) + 8 * lg;
    const int8_t *bp = q + mc * K + 8 * lg;
    int64_t orow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t n = n0 + 4 * lg + i;
        orow[i] = n < N ? n : N - 1;
    }

    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int64_t g = g_begin; g < g_end; ++g) {
        const uint2 wv = *reinterpret_cast<const uint2 *>(ap + 32 * g);
        uint2 b[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            b[p] = *reinterpret_cast<const uint2 *>(bp + kGroup * g + 32 * p);
            if (!mvalid) b[p] = make_uint2(0u, 0u);
        }
        const int tg = mvalid ? t[mc * G + g] : 0;
        float sm = 0.0f;
        uint16_t wsv[4];
        if (!DOTS) {
            sm = mvalid ? s[mc * G + g] : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) wsv[i] = ws[orow[i] * G + g];
        }
        const v4i a0 = planes_of(wv.x);
        const v4i a1 = planes_of(wv.y);
        const v4i b0 = {(int)b[0].x, (int)b[1].x, (int)b[2].x, (int)b[3].x};
        const v4i b1 = {(int)b[0].y, (int)b[1].y, (int)b[2].y, (int)b[3].y};
        v4i c = {-tg, -tg, -tg, -tg};
        c = mfma16x16x64(a0, b0, c);
        c = mfma16x16x64(a1, b1, c);
        if (DOTS) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t n = n0 + 4 * lg + i;
                if (mvalid && n < N) d[((int64_t)r * N + n) * G + g] = c[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[i] = fmaf((float)c[i], sm * half_bits_to_float(wsv[i]), acc[i]);
        }
    }

    if (!DOTS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) partial[DOTS ? 0 : wave][lane][i] = acc[i];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = partial[0][lane][i];
                for (int w = 1; w < NW; ++w) v += partial[w][lane][i];
                const int64_t n = n0 + 4 * lg + i;
                if (mvalid && n < N) y[(int64_t)r * N + n] = v;
            }
        }
    }
}

template <int NW>
hipError_t launch_nw(const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t blocks = (N + 15) / 16;
    if (out.d) {
        hipLaunchKernelGGL((small_mfma_kernel<NW, true>), dim3((unsigned)blocks),
                           dim3(NW * kWave), 0, stream, q, nullptr, t, codes, nullptr, nullptr,
                           out.d, M, N, K);
    } else {
        hipLaunchKernelGGL((small_mfma_kernel<NW, false>), dim3((unsigned)blocks),
                           dim3(NW * kWave), 0, stream, q, out.s, t, codes, out.ws, out.y,
                           nullptr, M, N, K);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_small(const int8_t *q, const int32_t *t, const uint8_t *codes,
                        const GemmOut &out, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
    // Split K over enough waves that the grid holds ~16 waves per CU, but give
    // every wave at least two groups.
    const int64_t G = K / kGroup;
    const int64_t tiles = (N + 15) / 16;
    int64_t nw = (4096 + tiles - 1) / tiles;
    if (nw > G / 2) nw = G / 2;
    if (nw >= 16) return launch_nw<16>(q, t, codes, out, M, N, K, stream);
    if (nw >= 8) return launch_nw<8>(q, t, codes, out, M, N, K, stream);
    if (nw >= 4) return launch_nw<4>(q, t, codes, out, M, N, K, stream);
    if (nw >= 2) return launch_nw<2>(q, t, codes, out, M, N, K, stream);
    return launch_nw<1>(q, t, codes, out, M, N, K, stream);
}

}  // namespace pq2
