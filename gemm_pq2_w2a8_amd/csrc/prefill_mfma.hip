// prefill_mfma.hip -- K4: tiled int8 MFMA GEMM for the PQ2_0 product at
// M >= 17 (prompt processing).
//
// Per group the work is a dense int8 contraction. As on the page "Making a
// ternary reasoning model fast in vLLM" (section "Prompt processing: check
// configuration and launch costs"), each 128-group is consumed as masked
// 2-bit planes of the code words against plane-order activations, with the
// -sum(q) correction, followed by the float32 scale epilogue; the page's
// kernels used 2-D tiles of 128 x 128 or 256 x 64 ("What did not work":
// four masked K=32 dots per group beat one K=128 dot on reshaped planes).
//
// gfx950 mapping:
//  * A block has WAVES_N x WAVES_M waves; a wave owns WN x WM tiles of
//    v_mfma_i32_16x16x64_i8 (16 weight rows x 16 tokens each), so the block
//    tile is (16*WN*WAVES_N) weight rows x (16*WM*WAVES_M) tokens.
//  * Operand layout (as in the small-batch kernel): lane (r = lane%16,
//    lg = lane/16) of a 16-row tile holds code words 4*(lg&1)..+3 of row r;
//    MFMA a (a = 0, 1) takes plane 2a + (lg>>1) of those words (shift + mask)
//    as A and the 16 plane-order activation bytes that pair with them as B
//    (one 16-byte LDS read). The accumulator is seeded with -t, so the two
//    MFMAs give the exact group dot; the float32 epilogue
//    acc += D * (s[m] * ws[n]) follows per group.
//  * Per group the block stages codes, activations and the group's scales
//    in LDS, double buffered: the global loads of group g+1 are in flight
//    while group g is computed, with one barrier per group.
//  * Tiles are numbered so that each XCD (blocks are dealt round-robin over
//    the 8 XCDs) gets a contiguous run of tiles along N for the same token
//    panel, which then stays in that XCD's L2.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

constexpr int kCodeStride = 48;          // LDS bytes per code row (32 + pad)
constexpr int kQStride = 144;            // LDS bytes per token row (128 + pad)
constexpr int kNumXcd = 8;

// Bijection from dispatch order to tile order: dispatch slot b runs on XCD
// b % 8; XCD x receives the x-th contiguous run of tile numbers.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t nb) {
    const int64_t xcd = b % kNumXcd, idx = b / kNumXcd;
    const int64_t per = nb / kNumXcd, rem = nb % kNumXcd;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

template <int WN, int WM, int WAVES_N, int WAVES_M>
struct PfCfg {
    static constexpr int kThreads = 64 * WAVES_N * WAVES_M;
    static constexpr int BN = 16 * WN * WAVES_N;
    static constexpr int BM = 16 * WM * WAVES_M;
    static constexpr int kCodeChunks = BN * 2;          // 16-byte chunks of codes per group
    static constexpr int kQChunks = BM * 8;             // 16-byte chunks of q per group
    static constexpr int kCodePer = (kCodeChunks + kThreads - 1) / kThreads;
    static constexpr int kQPer = (kQChunks + kThreads - 1) / kThreads;
    struct __align__(16) Stage {
        uint8_t codes[BN * kCodeStride];
        int8_t q[BM * kQStride];
        uint16_t ws[BN];
        float s[BM];
        int32_t t[BM];
    };
};

template <int WN, int WM, int WAVES_N, int WAVES_M, bool DOTS>
__global__ __launch_bounds__(64 * WAVES_N * WAVES_M) void prefill_mfma_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    int32_t *__restrict__ d, int64_t M, int64_t N, int64_t K) {
    using C = PfCfg<WN, WM, WAVES_N, WAVES_M>;
    using Stage = typename C::Stage;
    __shared__ Stage stage[2];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wn = wave % WAVES_N, wm = wave / WAVES_N;
    const int r = lane & 15, lg = lane >> 4;
    const int half = lg & 1;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);

    const int64_t tiles_n = (N + C::BN - 1) / C::BN;
    const int64_t tiles_m = (M + C::BM - 1) / C::BM;
    const int64_t tile = xcd_tile(blockIdx.x, tiles_n * tiles_m);
    const int64_t n0 = (tile % tiles_n) * C::BN;
    const int64_t m0 = (tile / tiles_n) * C::BM;

    // staging assignment: chunk c of codes is (row c/2, half c%2); chunk c of q
    // is (token c/8, 16-byte piece c%8)
    const uint4 *code_src[C::kCodePer];
    int code_dst[C::kCodePer];
#pragma unroll
    for (int i = 0; i < C::kCodePer; ++i) {
        int c = tid + i * C::kThreads;
        if (c >= C::kCodeChunks) c = C::kCodeChunks - 1;
        const int row = c >> 1, hh = c & 1;
        const int64_t gn = (n0 + row < N) ? n0 + row : N - 1;
        code_src[i] = reinterpret_cast<const uint4 *>(codes + gn * (K / 4) + 16 * hh);
        code_dst[i] = row * kCodeStride + 16 * hh;
    }
    const uint4 *q_src[C::kQPer];
    int q_dst[C::kQPer];
#pragma unroll
    for (int i = 0; i < C::kQPer; ++i) {
        int c = tid + i * C::kThreads;
        if (c >= C::kQChunks) c = C::kQChunks - 1;
        const int tok = c >> 3, piece = c & 7;
        const int64_t gm = (m0 + tok < M) ? m0 + tok : M - 1;
        q_src[i] = reinterpret_cast<const uint4 *>(q + gm * K + 16 * piece);
        q_dst[i] = tok * kQStride + 16 * piece;
    }

    // Staging loads and LDS writes are never predicated on g (the step after
    // the last group re-reads the last group into the idle buffer), which
    // keeps the staging registers out of scratch memory.
    constexpr bool kCodeRagged = (C::kCodeChunks % C::kThreads) != 0;
    constexpr bool kQRagged = (C::kQChunks % C::kThreads) != 0;
    const int64_t sn = (n0 + tid < N) ? n0 + tid : N - 1;     // ws row of this thread
    const int64_t sm = (m0 + tid < M) ? m0 + tid : M - 1;     // s/t token of this thread
#define PQ2_PF_FETCH(g)                                                             \
    do {                                                                          \
        _Pragma("unroll") for (int i = 0; i < C::kCodePer; ++i) rc[i] = code_src[i][2 * (g)]; \
        _Pragma("unroll") for (int i = 0; i < C::kQPer; ++i) rq[i] = q_src[i][8 * (g)];       \
        if (!DOTS && tid < C::BN) rws = ws[sn * G + (g)];                         \
        if (tid < C::BM) {                                                        \
            rt = t[sm * G + (g)];                                                 \
            if (!DOTS) rs_ = s[sm * G + (g)];                                     \
        }                                                                         \
    } while (0)
#define PQ2_PF_COMMIT(st)                                                           \
    do {                                                                          \
        _Pragma("unroll") for (int i = 0; i < C::kCodePer; ++i)                   \
            if (!kCodeRagged || tid + i * C::kThreads < C::kCodeChunks)           \
                *reinterpret_cast<uint4 *>((st).codes + code_dst[i]) = rc[i];     \
        _Pragma("unroll") for (int i = 0; i < C::kQPer; ++i)                      \
            if (!kQRagged || tid + i * C::kThreads < C::kQChunks)                 \
                *reinterpret_cast<uint4 *>((st).q + q_dst[i]) = rq[i];            \
        if (!DOTS && tid < C::BN) (st).ws[tid] = rws;                             \
        if (tid < C::BM) {                                                        \
            (st).t[tid] = rt;                                                     \
            if (!DOTS) (st).s[tid] = rs_;                                         \
        }                                                                         \
    } while (0)

    uint4 rc[C::kCodePer], rq[C::kQPer];
    uint16_t rws = 0;
    float rs_ = 0.0f;
    int32_t rt = 0;

    float acc[WN][WM][4];
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
        for (int b = 0; b < WM; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;

    PQ2_PF_FETCH(0);
    PQ2_PF_COMMIT(stage[0]);
    __syncthreads();

    const int row_base = 16 * WN * wn;     // wave's first row within the block tile
    const int tok_base = 16 * WM * wm;     // wave's first token within the block tile
    for (int g = 0; g < G; ++g) {
        const Stage &cur = stage[g & 1];
        const int gn1 = g + 1 < G ? g + 1 : g;
        PQ2_PF_FETCH(gn1);

        // A operands (and weight scales) of the wave's WN row tiles
        v4i a0[WN], a1[WN];
        float wsf[WN][4];
#pragma unroll
        for (int a = 0; a < WN; ++a) {
            const uint4 w = *reinterpret_cast<const uint4 *>(
                cur.codes + (row_base + 16 * a + r) * kCodeStride + 16 * half);
            const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t sh = wv[j] >> sh0;
                a0[a][j] = (int)(sh & kPlaneMask);
                a1[a][j] = (int)((sh >> 4) & kPlaneMask);
            }
            if (!DOTS) {
                const uint2 wsw = *reinterpret_cast<const uint2 *>(cur.ws + row_base + 16 * a + 4 * lg);
                wsf[a][0] = half_bits_to_float((uint16_t)(wsw.x & 0xffff));
                wsf[a][1] = half_bits_to_float((uint16_t)(wsw.x >> 16));
                wsf[a][2] = half_bits_to_float((uint16_t)(wsw.y & 0xffff));
                wsf[a][3] = half_bits_to_float((uint16_t)(wsw.y >> 16));
            }
        }
#pragma unroll
        for (int b = 0; b < WM; ++b) {
            const int tok = tok_base + 16 * b + r;
            const int8_t *qrow = cur.q + tok * kQStride + 16 * half + 16 * sh0;
            const uint4 q0 = *reinterpret_cast<const uint4 *>(qrow);
            const uint4 q1 = *reinterpret_cast<const uint4 *>(qrow + 64);
            const v4i b0 = {(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w};
            const v4i b1 = {(int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
            const int tneg = -cur.t[tok];
            const float sv = cur.s[tok];
#pragma unroll
            for (int a = 0; a < WN; ++a) {
                v4i c = {tneg, tneg, tneg, tneg};
                c = mfma16x16x64(a0[a], b0, c);
                c = mfma16x16x64(a1[a], b1, c);
                if (DOTS) {
                    const int64_t m = m0 + tok;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + row_base + 16 * a + 4 * lg + i;
                        if (m < M && n < N) d[(m * N + n) * G + g] = c[i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[a][b][i] = fmaf((float)c[i], sv * wsf[a][i], acc[a][b][i]);
                }
            }
        }

        PQ2_PF_COMMIT(stage[(g + 1) & 1]);
        __syncthreads();
    }
#undef PQ2_PF_FETCH
#undef PQ2_PF_COMMIT

    if (!DOTS) {
#pragma unroll
        for (int b = 0; b < WM; ++b) {
            const int64_t m = m0 + tok_base + 16 * b + r;
#pragma unroll
            for (int a = 0; a < WN; ++a) {
                const int64_t nb = n0 + row_base + 16 * a + 4 * lg;
                if (m < M) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (nb + i < N) y[m * N + nb + i] = acc[a][b][i];
                }
            }
        }
    }
}

template <int WN, int WM, int WAVES_N, int WAVES_M>
hipError_t launch_cfg(const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
    using C = PfCfg<WN, WM, WAVES_N, WAVES_M>;
    const int64_t blocks = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
    if (out.d) {
        hipLaunchKernelGGL((prefill_mfma_kernel<WN, WM, WAVES_N, WAVES_M, true>),
                           dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, q, nullptr, t,
                           codes, nullptr, nullptr, out.d, M, N, K);
    } else {
        hipLaunchKernelGGL((prefill_mfma_kernel<WN, WM, WAVES_N, WAVES_M, false>),
                           dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, q, out.s, t,
                           codes, out.ws, out.y, nullptr, M, N, K);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const int8_t *q, const int32_t *t, const uint8_t *codes,
                          const GemmOut &out, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream) {
    // Largest tile that still gives every CU at least one block.
    auto tiles = [&](int64_t bn, int64_t bm) { return ((N + bn - 1) / bn) * ((M + bm - 1) / bm); };
    constexpr int64_t kCUs = 256;
    if (tiles(128, 128) >= kCUs)
        return launch_cfg<4, 4, 2, 2>(q, t, codes, out, M, N, K, stream);   // 128 x 128
    if (tiles(64, 128) >= kCUs)
        return launch_cfg<2, 4, 2, 2>(q, t, codes, out, M, N, K, stream);   // 64 x 128
    return launch_cfg<1, 4, 2, 2>(q, t, codes, out, M, N, K, stream);       // 32 x 128
}

}  // namespace pq2
