// prefill_mfma.hip -- K4: tiled int8 MFMA GEMM for the PQ2_0 product at
// M >= 17 (prompt processing).
//
// Per group the work is a dense int8 contraction. As on the page "Making a
// ternary reasoning model fast in vLLM" (section "Prompt processing: check
// configuration and launch costs"), each 128-group is consumed as masked
// 2-bit planes of the code words against plane-order activations, with the
// -sum(q) correction, followed by the float32 scale epilogue; the page's
// kernels used 2-D tiles of 128 x 128 or 256 x 64.
//
// gfx950 mapping:
//  * 256 threads = 4 waves; block tile 128 weight rows x 128 tokens; each
//    wave owns 64 x 64 = 4 x 4 tiles of v_mfma_i32_16x16x64_i8.
//  * Per group, codes (128 x 32 B) and activations (128 x 128 B), plus the
//    group's weight scales and token s/t, are staged in LDS, double
//    buffered: the global loads of group g+1 are in flight while group g is
//    computed, with one barrier per group.
//  * A operands: the four 2-bit planes of one code word (shift + mask);
//    B operands: the matching plane-order activation words. The accumulator
//    is seeded with -t, so two MFMAs give the exact group dot; the float32
//    epilogue acc += D * (s[m] * ws[n]) follows per group.
//  * Tiles are numbered so that each XCD (blocks are dealt round-robin over
//    the 8 XCDs) gets a contiguous run of tiles along N for the same token
//    panel, which then stays in that XCD's L2.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

constexpr int kPfThreads = 256;
constexpr int kBN = 128;                 // weight rows per block
constexpr int kBM = 128;                 // tokens per block
constexpr int kCodeStride = 40;          // LDS bytes per code row (32 + pad)
constexpr int kQStride = 136;            // LDS bytes per token row (128 + pad)
constexpr int kNumXcd = 8;

struct __align__(16) PfStage {
    uint8_t codes[kBN * kCodeStride];
    int8_t q[kBM * kQStride];
    uint16_t ws[kBN];
    float s[kBM];
    int32_t t[kBM];
};

// Bijection from dispatch order to tile order: dispatch slot b runs on XCD
// b % 8; XCD x receives the x-th contiguous run of tile numbers.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t nb) {
    const int64_t xcd = b % kNumXcd, idx = b / kNumXcd;
    const int64_t per = nb / kNumXcd, rem = nb % kNumXcd;
    return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

template <bool DOTS>
__global__ __launch_bounds__(kPfThreads) void prefill_mfma_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    int32_t *__restrict__ d, int64_t M, int64_t N, int64_t K) {
    __shared__ PfStage stage[2];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wn = wave & 1, wm = wave >> 1;
    const int r = lane & 15, lg = lane >> 4;
    const int64_t G = K / kGroup;

    const int64_t tiles_n = (N + kBN - 1) / kBN;
    const int64_t tiles_m = (M + kBM - 1) / kBM;
    const int64_t tile = xcd_tile(blockIdx.x, tiles_n * tiles_m);
    const int64_t n0 = (tile % tiles_n) * kBN;
    const int64_t m0 = (tile / tiles_n) * kBM;

    // global -> LDS staging assignment (row/token = tid / 2, half = tid % 2)
    const int srow = tid >> 1, shalf = tid & 1;
    const int64_t gn = (n0 + srow < N) ? n0 + srow : N - 1;
    const int64_t gm = (m0 + srow < M) ? m0 + srow : M - 1;
    const uint8_t *code_src = codes + gn * (K / 4) + 16 * shalf;
    const int8_t *q_src = q + gm * K + 64 * shalf;
    // scales: threads 0..127 fetch ws of rows, 128..255 fetch s/t of tokens
    const int sidx = tid & 127;
    const int64_t sn = (n0 + sidx < N) ? n0 + sidx : N - 1;
    const int64_t sm = (m0 + sidx < M) ? m0 + sidx : M - 1;

    uint4 rc, rq[4];
    uint16_t rws = 0;
    float rs_ = 0.0f;
    int32_t rt = 0;
    auto fetch = [&](int64_t g) {
        rc = *reinterpret_cast<const uint4 *>(code_src + 32 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            rq[i] = *reinterpret_cast<const uint4 *>(q_src + kGroup * g + 16 * i);
        if (tid < 128) {
            if (!DOTS) rws = ws[sn * G + g];
        } else {
            rt = t[sm * G + g];
            if (!DOTS) rs_ = s[sm * G + g];
        }
    };
    auto commit = [&](PfStage &st) {
        uint2 *cdst = reinterpret_cast<uint2 *>(st.codes + srow * kCodeStride + 16 * shalf);
        cdst[0] = make_uint2(rc.x, rc.y);
        cdst[1] = make_uint2(rc.z, rc.w);
        uint2 *qdst = reinterpret_cast<uint2 *>(st.q + srow * kQStride + 64 * shalf);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qdst[2 * i] = make_uint2(rq[i].x, rq[i].y);
            qdst[2 * i + 1] = make_uint2(rq[i].z, rq[i].w);
        }
        if (tid < 128) {
            st.ws[sidx] = rws;
        } else {
            st.s[sidx] = rs_;
            st.t[sidx] = rt;
        }
    };

    float acc[4][4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;

    fetch(0);
    commit(stage[0]);
    __syncthreads();

    for (int64_t g = 0; g < G; ++g) {
        PfStage &cur = stage[g & 1];
        if (g + 1 < G) fetch(g + 1);

        // B operands and token scalars for the wave's four token blocks
        v4i b0[4], b1[4];
        int tneg[4];
        float sv[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int tok = 64 * wm + 16 * b + r;
            uint2 qq[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
                qq[p] = *reinterpret_cast<const uint2 *>(cur.q + tok * kQStride + 32 * p + 8 * lg);
            b0[b] = v4i{(int)qq[0].x, (int)qq[1].x, (int)qq[2].x, (int)qq[3].x};
            b1[b] = v4i{(int)qq[0].y, (int)qq[1].y, (int)qq[2].y, (int)qq[3].y};
            const int otok = 64 * wm + 16 * b + r;   // D column = token r of block b
            tneg[b] = -cur.t[otok];
            sv[b] = cur.s[otok];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int row = 64 * wn + 16 * a + r;
            const uint2 wv = *reinterpret_cast<const uint2 *>(cur.codes + row * kCodeStride + 8 * lg);
            const v4i a0 = planes_of(wv.x);
            const v4i a1 = planes_of(wv.y);
            const int orow = 64 * wn + 16 * a + 4 * lg;   // D rows orow .. orow+3
            float wsf[4];
            if (!DOTS) {
                const uint2 wsw = *reinterpret_cast<const uint2 *>(cur.ws + orow);
                wsf[0] = half_bits_to_float((uint16_t)(wsw.x & 0xffff));
                wsf[1] = half_bits_to_float((uint16_t)(wsw.x >> 16));
                wsf[2] = half_bits_to_float((uint16_t)(wsw.y & 0xffff));
                wsf[3] = half_bits_to_float((uint16_t)(wsw.y >> 16));
            }
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                v4i c = {tneg[b], tneg[b], tneg[b], tneg[b]};
                c = mfma16x16x64(a0, b0[b], c);
                c = mfma16x16x64(a1, b1[b], c);
                if (DOTS) {
                    const int64_t m = m0 + 64 * wm + 16 * b + r;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + orow + i;
                        if (m < M && n < N) d[(m * N + n) * G + g] = c[i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[a][b][i] = fmaf((float)c[i], sv[b] * wsf[i], acc[a][b][i]);
                }
            }
        }

        if (g + 1 < G) commit(stage[(g + 1) & 1]);
        __syncthreads();
    }

    if (!DOTS) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int64_t m = m0 + 64 * wm + 16 * b + r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t n = n0 + 64 * wn + 16 * a + 4 * lg + i;
                    if (m < M && n < N) y[m * N + n] = acc[a][b][i];
                }
            }
    }
}

}  // namespace

hipError_t launch_prefill(const int8_t *q, const int32_t *t, const uint8_t *codes,
                          const GemmOut &out, int64_t M, int64_t N, int64_t K,
                          hipStream_t stream) {
    const int64_t blocks = ((N + kBN - 1) / kBN) * ((M + kBM - 1) / kBM);
    if (out.d) {
        hipLaunchKernelGGL(prefill_mfma_kernel<true>, dim3((unsigned)blocks), dim3(kPfThreads),
                           0, stream, q, nullptr, t, codes, nullptr, nullptr, out.d, M, N, K);
    } else {
        hipLaunchKernelGGL(prefill_mfma_kernel<false>, dim3((unsigned)blocks), dim3(kPfThreads),
                           0, stream, q, out.s, t, codes, out.ws, out.y, nullptr, M, N, K);
    }
    return hipGetLastError();
}

}  // namespace pq2
