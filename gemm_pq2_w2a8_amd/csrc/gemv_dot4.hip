// gemv_dot4.hip -- K2: the PQ2_0 GEMV on v_dot4 for 1 to 4 token rows.
//
// Algorithm (page "Making a ternary reasoning model fast in vLLM", section
// "One token at a time: plain Triton is enough"): activations are in plane
// order, so plane s of a 32-bit code word -- the 2-bit fields at bits 2s of
// its four bytes -- lines up with four consecutive activation bytes and one
// int8 dot4 consumes them with no decode step; the -1 offset of the ternary
// code is one subtraction of sum(q) per 128-weight group; the group dot is
// then scaled by s[g] * ws[n][g] in float32 and summed over groups. The page
// also found independent dot4 accumulators and a one-stage loop best for one
// token (page "Chasing llama.cpp at batch one", section "The win: a program
// just for one token"). The same page series notes that plane dot products
// turn arithmetic-bound from about three tokens (section "One token at a
// time", last paragraph); on gfx950 the per-word bit work is shared by the
// tokens and the dot4 rate leaves room for up to four, so MT = 1, 2 or 4
// token rows run here and larger batches take the MFMA kernel.
//
// gfx950 mapping:
//  * A "chunk" is 16 bytes of one row = 4 code words = half a group. A wave
//    splits into RL = 64/CL row slots of CL lanes; lane cs of a slot handles
//    chunks cs, cs+CL, cs+2CL, ... of RP rows. CL = gcd(K/64, 64), so every
//    lane is busy on every iteration and each load instruction covers RL
//    contiguous runs of CL*16 bytes (coalesced HBM streaming).
//  * K is processed in LDS windows of up to 32768/MT activations per token
//    (one window for every K up to that). Per window the block stages the
//    MT token rows of q into LDS chunk-major by plane ([token][plane][chunk]
//    of 16 bytes, so the CL lanes of a slot read consecutive 16-byte words),
//    with s and t.
//  * Memory-level parallelism: a lane issues the code loads (and the weight
//    scale of each chunk's group) of IB chunk iterations x RP rows at once
//    (one batch) and the next batch is in flight while the current one is
//    computed. A window's first batch and all of its staging loads are
//    issued before the first wait: one memory round trip before compute.
//  * Planes 0 and 2 are masked to bits 0..1 (plane 2 after one shift by 4);
//    planes 1 and 3 are masked in place at bits 2..3, which is 4 * code, and
//    go to a second accumulator divided by 4 (exactly) before the two are
//    added: five bit operations per code word shared by all tokens, and four
//    v_dot4 per code word and token.
//  * The even lane of a chunk pair seeds its accumulators with -t[m][g]; the
//    two half-group sums meet through a DPP lane swap, giving the exact group
//    dot on both lanes. The even lane applies the float32 epilogue.
//  * Rows are reduced over their CL lanes with a fixed butterfly at the end.
//  * Token rows past M (M = 3 runs as MT = 4) read token M-1 and are never
//    stored.
//  * The fused variant (pq2_linear) reads float32 x instead of q, s, t: each
//    block quantises its window in LDS with the quantiser's own arithmetic
//    (quantize_groups32) while its first batch of code loads is in flight,
//    which saves the separate quantise launch of a decode step.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

// u / n for 0 <= u < MT * n, without a division: MT - 1 comparisons.
template <int MT>
__device__ __forceinline__ int token_of(int u, int n) {
    int m = 0;
#pragma unroll
    for (int i = 1; i < MT; ++i) m += u >= i * n ? 1 : 0;
    return m;
}

constexpr int kGemvThreads = 256;
constexpr int kGemvWaves = kGemvThreads / kWave;
constexpr int kLoadsPerBatch = 8;                 // uint4 code loads per lane per batch
constexpr int64_t kMaxStage = 32768;              // activations staged per window (all tokens)
constexpr int kQStagePer = kMaxStage / 16 / kGemvThreads;   // q chunks per thread

template <int LOG_CL, int RP>
struct GemvShape {
    static constexpr int CL = 1 << LOG_CL;
    static constexpr int RL = kWave / CL;
    static constexpr int ROWS_PER_WAVE = RL * RP;
    static constexpr int ROWS_PER_BLOCK = kGemvWaves * ROWS_PER_WAVE;
    static constexpr int IB = kLoadsPerBatch / RP;    // chunk iterations per batch
};

// LDS bytes per group and token of a window: q (128), s (4), t (4).
constexpr int64_t kLdsPerGroup = kGroup + 8;

// Groups quantised per 32-lane slot and pass in the fused variant.
constexpr int kXRound = 8;

template <int LOG_CL, int RP, int MT, bool DOTS, bool FUSED>
__global__ __launch_bounds__(kGemvThreads) void gemv_dot4_kernel(
    const float *__restrict__ x, const int8_t *__restrict__ q, const float *__restrict__ s,
    const int32_t *__restrict__ t, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ ws, float *__restrict__ y, int32_t *__restrict__ d, int64_t M,
    int64_t N, int64_t K, int64_t window) {
    static_assert(!(FUSED && DOTS), "the fused variant writes y");
    using S = GemvShape<LOG_CL, RP>;
    constexpr int CL = S::CL, RL = S::RL, IB = S::IB;
    extern __shared__ uint4 smem[];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int cs = lane & (CL - 1);
    const int rs = lane >> LOG_CL;
    const int h = cs & 1;                         // half of the group this lane holds
    const int64_t G = K / kGroup;
    const int64_t block_row0 = (int64_t)blockIdx.x * S::ROWS_PER_BLOCK;
    const int local0 = wave * S::ROWS_PER_WAVE + rs;     // first local row of this lane
    const int64_t row0 = block_row0 + local0;

    const uint4 *rowp[RP];
    const uint16_t *wsp[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int64_t row = row0 + (int64_t)r * RL;
        const int64_t rc = row < N ? row : N - 1;
        rowp[r] = reinterpret_cast<const uint4 *>(codes + rc * (K / 4));
        wsp[r] = ws + rc * G;
    }

    float facc[RP][MT];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) facc[r][m] = 0.0f;

    // Fused variant: the first pass of x loads goes out before the first code
    // batch. Loads complete in issue order for the wait counter, so the block
    // can then wait for x alone and quantise while the codes of its first
    // batch are still in flight (later windows and passes are serial).
    constexpr int kSlots = kGemvThreads / 32;
    const int lane32 = threadIdx.x & 31, slot = threadIdx.x >> 5;
    float4 xv[kXRound];
    auto load_x = [&](int64_t kx, int base) {
        const int wkx = (int)((K - kx < window) ? K - kx : window);
        const int wgx = wkx / kGroup, ngx = MT * wgx;
#pragma unroll
        for (int i = 0; i < kXRound; ++i) {
            int gi = base + slot + kSlots * i;
            gi = gi < ngx ? gi : ngx - 1;
            const int m = token_of<MT>(gi, wgx), gw = gi - m * wgx;
            const int64_t mc = m < M ? m : M - 1;
            xv[i] = *reinterpret_cast<const float4 *>(x + mc * K + kx + kGroup * gw + 4 * lane32);
        }
    };
    if constexpr (FUSED) {
        load_x(0, 0);
        // keep the x loads ahead of the codes (no pass moves loads across)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }

    for (int64_t k0 = 0; k0 < K; k0 += window) {
        // window extent; all wave-uniform, kept in scalar registers
        const int wk = __builtin_amdgcn_readfirstlane((int)((K - k0 < window) ? K - k0 : window));
        const int wg = wk / kGroup;                   // groups in window
        const int wchunks = wk / 64;
        const int iters = wchunks / CL;
        const int64_t g0 = k0 / kGroup;
        const uint4 *wrow[RP];                        // this lane's first chunk of the window
        const uint16_t *wsrow[RP];                    // the rows' scales of the window
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            wrow[r] = rowp[r] + k0 / 64 + cs;
            wsrow[r] = wsp[r] + g0;
        }

        // Loads are never predicated (a chunk past the window re-reads the
        // window's last chunk and is not used), so each batch is a fixed
        // number of loads and the compiler's wait counts stay exact.
        uint4 bufa[IB][RP], bufb[IB][RP];
        uint16_t wsa[IB][RP], wsb[IB][RP];
        auto load_batch = [&](uint4 (&buf)[IB][RP], uint16_t (&wsv)[IB][RP], int it0) {
#pragma unroll
            for (int b = 0; b < IB; ++b) {
                const int it = min(it0 + b, iters - 1);
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    buf[b][r] = wrow[r][CL * it];
                    if (!DOTS) wsv[b][r] = wsrow[r][(cs + CL * it) >> 1];
                }
            }
        };
        load_batch(bufa, wsa, 0);
        if constexpr (FUSED) __builtin_amdgcn_sched_barrier(0);

        // stage the window: q [token][plane][chunk], s [token][g],
        // t [token][g]; all loads of the staging are issued (clamped,
        // unpredicated) before any LDS store, so they share one memory round
        // trip with the first code batch
        float *s_l = reinterpret_cast<float *>(smem + 4 * MT * wchunks);
        int32_t *t_l = reinterpret_cast<int32_t *>(s_l + MT * wg);
        if constexpr (FUSED) {
            // quantise the window's MT x wg groups from x straight into the
            // LDS layout: 32 lanes per group, kXRound groups per slot and pass,
            // the same arithmetic as pq2_quantize_act (quantize_groups32)
            uint32_t *qw = reinterpret_cast<uint32_t *>(smem);
            const int ngr = MT * wg;
            auto quantize_pass = [&](int base) {
#pragma unroll
                for (int i = 0; i < kXRound; ++i) {
                    const int graw = base + slot + kSlots * i;
                    const float4 xi[1] = {xv[i]};
                    uint32_t word[1];
                    float sc[1];
                    int sm[1];
                    quantize_groups32<1>(xi, lane32, word, sc, sm);   // all 32 lanes
                    if (graw < ngr) {
                        const int m = token_of<MT>(graw, wg), gw = graw - m * wg;
                        const int p = lane32 & 3, j = lane32 >> 2;
                        qw[((m * 4 + p) * wchunks + 2 * gw + (j >> 2)) * 4 + (j & 3)] = word[0];
                        if (lane32 == 0) {
                            s_l[m * wg + gw] = sc[0];
                            t_l[m * wg + gw] = sm[0];
                        }
                    }
                }
            };
            // pass 0 on the x loads issued ahead of the code batch (straight
            // line, so the wait is for x alone); further passes load and wait
            quantize_pass(0);
            for (int base = kSlots * kXRound; base < ngr; base += kSlots * kXRound) {
                load_x(k0, base);
                quantize_pass(base);
            }
        } else
        {
            const int nq = wk / 16;                   // 16-byte q chunks per token
            uint4 qs[kQStagePer];
#pragma unroll
            for (int i = 0; i < kQStagePer; ++i) {
                int u = (int)threadIdx.x + i * kGemvThreads;
                u = u < MT * nq ? u : MT * nq - 1;
                const int m = token_of<MT>(u, nq), uu = u - m * nq;
                const int64_t mc = m < M ? m : M - 1;
                qs[i] = reinterpret_cast<const uint4 *>(q + mc * K + k0)[uu];
            }
            float sv = 0.0f;
            int32_t tv = 0;
            {
                int e = (int)threadIdx.x;
                e = e < MT * wg ? e : MT * wg - 1;
                const int m = token_of<MT>(e, wg), gi = e - m * wg;
                const int64_t mc = m < M ? m : M - 1;
                if (!DOTS) sv = s[mc * G + g0 + gi];
                tv = t[mc * G + g0 + gi];
            }
#pragma unroll
            for (int i = 0; i < kQStagePer; ++i) {
                const int u = threadIdx.x + i * kGemvThreads;
                if (u < MT * nq) {
                    const int m = token_of<MT>(u, nq), uu = u - m * nq;
                    const int g = uu >> 3, p = (uu >> 1) & 3, hh = uu & 1;
                    smem[(m * 4 + p) * wchunks + 2 * g + hh] = qs[i];
                }
            }
            if ((int)threadIdx.x < MT * wg) {
                if (!DOTS) s_l[threadIdx.x] = sv;
                t_l[threadIdx.x] = tv;
            }
        }
        __syncthreads();

        auto compute_batch = [&](const uint4 (&buf)[IB][RP], const uint16_t (&wsv)[IB][RP],
                                 int it0) {
#pragma unroll
            for (int b = 0; b < IB; ++b) {
                if (it0 + b >= iters) break;
                const int c = cs + CL * (it0 + b);    // chunk within window
                const int g = c >> 1;                 // group within window
                // the planes of every code word of the RP rows, shared by the tokens
                uint32_t pa0[RP][4], pa1[RP][4], pa2[RP][4], pa3[RP][4];
#pragma unroll
                for (int r = 0; r < RP; ++r) {
                    const uint4 w = buf[b][r];
                    const uint32_t wr[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const uint32_t wd = wr[jj];
                        const uint32_t hi = wd >> 4;
                        pa0[r][jj] = wd & kPlaneMask;
                        pa1[r][jj] = wd & kPlaneMaskX4;
                        pa2[r][jj] = hi & kPlaneMask;
                        pa3[r][jj] = hi & kPlaneMaskX4;
                    }
                }
                float cw[RP];
                if (!DOTS) {
#pragma unroll
                    for (int r = 0; r < RP; ++r) cw[r] = half_bits_to_float(wsv[b][r]);
                }
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    uint4 qv[4];
#pragma unroll
                    for (int p = 0; p < 4; ++p) qv[p] = smem[(m * 4 + p) * wchunks + c];
                    const int tg = t_l[m * wg + g];
                    float sg = 0.0f;
                    if (!DOTS) sg = s_l[m * wg + g];
                    const uint32_t p0[4] = {qv[0].x, qv[0].y, qv[0].z, qv[0].w};
                    const uint32_t p1[4] = {qv[1].x, qv[1].y, qv[1].z, qv[1].w};
                    const uint32_t p2[4] = {qv[2].x, qv[2].y, qv[2].z, qv[2].w};
                    const uint32_t p3[4] = {qv[3].x, qv[3].y, qv[3].z, qv[3].w};
#pragma unroll
                    for (int r = 0; r < RP; ++r) {
                        int da = h ? 0 : -tg;   // planes 0 and 2, and the -sum(q) offset
                        int db = 0;             // planes 1 and 3, in place: 4 * (their dot)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            da = dot4(pa0[r][jj], p0[jj], da);
                            db = dot4(pa1[r][jj], p1[jj], db);
                            da = dot4(pa2[r][jj], p2[jj], da);
                            db = dot4(pa3[r][jj], p3[jj], db);
                        }
                        const int half_dot = da + (db >> 2);            // db is a multiple of 4
                        const int dot = half_dot + dpp_xor1(half_dot);  // exact group dot
                        if (DOTS) {
                            const int64_t row = row0 + (int64_t)r * RL;
                            if (!h && m < M && row < N) d[(m * N + row) * G + g0 + g] = dot;
                        } else {
                            facc[r][m] = fmaf((float)dot, h ? 0.0f : sg * cw[r], facc[r][m]);
                        }
                    }
                }
            }
        };

        // ping-pong: the other buffer's loads are in flight during each
        // compute. Prefetches are unconditional (clamped), so the wait counts
        // inside the loop are static.
        if (iters <= IB) {
            compute_batch(bufa, wsa, 0);
        } else {
            for (int it0 = 0;; it0 += 2 * IB) {
                load_batch(bufb, wsb, it0 + IB);
                compute_batch(bufa, wsa, it0);
                if (it0 + IB >= iters) break;
                load_batch(bufa, wsa, it0 + 2 * IB);
                compute_batch(bufb, wsb, it0 + IB);
                if (it0 + 2 * IB >= iters) break;
            }
        }
        if constexpr (FUSED) {
            // the next window's first x pass (the last window reloads itself;
            // unconditional, so the pending loads are the same on every path)
            const int64_t last = ((K - 1) / window) * window;
            load_x(k0 + window < K ? k0 + window : last, 0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        if (k0 + window < K) __syncthreads();    // window buffer is reused
    }

    if (!DOTS) {
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            const int64_t row = row0 + (int64_t)r * RL;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float v = segment_sum<CL>(facc[r][m]);
                if (cs == 0 && m < M && row < N) y[m * N + row] = v;
            }
        }
    }
}

template <int LOG_CL, int RP, int MT>
hipError_t launch_cfg(const float *x, const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    using S = GemvShape<LOG_CL, RP>;
    const int64_t blocks = (N + S::ROWS_PER_BLOCK - 1) / S::ROWS_PER_BLOCK;
    constexpr int64_t kWindow = kMaxStage / MT;       // a multiple of 64 * CL for every CL
    const int64_t window = K < kWindow ? K : kWindow;
    const size_t lds = (size_t)(MT * (window / kGroup) * kLdsPerGroup);
    if (x) {
        hipLaunchKernelGGL((gemv_dot4_kernel<LOG_CL, RP, MT, false, true>), dim3((unsigned)blocks),
                           dim3(kGemvThreads), lds, stream, x, nullptr, nullptr, nullptr, codes,
                           out.ws, out.y, nullptr, M, N, K, window);
    } else if (out.d) {
        hipLaunchKernelGGL((gemv_dot4_kernel<LOG_CL, RP, MT, true, false>), dim3((unsigned)blocks),
                           dim3(kGemvThreads), lds, stream, nullptr, q, nullptr, t, codes,
                           nullptr, nullptr, out.d, M, N, K, window);
    } else {
        hipLaunchKernelGGL((gemv_dot4_kernel<LOG_CL, RP, MT, false, false>), dim3((unsigned)blocks),
                           dim3(kGemvThreads), lds, stream, nullptr, q, out.s, t, codes, out.ws,
                           out.y, nullptr, M, N, K, window);
    }
    return hipGetLastError();
}

// Two rows per lane when a row slot is wide (CL >= 32): each wave then still
// covers four rows, and every q word read from LDS serves both rows.
template <int LOG_CL>
hipError_t launch_cl(const float *x, const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    constexpr int RP = (LOG_CL >= 5) ? 2 : 1;
    if (M == 1) return launch_cfg<LOG_CL, RP, 1>(x, q, t, codes, out, M, N, K, stream);
    if (M == 2) return launch_cfg<LOG_CL, RP, 2>(x, q, t, codes, out, M, N, K, stream);
    return launch_cfg<LOG_CL, RP, 4>(x, q, t, codes, out, M, N, K, stream);
}

// x != nullptr: the fused variant (quantises x itself); else q, t from
// pq2_quantize_act.
hipError_t launch_any(const float *x, const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    // chunk lanes per row: the largest power of two <= 64 dividing K/64
    const int64_t chunks = K / 64;
    int64_t cl = chunks & -chunks;
    if (cl > 64) cl = 64;
    switch (cl) {
        case 2: return launch_cl<1>(x, q, t, codes, out, M, N, K, stream);
        case 4: return launch_cl<2>(x, q, t, codes, out, M, N, K, stream);
        case 8: return launch_cl<3>(x, q, t, codes, out, M, N, K, stream);
        case 16: return launch_cl<4>(x, q, t, codes, out, M, N, K, stream);
        case 32: return launch_cl<5>(x, q, t, codes, out, M, N, K, stream);
        default: return launch_cl<6>(x, q, t, codes, out, M, N, K, stream);
    }
}

}  // namespace

hipError_t launch_gemv(const int8_t *q, const int32_t *t, const uint8_t *codes,
                       const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return launch_any(nullptr, q, t, codes, out, M, N, K, stream);
}

hipError_t launch_gemv_fused(const float *x, const uint8_t *codes, const uint16_t *ws, float *y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const GemmOut out{y, nullptr, nullptr, ws};
    return launch_any(x, nullptr, nullptr, codes, out, M, N, K, stream);
}

}  // namespace pq2
