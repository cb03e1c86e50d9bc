// gemv_dot4.hip -- K2: the PQ2_0 GEMV on v_dot4 for 1 to 4 token rows.
//
// Algorithm (page "Making a ternary reasoning model fast in vLLM", section
// "One token at a time: plain Triton is enough"): activations are in plane
// order, so plane s of a 32-bit code word -- the 2-bit fields at bits 2s of
// its four bytes -- pairs with four adjacent plane-order activation bytes, and
// one int8 dot4 takes both with no decode step; the -1 offset of the ternary
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
//    contiguous runs of CL*16 bytes (coalesced HBM streaming). A block (four
//    waves) covers a row group of ROWS_PER_BLOCK rows.
//  * The MT token rows of q are staged in LDS chunk-major by plane
//    ([token][plane][chunk] of 16 bytes, so the CL lanes of a slot read
//    consecutive 16-byte words), with s and t, in windows of up to
//    kMaxStage / MT activations per token.
//  * When one window covers K (every shape of the decode and small-batch
//    workloads) the kernel is persistent: at most kPersistBlocks blocks each
//    stage q once and then walk row groups blockIdx.x, + gridDim.x, ...; the
//    staging is paid once per block instead of once per row group. Otherwise
//    each block takes one row group and loops over the windows.
//  * Memory-level parallelism: a lane issues the code loads (and the weight
//    scale of each chunk's group) of IB chunk iterations x RP rows at once
//    (one batch); the next batch -- of the same row group or the next one --
//    is in flight while the current one is computed. For one token row they
//    are buffer loads with a fixed per-lane offset (no address arithmetic
//    per load); the four-wave K = 5120 plan loads a row's scales together
//    and hands them out by lane permutes. The staging loads go
//    out first and the first batch right behind them, in one memory round
//    trip; the block computes on each code word as it arrives. Six loads
//    per batch: the decode shapes' rows then split into whole batches
//    (K = 6144: 3 iterations x 2 rows), so no lane re-reads a chunk whose
//    line is still in flight.
//  * Planes 0 and 2 are masked to bits 0..1 (plane 2 after one shift by 4);
//    planes 1 and 3 are masked in place at bits 2..3, which is 4 * code, and
//    go to a second accumulator divided by 4 (exactly) before the two are
//    added: five bit operations per code word shared by all tokens, and four
//    v_dot4 per code word and token.
//  * The even lane of a chunk pair seeds its accumulators with -t[m][g]; the
//    two half-group sums meet through a DPP lane swap, giving the exact group
//    dot on both lanes. The even lane applies the float32 epilogue.
//  * Rows are reduced over their CL lanes with a fixed butterfly when their
//    row group is done.
//  * Token rows past M (M = 3 runs as MT = 4) read token M-1 and are never
//    stored.
//  * The fused variant (pq2_linear) reads float32 x instead of q, s, t: each
//    block quantises its window in LDS with the quantiser's own arithmetic
//    (quantize_groups8, 8 lanes per group). The first pass of x loads is
//    issued before the first code batch (loads complete in issue order for
//    the wait counter), so the block quantises while its codes are in flight.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

#include <type_traits>

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

constexpr int kLoadsPerBatch = 6;                 // uint4 code loads per lane per batch
constexpr int64_t kMaxStage = 40960;              // activations staged per window (all tokens)
constexpr int64_t kPersistBlocks = 512;           // two blocks per CU
constexpr int kXRound = 2;                        // groups per 8-lane slot and pass (fused)

typedef __attribute__((address_space(3))) const v4i lds_v4i;

// NW waves per block (4 by default; 5 to 10 for the one-block-per-CU plans
// of the decode shapes, see launch_mt), IB0 chunk iterations per batch (0:
// kLoadsPerBatch / RP; those plans take a row's whole iteration count).
template <int LOG_CL, int RP, int NW, int IB0 = 0>
struct GemvShape {
    static constexpr int CL = 1 << LOG_CL;
    static constexpr int RL = kWave / CL;
    static constexpr int ROWS_PER_WAVE = RL * RP;
    static constexpr int ROWS_PER_BLOCK = NW * ROWS_PER_WAVE;
    static constexpr int IB = IB0 > 0 ? IB0 : kLoadsPerBatch / RP;   // chunk iterations per batch
    static constexpr int kThreads = NW * kWave;
    static constexpr int kQStagePer = (kMaxStage / 16 + kThreads - 1) / kThreads;   // q chunks per thread
    static constexpr int kSTStagePer = (kMaxStage / 128 + kThreads - 1) / kThreads; // s, t per thread
};

// LDS bytes per group and token of a window: q (128), s (4), t (4).
constexpr int64_t kLdsPerGroup = kGroup + 8;

template <int LOG_CL, int RP, int MT, bool DOTS, bool FUSED, bool Y16, int NW, int IB0>
__global__ __launch_bounds__(NW * kWave) void gemv_dot4_kernel(
    const float *__restrict__ x, const int8_t *__restrict__ q, const float *__restrict__ s,
    const int32_t *__restrict__ t, const uint8_t *__restrict__ codes,
    const uint16_t *__restrict__ ws, float *__restrict__ y, uint16_t *__restrict__ y16,
    int32_t *__restrict__ d, int64_t M,
    int64_t N, int64_t K, int64_t window) {
    static_assert(!(FUSED && DOTS), "the fused variant writes y");
    using S = GemvShape<LOG_CL, RP, NW, IB0>;
    constexpr int CL = S::CL, RL = S::RL, IB = S::IB;
    constexpr int kGemvThreads = S::kThreads;
    constexpr int kQStagePer = S::kQStagePer, kSTStagePer = S::kSTStagePer;
    extern __shared__ uint4 smem[];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int cs = lane & (CL - 1);
    const int rs = lane >> LOG_CL;
    const int h = cs & 1;                         // half of the group this lane holds
    const int64_t G = K / kGroup;
    const int local0 = wave * S::ROWS_PER_WAVE + rs;     // first row of this lane in a row group
    const int64_t n_rg = (N + S::ROWS_PER_BLOCK - 1) / S::ROWS_PER_BLOCK;
    const bool single = K <= window;              // uniform: one LDS window covers K

    float facc[RP][MT];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
        for (int m = 0; m < MT; ++m) facc[r][m] = 0.0f;

    // ---------------------------------------------------------------- loads
    // One row's weight scales for a whole-row batch of five 16-lane chunks
    // (K = 5120, the four-wave plan): its 40 halves are 20 dwords, which the
    // row's 16 lanes load in two instructions (lane i: dwords i and 16 + i % 4)
    // and hand out by lane permutes, instead of five 2-byte loads per lane
    // (34816 x 5120: 11.4 -> 11.1 us; the six- to ten-wave plans measured
    // slower this way and keep the 2-byte loads).
    constexpr bool kCoopWs =
        MT == 1 && !FUSED && !DOTS && LOG_CL == 4 && IB == 5 && RP == 1 && NW == 4;
    using WsT = typename std::conditional<kCoopWs, uint32_t, uint16_t>::type;
    // (native vectors: copies of the HIP uint4 struct can leave arrays in scratch)
    v4i bufa[IB][RP], bufb[IB][RP];
    WsT wsa[IB][RP], wsb[IB][RP];
    // Byte offsets of this lane's rows (local0 + r * RL) inside a row group's
    // codes and weight scales. For one token row (not fused) the loads are
    // buffer loads over the row group: the per-lane part is this fixed offset,
    // the chunk iteration and window are a wave-uniform offset, so a load
    // costs no address arithmetic; rows past N lie outside the resource and
    // read zeros (their sums are never stored). Every offset stays below 2^30
    // (K <= 2^24, at most 128 rows).
    int voff_c[RP], voff_w[RP];
#pragma unroll
    for (int r = 0; r < RP; ++r) {
        const int lr = local0 + r * RL;
        voff_c[r] = lr * (int)(K / 4) + 16 * cs;
        voff_w[r] = 2 * (lr * (int)G + (cs >> 1));
    }
    // code chunks of row group rg, window starting at k0, iterations it0..
    // (never predicated: past the window the last chunk is re-read, unused)
    auto load_batch = [&](v4i (&buf)[IB][RP], WsT (&wsv)[IB][RP], int64_t rg, int64_t k0,
                          int iters, int it0) __attribute__((always_inline)) {
        const int64_t rbase = rg * S::ROWS_PER_BLOCK;
        const int64_t nr = N - rbase < S::ROWS_PER_BLOCK ? N - rbase : S::ROWS_PER_BLOCK;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes + rbase * (K / 4), nr * (K / 4));
        const __amdgpu_buffer_rsrc_t rw = make_rsrc(ws + rbase * G, nr * G * 2);
#pragma unroll
        for (int r = 0; r < RP; ++r) {
            if constexpr (FUSED || MT > 1) {
                // (the fused variant and two or four token rows measured as
                // fast or faster with plain loads)
                const int64_t row = rbase + local0 + (int64_t)r * RL;
                const int64_t rcl = row < N ? row : N - 1;
                const v4i *cp = reinterpret_cast<const v4i *>(codes + rcl * (K / 4)) + k0 / 64 + cs;
                const uint16_t *wp = ws + rcl * G + k0 / kGroup;
#pragma unroll
                for (int b = 0; b < IB; ++b) {
                    const int it = min(it0 + b, iters - 1);
                    buf[b][r] = cp[CL * it];
                    wsv[b][r] = wp[(cs + CL * it) >> 1];
                }
            } else {
                if constexpr (kCoopWs) {
                    // (this plan runs for K = 5120 only: one batch per row, it0 = 0)
                    const int sb = (int)(k0 / 64) + CL * it0;
                    const int rowoff = 2 * local0 * (int)G;
                    wsv[0][0] = __builtin_amdgcn_raw_buffer_load_b32(rw, rowoff + 4 * cs, sb, 0);
                    wsv[1][0] = __builtin_amdgcn_raw_buffer_load_b32(rw, rowoff + 4 * (16 + (cs & 3)),
                                                                     sb, 0);
                }
#pragma unroll
                for (int b = 0; b < IB; ++b) {
                    const int it = min(it0 + b, iters - 1);
                    buf[b][r] = __builtin_bit_cast(
                        v4i, __builtin_amdgcn_raw_buffer_load_b128(rc, voff_c[r],
                                                                   (int)(k0 / 4) + 16 * CL * it, 0));
                    if (!DOTS && !kCoopWs)
                        wsv[b][r] = __builtin_amdgcn_raw_buffer_load_b16(
                            rw, voff_w[r], (int)(k0 / 64) + CL * it, 0);
                }
            }
        }
    };

    // x loads of the fused variant (first pass of window kx): 8-lane slots,
    // one group per slot and round, lane j of a slot loading the group's
    // activations 16j .. 16j + 15 (quantize_groups8)
    constexpr int kSlots = kGemvThreads / 8;
    // rounds per pass: kXRound, or the exact count where the plan fixes K (a
    // row's whole iteration count in one batch: G = IB0 * CL / 2 groups)
    constexpr int kXNeed = IB0 > 0 ? (MT * IB0 * CL / 2 + kSlots - 1) / kSlots : kXRound;
    constexpr int kXR = kXNeed < kXRound ? kXNeed : kXRound;
    const int lane8 = threadIdx.x & 7, slot = threadIdx.x >> 3;
    float4 xv[kXR][4];
    auto load_x = [&](int64_t kx, int base) __attribute__((always_inline)) {
        const int wkx = (int)((K - kx < window) ? K - kx : window);
        const int wgx = wkx / kGroup, ngx = MT * wgx;
        // rounds i with a group for some slot (a uniform bound); slots past
        // the last group load nothing and quantise zeros that are never stored
        const int rounds = (ngx - base + kSlots - 1) / kSlots;
#pragma unroll
        for (int i = 0; i < kXR; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[i][e] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            const int gi = base + slot + kSlots * i;
            if (i < rounds && gi < ngx) {
                const int m = token_of<MT>(gi, wgx), gw = gi - m * wgx;
                const int64_t mc = m < M ? m : M - 1;
                const float4 *src = reinterpret_cast<const float4 *>(x + mc * K + kx + kGroup * gw + 16 * lane8);
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[i][e] = src[e];
            }
        }
    };

    // ---------------------------------------------------------------- staging
    // q, s, t of window k0 into registers (the non-fused variant), issued
    // ahead of the first code batch: loads complete in issue order for the
    // wait counter, so the LDS stores below then wait only for these loads
    // and the block starts computing while its codes are still arriving.
    v4i qs[kQStagePer];
    float sv[kSTStagePer];
    int32_t tv[kSTStagePer];
    auto stage_load = [&](int64_t k0, int wk) __attribute__((always_inline)) {
        const int wg = wk / kGroup;
        const int nq = wk / 16;                   // 16-byte q chunks per token
        // only the passes the window needs (a uniform bound): a clamped load
        // past the end re-reads the last chunk, so every extra pass would
        // queue behind a line already in flight
        const int passes = (MT * nq + kGemvThreads - 1) / kGemvThreads;
        // a wave whose first chunk is past the end loads nothing: every
        // block's waves asking for the same last line keep one L2 channel busy
        const int wave0 = (int)threadIdx.x & ~(kWave - 1);
#pragma unroll
        for (int i = 0; i < kQStagePer; ++i) {
            if (i < passes && wave0 + i * kGemvThreads < MT * nq) {
                int u = (int)threadIdx.x + i * kGemvThreads;
                u = u < MT * nq ? u : MT * nq - 1;
                const int m = token_of<MT>(u, nq), uu = u - m * nq;
                const int64_t mc = m < M ? m : M - 1;
                qs[i] = reinterpret_cast<const v4i *>(q + mc * K + k0)[uu];
            }
        }
        const int st_passes = (MT * wg + kGemvThreads - 1) / kGemvThreads;
#pragma unroll
        for (int i = 0; i < kSTStagePer; ++i) {
            sv[i] = 0.0f;
            tv[i] = 0;
            if (i < st_passes && wave0 + i * kGemvThreads < MT * wg) {
                int e = (int)threadIdx.x + i * kGemvThreads;
                e = e < MT * wg ? e : MT * wg - 1;
                const int m = token_of<MT>(e, wg), gi = e - m * wg;
                const int64_t mc = m < M ? m : M - 1;
                if (!DOTS) sv[i] = s[mc * G + k0 / kGroup + gi];
                tv[i] = t[mc * G + k0 / kGroup + gi];
            }
        }
    };

    // window k0 of wk activations per token into LDS: q [token][plane][chunk],
    // s [token][g], t [token][g]. Ends with a barrier.
    auto stage = [&](int64_t k0, int wk) __attribute__((always_inline)) {
        const int wg = wk / kGroup;
        const int wchunks = wk / 64;
        float *s_l = reinterpret_cast<float *>(smem + 4 * MT * wchunks);
        int32_t *t_l = reinterpret_cast<int32_t *>(s_l + MT * wg);
        if constexpr (FUSED) {
            // quantise the window's MT x wg groups from x straight into the
            // LDS layout: 8 lanes per group, kXR groups per slot and pass
            uint32_t *qw = reinterpret_cast<uint32_t *>(smem);
            const int ngr = MT * wg;
            auto quantize_pass = [&](int base) __attribute__((always_inline)) {
                // rounds with a group for some slot (uniform, as in load_x)
                const int rounds = (ngr - base + kSlots - 1) / kSlots;
#pragma unroll
                for (int i = 0; i < kXR; ++i) {
                    if (i >= rounds) break;
                    const int graw = base + slot + kSlots * i;
                    uint32_t word[4];
                    float sc;
                    int sm;
                    quantize_groups8(xv[i], word, sc, sm);   // all 8 lanes
                    if (graw < ngr) {
                        const int m = token_of<MT>(graw, wg), gw = graw - m * wg;
#pragma unroll
                        for (int p = 0; p < 4; ++p)
                            qw[((m * 4 + p) * wchunks + 2 * gw + (lane8 >> 2)) * 4 + (lane8 & 3)] =
                                word[p];
                        if (lane8 == 0) {
                            s_l[m * wg + gw] = sc;
                            t_l[m * wg + gw] = sm;
                        }
                    }
                }
            };
            // pass 0 on x loads issued ahead of the first code batch
            quantize_pass(0);
            for (int base = kSlots * kXR; base < ngr; base += kSlots * kXR) {
                load_x(k0, base);
                quantize_pass(base);
            }
        } else {
            const int nq = wk / 16;                   // 16-byte q chunks per token
#pragma unroll
            for (int i = 0; i < kQStagePer; ++i) {
                const int u = threadIdx.x + i * kGemvThreads;
                if (u < MT * nq) {
                    const int m = token_of<MT>(u, nq), uu = u - m * nq;
                    const int g = uu >> 3, p = (uu >> 1) & 3, hh = uu & 1;
                    reinterpret_cast<v4i *>(smem)[(m * 4 + p) * wchunks + 2 * g + hh] = qs[i];
                }
            }
#pragma unroll
            for (int i = 0; i < kSTStagePer; ++i) {
                const int e = (int)threadIdx.x + i * kGemvThreads;
                if (e < MT * wg) {
                    if (!DOTS) s_l[e] = sv[i];
                    t_l[e] = tv[i];
                }
            }
        }
        __syncthreads();
    };

    // ---------------------------------------------------------------- compute
    auto compute_batch = [&](const v4i (&buf)[IB][RP], const WsT (&wsv)[IB][RP],
                             int64_t rg, int64_t k0, int wk, int it0) __attribute__((always_inline)) {
        const int wg = wk / kGroup;
        const int wchunks = wk / 64;
        const int iters = wchunks / CL;
        const float *s_l = reinterpret_cast<const float *>(smem + 4 * MT * wchunks);
        const int32_t *t_l = reinterpret_cast<const int32_t *>(s_l + MT * wg);
        const int64_t row0 = rg * S::ROWS_PER_BLOCK + local0;
        // this lane's chunk and group at b = 0; chunk b of the batch is CL * b
        // chunks and CL / 2 groups further (constant LDS offsets)
        const int cb = cs + CL * it0;
        const int32_t *t_b = t_l + (cb >> 1);
        const float *s_b = s_l + (cb >> 1);
        // the LDS address of each token's planes at b = 0, opaque to the
        // compiler: it would otherwise fold the constant b offsets into the
        // wave-uniform plane offsets and add both to the lane address per chunk
        lds_v4i *q_b[MT][4];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                q_b[m][p] = (lds_v4i *)smem + (m * 4 + p) * wchunks + cb;
                asm volatile("" : "+v"(q_b[m][p]));
            }
#pragma unroll
        for (int b = 0; b < IB; ++b) {
            if (it0 + b >= iters) break;
            // the planes of every code word of the RP rows, shared by the tokens
            uint32_t pa0[RP][4], pa1[RP][4], pa2[RP][4], pa3[RP][4];
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                const v4i w = buf[b][r];
                const uint32_t wr[4] = {(uint32_t)w[0], (uint32_t)w[1], (uint32_t)w[2], (uint32_t)w[3]};
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
                for (int r = 0; r < RP; ++r) {
                    if constexpr (kCoopWs) {
                        // half (cs >> 1) + 8 b of the row's batch: dword (cs >> 2) + 4 b
                        const int src = rs * 16 + (b < 4 ? 4 * b : 0) + (cs >> 2);
                        const uint32_t dw = (uint32_t)__builtin_amdgcn_ds_bpermute(
                            4 * src, (int)(b < 4 ? wsv[0][0] : wsv[1][0]));
                        cw[r] = half_bits_to_float((uint16_t)(dw >> (16 * ((cs >> 1) & 1))));
                    } else {
                        cw[r] = half_bits_to_float(wsv[b][r]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                v4i qv[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) qv[p] = q_b[m][p][CL * b];
                const int tg = t_b[m * wg + (CL / 2) * b];
                float sg = 0.0f;
                if (!DOTS) sg = s_b[m * wg + (CL / 2) * b];
                uint32_t p0[4], p1[4], p2[4], p3[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    p0[jj] = (uint32_t)qv[0][jj];
                    p1[jj] = (uint32_t)qv[1][jj];
                    p2[jj] = (uint32_t)qv[2][jj];
                    p3[jj] = (uint32_t)qv[3][jj];
                }
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
                        const int g = (cb >> 1) + (CL / 2) * b;   // group within window
                        if (!h && m < M && row < N) d[(m * N + row) * G + k0 / kGroup + g] = dot;
                    } else {
                        facc[r][m] = fmaf((float)dot, h ? 0.0f : sg * cw[r], facc[r][m]);
                    }
                }
            }
        }
    };

    // reduce the rows of row group rg over their CL lanes, store, reset
    auto finish = [&](int64_t rg) __attribute__((always_inline)) {
        if (!DOTS) {
            const int64_t row0 = rg * S::ROWS_PER_BLOCK + local0;
#pragma unroll
            for (int r = 0; r < RP; ++r) {
                const int64_t row = row0 + (int64_t)r * RL;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float v = segment_sum<CL>(facc[r][m]);
                    if (cs == 0 && m < M && row < N) {
                        if constexpr (Y16)
                            y16[m * N + row] = bf16_rne(v);
                        else
                            y[m * N + row] = v;
                    }
                    facc[r][m] = 0.0f;
                }
            }
        }
    };

    // This block's batches in order: row groups rg_first, + gridDim.x, ...
    // (rg_count of them), nb batches of IB iterations each.
    auto run = [&](int64_t k0, int wk, int64_t rg_first, int64_t rg_count,
                   bool last_window) __attribute__((always_inline)) {
        const int iters = wk / 64 / CL;
        const int nb = (iters + IB - 1) / IB;
        const int J = (int)(rg_count * nb);
        auto rg_of = [&](int j) __attribute__((always_inline)) { return rg_first + (int64_t)(j / nb) * gridDim.x; };
        auto it_of = [&](int j) __attribute__((always_inline)) { return (j % nb) * IB; };
        if (J == 1) {                  // one batch in all: nothing to prefetch
            compute_batch(bufa, wsa, rg_first, k0, wk, 0);
            if (last_window) finish(rg_first);
            return;
        }
        // ping-pong: the other buffer's loads are in flight during each
        // compute; prefetches are unconditional (clamped), so the wait counts
        // inside the loop are static
        for (int j = 0;; j += 2) {
            const int j1 = j + 1 < J ? j + 1 : J - 1;
            load_batch(bufb, wsb, rg_of(j1), k0, iters, it_of(j1));
            compute_batch(bufa, wsa, rg_of(j), k0, wk, it_of(j));
            if (last_window && j % nb == nb - 1) finish(rg_of(j));
            if (j + 1 >= J) break;
            const int j2 = j + 2 < J ? j + 2 : J - 1;
            load_batch(bufa, wsa, rg_of(j2), k0, iters, it_of(j2));
            compute_batch(bufb, wsb, rg_of(j + 1), k0, wk, it_of(j + 1));
            if (last_window && (j + 1) % nb == nb - 1) finish(rg_of(j + 1));
            if (j + 2 >= J) break;
        }
    };

    const int64_t rg0 = blockIdx.x;
    if (single) {
        // persistent: stage once, then every row group of this block
        const int wk = (int)K;
        const int64_t count = (n_rg - rg0 + gridDim.x - 1) / gridDim.x;
        if constexpr (FUSED) load_x(0, 0);
        else stage_load(0, wk);
        asm volatile("" ::: "memory");         // keep the staging loads ahead of the codes
        __builtin_amdgcn_sched_barrier(0);
        load_batch(bufa, wsa, rg0, 0, wk / 64 / CL, 0);
        __builtin_amdgcn_sched_barrier(0);
        stage(0, wk);
        run(0, wk, rg0, count, true);
    } else {
        // one row group per block, windows in turn
        for (int64_t k0 = 0; k0 < K; k0 += window) {
            const int wk = __builtin_amdgcn_readfirstlane((int)((K - k0 < window) ? K - k0 : window));
            if constexpr (FUSED) load_x(k0, 0);
            else stage_load(k0, wk);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            load_batch(bufa, wsa, rg0, k0, wk / 64 / CL, 0);
            __builtin_amdgcn_sched_barrier(0);
            stage(k0, wk);
            run(k0, wk, rg0, 1, k0 + window >= K);
            if (k0 + window < K) __syncthreads();    // window buffer is reused
        }
    }
}

// window: the largest multiple of 64 * CL activations per token within
// kMaxStage / MT (iterations then divide every window)
template <int LOG_CL, int MT>
constexpr int64_t gemv_window() {
    return (kMaxStage / MT) / (64 << LOG_CL) * (64 << LOG_CL);
}

template <int LOG_CL, int RP, int MT, int NW, int IB0 = 0>
hipError_t launch_cfg(const float *x, const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    using S = GemvShape<LOG_CL, RP, NW, IB0>;
    const int64_t n_rg = (N + S::ROWS_PER_BLOCK - 1) / S::ROWS_PER_BLOCK;
    constexpr int64_t kWindow = gemv_window<LOG_CL, MT>();
    static_assert(kWindow >= (64 << LOG_CL), "window");
    const int64_t window = K < kWindow ? K : kWindow;
    const int64_t blocks = K <= window ? (n_rg < kPersistBlocks ? n_rg : kPersistBlocks) : n_rg;
    const size_t lds = (size_t)(MT * (window / kGroup) * kLdsPerGroup);
    const dim3 threads(S::kThreads);
    if (x) {
        hipLaunchKernelGGL((gemv_dot4_kernel<LOG_CL, RP, MT, false, true, false, NW, IB0>), dim3((unsigned)blocks),
                           threads, lds, stream, x, nullptr, nullptr, nullptr, codes,
                           out.ws, out.y, nullptr, nullptr, M, N, K, window);
    } else if (out.d) {
        hipLaunchKernelGGL((gemv_dot4_kernel<LOG_CL, RP, MT, true, false, false, NW, IB0>), dim3((unsigned)blocks),
                           threads, lds, stream, nullptr, q, nullptr, t, codes,
                           nullptr, nullptr, nullptr, out.d, M, N, K, window);
    } else if (out.y16) {
        hipLaunchKernelGGL((gemv_dot4_kernel<LOG_CL, RP, MT, false, false, true, NW, IB0>), dim3((unsigned)blocks),
                           threads, lds, stream, nullptr, q, out.s, t, codes, out.ws,
                           nullptr, out.y16, nullptr, M, N, K, window);
    } else {
        hipLaunchKernelGGL((gemv_dot4_kernel<LOG_CL, RP, MT, false, false, false, NW, IB0>), dim3((unsigned)blocks),
                           threads, lds, stream, nullptr, q, out.s, t, codes, out.ws,
                           out.y, nullptr, nullptr, M, N, K, window);
    }
    return hipGetLastError();
}

// Launch plan. Where a row takes 3 (CL = 32) or 5 (CL = 16) chunk
// iterations and the rows split into 5 to 10 waves per compute unit: one
// block per CU with one row per lane, that many waves, and a row's whole
// iteration count in one batch (no clamped re-reads). Every CU then streams
// the same number of rows (with 16-row blocks of four waves, 5120 rows make
// 320 blocks and 64 CUs carry two) and each wave's compute after its last
// code word lands is short. MI355X, us per call, 64 rotating weight sets,
// M = 1: 5120 x 6144 4.82 against 5.08 with four-wave blocks of two rows per
// lane; 6144 x 5120 4.85 against 4.91. Otherwise four-wave blocks, two rows
// per lane when a row slot is wide (CL >= 32: every q word read from LDS
// then serves both rows), persistent over at most 512 blocks (17408 x 5120
// would need 17 waves per CU: 8.02 us this way).
template <int LOG_CL, int NW, int MT, int ITER>
hipError_t launch_nw(const float *x, const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    return launch_cfg<LOG_CL, 1, MT, NW, ITER>(x, q, t, codes, out, M, N, K, stream);
}

template <int LOG_CL, int MT, int ITER>
hipError_t launch_balanced(int64_t nw, const float *x, const int8_t *q, const int32_t *t,
                           const uint8_t *codes, const GemmOut &out, int64_t M, int64_t N,
                           int64_t K, hipStream_t stream) {
    switch (nw) {
        case 5: return launch_nw<LOG_CL, 5, MT, ITER>(x, q, t, codes, out, M, N, K, stream);
        case 6: return launch_nw<LOG_CL, 6, MT, ITER>(x, q, t, codes, out, M, N, K, stream);
        case 7:
        case 8: return launch_nw<LOG_CL, 8, MT, ITER>(x, q, t, codes, out, M, N, K, stream);
        default:
            if constexpr (ITER > 0)
                return launch_nw<LOG_CL, 10, MT, ITER>(x, q, t, codes, out, M, N, K, stream);
            else
                return hipErrorInvalidValue;      // never planned (nw <= 8 for ITER = 0)
    }
}

template <int LOG_CL, int MT>
hipError_t launch_mt(const float *x, const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if constexpr ((LOG_CL == 4 || LOG_CL == 5) && MT <= 2) {
        constexpr int64_t RL = kWave >> LOG_CL;
        constexpr int64_t kIter = LOG_CL == 5 ? 3 : 5;
        const int cus = device_cus();
        if (K <= gemv_window<LOG_CL, MT>() && cus > 0) {
            const int64_t units = (N + RL - 1) / RL;
            const int64_t nw = (units + cus - 1) / cus;
            if (nw >= 5 && nw <= 10) {
                // longer rows (5120 x 17408: 17 iterations of CL = 16) in
                // batches of six: 9.33 us against 9.62 for four-wave blocks
                if (K == kIter * (64 << LOG_CL))
                    return launch_balanced<LOG_CL, MT, kIter>(nw, x, q, t, codes, out, M, N, K,
                                                              stream);
                // (six-deep batches fit the registers of at most 8 waves)
                if constexpr (MT == 1)
                    if (nw <= 8)
                        return launch_balanced<LOG_CL, MT, 0>(nw, x, q, t, codes, out, M, N, K,
                                                              stream);
            }
        }
    }
    constexpr int RP = (LOG_CL >= 5) ? 2 : 1;
    // rows of 5 chunk iterations (K = 5120) in batches of exactly five loads:
    // a batch of the default six re-reads a clamped chunk (MI355X, M = 1:
    // 34816 x 5120 11.6 against 12.2 us; 17408 x 5120 7.75 against 8.08)
    if constexpr (LOG_CL == 4 && MT <= 2)
        if (K == 5 * (64 << LOG_CL))
            return launch_cfg<LOG_CL, RP, MT, 4, 5>(x, q, t, codes, out, M, N, K, stream);
    return launch_cfg<LOG_CL, RP, MT, 4>(x, q, t, codes, out, M, N, K, stream);
}

template <int LOG_CL>
hipError_t launch_cl(const float *x, const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    if (M == 1) return launch_mt<LOG_CL, 1>(x, q, t, codes, out, M, N, K, stream);
    if (M == 2) return launch_mt<LOG_CL, 2>(x, q, t, codes, out, M, N, K, stream);
    return launch_mt<LOG_CL, 4>(x, q, t, codes, out, M, N, K, stream);
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
