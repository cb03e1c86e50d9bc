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
//  * The float epilogue (convert, scale product, FMA per output and group;
//    the product widens the half scale inside one mixed-precision FMA) is
//    the VALU work that bounds this kernel, so everything else is kept
//    off the VALU: MFMA results stay in VGPRs (no accumulator-register
//    copies), global addresses are a uniform 64-bit base plus a fixed 32-bit
//    per-lane offset, and a lane's A operands are formed once per group and
//    reused across its WM token tiles.
//  * Scales are staged in LDS eight groups at a time (double buffered).
//  * Staging runs through two LDS stages with one barrier per group. With
//    DEPTH = 2 the global loads of group g+2 are issued into one of two
//    register sets while group g is computed and group g+1 is written from
//    the other set into the second stage; with DEPTH = 1 (large tiles, whose
//    accumulators leave no room for a second set) the loads of group g+1 are
//    in flight while group g is computed.
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
// Scales are staged kScaleChunk groups at a time: lanes walk along the group
// dimension of the [rows][G] scale arrays, so one load instruction touches a
// few cache lines instead of one line per lane.
constexpr int kScaleChunk = 8;

// s * ws for the epilogue as one mixed-precision FMA that widens the half
// scale itself (v_fma_mix_f32): the float32 product s * (float)ws with +0
// added, one instruction where a conversion and a multiply would be two.
__device__ __forceinline__ float scale_product(float sv, _Float16 w) {
    return fmaf(sv, (float)w, 0.0f);
}

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
    };
    // Scales of kScaleChunk consecutive groups, group-major: ws[j][row],
    // s[j][token], t[j][token] for group kScaleChunk * c + j.
    static constexpr int kWsElems = kScaleChunk * BN;
    static constexpr int kStElems = kScaleChunk * BM;
    static constexpr int kWsPer = (kWsElems + kThreads - 1) / kThreads;
    static constexpr int kStPer = (kStElems + kThreads - 1) / kThreads;
    struct __align__(16) Scales {
        uint16_t ws[kScaleChunk][BN];
        float s[kScaleChunk][BM];
        int32_t t[kScaleChunk][BM];
    };
};

// 16-byte staging chunks: global -> registers (buffer loads: fixed per-lane
// offset plus a uniform group offset), registers -> LDS. Native vector
// types: copies of the HIP uint4 struct become memcpys that can leave the
// staging registers in scratch memory.
template <int P>
__device__ __forceinline__ void load_chunks(v4i (&dst)[P], __amdgpu_buffer_rsrc_t rs,
                                            const uint32_t (&off)[P], uint32_t goff) {
#pragma unroll
    for (int i = 0; i < P; ++i)
        dst[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off[i], (int)goff, 0);
}

template <int CHUNKS, int THREADS, int P>
__device__ __forceinline__ void store_chunks(const v4i (&src)[P], uint8_t *lds,
                                             const int (&dst)[P], int tid) {
#pragma unroll
    for (int i = 0; i < P; ++i)
        if (CHUNKS % THREADS == 0 || tid + i * THREADS < CHUNKS)
            *reinterpret_cast<v4i *>(lds + dst[i]) = src[i];
}

// Per-lane constants of the compute step.
struct LaneCtx {
    int row_base, tok_base, r, lg, half, sh0, G;
    int64_t m0, n0, M, N;
    int32_t *d;
};

// One group from an LDS stage and the group's scale tables (ws_g, s_g, t_g:
// row / token-indexed LDS rows). Every LDS read of the group (code words and
// weight scales of the wave's WN row tiles, activations and token scales of
// its WM token tiles) is issued first, so their latency is paid once per
// group; then per token tile the 2 * WN MFMAs are issued before their
// epilogue (or the exact dots).
template <int WN, int WM, bool DOTS, class Stage>
__device__ __forceinline__ void compute_group(const Stage &cur, const uint16_t *ws_g,
                                              const float *s_g, const int32_t *t_g,
                                              float (&acc)[WN][WM][4], const LaneCtx &c_, int g) {
    v4i w[WN], b0[WM], b1[WM];
    uint2 wsw[WN];
    int tt[WM];
    float sv[WM];
#pragma unroll
    for (int a = 0; a < WN; ++a) {
        w[a] = *reinterpret_cast<const v4i *>(
            cur.codes + (c_.row_base + 16 * a + c_.r) * kCodeStride + 16 * c_.half);
        if (!DOTS)
            wsw[a] = *reinterpret_cast<const uint2 *>(ws_g + c_.row_base + 16 * a + 4 * c_.lg);
    }
#pragma unroll
    for (int b = 0; b < WM; ++b) {
        const int tok = c_.tok_base + 16 * b + c_.r;
        const int8_t *qrow = cur.q + tok * kQStride + 16 * c_.lg;
        b0[b] = *reinterpret_cast<const v4i *>(qrow);
        b1[b] = *reinterpret_cast<const v4i *>(qrow + 64);
        tt[b] = t_g[tok];
        sv[b] = DOTS ? 0.0f : s_g[tok];
    }
    __builtin_amdgcn_sched_barrier(0);
    v4i a0[WN], a1[WN];
    _Float16 wsh[WN][4];
#pragma unroll
    for (int a = 0; a < WN; ++a) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t sh = (uint32_t)w[a][j] >> c_.sh0;
            a0[a][j] = (int)(sh & kPlaneMask);
            a1[a][j] = (int)((sh >> 4) & kPlaneMask);
        }
        if (!DOTS) {
            wsh[a][0] = __builtin_bit_cast(_Float16, (uint16_t)(wsw[a].x & 0xffff));
            wsh[a][1] = __builtin_bit_cast(_Float16, (uint16_t)(wsw[a].x >> 16));
            wsh[a][2] = __builtin_bit_cast(_Float16, (uint16_t)(wsw[a].y & 0xffff));
            wsh[a][3] = __builtin_bit_cast(_Float16, (uint16_t)(wsw[a].y >> 16));
        }
    }
#pragma unroll
    for (int b = 0; b < WM; ++b) {
        const v4i seed = {-tt[b], -tt[b], -tt[b], -tt[b]};
        v4i c[WN];
#pragma unroll
        for (int a = 0; a < WN; ++a) c[a] = mfma16x16x64(a0[a], b0[b], seed);
#pragma unroll
        for (int a = 0; a < WN; ++a) c[a] = mfma16x16x64(a1[a], b1[b], c[a]);
#pragma unroll
        for (int a = 0; a < WN; ++a) {
            if (DOTS) {
                const int64_t m = c_.m0 + c_.tok_base + 16 * b + c_.r;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t n = c_.n0 + c_.row_base + 16 * a + 4 * c_.lg + i;
                    if (m < c_.M && n < c_.N) c_.d[(m * c_.N + n) * c_.G + g] = c[a][i];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[a][b][i] = fmaf((float)c[a][i], scale_product(sv[b], wsh[a][i]), acc[a][b][i]);
            }
        }
    }
}

template <int WN, int WM, int WAVES_N, int WAVES_M, int DEPTH, bool DOTS>
__global__ __launch_bounds__(64 * WAVES_N * WAVES_M) void prefill_mfma_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    uint16_t *__restrict__ y16, int32_t *__restrict__ d, int64_t M, int64_t N, int64_t K) {
    using C = PfCfg<WN, WM, WAVES_N, WAVES_M>;
    using Stage = typename C::Stage;
    using Scales = typename C::Scales;
    __shared__ Stage stage[2];
    __shared__ Scales scl[2];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wn = wave % WAVES_N, wm = wave / WAVES_N;
    const int r = lane & 15, lg = lane >> 4;
    const int half = lg & 1;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);
    const int64_t KB = K / 4;                // code bytes per row

    const int64_t tiles_n = (N + C::BN - 1) / C::BN;
    const int64_t tiles_m = (M + C::BM - 1) / C::BM;
    const int64_t tile = xcd_tile(blockIdx.x, tiles_n * tiles_m);
    const int64_t n0 = (tile % tiles_n) * C::BN;
    const int64_t m0 = (tile / tiles_n) * C::BM;

    // Buffer resources based at the block's first row and token; per-lane
    // 32-bit offsets (the host bounds K so that BN * K / 4 and BM * K fit in
    // 32 bits) and a uniform offset per group.
    const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(codes + n0 * KB, (N - n0) * KB);
    const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + m0 * K, (M - m0) * K);
    const __amdgpu_buffer_rsrc_t rs_t = make_rsrc(t + m0 * G, (M - m0) * G * 4);
    const __amdgpu_buffer_rsrc_t rs_ws = make_rsrc(DOTS ? nullptr : ws + n0 * G, DOTS ? 0 : (N - n0) * G * 2);
    const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(DOTS ? nullptr : s + m0 * G, DOTS ? 0 : (M - m0) * G * 4);

    // staging assignment: chunk c of codes is (row c/2, half c%2); chunk c of
    // q is (token c/8, 16-byte piece c%8). Rows and tokens past the end are
    // clamped to the last one (their results are never stored).
    uint32_t code_off[C::kCodePer];
    int code_dst[C::kCodePer];
#pragma unroll
    for (int i = 0; i < C::kCodePer; ++i) {
        int c = tid + i * C::kThreads;
        if (c >= C::kCodeChunks) c = C::kCodeChunks - 1;
        const int row = c >> 1, hh = c & 1;
        const int64_t rel = (n0 + row < N) ? row : N - 1 - n0;
        code_off[i] = (uint32_t)(rel * KB + 16 * hh);
        code_dst[i] = row * kCodeStride + 16 * hh;
    }
    uint32_t q_off[C::kQPer];
    int q_dst[C::kQPer];
#pragma unroll
    for (int i = 0; i < C::kQPer; ++i) {
        int c = tid + i * C::kThreads;
        if (c >= C::kQChunks) c = C::kQChunks - 1;
        const int tok = c >> 3, piece = c & 7;
        const int64_t rel = (m0 + tok < M) ? tok : M - 1 - m0;
        q_off[i] = (uint32_t)(rel * K + 16 * piece);
        q_dst[i] = tok * kQStride + 16 * piece;
    }
    // scale-chunk assignment: element e = tid + i * kThreads is (row or token
    // e / kScaleChunk, group offset e % kScaleChunk); kThreads is a multiple
    // of kScaleChunk, so a thread's group offset sc_j is the same for all i
    // and its rows step by kThreads / kScaleChunk.
    static_assert(C::kThreads % kScaleChunk == 0, "scale chunk layout");
    constexpr int kRowStep = C::kThreads / kScaleChunk;
    const int sc_j = tid % kScaleChunk, sc_row = tid / kScaleChunk;
    // Staging loads are never predicated (groups past the end are clamped to
    // the last group), which keeps their registers out of scratch memory and
    // the wait counts exact; only the LDS writes of ragged chunk counts are.
#define PQ2_PF_FETCH(gg, RC, RQ)                                                      \
    do {                                                                            \
        const uint32_t g_ = (uint32_t)((gg) < G ? (gg) : G - 1);                    \
        load_chunks(RC, rs_codes, code_off, 32u * g_);                              \
        load_chunks(RQ, rs_q, q_off, (uint32_t)kGroup * g_);                        \
        __builtin_amdgcn_sched_barrier(0);                                          \
    } while (0)
#define PQ2_PF_COMMIT(st, RC, RQ)                                                     \
    do {                                                                            \
        __builtin_amdgcn_sched_barrier(0);                                          \
        store_chunks<C::kCodeChunks, C::kThreads>(RC, (st).codes, code_dst, tid);   \
        store_chunks<C::kQChunks, C::kThreads>(RQ, (uint8_t *)(st).q, q_dst, tid);  \
    } while (0)
    // scale chunk cc: group kScaleChunk * cc + j, clamped to the last group
#define PQ2_PF_SCALE_FETCH(cc)                                                        \
    do {                                                                            \
        const int gi_ = kScaleChunk * (cc) + sc_j < G ? kScaleChunk * (cc) + sc_j : G - 1; \
        if (!DOTS) {                                                                \
            _Pragma("unroll") for (int i = 0; i < C::kWsPer; ++i) {                 \
                int row = sc_row + i * kRowStep;                                    \
                row = row < C::BN ? row : C::BN - 1;                                \
                row = n0 + row < N ? row : (int)(N - 1 - n0);                       \
                rws[i] = __builtin_amdgcn_raw_buffer_load_b16(                      \
                    rs_ws, (int)(2u * ((uint32_t)row * (uint32_t)G + (uint32_t)gi_)), 0, 0); \
            }                                                                       \
        }                                                                           \
        _Pragma("unroll") for (int i = 0; i < C::kStPer; ++i) {                     \
            int tok = sc_row + i * kRowStep;                                        \
            tok = tok < C::BM ? tok : C::BM - 1;                                    \
            tok = m0 + tok < M ? tok : (int)(M - 1 - m0);                           \
            const int off = (int)(4u * ((uint32_t)tok * (uint32_t)G + (uint32_t)gi_)); \
            if (!DOTS) rss[i] = __builtin_amdgcn_raw_buffer_load_b32(rs_s, off, 0, 0); \
            rts[i] = __builtin_amdgcn_raw_buffer_load_b32(rs_t, off, 0, 0);         \
        }                                                                           \
    } while (0)
#define PQ2_PF_SCALE_COMMIT(buf)                                                      \
    do {                                                                            \
        if (!DOTS) {                                                                \
            _Pragma("unroll") for (int i = 0; i < C::kWsPer; ++i)                   \
                if (C::kWsElems % C::kThreads == 0 || tid + i * C::kThreads < C::kWsElems) \
                    (buf).ws[sc_j][sc_row + i * kRowStep] = rws[i];                 \
        }                                                                           \
        _Pragma("unroll") for (int i = 0; i < C::kStPer; ++i)                       \
            if (C::kStElems % C::kThreads == 0 || tid + i * C::kThreads < C::kStElems) { \
                if (!DOTS) (buf).s[sc_j][sc_row + i * kRowStep] = __builtin_bit_cast(float, rss[i]); \
                (buf).t[sc_j][sc_row + i * kRowStep] = (int32_t)rts[i];             \
            }                                                                       \
    } while (0)
    // one group: scale chunk loads every kScaleChunk groups (committed in the
    // same iteration, into the buffer the previous chunk used)
#define PQ2_PF_STEP(gg, CUR, NXT, RC_F, RQ_F, RC_C, RQ_C, FETCH_G)                     \
    do {                                                                            \
        const int cc_ = (gg) / kScaleChunk, jj_ = (gg) % kScaleChunk;               \
        const bool sc_ = jj_ == 0 && (gg) + kScaleChunk < G;                        \
        if (sc_) PQ2_PF_SCALE_FETCH(cc_ + 1);                                       \
        PQ2_PF_FETCH(FETCH_G, RC_F, RQ_F);                                          \
        const Scales &sb_ = scl[cc_ & 1];                                           \
        compute_group<WN, WM, DOTS>(CUR, sb_.ws[jj_], sb_.s[jj_], sb_.t[jj_], acc, ctx, (gg)); \
        PQ2_PF_COMMIT(NXT, RC_C, RQ_C);                                             \
        if (sc_) PQ2_PF_SCALE_COMMIT(scl[(cc_ + 1) & 1]);                           \
        __syncthreads();                                                            \
    } while (0)

    float acc[WN][WM][4];
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
        for (int b = 0; b < WM; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;

    LaneCtx ctx;
    ctx.row_base = 16 * WN * wn;    // wave's first row within the block tile
    ctx.tok_base = 16 * WM * wm;    // wave's first token within the block tile
    ctx.r = r;
    ctx.lg = lg;
    ctx.half = half;
    ctx.sh0 = sh0;
    ctx.m0 = m0;
    ctx.n0 = n0;
    ctx.M = M;
    ctx.N = N;
    ctx.G = G;
    ctx.d = d;

    uint16_t rws[C::kWsPer];
    uint32_t rss[C::kStPer], rts[C::kStPer];
#pragma unroll
    for (int i = 0; i < C::kWsPer; ++i) rws[i] = 0;
#pragma unroll
    for (int i = 0; i < C::kStPer; ++i) rss[i] = rts[i] = 0;
    PQ2_PF_SCALE_FETCH(0);
    PQ2_PF_SCALE_COMMIT(scl[0]);

    v4i rcA[C::kCodePer], rqA[C::kQPer];
    int g = 0;
    if constexpr (DEPTH == 2) {
        v4i rcB[C::kCodePer], rqB[C::kQPer];
        PQ2_PF_FETCH(0, rcA, rqA);
        PQ2_PF_FETCH(1, rcB, rqB);
        PQ2_PF_COMMIT(stage[0], rcA, rqA);
        __syncthreads();
        for (; g + 1 < G; g += 2) {
            // stage 0 holds group g, set B carries group g+1, set A fetches g+2
            PQ2_PF_STEP(g, stage[0], stage[1], rcA, rqA, rcB, rqB, g + 2);
            // stage 1 holds group g+1, set A carries group g+2, set B fetches g+3
            PQ2_PF_STEP(g + 1, stage[1], stage[0], rcB, rqB, rcA, rqA, g + 3);
        }
        if (g < G) {   // odd G: the last group is in stage 0
            const Scales &sb = scl[(g / kScaleChunk) & 1];
            const int jj = g % kScaleChunk;
            compute_group<WN, WM, DOTS>(stage[0], sb.ws[jj], sb.s[jj], sb.t[jj], acc, ctx, g);
        }
    } else {
        PQ2_PF_FETCH(0, rcA, rqA);
        PQ2_PF_COMMIT(stage[0], rcA, rqA);
        __syncthreads();
        for (; g < G; ++g) PQ2_PF_STEP(g, stage[g & 1], stage[(g + 1) & 1], rcA, rqA, rcA, rqA, g + 1);
    }
#undef PQ2_PF_FETCH
#undef PQ2_PF_COMMIT
#undef PQ2_PF_SCALE_FETCH
#undef PQ2_PF_SCALE_COMMIT
#undef PQ2_PF_STEP

    if (!DOTS) {
#pragma unroll
        for (int b = 0; b < WM; ++b) {
            const int64_t m = m0 + ctx.tok_base + 16 * b + r;
#pragma unroll
            for (int a = 0; a < WN; ++a) {
                const int64_t nb = n0 + ctx.row_base + 16 * a + 4 * lg;
                if (m < M) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (nb + i < N) store_y(y, y16, m * N + nb + i, acc[a][b][i]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- ring variant
//
// Same tiles, operand mapping and arithmetic, but the per-group operands reach
// LDS by 16-byte buffer -> LDS copies (no VGPRs held), so R - 1 groups are in
// flight while one is computed. Every thread issues the same copies per
// group (lanes past a region read past the buffer range, which moves no
// memory), so one explicit vmcnt wait per group covers that group's copies.
// Stage layout (16-byte units; copy instruction i of wave w writes units
// 256 i + 64 w + lane of a region, or a sink when those lie past it): code
// unit 2 row + (half ^ ((row >> 2) & 1)), then q
// unit 8 token + (piece ^ (token & 7)) -- every 128-byte line is fetched by
// one instruction, and the 16-lane operand reads hit distinct LDS banks.
// Scales of groups 8c .. 8c + 7 travel as one chunk: ws unit row (8 halves),
// s and t units 2 token + h (4 floats each), issued at group 8c - 8 into the
// other of two chunk slots.
template <int BN, int BM, int T, bool DOTS>
struct PfRing {
    // copies per thread; a wave whose units of an instruction all lie past a
    // region copies into a shared 1 KB sink instead, so each region only
    // spans its units rounded up to a wave (64 units)
    static constexpr int kCodeInst = (2 * BN + T - 1) / T;
    static constexpr int kQInst = (8 * BM + T - 1) / T;
    static constexpr int kStageInst = kCodeInst + kQInst;
    static constexpr int kCodeUnits = (2 * BN + 63) / 64 * 64;
    static constexpr int kQUnits = (8 * BM + 63) / 64 * 64;
    static constexpr int kQBase = kCodeUnits;                      // first q unit
    static constexpr int kStageBytes = (kCodeUnits + kQUnits) * 16;
    static constexpr int kWsInst = DOTS ? 0 : (BN + T - 1) / T;
    static constexpr int kTokInst = (2 * BM + T - 1) / T;          // per s or t table
    static constexpr int kScaleInst = kWsInst + (DOTS ? 1 : 2) * kTokInst;
    static constexpr int kWsUnits = DOTS ? 0 : (BN + 63) / 64 * 64;
    static constexpr int kTokUnits = (2 * BM + 63) / 64 * 64;
    static constexpr int kSBase = kWsUnits;                        // first s unit
    static constexpr int kTBase = kSBase + (DOTS ? 0 : kTokUnits);
    static constexpr int kScaleBytes = (kTBase + kTokUnits) * 16;
    static constexpr int kSinkBytes = 1024;
};

template <int WN, int WM, int WAVES_N, int WAVES_M, int R, bool DOTS>
__global__ __launch_bounds__(64 * WAVES_N * WAVES_M) void prefill_ring_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    uint16_t *__restrict__ y16, int32_t *__restrict__ d, int64_t M, int64_t N, int64_t K) {
    using C = PfCfg<WN, WM, WAVES_N, WAVES_M>;
    constexpr int T = C::kThreads;
    using L = PfRing<C::BN, C::BM, T, DOTS>;
    static_assert(R >= 2 && R <= 8, "the scale chunk of group 8c + 8 must land before it");
    constexpr int CPS = L::kStageInst;
    constexpr int SI = L::kScaleInst;
    static_assert((R - 2) * CPS + SI < 64, "vmcnt holds 6 bits");
    // dynamic LDS: [R] stages, then [2] scale chunks (with static arrays the
    // compiler sees the copies' target and drains every copy before each read)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *const ring0 = smem;
    uint8_t *const scl0 = smem + R * L::kStageBytes;
    uint8_t *const sink = scl0 + 2 * L::kScaleBytes;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    // LDS destination of copy instruction i of this wave into a region of
    // `units` units at `base` (past the region: the sink)
    auto dst = [&](uint8_t *base, int units, int i) __attribute__((always_inline)) {
        const int u = i * T + kWave * wave;
        return u < units ? base + u * 16 : sink;
    };
    const int wn = wave % WAVES_N, wm = wave / WAVES_N;
    const int r = lane & 15, lg = lane >> 4;
    const int half = lg & 1;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);
    const int KB = (int)(K / 4);

    const int64_t tiles_n = (N + C::BN - 1) / C::BN;
    const int64_t tiles_m = (M + C::BM - 1) / C::BM;
    const int64_t tile = xcd_tile(blockIdx.x, tiles_n * tiles_m);
    const int64_t n0 = (tile % tiles_n) * C::BN;
    const int64_t m0 = (tile / tiles_n) * C::BM;
    const int rows = N - n0 < C::BN ? (int)(N - n0) : C::BN;
    const int toks = M - m0 < C::BM ? (int)(M - m0) : C::BM;

    const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(codes + n0 * KB, (int64_t)rows * KB);
    const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + m0 * K, (int64_t)toks * K);
    const __amdgpu_buffer_rsrc_t rs_t = make_rsrc(t + m0 * G, (int64_t)toks * G * 4);
    const __amdgpu_buffer_rsrc_t rs_ws = make_rsrc(DOTS ? nullptr : ws + n0 * G, DOTS ? 0 : (int64_t)rows * G * 2);
    const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(DOTS ? nullptr : s + m0 * G, DOTS ? 0 : (int64_t)toks * G * 4);

    // per-thread copy sources (group 0; group g adds 32 g or 128 g); rows and
    // tokens past the end read past the range (zeros, never stored)
    int coff[L::kCodeInst], qoff[L::kQInst];
#pragma unroll
    for (int i = 0; i < L::kCodeInst; ++i) {
        const int u = i * T + tid;
        const int row = u >> 1;
        const int h = (u & 1) ^ ((row >> 2) & 1);
        coff[i] = u < 2 * C::BN && row < rows ? row * KB + 16 * h : kCopyOob;
    }
#pragma unroll
    for (int i = 0; i < L::kQInst; ++i) {
        const int u = i * T + tid;
        const int tok = u >> 3;
        const int piece = (u & 7) ^ (tok & 7);
        qoff[i] = u < 8 * C::BM && tok < toks ? tok * (int)K + 16 * piece : kCopyOob;
    }
    // scale chunk sources (chunk 0; chunk c adds 16 c bytes for ws, 32 c for s / t)
    int wsoff[L::kWsInst > 0 ? L::kWsInst : 1], toff[L::kTokInst];
#pragma unroll
    for (int i = 0; i < L::kWsInst; ++i) {
        const int u = i * T + tid;
        wsoff[i] = u < C::BN && u < rows ? 2 * u * G : kCopyOob;
    }
#pragma unroll
    for (int i = 0; i < L::kTokInst; ++i) {
        const int u = i * T + tid;
        const int tok = u >> 1;
        toff[i] = u < 2 * C::BM && tok < toks ? 4 * (tok * G + 4 * (u & 1)) : kCopyOob;
    }

    auto issue_stage = [&](int g) __attribute__((always_inline)) {
        const bool live = g < G;
        uint8_t *st = ring0 + (g % R) * L::kStageBytes;
#pragma unroll
        for (int i = 0; i < L::kCodeInst; ++i)
            copy16_to_lds(rs_codes, dst(st, L::kCodeUnits, i),
                          live && coff[i] != kCopyOob ? coff[i] + 32 * g : kCopyOob);
#pragma unroll
        for (int i = 0; i < L::kQInst; ++i)
            copy16_to_lds(rs_q, dst(st + L::kQBase * 16, L::kQUnits, i),
                          live && qoff[i] != kCopyOob ? qoff[i] + kGroup * g : kCopyOob);
    };
    auto issue_scales = [&](int c) __attribute__((always_inline)) {
        const bool live = 8 * c < G;
        uint8_t *sc = scl0 + (c & 1) * L::kScaleBytes;
#pragma unroll
        for (int i = 0; i < L::kWsInst; ++i)
            copy16_to_lds(rs_ws, dst(sc, L::kWsUnits, i),
                          live && wsoff[i] != kCopyOob ? wsoff[i] + 16 * c : kCopyOob);
        if (!DOTS) {
#pragma unroll
            for (int i = 0; i < L::kTokInst; ++i)
                copy16_to_lds(rs_s, dst(sc + L::kSBase * 16, L::kTokUnits, i),
                              live && toff[i] != kCopyOob ? toff[i] + 32 * c : kCopyOob);
        }
#pragma unroll
        for (int i = 0; i < L::kTokInst; ++i)
            copy16_to_lds(rs_t, dst(sc + L::kTBase * 16, L::kTokUnits, i),
                          live && toff[i] != kCopyOob ? toff[i] + 32 * c : kCopyOob);
    };

    const int row_base = 16 * WN * wn;
    const int tok_base = 16 * WM * wm;
    float acc[WN][WM][4];
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
        for (int b = 0; b < WM; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;

    // a group's operands, read from its stage and scale chunk into VGPRs
    struct Ops {
        v4i w[WN], b0[WM], b1[WM];
        int tt[WM];
        float sv[WM];
        uint16_t wsh[WN][4];
    };
    auto load_ops = [&](int g, Ops &o) __attribute__((always_inline)) {
        const uint8_t *st = ring0 + (g % R) * L::kStageBytes;
        const uint8_t *sc = scl0 + ((g >> 3) & 1) * L::kScaleBytes;
        const int j = g & 7;
        const uint16_t *wsl = reinterpret_cast<const uint16_t *>(sc) + j;
        const float *sl = reinterpret_cast<const float *>(sc + L::kSBase * 16) + j;
        const int32_t *tl = reinterpret_cast<const int32_t *>(sc + L::kTBase * 16) + j;
#pragma unroll
        for (int a = 0; a < WN; ++a) {
            const int row = row_base + 16 * a + r;
            o.w[a] = *reinterpret_cast<const v4i *>(st + 16 * (2 * row + (half ^ ((row >> 2) & 1))));
            if (!DOTS) {
#pragma unroll
                for (int i = 0; i < 4; ++i) o.wsh[a][i] = wsl[8 * (row_base + 16 * a + 4 * lg + i)];
            }
        }
#pragma unroll
        for (int b = 0; b < WM; ++b) {
            const int tok = tok_base + 16 * b + r;
            const uint8_t *qrow = st + (L::kQBase + 8 * tok) * 16;
            o.b0[b] = *reinterpret_cast<const v4i *>(qrow + 16 * (lg ^ (tok & 7)));
            o.b1[b] = *reinterpret_cast<const v4i *>(qrow + 16 * ((lg + 4) ^ (tok & 7)));
            o.tt[b] = tl[8 * tok];
            o.sv[b] = DOTS ? 0.0f : sl[8 * tok];
        }
    };
    // plane decode, then per token tile the 2 WN MFMAs and their epilogue (the
    // compiler overlaps one tile's epilogue with the next tile's MFMAs; issuing
    // every MFMA of the group before any epilogue measured 1.5-1.9x slower)
    auto mma = [&](const Ops &o, int g) __attribute__((always_inline)) {
        v4i a0[WN], a1[WN];
        _Float16 wsh[WN][4];
#pragma unroll
        for (int a = 0; a < WN; ++a) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t sh = (uint32_t)o.w[a][k] >> sh0;
                a0[a][k] = (int)(sh & kPlaneMask);
                a1[a][k] = (int)((sh >> 4) & kPlaneMask);
            }
            if (!DOTS) {
#pragma unroll
                for (int i = 0; i < 4; ++i) wsh[a][i] = __builtin_bit_cast(_Float16, o.wsh[a][i]);
            }
        }
#pragma unroll
        for (int b = 0; b < WM; ++b) {
            const v4i seed = {-o.tt[b], -o.tt[b], -o.tt[b], -o.tt[b]};
            v4i c[WN];
#pragma unroll
            for (int a = 0; a < WN; ++a) c[a] = mfma16x16x64(a0[a], o.b0[b], seed);
#pragma unroll
            for (int a = 0; a < WN; ++a) c[a] = mfma16x16x64(a1[a], o.b1[b], c[a]);
#pragma unroll
            for (int a = 0; a < WN; ++a) {
                if (DOTS) {
                    const int64_t m = m0 + tok_base + 16 * b + r;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + row_base + 16 * a + 4 * lg + i;
                        if (m < M && n < N) d[(m * N + n) * G + g] = c[a][i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[a][b][i] = fmaf((float)c[a][i], scale_product(o.sv[b], wsh[a][i]),
                                            acc[a][b][i]);
                }
            }
        }
    };

    // prologue: scale chunk 0, then the first R - 1 stages
    issue_scales(0);
#pragma unroll
    for (int p = 0; p < R - 1; ++p) issue_stage(p);
    for (int g = 0; g < G; ++g) {
        // copies younger than stage g: stages g + 1 .. g + R - 2, and the
        // scale chunk issued at the last group 8c in [g - R + 1, g - 1]
        const bool scale_after = g >= 1 && ((g - 1) & ~7) >= g - R + 1;
        if (scale_after)
            wait_vmem<(R - 2) * CPS + SI>();
        else
            wait_vmem<(R - 2) * CPS>();
        ring_barrier();                          // stage g in LDS; stage g - 1 free
        issue_stage(g + R - 1);
        if ((g & 7) == 0) issue_scales((g >> 3) + 1);
        Ops o;
        load_ops(g, o);
        __builtin_amdgcn_sched_barrier(0);
        mma(o, g);
    }
    wait_vmem<0>();                              // no copy may land after the block ends

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
                        if (nb + i < N) store_y(y, y16, m * N + nb + i, acc[a][b][i]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- wide variant
//
// Block tile 256 weight rows x 128 tokens: four waves side by side along N,
// each owning 64 rows x 128 tokens (4 x 8 MFMA tiles), so the code words a
// wave decodes per group serve eight token tiles, and the block's buffer ->
// LDS copies move 24 KB per group for 32768 outputs (8 KB codes, 16 KB
// activations). The scale products s[m] * ws[n] come from the matrix core:
// per group, token tile and row tile one v_mfma_f32_4x4x1_16b forms the
// outer products of weight and token scales in sixteen 4 x 4 blocks, lane
// 4k + i supplying row i and column i of block k: with the weight scale of
// row 4 (lane / 16) + (lane % 4) and the token scale of token lane % 16 as
// operands, block k's result lands in the lanes and registers that hold the
// int8 results of the same outputs. That leaves the VALU one conversion and
// one FMA per output and group (measured here, MFMA and VALU time add up
// rather than overlap, so VALU work moved to the matrix core is time saved
// as long as it costs fewer cycles there). The product is the correctly
// rounded float32 product the other tiles form with a mixed-precision FMA,
// and the accumulation order over groups is the same: results are
// identical.
// Staging as in the ring variant, with two stages and the group offset of
// every copy in the SGPR operand: stage g + 1 (and every eight groups the
// next scale chunk) is copied while group g is computed.
template <bool DOTS, int WM_>
struct PfWide {
    static constexpr int T = 256, BN = 256, WN = 4, WM = WM_, BM = 16 * WM;
    static constexpr int kCodeInst = 2 * BN / T;          // code units per thread
    static constexpr int kQInst = 8 * BM / T;             // activation units per thread
    static constexpr int kStageInst = kCodeInst + kQInst;
    static constexpr int kQBase = 2 * BN * 16;            // activation bytes of a stage
    static constexpr int kStageBytes = kQBase + 8 * BM * 16;
    // scale chunk of 8 groups: ws unit per row (8 halves), then s and t in
    // two units per token (8 values each)
    static constexpr int kSBase = BN * 16;
    static constexpr int kTBase = kSBase + BM * 32;
    static constexpr int kScaleBytes = kTBase + BM * 32;
    static constexpr int kScaleInst = DOTS ? 1 : 3;
    // s and t have 2 BM units: with fewer than T, the waves past them copy
    // into a 1 KB sink (their lanes read no memory)
    static constexpr int kSinkBase = 2 * kStageBytes + 2 * kScaleBytes;
    static constexpr int kLdsBytes = kSinkBase + (2 * BM < T ? 1024 : 0);
    static_assert(T == BN && 2 * BM <= T && (2 * BM) % kWave == 0, "scale units per thread");
};

typedef float v4f __attribute__((ext_vector_type(4)));

// K split of the last tiles of the wide variant (see prefill_wide_kernel);
// full = every tile and chunks = 1 when nothing is split.
struct WideSplit {
    int64_t full;        // tiles computed whole
    int chunks;          // K chunks per remaining tile
    int chunk_groups;    // groups per chunk (even)
    float *part;         // (tiles - full) * chunks partial [BM][BN] tiles
};

// y of the split tiles: the chunks' partial sums added in chunk order. One
// block per (tile, token row), one thread per weight row.
template <int BM>
__global__ __launch_bounds__(256) void wide_tail_sum_kernel(const float *__restrict__ part,
                                                            float *__restrict__ y,
                                                            uint16_t *__restrict__ y16, int64_t M,
                                                            int64_t N, WideSplit sp) {
    constexpr int BN = 256;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t v = blockIdx.x / BM;                 // split tile index
    const int ml = blockIdx.x % BM;
    const int64_t tile = sp.full + v;
    const int64_t m = (tile / tiles_n) * BM + ml;
    const int64_t n = (tile % tiles_n) * BN + threadIdx.x;
    if (m >= M || n >= N) return;
    const float *p = part + v * sp.chunks * (BM * BN) + ml * BN + threadIdx.x;
    float acc = p[0];
    for (int c = 1; c < sp.chunks; ++c) acc += p[(int64_t)c * (BM * BN)];
    store_y(y, y16, m * N + n, acc);
}

template <bool DOTS, int WM_>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void prefill_wide_kernel(const int8_t *__restrict__ q, const float *__restrict__ s,
                         const int32_t *__restrict__ t, const uint8_t *__restrict__ codes,
                         const uint16_t *__restrict__ ws, float *__restrict__ y,
                         uint16_t *__restrict__ y16, int32_t *__restrict__ d, int64_t M,
                         int64_t N, int64_t K, WideSplit sp) {
    using L = PfWide<DOTS, WM_>;
    constexpr int T = L::T, WN = L::WN, WM = L::WM;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    uint8_t *const stage0 = smem;
    uint8_t *const stage1 = smem + L::kStageBytes;
    uint8_t *const scl0 = smem + 2 * L::kStageBytes;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int r = lane & 15, lg = lane >> 4;
    const int half = lg & 1;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);
    const int KB = (int)(K / 4);

    const int64_t tiles_n = (N + L::BN - 1) / L::BN;
    // Dispatch slots below sp.full run whole tiles 0 .. sp.full - 1 (in XCD
    // order); slot sp.full + u runs K chunk u % sp.chunks (groups
    // chunk * sp.chunk_groups onward) of tile sp.full + u / sp.chunks and
    // leaves its partial sums in sp.part[u] ([BM][BN] float32).
    int64_t tile;
    int g0 = 0, g1 = G;
    float *partial = nullptr;
    if ((int64_t)blockIdx.x < sp.full) {
        tile = xcd_tile(blockIdx.x, sp.full);
    } else {
        const int64_t u = (int64_t)blockIdx.x - sp.full;
        tile = sp.full + u / sp.chunks;
        g0 = (int)(u % sp.chunks) * sp.chunk_groups;
        g1 = g0 + sp.chunk_groups < G ? g0 + sp.chunk_groups : G;
        partial = sp.part + u * (L::BM * L::BN);
    }
    const int64_t n0 = (tile % tiles_n) * L::BN;
    const int64_t m0 = (tile / tiles_n) * L::BM;
    const int rows = N - n0 < L::BN ? (int)(N - n0) : L::BN;
    const int toks = M - m0 < L::BM ? (int)(M - m0) : L::BM;

    const __amdgpu_buffer_rsrc_t rs_codes = make_rsrc(codes + n0 * KB, (int64_t)rows * KB);
    const __amdgpu_buffer_rsrc_t rs_q = make_rsrc(q + m0 * K, (int64_t)toks * K);
    const __amdgpu_buffer_rsrc_t rs_t = make_rsrc(t + m0 * G, (int64_t)toks * G * 4);
    const __amdgpu_buffer_rsrc_t rs_ws = make_rsrc(DOTS ? nullptr : ws + n0 * G, DOTS ? 0 : (int64_t)rows * G * 2);
    const __amdgpu_buffer_rsrc_t rs_s = make_rsrc(DOTS ? nullptr : s + m0 * G, DOTS ? 0 : (int64_t)toks * G * 4);

    // Copy sources of group 0 (group g adds 32 g or 128 g through the SGPR
    // offset). Unit u of copy instruction i is i * T + tid; code unit
    // 2 row + (half ^ ((row >> 2) & 1)), activation unit 8 token +
    // (piece ^ (token & 7)), as in the ring variant. Rows and tokens past the
    // end are never read (their LDS units receive zeros).
    int coff[L::kCodeInst], qoff[L::kQInst];
#pragma unroll
    for (int i = 0; i < L::kCodeInst; ++i) {
        const int u = i * T + tid;
        const int row = u >> 1;
        const int h = (u & 1) ^ ((row >> 2) & 1);
        coff[i] = row < rows ? row * KB + 16 * h : kCopyOob;
    }
#pragma unroll
    for (int i = 0; i < L::kQInst; ++i) {
        const int u = i * T + tid;
        const int tok = u >> 3;
        const int piece = (u & 7) ^ (tok & 7);
        qoff[i] = tok < toks ? tok * (int)K + 16 * piece : kCopyOob;
    }
    // scale chunk c: ws unit tid = row tid, groups 8c .. 8c + 7 (byte offset
    // 2 (row G + 8c)); s / t unit tid = token tid / 2, groups 8c + 4 (tid & 1)
    // .. + 3 (byte offset 4 (token G + 8c + 4 (tid & 1)))
    const int wsoff = tid < rows ? 2 * tid * G : kCopyOob;
    const int tokoff = (tid >> 1) < toks ? 4 * ((tid >> 1) * G + 4 * (tid & 1)) : kCopyOob;

    auto issue_stage = [&](int g, uint8_t *st) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < L::kCodeInst; ++i)
            copy16_to_lds_at(rs_codes, st + 16 * (i * T + kWave * wave), coff[i], 32 * g);
#pragma unroll
        for (int i = 0; i < L::kQInst; ++i)
            copy16_to_lds_at(rs_q, st + L::kQBase + 16 * (i * T + kWave * wave), qoff[i],
                             kGroup * g);
    };
    const bool tok_wave = kWave * wave < 2 * L::BM;   // this wave's s / t units exist
    auto issue_scales = [&](int c) __attribute__((always_inline)) {
        uint8_t *sc = scl0 + (c & 1) * L::kScaleBytes + 16 * kWave * wave;
        uint8_t *sink = smem + L::kSinkBase;
        if (!DOTS) {
            copy16_to_lds_at(rs_ws, sc, wsoff, 16 * c);
            copy16_to_lds_at(rs_s, tok_wave ? sc + L::kSBase : sink, tokoff, 32 * c);
        }
        copy16_to_lds_at(rs_t, tok_wave ? sc + L::kTBase : sink, tokoff, 32 * c);
    };

    const int row_base = 64 * wave;
    // per-lane LDS byte offsets: code words of row tile a at cbase + 512 a;
    // activation pieces lg and lg + 4 of token tile b at qb0 / qb1 + 2048 b;
    // s / t of token tile b, group j at tokb + 512 b + 4 j; the outer-product
    // weight scale of row tile a at wsb + 256 a + 2 j
    const int cbase = 32 * (row_base + r) + 16 * (half ^ ((r >> 2) & 1));
    const int qb0 = L::kQBase + 128 * r + 16 * (lg ^ (r & 7));
    const int qb1 = L::kQBase + 128 * r + 16 * ((lg + 4) ^ (r & 7));
    const int tokb = 32 * r;
    const int wsb = 16 * (row_base + 4 * lg + (lane & 3));

    float acc[WN][WM][4];
#pragma unroll
    for (int a = 0; a < WN; ++a)
#pragma unroll
        for (int b = 0; b < WM; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] = 0.0f;

    auto compute = [&](const uint8_t *st, int g) __attribute__((always_inline)) {
        const uint8_t *sc = scl0 + ((g >> 3) & 1) * L::kScaleBytes;
        const int j = g & 7;
        v4i w[WN];
#pragma unroll
        for (int a = 0; a < WN; ++a) w[a] = *reinterpret_cast<const v4i *>(st + cbase + 512 * a);
        // weight-scale operand of the outer products: lane 4k + i of row tile a
        // supplies ws of row 16 a + 4 (lane / 16) + i
        float wsa[WN];
        float sv[WM];
        if (!DOTS) {
#pragma unroll
            for (int a = 0; a < WN; ++a)
                wsa[a] = half_bits_to_float(
                    *reinterpret_cast<const uint16_t *>(sc + wsb + 256 * a + 2 * j));
#pragma unroll
            for (int b = 0; b < WM; ++b)
                sv[b] = *reinterpret_cast<const float *>(sc + L::kSBase + tokb + 512 * b + 4 * j);
        }
        v4i a0[WN], a1[WN];
#pragma unroll
        for (int a = 0; a < WN; ++a) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t sh = (uint32_t)w[a][k] >> sh0;
                a0[a][k] = (int)(sh & kPlaneMask);
                a1[a][k] = (int)((sh >> 4) & kPlaneMask);
            }
        }
        // token-tile pipeline: activations of tile b + 2 are read and the
        // MFMAs of tile b + 1 issued before tile b's epilogue
        v4i bq0[2], bq1[2];
        int ttq[2];
        auto load_tile = [&](int b, int slot) __attribute__((always_inline)) {
            bq0[slot] = *reinterpret_cast<const v4i *>(st + qb0 + 2048 * b);
            bq1[slot] = *reinterpret_cast<const v4i *>(st + qb1 + 2048 * b);
            ttq[slot] = *reinterpret_cast<const int32_t *>(sc + L::kTBase + tokb + 512 * b + 4 * j);
        };
        v4i c[2][WN];
        auto mma = [&](int slot) __attribute__((always_inline)) {
            const int tt = ttq[slot];
            const v4i seed = {-tt, -tt, -tt, -tt};
#pragma unroll
            for (int a = 0; a < WN; ++a) c[slot][a] = mfma16x16x64(a0[a], bq0[slot], seed);
#pragma unroll
            for (int a = 0; a < WN; ++a) c[slot][a] = mfma16x16x64(a1[a], bq1[slot], c[slot][a]);
        };
        load_tile(0, 0);
        load_tile(1, 1);
        mma(0);
#pragma unroll
        for (int b = 0; b < WM; ++b) {
            const int cur = b & 1;
            if (b + 2 < WM) load_tile(b + 2, cur);
            if (b + 1 < WM) mma(cur ^ 1);
            if (DOTS) {
                const int64_t m = m0 + 16 * b + r;
                int64_t at = (m * N + n0 + row_base + 4 * lg) * G + g;
                // recomputed per tile: hoisted, the 128 store addresses of a group
                // would not fit in registers
                asm volatile("" : "+v"(at));
#pragma unroll
                for (int a = 0; a < WN; ++a)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + row_base + 16 * a + 4 * lg + i;
                        if (m < M && n < N) d[at + (int64_t)(16 * a + i) * G] = c[cur][a][i];
                    }
            } else {
#pragma unroll
                for (int a = 0; a < WN; ++a) {
                    const v4f sp = __builtin_amdgcn_mfma_f32_4x4x1f32(wsa[a], sv[b], v4f{}, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[a][b][i] = fmaf((float)c[cur][a][i], sp[i], acc[a][b][i]);
                    // keeps the tile's epilogue here: left free, the compiler sinks it
                    // past the next group's barrier and holds every MFMA result of the
                    // group in scratch memory meanwhile
                    asm volatile("" : "+v"(acc[a][b][0]), "+v"(acc[a][b][1]), "+v"(acc[a][b][2]),
                                 "+v"(acc[a][b][3]));
                }
            }
            // issue order: the LDS reads, then one MFMA per three VALU
            // instructions, so the epilogue's VALU work goes out between
            // the next tile's MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
            for (int k = 0; k < 12; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // whether the step of group g issues the next scale chunk (chunk g / 8 + 1)
    auto scales_at = [&](int g) __attribute__((always_inline)) {
        return (g & 7) == 0 && g + 8 < g1;
    };
    // one group: stage g in LDS once this wave's copies older than the last
    // scale chunk have landed and every wave has passed the barrier
    auto step = [&](int g, const uint8_t *cur, uint8_t *nxt) __attribute__((always_inline)) {
        if (g > g0 && scales_at(g - 1))
            wait_vmem<L::kScaleInst>();          // that chunk may still be in flight
        else
            wait_vmem<0>();
        ring_barrier();
        if (g + 1 < g1) issue_stage(g + 1, nxt);
        if (scales_at(g)) issue_scales((g >> 3) + 1);
        compute(cur, g);
    };

    // scale chunk of group g0, and the next one when g0 starts mid-chunk
    // (the loop issues chunks only at multiples of 8)
    issue_scales(g0 >> 3);
    if ((g0 & 7) != 0 && ((g0 >> 3) + 1) * 8 < g1) issue_scales((g0 >> 3) + 1);
    issue_stage(g0, stage0);
    for (int g = g0; g < g1; g += 2) {           // g0 and g1 - g0 are even
        step(g, stage0, stage1);
        step(g + 1, stage1, stage0);
    }
    wait_vmem<0>();

    if (!DOTS && partial) {
#pragma unroll
        for (int b = 0; b < WM; ++b)
#pragma unroll
            for (int a = 0; a < WN; ++a)
                *reinterpret_cast<float4 *>(partial + (16 * b + r) * L::BN + row_base + 16 * a + 4 * lg) =
                    make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
        return;
    }
    if (!DOTS) {
        // four outputs of a lane as one 16-byte store where y allows it
        const bool vec_y = !y16 && (N & 3) == 0 && ((uintptr_t)y & 15) == 0;
#pragma unroll
        for (int b = 0; b < WM; ++b) {
            const int64_t m = m0 + 16 * b + r;
            if (m >= M) continue;
#pragma unroll
            for (int a = 0; a < WN; ++a) {
                const int64_t nb = n0 + row_base + 16 * a + 4 * lg;
                if (vec_y && nb + 3 < N) {
                    *reinterpret_cast<float4 *>(y + m * N + nb) =
                        make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (nb + i < N) store_y(y, y16, m * N + nb + i, acc[a][b][i]);
                }
            }
        }
    }
}

constexpr int64_t kWideBN = 256;

int64_t wide_tiles(int64_t M, int64_t N, int64_t bm) {
    return ((N + kWideBN - 1) / kWideBN) * ((M + bm - 1) / bm);
}

// K split of the wide variant's last tiles within work_bytes of partial sums.
// Two blocks fit per CU, so P = 2 * CUs blocks run at once and T tiles leave
// T % P of them for a last round that keeps part of the GPU idle; splitting
// the K range of those tiles into S chunks (S <= P / (T % P), at most 4, at
// least 10 groups and whole pairs of groups per chunk) fills that round with
// S times as many blocks of 1 / S of the work each. Measured (K = 5120): the
// 256 x 128 tile at M = 4096, N = 17408 523 us against 560 unsplit, M =
// 1024 138 against 182; the 256 x 64 tile at M = 512, N = 17408 84 against
// 111, M = 2048, N = 5120 95 against 105. Shorter chunks lost: 8 groups (M =
// 600, N = 17300, K = 2048) 58 against 51 us, 2 groups (K = 1024) 60
// against 51.
WideSplit wide_split(int64_t M, int64_t N, int64_t K, int64_t bm, float *work,
                     size_t work_bytes) {
    const int64_t T = wide_tiles(M, N, bm);
    const int G = (int)(K / kGroup);
    WideSplit sp{T, 1, G, nullptr};
    const int cus = device_cus() > 0 ? device_cus() : 256;
    const int64_t P = 2 * (int64_t)cus;
    const int64_t tail = T % P;
    if (T < P || tail == 0) return sp;
    const uint64_t per = (uint64_t)tail * bm * kWideBN * sizeof(float);
    int64_t S = P / tail < 4 ? P / tail : 4;
    if (S > G / 10) S = G / 10;
    if ((uint64_t)S > work_bytes / per) S = (int64_t)(work_bytes / per);
    if (S < 2) return sp;
    int cg = (G + (int)S - 1) / (int)S;
    cg += cg & 1;
    S = (G + cg - 1) / cg;
    if (S < 2) return sp;
    sp.full = T - tail;
    sp.chunks = (int)S;
    sp.chunk_groups = cg;
    sp.part = work;
    return sp;
}

template <bool DOTS, int WM>
hipError_t launch_wide_dots(const int8_t *q, const int32_t *t, const uint8_t *codes,
                            const GemmOut &out, int64_t M, int64_t N, int64_t K,
                            const WideSplit &sp, hipStream_t stream) {
    using L = PfWide<DOTS, WM>;
    static_assert(L::BN == kWideBN, "tile sizes");
    const int64_t T = wide_tiles(M, N, L::BM);
    const int64_t blocks = sp.full + (T - sp.full) * sp.chunks;
    hipLaunchKernelGGL((prefill_wide_kernel<DOTS, WM>), dim3((unsigned)blocks), dim3(L::T),
                       (size_t)L::kLdsBytes, stream, q, DOTS ? nullptr : out.s, t, codes,
                       DOTS ? nullptr : out.ws, DOTS ? nullptr : out.y,
                       DOTS ? nullptr : out.y16, DOTS ? out.d : nullptr, M, N, K, sp);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || DOTS || sp.chunks == 1) return e;
    hipLaunchKernelGGL(wide_tail_sum_kernel<L::BM>, dim3((unsigned)((T - sp.full) * L::BM)),
                       dim3((unsigned)kWideBN), 0, stream, sp.part, out.y, out.y16, M, N, sp);
    return hipGetLastError();
}

// WM token tiles of 16 per wave: block tile 256 x 16 WM
template <int WM>
hipError_t launch_wide(const int8_t *q, const int32_t *t, const uint8_t *codes,
                       const GemmOut &out, int64_t M, int64_t N, int64_t K, float *work,
                       size_t work_bytes, hipStream_t stream) {
    if (out.d) {
        const WideSplit whole{wide_tiles(M, N, 16 * WM), 1, (int)(K / kGroup), nullptr};
        return launch_wide_dots<true, WM>(q, t, codes, out, M, N, K, whole, stream);
    }
    const WideSplit sp = wide_split(M, N, K, 16 * WM, work, work ? work_bytes : 0);
    return launch_wide_dots<false, WM>(q, t, codes, out, M, N, K, sp, stream);
}

template <int WN, int WM, int WAVES_N, int WAVES_M, int R>
hipError_t launch_ring_cfg(const int8_t *q, const int32_t *t, const uint8_t *codes,
                           const GemmOut &out, int64_t M, int64_t N, int64_t K,
                           hipStream_t stream) {
    using C = PfCfg<WN, WM, WAVES_N, WAVES_M>;
    const int64_t blocks = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
    if (out.d) {
        using L = PfRing<C::BN, C::BM, C::kThreads, true>;
        const size_t lds = (size_t)R * L::kStageBytes + 2 * L::kScaleBytes + L::kSinkBytes;
        hipLaunchKernelGGL((prefill_ring_kernel<WN, WM, WAVES_N, WAVES_M, R, true>),
                           dim3((unsigned)blocks), dim3(C::kThreads), lds, stream, q, nullptr, t,
                           codes, nullptr, nullptr, nullptr, out.d, M, N, K);
    } else {
        using L = PfRing<C::BN, C::BM, C::kThreads, false>;
        const size_t lds = (size_t)R * L::kStageBytes + 2 * L::kScaleBytes + L::kSinkBytes;
        hipLaunchKernelGGL((prefill_ring_kernel<WN, WM, WAVES_N, WAVES_M, R, false>),
                           dim3((unsigned)blocks), dim3(C::kThreads), lds, stream, q, out.s, t,
                           codes, out.ws, out.y, out.y16, nullptr, M, N, K);
    }
    return hipGetLastError();
}

template <int WN, int WM, int WAVES_N, int WAVES_M, int DEPTH>
hipError_t launch_cfg(const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t M, int64_t N, int64_t K,
                      hipStream_t stream) {
    using C = PfCfg<WN, WM, WAVES_N, WAVES_M>;
    const int64_t blocks = ((N + C::BN - 1) / C::BN) * ((M + C::BM - 1) / C::BM);
    if (out.d) {
        hipLaunchKernelGGL((prefill_mfma_kernel<WN, WM, WAVES_N, WAVES_M, DEPTH, true>),
                           dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, q, nullptr, t,
                           codes, nullptr, nullptr, nullptr, out.d, M, N, K);
    } else {
        hipLaunchKernelGGL((prefill_mfma_kernel<WN, WM, WAVES_N, WAVES_M, DEPTH, false>),
                           dim3((unsigned)blocks), dim3(C::kThreads), 0, stream, q, out.s, t,
                           codes, out.ws, out.y, out.y16, nullptr, M, N, K);
    }
    return hipGetLastError();
}

}  // namespace

// Tile configurations (rows x tokens, waves, prefetch depth):
//  10: 256 x 128, 4 x 1 waves of 64 x 128, ring of 2 stages, scale products
//      on the matrix core (the wide variant)
//  12: 256 x 64, 4 x 1 waves of 64 x 64, the wide variant
//   0: 128 x 128, 2 x 2 waves of 64 x 64, depth 1
//   6: 128 x 128, 2 x 2 waves of 64 x 64, ring of 2 stages (buffer -> LDS copies)
//   7:  64 x 64,  2 x 2 waves of 32 x 32, depth 2
//   8:  64 x 64,  2 x 2 waves of 32 x 32, ring of 2 stages
//   9:  32 x 32,  2 x 2 waves of 16 x 16, depth 2
namespace {

constexpr int64_t kPrefillCUs = 256;

// The tile rule below as block counts: 128 x 128 tiles where that gives four
// per CU, else 64 x 64 where that gives two, else 32 x 32.
int64_t prefill_tiles(int64_t M, int64_t N, int64_t bn, int64_t bm) {
    return ((N + bn - 1) / bn) * ((M + bm - 1) / bm);
}

}  // namespace

int64_t prefill_blocks(int64_t M, int64_t N) {
    if (prefill_tiles(M, N, 128, 128) >= 4 * kPrefillCUs) return prefill_tiles(M, N, 128, 128);
    if (prefill_tiles(M, N, 64, 64) >= 2 * kPrefillCUs) return prefill_tiles(M, N, 64, 64);
    return prefill_tiles(M, N, 32, 32);
}

namespace {

// Tile choice (MI355X sweeps over M = 128 / 512 / 4096 on the 5120 and 17408
// shapes): 128 x 128 where that gives at least four tiles per CU, else
// 64 x 64 where that gives two, else 32 x 32 -- at these sizes more,
// smaller tiles keep more waves per CU busy (M = 128, N = 17408: 43.7 us
// against 54.2 with 64 x 128; M = 128, N = 5120: 20.4 against 27.0).
// Ring forms (stages and scale chunks by buffer -> LDS copies) where G is
// a multiple of 8 and offsets stay below their sentinel: 3-20 % faster;
// the 64 x 64 ring (88 VGPRs, 31 KB of LDS) runs five blocks per CU. Ring
// forms of the 32 x 32, 64 x 128 tiles and a 3-stage 64 x 64 ring were
// slower. The wide variant (256 weight rows x 128 or 64 tokens), where its
// tiles fill at least 7/8 of a round of two blocks per CU, is faster again
// (K = 5120, with the K split of its last round): M = 4096, N = 17408 523 us
// against 672 for the 128 x 128 ring; M = 3072, N = 5120 118 against 160
// (480 tiles of 128 tokens: one round; the 64-token tile 130); M = 2048,
// N = 5120 95 (64 tokens) against 114 for the 64 x 64 ring; M = 512,
// N = 17408 84 (64 tokens) against 113. With fewer tiles the 64 x 64 ring
// stays faster (M = 512 / 1024, N = 5120: 42 / 66 us against 47 / 69).
int prefill_cfg(int64_t M, int64_t N, int64_t K) {
    auto tiles = [&](int64_t bn, int64_t bm) { return prefill_tiles(M, N, bn, bm); };
    constexpr int64_t kCUs = kPrefillCUs;
    const bool ring = (K / kGroup) % 8 == 0 && K <= 65536;
    // the wide tiles where they fill at least 7/8 of a round of two blocks
    // per CU: 256 x 128 first, else 256 x 64
    const int64_t wide_min = 7 * (2 * kCUs) / 8;
    return ring && tiles(256, 128) >= wide_min ? 10
         : ring && tiles(256, 64) >= wide_min  ? 12
         : tiles(128, 128) >= 4 * kCUs ? (ring ? 6 : 0)
         : tiles(64, 64) >= 2 * kCUs   ? (ring ? 8 : 7)
                                       : 9;
}

}  // namespace

size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int cfg = prefill_cfg(M, N, K);
    if (cfg != 10 && cfg != 12) return 0;
    const int64_t bm = cfg == 10 ? 128 : 64;
    const WideSplit sp = wide_split(M, N, K, bm, nullptr, SIZE_MAX);
    if (sp.chunks == 1) return 0;
    return (size_t)(wide_tiles(M, N, bm) - sp.full) * sp.chunks * bm * kWideBN * sizeof(float);
}

hipError_t launch_prefill(const int8_t *q, const int32_t *t, const uint8_t *codes,
                          const GemmOut &out, int64_t M, int64_t N, int64_t K, float *work,
                          size_t work_bytes, hipStream_t stream) {
    switch (prefill_cfg(M, N, K)) {
        case 10: return launch_wide<8>(q, t, codes, out, M, N, K, work, work_bytes, stream);
        case 12: return launch_wide<4>(q, t, codes, out, M, N, K, work, work_bytes, stream);
        case 6: return launch_ring_cfg<4, 4, 2, 2, 2>(q, t, codes, out, M, N, K, stream);
        case 7: return launch_cfg<2, 2, 2, 2, 2>(q, t, codes, out, M, N, K, stream);
        case 8: return launch_ring_cfg<2, 2, 2, 2, 2>(q, t, codes, out, M, N, K, stream);
        case 9: return launch_cfg<1, 1, 2, 2, 2>(q, t, codes, out, M, N, K, stream);
        default: return launch_cfg<4, 4, 2, 2, 1>(q, t, codes, out, M, N, K, stream);
    }
}

}  // namespace pq2
