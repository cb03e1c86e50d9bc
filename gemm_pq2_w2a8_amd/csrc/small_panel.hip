// small_panel.hip -- K3, persistent form: PQ2_0 product for up to 16 token
// rows on int8 MFMA with the whole activation panel resident in LDS.
//
// Same arithmetic as the small-batch kernel (page "Making a ternary reasoning
// model fast in vLLM", section "Small batches: make the register layout
// explicit": code bytes go straight into matrix-instruction operand registers,
// one shift and one mask per plane; every weight is loaded once for all token
// rows). What changes is where the activations come from. A 16-row tile
// needs 16 * 128 activation bytes per group against 512 code bytes, so a
// kernel that fetches activation fragments per tile moves several times more
// bytes into the CUs than the weights it streams. Here each block copies the
// M x K int8 panel and the tokens' s and t into LDS once, then walks weight
// tiles blockIdx.x, blockIdx.x + gridDim.x, ... with one block per CU, so the
// inbound bytes are the codes plus one panel per CU.
//
// gfx950 mapping (v_mfma_i32_16x16x64_i8):
//  * Operand A = activations (rows = tokens, read from LDS), operand B =
//    code planes (columns = weight rows c = lane % 16). For group g, lane
//    group lg = lane / 16 holds code words 4*(lg&1) .. 4*(lg&1)+3 of row c and
//    takes plane lg>>1 (first MFMA) and 2 + lg>>1 (second MFMA) of them; its
//    A fragments are plane-order activation bytes 16*lg .. 16*lg+15 and
//    64 + 16*lg .. of the group for token c. A and B use the same k order, so
//    the pair of MFMAs gives the exact group dot.
//  * Codes arrive two groups at a time: one 16-byte load per lane covers 64
//    contiguous bytes of each of the 16 rows (lanes 0-31: group 2p, lanes
//    32-63: group 2p+1), so no lane loads a byte another lane loads. One
//    v_permlane32_swap per register then copies the low half-wave to the high
//    half for group 2p and the high half to the low half for group 2p+1.
//    (Lanes that load the same bytes, or consecutive loads that each touch a
//    quarter of a cache line, keep the L1 waiting on lines already in flight.)
//  * The accumulator is seeded with -t, so D[m][n] = dot - t exactly. Lane
//    (lg, c) holds D for tokens 4*lg .. 4*lg+3 of weight row c and adds
//    D * (s[m][g] * ws[n][g]) to its four float partials; token scales come
//    from LDS, weight scales from an LDS copy of the tile's [16][G] scale
//    block, loaded with one coalesced 16-byte load per thread a tile ahead.
//  * The NW waves of a block split the group pairs of every tile; at the end
//    of a tile each wave writes its partials to LDS and, after one barrier,
//    256 threads sum them in wave order (a fixed order: deterministic
//    results) and store y. Partials and weight scales alternate between two
//    LDS buffers, so one barrier per tile is enough.
//  * Codes are prefetched R - 1 tiles ahead through a ring of register
//    buffers; every load is unconditional, so the wait counts stay exact
//    across the loop back edge.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

#include <type_traits>
#include <mutex>

namespace pq2 {

namespace {

constexpr int kPanelPad = 16;       // LDS row stride of the panel: K + 16 bytes

// LDS bytes for K chunks of up to gc groups: panel [Mr][128 gc + 16]; s and -t
// tables [gc][16]; weight scales of two tiles [2][16][gc + 1] floats;
// partials [2][NW][64][4] floats.
__host__ __device__ constexpr int64_t panel_lds_bytes(int64_t Mr, int64_t gc, int nw) {
    return Mr * (kGroup * gc + kPanelPad) + 2 * 16 * gc * 4 + 2 * 16 * (gc + 1) * 4 +
           2 * (int64_t)nw * kWave * 16;
}

// Split-K: the G groups are cut into chunks of gsplit groups (the last one
// shorter); blocks [s * bps, (s + 1) * bps) take chunk s for every tile
// (tiles bl, bl + bps, ... for block bl of the chunk) and write their sums to
// part[s][M][N] instead of y. One chunk (gsplit = G, bps = gridDim.x) is the
// plain case.
template <int NW, int GS, int R, bool DOTS>
__global__ __launch_bounds__(NW * kWave) void small_panel_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    uint16_t *__restrict__ y16, int32_t *__restrict__ d, float *__restrict__ part_out, int64_t M,
    int64_t N, int64_t K,
    int gsplit, int bps) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int T = NW * kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = lane & 15;
    const int lg = lane >> 4;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);
    const int KB = (int)(K / 4);                 // code bytes per weight row
    const int Mr = M < 16 ? (int)M : 16;
    const int64_t NT = (N + 15) / 16;
    const int bid = blockIdx.x;
    const int sidx = bid / bps;                  // K chunk of this block
    const int bl = bid - sidx * bps;             // block within the chunk
    const int g0 = sidx * gsplit;                // first group of the chunk
    const int Gc = G - g0 < gsplit ? G - g0 : gsplit;
    const int GP = Gc + 1;
    const int RS = kGroup * gsplit + kPanelPad;  // panel row stride
    const int cnt = (int)((NT - bl + bps - 1) / bps);    // tiles of this block (>= 1)

    int8_t *panel = reinterpret_cast<int8_t *>(smem);                          // [Mr][RS]
    float *s_l = reinterpret_cast<float *>(smem + (int64_t)Mr * RS);           // [Gc][16]
    int32_t *tn_l = reinterpret_cast<int32_t *>(s_l + 16 * gsplit);            // [Gc][16], -t
    float *wsl = reinterpret_cast<float *>(tn_l + 16 * gsplit);                // [2][16][GP]
    float *part = wsl + 2 * 16 * (gsplit + 1);                                 // [2][NW][64][4]

    // This wave's group pairs of the chunk: [p_lo, p_lo + np), 1 <= np <= GS
    // (the last pair has one group when Gc is odd).
    const int NP = (Gc + 1) / 2;
    const int p_lo = (NP * wave) / NW;
    const int np = (NP * (wave + 1)) / NW - p_lo;
    const int voff_c = c * KB + 32 * g0 + 16 * lg;

    // Weight scales of a tile's chunk, [16][Gc] halves, as 16-byte chunks of
    // eight groups. With G % 8 == 0 (every split shape) each row's part is
    // whole chunks: thread tid < 2 Gc takes row tid / (Gc/8), chunk tid %
    // (Gc/8). Otherwise (one chunk only) the tile's 16 G halves are
    // contiguous and thread tid < 2G takes elements 8 tid .. 8 tid + 7, at
    // (row, column) = divmod(8 tid, G). Only the waves that hold a chunk load.
    const bool rowwise = G % 8 == 0;
    const int nwc = 2 * Gc;
    const bool ws_wave = !DOTS && wave * kWave < nwc;
    int w_row0 = 0, w_col0 = 0, w_off = 0;
    if (!DOTS) {
        if (rowwise) {
            const int cpr8 = Gc / 8;
            w_row0 = tid / cpr8;
            w_col0 = 8 * (tid - w_row0 * cpr8);
            w_off = 2 * (w_row0 * G + g0 + w_col0);
        } else {
            w_row0 = (8 * tid) / G;
            w_col0 = 8 * tid - w_row0 * G;
            w_off = 16 * tid;
        }
    }

    v4i cb[R][GS];
    v4i wv[R];
    // Past the block's last tile the code loads still issue (so the wait
    // counts stay exact) but every lane reads the first bytes of the last
    // tile: one cache line per instruction instead of a tile slice.
    auto load_tile = [&](v4i (&cbs)[GS], v4i &wvs, int j) __attribute__((always_inline)) {
        const bool live = j < cnt;
        const int jj = live ? j : cnt - 1;
        const int64_t n0 = (int64_t)(bl + (int64_t)jj * bps) * 16;
        const int64_t rows = N - n0 < 16 ? N - n0 : 16;
        if (ws_wave) {
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(ws + n0 * G, rows * G * 2);
            wvs = __builtin_amdgcn_raw_buffer_load_b128(rw, tid < nwc ? w_off : 0, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes + n0 * KB, rows * KB);
        const int oc = live ? voff_c : 0;
#pragma unroll
        for (int b = 0; b < GS; ++b) {
            const int p = live ? p_lo + (b < np ? b : np - 1) : 0;
            cbs[b] = __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 64 * p, 0);
        }
    };
    // Eight halves of a weight-scale chunk -> floats in wsl[buf][row][col].
    auto store_ws = [&](const v4i &wvs, int buf) __attribute__((always_inline)) {
        if (ws_wave && tid < nwc) {
            float *dst = wsl + buf * 16 * GP;
            int row = w_row0, col = w_col0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t word = (uint32_t)wvs[k >> 1];
                dst[row * GP + col] = half_bits_to_float((uint16_t)((k & 1) ? word >> 16 : word));
                if (++col == Gc) {
                    col = 0;
                    ++row;
                }
            }
        }
    };

    // Prefetch the first R - 1 tiles, then stage the panel chunk, the token
    // tables and the first tile's weight scales.
#pragma unroll
    for (int u = 0; u < R - 1; ++u) load_tile(cb[u], wv[u], u);

    {
        const int cpr = 8 * Gc;                  // 16-byte chunks per token row of the chunk
        const int total = Mr * cpr;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, (int64_t)Mr * K);
        // chunk e = tid + i*T sits at (row, col) = divmod(e, cpr), advanced by
        // (T / cpr, T % cpr) per step
        const int dr = T / cpr, dc = T - dr * cpr;
        int row = tid / cpr, col = tid - row * cpr;
        for (int e0 = 0; e0 < total; e0 += 8 * T) {
            // a chunk past the end is the last chunk again, loaded and stored
            // unconditionally (a conditional store lets the compiler sink the
            // load next to it), the same bytes twice
            int rr[8], cc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool in = e0 + tid + i * T < total;
                rr[i] = in ? row : Mr - 1;
                cc[i] = in ? col : cpr - 1;
                row += dr;
                col += dc;
                if (col >= cpr) {
                    col -= cpr;
                    ++row;
                }
            }
            v4i v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, rr[i] * (int)K + kGroup * g0 + 16 * cc[i], 0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<v4i *>(panel + rr[i] * RS + 16 * cc[i]) = v[i];
        }
        // tables [g][m]: tokens m >= M hold 0 (their outputs are never stored)
        for (int e = tid; e < 16 * Gc; e += T) {
            const int g = e >> 4, m = e & 15;
            const bool ok = m < Mr;
            if (!DOTS) s_l[e] = ok ? s[m * G + g0 + g] : 0.0f;
            tn_l[e] = ok ? -t[m * G + g0 + g] : 0;
        }
        store_ws(wv[0], 0);
    }
    __syncthreads();

    const int arow = c < Mr ? c : Mr - 1;   // padded tokens read the last real row
    const int8_t *abase = panel + arow * RS + 16 * lg;

    // One group (g within the chunk): planes of this lane's four code words
    // (w), two MFMAs, epilogue.
    auto group = [&](const v4i &w, int g, int64_t n0, const float *wrow, float (&acc)[4])
        __attribute__((always_inline)) {
        const v4i a0 = *reinterpret_cast<const v4i *>(abase + kGroup * g);
        const v4i a1 = *reinterpret_cast<const v4i *>(abase + kGroup * g + 64);
        const v4i seed = *reinterpret_cast<const v4i *>(tn_l + 16 * g + 4 * lg);
        v4i b0, b1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t sh = (uint32_t)w[k] >> sh0;
            b0[k] = (int)(sh & kPlaneMask);
            b1[k] = (int)((sh >> 4) & kPlaneMask);
        }
        v4i dd = mfma16x16x64(a0, b0, seed);
        dd = mfma16x16x64(a1, b1, dd);
        if (DOTS) {
            const int64_t n = n0 + c;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * lg + i;
                if (m < M && n < N) d[((int64_t)m * N + n) * G + g0 + g] = dd[i];
            }
        } else {
            const float4 sv = *reinterpret_cast<const float4 *>(s_l + 16 * g + 4 * lg);
            const float wsf = wrow[g];
            acc[0] = fmaf((float)dd[0], sv.x * wsf, acc[0]);
            acc[1] = fmaf((float)dd[1], sv.y * wsf, acc[1]);
            acc[2] = fmaf((float)dd[2], sv.z * wsf, acc[2]);
            acc[3] = fmaf((float)dd[3], sv.w * wsf, acc[3]);
        }
    };

    auto compute_tile = [&](const v4i (&cbs)[GS], int j) __attribute__((always_inline)) {
        const int64_t n0 = (int64_t)(bl + (int64_t)j * bps) * 16;
        const float *wrow = wsl + (j & 1) * 16 * GP + c * GP;
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < GS; ++b) {
            if (b < np) {
                const int g = 2 * (p_lo + b);
                v4i lo, hi;     // group g in every lane, group g + 1 in every lane
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const auto sw = __builtin_amdgcn_permlane32_swap((uint32_t)cbs[b][k],
                                                                     (uint32_t)cbs[b][k], false, false);
                    lo[k] = (int)sw[0];
                    hi[k] = (int)sw[1];
                }
                group(lo, g, n0, wrow, acc);
                if (g + 1 < Gc) group(hi, g + 1, n0, wrow, acc);
            }
        }
        if (!DOTS) {
            float *pb = part + (j & 1) * (NW * kWave * 4);
            *reinterpret_cast<float4 *>(pb + (wave * kWave + lane) * 4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    };

    float *out = part_out ? part_out + (int64_t)sidx * M * N : y;
    uint16_t *out16 = part_out ? nullptr : y16;   // partial sums stay float32
    auto reduce_tile = [&](int j) __attribute__((always_inline)) {
        if (!DOTS && tid < 256) {
            const int64_t n0 = (int64_t)(bl + (int64_t)j * bps) * 16;
            const float *pb = part + (j & 1) * (NW * kWave * 4);
            // output (token m, row cc) sits in lane cc + 16 * (m / 4), slot m % 4
            const int m = tid >> 4, cc = tid & 15;
            const int at = (cc + 16 * (m >> 2)) * 4 + (m & 3);
            float v = pb[at];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += pb[w * kWave * 4 + at];
            const int64_t n = n0 + cc;
            if (m < M && n < N) store_y(out, out16, (int64_t)m * N + n, v);
        }
    };

    for (int j0 = 0; j0 < cnt; j0 += R) {
#pragma unroll
        for (int u = 0; u < R; ++u) {
            load_tile(cb[(u + R - 1) % R], wv[(u + R - 1) % R], j0 + u + R - 1);
            if (j0 + u < cnt) {
                compute_tile(cb[u], j0 + u);
                store_ws(wv[(u + 1) % R], (j0 + u + 1) & 1);   // the next tile's scales
                __syncthreads();
                reduce_tile(j0 + u);
            }
        }
    }
}

// LDS bytes of the staged-codes variant for TT token tiles: panel
// [Mr][128 gc + 16]; s and -t tables [gc][16 TT]; weight scales of two tiles
// [2][16][gc + 1]; partials [NW][64][4] floats; one [16][32 gc + 16] code
// tile.
__host__ __device__ constexpr int64_t panel_lds_bytes_sc(int64_t Mr, int64_t gc, int nw, int tt) {
    return Mr * (kGroup * gc + kPanelPad) + 2 * 16 * tt * gc * 4 + 2 * 16 * (gc + 1) * 4 +
           (int64_t)nw * kWave * 16 + 16 * (32 * gc + kPanelPad);
}

// Staged-codes variant: same arithmetic and split-K scheme, but each 16-row
// code tile (its chunk of K) is read with fully coalesced 16-byte loads --
// every cache line is requested by exactly one instruction -- into LDS, and
// each wave reads its MFMA B operands from there (row c, bytes 32 g + 16 (lg
// & 1) of group g). A load that covers part of a line which another load has
// in flight stalls the L1 until the line arrives; the register layout of the
// operands cannot be loaded in whole lines. Waves split the chunk's groups
// (not pairs); the next code tile is prefetched in registers, and a tile
// takes two barriers (partials and code buffer, then the next tile's codes
// in LDS).
// TT token tiles (M <= 16 TT): wave w computes token tile w % TT over its
// share of the chunk's groups (the NW / TT waves of a token tile split the
// groups), so each wave keeps one float partial per lane whatever TT is.
template <int NW, int GSG, int CPT, int TT, bool DOTS>
__global__ __launch_bounds__(NW * kWave) void small_panel_sc_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    uint16_t *__restrict__ y16, int32_t *__restrict__ d, float *__restrict__ part_out, int64_t M,
    int64_t N, int64_t K,
    int gsplit, int bps) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int T = NW * kWave;
    constexpr int TM = 16 * TT;                  // tokens held
    constexpr int KW = NW / TT;                  // waves per token tile
    static_assert(KW * TT == NW, "token tiles must divide the waves");
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int tt = wave % TT;
    const int kw = wave / TT;
    const int c = lane & 15;
    const int lg = lane >> 4;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);
    const int KB = (int)(K / 4);
    const int Mr = M < TM ? (int)M : TM;
    const int64_t NT = (N + 15) / 16;
    const int bid = blockIdx.x;
    const int sidx = bid / bps;
    const int bl = bid - sidx * bps;
    const int g0 = sidx * gsplit;
    const int Gc = G - g0 < gsplit ? G - g0 : gsplit;
    const int GP = Gc + 1;
    const int RS = kGroup * gsplit + kPanelPad;
    const int RSC = 32 * gsplit + kPanelPad;     // code tile row stride in LDS
    const int cnt = (int)((NT - bl + bps - 1) / bps);

    int8_t *panel = reinterpret_cast<int8_t *>(smem);                          // [Mr][RS]
    float *s_l = reinterpret_cast<float *>(smem + (int64_t)Mr * RS);           // [Gc][TM]
    int32_t *tn_l = reinterpret_cast<int32_t *>(s_l + TM * gsplit);            // [Gc][TM], -t
    float *wsl = reinterpret_cast<float *>(tn_l + TM * gsplit);                // [2][16][GP]
    float *part = wsl + 2 * 16 * (gsplit + 1);                                 // [NW][64][4]
    uint8_t *codes_l = reinterpret_cast<uint8_t *>(part + NW * kWave * 4);     // [16][RSC]

    // this wave's groups of the chunk: [g_lo, g_lo + ng), 1 <= ng <= GSG
    const int g_lo = (Gc * kw) / KW;
    const int ng = (Gc * (kw + 1)) / KW - g_lo;

    // code tile chunks: e = tid + i*T < 32 Gc is (row e / (2 Gc), 16-byte
    // column e % (2 Gc)); past the end a lane re-reads the last chunk in the
    // same instruction
    const int nch = 32 * Gc;
    int goff[CPT], loff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        int e = tid + i * T;
        e = e < nch ? e : nch - 1;
        const int row = e / (2 * Gc), col = e - row * 2 * Gc;
        goff[i] = row * KB + 32 * g0 + 16 * col;
        loff[i] = row * RSC + 16 * col;
    }

    // weight scales as in the register-operand kernel
    const bool rowwise = G % 8 == 0;
    const int nwc = 2 * Gc;
    const bool ws_wave = !DOTS && wave * kWave < nwc;
    int w_row0 = 0, w_col0 = 0, w_off = 0;
    if (!DOTS) {
        if (rowwise) {
            const int cpr8 = Gc / 8;
            w_row0 = tid / cpr8;
            w_col0 = 8 * (tid - w_row0 * cpr8);
            w_off = 2 * (w_row0 * G + g0 + w_col0);
        } else {
            w_row0 = (8 * tid) / G;
            w_col0 = 8 * tid - w_row0 * G;
            w_off = 16 * tid;
        }
    }

    v4i cr[CPT];
    v4i wv;
    // tile j's codes (and scales) into registers; past the block's last tile
    // every lane reads the first 16 bytes of the last tile (one line)
    auto load_tile = [&](int j) __attribute__((always_inline)) {
        const bool live = j < cnt;
        const int jj = live ? j : cnt - 1;
        const int64_t n0 = (int64_t)(bl + (int64_t)jj * bps) * 16;
        const int64_t rows = N - n0 < 16 ? N - n0 : 16;
        if (ws_wave) {
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(ws + n0 * G, rows * G * 2);
            wv = __builtin_amdgcn_raw_buffer_load_b128(rw, tid < nwc ? w_off : 0, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes + n0 * KB, rows * KB);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            cr[i] = __builtin_amdgcn_raw_buffer_load_b128(rc, live ? goff[i] : 0, 0, 0);
    };
    auto store_codes = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) *reinterpret_cast<v4i *>(codes_l + loff[i]) = cr[i];
    };
    auto store_ws = [&](int buf) __attribute__((always_inline)) {
        if (ws_wave && tid < nwc) {
            float *dst = wsl + buf * 16 * GP;
            int row = w_row0, col = w_col0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t word = (uint32_t)wv[k >> 1];
                dst[row * GP + col] = half_bits_to_float((uint16_t)((k & 1) ? word >> 16 : word));
                if (++col == Gc) {
                    col = 0;
                    ++row;
                }
            }
        }
    };

    // prologue: tile 0 in flight, the panel chunk and tables, tile 0 into
    // LDS, its registers refilled with tile 1
    load_tile(0);
    {
        const int cpr = 8 * Gc;
        const int total = Mr * cpr;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, (int64_t)Mr * K);
        const int dr = T / cpr, dc = T - dr * cpr;
        int row = tid / cpr, col = tid - row * cpr;
        for (int e0 = 0; e0 < total; e0 += 8 * T) {
            int rr[8], cc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool in = e0 + tid + i * T < total;
                rr[i] = in ? row : Mr - 1;
                cc[i] = in ? col : cpr - 1;
                row += dr;
                col += dc;
                if (col >= cpr) {
                    col -= cpr;
                    ++row;
                }
            }
            v4i v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                v[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, rr[i] * (int)K + kGroup * g0 + 16 * cc[i], 0, 0);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<v4i *>(panel + rr[i] * RS + 16 * cc[i]) = v[i];
        }
        // tables [g][m]: tokens m >= M hold 0 (their outputs are never stored)
        for (int e = tid; e < TM * Gc; e += T) {
            const int g = e / TM, m = e - g * TM;
            const bool ok = m < Mr;
            if (!DOTS) s_l[e] = ok ? s[m * G + g0 + g] : 0.0f;
            tn_l[e] = ok ? -t[m * G + g0 + g] : 0;
        }
        store_codes();
        store_ws(0);
        load_tile(1);
    }
    __syncthreads();

    const int arow = 16 * tt + c < Mr ? 16 * tt + c : Mr - 1;   // padded tokens: last real row
    const int8_t *abase = panel + arow * RS + 16 * lg;
    const uint8_t *bbase = codes_l + c * RSC + 16 * (lg & 1);
    const int32_t *tnbase = tn_l + 16 * tt + 4 * lg;
    const float *sbase = s_l + 16 * tt + 4 * lg;

    auto compute_tile = [&](int j) __attribute__((always_inline)) {
        const int64_t n0 = (int64_t)(bl + (int64_t)j * bps) * 16;
        const float *wrow = wsl + (j & 1) * 16 * GP + c * GP;
        float acc0 = 0.0f, acc1 = 0.0f, acc2 = 0.0f, acc3 = 0.0f;
#pragma unroll
        for (int b = 0; b < GSG; ++b) {
            if (b < ng) {
                const int g = g_lo + b;
                const v4i w = *reinterpret_cast<const v4i *>(bbase + 32 * g);
                const v4i a0 = *reinterpret_cast<const v4i *>(abase + kGroup * g);
                const v4i a1 = *reinterpret_cast<const v4i *>(abase + kGroup * g + 64);
                const v4i seed = *reinterpret_cast<const v4i *>(tnbase + TM * g);
                v4i b0, b1;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t sh = (uint32_t)w[k] >> sh0;
                    b0[k] = (int)(sh & kPlaneMask);
                    b1[k] = (int)((sh >> 4) & kPlaneMask);
                }
                v4i dd = mfma16x16x64(a0, b0, seed);
                dd = mfma16x16x64(a1, b1, dd);
                if (DOTS) {
                    const int64_t n = n0 + c;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int m = 16 * tt + 4 * lg + i;
                        if (m < M && n < N) d[((int64_t)m * N + n) * G + g0 + g] = dd[i];
                    }
                } else {
                    const float wsf = wrow[g];
                    const float4 sv = *reinterpret_cast<const float4 *>(sbase + TM * g);
                    acc0 = fmaf((float)dd[0], sv.x * wsf, acc0);
                    acc1 = fmaf((float)dd[1], sv.y * wsf, acc1);
                    acc2 = fmaf((float)dd[2], sv.z * wsf, acc2);
                    acc3 = fmaf((float)dd[3], sv.w * wsf, acc3);
                }
            }
        }
        if (!DOTS)
            *reinterpret_cast<float4 *>(part + (wave * kWave + lane) * 4) =
                make_float4(acc0, acc1, acc2, acc3);
    };

    float *out = part_out ? part_out + (int64_t)sidx * M * N : y;
    uint16_t *out16 = part_out ? nullptr : y16;   // partial sums stay float32
    auto reduce_tile = [&](int j) __attribute__((always_inline)) {
        if (!DOTS) {
            const int64_t n0 = (int64_t)(bl + (int64_t)j * bps) * 16;
            // output (token 16 u + ml, row cc) sits in lane cc + 16 (ml / 4),
            // slot ml % 4 of waves u, u + TT, ..., summed in wave order
            for (int e = tid; e < TT * 256; e += T) {
                const int u = e >> 8, ml = (e >> 4) & 15, cc = e & 15;
                const int at = (u * kWave + cc + 16 * (ml >> 2)) * 4 + (ml & 3);
                float v = part[at];
#pragma unroll
                for (int w = 1; w < KW; ++w) v += part[w * TT * kWave * 4 + at];
                const int64_t m = 16 * u + ml, n = n0 + cc;
                if (m < M && n < N) store_y(out, out16, m * N + n, v);
            }
        }
    };

    // tile j's codes are in LDS, tile j + 1's in registers
    for (int j = 0; j < cnt; ++j) {
        compute_tile(j);
        __syncthreads();            // code buffer free, partials visible
        reduce_tile(j);
        store_codes();
        store_ws((j + 1) & 1);
        load_tile(j + 2);
        __syncthreads();            // tile j + 1 in LDS; partials free again
    }
}

// ---------------------------------------------------------------- ring variant

// Code tiles in LDS: one being computed, one in flight. MI355X sweeps over
// the 5120 / 6144 / 17408 shapes: 2 slots beat 3, 4 and 5 by 5-15 % (more
// copies in flight per CU made every tile land later), also when only tile 0
// is issued ahead of the first compute and with non-temporal copies.
constexpr int kRingSlots = 2;
constexpr int kRingMaxGs = 6;                // groups per wave: A, seeds, scales and NG MFMA
                                             // chains in at most 256 VGPRs
// f(std::integral_constant<int, n>) for the run-time n in [1, NG].
template <int NG, typename F>
__device__ __forceinline__ void with_count(int n, F &&f) {
    if constexpr (NG >= 1) {
        if (n == NG) {
            f(std::integral_constant<int, NG>{});
            return;
        }
        with_count<NG - 1>(n, f);
    }
}

// LDS bytes of the ring variant: R code slots of CPT * NW / 2 KB and R
// weight-scale slots of 2 KB, a 1 KB sink for copies of idle waves, partials
// [2][NW][4][64] floats.
__host__ __device__ constexpr int64_t ring_lds_bytes(int cpt, int nw) {
    return (int64_t)kRingSlots * (cpt * nw / 2 * 1024 + 2048) + 1024 + 2 * nw * 1024;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// v_permlane32_swap(a, b): lanes 32..63 of a trade places with lanes 0..31
// of b. Returns the new a and b. (The elements of the builtin's result are
// read into scalars before any bit cast: a bit cast applied to a vector
// element expression reads element 0.)
__device__ __forceinline__ void swap_halves(uint32_t &a, uint32_t &b) {
    const auto sw = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    const uint32_t na = sw[0], nb = sw[1];
    a = na;
    b = nb;
}

// Max and sum of this lane's value and that of lane ^ 32: with a == b, the
// swap leaves the lower half's value in a and the upper half's in b.
__device__ __forceinline__ float max_halves(float v) {
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    swap_halves(a, b);
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ int sum_halves(int v) {
    uint32_t a = (uint32_t)v, b = a;
    swap_halves(a, b);
    return (int)a + (int)b;
}

// In-register quantisation of one 128-activation group of one token into the
// ring variant's A fragments (the fused entry). Lanes c, c + 16, c + 32 and
// c + 48 (lane group lg = 0..3) hold token c's group between them: lane lg
// has loaded the 32 activations [64 h + 32 u, 64 h + 32 u + 32) of it as
// f[j] = x[64 h + 32 u + 4 j .. + 3] (h = lg & 1, u = lg >> 1). Its
// fragments need planes p0 = u and p0 + 2 at plane positions 16 h .. 16 h +
// 15, i.e. activations 64 h + 4 i + p0 (a0 byte i) and 64 h + 4 i + p0 + 2
// (a1 byte i), i = 0..15; for i >= 8 they sit in lane ^ 32 (same h, other
// u), which in turn needs this lane's other two planes. One
// v_permlane32_swap per component pair trades them, after which
// a0 byte i comes from f[i].x (i < 8) or f[i - 8].y and a1 byte i from f[i].z
// or f[i - 8].w, in every lane. amax and sum(q) are reductions over the four
// lanes (lane ^ 16 by ds_swizzle, lane ^ 32 by v_permlane32_swap); the
// rounding is the quantiser's own (quant_* helpers), so q, s and t are those
// pq2_quantize_act writes, bit for bit. Returns s and t of token c in every
// lane of the token.
__device__ __forceinline__ void quantize_ring_frag(v4f (&f)[8], v4i &a0, v4i &a1, float &scale,
                                                   int &tsum) {
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        a = fmaxf(a, fmaxf(fmaxf(fabsf(f[j].x), fabsf(f[j].y)), fmaxf(fabsf(f[j].z), fabsf(f[j].w))));
    a = fmaxf(a, __builtin_bit_cast(float, swizzle_xor16(__builtin_bit_cast(int, a))));
    a = max_halves(a);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float fx = f[j].x, fy = f[j].y, fz = f[j].z, fw = f[j].w;
        uint32_t x0 = __builtin_bit_cast(uint32_t, fx), y0 = __builtin_bit_cast(uint32_t, fy);
        uint32_t z0 = __builtin_bit_cast(uint32_t, fz), w0 = __builtin_bit_cast(uint32_t, fw);
        swap_halves(x0, y0);
        swap_halves(z0, w0);
        f[j] = v4f{__builtin_bit_cast(float, x0), __builtin_bit_cast(float, y0),
                   __builtin_bit_cast(float, z0), __builtin_bit_cast(float, w0)};
    }
    scale = a / 127.0f;                             // IEEE division
    const float rc = __builtin_amdgcn_rcpf(scale);
    const bool tiny = quant_tiny(scale);
    // element i of fragment p: p = 0 planes p0, p = 1 planes p0 + 2
    auto elem = [&](int p, int i) __attribute__((always_inline)) {
        const v4f &v = f[i & 7];
        return p == 0 ? (i < 8 ? v.x : v.y) : (i < 8 ? v.z : v.w);
    };
    float qf[2][16];
    bool slow = false;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            bool ok;
            qf[p][i] = quant_round_fast(elem(p, i), rc, tiny, ok);
            slow |= !ok && scale != 0.0f;
        }
    if (__any(slow)) {                              // rare: the IEEE division decides
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                bool ok;
                quant_round_fast(elem(p, i), rc, tiny, ok);
                if (!ok && scale != 0.0f) qf[p][i] = rintf(elem(p, i) / scale);
            }
    }
    v4i w[2];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                word |= ((uint32_t)quant_clamp(qf[p][4 * k + e], scale) & 0xffu) << (8 * e);
            w[p][k] = (int)word;
        }
    a0 = w[0];
    a1 = w[1];
    int t = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        t = dot4((uint32_t)w[0][k], 0x01010101u, t);
        t = dot4((uint32_t)w[1][k], 0x01010101u, t);
    }
    t += swizzle_xor16(t);
    tsum = sum_halves(t);
}

// Ring variant (M <= 16, chunks of a multiple of 8 groups): same arithmetic,
// but the A side never moves again once loaded. Wave w owns groups
// [g_lo, g_lo + ng) of the chunk for every tile, so its A fragments, -t seeds
// and token scales for those groups live in VGPRs from the prologue on. Code
// tiles stream through a ring of LDS slots by buffer -> LDS copies (16 bytes
// per lane, no VGPRs held), kRingSlots - 1 tiles ahead of the one being
// computed; each copy thread issues the same number of copies per tile (lanes
// past the tile read past the buffer range, which moves no memory), so one
// vmcnt wait per tile covers exactly the copies of that tile. Unit u (16 bytes) of a slot holds
// row r = u / (2 Gc), column (u % (2 Gc)) ^ (r % 16) of the tile's chunk: every
// 128-byte line is still fetched by one instruction, and the 16 rows of one
// B read land in different LDS banks. The tile's [16][Gc] weight scales ride
// in the same round, one copy per wave (waves past the block's 2 Gc scale units
// copy into a sink). One barrier per tile: before it, each wave waits for its
// own copies of the tile; after it, tile j - 1's slot is free for tile
// j + kRingSlots - 1, and tile j - 1's partials (double-buffered) are summed
// and stored.
template <int NW, int GSG, int CPT, bool DOTS, bool FUSED>
__global__ __launch_bounds__(NW * kWave) void small_panel_ring_kernel(
    const float *__restrict__ x,
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    uint16_t *__restrict__ y16, int32_t *__restrict__ d, float *__restrict__ part_out, int64_t M,
    int64_t N, int64_t K,
    int gsplit, int bps) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int T = NW * kWave;
    constexpr int R = kRingSlots;
    constexpr int TC = T / 2;                    // copy threads: waves NW/2 .. NW-1
    constexpr int LPT = CPT + (DOTS ? 0 : 1);     // copies per copy thread and tile
    constexpr int SLOT = CPT * TC * 16;          // code slot bytes
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = lane & 15;
    const int lg = lane >> 4;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);
    const int KB = (int)(K / 4);
    const int Mr = M < 16 ? (int)M : 16;
    const int64_t NT = (N + 15) / 16;
    const int bid = blockIdx.x;
    const int sidx = bid / bps;
    const int bl = bid - sidx * bps;
    const int g0 = sidx * gsplit;
    const int Gc = G - g0 < gsplit ? G - g0 : gsplit;
    const int cnt = (int)((NT - bl + bps - 1) / bps);

    uint8_t *ring = smem;                                               // [R][SLOT]
    uint8_t *wsr = smem + R * SLOT;                                     // [R][2048]
    uint8_t *sink = wsr + R * 2048;                                     // 1 KB
    float *part = reinterpret_cast<float *>(sink + 1024);               // [2][NW][4][64]

    // this wave's groups of the chunk: [g_lo, g_lo + ng), 1 <= ng <= GSG
    const int g_lo = (Gc * wave) / NW;
    const int ng = (Gc * (wave + 1)) / NW - g_lo;

    // Roles: the upper half of the waves issues every copy, the lower half
    // sums and stores the outputs, so a copy wave's vmcnt counts copies only
    // (no store between them) and its waits are exact; the summing waves
    // never wait on the copies, the barrier orders them.
    const bool copier = wave >= NW / 2;
    const int tc = tid - TC;                     // copy thread index
    const int cw = wave - NW / 2;                // copy wave index
    // copy sources: code unit u = i TC + tc of a slot, weight-scale unit tc
    const int ncu = 32 * Gc;
    const int rc2 = 2 * Gc;
    int coff[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int u = i * TC + tc;
        const int r = u / rc2;
        const int col = (u - r * rc2) ^ (r & 15);
        coff[i] = copier && u < ncu ? r * KB + 32 * g0 + 16 * col : kCopyOob;
    }
    int woff = kCopyOob;
    if (!DOTS && copier && tc < 2 * Gc) {
        const int cpr8 = Gc / 8;
        const int r = tc / cpr8;
        woff = 2 * (r * G + g0 + 8 * (tc - r * cpr8));
    }
    const bool ws_wave = kWave * cw < 2 * Gc;

    // tile j's copies into slot j % R; past the block's last tile every copy
    // reads past the range (zeros into the slot, no memory traffic)
    auto issue = [&](int j) __attribute__((always_inline)) {
        const bool live = j < cnt;
        const int64_t n0 = (int64_t)(bl + (int64_t)(live ? j : 0) * bps) * 16;
        const int64_t rows = N - n0 < 16 ? N - n0 : 16;
        const int slot = j % R;
        const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes + n0 * KB, rows * KB);
#pragma unroll
        for (int i = 0; i < CPT; ++i)
            copy16_to_lds(rc, ring + slot * SLOT + (i * TC + kWave * cw) * 16,
                          live ? coff[i] : kCopyOob);
        if (!DOTS) {
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(ws + n0 * G, rows * G * 2);
            uint8_t *dst = ws_wave ? wsr + slot * 2048 + 1024 * cw : sink;
            copy16_to_lds(rw, dst, live ? woff : kCopyOob);
        }
    };

    // prologue: the A fragments, -t seeds and token scales of this wave's
    // groups straight into VGPRs (tokens past M read past the buffer ranges:
    // zero seeds and scales, A repeats the last row; their outputs are never
    // stored), then the first R - 1 tiles' copies behind them.
    const int arow = c < Mr ? c : Mr - 1;
    v4i a0[GSG], a1[GSG], seed[GSG];
    v4f sv[GSG];
    if constexpr (FUSED) {
        // float32 x instead: the loads of the first two groups, the first
        // tiles' copies behind them, then each group quantised in registers
        // (quantize_ring_frag) while the loads of the group after next are
        // in flight; -t and s of the lane's output tokens 4 lg + i come from
        // lane 4 lg + i, which quantised that token.
        const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (int64_t)Mr * K * 4);
        const int xlane = arow * (int)K * 4 + 256 * (lg & 1) + 128 * (lg >> 1);
        v4f xf[2][8];
        auto load_x = [&](v4f (&f)[8], int b) __attribute__((always_inline)) {
            const int off = xlane + 512 * (g0 + g_lo + (b < ng ? b : ng - 1));
#pragma unroll
            for (int j = 0; j < 8; ++j)
                f[j] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rx, off + 16 * j, 0, 0));
        };
        load_x(xf[0], 0);
        if constexpr (GSG > 1) load_x(xf[1], 1);
        __builtin_amdgcn_sched_barrier(0);
        if (copier) {
#pragma unroll
            for (int p = 0; p < R - 1; ++p) issue(p);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int b = 0; b < GSG; ++b) {
            float sc;
            int ts;
            quantize_ring_frag(xf[b & 1], a0[b], a1[b], sc, ts);
            if (b + 2 < GSG) load_x(xf[b & 1], b + 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                seed[b][i] = -__shfl(ts, 4 * lg + i, kWave);
                sv[b][i] = __shfl(sc, 4 * lg + i, kWave);
            }
        }
    } else {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, (int64_t)Mr * K);
        const __amdgpu_buffer_rsrc_t rt = make_rsrc(t, (int64_t)Mr * G * 4);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(s, DOTS ? 0 : (int64_t)Mr * G * 4);
#pragma unroll
        for (int b = 0; b < GSG; ++b) {
            const int g = g0 + g_lo + (b < ng ? b : ng - 1);
            const int off = arow * (int)K + kGroup * g + 16 * lg;
            a0[b] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
            a1[b] = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 64, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * lg + i;
                const int toff = m < Mr ? 4 * (m * G + g) : kCopyOob;
                seed[b][i] = -__builtin_amdgcn_raw_buffer_load_b32(rt, toff, 0, 0);
                if (!DOTS)
                    sv[b][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, toff, 0, 0));
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the copies behind these loads
        if (copier) {
#pragma unroll
            for (int p = 0; p < R - 1; ++p) issue(p);
        }
    }
    // Hand the fragments to the loop as plain register values: the compiler
    // waits for their loads here (only the copies behind them may stay in
    // flight) instead of draining every copy before the loop.
#pragma unroll
    for (int b = 0; b < GSG; ++b) {
        asm volatile("" : "+v"(a0[b]), "+v"(a1[b]), "+v"(seed[b]));
        if (!DOTS) asm volatile("" : "+v"(sv[b]));
    }

    // the tile's groups in straight-line code for the wave's exact count NG:
    // every B read and weight scale first, then NG independent MFMA chains,
    // then the epilogues (no per-group branch or LDS round trip in between)
    auto compute_tile = [&](int j, auto ngc) __attribute__((always_inline)) {
        constexpr int NG = decltype(ngc)::value;
        const int64_t n0 = (int64_t)(bl + (int64_t)j * bps) * 16;
        const uint8_t *cs = ring + (j % R) * SLOT + c * rc2 * 16;
        const uint16_t *wrow = reinterpret_cast<const uint16_t *>(wsr + (j % R) * 2048) + c * Gc;
        v4i w[NG];
#pragma unroll
        for (int b = 0; b < NG; ++b)
            w[b] = *reinterpret_cast<const v4i *>(cs + 16 * ((2 * (g_lo + b) + (lg & 1)) ^ c));
        float wsf[NG];
        if (!DOTS) {
#pragma unroll
            for (int b = 0; b < NG; ++b) wsf[b] = half_bits_to_float(wrow[g_lo + b]);
        }
        v4i dd[NG];
#pragma unroll
        for (int b = 0; b < NG; ++b) {
            v4i b0, b1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t sh = (uint32_t)w[b][k] >> sh0;
                b0[k] = (int)(sh & kPlaneMask);
                b1[k] = (int)((sh >> 4) & kPlaneMask);
            }
            dd[b] = mfma16x16x64(a0[b], b0, seed[b]);
            dd[b] = mfma16x16x64(a1[b], b1, dd[b]);
        }
        if (DOTS) {
            const int64_t n = n0 + c;
#pragma unroll
            for (int b = 0; b < NG; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int m = 4 * lg + i;
                    if (m < M && n < N) d[((int64_t)m * N + n) * G + g0 + g_lo + b] = dd[b][i];
                }
        } else {
            float acc0 = 0.0f, acc1 = 0.0f, acc2 = 0.0f, acc3 = 0.0f;
#pragma unroll
            for (int b = 0; b < NG; ++b) {
                acc0 = fmaf((float)dd[b][0], sv[b][0] * wsf[b], acc0);
                acc1 = fmaf((float)dd[b][1], sv[b][1] * wsf[b], acc1);
                acc2 = fmaf((float)dd[b][2], sv[b][2] * wsf[b], acc2);
                acc3 = fmaf((float)dd[b][3], sv[b][3] * wsf[b], acc3);
            }
            float *pw = part + ((j & 1) * NW + wave) * 4 * kWave + lane;
            pw[0] = acc0;
            pw[kWave] = acc1;
            pw[2 * kWave] = acc2;
            pw[3 * kWave] = acc3;
        }
    };

    float *out = part_out ? part_out + (int64_t)sidx * M * N : y;
    uint16_t *out16 = part_out ? nullptr : y16;   // partial sums stay float32
    // summing wave i (< 4) adds slot i of every lane's partials (token
    // 4 (lane / 16) + i, row lane % 16) in wave order; the reads go out
    // before the next tile's compute, the sum and store follow it
    auto read_partials = [&](int j, float (&pv)[NW]) __attribute__((always_inline)) {
        const float *pr = part + (j & 1) * NW * 4 * kWave + wave * kWave + lane;
#pragma unroll
        for (int w = 0; w < NW; ++w) pv[w] = pr[w * 4 * kWave];
    };
    auto store_sum = [&](int j, const float (&pv)[NW]) __attribute__((always_inline)) {
        const int64_t n0 = (int64_t)(bl + (int64_t)j * bps) * 16;
        float v = pv[0];
#pragma unroll
        for (int w = 1; w < NW; ++w) v += pv[w];
        const int64_t m = 4 * lg + wave, n = n0 + c;
        if (m < M && n < N) store_y(out, out16, m * N + n, v);
    };

    static_assert(NW == 8, "four summing waves, one per partial slot");
    static_assert(!(FUSED && DOTS), "the fused variant writes y");
    if (copier) {
        for (int j = 0; j < cnt; ++j) {
            wait_vmem<(R - 2) * LPT>();  // this thread's copies of tile j have landed
            ring_barrier();              // ... and every copier's; tile j - 1 is done
            issue(j + R - 1);            // into tile j - 1's slot
            with_count<GSG>(ng, [&](auto ngc) { compute_tile(j, ngc); });
        }
        wait_vmem<0>();                  // no copy may land after the block ends
        ring_barrier();
    } else {
        for (int j = 0; j < cnt; ++j) {
            ring_barrier();
            float pv[NW];
            if (!DOTS && j > 0) read_partials(j - 1, pv);
            with_count<GSG>(ng, [&](auto ngc) { compute_tile(j, ngc); });
            if (!DOTS && j > 0) store_sum(j - 1, pv);
        }
        ring_barrier();
        if (!DOTS) {
            float pv[NW];
            read_partials(cnt - 1, pv);
            store_sum(cnt - 1, pv);
        }
    }
}

// y = sum over the S chunks of part[s] (fixed order s = 0, 1, ...).
__global__ __launch_bounds__(256) void panel_split_sum_kernel(const float *__restrict__ part,
                                                              float *__restrict__ y,
                                                              uint16_t *__restrict__ y16, int64_t MN,
                                                              int S) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float v = part[i];
    for (int k = 1; k < S; ++k) v += part[(int64_t)k * MN + i];
    store_y(y, y16, i, v);
}

struct DevLimits {
    int cus = 0;
    int lds_block = 0;
    int lds_cu = 0;
};

// Compute units and LDS limits of the current device, read once per device.
DevLimits dev_limits() {
    static DevLimits cache[64];
    static std::mutex mu;             // host threads may plan launches concurrently
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DevLimits();
    std::lock_guard<std::mutex> lock(mu);
    DevLimits &l = cache[dev];
    if (l.cus == 0) {
        DevLimits v;
        if (hipDeviceGetAttribute(&v.lds_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) ==
                hipSuccess &&
            hipDeviceGetAttribute(&v.lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) == hipSuccess &&
            hipDeviceGetAttribute(&v.cus, hipDeviceAttributeMultiprocessorCount, dev) ==
                hipSuccess)
            l = v;
    }
    return l;
}

template <int NW, int GS, int R>
hipError_t launch_cfg(const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, float *part, int64_t M, int64_t N, int64_t K,
                      int gsplit, int bps, int64_t blocks, size_t lds, hipStream_t stream) {
    if (out.d) {
        hipLaunchKernelGGL((small_panel_kernel<NW, GS, R, true>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, nullptr, t, codes, nullptr, nullptr,
                           nullptr, out.d, nullptr, M, N, K, gsplit, bps);
    } else {
        hipLaunchKernelGGL((small_panel_kernel<NW, GS, R, false>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, out.s, t, codes, out.ws, out.y,
                           out.y16, nullptr, part, M, N, K, gsplit, bps);
    }
    return hipGetLastError();
}

// GS = ceil(pairs per chunk / NW) exactly: a wave's short slice costs at most
// one repeated load.
template <int NW, int R>
hipError_t launch_gs(int64_t gs, const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, float *part, int64_t M, int64_t N, int64_t K,
                     int gsplit, int bps, int64_t blocks, size_t lds, hipStream_t stream) {
#define PQ2_PANEL_GS(V)                                                                        \
    case V:                                                                                    \
        return launch_cfg<NW, V, R>(q, t, codes, out, part, M, N, K, gsplit, bps, blocks, lds, \
                                    stream);
    switch (gs) {
        PQ2_PANEL_GS(1)
        PQ2_PANEL_GS(2)
        PQ2_PANEL_GS(3)
        PQ2_PANEL_GS(4)
        PQ2_PANEL_GS(5)
        PQ2_PANEL_GS(6)
        PQ2_PANEL_GS(7)
        PQ2_PANEL_GS(8)
        PQ2_PANEL_GS(9)
        default: return hipErrorInvalidValue;
    }
#undef PQ2_PANEL_GS
}

template <int NW, int GSG, int TT>
hipError_t launch_sc_cfg(const int8_t *q, const int32_t *t, const uint8_t *codes,
                         const GemmOut &out, float *part, int64_t M, int64_t N, int64_t K,
                         int gsplit, int bps, int64_t blocks, size_t lds, hipStream_t stream) {
    // 16-byte code chunks per thread: 32 gsplit <= 32 GSG NW / TT chunks
    constexpr int CPT = (32 * GSG * (NW / TT) + NW * kWave - 1) / (NW * kWave);
    if (out.d) {
        hipLaunchKernelGGL((small_panel_sc_kernel<NW, GSG, CPT, TT, true>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, nullptr, t, codes, nullptr, nullptr,
                           nullptr, out.d, nullptr, M, N, K, gsplit, bps);
    } else {
        hipLaunchKernelGGL((small_panel_sc_kernel<NW, GSG, CPT, TT, false>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, out.s, t, codes, out.ws, out.y,
                           out.y16, nullptr, part, M, N, K, gsplit, bps);
    }
    return hipGetLastError();
}

template <int NW, int TT>
hipError_t launch_sc(int64_t gs, const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, float *part, int64_t M, int64_t N, int64_t K,
                     int gsplit, int bps, int64_t blocks, size_t lds, hipStream_t stream) {
#define PQ2_PANEL_SC(V)                                                                          \
    case V:                                                                                      \
        return launch_sc_cfg<NW, V, TT>(q, t, codes, out, part, M, N, K, gsplit, bps, blocks, lds, \
                                        stream);
    switch (gs) {
        PQ2_PANEL_SC(1)
        PQ2_PANEL_SC(2)
        PQ2_PANEL_SC(3)
        PQ2_PANEL_SC(4)
        PQ2_PANEL_SC(5)
        PQ2_PANEL_SC(6)
        PQ2_PANEL_SC(7)
        PQ2_PANEL_SC(8)
        PQ2_PANEL_SC(9)
        default: return hipErrorInvalidValue;
    }
#undef PQ2_PANEL_SC
}

template <int NW, int GSG, bool DOTS, bool FUSED>
hipError_t launch_ring_cfg(const float *x, const int8_t *q, const int32_t *t,
                           const uint8_t *codes, const GemmOut &out, float *part, int64_t M,
                           int64_t N, int64_t K, int gsplit, int bps, int64_t blocks, size_t lds,
                           hipStream_t stream) {
    constexpr int CPT = GSG;     // 32 * 8 GSG code units over the 256 copy threads, NW = 8
    hipLaunchKernelGGL((small_panel_ring_kernel<NW, GSG, CPT, DOTS, FUSED>), dim3((unsigned)blocks),
                       dim3(NW * kWave), lds, stream, x, q, DOTS ? nullptr : out.s, t, codes,
                       DOTS ? nullptr : out.ws, DOTS ? nullptr : out.y, DOTS ? nullptr : out.y16,
                       out.d, part, M, N, K,
                       gsplit, bps);
    return hipGetLastError();
}

// x != nullptr: the fused variant (quantises x itself; q and t unused).
template <int NW>
hipError_t launch_ring(int64_t gs, const float *x, const int8_t *q, const int32_t *t,
                       const uint8_t *codes, const GemmOut &out, float *part, int64_t M,
                       int64_t N, int64_t K, int gsplit, int bps, int64_t blocks, size_t lds,
                       hipStream_t stream) {
#define PQ2_PANEL_RING(V)                                                                       \
    case V:                                                                                     \
        if (out.d)                                                                              \
            return launch_ring_cfg<NW, V, true, false>(nullptr, q, t, codes, out, part, M, N,   \
                                                       K, gsplit, bps, blocks, lds, stream);    \
        if (x)                                                                                  \
            return launch_ring_cfg<NW, V, false, true>(x, nullptr, nullptr, codes, out, part,   \
                                                       M, N, K, gsplit, bps, blocks, lds,       \
                                                       stream);                                 \
        return launch_ring_cfg<NW, V, false, false>(nullptr, q, t, codes, out, part, M, N, K,   \
                                                    gsplit, bps, blocks, lds, stream);
    switch (gs) {
        PQ2_PANEL_RING(1)
        PQ2_PANEL_RING(2)
        PQ2_PANEL_RING(3)
        PQ2_PANEL_RING(4)
        PQ2_PANEL_RING(5)
        PQ2_PANEL_RING(6)
        default: return hipErrorInvalidValue;
    }
#undef PQ2_PANEL_RING
}

constexpr int kPanelWaves = 8;
constexpr int kPanelMaxGs = 9;

// 16-token tiles of the staged-codes kernel: 1, 2 or 4 (M <= 16, 32, 64;
// the tiles must divide the 8 waves)
int panel_token_tiles(int64_t M) { return M <= 16 ? 1 : M <= 32 ? 2 : 4; }

struct PanelPlan {
    int S = 0;            // K chunks (0: no plan fits)
    int tt = 1;           // 16-token tiles (staged-codes kernel)
    int gsplit = 0;       // groups per chunk (the last one may be shorter)
    int bps = 0;          // blocks per chunk
    int64_t lds = 0;
    int64_t gs = 0;       // group pairs per wave and tile
};

// Whether K can be cut into S chunks here: chunks of a multiple of 8 groups
// (whole 16-byte scale chunks per row) and at least 16 groups each (every
// wave gets a pair; the staged-codes kernel needs one group per wave of a
// token tile, 8 suffice), at most 9 pairs or groups per wave, LDS within the
// block limit. Only the staged-codes kernel takes M > 16.
PanelPlan plan_for(int S, int64_t M, int64_t N, int64_t K, const DevLimits &l, bool sc) {
    PanelPlan p;
    const int tt = sc ? panel_token_tiles(M) : 1;
    const int64_t G = K / kGroup, NT = (N + 15) / 16, Mr = M < 16 * tt ? M : 16 * tt;
    if (M > 16 * tt) return p;
    if (S > 1 && G % 8 != 0) return p;
    const int64_t gsplit = S == 1 ? G : ((G + S - 1) / S + 7) / 8 * 8;
    if ((G + gsplit - 1) / gsplit != S) return p;
    const int64_t last = G - (S - 1) * gsplit;
    if ((gsplit < last ? gsplit : last) < (sc && S > 1 ? 8 : 16)) return p;
    // register-operand kernel: group pairs per wave; staged codes: groups per
    // wave of a token tile
    const int64_t kw = kPanelWaves / tt;
    const int64_t gs = sc ? (gsplit + kw - 1) / kw
                          : ((gsplit + 1) / 2 + kPanelWaves - 1) / kPanelWaves;
    if (gs > kPanelMaxGs) return p;
    const int64_t lds = sc ? panel_lds_bytes_sc(Mr, gsplit, kPanelWaves, tt)
                           : panel_lds_bytes(Mr, gsplit, kPanelWaves);
    if (lds > l.lds_block) return p;
    const int64_t per_cu = (S == 1 && l.lds_cu / lds >= 2) ? 2 : 1;
    int64_t bps = l.cus * per_cu / S;
    if (bps > NT) bps = NT;
    if (bps < 1) return p;
    p.S = S;
    p.tt = tt;
    p.gsplit = (int)gsplit;
    p.bps = (int)bps;
    p.lds = lds;
    p.gs = gs;
    return p;
}

// The split count (MI355X sweeps over the 5120 / 6144 / 17408 shapes at M = 4,
// 8, 16): chunks of about 48 groups win -- K = 5120 and 6144 unsplit (a
// split's partial sums and extra summing launch cost more than the uneven
// tile count saves), K = 17408 in three chunks (14.3-15.8 us against 15.6-17.4
// for two or four, 17.0 unsplit where it fits). The count nearest to G / 48
// that fits, preferring more chunks.
PanelPlan plan_panel(int64_t M, int64_t N, int64_t K, const DevLimits &l, int max_splits,
                     bool sc) {
    PanelPlan none;
    if (l.cus <= 0 || M < 1 || M > (sc ? kPanelMaxM : 16) || max_splits < 1) return none;
    const int cap = max_splits < kPanelMaxSplits ? max_splits : kPanelMaxSplits;
    const int64_t G = K / kGroup;
    int target = (int)((G + 24) / 48);
    target = target < 1 ? 1 : target > cap ? cap : target;
    for (int S = target; S <= cap; ++S) {
        const PanelPlan p = plan_for(S, M, N, K, l, sc);
        if (p.S) return p;
    }
    for (int S = target - 1; S >= 1; --S) {
        const PanelPlan p = plan_for(S, M, N, K, l, sc);
        if (p.S) return p;
    }
    return none;
}

// Ring variant: M <= 16, chunks of a multiple of 8 groups (the column swizzle
// permutes within 16-unit blocks of a row), at most 8 groups per wave, LDS
// within the block limit; same split rule as the other variants.
PanelPlan plan_ring_for(int S, int64_t M, int64_t N, int64_t K, const DevLimits &l) {
    PanelPlan p;
    const int64_t G = K / kGroup, NT = (N + 15) / 16;
    if (M > 16 || G % 8 != 0) return p;
    const int64_t gsplit = ((G + S - 1) / S + 7) / 8 * 8;
    if ((G + gsplit - 1) / gsplit != S) return p;
    const int64_t gs = gsplit / kPanelWaves;
    if (gs < 1 || gs > kRingMaxGs) return p;
    const int64_t lds = ring_lds_bytes((int)gs, kPanelWaves);
    if (lds > l.lds_block) return p;
    int64_t bps = l.cus / S;
    if (bps > NT) bps = NT;
    if (bps < 1) return p;
    p.S = S;
    p.gsplit = (int)gsplit;
    p.bps = (int)bps;
    p.lds = lds;
    p.gs = gs;
    return p;
}

PanelPlan plan_ring(int64_t M, int64_t N, int64_t K, const DevLimits &l, int max_splits) {
    PanelPlan none;
    if (l.cus <= 0 || M < 1 || M > 16 || max_splits < 1) return none;
    const int cap = max_splits < kPanelMaxSplits ? max_splits : kPanelMaxSplits;
    const int64_t G = K / kGroup;
    int target = (int)((G + 24) / 48);
    target = target < 1 ? 1 : target > cap ? cap : target;
    for (int S = target; S <= cap; ++S) {
        const PanelPlan p = plan_ring_for(S, M, N, K, l);
        if (p.S) return p;
    }
    return none;
}

}  // namespace

hipError_t launch_split_sum(const float *part, float *y, uint16_t *y16, int64_t MN, int splits,
                            hipStream_t stream) {
    hipLaunchKernelGGL(panel_split_sum_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0,
                       stream, part, y, y16, MN, splits);
    return hipGetLastError();
}

int device_cus() { return dev_limits().cus; }

bool small_panel_ring_fits(int64_t M, int64_t K, int max_splits) {
    if (M < 1 || M > 16 || K > kPanelMaxK || K / kGroup < 16) return false;
    return plan_ring(M, 16, K, dev_limits(), max_splits).S > 0;
}

bool small_panel_fits(int64_t M, int64_t K, int max_splits) {
    if (M < 1 || M > kPanelMaxM || K > kPanelMaxK || K / kGroup < 16) return false;
    // M <= 16: the register-operand kernel's plan (the fallback) must exist
    return plan_panel(M, 16, K, dev_limits(), max_splits, M > 16).S > 0;
}

namespace {

// The plan launch_small_panel runs: the ring variant where it has a plan,
// else the staged-codes kernel (MI355X sweeps: 2-14 % faster than the
// register-operand kernel on five of the nine 5120 / 6144 / 17408 shapes at
// M = 4, 8, 16, slower on one; one tile of register prefetch beat two on all
// nine), else the register-operand kernel.
enum class PanelKind { kNone, kRing, kStaged, kRegs };

PanelPlan choose_panel(int64_t M, int64_t N, int64_t K, int max_splits, PanelKind &kind) {
    const DevLimits l = dev_limits();
    PanelPlan plan = plan_ring(M, N, K, l, max_splits);
    kind = PanelKind::kRing;
    if (plan.S == 0) {
        plan = plan_panel(M, N, K, l, max_splits, true);
        kind = PanelKind::kStaged;
    }
    if (plan.S == 0) {
        plan = plan_panel(M, N, K, l, max_splits, false);
        kind = PanelKind::kRegs;
    }
    if (plan.S == 0) kind = PanelKind::kNone;
    return plan;
}

}  // namespace

// Split-K partial sums of the allocation-free entry: a file-scope device
// array (one copy per device, alive until the process ends). Host code never
// passes the array's name to a kernel -- in host code it is a stand-in, not
// a device address -- but the address hipGetSymbolAddress returns for the
// current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

float *scratch_address(hipError_t *err) {
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess && (dev < 0 || dev >= 64)) e = hipErrorInvalidDevice;
    if (e != hipSuccess) {
        *err = e;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
            return nullptr;
        }
        addr[dev] = p;
    }
    *err = hipSuccess;
    return static_cast<float *>(addr[dev]);
}

int small_panel_splits(int64_t M, int64_t N, int64_t K, int max_splits) {
    if (!small_panel_fits(M, K, max_splits)) return 0;
    PanelKind kind;
    return choose_panel(M, N, K, max_splits, kind).S;
}

// One block of 8 waves per CU (two when two panels fit in a CU's LDS and K
// is not split). Two tiles in flight per wave (R = 2): sweeps on MI355X found
// deeper rings, 16-wave blocks and two blocks per CU all slower on the
// 5120 / 6144 / 17408 shapes.
hipError_t launch_small_panel(const int8_t *q, const int32_t *t, const uint8_t *codes,
                              const GemmOut &out, int64_t M, int64_t N, int64_t K,
                              int max_splits, float *work, hipStream_t stream) {
    PanelKind kind;
    const PanelPlan plan = choose_panel(M, N, K, max_splits, kind);
    if (kind == PanelKind::kNone) return hipErrorInvalidValue;
    const bool rg = kind == PanelKind::kRing, sc = kind == PanelKind::kStaged;
    // the exact group dots go straight to d per chunk; float partials need
    // the caller's workspace
    float *part = nullptr;
    if (plan.S > 1 && !out.d) {
        if (!work) return hipErrorInvalidValue;
        part = work;
    }
    const int64_t blocks = (int64_t)plan.bps * plan.S;
    hipError_t e;
    if (rg)
        e = launch_ring<kPanelWaves>(plan.gs, nullptr, q, t, codes, out, part, M, N, K, plan.gsplit,
                                     plan.bps, blocks, plan.lds, stream);
    else if (sc && plan.tt == 1)
        e = launch_sc<kPanelWaves, 1>(plan.gs, q, t, codes, out, part, M, N, K, plan.gsplit,
                                      plan.bps, blocks, plan.lds, stream);
    else if (sc && plan.tt == 2)
        e = launch_sc<kPanelWaves, 2>(plan.gs, q, t, codes, out, part, M, N, K, plan.gsplit,
                                      plan.bps, blocks, plan.lds, stream);
    else if (sc)
        e = launch_sc<kPanelWaves, 4>(plan.gs, q, t, codes, out, part, M, N, K, plan.gsplit,
                                      plan.bps, blocks, plan.lds, stream);
    else
        e = launch_gs<kPanelWaves, 2>(plan.gs, q, t, codes, out, part, M, N, K, plan.gsplit,
                                      plan.bps, blocks, plan.lds, stream);
    if (e != hipSuccess || !part) return e;
    return launch_split_sum(part, out.y, out.y16, M * N, plan.S, stream);
}

int small_panel_fused_splits(int64_t M, int64_t N, int64_t K, int max_splits) {
    if (!small_panel_ring_fits(M, K, max_splits)) return 0;
    return plan_ring(M, N, K, dev_limits(), max_splits).S;
}

// The ring variant's plan for this shape, with the fused prologue: the same
// tiles, chunks and split sums as launch_small_panel's ring plan.
hipError_t launch_small_panel_fused(const float *x, const uint8_t *codes, const uint16_t *ws,
                                    float *y, int64_t M, int64_t N, int64_t K, int max_splits,
                                    float *work, hipStream_t stream) {
    if (!small_panel_ring_fits(M, K, max_splits)) return hipErrorInvalidValue;
    const PanelPlan plan = plan_ring(M, N, K, dev_limits(), max_splits);
    if (plan.S == 0) return hipErrorInvalidValue;
    float *part = nullptr;
    if (plan.S > 1) {
        if (!work) return hipErrorInvalidValue;
        part = work;
    }
    const GemmOut out{y, nullptr, nullptr, ws};
    const int64_t blocks = (int64_t)plan.bps * plan.S;
    hipError_t e = launch_ring<kPanelWaves>(plan.gs, x, nullptr, nullptr, codes, out, part, M, N,
                                            K, plan.gsplit, plan.bps, blocks, plan.lds, stream);
    if (e != hipSuccess || !part) return e;
    return launch_split_sum(part, y, nullptr, M * N, plan.S, stream);
}

}  // namespace pq2
