// small_mfma.hip -- K3: PQ2_0 product for 2..16 token rows on int8 MFMA.
//
// Plane dot products become arithmetic-bound from about three tokens (page
// "Making a ternary reasoning model fast in vLLM", section "One token at a
// time", last paragraph); the small-batch path instead places code bytes
// directly in the matrix-instruction operand registers, where a shift and a
// mask per register pull one 2-bit plane out (section "Small batches: make
// the register layout explicit"), and loads every weight once for all token
// rows.
//
// gfx950 mapping (v_mfma_i32_16x16x64_i8, tokens padded to 16):
//  * A block owns 16*TILES weight rows and all tokens; its NW waves split the
//    K groups between them and their float partials are summed through LDS
//    in wave order (a fixed order, so results are deterministic). Each wave
//    covers all TILES 16-row tiles of the block, so every activation fragment
//    it loads serves TILES MFMA tiles: the L2->CU traffic for activations
//    drops from 4x the code bytes (one tile per load at 16 tokens) to 4/TILES.
//  * Per group, lane (r = lane % 16, lane group lg = lane / 16) loads 16 bytes
//    of row r: code words 4*(lg&1) .. 4*(lg&1)+3. MFMA a (a = 0, 1) takes
//    plane p = 2a + (lg>>1) of those four words as its A operand (one shift
//    and one mask per word); its B operand is the 16 plane-order activation
//    bytes of token r that pair with them, bytes 32p + 16*(lg&1) .. +15 of
//    the group: a single 16-byte load. Across the four lane groups MFMA 0
//    covers planes 0-1 and MFMA 1 planes 2-3 of the group. The k order inside
//    the instruction is the same function of (lane group, register, byte)
//    for A and B, so any such order gives the exact dot.
//  * The accumulator is seeded with -t[m][g]; two MFMAs give the exact group
//    dot D[n][m]. Lane (lg, m) then holds rows 4lg..4lg+3 of token m and
//    applies acc += D * (s[m][g] * ws[n][g]).
//  * The main loop issues only 16-byte loads: TILES code loads and the two
//    B fragments per group. The block's weight scales and the tokens' s and
//    t are staged in LDS once per block, with straight-line loads issued in
//    the same memory round trip as the first batch of GB groups.
#include "pq2_device.hpp"
#include "pq2_launch.hpp"

namespace pq2 {

namespace {

// LDS words: weight scales [16*TILES][GP], token s and t [16][GP] (GP = G + 1,
// odd, so the 16 lanes of a lane group read 16 different rows without bank
// conflicts); reused for the wave partials [NW][64][4*TILES] after compute.
__host__ __device__ constexpr int small_lds_words(int G, int tiles, int nw) {
    const int tables = (16 * tiles + 32) * (G + 1);
    const int parts = nw * 64 * 4 * tiles;
    return tables > parts ? tables : parts;
}

template <int NW, int TILES, int GB, int PER, bool DOTS>
__global__ __launch_bounds__(NW * kWave) void small_mfma_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    uint16_t *__restrict__ y16,
    int32_t *__restrict__ d, int64_t M, int64_t N, int64_t K) {
    extern __shared__ float sm[];
    constexpr int T = NW * kWave;      // threads per block
    constexpr int ROWS = 16 * TILES;   // weight rows per block
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r = lane & 15;           // A row within a tile, and B token
    const int lg = lane >> 4;          // lane group
    const int half = lg & 1;           // which four code words of the group
    const int sh0 = 2 * (lg >> 1);     // plane of MFMA 0 is lg>>1, of MFMA 1 is 2 + lg>>1
    const int G = (int)(K / kGroup);
    const int GP = G + 1;
    const int64_t n0 = (int64_t)blockIdx.x * ROWS;
    const bool mvalid = r < M;
    // a padded token (r >= M) reads token M-1: its B column only feeds its
    // own D column, which is never stored
    const int64_t mc = mvalid ? r : M - 1;
    const int g_begin = (G * wave) / NW;
    const int g_end = (G * (wave + 1)) / NW;
    const int ng = g_end - g_begin;

    float *ws_l = sm;                                           // [ROWS][GP]
    float *s_l = ws_l + ROWS * GP;                              // [16][GP]
    int32_t *t_l = reinterpret_cast<int32_t *>(s_l + 16 * GP);  // [16][GP]

    const uint4 *ap[TILES];
#pragma unroll
    for (int ti = 0; ti < TILES; ++ti) {
        const int64_t row = n0 + 16 * ti + r;
        ap[ti] = reinterpret_cast<const uint4 *>(codes + (row < N ? row : N - 1) * (K / 4) +
                                                 16 * half);
    }
    const int8_t *bp = q + mc * K + 16 * half + 16 * sh0;

    // One batch: the codes of TILES tiles and both B fragments of GB groups,
    // loaded straight-line (indices clamped, never predicated).
    uint4 cb[GB][TILES], qb0[GB], qb1[GB];
    auto load_batch = [&](int i0) {
#pragma unroll
        for (int b = 0; b < GB; ++b) {
            const int g = g_begin + min(i0 + b, ng - 1);
#pragma unroll
            for (int ti = 0; ti < TILES; ++ti) cb[b][ti] = ap[ti][2 * g];
            qb0[b] = *reinterpret_cast<const uint4 *>(bp + kGroup * g);
            qb1[b] = *reinterpret_cast<const uint4 *>(bp + kGroup * g + 64);
        }
    };
    load_batch(0);     // ng >= 1: the host gives every wave a group

    // Stage the scales of the block's rows and the tokens. Straight-line: PER
    // elements per thread and table (the host guarantees ROWS*G <= PER*T and
    // 16*G <= PER*T), loads clamped and unpredicated and issued before any
    // store, so they share the first batch's memory round trip. Element
    // e = threadIdx.x + i*T of a [rows][G] table sits at (row, col) =
    // divmod(e, G), advanced by (T / G, T % G) per step.
    {
        const int mrows = M < 16 ? (int)M : 16;
        const int nrows = (N - n0) < ROWS ? (int)(N - n0) : ROWS;
        const int cnt_w = nrows * G, cnt_m = mrows * G;
        const uint16_t *wsrc = ws + n0 * G;
        uint16_t wv[PER];
        float sv[PER];
        int32_t tv[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (int)threadIdx.x + i * T;
            if (!DOTS) {
                wv[i] = wsrc[min(e, cnt_w - 1)];
                sv[i] = s[min(e, cnt_m - 1)];
            }
            tv[i] = t[min(e, cnt_m - 1)];
        }
        const int dr = T / G, dc = T - dr * G;
        int row = (int)threadIdx.x / G, col = (int)threadIdx.x - row * G;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = (int)threadIdx.x + i * T;
            const int at = row * GP + col;
            if (!DOTS && e < cnt_w) ws_l[at] = half_bits_to_float(wv[i]);
            if (e < cnt_m) {
                if (!DOTS) s_l[at] = sv[i];
                t_l[at] = tv[i];
            }
            row += dr;
            col += dc;
            if (col >= G) {
                col -= G;
                ++row;
            }
        }
    }
    __syncthreads();

    float acc[TILES][4];
#pragma unroll
    for (int ti = 0; ti < TILES; ++ti)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[ti][i] = 0.0f;

    auto compute_batch = [&](int i0) {
#pragma unroll
        for (int b = 0; b < GB; ++b) {
            if (i0 + b >= ng) break;
            const int g = g_begin + i0 + b;
            const v4i b0 = {(int)qb0[b].x, (int)qb0[b].y, (int)qb0[b].z, (int)qb0[b].w};
            const v4i b1 = {(int)qb1[b].x, (int)qb1[b].y, (int)qb1[b].z, (int)qb1[b].w};
            const int tneg = -t_l[r * GP + g];
            const v4i seed = {tneg, tneg, tneg, tneg};
            float sg = 0.0f;
            if (!DOTS) sg = s_l[r * GP + g];
#pragma unroll
            for (int ti = 0; ti < TILES; ++ti) {
                const uint4 w = cb[b][ti];
                const uint32_t wv4[4] = {w.x, w.y, w.z, w.w};
                v4i a0, a1;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t sh = wv4[j] >> sh0;
                    a0[j] = (int)(sh & kPlaneMask);
                    a1[j] = (int)((sh >> 4) & kPlaneMask);
                }
                v4i dd = mfma16x16x64(a0, b0, seed);
                dd = mfma16x16x64(a1, b1, dd);
                const int lrow = 16 * ti + 4 * lg;      // block-local D rows lrow .. lrow+3
                if (DOTS) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int64_t n = n0 + lrow + i;
                        if (mvalid && n < N) d[((int64_t)r * N + n) * G + g] = dd[i];
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc[ti][i] = fmaf((float)dd[i], sg * ws_l[(lrow + i) * GP + g], acc[ti][i]);
                }
            }
        }
    };

    compute_batch(0);
    for (int i0 = GB; i0 < ng; i0 += GB) {
        load_batch(i0);
        compute_batch(i0);
    }

    if (!DOTS) {
        __syncthreads();                  // the tables are dead: reuse LDS for partials
        float *part = sm;                 // [NW][64][4*TILES]
#pragma unroll
        for (int ti = 0; ti < TILES; ++ti)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part[(wave * kWave + lane) * 4 * TILES + 4 * ti + i] = acc[ti][i];
        __syncthreads();
        // wave w sums tiles w, w + NW, ... over all waves in wave order
        for (int ti = wave; ti < TILES; ti += NW) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = part[lane * 4 * TILES + 4 * ti + i];
                for (int w = 1; w < NW; ++w) v += part[(w * kWave + lane) * 4 * TILES + 4 * ti + i];
                const int64_t n = n0 + 16 * ti + 4 * lg + i;
                if (mvalid && n < N) store_y(y, y16, (int64_t)r * N + n, v);
            }
        }
    }
}

template <int NW, int TILES, int GB, int PER>
hipError_t launch_cfg(const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t blocks = (N + 16 * TILES - 1) / (16 * TILES);
    const int G = (int)(K / kGroup);
    const size_t lds = (size_t)small_lds_words(G, TILES, NW) * 4;
    if (out.d) {
        hipLaunchKernelGGL((small_mfma_kernel<NW, TILES, GB, PER, true>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, nullptr, t, codes, nullptr, nullptr,
                           nullptr, out.d, M, N, K);
    } else {
        hipLaunchKernelGGL((small_mfma_kernel<NW, TILES, GB, PER, false>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, out.s, t, codes, out.ws, out.y,
                           out.y16, nullptr, M, N, K);
    }
    return hipGetLastError();
}

// Staging elements per thread: the smallest of 2, 4, 8, 16 covering the
// largest table (16*TILES rows of G).
template <int NW, int TILES, int GB>
hipError_t launch_per(const int8_t *q, const int32_t *t, const uint8_t *codes,
                      const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
    const int64_t per = (16 * TILES * (K / kGroup) + NW * kWave - 1) / (NW * kWave);
    if (per <= 2) return launch_cfg<NW, TILES, GB, 2>(q, t, codes, out, M, N, K, stream);
    if (per <= 4) return launch_cfg<NW, TILES, GB, 4>(q, t, codes, out, M, N, K, stream);
    if (per <= 8) return launch_cfg<NW, TILES, GB, 8>(q, t, codes, out, M, N, K, stream);
    return launch_cfg<NW, TILES, GB, 16>(q, t, codes, out, M, N, K, stream);
}

}  // namespace

// Block shape (from sweeps on MI355X): 16 rows (TILES = 1) with NW waves
// splitting K so the grid holds ~2048 waves; 32 rows (TILES = 2, NW = 8) for
// K > 8192 at M > 4, where the activation re-reads of 16-row tiles dominate.
// (64-row blocks halve the activation traffic again but leave too few blocks
// for a single occupancy round on the N = 5120 / 17408 shapes.) Every wave
// gets at least one group, and NW covers the staging bound (PER = 16 covers
// 1024 * NW elements of a table).
template <int TILES>
hipError_t launch_tiles(int64_t nw, const int8_t *q, const int32_t *t, const uint8_t *codes,
                        const GemmOut &out, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
    if (nw >= 8) return launch_per<8, TILES, 4>(q, t, codes, out, M, N, K, stream);
    if (nw >= 4) return launch_per<4, TILES, 4>(q, t, codes, out, M, N, K, stream);
    if (nw >= 2) return launch_per<2, TILES, 4>(q, t, codes, out, M, N, K, stream);
    return launch_per<1, TILES, 4>(q, t, codes, out, M, N, K, stream);
}

hipError_t launch_small(const int8_t *q, const int32_t *t, const uint8_t *codes,
                        const GemmOut &out, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream) {
    const int64_t G = K / kGroup;
    int tiles = 1;
    if (M > 4 && G > 64 && (N + 31) / 32 >= 128) tiles = 2;
    int64_t nw;
    if (tiles > 1) {
        nw = 8;
    } else {
        const int64_t nt = (N + 15) / 16;
        nw = (2048 + nt - 1) / nt;
        nw = nw >= 8 ? 8 : nw >= 4 ? 4 : nw >= 2 ? 2 : 1;
    }
    while (tiles > 1 && small_lds_words((int)G, tiles, 8) * 4 > 65536) tiles /= 2;
    while (nw > 1 && nw > G) nw /= 2;
    while (nw * 1024 < 16 * tiles * G) nw *= 2;
    if (tiles == 2) return launch_tiles<2>(nw, q, t, codes, out, M, N, K, stream);
    return launch_tiles<1>(nw, q, t, codes, out, M, N, K, stream);
}

}  // namespace pq2
