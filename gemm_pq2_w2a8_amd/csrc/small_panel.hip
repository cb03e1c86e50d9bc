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

namespace pq2 {

namespace {

#ifndef PANEL_TUNE_OVERRIDE
#define PANEL_TUNE_OVERRIDE
#endif

constexpr int kPanelPad = 16;       // LDS row stride of the panel: K + 16 bytes

// LDS bytes: panel [Mr][K + 16]; s and -t tables [G][16]; weight scales of two
// tiles [2][16][G + 1] floats; partials [2][NW][64][4] floats.
__host__ __device__ constexpr int64_t panel_lds_bytes(int64_t Mr, int64_t K, int nw) {
    return Mr * (K + kPanelPad) + 2 * 16 * (K / kGroup) * 4 + 2 * 16 * (K / kGroup + 1) * 4 +
           2 * (int64_t)nw * kWave * 16;
}

template <int NW, int GS, int R, bool DOTS>
__global__ __launch_bounds__(NW * kWave) void small_panel_kernel(
    const int8_t *__restrict__ q, const float *__restrict__ s, const int32_t *__restrict__ t,
    const uint8_t *__restrict__ codes, const uint16_t *__restrict__ ws, float *__restrict__ y,
    int32_t *__restrict__ d, int64_t M, int64_t N, int64_t K) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    constexpr int T = NW * kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c = lane & 15;
    const int lg = lane >> 4;
    const int sh0 = 2 * (lg >> 1);
    const int G = (int)(K / kGroup);
    const int GP = G + 1;
    const int KB = (int)(K / 4);                 // code bytes per weight row
    const int RS = (int)K + kPanelPad;
    const int Mr = M < 16 ? (int)M : 16;
    const int64_t NT = (N + 15) / 16;
    const int B = gridDim.x;
    const int bid = blockIdx.x;
    const int cnt = (int)((NT - bid + B - 1) / B);    // tiles of this block (>= 1)

    int8_t *panel = reinterpret_cast<int8_t *>(smem);                        // [Mr][RS]
    float *s_l = reinterpret_cast<float *>(smem + (int64_t)Mr * RS);         // [G][16]
    int32_t *tn_l = reinterpret_cast<int32_t *>(s_l + 16 * G);               // [G][16], -t
    float *wsl = reinterpret_cast<float *>(tn_l + 16 * G);                   // [2][16][GP]
    float *part = wsl + 2 * 16 * GP;                                         // [2][NW][64][4]

    // This wave's group pairs of every tile: [p_lo, p_lo + np), 1 <= np <= GS
    // (the last pair has one group when G is odd).
    const int NP = (G + 1) / 2;
    const int p_lo = (NP * wave) / NW;
    const int np = (NP * (wave + 1)) / NW - p_lo;
    const int voff_c = c * KB + 16 * lg;

    // Weight scales of a tile: 16 * G halves, contiguous, as 2G 16-byte
    // chunks; thread tid < 2G loads chunk tid, elements 8 * tid .. + 7, whose
    // (row, column) in the [16][G] block starts at divmod(8 * tid, G).
    const int nwc = 2 * G;
    int w_row0 = 0, w_col0 = 0;
    if (!DOTS) {
        w_row0 = (8 * tid) / G;
        w_col0 = 8 * tid - w_row0 * G;
    }

    v4i cb[R][GS];
    v4i wv[R];
    // Past the block's last tile the loads still issue (so the wait counts
    // stay exact) but every lane reads the first bytes of the last tile:
    // one cache line per instruction instead of a tile slice.
    auto load_tile = [&](v4i (&cbs)[GS], v4i &wvs, int j) __attribute__((always_inline)) {
        const bool live = j < cnt;
        const int jj = live ? j : cnt - 1;
        const int64_t n0 = (int64_t)(bid + (int64_t)jj * B) * 16;
        const int64_t rows = N - n0 < 16 ? N - n0 : 16;
        if (!DOTS) {
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(ws + n0 * G, rows * G * 2);
            wvs = __builtin_amdgcn_raw_buffer_load_b128(rw, live && tid < nwc ? 16 * tid : 0, 0, 0);
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
        if (!DOTS && tid < nwc) {
            float *dst = wsl + buf * 16 * GP;
            int row = w_row0, col = w_col0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t word = (uint32_t)wvs[k >> 1];
                dst[row * GP + col] = half_bits_to_float((uint16_t)((k & 1) ? word >> 16 : word));
                if (++col == G) {
                    col = 0;
                    ++row;
                }
            }
        }
    };

    // Prefetch the first R - 1 tiles, then stage the panel, the token tables
    // and the first tile's weight scales.
#pragma unroll
    for (int u = 0; u < R - 1; ++u) load_tile(cb[u], wv[u], u);

    {
        const int cpr = (int)(K / 16);           // 16-byte chunks per token row
        const int total = Mr * cpr;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q, (int64_t)Mr * K);
        // chunk e = tid + i*T sits at (row, col) = divmod(e, cpr), advanced by
        // (T / cpr, T % cpr) per step
        const int dr = T / cpr, dc = T - dr * cpr;
        int row = tid / cpr, col = tid - row * cpr;
        for (int e0 = 0; e0 < total; e0 += 8 * T) {
            v4i v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = e0 + tid + i * T;
                v[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * (e < total ? e : total - 1), 0, 0);
            }
            // unconditional stores (a conditional one lets the compiler sink its
            // load next to it): a chunk past the end was loaded as the last
            // chunk and is stored there again, the same bytes
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const bool in = e0 + tid + i * T < total;
                *reinterpret_cast<v4i *>(panel + (in ? row : Mr - 1) * RS +
                                         16 * (in ? col : cpr - 1)) = v[i];
                row += dr;
                col += dc;
                if (col >= cpr) {
                    col -= cpr;
                    ++row;
                }
            }
        }
        // tables [g][m]: tokens m >= M hold 0 (their outputs are never stored)
        for (int e = tid; e < 16 * G; e += T) {
            const int g = e >> 4, m = e & 15;
            const bool ok = m < Mr;
            if (!DOTS) s_l[e] = ok ? s[m * G + g] : 0.0f;
            tn_l[e] = ok ? -t[m * G + g] : 0;
        }
        store_ws(wv[0], 0);
    }
    __syncthreads();

    const int arow = c < Mr ? c : Mr - 1;   // padded tokens read the last real row
    const int8_t *abase = panel + arow * RS + 16 * lg;

    // One group: planes of this lane's four code words (w), two MFMAs, epilogue.
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
                if (m < M && n < N) d[((int64_t)m * N + n) * G + g] = dd[i];
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
        const int64_t n0 = (int64_t)(bid + (int64_t)j * B) * 16;
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
                if (g + 1 < G) group(hi, g + 1, n0, wrow, acc);
            }
        }
        if (!DOTS) {
            float *pb = part + (j & 1) * (NW * kWave * 4);
            *reinterpret_cast<float4 *>(pb + (wave * kWave + lane) * 4) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    };

    auto reduce_tile = [&](int j) __attribute__((always_inline)) {
        if (!DOTS && tid < 256) {
            const int64_t n0 = (int64_t)(bid + (int64_t)j * B) * 16;
            const float *pb = part + (j & 1) * (NW * kWave * 4);
            // output (token m, row cc) sits in lane cc + 16 * (m / 4), slot m % 4
            const int m = tid >> 4, cc = tid & 15;
            const int at = (cc + 16 * (m >> 2)) * 4 + (m & 3);
            float v = pb[at];
#pragma unroll
            for (int w = 1; w < NW; ++w) v += pb[w * kWave * 4 + at];
            const int64_t n = n0 + cc;
            if (m < M && n < N) y[(int64_t)m * N + n] = v;
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

struct DevLimits {
    int cus = 0;
    int lds_block = 0;
    int lds_cu = 0;
};

// Compute units and LDS limits of the current device, read once per device.
const DevLimits &dev_limits() {
    static DevLimits cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        static DevLimits none;
        return none;
    }
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
                      const GemmOut &out, int64_t M, int64_t N, int64_t K, int64_t blocks,
                      size_t lds, hipStream_t stream) {
    if (out.d) {
        hipLaunchKernelGGL((small_panel_kernel<NW, GS, R, true>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, nullptr, t, codes, nullptr, nullptr,
                           out.d, M, N, K);
    } else {
        hipLaunchKernelGGL((small_panel_kernel<NW, GS, R, false>), dim3((unsigned)blocks),
                           dim3(NW * kWave), lds, stream, q, out.s, t, codes, out.ws, out.y,
                           nullptr, M, N, K);
    }
    return hipGetLastError();
}

// GS = ceil(pairs / NW) exactly: a wave's short slice costs at most one repeated load.
template <int NW, int R>
hipError_t launch_gs(int64_t gs, const int8_t *q, const int32_t *t, const uint8_t *codes,
                     const GemmOut &out, int64_t M, int64_t N, int64_t K, int64_t blocks,
                     size_t lds, hipStream_t stream) {
    switch (gs) {
        case 1: return launch_cfg<NW, 1, R>(q, t, codes, out, M, N, K, blocks, lds, stream);
        case 2: return launch_cfg<NW, 2, R>(q, t, codes, out, M, N, K, blocks, lds, stream);
        case 3: return launch_cfg<NW, 3, R>(q, t, codes, out, M, N, K, blocks, lds, stream);
        case 4: return launch_cfg<NW, 4, R>(q, t, codes, out, M, N, K, blocks, lds, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool small_panel_fits(int64_t M, int64_t K) {
    if (M < 1 || M > 16 || K > kPanelMaxK || K / kGroup < 16) return false;
    const DevLimits &l = dev_limits();
    return l.cus > 0 && panel_lds_bytes(M, K, 8) <= l.lds_block;
}

// One block of 8 waves per CU (two when two panels fit in a CU's LDS), at
// most one block per 16-row tile; each wave gets (G / 2) / 8 group pairs per
// tile (G >= 16 is required; K <= 8192 keeps that at most 4). Two tiles in
// flight per wave (R = 2): sweeps on MI355X found deeper rings, 16-wave
// blocks and two blocks per CU all slower on the 5120 / 6144 / 17408 shapes.
hipError_t launch_small_panel(const int8_t *q, const int32_t *t, const uint8_t *codes,
                              const GemmOut &out, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream) {
    constexpr int kNW = 8;
    const DevLimits &l = dev_limits();
    const int64_t Mr = M < 16 ? M : 16;
    const int64_t G = K / kGroup;
    const int64_t lds = panel_lds_bytes(Mr, K, kNW);
    if (l.cus <= 0 || lds > l.lds_block || (G + 1) / 2 < kNW) return hipErrorInvalidValue;
    int64_t blocks = l.cus * (l.lds_cu / lds >= 2 ? 2 : 1);
    PANEL_TUNE_OVERRIDE
    const int64_t NT = (N + 15) / 16;
    if (blocks > NT) blocks = NT;
    const int64_t gs = ((G + 1) / 2 + kNW - 1) / kNW;
    return launch_gs<kNW, 2>(gs, q, t, codes, out, M, N, K, blocks, lds, stream);
}

}  // namespace pq2
