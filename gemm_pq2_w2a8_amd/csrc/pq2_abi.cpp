// pq2_abi.cpp -- the C ABI declared in include/pq2.h: host-side argument
// validation and dispatch to the gfx950 kernels. Validation happens before
// anything is enqueued; the library allocates nothing and keeps no mutable
// state (the device-limit cache of the panel planner is written once per
// device and read-only after that).
#include "../../include/pq2.h"

#include <hip/hip_runtime.h>

#include "pq2_launch.hpp"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

pq2_status check_mnk(int64_t M, int64_t N, int64_t K) {
    if (M < 1 || N < 1 || K < PQ2_GROUP || K % PQ2_GROUP != 0) return PQ2_ERR_SHAPE;
    if (M > PQ2_MAX_DIM || N > PQ2_MAX_DIM || K > PQ2_MAX_K) return PQ2_ERR_SHAPE;
    // no buffer beyond 2^40 elements (every grid then stays below 2^31 blocks)
    if (M * N > PQ2_MAX_ELEMS || M * K > PQ2_MAX_ELEMS || N * (K / 4) > PQ2_MAX_ELEMS)
        return PQ2_ERR_SHAPE;
    return PQ2_OK;
}

pq2_status from_hip(hipError_t e) { return e == hipSuccess ? PQ2_OK : PQ2_ERR_HIP; }

// K chunks the caller's workspace allows the panel kernel: S chunks need
// S * M * N float32 partial sums; no workspace means unsplit plans only.
int splits_for_bytes(size_t work_bytes, int64_t M, int64_t N) {
    const uint64_t per = (uint64_t)M * (uint64_t)N * sizeof(float);
    const uint64_t s = work_bytes / per;
    return s < 1 ? 1 : s > (uint64_t)pq2::kPanelMaxSplits ? pq2::kPanelMaxSplits : (int)s;
}

int max_splits(const void *work, size_t work_bytes, int64_t M, int64_t N) {
    return work ? splits_for_bytes(work_bytes, M, N) : 1;
}

// work / work_bytes: the caller's workspace (nullptr / 0 when none); max_s:
// the K chunks of M x N partial sums it holds for the panel kernel.
pq2_status run_path(int path, const int8_t *q, const int32_t *t, const uint8_t *codes,
                    const pq2::GemmOut &out, int64_t M, int64_t N, int64_t K, int max_s,
                    float *work, size_t work_bytes, hipStream_t stream) {
    switch (path) {
        case PQ2_PATH_GEMV:
            return from_hip(pq2::launch_gemv(q, t, codes, out, M, N, K, stream));
        case PQ2_PATH_SMALL:
            return from_hip(pq2::launch_small(q, t, codes, out, M, N, K, stream));
        case PQ2_PATH_PREFILL:
            return from_hip(pq2::launch_prefill(q, t, codes, out, M, N, K, work,
                                                work ? work_bytes : 0, stream));
        case PQ2_PATH_PANEL:
            return from_hip(pq2::launch_small_panel(q, t, codes, out, M, N, K, max_s, work,
                                                    stream));
        default:
            return PQ2_ERR_ARG;
    }
}

// Kernel choice of pq2_gemm (from MI355X measurements on the decode and
// small-batch shapes): the dot4 GEMV reads only the real token rows and wins
// for M <= 2 everywhere. For 3 <= M <= 16 the panel kernel's ring variant
// (K chunks of whole multiples of 8 groups) beats the GEMV and the 16-token
// kernel on every shape measured (5120 x 6144 at M = 3: 7.0 us against 8.4);
// where only its other variants run it wins on large matrices (N*K > 2^25)
// and, from M = 8, on every size it can hold (K from 2048 to 18432, within
// LDS); otherwise the dot4 GEMV for M = 3..4 on large matrices with K too
// large for the panel, else the 16-token MFMA kernel. For 17 <= M <= 64 the
// panel kernel in 2 or 4 token tiles wins where the tiled GEMM has fewer than
// two blocks per CU (5120 x 6144 at M = 32: 12.9 us against 16.4; 5120 x
// 17408: 23.0 against 46.1); with more the tiled GEMM wins (17408 x 5120 at
// M = 32: 21.0 against 24.5). Plans that split K count only where the
// caller's workspace holds their partial sums (max_s chunks).
int auto_path(int64_t M, int64_t N, int64_t K, int max_s) {
    if (M <= 2) return PQ2_PATH_GEMV;
    if (M <= 16 && pq2::small_panel_ring_fits(M, K, max_s)) return PQ2_PATH_PANEL;
    const bool large = N * K > (int64_t(1) << 25);
    if (M <= 16 && (large || M >= 8) && pq2::small_panel_fits(M, K, max_s)) return PQ2_PATH_PANEL;
    if (M <= pq2::kGemvMaxM && large) return PQ2_PATH_GEMV;
    if (M <= 16 && K <= pq2::kSmallMaxK) return PQ2_PATH_SMALL;
    if (M <= pq2::kPanelMaxM && pq2::prefill_blocks(M, N) < 512 &&
        pq2::small_panel_fits(M, K, max_s))
        return PQ2_PATH_PANEL;
    return PQ2_PATH_PREFILL;
}

// Resolves PQ2_PATH_AUTO and rejects a path that cannot run this shape.
pq2_status resolve_path(int &path, int64_t M, int64_t N, int64_t K, int max_s) {
    if (path == PQ2_PATH_AUTO) path = auto_path(M, N, K, max_s);
    if (path == PQ2_PATH_GEMV && M > pq2::kGemvMaxM) return PQ2_ERR_ARG;
    if (path == PQ2_PATH_SMALL && (M > 16 || K > pq2::kSmallMaxK)) return PQ2_ERR_ARG;
    if (path == PQ2_PATH_PANEL && !pq2::small_panel_fits(M, K, max_s)) return PQ2_ERR_ARG;
    if (path < PQ2_PATH_GEMV || path > PQ2_PATH_PANEL) return PQ2_ERR_ARG;
    return PQ2_OK;
}

// Bytes of partial sums pq2_gemm's plan for this shape writes when the
// workspace is large enough (0: its plan does not split K).
size_t workspace_need(int64_t M, int64_t N, int64_t K) {
    const int path = auto_path(M, N, K, pq2::kPanelMaxSplits);
    if (path == PQ2_PATH_PREFILL) return pq2::prefill_workspace_bytes(M, N, K);
    if (path != PQ2_PATH_PANEL) return 0;
    const int S = pq2::small_panel_splits(M, N, K, pq2::kPanelMaxSplits);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

// Checks shared by the GEMM entries (y: float32 needs 4-byte, bfloat16
// 2-byte alignment; the workspace 16 bytes when given).
pq2_status check_gemm(const int8_t *q, const float *s, const int32_t *t, const uint8_t *codes,
                      const uint16_t *wscale, const void *y, uintptr_t y_align, const void *work,
                      int64_t M, int64_t N, int64_t K) {
    if (!q || !s || !t || !codes || !wscale || !y) return PQ2_ERR_NULL;
    pq2_status st = check_mnk(M, N, K);
    if (st != PQ2_OK) return st;
    if (!aligned(q, 16) || !aligned(codes, 16) || !aligned(s, 4) || !aligned(t, 4) ||
        !aligned(wscale, 2) || !aligned(y, y_align) || (work && !aligned(work, 16)))
        return PQ2_ERR_ALIGN;
    return PQ2_OK;
}

// Kernel of pq2_linear: the fused dot4 GEMV for one or two token rows (it
// reads only the real rows) and, without a ring plan, for three or four;
// the fused ring variant of the panel kernel for 3 to 16 rows where it has
// a plan with the K chunks the workspace holds (max_s); 0: no fused kernel.
enum LinearKernel { kLinearNone = 0, kLinearGemv = 1, kLinearRing = 2 };

LinearKernel linear_kernel(int64_t M, int64_t N, int64_t K, int max_s) {
    if (M <= 2) return kLinearGemv;
    if (M <= PQ2_LINEAR_MAX_M && pq2::small_panel_fused_splits(M, N, K, max_s) > 0)
        return kLinearRing;
    if (M <= pq2::kGemvMaxM) return kLinearGemv;
    return kLinearNone;
}

}  // namespace

extern "C" {

int pq2_abi_version(void) { return PQ2_ABI_VERSION; }

const char *pq2_status_str(int status) {
    switch (status) {
        case PQ2_OK: return "PQ2_OK";
        case PQ2_ERR_NULL: return "PQ2_ERR_NULL: a required pointer is NULL";
        case PQ2_ERR_SHAPE: return "PQ2_ERR_SHAPE: need M >= 1, N >= 1, K a positive multiple of 128, K <= 2^24";
        case PQ2_ERR_ALIGN: return "PQ2_ERR_ALIGN: a base pointer is misaligned";
        case PQ2_ERR_HIP: return "PQ2_ERR_HIP: the HIP runtime rejected a launch";
        case PQ2_ERR_ARG: return "PQ2_ERR_ARG: invalid path selector for this shape and workspace, no fused kernel of pq2_linear for this shape and workspace, or unknown activation format";
        case PQ2_ERR_SCRATCH: return "PQ2_ERR_SCRATCH: the shape needs more split-K scratch than pq2_gemm_noalloc holds (PQ2_NOALLOC_SCRATCH_BYTES)";
        default: return "PQ2 unknown status";
    }
}

pq2_status pq2_quantize_act(const float *x, int8_t *q, float *s, int32_t *t, int64_t M,
                            int64_t K, void *hip_stream) {
    if (!x || !q || !s || !t) return PQ2_ERR_NULL;
    pq2_status st = check_mnk(M, 1, K);
    if (st != PQ2_OK) return st;
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4) || !aligned(t, 4))
        return PQ2_ERR_ALIGN;
    return from_hip(pq2::launch_quantize(x, 0, q, s, t, M, K, static_cast<hipStream_t>(hip_stream)));
}

pq2_status pq2_quantize_act_16(const uint16_t *x, int x_format, int8_t *q, float *s, int32_t *t,
                               int64_t M, int64_t K, void *hip_stream) {
    if (!x || !q || !s || !t) return PQ2_ERR_NULL;
    pq2_status st = check_mnk(M, 1, K);
    if (st != PQ2_OK) return st;
    if (!aligned(x, 8) || !aligned(q, 16) || !aligned(s, 4) || !aligned(t, 4))
        return PQ2_ERR_ALIGN;
    if (x_format != PQ2_ACT_BF16 && x_format != PQ2_ACT_F16) return PQ2_ERR_ARG;
    return from_hip(pq2::launch_quantize(x, x_format, q, s, t, M, K,
                                         static_cast<hipStream_t>(hip_stream)));
}

size_t pq2_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_mnk(M, N, K) != PQ2_OK) return 0;
    return workspace_need(M, N, K);
}

pq2_status pq2_gemm(const int8_t *q, const float *s, const int32_t *t, const uint8_t *codes,
                    const uint16_t *wscale, float *y, int64_t M, int64_t N, int64_t K,
                    void *workspace, size_t workspace_bytes, void *hip_stream) {
    pq2_status st = check_gemm(q, s, t, codes, wscale, y, 4, workspace, M, N, K);
    if (st != PQ2_OK) return st;
    const int max_s = max_splits(workspace, workspace_bytes, M, N);
    const pq2::GemmOut out{y, nullptr, s, wscale};
    return run_path(auto_path(M, N, K, max_s), q, t, codes, out, M, N, K, max_s,
                    static_cast<float *>(workspace), workspace_bytes,
                    static_cast<hipStream_t>(hip_stream));
}

pq2_status pq2_gemm_bf16(const int8_t *q, const float *s, const int32_t *t, const uint8_t *codes,
                         const uint16_t *wscale, uint16_t *y, int64_t M, int64_t N, int64_t K,
                         void *workspace, size_t workspace_bytes, void *hip_stream) {
    pq2_status st = check_gemm(q, s, t, codes, wscale, y, 2, workspace, M, N, K);
    if (st != PQ2_OK) return st;
    const int max_s = max_splits(workspace, workspace_bytes, M, N);
    pq2::GemmOut out{nullptr, nullptr, s, wscale};
    out.y16 = y;
    return run_path(auto_path(M, N, K, max_s), q, t, codes, out, M, N, K, max_s,
                    static_cast<float *>(workspace), workspace_bytes,
                    static_cast<hipStream_t>(hip_stream));
}

pq2_status pq2_gemm_noalloc(const int8_t *q, const float *s, const int32_t *t,
                            const uint8_t *codes, const uint16_t *wscale, float *y, int64_t M,
                            int64_t N, int64_t K, void *hip_stream) {
    static_assert(PQ2_NOALLOC_SCRATCH_BYTES == pq2::kScratchBytes, "scratch size in the header");
    pq2_status st = check_gemm(q, s, t, codes, wscale, y, 4, nullptr, M, N, K);
    if (st != PQ2_OK) return st;
    // The prefill plan splits only as far as its partial sums fit the scratch
    // array (down to no split); a panel plan that needs more is refused.
    const bool prefill = auto_path(M, N, K, pq2::kPanelMaxSplits) == PQ2_PATH_PREFILL;
    size_t need = workspace_need(M, N, K);
    if (prefill && need > pq2::kScratchBytes) need = pq2::kScratchBytes;
    if (need > pq2::kScratchBytes) return PQ2_ERR_SCRATCH;
    float *work = nullptr;
    if (need > 0) {
        hipError_t e = hipSuccess;
        work = pq2::scratch_address(&e);
        if (!work) return PQ2_ERR_HIP;
    }
    // the same plan pq2_gemm takes with a workspace of exactly `need` bytes
    const int max_s = need > 0 ? splits_for_bytes(need, M, N) : 1;
    const pq2::GemmOut out{y, nullptr, s, wscale};
    return run_path(auto_path(M, N, K, max_s), q, t, codes, out, M, N, K, max_s, work, need,
                    static_cast<hipStream_t>(hip_stream));
}

int pq2_gemm_kernel_path(int64_t M, int64_t N, int64_t K, size_t workspace_bytes) {
    if (check_mnk(M, N, K) != PQ2_OK) return -1;
    return auto_path(M, N, K, splits_for_bytes(workspace_bytes, M, N));
}

pq2_status pq2_gemm_path(const int8_t *q, const float *s, const int32_t *t, const uint8_t *codes,
                         const uint16_t *wscale, float *y, int64_t M, int64_t N, int64_t K,
                         int path, void *workspace, size_t workspace_bytes, void *hip_stream) {
    pq2_status st = check_gemm(q, s, t, codes, wscale, y, 4, workspace, M, N, K);
    if (st != PQ2_OK) return st;
    const int max_s = max_splits(workspace, workspace_bytes, M, N);
    st = resolve_path(path, M, N, K, max_s);
    if (st != PQ2_OK) return st;
    const pq2::GemmOut out{y, nullptr, s, wscale};
    return run_path(path, q, t, codes, out, M, N, K, max_s, static_cast<float *>(workspace),
                    workspace_bytes, static_cast<hipStream_t>(hip_stream));
}

size_t pq2_linear_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (check_mnk(M, N, K) != PQ2_OK || M > PQ2_LINEAR_MAX_M) return 0;
    if (linear_kernel(M, N, K, pq2::kPanelMaxSplits) != kLinearRing) return 0;
    const int S = pq2::small_panel_fused_splits(M, N, K, pq2::kPanelMaxSplits);
    return S > 1 ? (size_t)S * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int pq2_linear_kernel_path(int64_t M, int64_t N, int64_t K, size_t workspace_bytes) {
    if (check_mnk(M, N, K) != PQ2_OK || M > PQ2_LINEAR_MAX_M) return -1;
    switch (linear_kernel(M, N, K, splits_for_bytes(workspace_bytes, M, N))) {
        case kLinearGemv: return PQ2_PATH_GEMV;
        case kLinearRing: return PQ2_PATH_PANEL;
        default: return -1;
    }
}

pq2_status pq2_linear(const float *x, const uint8_t *codes, const uint16_t *wscale, float *y,
                      int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                      void *hip_stream) {
    if (!x || !codes || !wscale || !y) return PQ2_ERR_NULL;
    pq2_status st = check_mnk(M, N, K);
    if (st != PQ2_OK) return st;
    if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(wscale, 2) || !aligned(y, 4) ||
        (workspace && !aligned(workspace, 16)))
        return PQ2_ERR_ALIGN;
    if (M > PQ2_LINEAR_MAX_M) return PQ2_ERR_ARG;
    const int max_s = max_splits(workspace, workspace_bytes, M, N);
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    switch (linear_kernel(M, N, K, max_s)) {
        case kLinearGemv:
            return from_hip(pq2::launch_gemv_fused(x, codes, wscale, y, M, N, K, stream));
        case kLinearRing:
            return from_hip(pq2::launch_small_panel_fused(x, codes, wscale, y, M, N, K, max_s,
                                                          static_cast<float *>(workspace),
                                                          stream));
        default:
            return PQ2_ERR_ARG;
    }
}

pq2_status pq2_gemm_group_dots(const int8_t *q, const int32_t *t, const uint8_t *codes,
                               int32_t *d, int64_t M, int64_t N, int64_t K, int path,
                               void *hip_stream) {
    if (!q || !t || !codes || !d) return PQ2_ERR_NULL;
    pq2_status st = check_mnk(M, N, K);
    if (st != PQ2_OK) return st;
    if (!aligned(q, 16) || !aligned(codes, 16) || !aligned(t, 4) || !aligned(d, 4))
        return PQ2_ERR_ALIGN;
    // the exact dots of each K chunk go straight to d: no workspace needed,
    // so every chunk count is open to the planner
    st = resolve_path(path, M, N, K, pq2::kPanelMaxSplits);
    if (st != PQ2_OK) return st;
    const pq2::GemmOut out{nullptr, d, nullptr, nullptr};
    return run_path(path, q, t, codes, out, M, N, K, pq2::kPanelMaxSplits, nullptr, 0,
                    static_cast<hipStream_t>(hip_stream));
}

}  // extern "C"
