// pq2_launch.hpp -- host-side launchers of the PQ2_0 kernels. Arguments are
// validated by the C ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pq2 {

// Epilogue of a GEMM launch: the float32 scale epilogue into y, or the exact
// int32 group dots into d (test and diagnostic path).
struct GemmOut {
    float *y;        // [M][N] or nullptr
    int32_t *d;      // [M][N][G] or nullptr
    const float *s;  // [M][G], unused when d is set
    const uint16_t *ws;  // [N][G], unused when d is set
    uint16_t *y16 = nullptr;  // bfloat16 [M][N] instead of y, when set
};

// Compute units of the current device (read once per device; 0 if unknown).
int device_cus();

// format 0: float32 x; 1: bfloat16; 2: IEEE binary16 (each widened exactly).
hipError_t launch_quantize(const void *x, int format, int8_t *q, float *s, int32_t *t,
                           int64_t M, int64_t K, hipStream_t stream);

// The dot4 GEMV runs 1 to kGemvMaxM token rows.
constexpr int64_t kGemvMaxM = 4;

hipError_t launch_gemv(const int8_t *q, const int32_t *t, const uint8_t *codes,
                       const GemmOut &out, int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Quantise + GEMV in one launch (M <= kGemvMaxM): y from float32 x.
hipError_t launch_gemv_fused(const float *x, const uint8_t *codes, const uint16_t *ws, float *y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);

// The small-batch kernel stages 3 * 16 * (G + 1) words of scales in LDS.
constexpr int64_t kSmallMaxK = 32768;

hipError_t launch_small(const int8_t *q, const int32_t *t, const uint8_t *codes,
                        const GemmOut &out, int64_t M, int64_t N, int64_t K,
                        hipStream_t stream);

// The persistent small-batch kernel keeps the M x K activation panel (or a
// K chunk of it) in LDS: K <= kPanelMaxK, K >= 16 * 128, M <= kPanelMaxM,
// and a split of K into at most kPanelMaxSplits chunks whose panel plus
// tables fit the device's LDS per block (small_panel_fits checks all of it).
// A split into S > 1 chunks writes S * M * N float32 partial sums to a
// caller-owned workspace, so every planner takes the largest chunk count
// the caller's workspace allows (max_splits >= 1; 1 = unsplit only).
constexpr int64_t kPanelMaxK = 18432;
constexpr int64_t kPanelMaxM = 64;
constexpr int kPanelMaxSplits = 16;

bool small_panel_fits(int64_t M, int64_t K, int max_splits);
// Whether the panel kernel runs its ring variant (A fragments resident in
// VGPRs, codes through an LDS ring): M <= 16 and K chunks of whole multiples
// of 8 groups within the LDS bound.
bool small_panel_ring_fits(int64_t M, int64_t K, int max_splits);
// K chunks of the plan launch_small_panel takes (0: none fits).
int small_panel_splits(int64_t M, int64_t N, int64_t K, int max_splits);

// work: device buffer of at least small_panel_splits(...) * M * N floats when
// that is above 1 and out.d is not set (the chunks' partial sums), else unused.
hipError_t launch_small_panel(const int8_t *q, const int32_t *t, const uint8_t *codes,
                              const GemmOut &out, int64_t M, int64_t N, int64_t K,
                              int max_splits, float *work, hipStream_t stream);

// Quantise + ring-variant panel kernel in one launch (plus the split sum when
// K is cut into chunks): y from float32 x, M <= 16, where the ring variant
// has a plan (small_panel_ring_fits). small_panel_fused_splits gives its K
// chunks (0: no plan); work holds that many M x N float32 partial sums when
// above 1.
int small_panel_fused_splits(int64_t M, int64_t N, int64_t K, int max_splits);
hipError_t launch_small_panel_fused(const float *x, const uint8_t *codes, const uint16_t *ws,
                                    float *y, int64_t M, int64_t N, int64_t K, int max_splits,
                                    float *work, hipStream_t stream);

// The allocation-free entry's split-K buffer: kScratchBytes of device memory
// per device (a file-scope array), its address on the current device looked
// up once per device (nullptr and *err set if the lookup fails).
constexpr size_t kScratchBytes = size_t(16) << 20;
float *scratch_address(hipError_t *err);

// y = sum over the chunks of part[c][M*N], added in chunk order.
hipError_t launch_split_sum(const float *part, float *y, uint16_t *y16, int64_t MN, int splits,
                            hipStream_t stream);

// Blocks the tiled prefill kernel launches for M x N (its tile rule).
int64_t prefill_blocks(int64_t M, int64_t N);

// Bytes of partial sums the prefill plan for M x N x K uses when it splits
// the K range of its last tiles (0: its plan does not split).
size_t prefill_workspace_bytes(int64_t M, int64_t N, int64_t K);

// work: device buffer of work_bytes (or nullptr); the plan splits its last
// tiles into as many K chunks as their partial sums fit there (with no room,
// or for group dots, nothing is split).
hipError_t launch_prefill(const int8_t *q, const int32_t *t, const uint8_t *codes,
                          const GemmOut &out, int64_t M, int64_t N, int64_t K, float *work,
                          size_t work_bytes, hipStream_t stream);

}  // namespace pq2
