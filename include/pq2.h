/*
 * pq2.h -- C ABI of the PQ2_0 ternary-weight x int8-activation GEMM for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "Making a ternary reasoning model fast in vLLM -- from
 * CUDA to Triton and Gluon", section "One token at a time: plain Triton is
 * enough"; per-call buffers from section "Prompt processing: check
 * configuration and launch costs"):
 *
 *   x float32 [M][K]  --pq2_quantize_act-->  q int8 [M][K] (plane order),
 *                                            s float32 [M][G], t int32 [M][G]
 *   q, s, t + codes + wscale  --pq2_gemm-->  y float32 [M][N]
 *
 *   y[m][n] = sum_g  s[m][g] * wscale[n][g] * D[m][n][g]
 *   D[m][n][g] = sum_{k in group g} code[n][k] * q[m][k]  -  t[m][g]
 *              = sum_{k in group g} (code[n][k] - 1) * q[m][k]
 *
 * G = K / 128. All arrays are dense and row-major, in device memory, owned
 * by the caller, and so is the optional split-K workspace (see pq2_gemm).
 * Every call only enqueues kernels on the given stream (NULL = the null
 * stream); the library never allocates, frees or synchronises and keeps no
 * mutable state (a per-device cache of device limits is filled once, under a
 * lock, and only read after that), so calls are thread-safe and may be
 * captured in HIP graphs. Inputs must not overlap outputs or the workspace.
 *
 * LAYOUTS (fixed):
 *  codes   uint8 [N][K/4]. The 2-bit code of weight k of row n (code c means
 *          the weight c-1; codes are 0, 1, 2) sits in byte n*K/4 + k/4 at
 *          bits 2*(k%4) .. 2*(k%4)+1. Viewed as little-endian 32-bit words,
 *          group g of a row is words 8g .. 8g+7. Base 16-byte aligned.
 *  wscale  IEEE binary16 bit patterns [N][G], one scale per (row, group).
 *          Base 2-byte aligned.
 *  x       float32 [M][K]. Base 16-byte aligned.
 *  q       int8 [M][K] in plane order: inside group g (bytes 128g..128g+127
 *          of a row), the activation of weight 4*b+s (b = 0..31, s = 0..3)
 *          is stored at byte 128g + 32*s + b. Base 16-byte aligned.
 *  s       float32 [M][G]; t int32 [M][G]. Base 4-byte aligned.
 *  y       float32 [M][N], overwritten. Base 4-byte aligned.
 *
 * ERRORS: arguments are validated on the host before anything is enqueued:
 *  PQ2_ERR_NULL  a required pointer is NULL;
 *  PQ2_ERR_SHAPE M < 1, N < 1, K < 128, K % 128 != 0, M or N above
 *                PQ2_MAX_DIM, K above PQ2_MAX_K (the kernels address a
 *                block's rows with 32-bit offsets), or M*N, M*K or N*K/4
 *                above PQ2_MAX_ELEMS (larger than any device memory; keeps
 *                every launch grid below 2^31 blocks);
 *  PQ2_ERR_ALIGN a base pointer breaks the alignment stated above (a
 *                workspace, when given, must be 16-byte aligned);
 *  PQ2_ERR_ARG   an invalid path selector (pq2_gemm_group_dots), a shape
 *                and workspace no fused kernel of pq2_linear runs, or an
 *                unknown activation format (pq2_quantize_act_16);
 *  PQ2_ERR_SCRATCH (pq2_gemm_noalloc) the small-batch plan's split-K partial
 *                sums need more than PQ2_NOALLOC_SCRATCH_BYTES;
 *  PQ2_ERR_HIP   a kernel launch was rejected by the HIP runtime.
 * Nothing is enqueued when a status other than PQ2_OK is returned, except for
 * PQ2_ERR_HIP. A fault during execution surfaces at the caller's next
 * synchronisation, as for any HIP kernel. No C++ exception crosses the ABI.
 */
#ifndef PQ2_H
#define PQ2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQ2_ABI_VERSION 3
#define PQ2_GROUP 128
#define PQ2_MAX_DIM (1LL << 30)
#define PQ2_MAX_K (1LL << 24)
#define PQ2_MAX_ELEMS (1LL << 40)

typedef enum {
    PQ2_OK = 0,
    PQ2_ERR_NULL = 1,
    PQ2_ERR_SHAPE = 2,
    PQ2_ERR_ALIGN = 3,
    PQ2_ERR_HIP = 4,
    PQ2_ERR_ARG = 5,
    PQ2_ERR_SCRATCH = 6
} pq2_status;

/* Kernel path selectors for pq2_gemm_group_dots. */
enum {
    PQ2_PATH_AUTO = 0,      /* pq2_gemm's choice for the given workspace */
    PQ2_PATH_GEMV = 1,      /* M <= 4 only: the v_dot4 GEMV */
    PQ2_PATH_SMALL = 2,     /* M <= 16, K <= 32768: the small-batch MFMA kernel */
    PQ2_PATH_PREFILL = 3,   /* any M: the tiled MFMA GEMM */
    PQ2_PATH_PANEL = 4      /* M <= 64, 2048 <= K <= 18432: the persistent
                               small-batch MFMA kernel (activation panel in LDS) */
};

/* Returns PQ2_ABI_VERSION of the loaded library. */
int pq2_abi_version(void);

/* Static, human-readable name of a status code. Never NULL. */
const char *pq2_status_str(int status);

/*
 * Per-128-group int8 quantisation of activations, fused with the plane-order
 * permutation (page "Making a ternary reasoning model fast in vLLM -- from
 * CUDA to Triton and Gluon": section "One token at a time" for the layout,
 * section "Prompt processing" for the q/s/t buffers). For each row m and group g:
 *   amax = max |x|;  s = amax / 127 (float32, correctly rounded division);
 *   q = clamp(round_half_even(x / s), -127, 127) (float32 division);
 *   t = sum of the group's q.   A group with s == 0 gets q = 0, t = 0.
 * x must be finite. Writes q (plane order), s and t.
 */
pq2_status pq2_quantize_act(const float *x, int8_t *q, float *s, int32_t *t,
                            int64_t M, int64_t K, void *hip_stream);

/*
 * pq2_quantize_act for 16-bit activations, as a model running in bfloat16 or
 * float16 holds them (the pages' projections take the activation dtype; see
 * the page "Making a ternary reasoning model fast in vLLM", section "Prompt
 * processing: check configuration and launch costs", for the quantiser's
 * place in the step). Every element is first widened exactly to float32
 * (bfloat16: its bits are the upper half of the float32's; binary16: the IEEE
 * conversion, subnormals included), then quantised by the rule above, so q,
 * s and t are those pq2_quantize_act gives for the widened x.
 *   x_format  PQ2_ACT_BF16 or PQ2_ACT_F16 (else PQ2_ERR_ARG);
 *   x         uint16 bit patterns [M][K], 8-byte aligned; q, s, t as above.
 */
#define PQ2_ACT_BF16 1
#define PQ2_ACT_F16 2
pq2_status pq2_quantize_act_16(const uint16_t *x, int x_format, int8_t *q, float *s, int32_t *t,
                               int64_t M, int64_t K, void *hip_stream);

/*
 * Device workspace, in bytes, that pq2_gemm (and pq2_gemm_bf16) needs to run
 * its fastest plan for this shape: the persistent small-batch kernel splits
 * K into S chunks for some shapes (K = 17408 at 3..16 token rows: S = 3;
 * 17..64 rows: most K) and writes S * M * N float32 partial sums, which a
 * second small launch adds in chunk order; the tiled prefill GEMM splits the
 * K range of its leftover 256 x 128 tiles (M = 4096, K = 5120, N = 17408 or
 * 5120: 128 tiles x 4 chunks, 64 MiB). 0 when the plan does not split K, or
 * when the shape is invalid. Pure host query; enqueues nothing. (The
 * page "Making a ternary reasoning model fast in vLLM", section "Measure at
 * the clock speeds used in serving", counts the split-K reduction launches;
 * its section "Speed up a small unquantised projection" sums splits in a
 * fixed order and rounds once.)
 */
size_t pq2_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * y = the PQ2_0 product defined above. The kernel depends on M:
 *   M <= 2        -> GEMV streaming code words into v_dot4 (2-bit planes
 *                    masked out of each 32-bit word, no decode step; each
 *                    word serves every token row);
 *   3 <= M <= 16  -> persistent small-batch kernel on int8 MFMA
 *                    (PQ2_PATH_PANEL) whenever 2048 <= K <= 18432 and G is
 *                    a multiple of 8 (its activation fragments stay in
 *                    registers, code tiles stream through LDS); for other G
 *                    runs it when N*K > 2^25 or M >= 8 and the activation panel
 *                    fits LDS (the bound below); else the GEMV for M <= 4
 *                    with N*K > 2^25; else the 16-token MFMA kernel
 *                    (K <= 32768);
 *   17 <= M <= 64 -> the same persistent kernel in 2 or 4 token tiles where
 *                    the panel fits and the tiled GEMM below would launch
 *                    fewer than 512 blocks (2 per CU);
 *   otherwise     -> tiled int8 MFMA GEMM (prefill).
 * pq2_gemm_kernel_path reports the choice.
 * Group dots are exact int32; the float32 epilogue sums the G terms in an
 * order that differs from a sequential sum only by float32 rounding (a fixed
 * order: repeated calls give identical y).
 * Workspace: a caller-owned device buffer of workspace_bytes bytes, 16-byte
 * aligned, or NULL, that holds float32 partial sums of plans splitting K.
 * The persistent small-batch kernel splits K into S chunks only when
 * S * M * N * 4 <= workspace_bytes (the largest chunk count that fits, at
 * most 16). The tiled prefill GEMM, on its 256 x 128 tile, splits the K range
 * of the tiles left over after whole rounds of two blocks per CU into up to
 * 4 chunks, each chunk's partial tile (128 x 256 float32) in the workspace,
 * and takes as many chunks as fit. pq2_gemm_workspace_bytes gives the size
 * of the fastest plan. With NULL, or a buffer too small for any split,
 * pq2_gemm takes a plan that does not split K (same result up to float32
 * summation order; slower on some shapes, e.g. K = 17408 at 3..16 rows). The workspace's contents
 * before and after a call are unspecified; calls that may run concurrently
 * (different streams) need different workspaces, calls on one stream may
 * share one.
 */
pq2_status pq2_gemm(const int8_t *q, const float *s, const int32_t *t,
                    const uint8_t *codes, const uint16_t *wscale, float *y,
                    int64_t M, int64_t N, int64_t K,
                    void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * pq2_gemm for callers that cannot allocate device memory or hold a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments as pq2_gemm without the workspace,
 * same plan as pq2_gemm given min(pq2_gemm_workspace_bytes(M, N, K),
 * PQ2_NOALLOC_SCRATCH_BYTES) bytes of workspace, so y is bit-identical to
 * that call. The split-K partial sums go to a buffer of
 * PQ2_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one per
 * device (part of the loaded library, alive until the process ends); its
 * address is looked up on the first call on each device. Prefill shapes
 * split only as far as their partial tiles fit that buffer (or not at all);
 * small-batch shapes whose pq2_gemm_workspace_bytes exceeds
 * PQ2_NOALLOC_SCRATCH_BYTES return PQ2_ERR_SCRATCH (nothing enqueued). Nothing is allocated or freed. Every
 * call on a device shares that device's buffer: calls that may overlap on one
 * device (different streams, or host threads) race on it and must be
 * serialised by the caller; calls on one stream are ordered and safe. The
 * buffer needs no clearing (every call writes all partial sums it reads).
 */
#define PQ2_NOALLOC_SCRATCH_BYTES (16u << 20)
pq2_status pq2_gemm_noalloc(const int8_t *q, const float *s, const int32_t *t,
                            const uint8_t *codes, const uint16_t *wscale, float *y,
                            int64_t M, int64_t N, int64_t K, void *hip_stream);

/*
 * pq2_gemm with a bfloat16 output, for callers whose activations are bfloat16
 * (the pages' projections return the activation dtype; page "Making a ternary
 * reasoning model fast in vLLM", section "One token at a time: plain Triton
 * is enough"): the same kernels and the same float32 accumulation as
 * pq2_gemm, each output rounded to nearest-even bfloat16 at its final store
 * (split-K partial sums stay float32 until the summing launch), so y is
 * exactly pq2_gemm's y rounded to bfloat16.
 *   y  bfloat16 bit patterns [M][N], 2-byte aligned, overwritten.
 * Everything else, the workspace included, as for pq2_gemm.
 */
pq2_status pq2_gemm_bf16(const int8_t *q, const float *s, const int32_t *t,
                         const uint8_t *codes, const uint16_t *wscale, uint16_t *y,
                         int64_t M, int64_t N, int64_t K,
                         void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Quantise and multiply without the separate quantiser launch, for decode
 * batches of 1 to 16 token rows (PQ2_LINEAR_MAX_M): y = the PQ2_0 product of
 * x quantised exactly as pq2_quantize_act would (page "Making a ternary
 * reasoning model fast in vLLM", section "Prompt processing: check
 * configuration and launch costs", counts a quantiser launch per projection;
 * section "Choose the configuration with the proxy" charges its time to the
 * matmul). The GEMM kernel quantises the activations it needs itself, with
 * the quantiser's arithmetic, so q, s and t -- never written anywhere -- are
 * bit for bit those of pq2_quantize_act, and y is bit-identical to
 * pq2_quantize_act followed by pq2_gemm on the same kernel path:
 *   M = 1, 2 (and 3, 4 where the panel kernel below has no plan): the v_dot4
 *     GEMV; every block quantises the whole activation row into LDS.
 *   M = 3 .. 16 with K a multiple of 1024 in [2048, 18432]: the persistent
 *     panel kernel (PQ2_PATH_PANEL, its ring variant), each wave quantising
 *     its own groups of every token in registers. Its K chunks and their
 *     split sum are those of pq2_gemm: K up to 6144 runs in one launch, a
 *     longer K in chunks whose partial sums go to the workspace (then a
 *     second, summing launch).
 * Every compute unit quantises the activations it consumes, so the work of
 * the quantiser is repeated once per unit: on MI355X this pays at one token
 * row (decode 5120 x 6144: 5.07 against 6.57 us for the two launches) and
 * at two rows of that shape (7.21 against 7.53 us); on the larger shapes
 * and from four rows on it costs more than the launch it saves (see the
 * bench's fused_step_us).
 *   x  float32 [M][K], 16-byte aligned; codes, wscale, y as for pq2_gemm.
 *   workspace, workspace_bytes  as for pq2_gemm, sized by
 *      pq2_linear_workspace_bytes (0 for M <= 2 and for K <= 6144).
 * PQ2_ERR_ARG when M > PQ2_LINEAR_MAX_M, or when 5 <= M <= 16 and no panel
 * plan runs this K with this workspace (use pq2_quantize_act and pq2_gemm).
 */
#define PQ2_LINEAR_MAX_M 16
pq2_status pq2_linear(const float *x, const uint8_t *codes, const uint16_t *wscale, float *y,
                      int64_t M, int64_t N, int64_t K, void *workspace, size_t workspace_bytes,
                      void *hip_stream);

/*
 * Bytes of split-K partial sums pq2_linear's plan for this shape writes to
 * its workspace (0: the plan needs none). Pure host query; 0 for invalid
 * shapes and M above PQ2_LINEAR_MAX_M.
 */
size_t pq2_linear_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * The kernel path pq2_linear takes for this shape given a workspace of
 * workspace_bytes bytes: PQ2_PATH_GEMV or PQ2_PATH_PANEL, whose pq2_gemm_path
 * result (same workspace) its y equals bit for bit, or -1 where it returns
 * PQ2_ERR_SHAPE or PQ2_ERR_ARG. Pure host query; enqueues nothing.
 */
int pq2_linear_kernel_path(int64_t M, int64_t N, int64_t K, size_t workspace_bytes);

/*
 * The PQ2_PATH_* kernel path pq2_gemm takes for this shape on the current
 * device when given a workspace of workspace_bytes bytes (0: none), or -1
 * when pq2_gemm would reject the shape (PQ2_ERR_SHAPE). Pure host query;
 * enqueues nothing.
 */
int pq2_gemm_kernel_path(int64_t M, int64_t N, int64_t K, size_t workspace_bytes);

/*
 * Test and tuning entry: pq2_gemm through the selected kernel path instead of
 * pq2_gemm's own choice. Arguments, layouts, workspace and results as for
 * pq2_gemm; path is one of PQ2_PATH_* with the limits listed for
 * pq2_gemm_group_dots, where the panel kernel's K chunks are limited by the
 * workspace as in pq2_gemm (PQ2_ERR_ARG when no plan runs).
 */
pq2_status pq2_gemm_path(const int8_t *q, const float *s, const int32_t *t,
                         const uint8_t *codes, const uint16_t *wscale, float *y,
                         int64_t M, int64_t N, int64_t K, int path,
                         void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Test and diagnostic entry: runs the main loop of the selected kernel path
 * but stores the exact per-group dots instead of the float epilogue:
 *   d int32 [M][N][G],  d[m][n][g] = D[m][n][g] as defined above.
 * Every K chunk writes its own groups of d, so no workspace is involved:
 * PQ2_PATH_AUTO is pq2_gemm's choice with a workspace of
 * pq2_gemm_workspace_bytes(M, N, K) bytes.
 * path is one of PQ2_PATH_*; PQ2_PATH_GEMV requires M <= 4,
 * PQ2_PATH_SMALL requires M <= 16 and K <= 32768, PQ2_PATH_PANEL requires
 * M <= 64, 2048 <= K <= 18432 and a device whose LDS per block holds the
 * activation panel of one K chunk and its tables. Chunks are whole multiples
 * of 8 groups, at most 16 of them; an unsplit K (any G >= 16) needs, on
 * MI355X (160 KiB), M * (K + 16) + 320 * K / 128 + 16512 bytes for M <= 16.
 * Else PQ2_ERR_ARG.
 */
pq2_status pq2_gemm_group_dots(const int8_t *q, const int32_t *t,
                               const uint8_t *codes, int32_t *d,
                               int64_t M, int64_t N, int64_t K,
                               int path, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ2_H */
