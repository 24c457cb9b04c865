/*
 * dense_gemm.h — C ABI of the gfx950 (MI355X) dense GEMM library.
 *
 * Operation (the general GEMM of "GEMM on NVIDIA GPUs: from a naive kernel to
 * a tiled pipeline", section 1):
 *
 *     D = alpha * op(A) * op(B) + beta * C
 *     D_ij = alpha * sum_{k=0}^{K-1} op(A)_ik op(B)_kj + beta * C_ij
 *
 * with op(X) = X or X^T, op(A) of size M x K, op(B) of size K x N, C and D of
 * size M x N.  Throughput is counted as 2*M*N*K floating-point operations
 * (alpha/beta work excluded, as in that section).
 *
 * Precisions (input / accumulate / output, the triple named in its section 5):
 *   GEMM_DTYPE_F32       : A, B fp32 / fp32 / C, D fp32
 *   GEMM_DTYPE_BF16_F32  : A, B bfloat16 (raw 16-bit patterns) / fp32 / C, D fp32
 *   GEMM_DTYPE_BF16_BF16 : A, B bfloat16 / fp32 / C, D bfloat16 — the section's
 *                          example triple; alpha*acc + beta*C is formed in fp32
 *                          and rounded once to bfloat16 (nearest even).  Needs
 *                          element-aligned operands whose panels the
 *                          direct-to-LDS kernels can address (every leading
 *                          dimension below 2^31 / 256 elements is), else
 *                          GEMM_ERR_NOT_SUPPORTED.  As stream-K, the partial
 *                          sums handed between workgroups stay fp32.
 * The order in which the K products are summed is not specified; results are
 * bitwise reproducible run to run for the same call and kernel variant.
 *
 * Storage: every matrix is row-major (element (r, c) at ptr[r*ld + c]).
 *   transA == GEMM_OP_N : A stored M x K, lda >= max(1, K)
 *   transA == GEMM_OP_T : A stored K x M, lda >= max(1, M)
 *   transB == GEMM_OP_N : B stored K x N, ldb >= max(1, N)
 *   transB == GEMM_OP_T : B stored N x K, ldb >= max(1, K)
 *   C, D stored M x N, ldc >= max(1, N) (when C is read), ldd >= max(1, N)
 * A column-major caller obtains the same result by computing
 * D^T = op(B)^T op(A)^T, i.e. by swapping the operands.
 *
 * Ownership: A, B, C and D are device pointers owned by the caller; the
 * library never allocates, frees or retains them.  A handle owns only the
 * kernel-choice state below.  alpha and beta are host values.
 *
 * Execution: gemm_run validates its arguments on the host, then enqueues its
 * kernel(s) on `stream` (0 = the default stream) and returns without waiting.
 * The caller synchronizes before reading D.  Different handles may be used
 * concurrently from different threads.
 *
 * Semantics of degenerate calls:
 *   M == 0 or N == 0 : nothing is enqueued, GEMM_OK.
 *   K == 0 or alpha == 0 : D = beta * C (D = 0 when beta == 0); A and B are
 *                          not read and may be NULL.
 *   beta == 0 : C is never read and may be NULL; NaN/Inf in C cannot reach D.
 *   C == D (in place) is allowed when ldc == ldd; any other overlap of the C
 *   and D address ranges is rejected.
 *
 * Errors: every entry point returns a status; nothing aborts or throws.
 *   GEMM_ERR_INVALID_VALUE : checked before anything is enqueued — NULL
 *       handle or output pointer, unknown enum, negative size, leading
 *       dimension too small, NULL operand that must be read, overlapping C/D.
 *   GEMM_ERR_NOT_SUPPORTED : a size beyond the library's limits (M, N, K and
 *       every leading dimension below 2^31) or a forced kernel variant that
 *       does not handle the call's dtype.
 *   GEMM_ERR_HIP : the HIP runtime rejected the kernel launch.
 *   GEMM_ERR_ALLOC : gemm_create could not allocate its handle.
 *   GEMM_ERR_STREAM_K : reported by gemm_stream_k_status only: a stream-K
 *       finisher gave up waiting for a contributor (see that function).
 * Pointer alignment is never an error: misaligned operands select kernels
 * with narrower memory accesses.
 */
#ifndef DENSE_GEMM_H
#define DENSE_GEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemm_handle_s* gemm_handle_t;

typedef enum { GEMM_OP_N = 0, GEMM_OP_T = 1 } gemm_op_t;

typedef enum {
    GEMM_DTYPE_F32 = 0,       /* A, B fp32; C, D fp32; fp32 accumulate */
    GEMM_DTYPE_BF16_F32 = 1,  /* A, B bf16; C, D fp32; fp32 accumulate */
    GEMM_DTYPE_BF16_BF16 = 2  /* A, B bf16; C, D bf16; fp32 accumulate */
} gemm_dtype_t;

typedef enum {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_VALUE = 1,
    GEMM_ERR_NOT_SUPPORTED = 2,
    GEMM_ERR_HIP = 3,
    GEMM_ERR_ALLOC = 4,
    GEMM_ERR_STREAM_K = 5
} gemm_status_t;

/* Create a handle (*out receives it).  Makes no HIP call.  Two environment
 * variables, read here (set, non-empty and not "0" turns them on), apply to
 * every call made through the handle:
 *   GEMM_LOG               : after each launch, one line on stderr naming the
 *                            variant, layout, shape, dtype, grid, stream-K
 *                            workgroups and whether NN ran as D^T;
 *   GEMM_DEBUG_FAIL_LAUNCH : calls that pass their checks return GEMM_ERR_HIP
 *                            instead of launching (D is left untouched), so
 *                            callers can exercise their launch-failure path
 *                            without a real fault. */
gemm_status_t gemm_create(gemm_handle_t* out);

/* Release a handle.  NULL is accepted and ignored.  Pending work on streams
 * is not affected (the handle is not referenced by enqueued kernels). */
gemm_status_t gemm_destroy(gemm_handle_t h);

/* D = alpha*op(A)*op(B) + beta*C, enqueued on `stream`.  See the header
 * comment for layouts, degenerate cases and errors.  A and B point to float
 * (GEMM_DTYPE_F32) or to 16-bit bfloat16 patterns (both bf16 dtypes); C and D
 * point to float, or to bfloat16 patterns for GEMM_DTYPE_BF16_BF16. */
gemm_status_t gemm_run(gemm_handle_t h, gemm_op_t transA, gemm_op_t transB,
                       int64_t M, int64_t N, int64_t K, float alpha,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       float beta, const void* C, int64_t ldc,
                       void* D, int64_t ldd, gemm_dtype_t dtype, hipStream_t stream);

/* ---- fused epilogue ------------------------------------------------------
 * "GEMM on NVIDIA GPUs: from a naive kernel to a tiled pipeline" (section 4,
 * epilogue) lists alpha, beta, bias, activation, clamp and the dtype
 * conversion as work the store step can do in place, saving the round trip
 * of a second kernel through D.  gemm_run_epilogue computes, per element,
 *     D_ij = convert(clamp(act(alpha*op(A)op(B)_ij + beta*C_ij + bias_j)))
 * in that order, every step in fp32, with one conversion to D's type at the
 * end (nearest even for bf16).
 *   bias       : device pointer to N elements of D's element type (float, or
 *                bfloat16 for GEMM_DTYPE_BF16_BF16), bias[j] added to column
 *                j of every row; NULL for none.  Caller-owned; it must not
 *                overlap D (GEMM_ERR_INVALID_VALUE) and must be element
 *                aligned (GEMM_ERR_NOT_SUPPORTED otherwise).
 *   activation : GEMM_ACT_NONE; GEMM_ACT_RELU max(x, 0); GEMM_ACT_GELU
 *                x*Phi(x) = x/2 * (1 + erf(x/sqrt(2))) (the erf form).  Any
 *                other value: GEMM_ERR_INVALID_VALUE.
 *   clamp      : nonzero clamps to [clamp_lo, clamp_hi]; clamp_lo > clamp_hi
 *                or a NaN bound: GEMM_ERR_INVALID_VALUE.
 * A NULL epilogue (or one with no bias, no activation and no clamp) is
 * gemm_run.  Everything else -- layouts, degenerate cases (K == 0 or
 * alpha == 0 gives clamp(act(beta*C + bias))), errors -- is as for gemm_run.
 * The fused epilogue runs in the whole-tile direct-to-LDS kernels the
 * selector uses for element-aligned operands (also as stream-K, the
 * finishing workgroup applying it after the partial sums); where
 * gemm_run would take another kernel (operands not element-aligned, panel
 * offsets beyond 32 bits, a forced sweep variant) it returns
 * GEMM_ERR_NOT_SUPPORTED.                                                   */
typedef enum {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1,
    GEMM_ACT_GELU = 2
} gemm_activation_t;

typedef struct {
    const void* bias;
    gemm_activation_t activation;
    int clamp;
    float clamp_lo, clamp_hi;
} gemm_epilogue_t;

gemm_status_t gemm_run_epilogue(gemm_handle_t h, gemm_op_t transA, gemm_op_t transB,
                                int64_t M, int64_t N, int64_t K, float alpha,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                float beta, const void* C, int64_t ldc,
                                void* D, int64_t ldd, gemm_dtype_t dtype,
                                const gemm_epilogue_t* epilogue, hipStream_t stream);

/* Static, human-readable text for a status code ("unknown status" otherwise). */
const char* gemm_status_string(gemm_status_t s);

/* ---- kernel variants (per-shape tile and occupancy selection) -------------
 * The library holds a table of kernel variants (tile shape, wave grid,
 * instruction kind).  By default gemm_run picks one per call from the dtype,
 * transposes and M, N, K; a handle can instead force one (tests use this to
 * exercise every variant, benchmarks to sweep them).                        */

/* Number of variants in the table. */
int gemm_variant_count(void);

/* Static name of variant `id` (NULL when out of range), e.g.
 * "bf16_mfma16x16x32_256x256x64_w2x2". */
const char* gemm_variant_name(int id);

/* dtype handled by variant `id` (-1 when out of range). */
int gemm_variant_dtype(int id);

/* Tile shape of variant `id` into bm/bn/bk (any may be NULL). */
gemm_status_t gemm_variant_tile(int id, int* bm, int* bn, int* bk);

/* Software pipeline of variant `id`: LDS stages in its ring (*stages) and
 * K-steps between a step's copy into LDS and its first use (*ahead; S for a
 * barrier late in the step, S-1 for one half way).  Variants that copy
 * k-contiguous operands two K-steps at a time into pair buffers report the
 * ring of their other operands; a pair is copied three steps (with three
 * pair buffers five steps) ahead of its first step.  Any may be NULL.
 * GEMM_ERR_INVALID_VALUE for an unknown id. */
gemm_status_t gemm_variant_pipeline(int id, int* stages, int* ahead);

/* Workgroups of variant `id` (its NN kernel with 16-byte access) that fit on
 * one compute unit of the current device, from the HIP occupancy query: the
 * occupancy the pipeline depth trades against ("High-Performance FP16 GEMM
 * on NVIDIA Ada Lovelace", key results).  -1 for an unknown id or when the
 * device cannot be queried. */
int gemm_variant_occupancy(int id);

/* Planning model: what the planner behind gemm_run and gemm_select_variant
 * assumes about the device in place of querying it -- `cus` compute units
 * (0: the device attribute) and, per variant, occupancy[id] workgroups per
 * compute unit for its data-parallel kernel (0: the HIP occupancy query, as
 * gemm_variant_occupancy reports it).  The choices then follow the same
 * rules ("GEMM on NVIDIA GPUs", section 5: waves of tiles over the compute
 * units) for that model: planning on a host without the device, e.g. tests
 * of the selection rules, or for another device's figures.  `occupancy`
 * holds `count` == gemm_variant_count() entries, all >= 0, and is copied;
 * occupancy = NULL with cus = 0 clears the model.  Process-wide (every
 * handle); not meant to change while another thread plans a call.
 * GEMM_ERR_INVALID_VALUE for a negative cus or entry, or a wrong count. */
gemm_status_t gemm_set_planning_model(int cus, const int* occupancy, int count);

/* Force variant `id` for later gemm_run calls on h; -1 restores automatic
 * selection.  GEMM_ERR_INVALID_VALUE for an unknown id or NULL handle. */
gemm_status_t gemm_set_variant(gemm_handle_t h, int id);

/* Variant used by the last successful gemm_run on h (-1 if none or if that
 * call launched no GEMM kernel). */
int gemm_last_variant(gemm_handle_t h);

/* The variant gemm_run's automatic selection takes for this problem on a
 * handle without a workspace and without a forced variant, for A and B at
 * 16-byte-aligned addresses with tightly packed rows (lda, ldb = the stored
 * row length) and no fused epilogue: the same host logic gemm_run uses, so a
 * call of that kind reports this variant through gemm_last_variant.  It
 * queries the current device's compute-unit count and the variants'
 * occupancy (assuming 256 compute units and one workgroup when no device
 * answers); -1 for an invalid dtype, transpose or negative size. */
int gemm_select_variant(gemm_dtype_t dtype, gemm_op_t transA, gemm_op_t transB,
                        int64_t M, int64_t N, int64_t K);

/* ---- stream-K (split-K with an even split of the whole iteration space) ----
 * "GEMM on NVIDIA GPUs: from a naive kernel to a tiled pipeline", section 5:
 * split-K lets several workers share one output tile's K range, each forming
 * a partial sum P^(s)_ij over its range K_s, and reduces P_ij = sum_s P^(s)_ij
 * afterwards; stream-K divides all (tile, K-step) iterations evenly over the
 * workers at the price of that fix-up.  Its section 6 lists the workspace
 * limit among the fields that decide a GEMM configuration.
 *
 * A handle with a workspace may run a call as stream-K: a grid of about one
 * workgroup per workgroup slot of the GPU, each taking an equal run of the
 * iterations; a tile split between workgroups is finished by the one that
 * reaches its last K-step, which adds the others' partial sums in a fixed
 * order (results stay bitwise reproducible for a given call, variant and GPU).
 * Automatic mode uses it only when whole tiles would leave at least a tenth
 * of the last wave's slots idle.  Only 16-byte-capable direct-to-LDS variants
 * have stream-K kernels; other calls run data-parallel as before.          */

/* Bytes of workspace that let every stream-K variant run at its full grid on
 * the current device (a smaller workspace restricts stream-K to the calls it
 * can hold). */
size_t gemm_stream_k_workspace_bytes(void);

/* Give h a device workspace: caller-owned memory of `bytes` bytes, 256-byte
 * aligned, used by h's stream-K calls until replaced or cleared (ws == NULL or
 * bytes == 0).  Enqueues one small kernel on `stream` that clears the
 * workspace's flag area; the calls that use it must be ordered after that
 * kernel.  Layout: 4096 32-bit flags, one 32-bit sticky error word (then
 * padding to byte 16640), then one BM*BN fp32 partial-sum slot per
 * workgroup.  Each stream-K call leaves every flag zero again unless a
 * finisher's bounded wait gave up (gemm_stream_k_status).  Calls that
 * share a workspace must not overlap in time (use one handle and workspace
 * per concurrently used stream).  GEMM_ERR_INVALID_VALUE: NULL handle, a
 * misaligned pointer or fewer bytes than the flag area; GEMM_ERR_HIP: the
 * clearing kernel could not be launched. */
gemm_status_t gemm_set_workspace(gemm_handle_t h, void* ws, size_t bytes, hipStream_t stream);

/* Stream-K policy of h: -1 automatic (default), 0 never, 1 whenever the
 * variant and the workspace allow (tests use this to exercise the split on
 * small shapes).  GEMM_ERR_INVALID_VALUE for another mode or a NULL handle. */
gemm_status_t gemm_set_stream_k(gemm_handle_t h, int mode);

/* Stream-K workgroups used by the last gemm_run on h (0: data-parallel tiles;
 * -1 for a NULL handle). */
int gemm_last_stream_k(gemm_handle_t h);

/* Failure report of h's stream-K calls.  A finisher waits for each
 * contributor's flag a bounded number of polls (about 100 ns each).  Every
 * contributor of a stream-K grid is resident at the same time as its
 * finisher, so the bound is never reached in a correct run; if it is, the
 * finisher adds no partial sum and clears no flag, writes NaN in place of its
 * tile (where the fused epilogue's activation or clamp does not map NaN to a
 * number) and sets the workspace's sticky error word.  This call waits for
 * `stream`, reads that word and, when it is set, clears the whole flag area
 * and the word on `stream` (waiting again) and returns GEMM_ERR_STREAM_K: the
 * results of the stream-K calls since the last check are not to be trusted.
 * The same is done for the current device's gemm_run_no_alloc array once a
 * call has set it up.
 * GEMM_OK when the word is clear or h has no workspace; GEMM_ERR_HIP when the
 * copy or the clearing kernel fails; GEMM_ERR_INVALID_VALUE for a NULL
 * handle.  Synchronizing: not for use inside graph capture. */
gemm_status_t gemm_stream_k_status(gemm_handle_t h, hipStream_t stream);

/* ---- a gemm_run that allocates nothing ----------------------------------
 * For callers that cannot allocate device memory at call time (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * gemm_run_no_alloc takes gemm_run's arguments and computes the same result
 * with the same kernel choice, except that its stream-K workspace is the
 * library's own: a static device array of GEMM_NO_ALLOC_SCRATCH_BYTES per GPU
 * (the 16640-byte flag area, then 16 MiB of partial-sum slots: 64 slots of
 * 256x256 fp32 or 256 of 128x128), which each GPU the library runs on holds
 * until the process ends.  The handle's own workspace, if any, is not used.
 * The automatic choice only takes stream-K grids whose slots fit in it, as it
 * does for a caller's workspace of that size; should a plan need more, the
 * call returns GEMM_ERR_NOT_SUPPORTED before enqueuing anything.  It makes no
 * hipMalloc, hipFree or other allocating call.  The first call on a device
 * looks up that device's copy (hipGetSymbolAddress) and enqueues one small
 * kernel on `stream` that clears its flag area; later stream-K calls leave the
 * flags zero again.  Every call on a GPU shares that GPU's copy: calls that
 * may overlap in time on one GPU (several streams, several threads) race and
 * must be serialized by the caller.  gemm_stream_k_status reports and clears
 * a failed wait in the current device's copy as well.  Errors as for
 * gemm_run, plus GEMM_ERR_HIP when the first call on a device cannot set the
 * array up. */
#define GEMM_NO_ALLOC_SCRATCH_BYTES ((size_t)16640 + ((size_t)16 << 20))

gemm_status_t gemm_run_no_alloc(gemm_handle_t h, gemm_op_t transA, gemm_op_t transB,
                                int64_t M, int64_t N, int64_t K, float alpha,
                                const void* A, int64_t lda, const void* B, int64_t ldb,
                                float beta, const void* C, int64_t ldc,
                                void* D, int64_t ldd, gemm_dtype_t dtype, hipStream_t stream);

/* Bound on a stream-K finisher's wait, in polls per contributor, for h's later
 * calls: -1 restores the default (2^20); 0 makes every finisher that has
 * contributors give up at once, which lets a test exercise the failure report
 * with every kernel ending normally.  GEMM_ERR_INVALID_VALUE for a NULL handle
 * or a value below -1. */
gemm_status_t gemm_set_stream_k_poll_limit(gemm_handle_t h, int polls);

#ifdef __cplusplus
}
#endif

#endif /* DENSE_GEMM_H */
