/*
 * dg.h -- C ABI of the MI355X (gfx950) dense GEMM library.
 *
 * Computes  C <- alpha * A * B + beta * C  for FP16/BF16 inputs with FP32
 * accumulation, and an FP8 E4M3 variant whose per-token and per-block FP32
 * scale factors are applied inside the kernel.
 *
 * Sources (pages cited by title and section):
 *  - The operation, C = alpha*op(A)*op(B) + beta*C with op() folded into
 *    strides: DeepGEMM view-native GEMM article (kwkr.cn), sections 2.3 and
 *    4.1; "DeepGEMM: GEMM micro-kernel modelling and generation methodology for
 *    heterogeneous chips" (xdnf.cn), section 3.1; "DeepGEMM deep dive: from
 *    GEMM fundamentals to Tensor Core performance" (sheratonhq.com), section 1.1.
 *  - Operands as views {ptr, shape[<=4], byte stride[<=4], dtype}: kwkr.cn
 *    article, sections 2.1 and 3.2 (strides are bytes, not elements).
 *  - FP8 with scale factors applied in the kernel: sheratonhq.com deep dive,
 *    section 2.4.
 *  - Bias + activation fused into the GEMM's epilogue: "DeepGEMM is not a new
 *    model" article (cf-1.com), section 3.3.
 *
 * Conventions shared by every entry point
 *  - Views are borrowed for the duration of the call only; the caller owns all
 *    memory.  `ptr` is a device pointer (any HIP device allocation, e.g. a
 *    PyTorch tensor's data_ptr()).  Buffers must stay valid until `stream`
 *    has executed the launched work.
 *  - A view's logical matrix: rows = row-major flattening of dims 0..ndim-2,
 *    cols = dim ndim-1 (ndim == 1 is a single row).  Leading dims must merge
 *    into one row stride (stride[i] == stride[i+1] * shape[i+1]) once size-1
 *    dims are dropped; otherwise DG_ERR_UNSUPPORTED_VIEW.
 *  - A is M x K, B is K x N, C is M x N.  Any strides >= 0 (transposes are
 *    just strides); input views may use stride 0 (broadcast).  C must not use
 *    stride 0 on an extent > 1 and must not overlap itself.
 *  - alpha and beta are FP32 and must be finite.  beta == 0: C is not read
 *    (NaN garbage in C is ignored).  alpha == 0 or K == 0: A and B are not
 *    read and C <- beta * C.  M == 0 or N == 0: nothing happens.
 *  - NaN/Inf in the data propagate per IEEE; nothing on the hot path checks.
 *  - Work is enqueued on `stream` (0 = null stream) and the call returns
 *    without synchronizing.  Launch errors are reported as DG_ERR_HIP; faults
 *    during execution surface at the caller's next synchronization.
 *  - On any error return, C has not been touched and nothing was enqueued.
 *  - Thread safety: every entry point may be called concurrently from several
 *    host threads and on several streams.  Split-K scratch memory (partial
 *    sums and arrival counters) is library-owned device memory per (device,
 *    stream), allocated in stream order on that stream (hipMallocAsync) on
 *    first need.  When a call needs more, the larger block is allocated and
 *    the old one released with hipFreeAsync, both on the stream, so the old
 *    block is freed only after the work already enqueued there; the host never
 *    waits.  A call holds its stream's scratch from lookup until its kernels
 *    are enqueued, so two host threads may share one stream.  Calls on
 *    different streams never share scratch.  Scratch is kept until the process
 *    ends.  (kwkr.cn article, troubleshooting table in section 5.1: state that
 *    host threads share must be thread-safe; sheratonhq.com deep dive, section
 *    5.2: split-K partials in a workspace.)
 */
#ifndef DG_H
#define DG_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DG_VERSION 10000 /* 1.0.0 */

typedef enum {
    DG_F32 = 0,
    DG_F16 = 1,     /* IEEE binary16 */
    DG_BF16 = 2,    /* bfloat16 */
    DG_F8E4M3 = 3   /* OCP E4M3FN: bias 7, 3 mantissa bits, max 448, no Inf */
} dg_dtype;

typedef enum {
    DG_SUCCESS = 0,
    DG_ERR_NULL = 1,              /* null view, or null ptr with nonzero extent */
    DG_ERR_NDIM = 2,              /* ndim outside 1..4 */
    DG_ERR_STRIDE = 3,            /* negative stride, stride not a multiple of the element
                                     size, negative extent, or C that overlaps itself
                                     (e.g. stride 0 on an extent > 1) */
    DG_ERR_SHAPE_MISMATCH = 4,    /* K, M or N disagree; scale views of the wrong shape */
    DG_ERR_DTYPE = 5,             /* unsupported dtype or dtype combination */
    DG_ERR_MISALIGNED = 6,        /* ptr not aligned to the element size */
    DG_ERR_ALIAS = 7,             /* C's byte span overlaps A, B or a scale view */
    DG_ERR_NONFINITE_SCALAR = 8,  /* alpha or beta is NaN or Inf */
    DG_ERR_OVERFLOW = 9,          /* an extent or byte offset overflows 64 bits */
    DG_ERR_UNSUPPORTED_VIEW = 10, /* leading dims do not merge into one row stride */
    DG_ERR_POINTER = 11,          /* not a device pointer (checked only if DG_CHECK_POINTERS=1) */
    DG_ERR_ARCH = 12,             /* current device is not gfx950 */
    DG_ERR_HIP = 13,              /* a HIP runtime call or kernel launch failed */
    DG_ERR_INVALID_ARG = 14,      /* other invalid argument (e.g. a null output buffer) */
    DG_ERR_SCRATCH = 15           /* dg_gemm_noalloc: the plan needs more split-K scratch
                                     than the fixed buffer holds */
} dg_status;

/* A tensor view: up to 4 dims, strides in BYTES (kwkr.cn article, section 3.2). */
typedef struct {
    void *ptr;           /* address of element (0,...,0) */
    int32_t ndim;        /* 1..4 */
    int64_t shape[4];    /* extents; entries >= ndim are ignored */
    int64_t stride[4];   /* byte strides; entries >= ndim are ignored */
    dg_dtype dtype;
} dg_view;

/*
 * C <- alpha * A * B + beta * C, FP32 accumulation.
 *   A: M x K, B: K x N, both DG_F16 or both DG_BF16.
 *   C: M x N, DG_F32, DG_F16 or DG_BF16; results are rounded to nearest even.
 * Definition: kwkr.cn article, sections 2.3 and 4.1; xdnf.cn methodology, 3.1.
 */
dg_status dg_gemm(const dg_view *A, const dg_view *B, const dg_view *C,
                  float alpha, float beta, hipStream_t stream);

/*
 * FP8 E4M3 GEMM with block scales applied in the kernel:
 *   C[m,n] <- alpha * sum_k (qA[m,k] * sA[m, k/128]) * (qB[k,n] * sB[k/128, n/128])
 *             + beta * C[m,n]
 *   A (qA): M x K DG_F8E4M3;  A_scale (sA): M x ceil(K/128) DG_F32 (per token,
 *   one scale per row and 128-wide K block);  B (qB): K x N DG_F8E4M3;
 *   B_scale (sB): ceil(K/128) x ceil(N/128) DG_F32 (one scale per 128 x 128
 *   block).  Scale views take any strides.  C: DG_BF16, DG_F32 or DG_F16.
 * Each K block of 128 is summed on the matrix cores and promoted into the FP32
 * accumulator with its scale product exactly once (sheratonhq.com deep dive,
 * sections 2.4 and 4.2).
 */
dg_status dg_gemm_fp8(const dg_view *A, const dg_view *A_scale, const dg_view *B,
                      const dg_view *B_scale, const dg_view *C, float alpha, float beta,
                      hipStream_t stream);

/* Activation of the fused epilogue (dg_gemm_epilogue, dg_gemm_fp8_epilogue). */
typedef enum {
    DG_ACT_NONE = 0,
    DG_ACT_RELU = 1,       /* x < 0 ? 0 : x (NaN stays NaN) */
    DG_ACT_GELU_TANH = 2   /* GELU, tanh form (Hendrycks and Gimpel, 2016):
                              0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))) */
} dg_act;

/*
 * GEMM with a fused epilogue: the bias add and the activation run on the
 * accumulators in registers, and C is written once ("DeepGEMM is not a new
 * model" article, cf-1.com, section 3.3: GEMM + BiasAdd + GeLU in one kernel
 * instead of three global-memory round trips):
 *
 *   C[m,n] <- act(alpha * (A*B)[m,n] + beta * C[m,n] + bias[n])
 *
 * (A*B)[m,n] is the FP32-accumulated product of dg_gemm (FP16/BF16 A and B),
 * or of dg_gemm_fp8 with its scales (the _fp8 form).  The sum is formed in
 * FP32 in that order (alpha * AB, then + beta * C with one rounding, then
 * + bias), the activation is evaluated in FP32 and the result rounded once to
 * C's dtype.
 *   bias: NULL (no bias), or a view of N elements (shape [N] or [1, N]) of
 *         dtype DG_F32, DG_F16 or DG_BF16 with any element stride >= 0
 *         (0: one value for every column).  Read only; it must not overlap C.
 *   act:  a dg_act value.
 * alpha == 0 or K == 0: C <- act(beta * C + bias).  With bias == NULL and
 * act == DG_ACT_NONE the result is bit for bit that of dg_gemm / dg_gemm_fp8.
 * Every other argument, rule and error as for dg_gemm / dg_gemm_fp8, plus:
 * DG_ERR_INVALID_ARG (act not a dg_act value), DG_ERR_DTYPE (bias dtype),
 * DG_ERR_SHAPE_MISMATCH (bias not 1 x N), DG_ERR_ALIAS (bias overlaps C), and
 * the view errors of the bias view itself.
 */
dg_status dg_gemm_epilogue(const dg_view *A, const dg_view *B, const dg_view *C,
                           const dg_view *bias, dg_act act, float alpha, float beta,
                           hipStream_t stream);

dg_status dg_gemm_fp8_epilogue(const dg_view *A, const dg_view *A_scale, const dg_view *B,
                               const dg_view *B_scale, const dg_view *C, const dg_view *bias,
                               dg_act act, float alpha, float beta, hipStream_t stream);

/*
 * Grouped GEMM: G independent problems in one call,
 *
 *   C[g] <- alpha * A[g] * B[g] + beta * C[g],   g = 0 .. G-1,
 *
 * e.g. the experts of an MoE layer applied to the tokens routed to each: the
 * "DeepGEMM is not a new model" article (cf-1.com), section 1, singles out the
 * small per-expert GEMM [1,512] x [512,4096] issued once per expert, whose cost
 * is dominated by launching it (about 1.2 us per launch, its section 5.1).
 *   A, B, C: host arrays of G views each (read during the call only).  Every
 *         group obeys every rule of dg_gemm; groups may differ in M, N, K,
 *         strides and C dtype, but A and B have one dtype (DG_F16 or DG_BF16)
 *         across all groups.  Input views may be shared between groups (one
 *         token row sent to several experts); no group's C may overlap any
 *         group's A, B or C.
 *   G == 0: nothing happens.
 * Execution: groups with M <= 8 whose B is N-contiguous with 16-byte aligned
 * rows run together in one launch per M class (1, 2, 4, 8) and per 16 groups.
 * Every other group is planned for its share of the CUs (its M*N over the sum
 * of theirs); those whose plan is then the matrix-core kernel with direct
 * HBM -> LDS loads and no K split run together, one launch per tile
 * configuration (tile size, operand storage orders) and per 16 groups, when at
 * least two share it (the experts of an MoE layer with more than a few tokens
 * each).  The rest run through their own dg_gemm plan, in order, on `stream`.
 * Results equal those of G separate dg_gemm calls within the dg_gemm tolerance
 * (a group's tile and K split may differ), and are bitwise reproducible.
 * Errors: DG_ERR_INVALID_ARG (G < 0), DG_ERR_NULL (an array is NULL with
 * G > 0), the dg_gemm error of the first invalid group, DG_ERR_DTYPE (A/B
 * dtypes differ between groups), DG_ERR_ALIAS (a C overlaps another group's
 * operand).  Validation errors enqueue nothing; a launch failure (DG_ERR_HIP)
 * may leave earlier launches of the call enqueued.
 */
dg_status dg_gemm_grouped(int32_t G, const dg_view *A, const dg_view *B, const dg_view *C,
                          float alpha, float beta, hipStream_t stream);

/* Validate as dg_gemm_grouped does and describe its launches (batches of
 * grouped groups with their K splits, and the groups run alone) in buf,
 * without launching anything.  buf may be NULL only if len == 0. */
dg_status dg_gemm_grouped_plan(int32_t G, const dg_view *A, const dg_view *B, const dg_view *C,
                               float alpha, float beta, char *buf, size_t len);

/*
 * Plan choices and autotuning.
 *
 * A plan is a kernel path with its tile and K split; the library picks one per
 * problem with a built-in heuristic.  Fixed tile sizes cannot be best for every
 * shape, so a problem can be tuned: a small set of candidate plans is run on
 * the device with the real shape and precision and the fastest is kept, keyed
 * by device (architecture and CU count) and problem (M, N, K, byte strides,
 * alignments, dtypes), and can be saved to a file so that a process does not
 * search again at every start ("DeepGEMM deep dive" article, sheratonhq.com,
 * section 5.3; the "DeepGEMM is not a new model" article, cf-1.com, section
 * 5.2, probes the best tile per shape at warm-up and warns that probing only
 * pays when amortized).  Every later dg_gemm, dg_gemm_fp8 or
 * dg_gemm_epilogue call with the same key uses the tuned plan; its results
 * stay within the documented bound and are bitwise reproducible per plan.
 *
 * These entry points take the FP8 scale views as optional: A_scale and
 * B_scale both NULL for FP16/BF16 inputs, both given for FP8 (dg_gemm_fp8's
 * rules); one NULL and not the other is DG_ERR_NULL.
 */
typedef struct {
    int32_t path;     /* 0 built-in, 1 streaming kernel (thin shapes), 2 matrix-core kernel */
    int32_t tile;     /* -1 built-in, else 0: 256x256, 1: 128x128, 2: 64x64, 3: 128x64, 4: 64x128
                         (where the selected kernel has that tile; otherwise ignored) */
    int32_t splits;   /* 0 built-in, else the number of K splits (clamped to the K tiles; the
                         matrix-core 256x256 direct kernel never splits) */
    int32_t tail;     /* -1 built-in, 0 never split the tail of the last wave of tiles */
} dg_plan_choice;

typedef struct {
    double default_us;   /* average launch duration of the built-in plan */
    double best_us;      /* ... of the chosen plan (<= default_us) */
    double tune_ms;      /* wall time of the whole tuning call */
    int32_t candidates;  /* plans timed */
    int32_t chosen;      /* index of the chosen plan in dg_gemm_candidates' list */
    int32_t sets;        /* operand sets the timing rotated over (1: the caller's only) */
    char plan[512];      /* description of the chosen plan (dg_gemm_plan's format) */
} dg_tune_result;

/* The candidate plans the tuner times for this problem, built-in plan first,
 * no two alike: up to `max` written to out[], their number to *count.  Needs
 * no GPU (plans for a 256-CU gfx950 when no device is visible).
 * Errors: DG_ERR_NULL (count NULL, or out NULL with max > 0, or max < 0), and
 * the validation errors of dg_gemm / dg_gemm_fp8. */
dg_status dg_gemm_candidates(const dg_view *A, const dg_view *A_scale, const dg_view *B,
                             const dg_view *B_scale, const dg_view *C, dg_plan_choice *out,
                             int32_t max, int32_t *count);

/* dg_gemm / dg_gemm_fp8 with an explicit plan choice (any choice is valid: a
 * field that the selected kernel cannot honour is ignored).  Same semantics,
 * bound and errors, plus DG_ERR_NULL (choice NULL) and DG_ERR_INVALID_ARG
 * (path outside 0..2, tile outside -1..4, splits outside 0..64). */
dg_status dg_gemm_with_choice(const dg_view *A, const dg_view *A_scale, const dg_view *B,
                              const dg_view *B_scale, const dg_view *C, const dg_plan_choice *choice,
                              float alpha, float beta, hipStream_t stream);

/* Tune this problem on the current device: run the built-in plan for about
 * 30 ms (the clocks rise under sustained load), then time every candidate
 * twice, each time one untimed launch and max(reps, sets) launches between two
 * events on `stream` (reps 0: 5), keep the fastest for the problem's key (by
 * each candidate's better time), fill *result.  Successive launches run on
 * distinct copies of the operands (at least 1 GiB of them in total, at most
 * 64 sets; none for a problem of 512 MB or more), so that every candidate
 * reads its operands from HBM, as in a workload, and not from the last-level
 * cache: the ranking of plans for bandwidth-bound shapes depends on it
 * (sheratonhq.com deep dive, section 5.3: tune on the target device with the
 * real shape; cf-1.com article, section 5.2).  The copies are allocated with
 * hipMalloc and freed before the call returns.  C (and its copies) is
 * overwritten with A*B (alpha 1, beta 0; its earlier contents are lost); A and
 * B are only read.  Synchronizes `stream`.  Problems with M, N or K equal to 0 have nothing to
 * tune (result->candidates = 0).
 * Errors: DG_ERR_NULL (result NULL), DG_ERR_INVALID_ARG (reps outside
 * 0..1000), the validation errors of dg_gemm / dg_gemm_fp8, DG_ERR_HIP. */
dg_status dg_gemm_tune(const dg_view *A, const dg_view *A_scale, const dg_view *B,
                       const dg_view *B_scale, const dg_view *C, int32_t reps,
                       dg_tune_result *result, hipStream_t stream);

/* Write every tuned plan to a text file (one line per entry), or add the
 * entries of such a file (a malformed file adds nothing: DG_ERR_INVALID_ARG;
 * entries for other devices are kept and match no problem here).
 * Errors: DG_ERR_NULL (path NULL), DG_ERR_INVALID_ARG (cannot open, write or
 * parse the file). */
dg_status dg_tune_save(const char *path);
dg_status dg_tune_load(const char *path);
/* Forget every tuned plan; later calls use the built-in selection again. */
void dg_tune_clear(void);
/* Number of tuned plans held. */
int32_t dg_tune_count(void);

/*
 * dg_gemm / dg_gemm_fp8 for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  A_scale and B_scale: both NULL for FP16/BF16 inputs, both given
 * for FP8 (dg_gemm_fp8's rules; one NULL and not the other is DG_ERR_NULL).
 * Same plan, kernels, results (bit for bit), bound and errors as dg_gemm /
 * dg_gemm_fp8, but the split-K scratch is a fixed device array inside the
 * library instead of the stream's workspace, and the call allocates nothing
 * (no hipMalloc, hipMallocAsync or allocating library routine).
 *  - The fixed array holds 16 MiB of FP32 partial sums and 16384 arrival
 *    counters per device, from the library's load until the process ends.  A
 *    problem whose plan needs more returns DG_ERR_SCRATCH and enqueues nothing.
 *  - Every dg_gemm_noalloc call on one device shares that device's array: two
 *    calls whose work overlaps in time on one device (different streams, or
 *    different host threads with no ordering between them) race and may
 *    return wrong results.  Calls ordered on one stream are safe.
 *  - The first call on a device enqueues a zeroing of the counters on its
 *    stream; every kernel that uses them leaves them at zero.
 */
dg_status dg_gemm_noalloc(const dg_view *A, const dg_view *A_scale, const dg_view *B,
                          const dg_view *B_scale, const dg_view *C, float alpha, float beta,
                          hipStream_t stream);

/*
 * Validate the arguments of dg_gemm exactly as dg_gemm does and write a
 * one-line, NUL-terminated description of the chosen plan (path, tiles,
 * split-K, grid, canonical operand layouts) into buf[0..len-1], without
 * launching anything.  The pages check a problem against its views before any
 * kernel runs (a K disagreement is an error when the kernel is specialized,
 * not an assertion at run time) and pick the kernel variant per shape and
 * dtype from a cache (kwkr.cn article, sections 4.2 and 6.1); this call
 * exposes that step on its own.  Needs no GPU: with no device visible it plans for a
 * 256-CU gfx950.  Returns the status dg_gemm would return before launching.
 * buf may be NULL only if len == 0.  A tuned plan (dg_gemm_tune,
 * dg_tune_load) of the same key is the one described.
 */
dg_status dg_gemm_plan(const dg_view *A, const dg_view *B, const dg_view *C,
                       float alpha, float beta, char *buf, size_t len);

/* Same as dg_gemm_plan for the arguments of dg_gemm_fp8 (kwkr.cn article,
 * sections 4.2 and 6.1; the FP8 operands and scales of sheratonhq.com deep
 * dive, section 2.4). */
dg_status dg_gemm_fp8_plan(const dg_view *A, const dg_view *A_scale, const dg_view *B,
                           const dg_view *B_scale, const dg_view *C, float alpha, float beta,
                           char *buf, size_t len);

/*
 * FP8 E4M3 quantization of X, the producer of dg_gemm_fp8's operands: FP8 GEMM
 * needs per-token or per-block FP32 scale factors that squeeze each block into
 * the representable range, and a dedicated kernel applies them without an
 * extra pass (sheratonhq.com deep dive, sections 2.4 and 5.4).  The blocks are
 * those of dg_gemm_fp8's scale views: 1 x 128 (token) and 128 x 128.
 *
 *   X: M x K, DG_F32, DG_F16 or DG_BF16 (any strides; read only).
 *   Q: M x K, DG_F8E4M3 (written; must not overlap itself, X or S).
 *   S: FP32 scales (written; must not overlap itself, X or Q):
 *        DG_QUANT_TOKEN  [M][ceil(K/128)]: one per row and 128-wide block of K
 *                        (dg_gemm_fp8's A_scale when X is A);
 *        DG_QUANT_BLOCK  [ceil(M/128)][ceil(K/128)]: one per 128x128 block
 *                        (dg_gemm_fp8's B_scale when X is B as [K][N]).
 * For each block, in FP32 with IEEE operations:
 *   amax = max |x| over the block's elements (a partial block covers only the
 *          elements inside X);
 *   s    = max(amax, 1e-12) / 448;
 *   q    = E4M3(min(max(x / s, -448), 448)), rounded to nearest, ties to an
 *          even code; -0 keeps its sign.
 * X must be finite: for a block holding NaN or Inf the codes and scale are
 * unspecified (the call still completes).  M == 0 or K == 0: nothing happens.
 * Same conventions as the GEMM entry points (asynchronous on `stream`, C
 * untouched on error -- here Q and S).
 */
typedef enum { DG_QUANT_TOKEN = 0, DG_QUANT_BLOCK = 1 } dg_quant_mode;

dg_status dg_quant_fp8(const dg_view *X, const dg_view *Q, const dg_view *S, dg_quant_mode mode,
                       hipStream_t stream);

/* Helper (no page passage): static, human-readable name of a status code
 * ("DG_ERR_ALIAS", ...); "DG_ERR_UNKNOWN" for a value outside dg_status. */
const char *dg_status_str(dg_status s);

/* Helper (no page passage): DG_VERSION of the built library. */
int dg_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DG_H */
