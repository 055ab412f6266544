/*
 * libgemv — dense matrix-vector products on AMD Instinct MI355X (gfx950).
 *
 *   y = A·x (+ bias)                 gemv_f32 / gemv_f16 / gemv_bf16
 *   Y = A·X (+ bias), 1..64 vectors   gemv_batched_f16 / gemv_batched_bf16
 *   several y_i = A_i·x in one launch gemv_multi_*
 *   h = silu(A_gate·x) ⊙ (A_up·x)     gemv_gate_up_silu_*
 *   y = A·x for few, long rows        gemv_splitk_* (caller's workspace)
 *   y = scale ⊙ (Q·x), int8 Q         gemv_q8_f32 / gemv_q8_f16 / gemv_q8_bf16
 *
 * The operation.  Output m is the dot product of row m of A with x (page
 * "SGEMV CUDA代码学习", section "问题定义: 一行一个点积": A is M×K, x is K×1,
 * y is M×1), plus bias[m] when a bias is given; the bias may be absent, in
 * which case nothing is added (page "第 3 课：GEMV 与行级并行", section
 * "核心心智模型" item 1 for y = A x + bias, section "3. 正确性边界与指针安全性"
 * for the absent bias).  The batched form applies one pass over A to up to 64
 * right-hand vectors: the small-batch decode case measured on page "GEMM、
 * GEMV、dtype 与算术强度", section "可运行 CUDA 实验" (m = 16), and beyond it
 * the batches of 16 to 32 at which page "第 3 课" section "4. 性能与工程权舍"
 * moves to a matrix-core GEMM (here: the matrix-core kernel, still one
 * pass over A).
 *
 * Arithmetic.  fp16 and bf16 elements are multiplied and summed in fp32, the
 * wider accumulator that page "GEMM、GEMV、dtype 与算术强度", section "dtype
 * 改变什么", calls for; fp32 is true IEEE fp32 (never a reduced-precision
 * matrix mode).  Products may be fused (FMA) and the summation order is the
 * library's own, so results differ from a sequential sum by rounding only:
 * for every output |y − exact| <= 1e-5·Σ_k|A[m,k]·x[k]| + 1e-6.  Results are
 * deterministic: the same inputs give the same bits on every call.  No
 * atomics are used; each output is written by exactly one lane.
 *
 * Layouts.
 *   A     row-major: element (m, k) at A[(int64)m·lda + k], lda >= K.
 *         Elements K..lda-1 of each row are never read.
 *   x     K contiguous elements.
 *   X     K×nvec column-major: column j at X + (int64)j·K.
 *   bias  M contiguous fp32 values, or NULL.
 *   y     M contiguous fp32 values (written, never read).
 *   Y     M×nvec column-major fp32: column j at Y + (int64)j·M.
 *   fp16 / bf16 elements are passed as their raw 16-bit patterns (uint16_t):
 *   IEEE binary16, and bfloat16 (the upper half of a binary32 word).
 *   Outputs and bias are fp32 for every input type.
 *
 * Pointers and ownership.  A, x/X, bias and y/Y are device pointers (memory
 * from hipMalloc or a device allocator such as PyTorch's), owned by the
 * caller.  The library never allocates, frees, retains or synchronises: a
 * call only enqueues its kernel on `stream` (NULL = the null stream; split-K
 * enqueues two) and returns.  y/Y must not overlap A, x/X or bias.  Pointers must be aligned
 * to their element size; any further alignment is optional (16-byte aligned
 * A and x/X select the widest loads, for any row pitch and K; the matrix
 * cores, for several vectors, also need lda·element_size and K·element_size
 * to be multiples of 16 bytes and K % 8 == 0).
 *
 * Errors.  Every entry point validates its arguments before touching the
 * GPU.  GEMV_ERROR_INVALID_VALUE (nothing enqueued, y untouched) for:
 * M < 0, K < 0, lda < K, nvec outside [1, 64], a NULL A or x when
 * M > 0 and K > 0, a NULL y when M > 0, or a pointer not aligned to its
 * element size.  M == 0 succeeds without enqueuing anything.  K == 0 writes
 * y = bias (or 0): the empty sum.  GEMV_ERROR_LAUNCH_FAILURE if the HIP
 * runtime refuses the launch (nothing was enqueued; the runtime's own "last
 * error" is cleared again, see gemv_last_hip_error).  The library is
 * stateless and reentrant.
 */
#ifndef LIBGEMV_GEMV_H
#define LIBGEMV_GEMV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GEMV_SUCCESS = 0,
    GEMV_ERROR_INVALID_VALUE = 1,
    GEMV_ERROR_LAUNCH_FAILURE = 2
} gemv_status_t;

/* Static, NUL-terminated description of a status code. */
const char *gemv_status_string(gemv_status_t status);

/* The hipError_t value behind the calling thread's most recent
 * GEMV_ERROR_LAUNCH_FAILURE (0 = hipSuccess if there was none), and the HIP
 * runtime's name for it.  Thread-local; other calls do not reset it. */
int gemv_last_hip_error(void);
const char *gemv_last_hip_error_string(void);

/* y = A·x (+ bias); A, x fp32. */
gemv_status_t gemv_f32(const float *A, int lda, const float *x,
                       const float *bias, float *y, int M, int K,
                       hipStream_t stream);

/* y = A·x (+ bias); A, x IEEE binary16 bit patterns; fp32 accumulate/output. */
gemv_status_t gemv_f16(const uint16_t *A, int lda, const uint16_t *x,
                       const float *bias, float *y, int M, int K,
                       hipStream_t stream);

/* y = A·x (+ bias); A, x bfloat16 bit patterns; fp32 accumulate/output. */
gemv_status_t gemv_bf16(const uint16_t *A, int lda, const uint16_t *x,
                        const float *bias, float *y, int M, int K,
                        hipStream_t stream);

/* Y = A·X (+ bias added to every column); 1 <= nvec <= 64.  With 16-byte
 * aligned A and X, a row pitch of whole 16-byte units and K % 8 == 0, A is
 * read from memory once for all nvec vectors (matrix cores); otherwise the
 * vectors run in blocks of 16, one pass over A per block.  nvec == 1
 * computes what gemv_f16 does. */
gemv_status_t gemv_batched_f16(const uint16_t *A, int lda, const uint16_t *X,
                               const float *bias, float *Y, int M, int K,
                               int nvec, hipStream_t stream);

/* As gemv_batched_f16, for bfloat16 A and X. */
gemv_status_t gemv_batched_bf16(const uint16_t *A, int lda, const uint16_t *X,
                                const float *bias, float *Y, int M, int K,
                                int nvec, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Fused forms for one decode step.  Page "GEMM、GEMV、dtype 与算术强度",
 * section "可运行 CUDA 实验", shows a 4096×4096 GEMV taking about the same
 * time at 1 and 16 vectors: at decode sizes a launch's fixed cost is a large
 * share of the call.  The lqnn.cn NPU MatMul essay (sections 4.2 and 5.1)
 * fuses the QKV projections into one operator and the FFN's MatMuls with
 * their activation; these entry points do that on one GPU launch.
 * ------------------------------------------------------------------------ */

#define GEMV_MAX_SEGMENTS 8

/* One matrix of a multi-GEMV: y = A·x (+ bias), A M×K with row stride lda. */
typedef struct {
    const void *A;      /* device pointer, the call's element type */
    int lda;            /* >= K */
    int M;              /* >= 0; 0 = nothing to do for this segment */
    const float *bias;  /* M values, or NULL */
    float *y;           /* M values, written */
} gemv_segment_t;

/* y_i = A_i·x (+ bias_i) for every segment i < count (1..GEMV_MAX_SEGMENTS),
 * all with the same K and the same x (e.g. the q, k and v projections of one
 * token), in one launch.  The segment table is read on the host during the
 * call.  Each segment is validated like a gemv_* call; results are those of
 * separate calls up to summation order (the same tolerance).  No output may
 * overlap another output or any input. */
gemv_status_t gemv_multi_f32(const gemv_segment_t *segments, int count,
                             const float *x, int K, hipStream_t stream);
gemv_status_t gemv_multi_f16(const gemv_segment_t *segments, int count,
                             const uint16_t *x, int K, hipStream_t stream);
gemv_status_t gemv_multi_bf16(const gemv_segment_t *segments, int count,
                              const uint16_t *x, int K, hipStream_t stream);

/* h[m] = silu(g[m]) · u[m], g = A_gate·x, u = A_up·x, silu(g) = g/(1+e^-g):
 * the gated FFN projection pair in one pass over both M×K matrices (same
 * row stride lda), x read once for both.  h is fp32.  The tolerance follows
 * from the GEMV one: with t_g, t_u the bounds of g and u,
 * |h - h_exact| <= 1.1·t_g·(|u| + t_u) + |silu(g)|·t_u + 1e-6·|h| + 1e-6. */
gemv_status_t gemv_gate_up_silu_f32(const float *A_gate, const float *A_up,
                                    int lda, const float *x, float *h, int M,
                                    int K, hipStream_t stream);
gemv_status_t gemv_gate_up_silu_f16(const uint16_t *A_gate,
                                    const uint16_t *A_up, int lda,
                                    const uint16_t *x, float *h, int M, int K,
                                    hipStream_t stream);
gemv_status_t gemv_gate_up_silu_bf16(const uint16_t *A_gate,
                                     const uint16_t *A_up, int lda,
                                     const uint16_t *x, float *h, int M, int K,
                                     hipStream_t stream);

typedef enum { GEMV_DTYPE_F32 = 0, GEMV_DTYPE_F16 = 1, GEMV_DTYPE_BF16 = 2 } gemv_dtype_t;

/* ------------------------------------------------------------------------
 * Split-K, for few rows of many elements.  Page "SGEMV CUDA代码学习",
 * section "Kernel 1: k32", points out that with one row per warp a small M
 * (its example: M = 8) starts only a handful of blocks and leaves the rest
 * of the GPU idle.  Here each row is cut into `splits` slices of K; one
 * workgroup per (two rows, slice) writes their partial sums into a
 * caller-provided workspace, and a second kernel adds each row's partials
 * in a fixed order and the bias (two kernels on `stream`, no atomics).  The result is
 * y = A·x (+ bias) with the same tolerance as gemv_*, and identical bits on
 * every call with the same `splits`.
 *
 * splits: 0 = let the library choose (1 when M already fills the GPU or the
 * rows are short; then the call is exactly a gemv_* call and needs no
 * workspace); >= 1 = that many slices, rounded so that each slice is a whole
 * number of 16-byte loads (at most 1024; the effective count may be lower).
 * ------------------------------------------------------------------------ */

/* Bytes of workspace gemv_splitk_* needs for these arguments: 4·M·(effective
 * splits), or 0 when a single slice is used.  GEMV_ERROR_INVALID_VALUE for
 * M < 0, K < 0, splits < 0, a bad dtype or a NULL `bytes`. */
gemv_status_t gemv_splitk_workspace_size(gemv_dtype_t dtype, int M, int K,
                                         int splits, size_t *bytes);

/* y = A·x (+ bias) by split-K.  workspace: device memory of at least the
 * size above, 4-byte aligned, owned by the caller, not overlapping any
 * argument; it is overwritten (no initial contents are needed) and may be
 * reused once the call's kernels have finished on `stream`; two calls in
 * flight at the same time need separate workspaces.  Errors as for gemv_*,
 * plus GEMV_ERROR_INVALID_VALUE for splits < 0 or a NULL, misaligned or too
 * small workspace when one is needed. */
gemv_status_t gemv_splitk_f32(const float *A, int lda, const float *x,
                              const float *bias, float *y, int M, int K,
                              int splits, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);
gemv_status_t gemv_splitk_f16(const uint16_t *A, int lda, const uint16_t *x,
                              const float *bias, float *y, int M, int K,
                              int splits, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);
gemv_status_t gemv_splitk_bf16(const uint16_t *A, int lda, const uint16_t *x,
                               const float *bias, float *y, int M, int K,
                               int splits, void *workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Split-K for callers that cannot allocate (code under stream capture,
 * tight serving loops, harnesses that forbid hipMalloc): y = A·x (+ bias)
 * exactly as gemv_splitk_* with the same `splits` (the same kernels, the
 * same bits), A, x, bias and y of element type `dtype`, with no workspace
 * argument: the partial sums live in a static device buffer of
 * GEMV_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  The call allocates and frees nothing.  Its first
 * call on a device looks the buffer's address up (hipGetSymbolAddress) and
 * keeps it.  The buffer needs no clearing: each call writes every partial
 * it reads.  Every call on one GPU shares that GPU's buffer, so calls that
 * may run at the same time on one GPU (other streams, other host threads)
 * race and give wrong results: serialise them (one stream).  Errors as for
 * gemv_splitk_*, plus GEMV_ERROR_INVALID_VALUE when the call needs more than
 * GEMV_NOALLOC_SCRATCH_BYTES (4·M·splits bytes with the effective slice
 * count; gemv_splitk_workspace_size gives it).  The stream may belong to any
 * device. */
#define GEMV_NOALLOC_SCRATCH_BYTES (256 * 1024)
gemv_status_t gemv_splitk_noalloc(gemv_dtype_t dtype, const void *A, int lda,
                                  const void *x, const float *bias, float *y,
                                  int M, int K, int splits, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Weight-only int8.  The lqnn.cn NPU MatMul essay (sections 1.2, 4.2 and
 * 5.2) stores weights as int8 with a per-channel scale while activations
 * stay in floating point and the accumulator is fp32: at decode the weight
 * bytes halve against fp16/bf16, and the GEMV is bound by those bytes.
 *
 *   y[m] = scale[m] · Σ_k Q[m,k]·x[k] (+ bias[m])
 *
 * Q     row-major int8 (two's complement), element (m, k) at Q[m·ldq + k],
 *       ldq >= K (bytes K..ldq-1 of a row never read).  No zero point.
 * scale M fp32 values, one per row, applied after the row's sum.
 * x     K elements of the float type in the name (fp32 words, binary16 or
 *       bfloat16 bit patterns).
 * Products q·x are exact in fp32 and summed in fp32 in the library's own
 * order; |y - exact| <= 1e-5·|scale[m]|·Σ_k|Q[m,k]·x[k]| + 1e-6.
 * Errors as for gemv_*, plus a NULL scale when M > 0.  16-byte aligned Q
 * and x select the widest loads (for any ldq); any other alignment works.
 * ------------------------------------------------------------------------ */
gemv_status_t gemv_q8_f32(const int8_t *Q, int ldq, const float *scale,
                          const float *x, const float *bias, float *y, int M,
                          int K, hipStream_t stream);
gemv_status_t gemv_q8_f16(const int8_t *Q, int ldq, const float *scale,
                          const uint16_t *x, const float *bias, float *y,
                          int M, int K, hipStream_t stream);
gemv_status_t gemv_q8_bf16(const int8_t *Q, int ldq, const float *scale,
                           const uint16_t *x, const float *bias, float *y,
                           int M, int K, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Introspection and testing.  These do not change what the entry points
 * above compute; they expose how the library maps a problem onto the GPU so
 * that the mapping can be checked without a GPU and every kernel family can
 * be exercised at every shape it supports.
 * ------------------------------------------------------------------------ */

/* Kernel families.  Page "SGEMV CUDA代码学习", section "三 kernel 的设计空间
 * 总结", frames GEMV's only design choice as how many lanes share one row;
 * these are the gfx950 (64-lane wavefront) points on that axis. */
typedef enum {
    GEMV_FAMILY_AUTO = -1,
    GEMV_FAMILY_ROWS_PER_WAVE = 0, /* 64/L rows per wavefront, L lanes per row */
    GEMV_FAMILY_WAVE_PER_ROW = 1,  /* one 64-lane wavefront per row */
    GEMV_FAMILY_GROUP_PER_ROW = 2, /* one workgroup per row, LDS reduction */
    GEMV_FAMILY_BATCHED = 3,       /* 1-2 rows × nvec vectors per wave, or few rows split over 2-4 waves */
    GEMV_FAMILY_BATCHED_MFMA = 4,  /* 4-32 rows × 16 vectors per tile on the matrix cores */
    GEMV_FAMILY_GATED_SILU = 5,    /* a row of A_gate and of A_up per workgroup */
    GEMV_FAMILY_SPLIT_K = 6        /* a workgroup per two rows and K-slice, then a reduce */
} gemv_family_t;

typedef struct {
    int family;          /* gemv_family_t */
    int vector_loads;    /* 1: 16-byte loads; 0: one element per load */
    int chunk_elems;     /* elements per load (16/size, or 1) */
    int lanes_per_row;   /* lanes that share one row's dot product (batched
                            on the vector ALUs: 128 or 256 when a row's K
                            is split over 2 or 4 wavefronts) */
    int rows_per_wave;   /* rows one wavefront covers per row tile (matrix
                            cores: the workgroup's rows, which its wavefronts
                            share, each taking a slice of K) */
    int row_tiles;       /* row tiles each wavefront takes in one pass
                            (workgroup per row: rows per workgroup; matrix
                            cores: groups of 4 or 8 rows per workgroup, 1,
                            2 or 4 of them) */
    int waves_per_group; /* wavefronts per workgroup */
    int rows_per_group;  /* rows one workgroup produces */
    int batch;           /* loads per lane kept in flight per row */
    int passes;          /* loop trips per lane over one row's full chunks */
    int block;           /* threads per workgroup */
    int lds_bytes;       /* static + dynamic LDS per workgroup */
    int splits;          /* K-slices per row (split-K), else 1 */
    int slice_elems;     /* elements per K-slice (the last may be shorter), else K */
    int x_in_registers;  /* workgroup per row: 1 if each lane keeps its x chunks in
                            registers while the workgroup walks its rows */
    int rounding_chain;  /* n such that no product passes through more than n fp32
                            roundings on its way to its output, so that
                            |y - exact| <= γ_n·Σ_k|A[m,k]·x[k]|, γ_n ≈ n·2^-24;
                            at most 150 for every plan (the tolerance's 1e-5
                            holds up to n = 167) */
    int column_blocks;   /* batched: launches, each one pass over A for a block of
                            the vectors (1 = all vectors in one pass) */
    int64_t grid;        /* workgroups (split-K: ceil(rows / rows_per_group) × slices) */
} gemv_plan_t;

/* Compute, on the host only, the mapping a call with these arguments would
 * launch (family = GEMV_FAMILY_AUTO), or the mapping of a forced family.
 * The pointer arguments are inspected for alignment only (they may be any
 * value, including host addresses or NULL).  Returns GEMV_ERROR_INVALID_VALUE
 * for arguments the entry points would reject or a family that cannot run
 * this shape (e.g. GEMV_FAMILY_BATCHED for fp32, or a single-vector family
 * with nvec > 1; the gated and split-K families have their own calls). */
gemv_status_t gemv_plan(gemv_dtype_t dtype, int M, int K, int lda, int nvec,
                        const void *A, const void *X, int family,
                        gemv_plan_t *plan);

/* The mapping gemv_splitk_* would launch: family GEMV_FAMILY_SPLIT_K with
 * its splits and slice length, or (one slice) the gemv_* mapping. */
gemv_status_t gemv_plan_splitk(gemv_dtype_t dtype, int M, int K, int lda,
                               int splits, const void *A, const void *x,
                               gemv_plan_t *plan);

/* The mapping gemv_q8_* would launch for x of type xdtype (or a forced
 * family: rows per wavefront, wave per row or workgroup per row), and a run
 * with a forced family; same contracts as the entry points. */
gemv_status_t gemv_plan_q8(gemv_dtype_t xdtype, int M, int K, int ldq,
                           const void *Q, const void *x, int family,
                           gemv_plan_t *plan);
gemv_status_t gemv_q8_run_family(gemv_dtype_t xdtype, int family,
                                 const int8_t *Q, int ldq, const float *scale,
                                 const void *x, const float *bias, float *y,
                                 int M, int K, hipStream_t stream);

/* Read probe (measurement only): stream `bytes` of device memory from
 * `buffer` once, in the access pattern of the GEMV kernels (64-lane
 * wavefronts with eight 1 KiB nontemporal loads in flight each), and write
 * nothing; `sink` (4 device bytes) is written only if the folded data equal
 * one fixed 32-bit value.  Timed beside a GEMV of the same bytes it separates
 * what streaming those bytes costs on this GPU from what the GEMV adds
 * (page "GEMM、GEMV、dtype 与算术强度", section "FLOPs、最低字节数与算术强度":
 * the minimum byte count is an algorithmic bound, not what a kernel
 * achieves).  bytes == 0 enqueues nothing; a NULL buffer or sink, bytes not
 * a multiple of 16, or a buffer not 16-byte aligned gives
 * GEMV_ERROR_INVALID_VALUE. */
gemv_status_t gemv_read_probe(const void *buffer, size_t bytes, unsigned *sink,
                              hipStream_t stream);

/* Read-probe variants (measurement only): the read probe's job with other
 * read patterns, to map the streaming cost of `bytes` against the pattern.
 * loads_per_lane: 2, 4, 8 or 16 sixteen-byte loads in flight per lane (that
 * many KiB per wavefront); waves_per_group: 1, 2, 4, 8 or 16;
 * blocks_per_wave >= 1 blocks of loads_per_lane KiB per wavefront;
 * flags: bit 0 plain (cached) loads instead of nontemporal ones, bit 1 the
 * wavefront's priority raised while it issues its loads, bit 2 blocks dealt
 * grid-stride (block w + b·wavefronts) instead of consecutively.  The grid
 * has ceil(ceil(bytes / (1024·loads_per_lane·blocks_per_wave)) /
 * waves_per_group) workgroups.  wave_times (NULL, or 8-byte aligned device
 * memory of at least 2 × workgroups × waves_per_group entries, given in
 * wave_times_len): wavefront w writes its start and end readings of the
 * GPU's constant-rate real-time counter to entries 2w and 2w + 1.  Nothing
 * else is written (as gemv_read_probe).  Other values give
 * GEMV_ERROR_INVALID_VALUE. */
gemv_status_t gemv_read_probe_variant(const void *buffer, size_t bytes,
                                      unsigned *sink, int loads_per_lane,
                                      int waves_per_group, int blocks_per_wave,
                                      int flags, unsigned long long *wave_times,
                                      size_t wave_times_len, hipStream_t stream);

/* Error-path check (testing only): asks the HIP runtime for a launch it
 * must refuse before anything reaches the GPU (a workgroup of 2048 threads;
 * the hardware allows 1024) through the same launch path as every entry
 * point, and returns what an entry point returns when a launch is refused:
 * GEMV_ERROR_LAUNCH_FAILURE, with the runtime's error available from
 * gemv_last_hip_error().  The runtime's own "last error" is cleared, as after
 * any refused launch of this library, so later calls are unaffected. */
gemv_status_t gemv_test_refused_launch(hipStream_t stream);

/* Run with a forced family (GEMV_FAMILY_AUTO = what the entry points do).
 * Same arguments, validation and results contract as the entry points;
 * for tests and benchmarks. */
gemv_status_t gemv_run_family(gemv_dtype_t dtype, int family, const void *A,
                              int lda, const void *X, const float *bias,
                              float *Y, int M, int K, int nvec,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBGEMV_GEMV_H */
