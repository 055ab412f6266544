// libgemv C ABI: argument validation, mapping selection and kernel launch.
//
// The launcher shape follows page "第 3 课：GEMV 与行级并行", section "实践任务"
// (a host function taking A, x, bias, y, M, N and a stream), with an explicit
// row pitch, status codes instead of unchecked launches, and the mapping
// chosen by row length and row count (gemv_plan.hpp).
#include <hip/hip_runtime.h>

#include "../../include/gemv.h"
#include "gemv_kernels.hpp"
#include "gemv_plan.hpp"

namespace {

thread_local hipError_t g_last_launch_error = hipSuccess;

using gemvdev::TBF16;
using gemvdev::TF16;
using gemvdev::TF32;
using gemvplan::Plan;

struct Args {
    const void* A;
    int64_t lda;
    const void* X;
    const float* bias;
    float* Y;
    int M;
    int K;
    int nvec;
};

// Every kernel takes (A, lda, X, bias, Y, M, K); the matrix-core kernel also
// takes nvec (the others have it as a template parameter or do not need it).
hipError_t launch(const void* fn, const Plan& p, hipStream_t stream, const Args& a) {
    const void* A = a.A;
    int64_t lda = a.lda;
    const void* X = a.X;
    const float* bias = a.bias;
    float* Y = a.Y;
    int M = a.M;
    int K = a.K;
    int nvec = a.nvec;
    void* argv[] = {(void*)&A, (void*)&lda, (void*)&X, (void*)&bias, (void*)&Y, (void*)&M, (void*)&K,
                    (void*)&nvec};
    return hipLaunchKernel(fn, dim3((unsigned)p.grid), dim3((unsigned)p.block), argv, 0, stream);
}

// ---- rows-per-wave / wave-per-row ----------------------------------------

template <class D, int L, bool VEC>
const void* rows_fn(int tiles) {
    if constexpr (L == 64) {
        // one wavefront per row: a single row tile, kWaveBatch loads in flight
        if (tiles != 1) return nullptr;
        return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, gemvplan::kWaveBatch, VEC>;
    } else {
        // several rows per wavefront: one load per row tile, several tiles
        switch (tiles) {
        case 1: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 1, 1, VEC>;
        case 2: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 2, 1, VEC>;
        case 4: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 4, 1, VEC>;
        case 8: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 8, 1, VEC>;
        default: return nullptr;
        }
    }
}

template <class D, bool VEC>
const void* rows_fn(int lanes, int tiles) {
    switch (lanes) {
    case 1: return rows_fn<D, 1, VEC>(tiles);
    case 2: return rows_fn<D, 2, VEC>(tiles);
    case 4: return rows_fn<D, 4, VEC>(tiles);
    case 8: return rows_fn<D, 8, VEC>(tiles);
    case 16: return rows_fn<D, 16, VEC>(tiles);
    case 32: return rows_fn<D, 32, VEC>(tiles);
    case 64: return rows_fn<D, 64, VEC>(tiles);
    default: return nullptr;
    }
}

// ---- batched ----------------------------------------------------------------

template <class D, int NV, bool VEC>
const void* batched_fn_nv() {
    return (const void*)&gemvdev::gemv_batched_kernel<D, NV, gemvplan::batched_rows(NV),
                                                      gemvplan::kBatchedBatch, VEC>;
}

template <class D, bool VEC>
const void* batched_fn(int nvec) {
    switch (nvec) {
    case 1: return batched_fn_nv<D, 1, VEC>();
    case 2: return batched_fn_nv<D, 2, VEC>();
    case 3: return batched_fn_nv<D, 3, VEC>();
    case 4: return batched_fn_nv<D, 4, VEC>();
    case 5: return batched_fn_nv<D, 5, VEC>();
    case 6: return batched_fn_nv<D, 6, VEC>();
    case 7: return batched_fn_nv<D, 7, VEC>();
    case 8: return batched_fn_nv<D, 8, VEC>();
    case 9: return batched_fn_nv<D, 9, VEC>();
    case 10: return batched_fn_nv<D, 10, VEC>();
    case 11: return batched_fn_nv<D, 11, VEC>();
    case 12: return batched_fn_nv<D, 12, VEC>();
    case 13: return batched_fn_nv<D, 13, VEC>();
    case 14: return batched_fn_nv<D, 14, VEC>();
    case 15: return batched_fn_nv<D, 15, VEC>();
    case 16: return batched_fn_nv<D, 16, VEC>();
    default: return nullptr;
    }
}

// ---- family/type dispatch ------------------------------------------------

template <class D, bool VEC>
const void* kernel_for(const Plan& p, int nvec) {
    switch (p.family) {
    case gemvplan::ROWS_PER_WAVE:
    case gemvplan::WAVE_PER_ROW:
        return rows_fn<D, VEC>(p.lanes_per_row, p.row_tiles);
    case gemvplan::GROUP_PER_ROW:
        switch (p.batch) {
        case 1: return (const void*)&gemvdev::gemv_group_kernel<D, gemvplan::kGroupWaves, 1, VEC>;
        case 2: return (const void*)&gemvdev::gemv_group_kernel<D, gemvplan::kGroupWaves, 2, VEC>;
        case 4: return (const void*)&gemvdev::gemv_group_kernel<D, gemvplan::kGroupWaves, 4, VEC>;
        case 8: return (const void*)&gemvdev::gemv_group_kernel<D, gemvplan::kGroupWaves, 8, VEC>;
        default: return nullptr;
        }
    case gemvplan::BATCHED:
        if constexpr (D::bytes == 2) return batched_fn<D, VEC>(nvec);
        return nullptr;
    case gemvplan::BATCHED_MFMA:
        if constexpr (D::bytes == 2 && VEC)
            return (const void*)&gemvdev::gemv_batched_mfma_kernel<D, gemvplan::kMfmaWaves,
                                                                   gemvplan::kMfmaChunk>;
        return nullptr;
    default:
        return nullptr;
    }
}

template <class D>
const void* kernel_for(const Plan& p, int nvec) {
    return p.vector_loads ? kernel_for<D, true>(p, nvec) : kernel_for<D, false>(p, nvec);
}

static_assert(gemvplan::kBlock == gemvdev::kRowsWaves * 64,
              "the planner's workgroup size is the one the rows kernels are compiled for");

gemv_status_t run(int dtype, int family, const void* A, int lda, const void* X,
                  const float* bias, float* Y, int M, int K, int nvec,
                  hipStream_t stream) {
    if (gemvplan::validate(dtype, M, K, lda, nvec, (uintptr_t)A, (uintptr_t)X,
                           (uintptr_t)bias, (uintptr_t)Y) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    if (M == 0) return GEMV_SUCCESS;
    Plan p;
    if (gemvplan::make_plan(dtype, M, K, lda, nvec, (uintptr_t)A, (uintptr_t)X, family, &p) !=
        gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    const void* fn = nullptr;
    switch (dtype) {
    case gemvplan::F32: fn = kernel_for<TF32>(p, nvec); break;
    case gemvplan::F16: fn = kernel_for<TF16>(p, nvec); break;
    case gemvplan::BF16: fn = kernel_for<TBF16>(p, nvec); break;
    default: break;
    }
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
    const Args args{A, (int64_t)lda, X, bias, Y, M, K, nvec};
    const hipError_t err = launch(fn, p, stream, args);
    if (err != hipSuccess) {
        g_last_launch_error = err;
        return GEMV_ERROR_LAUNCH_FAILURE;
    }
    return GEMV_SUCCESS;
}

}  // namespace

extern "C" {

const char* gemv_status_string(gemv_status_t status) {
    switch (status) {
    case GEMV_SUCCESS: return "GEMV_SUCCESS: the kernel was enqueued (or there was nothing to do)";
    case GEMV_ERROR_INVALID_VALUE: return "GEMV_ERROR_INVALID_VALUE: an argument is out of range, NULL or misaligned; nothing was enqueued";
    case GEMV_ERROR_LAUNCH_FAILURE: return "GEMV_ERROR_LAUNCH_FAILURE: the HIP runtime refused the kernel launch";
    default: return "unknown gemv_status_t value";
    }
}

int gemv_last_hip_error(void) { return (int)g_last_launch_error; }

const char* gemv_last_hip_error_string(void) { return hipGetErrorName(g_last_launch_error); }

gemv_status_t gemv_f32(const float* A, int lda, const float* x, const float* bias, float* y,
                       int M, int K, hipStream_t stream) {
    return run(gemvplan::F32, gemvplan::AUTO, A, lda, x, bias, y, M, K, 1, stream);
}

gemv_status_t gemv_f16(const uint16_t* A, int lda, const uint16_t* x, const float* bias,
                       float* y, int M, int K, hipStream_t stream) {
    return run(gemvplan::F16, gemvplan::AUTO, A, lda, x, bias, y, M, K, 1, stream);
}

gemv_status_t gemv_bf16(const uint16_t* A, int lda, const uint16_t* x, const float* bias,
                        float* y, int M, int K, hipStream_t stream) {
    return run(gemvplan::BF16, gemvplan::AUTO, A, lda, x, bias, y, M, K, 1, stream);
}

gemv_status_t gemv_batched_f16(const uint16_t* A, int lda, const uint16_t* X, const float* bias,
                               float* Y, int M, int K, int nvec, hipStream_t stream) {
    return run(gemvplan::F16, gemvplan::AUTO, A, lda, X, bias, Y, M, K, nvec, stream);
}

gemv_status_t gemv_batched_bf16(const uint16_t* A, int lda, const uint16_t* X, const float* bias,
                                float* Y, int M, int K, int nvec, hipStream_t stream) {
    return run(gemvplan::BF16, gemvplan::AUTO, A, lda, X, bias, Y, M, K, nvec, stream);
}

gemv_status_t gemv_plan(gemv_dtype_t dtype, int M, int K, int lda, int nvec, const void* A,
                        const void* X, int family, gemv_plan_t* plan) {
    if (plan == nullptr) return GEMV_ERROR_INVALID_VALUE;
    Plan p;
    if (gemvplan::make_plan((int)dtype, M, K, lda, nvec, (uintptr_t)A, (uintptr_t)X, family,
                            &p) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    plan->family = p.family;
    plan->vector_loads = p.vector_loads;
    plan->chunk_elems = p.chunk_elems;
    plan->lanes_per_row = p.lanes_per_row;
    plan->rows_per_wave = p.rows_per_wave;
    plan->row_tiles = p.row_tiles;
    plan->waves_per_group = p.waves_per_group;
    plan->rows_per_group = p.rows_per_group;
    plan->batch = p.batch;
    plan->passes = p.passes;
    plan->block = p.block;
    plan->lds_bytes = p.lds_bytes;
    plan->grid = p.grid;
    return GEMV_SUCCESS;
}

gemv_status_t gemv_run_family(gemv_dtype_t dtype, int family, const void* A, int lda,
                              const void* X, const float* bias, float* Y, int M, int K,
                              int nvec, hipStream_t stream) {
    return run((int)dtype, family, A, lda, X, bias, Y, M, K, nvec, stream);
}

}  // extern "C"
