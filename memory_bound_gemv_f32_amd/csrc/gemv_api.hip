// libgemv C ABI: argument validation, mapping selection and kernel launch.
//
// The launcher shape follows page "第 3 课：GEMV 与行级并行", section "实践任务"
// (a host function taking A, x, bias, y, M, N and a stream), with an explicit
// row pitch, status codes instead of unchecked launches, and the mapping
// chosen by row length and row count (gemv_plan.hpp).
#include <hip/hip_runtime.h>

#include <mutex>
#include <type_traits>

#include "../../include/gemv.h"
#include "gemv_kernels.hpp"
#include "gemv_plan.hpp"

namespace {

thread_local hipError_t g_last_launch_error = hipSuccess;

using gemvdev::Segments;
using gemvdev::TBF16;
using gemvdev::TF16;
using gemvdev::TF32;
using gemvplan::Plan;

static_assert(gemvplan::kBlock == gemvdev::kRowsWaves * 64,
              "the planner's workgroup size is the one the rows kernels are compiled for");
static_assert(GEMV_MAX_SEGMENTS == gemvdev::kMaxSegments, "segment table size");

template <class D>
constexpr int dtype_code() {
    return std::is_same<D, TF32>::value ? gemvplan::F32
           : std::is_same<D, TF16>::value ? gemvplan::F16 : gemvplan::BF16;
}

hipError_t launch(const void* fn, const Plan& p, hipStream_t stream, void** argv) {
    return hipLaunchKernel(fn, dim3((unsigned)p.grid), dim3((unsigned)p.block), argv, 0, stream);
}

gemv_status_t finish(hipError_t err) {
    if (err != hipSuccess) {
        g_last_launch_error = err;
        // the runtime also keeps the error as the thread's "last error";
        // reported here, it is cleared there, so that it does not surface
        // later as the failure of someone else's unrelated call
        (void)hipGetLastError();
        return GEMV_ERROR_LAUNCH_FAILURE;
    }
    return GEMV_SUCCESS;
}

// ---- rows-per-wave / wave-per-row / workgroup-per-row ----------------------

// NSEG selects the kernels for several matrices sharing x: 0 the one-matrix
// kernels, kFewSegments the kernels that take up to three segments as scalar
// arguments, any other value the segment-table kernels whose select chains
// cover NSEG entries.
// one wavefront per row: B loads per lane in flight per batch
template <class D, bool VEC, int NSEG, int B>
const void* wave_fn_b() {
    if constexpr (NSEG == gemvdev::kFewSegments)
        return (const void*)&gemvdev::gemv_rows_multi3_kernel<D, 64, 1, B, VEC>;
    else if constexpr (NSEG > 0)
        return (const void*)&gemvdev::gemv_rows_multi_kernel<D, 64, 1, B, VEC, NSEG>;
    else
        return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, B, VEC>;
}

// several rows per wavefront (U row tiles, U·B <= 8 loads per lane in
// flight), one matrix only
template <class D, bool VEC>
const void* wave_tiles_fn(int tiles, int batch) {
    switch (tiles * 16 + batch) {
    case 2 * 16 + 1: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 2, 1, VEC>;
    case 2 * 16 + 2: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 2, 2, VEC>;
    case 2 * 16 + 3: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 2, 3, VEC>;
    case 2 * 16 + 4: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 2, 4, VEC>;
    case 4 * 16 + 1: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 4, 1, VEC>;
    case 4 * 16 + 2: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 4, 2, VEC>;
    case 8 * 16 + 1: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 8, 1, VEC>;
    default: return nullptr;
    }
}

template <class D, bool VEC, int NSEG>
const void* wave_fn(int batch) {
    static_assert(gemvplan::kWaveBatch == 8, "wave-per-row kernels are built for batches of 1 to 8");
    switch (batch) {
    case 1: return wave_fn_b<D, VEC, NSEG, 1>();
    case 2: return wave_fn_b<D, VEC, NSEG, 2>();
    case 3: return wave_fn_b<D, VEC, NSEG, 3>();
    case 4: return wave_fn_b<D, VEC, NSEG, 4>();
    case 5: return wave_fn_b<D, VEC, NSEG, 5>();
    case 6: return wave_fn_b<D, VEC, NSEG, 6>();
    case 7: return wave_fn_b<D, VEC, NSEG, 7>();
    case 8: return wave_fn_b<D, VEC, NSEG, 8>();
    default: return nullptr;
    }
}

template <class D, int L, bool VEC, int NSEG>
const void* rows_fn(int tiles, int batch) {
    if constexpr (L == 64) {
        // one wavefront per row
        if (tiles == 1) return wave_fn<D, VEC, NSEG>(batch);
        if constexpr (NSEG == 0) return wave_tiles_fn<D, VEC>(tiles, batch);
        return nullptr;
    } else if constexpr (NSEG > 0) {
        // per-lane segment lookups cost registers: at most two row tiles
        if constexpr (NSEG == gemvdev::kFewSegments) {
            switch (tiles) {
            case 1: return (const void*)&gemvdev::gemv_rows_multi3_kernel<D, L, 1, 1, VEC>;
            case 2: return (const void*)&gemvdev::gemv_rows_multi3_kernel<D, L, 2, 1, VEC>;
            default: return nullptr;
            }
        }
        switch (tiles) {
        case 1: return (const void*)&gemvdev::gemv_rows_multi_kernel<D, L, 1, 1, VEC, NSEG>;
        case 2: return (const void*)&gemvdev::gemv_rows_multi_kernel<D, L, 2, 1, VEC, NSEG>;
        default: return nullptr;
        }
    } else {
        // rows of a load count that is not a power of two: several loads
        // per lane, one row tile
        if (batch > 1) {
            if constexpr (L >= gemvplan::kRowsMinSplitLanes && L < 32 && VEC) {
                static_assert(gemvplan::kRowsMaxBatch == 6, "split rows are built for batches of 2 to 6");
                if (tiles != 1) return nullptr;
                switch (batch) {
                case 2: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 1, 2, VEC>;
                case 3: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 1, 3, VEC>;
                case 4: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 1, 4, VEC>;
                case 5: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 1, 5, VEC>;
                case 6: return (const void*)&gemvdev::gemv_rows_kernel<D, L, 1, 6, VEC>;
                default: return nullptr;
                }
            }
            return nullptr;
        }
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

template <class D, bool VEC, int NSEG>
const void* rows_fn(int lanes, int tiles, int batch) {
    // several rows per wavefront: one load per lane per row tile, or (rows
    // of a load count that is not a power of two) several, one row tile
    switch (lanes) {
    case 1: return rows_fn<D, 1, VEC, NSEG>(tiles, batch);
    case 2: return rows_fn<D, 2, VEC, NSEG>(tiles, batch);
    case 4: return rows_fn<D, 4, VEC, NSEG>(tiles, batch);
    case 8: return rows_fn<D, 8, VEC, NSEG>(tiles, batch);
    case 16: return rows_fn<D, 16, VEC, NSEG>(tiles, batch);
    case 32: return rows_fn<D, 32, VEC, NSEG>(tiles, batch);
    case 64: return rows_fn<D, 64, VEC, NSEG>(tiles, batch);
    default: return nullptr;
    }
}

template <class D, bool VEC, int NSEG, int B>
const void* group_fn_b(int rows, int waves) {
    constexpr int W = gemvplan::kGroupWaves;
    // few long rows (plain GEMV only): 16 wavefronts for one row, 8 for two
    if (waves != W) {
        if constexpr (NSEG == 0) {
            constexpr int W1 = gemvplan::kGroupWideWaves, W2 = gemvplan::kGroupWidePairWaves;
            if (waves == W1 && rows == 1)
                return (const void*)&gemvdev::gemv_group_kernel<D, W1, 1, B, VEC>;
            if constexpr (2 * B <= gemvplan::kGroupTileLoads)
                if (waves == W2 && rows == 2)
                    return (const void*)&gemvdev::gemv_group_kernel<D, W2, 2, B, VEC>;
        }
        return nullptr;
    }
    if constexpr (NSEG == gemvdev::kFewSegments) {
        return rows == 1 ? (const void*)&gemvdev::gemv_group_multi3_kernel<D, W, B, VEC> : nullptr;
    } else if constexpr (NSEG > 0) {
        return rows == 1 ? (const void*)&gemvdev::gemv_group_multi_kernel<D, W, B, VEC, NSEG> : nullptr;
    } else {
        switch (rows) {
        case 1: return (const void*)&gemvdev::gemv_group_kernel<D, W, 1, B, VEC>;
        case 2:
            static_assert(gemvplan::kGroupMaxTileRows == 2, "group kernels are built for 1 or 2 rows");
            if constexpr (2 * B <= gemvplan::kGroupTileLoads)
                return (const void*)&gemvdev::gemv_group_kernel<D, W, 2, B, VEC>;
            return nullptr;
        default: return nullptr;
        }
    }
}

template <class D, bool VEC, int NSEG>
const void* group_fn(int batch, int rows, int waves) {
    static_assert(gemvplan::kGroupBatch == 8, "workgroup-per-row kernels are built for batches of 1 to 8");
    switch (batch) {
    case 1: return group_fn_b<D, VEC, NSEG, 1>(rows, waves);
    case 2: return group_fn_b<D, VEC, NSEG, 2>(rows, waves);
    case 3: return group_fn_b<D, VEC, NSEG, 3>(rows, waves);
    case 4: return group_fn_b<D, VEC, NSEG, 4>(rows, waves);
    case 5: return group_fn_b<D, VEC, NSEG, 5>(rows, waves);
    case 6: return group_fn_b<D, VEC, NSEG, 6>(rows, waves);
    case 7: return group_fn_b<D, VEC, NSEG, 7>(rows, waves);
    case 8: return group_fn_b<D, VEC, NSEG, 8>(rows, waves);
    default: return nullptr;
    }
}

// workgroup per row with x in registers: NX chunks of x per lane, R rows
template <class D, int NX>
const void* group_stream_fn_nx(int rows) {
    constexpr int W = gemvplan::kGroupStreamWaves;
    static_assert(gemvplan::kGroupStreamRows == 4, "streaming kernels are built for 2 or 4 rows");
    switch (rows) {
    case 2: return (const void*)&gemvdev::gemv_group_stream_kernel<D, W, NX, 2>;
    case 4: return (const void*)&gemvdev::gemv_group_stream_kernel<D, W, NX, 4>;
    default: return nullptr;
    }
}

template <class D>
const void* group_stream_fn(int chunks, int rows) {
    // x longer than 8 KiB: at least 3 chunks per lane of 4 wavefronts
    static_assert(gemvplan::kGroupStreamMaxChunks == 6, "streaming kernels hold up to 6 x chunks");
    switch (chunks) {
    case 3: return group_stream_fn_nx<D, 3>(rows);
    case 4: return group_stream_fn_nx<D, 4>(rows);
    case 5: return group_stream_fn_nx<D, 5>(rows);
    case 6: return group_stream_fn_nx<D, 6>(rows);
    default: return nullptr;
    }
}

// one row per wavefront, workgroups of kNarrowRowsWaves wavefronts (one
// matrix, one row tile, 16-byte loads)
template <class D>
const void* narrow_wave_fn(int batch) {
    constexpr int NW = gemvplan::kNarrowRowsWaves;
    switch (batch) {
    case 1: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 1, true, NW>;
    case 2: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 2, true, NW>;
    case 3: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 3, true, NW>;
    case 4: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 4, true, NW>;
    case 5: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 5, true, NW>;
    case 6: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 6, true, NW>;
    case 7: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 7, true, NW>;
    case 8: return (const void*)&gemvdev::gemv_rows_kernel<D, 64, 1, 8, true, NW>;
    default: return nullptr;
    }
}

template <class D, bool VEC, int NSEG>
const void* single_fn(const Plan& p) {
    switch (p.family) {
    case gemvplan::ROWS_PER_WAVE:
    case gemvplan::WAVE_PER_ROW:
        if (p.waves_per_group == gemvplan::kNarrowRowsWaves) {
            if constexpr (NSEG == 0 && VEC)
                if (p.family == gemvplan::WAVE_PER_ROW && p.row_tiles == 1) return narrow_wave_fn<D>(p.batch);
            return nullptr;
        }
        if (p.waves_per_group != gemvdev::kRowsWaves) return nullptr;
        return rows_fn<D, VEC, NSEG>(p.lanes_per_row, p.row_tiles, p.batch);
    case gemvplan::GROUP_PER_ROW:
        if (p.x_in_registers) {
            if constexpr (NSEG == 0 && VEC) return group_stream_fn<D>(p.batch, p.row_tiles);
            return nullptr;
        }
        return group_fn<D, VEC, NSEG>(p.batch, p.row_tiles, p.waves_per_group);
    default: return nullptr;
    }
}

template <class D, int NSEG>
const void* single_fn(const Plan& p) {
    return p.vector_loads ? single_fn<D, true, NSEG>(p) : single_fn<D, false, NSEG>(p);
}

// ---- batched ----------------------------------------------------------------

template <class D, int NV, int R, bool VEC, int KS>
const void* batched_fn_nv() {
    constexpr int B = gemvplan::batched_batch(NV);
    constexpr int E = VEC ? gemvplan::kLoadBytes / D::bytes : 1;
    return (const void*)&gemvdev::gemv_batched_kernel<D, NV, R, B, gemvplan::batched_x_ahead(NV), VEC,
                                                      gemvplan::batched_run(NV, B, E), KS>;
}

template <class D, int R, bool VEC, int KS = 1>
const void* batched_fn(int nvec) {
    switch (nvec) {
    case 1: return batched_fn_nv<D, 1, R, VEC, KS>();
    case 2: return batched_fn_nv<D, 2, R, VEC, KS>();
    case 3: return batched_fn_nv<D, 3, R, VEC, KS>();
    case 4: return batched_fn_nv<D, 4, R, VEC, KS>();
    case 5: return batched_fn_nv<D, 5, R, VEC, KS>();
    case 6: return batched_fn_nv<D, 6, R, VEC, KS>();
    case 7: return batched_fn_nv<D, 7, R, VEC, KS>();
    case 8: return batched_fn_nv<D, 8, R, VEC, KS>();
    case 9: return batched_fn_nv<D, 9, R, VEC, KS>();
    case 10: return batched_fn_nv<D, 10, R, VEC, KS>();
    case 11: return batched_fn_nv<D, 11, R, VEC, KS>();
    case 12: return batched_fn_nv<D, 12, R, VEC, KS>();
    case 13: return batched_fn_nv<D, 13, R, VEC, KS>();
    case 14: return batched_fn_nv<D, 14, R, VEC, KS>();
    case 15: return batched_fn_nv<D, 15, R, VEC, KS>();
    case 16: return batched_fn_nv<D, 16, R, VEC, KS>();
    default: return nullptr;
    }
}

static_assert(gemvplan::kBatchedSplit == gemvdev::kRowsWaves && gemvplan::kBlock == gemvdev::kRowsWaves * 64,
              "the K-split batched form splits each row over the workgroup's wavefronts");

// R rows per wavefront (1 or 2), or one row per workgroup whose wavefronts
// split K (lanes per row 64·kBatchedSplit), from the plan
template <class D, bool VEC>
const void* batched_fn(int nvec, int rows, int lanes) {
    if (lanes == gemvplan::kWave * gemvplan::kBatchedSplit && rows == 1)
        return batched_fn<D, 1, VEC, gemvplan::kBatchedSplit>(nvec);
    if (lanes == gemvplan::kWave * 2 && rows == 1) return batched_fn<D, 1, VEC, 2>(nvec);
    if (lanes != gemvplan::kWave) return nullptr;
    if (rows == 1) return batched_fn<D, 1, VEC>(nvec);
    if (rows == 2) return batched_fn<D, 2, VEC>(nvec);
    return nullptr;
}

// matrix-core kernels of W wavefronts and Q groups of RG rows per workgroup
template <class D, int W, int Q, int RG>
const void* mfma_fn(int nvec) {
    if constexpr (Q == 4) {
        // four groups: one tile of vectors staged in LDS, half-size chunks
        if (nvec > gemvplan::kMfmaFewVectors && gemvplan::mfma_tiles(nvec) == 1)
            return (const void*)&gemvdev::gemv_batched_mfma_kernel<D, W, 1, gemvplan::mfma_chunk(16, 4),
                                                                   false, Q, RG>;
        return nullptr;
    } else {
        if (nvec <= gemvplan::kMfmaFewVectors) {
            // (groups of 4 rows only with X staged in LDS)
            if constexpr (RG == 8)
                return (const void*)&gemvdev::gemv_batched_mfma_kernel<D, W, 1, gemvplan::mfma_chunk(16), true, Q, RG>;
            return nullptr;
        }
        switch (gemvplan::mfma_tiles(nvec)) {
        case 1: return (const void*)&gemvdev::gemv_batched_mfma_kernel<D, W, 1, gemvplan::mfma_chunk(16), false, Q, RG>;
        case 2: return (const void*)&gemvdev::gemv_batched_mfma_kernel<D, W, 2, gemvplan::mfma_chunk(32), false, Q, RG>;
        case 4: return (const void*)&gemvdev::gemv_batched_mfma_kernel<D, W, 4, gemvplan::mfma_chunk(64), false, Q, RG>;
        default: return nullptr;
        }
    }
}
template <class D, int W>
const void* mfma_fn(int nvec, int groups, int rows) {
    if (groups == 2 && rows == 16) return mfma_fn<D, W, 2, 8>(nvec);
    if (groups == 1 && rows == 8) return mfma_fn<D, W, 1, 8>(nvec);
    // four groups only with more workgroups than compute units
    if constexpr (W == gemvplan::kMfmaManyTilesWaves)
        if (groups == 4 && rows == 32) return mfma_fn<D, W, 4, 8>(nvec);
    // one group of 4 rows only at one workgroup per compute unit or fewer
    if constexpr (W == gemvplan::kMfmaWaves)
        if (groups == 1 && rows == 4) return mfma_fn<D, W, 1, 4>(nvec);
    return nullptr;
}

template <class D>
const void* batched_kernel(const Plan& p, int nvec) {
    if constexpr (D::bytes == 2) {
        if (p.family == gemvplan::BATCHED)
            return p.vector_loads ? batched_fn<D, true>(nvec, p.rows_per_wave, p.lanes_per_row)
                                  : batched_fn<D, false>(nvec, p.rows_per_wave, p.lanes_per_row);
        if (p.family == gemvplan::BATCHED_MFMA && p.vector_loads) {
            if (p.waves_per_group == gemvplan::kMfmaWaves)
                return mfma_fn<D, gemvplan::kMfmaWaves>(nvec, p.row_tiles, p.rows_per_group);
            if (p.waves_per_group == gemvplan::kMfmaManyTilesWaves)
                return mfma_fn<D, gemvplan::kMfmaManyTilesWaves>(nvec, p.row_tiles, p.rows_per_group);
        }
    }
    return nullptr;
}

// ---- gated pair ---------------------------------------------------------------

template <class D, int W, bool VEC>
const void* gated_fn(int batch) {
    switch (batch) {
    case 1: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 1, VEC>;
    case 2: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 2, VEC>;
    case 3: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 3, VEC>;
    case 4: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 4, VEC>;
    case 5: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 5, VEC>;
    case 6: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 6, VEC>;
    case 7: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 7, VEC>;
    case 8: return (const void*)&gemvdev::gemv_gated_silu_kernel<D, W, 8, VEC>;
    default: return nullptr;
    }
}

template <class D>
const void* gated_kernel(const Plan& p) {
    if (p.waves_per_group == 1)
        return p.vector_loads ? gated_fn<D, 1, true>(p.batch) : gated_fn<D, 1, false>(p.batch);
    if (p.waves_per_group == gemvplan::kGroupWaves)
        return p.vector_loads ? gated_fn<D, gemvplan::kGroupWaves, true>(p.batch)
                              : gated_fn<D, gemvplan::kGroupWaves, false>(p.batch);
    return nullptr;
}

// ---- int8 weights ------------------------------------------------------------

template <class X, int L, bool VEC>
const void* q8_rows_fn(int tiles, int batch) {
    if constexpr (L == 64) {
        if (tiles != 1 && tiles != 2) return nullptr;
        switch (batch * 4 + tiles) {
        case 1 * 4 + 1: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 1, 1, VEC>;
        case 2 * 4 + 1: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 1, 2, VEC>;
        case 3 * 4 + 1: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 1, 3, VEC>;
        case 4 * 4 + 1: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 1, 4, VEC>;
        case 1 * 4 + 2: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 2, 1, VEC>;
        case 2 * 4 + 2: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 2, 2, VEC>;
        case 3 * 4 + 2: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 2, 3, VEC>;
        case 4 * 4 + 2: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, 64, 2, 4, VEC>;
        default: return nullptr;
        }
    } else {
        if (batch != 1) return nullptr;
        switch (tiles) {
        case 1: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, L, 1, 1, VEC>;
        case 2: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, L, 2, 1, VEC>;
        case 4: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, L, 4, 1, VEC>;
        case 8: return (const void*)&gemvdev::gemv_rows_q8_kernel<X, L, 8, 1, VEC>;
        default: return nullptr;
        }
    }
}

template <class X, int U, bool VEC, int W = gemvplan::kGroupWaves>
const void* q8_group_fn(int batch) {
    switch (batch) {
    case 1: return (const void*)&gemvdev::gemv_group_q8_kernel<X, W, U, 1, VEC>;
    case 2: return (const void*)&gemvdev::gemv_group_q8_kernel<X, W, U, 2, VEC>;
    case 3: return (const void*)&gemvdev::gemv_group_q8_kernel<X, W, U, 3, VEC>;
    case 4: return (const void*)&gemvdev::gemv_group_q8_kernel<X, W, U, 4, VEC>;
    default: return nullptr;
    }
}

// int8 weights, x in registers: NX chunks of x per lane (at most
// kQ8StreamMaxChunks, or kQ8StreamMaxChunksWideX of fp32 x), R rows
template <class X, int NX>
const void* q8_stream_fn_nx(int rows) {
    constexpr int W = gemvplan::kGroupStreamWaves;
    if constexpr (NX > (X::bytes == 4 ? gemvplan::kQ8StreamMaxChunksWideX : gemvplan::kQ8StreamMaxChunks)) {
        return nullptr;
    } else {
        switch (rows) {
        case 2: return (const void*)&gemvdev::gemv_group_stream_q8_kernel<X, W, NX, 2>;
        case 4: return (const void*)&gemvdev::gemv_group_stream_q8_kernel<X, W, NX, 4>;
        default: return nullptr;
        }
    }
}
template <class X>
const void* q8_stream_fn(int chunks, int rows) {
    static_assert(gemvplan::kQ8StreamMaxChunks == 4, "int8 streaming kernels hold up to 4 x chunks");
    switch (chunks) {
    case 1: return q8_stream_fn_nx<X, 1>(rows);
    case 2: return q8_stream_fn_nx<X, 2>(rows);
    case 3: return q8_stream_fn_nx<X, 3>(rows);
    case 4: return q8_stream_fn_nx<X, 4>(rows);
    default: return nullptr;
    }
}

template <class X, bool VEC>
const void* q8_fn(const Plan& p) {
    if (p.family == gemvplan::GROUP_PER_ROW) {
        if (p.x_in_registers) {
            if constexpr (VEC) return q8_stream_fn<X>(p.batch, p.row_tiles);
            return nullptr;
        }
        if (p.waves_per_group == gemvplan::kGroupWaves) {
            if (p.row_tiles == 1) return q8_group_fn<X, 1, VEC>(p.batch);
            // two rows per workgroup only with 16-byte loads
            if constexpr (VEC)
                if (p.row_tiles == 2) return q8_group_fn<X, 2, VEC>(p.batch);
        }
        // narrow workgroups (one row, 16-byte loads)
        if constexpr (VEC)
            if (p.waves_per_group == gemvplan::kQ8NarrowWaves && p.row_tiles == 1)
                return q8_group_fn<X, 1, VEC, gemvplan::kQ8NarrowWaves>(p.batch);
        return nullptr;
    }
    if (p.family != gemvplan::ROWS_PER_WAVE && p.family != gemvplan::WAVE_PER_ROW) return nullptr;
    switch (p.lanes_per_row) {
    case 1: return q8_rows_fn<X, 1, VEC>(p.row_tiles, p.batch);
    case 2: return q8_rows_fn<X, 2, VEC>(p.row_tiles, p.batch);
    case 4: return q8_rows_fn<X, 4, VEC>(p.row_tiles, p.batch);
    case 8: return q8_rows_fn<X, 8, VEC>(p.row_tiles, p.batch);
    case 16: return q8_rows_fn<X, 16, VEC>(p.row_tiles, p.batch);
    case 32: return q8_rows_fn<X, 32, VEC>(p.row_tiles, p.batch);
    case 64: return q8_rows_fn<X, 64, VEC>(p.row_tiles, p.batch);
    default: return nullptr;
    }
}

// ---- split-K ------------------------------------------------------------------

template <class D, int U, bool VEC>
const void* splitk_fn_u(int batch) {
    switch (batch) {
    case 1: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 1, VEC>;
    case 2: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 2, VEC>;
    case 3: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 3, VEC>;
    case 4: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 4, VEC>;
    case 5: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 5, VEC>;
    case 6: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 6, VEC>;
    case 7: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 7, VEC>;
    case 8: return (const void*)&gemvdev::gemv_splitk_partial_kernel<D, U, 8, VEC>;
    default: return nullptr;
    }
}

template <class D, bool VEC>
const void* splitk_fn(int rows, int batch) {
    static_assert(gemvplan::kSplitRowsPerGroup == 2, "split-K is instantiated for 1 and 2 rows");
    switch (rows) {
    case 1: return splitk_fn_u<D, 1, VEC>(batch);
    case 2: return splitk_fn_u<D, 2, VEC>(batch);
    default: return nullptr;
    }
}

static_assert(gemvplan::kQ8Batch == 4, "the int8 kernels are instantiated for batches 1 to 4");
static_assert(gemvplan::kGroupWaves == gemvdev::kGroupWavesDev,
              "the planner's split-K workgroup is the one the kernel is compiled for");

// ---- entry points -------------------------------------------------------------

template <class D>
gemv_status_t run_single(const Plan& p, const void* A, int lda, const void* X, const float* bias,
                         float* Y, int M, int K, int nvec, hipStream_t stream) {
    if (p.family == gemvplan::BATCHED_MFMA) {
        // one launch, or (long rows and more than 32 vectors) one per block of
        // 32 vectors: columns j0 .. j0 + nb - 1 start at X + j0·K and Y + j0·M
        using S = typename D::storage;
        const int per = p.column_blocks > 1 ? (nvec + p.column_blocks - 1) / p.column_blocks : nvec;
        for (int j0 = 0; j0 < nvec; j0 += per) {
            int nb = nvec - j0 < per ? nvec - j0 : per;
            const void* fn = batched_kernel<D>(p, nb);
            if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
            int64_t lda64 = lda;
            const S* Xb = static_cast<const S*>(X) + (int64_t)j0 * K;
            float* Yb = Y + (int64_t)j0 * M;
            void* argv[] = {(void*)&A, (void*)&lda64, (void*)&Xb, (void*)&bias, (void*)&Yb,
                            (void*)&M, (void*)&K, (void*)&nb};
            const gemv_status_t st = finish(launch(fn, p, stream, argv));
            if (st != GEMV_SUCCESS) return st;
        }
        return GEMV_SUCCESS;
    }
    if (p.family == gemvplan::BATCHED) {
        // column blocks of at most kValuVectors vectors, one launch each
        // (X and Y columns j0 .. j0 + nv - 1 start at X + j0·K and Y + j0·M)
        using S = typename D::storage;
        for (int j0 = 0; j0 < nvec; j0 += gemvplan::kValuVectors) {
            int nv = nvec - j0 < gemvplan::kValuVectors ? nvec - j0 : gemvplan::kValuVectors;
            Plan pb;
            if (gemvplan::make_plan_vec(dtype_code<D>(), M, K, nv,
                                        p.vector_loads != 0, gemvplan::BATCHED, &pb) != gemvplan::OK)
                return GEMV_ERROR_INVALID_VALUE;
            const void* fn = batched_kernel<D>(pb, nv);
            if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
            int64_t lda64 = lda, M64 = M;
            const S* Xb = static_cast<const S*>(X) + (int64_t)j0 * K;
            float* Yb = Y + (int64_t)j0 * M;
            void* argv[] = {(void*)&A, (void*)&lda64, (void*)&Xb, (void*)&bias, (void*)&Yb,
                            (void*)&M64, (void*)&K};
            const gemv_status_t st = finish(launch(fn, pb, stream, argv));
            if (st != GEMV_SUCCESS) return st;
        }
        return GEMV_SUCCESS;
    }
    const void* fn = single_fn<D, 0>(p);
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
    int64_t lda64 = lda, M64 = M;
    void* argv[] = {(void*)&A, (void*)&lda64, (void*)&bias, (void*)&Y, (void*)&M64, (void*)&X,
                    (void*)&K};
    return finish(launch(fn, p, stream, argv));
}

gemv_status_t run(int dtype, int family, const void* A, int lda, const void* X,
                  const float* bias, float* Y, int M, int K, int nvec,
                  hipStream_t stream) {
    // the gated and split-K families have entry points of their own
    if (family == gemvplan::GATED_SILU || family == gemvplan::SPLIT_K)
        return GEMV_ERROR_INVALID_VALUE;
    if (gemvplan::validate(dtype, M, K, lda, nvec, (uintptr_t)A, (uintptr_t)X,
                           (uintptr_t)bias, (uintptr_t)Y) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    if (M == 0) return GEMV_SUCCESS;
    Plan p;
    if (gemvplan::make_plan(dtype, M, K, lda, nvec, (uintptr_t)A, (uintptr_t)X, family, &p) !=
        gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    switch (dtype) {
    case gemvplan::F32: return run_single<TF32>(p, A, lda, X, bias, Y, M, K, nvec, stream);
    case gemvplan::F16: return run_single<TF16>(p, A, lda, X, bias, Y, M, K, nvec, stream);
    case gemvplan::BF16: return run_single<TBF16>(p, A, lda, X, bias, Y, M, K, nvec, stream);
    default: return GEMV_ERROR_INVALID_VALUE;
    }
}

template <class D, int NSEG>
gemv_status_t launch_multi(const gemv_segment_t* segs, int count, const void* x, int K, int total,
                           bool vec, hipStream_t stream) {
    using S = typename D::storage;
    Segments<S, NSEG> rows{};
    rows.x = static_cast<const S*>(x);
    rows.K = K;
    rows.M = total;
    int end = 0;
    for (int i = 0; i < count; ++i) {
        end += segs[i].M;
        rows.seg[i] = gemvdev::SegEntry<S>{static_cast<const S*>(segs[i].A), end, segs[i].lda};
        rows.bias[i] = segs[i].bias;
        rows.y[i] = segs[i].y;
    }
    // unused entries end at the last row, so no row selects the entry after them
    for (int i = count; i < gemvdev::kMaxSegments; ++i) rows.seg[i] = gemvdev::SegEntry<S>{nullptr, total, 0};
    Plan p;
    if (gemvplan::make_plan_vec(dtype_code<D>(), total, K, 1, vec, gemvplan::AUTO, &p,
                                gemvplan::kMultiMaxRowTiles, 1, 1, gemvplan::kGroupWaves) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    const void* fn = single_fn<D, NSEG>(p);
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
    void* argv[] = {(void*)&rows};
    return finish(launch(fn, p, stream, argv));
}

template <class D>
gemv_status_t launch_multi3(const gemv_segment_t* segs, int count, const void* x, int K, int total,
                            int lda, bool vec, hipStream_t stream) {
    using S = typename D::storage;
    // absent segments (count < 3) are empty: they end at the last row and are
    // never selected
    const S* A[3] = {nullptr, nullptr, nullptr};
    int end[3] = {total, total, total};
    const float* b[3] = {nullptr, nullptr, nullptr};
    float* y[3] = {nullptr, nullptr, nullptr};
    int e = 0;
    for (int i = 0; i < count; ++i) {
        e += segs[i].M;
        A[i] = static_cast<const S*>(segs[i].A);
        end[i] = e;
        b[i] = segs[i].bias;
        y[i] = segs[i].y;
    }
    Plan p;
    if (gemvplan::make_plan_vec(dtype_code<D>(), total, K, 1, vec, gemvplan::AUTO, &p,
                                gemvplan::kMultiMaxRowTiles, 1, 1, gemvplan::kGroupWaves) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    const void* fn = single_fn<D, gemvdev::kFewSegments>(p);
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
    const S* xs = static_cast<const S*>(x);
    int has_bias = b[0] != nullptr || b[1] != nullptr || b[2] != nullptr;
    void* argv[] = {(void*)&xs,   (void*)&A[0], (void*)&A[1],     (void*)&A[2], (void*)&end[0],
                    (void*)&end[1], (void*)&lda, (void*)&K,      (void*)&total, (void*)&has_bias,
                    (void*)&b[0], (void*)&b[1], (void*)&b[2],     (void*)&y[0], (void*)&y[1],
                    (void*)&y[2]};
    return finish(launch(fn, p, stream, argv));
}

template <class D>
gemv_status_t run_multi(const gemv_segment_t* segs, int count, const void* x, int K,
                        hipStream_t stream) {
    constexpr int dtype = dtype_code<D>();
    if (segs == nullptr || count < 1 || count > GEMV_MAX_SEGMENTS || K < 0)
        return GEMV_ERROR_INVALID_VALUE;
    int64_t total = 0;
    bool vec = ((uintptr_t)x % gemvplan::kLoadBytes) == 0;
    for (int i = 0; i < count; ++i) {
        const gemv_segment_t& s = segs[i];
        if (gemvplan::validate(dtype, s.M, K, s.lda, 1, (uintptr_t)s.A, (uintptr_t)x,
                               (uintptr_t)s.bias, (uintptr_t)s.y) != gemvplan::OK)
            return GEMV_ERROR_INVALID_VALUE;
        // a segment of one row never steps by its pitch: only its A pointer
        // must be aligned for 16-byte loads
        if (s.M > 1)
            vec = vec && gemvplan::vector_ok(dtype, K, s.lda, 1, (uintptr_t)s.A, (uintptr_t)x);
        else if (s.M == 1)
            vec = vec && ((uintptr_t)s.A % gemvplan::kLoadBytes) == 0;
        total += s.M;
    }
    if (total > 0x7fffffff) return GEMV_ERROR_INVALID_VALUE;
    if (total == 0) return GEMV_SUCCESS;
    // up to three segments with one row pitch (segments of at most one row
    // never step by theirs): the scalar-argument kernels
    int pitch = -1;
    bool one_pitch = true;
    for (int i = 0; i < count; ++i) {
        if (segs[i].M <= 1) continue;
        if (pitch < 0) pitch = segs[i].lda;
        one_pitch = one_pitch && segs[i].lda == pitch;
    }
    if (count <= gemvdev::kFewSegments && one_pitch)
        return launch_multi3<D>(segs, count, x, K, (int)total, pitch < 0 ? K : pitch, vec, stream);
    return launch_multi<D, gemvdev::kMaxSegments>(segs, count, x, K, (int)total, vec, stream);
}

template <class D>
gemv_status_t run_gated(const void* Ag, const void* Au, int lda, const void* x, float* h, int M,
                        int K, hipStream_t stream) {
    constexpr int dtype = dtype_code<D>();
    if (gemvplan::validate(dtype, M, K, lda, 1, (uintptr_t)Ag, (uintptr_t)x, 0, (uintptr_t)h) !=
            gemvplan::OK ||
        gemvplan::validate(dtype, M, K, lda, 1, (uintptr_t)Au, (uintptr_t)x, 0, (uintptr_t)h) !=
            gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    if (M == 0) return GEMV_SUCCESS;
    const bool vec = gemvplan::vector_ok(dtype, K, lda, 1, (uintptr_t)Ag, (uintptr_t)x) &&
                     gemvplan::vector_ok(dtype, K, lda, 1, (uintptr_t)Au, (uintptr_t)x);
    Plan p;
    if (gemvplan::make_plan_vec(dtype, M, K, 1, vec, gemvplan::GATED_SILU, &p) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    const void* fn = gated_kernel<D>(p);
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
    int64_t lda64 = lda, M64 = M;
    void* argv[] = {(void*)&Ag, (void*)&Au, (void*)&lda64, (void*)&h, (void*)&M64, (void*)&x,
                    (void*)&K};
    return finish(launch(fn, p, stream, argv));
}

// ---- scratch for the entry point that allocates nothing ---------------------
//
// gemv_splitk_noalloc keeps split-K's partial sums here instead of in a
// caller's workspace: a file-scope device array of kScratchBytes, of which
// every GPU the library runs on holds its own copy until the process ends.
// Its address on a device is looked up once (hipGetSymbolAddress, with that
// device current) and kept; host code uses only that address, never the
// array's name (which on the host is a stand-in, not a device address).
constexpr size_t kScratchBytes = 256 * 1024;
static_assert(kScratchBytes == GEMV_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device that `stream` belongs to (the current
// device for the null stream).
gemv_status_t device_scratch(hipStream_t stream, void** out) {
    int current = 0;
    hipError_t err = hipGetDevice(&current);
    if (err != hipSuccess) return finish(err);
    int dev = current;
    if (stream != nullptr) {
        hipDevice_t d = 0;
        err = hipStreamGetDevice(stream, &d);
        if (err != hipSuccess) return finish(err);
        dev = (int)d;
    }
    if (dev < 0 || dev >= kMaxDevices) return GEMV_ERROR_INVALID_VALUE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != current && (err = hipSetDevice(dev)) != hipSuccess) return finish(err);
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        const hipError_t back = dev != current ? hipSetDevice(current) : hipSuccess;
        if (err != hipSuccess) return finish(err);
        if (back != hipSuccess) return finish(back);
        if (p == nullptr) return GEMV_ERROR_LAUNCH_FAILURE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return GEMV_SUCCESS;
}

template <class D>
gemv_status_t run_splitk(const void* A, int lda, const void* x, const float* bias, float* y, int M,
                         int K, int splits, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    constexpr int dtype = dtype_code<D>();
    if (splits < 0 ||
        gemvplan::validate(dtype, M, K, lda, 1, (uintptr_t)A, (uintptr_t)x, (uintptr_t)bias,
                           (uintptr_t)y) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    if (M == 0) return GEMV_SUCCESS;
    const bool vec = gemvplan::vector_ok(dtype, K, lda, 1, (uintptr_t)A, (uintptr_t)x);
    Plan p;
    if (gemvplan::make_split_plan(dtype, M, K, vec, splits, &p) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    if (p.splits == 1) return run_single<D>(p, A, lda, x, bias, y, M, K, 1, stream);

    const int64_t need = gemvplan::split_workspace_bytes(M, p.splits);
    if (workspace == nullptr || (uintptr_t)workspace % sizeof(float) != 0 ||
        workspace_bytes < (size_t)need)
        return GEMV_ERROR_INVALID_VALUE;
    const void* fn = p.vector_loads ? splitk_fn<D, true>(p.rows_per_group, p.batch)
                                    : splitk_fn<D, false>(p.rows_per_group, p.batch);
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;

    float* ws = static_cast<float*>(workspace);
    int64_t lda64 = lda, M64 = M;
    int slice = p.slice_elems, nsplit = p.splits;
    void* argv1[] = {(void*)&A, (void*)&lda64, (void*)&ws, (void*)&M64, (void*)&x, (void*)&K,
                     (void*)&slice, (void*)&nsplit};
    hipError_t err = hipLaunchKernel(fn, dim3((unsigned)p.grid), dim3((unsigned)p.block), argv1, 0,
                                     stream);
    if (err != hipSuccess) return finish(err);
    const float* wsc = ws;
    void* argv2[] = {(void*)&wsc, (void*)&nsplit, (void*)&bias, (void*)&y, (void*)&M64};
    const unsigned groups = (unsigned)gemvplan::ceil_div(M, gemvdev::kRowsWaves);
    return finish(hipLaunchKernel((const void*)&gemvdev::gemv_splitk_reduce_kernel, dim3(groups),
                                  dim3(gemvdev::kRowsWaves * 64), argv2, 0, stream));
}

int q8_plan(int xdtype, int M, int K, int ldq, const void* Q, const void* x, int family, Plan* p) {
    if (xdtype < gemvplan::F32 || xdtype > gemvplan::BF16 || ldq < K) return gemvplan::INVALID;
    const bool vec = gemvplan::vector_ok_q8(ldq, (uintptr_t)Q, (uintptr_t)x);
    return gemvplan::make_plan_vec(gemvplan::Q8, M, K, 1, vec, family, p, 8, gemvplan::kGroupStreamRows,
                                   gemvplan::kWaveBatch, gemvplan::kGroupWideWaves, false,
                                   gemvplan::element_bytes(xdtype));
}

template <class X>
gemv_status_t run_q8(int family, const int8_t* Q, int ldq, const float* scale, const void* x,
                     const float* bias, float* y, int M, int K, hipStream_t stream) {
    constexpr int xdtype = dtype_code<X>();
    if (gemvplan::validate_q8(xdtype, M, K, ldq, (uintptr_t)Q, (uintptr_t)scale, (uintptr_t)x,
                              (uintptr_t)bias, (uintptr_t)y) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    if (M == 0) return GEMV_SUCCESS;
    Plan p;
    if (q8_plan(xdtype, M, K, ldq, Q, x, family, &p) != gemvplan::OK) return GEMV_ERROR_INVALID_VALUE;
    const void* fn = p.vector_loads ? q8_fn<X, true>(p) : q8_fn<X, false>(p);
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
    int64_t ldq64 = ldq, M64 = M;
    void* argv[] = {(void*)&Q, (void*)&ldq64, (void*)&x, (void*)&M64, (void*)&K, (void*)&scale,
                    (void*)&bias, (void*)&y};
    return finish(launch(fn, p, stream, argv));
}

void export_plan(const Plan& p, gemv_plan_t* plan) {
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
    plan->splits = p.splits;
    plan->slice_elems = p.slice_elems;
    plan->x_in_registers = p.x_in_registers;
    plan->rounding_chain = p.rounding_chain;
    plan->column_blocks = p.column_blocks;
    plan->grid = p.grid;
}

// Whether the library holds a compiled kernel for a plan (the host-side plan
// calls answer only for plans the entry points can launch).
template <class D>
bool has_kernel(const Plan& p, int nvec) {
    if (p.family == gemvplan::BATCHED_MFMA) {
        const int per = p.column_blocks > 1 ? (nvec + p.column_blocks - 1) / p.column_blocks : nvec;
        return batched_kernel<D>(p, per) != nullptr &&
               batched_kernel<D>(p, nvec - (p.column_blocks - 1) * per) != nullptr;
    }
    if (p.family == gemvplan::BATCHED)
        return batched_kernel<D>(p, nvec < gemvplan::kValuVectors ? nvec : gemvplan::kValuVectors) !=
               nullptr;
    return single_fn<D, 0>(p) != nullptr;
}

bool has_kernel(int dtype, const Plan& p, int nvec) {
    switch (dtype) {
    case gemvplan::F32: return has_kernel<TF32>(p, nvec);
    case gemvplan::F16: return has_kernel<TF16>(p, nvec);
    case gemvplan::BF16: return has_kernel<TBF16>(p, nvec);
    default: return false;
    }
}

bool has_q8_kernel(int xdtype, const Plan& p) {
    switch (xdtype) {
    case gemvplan::F32: return (p.vector_loads ? q8_fn<TF32, true>(p) : q8_fn<TF32, false>(p)) != nullptr;
    case gemvplan::F16: return (p.vector_loads ? q8_fn<TF16, true>(p) : q8_fn<TF16, false>(p)) != nullptr;
    case gemvplan::BF16: return (p.vector_loads ? q8_fn<TBF16, true>(p) : q8_fn<TBF16, false>(p)) != nullptr;
    default: return false;
    }
}

bool has_splitk_kernel(int dtype, const Plan& p) {
    if (p.family != gemvplan::SPLIT_K) return has_kernel(dtype, p, 1);
    switch (dtype) {
    case gemvplan::F32:
        return (p.vector_loads ? splitk_fn<TF32, true>(p.rows_per_group, p.batch)
                               : splitk_fn<TF32, false>(p.rows_per_group, p.batch)) != nullptr;
    case gemvplan::F16:
        return (p.vector_loads ? splitk_fn<TF16, true>(p.rows_per_group, p.batch)
                               : splitk_fn<TF16, false>(p.rows_per_group, p.batch)) != nullptr;
    case gemvplan::BF16:
        return (p.vector_loads ? splitk_fn<TBF16, true>(p.rows_per_group, p.batch)
                               : splitk_fn<TBF16, false>(p.rows_per_group, p.batch)) != nullptr;
    default: return false;
    }
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

gemv_status_t gemv_multi_f32(const gemv_segment_t* segments, int count, const float* x, int K,
                             hipStream_t stream) {
    return run_multi<TF32>(segments, count, x, K, stream);
}

gemv_status_t gemv_multi_f16(const gemv_segment_t* segments, int count, const uint16_t* x, int K,
                             hipStream_t stream) {
    return run_multi<TF16>(segments, count, x, K, stream);
}

gemv_status_t gemv_multi_bf16(const gemv_segment_t* segments, int count, const uint16_t* x,
                              int K, hipStream_t stream) {
    return run_multi<TBF16>(segments, count, x, K, stream);
}

gemv_status_t gemv_gate_up_silu_f32(const float* A_gate, const float* A_up, int lda,
                                    const float* x, float* h, int M, int K, hipStream_t stream) {
    return run_gated<TF32>(A_gate, A_up, lda, x, h, M, K, stream);
}

gemv_status_t gemv_gate_up_silu_f16(const uint16_t* A_gate, const uint16_t* A_up, int lda,
                                    const uint16_t* x, float* h, int M, int K,
                                    hipStream_t stream) {
    return run_gated<TF16>(A_gate, A_up, lda, x, h, M, K, stream);
}

gemv_status_t gemv_gate_up_silu_bf16(const uint16_t* A_gate, const uint16_t* A_up, int lda,
                                     const uint16_t* x, float* h, int M, int K,
                                     hipStream_t stream) {
    return run_gated<TBF16>(A_gate, A_up, lda, x, h, M, K, stream);
}

gemv_status_t gemv_q8_f32(const int8_t* Q, int ldq, const float* scale, const float* x,
                          const float* bias, float* y, int M, int K, hipStream_t stream) {
    return run_q8<TF32>(gemvplan::AUTO, Q, ldq, scale, x, bias, y, M, K, stream);
}

gemv_status_t gemv_q8_f16(const int8_t* Q, int ldq, const float* scale, const uint16_t* x,
                          const float* bias, float* y, int M, int K, hipStream_t stream) {
    return run_q8<TF16>(gemvplan::AUTO, Q, ldq, scale, x, bias, y, M, K, stream);
}

gemv_status_t gemv_q8_bf16(const int8_t* Q, int ldq, const float* scale, const uint16_t* x,
                           const float* bias, float* y, int M, int K, hipStream_t stream) {
    return run_q8<TBF16>(gemvplan::AUTO, Q, ldq, scale, x, bias, y, M, K, stream);
}

gemv_status_t gemv_q8_run_family(gemv_dtype_t xdtype, int family, const int8_t* Q, int ldq,
                                 const float* scale, const void* x, const float* bias, float* y,
                                 int M, int K, hipStream_t stream) {
    switch ((int)xdtype) {
    case gemvplan::F32: return run_q8<TF32>(family, Q, ldq, scale, x, bias, y, M, K, stream);
    case gemvplan::F16: return run_q8<TF16>(family, Q, ldq, scale, x, bias, y, M, K, stream);
    case gemvplan::BF16: return run_q8<TBF16>(family, Q, ldq, scale, x, bias, y, M, K, stream);
    default: return GEMV_ERROR_INVALID_VALUE;
    }
}

gemv_status_t gemv_plan_q8(gemv_dtype_t xdtype, int M, int K, int ldq, const void* Q,
                           const void* x, int family, gemv_plan_t* plan) {
    Plan p;
    if (plan == nullptr || M < 0 ||
        q8_plan((int)xdtype, M, K, ldq, Q, x, family, &p) != gemvplan::OK ||
        !has_q8_kernel((int)xdtype, p))
        return GEMV_ERROR_INVALID_VALUE;
    export_plan(p, plan);
    return GEMV_SUCCESS;
}

gemv_status_t gemv_read_probe(const void* buffer, size_t bytes, unsigned* sink,
                              hipStream_t stream) {
    if (bytes == 0) return GEMV_SUCCESS;
    if (buffer == nullptr || sink == nullptr || bytes % 16 != 0 ||
        (uintptr_t)buffer % 16 != 0 || (uintptr_t)sink % 4 != 0)
        return GEMV_ERROR_INVALID_VALUE;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t per_group = (int64_t)gemvdev::kRowsWaves * 8 * 64;  // 16-byte units
    Plan p;
    p.grid = (n16 + per_group - 1) / per_group;
    p.block = gemvdev::kRowsWaves * 64;
    if (p.grid > 0x7fffffff) return GEMV_ERROR_INVALID_VALUE;
    const gemvdev::quad* q = static_cast<const gemvdev::quad*>(buffer);
    void* argv[] = {(void*)&q, (void*)&n16, (void*)&sink};
    return finish(launch((const void*)&gemvdev::gemv_read_probe_kernel, p, stream, argv));
}

}  // extern "C"

namespace {

template <int LOADS, int W>
const void* probe_variant_fn(int flags) {
    switch (flags & 3) {
    case 0: return (const void*)&gemvdev::gemv_read_probe_variant_kernel<LOADS, W, false, false>;
    case 1: return (const void*)&gemvdev::gemv_read_probe_variant_kernel<LOADS, W, true, false>;
    case 2: return (const void*)&gemvdev::gemv_read_probe_variant_kernel<LOADS, W, false, true>;
    default: return (const void*)&gemvdev::gemv_read_probe_variant_kernel<LOADS, W, true, true>;
    }
}

template <int LOADS>
const void* probe_variant_fn(int waves, int flags) {
    switch (waves) {
    case 1: return probe_variant_fn<LOADS, 1>(flags);
    case 2: return probe_variant_fn<LOADS, 2>(flags);
    case 4: return probe_variant_fn<LOADS, 4>(flags);
    case 8: return probe_variant_fn<LOADS, 8>(flags);
    case 16: return probe_variant_fn<LOADS, 16>(flags);
    default: return nullptr;
    }
}

const void* probe_variant_fn(int loads, int waves, int flags) {
    switch (loads) {
    case 2: return probe_variant_fn<2>(waves, flags);
    case 4: return probe_variant_fn<4>(waves, flags);
    case 8: return probe_variant_fn<8>(waves, flags);
    case 16: return probe_variant_fn<16>(waves, flags);
    default: return nullptr;
    }
}

}  // namespace

extern "C" {

gemv_status_t gemv_read_probe_variant(const void* buffer, size_t bytes, unsigned* sink,
                                      int loads_per_lane, int waves_per_group, int blocks_per_wave,
                                      int flags, unsigned long long* wave_times,
                                      size_t wave_times_len, hipStream_t stream) {
    if (bytes == 0) return GEMV_SUCCESS;
    if (buffer == nullptr || sink == nullptr || bytes % 16 != 0 || (uintptr_t)buffer % 16 != 0 ||
        (uintptr_t)sink % 4 != 0 || blocks_per_wave < 1 || (flags & ~7) != 0)
        return GEMV_ERROR_INVALID_VALUE;
    const void* fn = probe_variant_fn(loads_per_lane, waves_per_group, flags);
    if (fn == nullptr) return GEMV_ERROR_INVALID_VALUE;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t per_wave = (int64_t)loads_per_lane * 64 * blocks_per_wave;
    const int64_t waves = (n16 + per_wave - 1) / per_wave;
    Plan p;
    p.grid = (waves + waves_per_group - 1) / waves_per_group;
    p.block = waves_per_group * 64;
    if (p.grid > 0x7fffffff) return GEMV_ERROR_INVALID_VALUE;
    if (wave_times != nullptr &&
        ((uintptr_t)wave_times % 8 != 0 || wave_times_len < (size_t)(2 * p.grid * waves_per_group)))
        return GEMV_ERROR_INVALID_VALUE;
    const gemvdev::quad* q = static_cast<const gemvdev::quad*>(buffer);
    int blocks = blocks_per_wave, stride = (flags & 4) ? 1 : 0;
    void* argv[] = {(void*)&q, (void*)&n16, (void*)&sink, (void*)&blocks, (void*)&stride,
                    (void*)&wave_times};
    return finish(launch(fn, p, stream, argv));
}

gemv_status_t gemv_plan(gemv_dtype_t dtype, int M, int K, int lda, int nvec, const void* A,
                        const void* X, int family, gemv_plan_t* plan) {
    if (plan == nullptr || (int)dtype > gemvplan::BF16) return GEMV_ERROR_INVALID_VALUE;
    Plan p;
    if (gemvplan::make_plan((int)dtype, M, K, lda, nvec, (uintptr_t)A, (uintptr_t)X, family,
                            &p) != gemvplan::OK ||
        !has_kernel((int)dtype, p, nvec))
        return GEMV_ERROR_INVALID_VALUE;
    export_plan(p, plan);
    return GEMV_SUCCESS;
}

gemv_status_t gemv_plan_splitk(gemv_dtype_t dtype, int M, int K, int lda, int splits,
                               const void* A, const void* x, gemv_plan_t* plan) {
    if (plan == nullptr || lda < K) return GEMV_ERROR_INVALID_VALUE;
    Plan p;
    const bool vec = gemvplan::vector_ok((int)dtype, K, lda, 1, (uintptr_t)A, (uintptr_t)x);
    if (gemvplan::make_split_plan((int)dtype, M, K, vec, splits, &p) != gemvplan::OK ||
        !has_splitk_kernel((int)dtype, p))
        return GEMV_ERROR_INVALID_VALUE;
    export_plan(p, plan);
    return GEMV_SUCCESS;
}

gemv_status_t gemv_splitk_workspace_size(gemv_dtype_t dtype, int M, int K, int splits,
                                         size_t* bytes) {
    int n = 1, slice = 0;
    if (bytes == nullptr ||
        gemvplan::split_geometry((int)dtype, M, K, splits, &n, &slice) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    *bytes = (size_t)gemvplan::split_workspace_bytes(M, n);
    return GEMV_SUCCESS;
}

gemv_status_t gemv_splitk_f32(const float* A, int lda, const float* x, const float* bias,
                              float* y, int M, int K, int splits, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    return run_splitk<TF32>(A, lda, x, bias, y, M, K, splits, workspace, workspace_bytes, stream);
}

gemv_status_t gemv_splitk_f16(const uint16_t* A, int lda, const uint16_t* x, const float* bias,
                              float* y, int M, int K, int splits, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
    return run_splitk<TF16>(A, lda, x, bias, y, M, K, splits, workspace, workspace_bytes, stream);
}

gemv_status_t gemv_splitk_bf16(const uint16_t* A, int lda, const uint16_t* x, const float* bias,
                               float* y, int M, int K, int splits, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
    return run_splitk<TBF16>(A, lda, x, bias, y, M, K, splits, workspace, workspace_bytes, stream);
}

gemv_status_t gemv_test_refused_launch(hipStream_t stream) {
    // A workgroup of 2048 threads, twice what the hardware allows: the
    // runtime refuses the launch before anything reaches the GPU.  The kernel
    // is the split-K reduce with no rows (M = 0), which would touch no memory
    // even if it ran.
    const float* ws = nullptr;
    const float* bias = nullptr;
    float* y = nullptr;
    int splits = 1;
    int64_t M = 0;
    void* argv[] = {(void*)&ws, (void*)&splits, (void*)&bias, (void*)&y, (void*)&M};
    return finish(hipLaunchKernel((const void*)&gemvdev::gemv_splitk_reduce_kernel, dim3(1),
                                  dim3(2048), argv, 0, stream));
}

gemv_status_t gemv_splitk_noalloc(gemv_dtype_t dtype, const void* A, int lda, const void* x,
                                  const float* bias, float* y, int M, int K, int splits,
                                  hipStream_t stream) {
    // the checks and the plan of gemv_splitk_*, before the scratch is touched
    if (splits < 0 || gemvplan::validate((int)dtype, M, K, lda, 1, (uintptr_t)A, (uintptr_t)x,
                                         (uintptr_t)bias, (uintptr_t)y) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    if (M == 0) return GEMV_SUCCESS;
    int n = 1, slice = 0;
    if (gemvplan::split_geometry((int)dtype, M, K, splits, &n, &slice) != gemvplan::OK)
        return GEMV_ERROR_INVALID_VALUE;
    const int64_t need = gemvplan::split_workspace_bytes(M, n);
    if (need > (int64_t)kScratchBytes) return GEMV_ERROR_INVALID_VALUE;
    void* ws = nullptr;
    if (need > 0) {
        const gemv_status_t st = device_scratch(stream, &ws);
        if (st != GEMV_SUCCESS) return st;
    }
    switch ((int)dtype) {
    case gemvplan::F32: return run_splitk<TF32>(A, lda, x, bias, y, M, K, splits, ws, kScratchBytes, stream);
    case gemvplan::F16: return run_splitk<TF16>(A, lda, x, bias, y, M, K, splits, ws, kScratchBytes, stream);
    case gemvplan::BF16: return run_splitk<TBF16>(A, lda, x, bias, y, M, K, splits, ws, kScratchBytes, stream);
    default: return GEMV_ERROR_INVALID_VALUE;
    }
}

gemv_status_t gemv_run_family(gemv_dtype_t dtype, int family, const void* A, int lda,
                              const void* X, const float* bias, float* Y, int M, int K,
                              int nvec, hipStream_t stream) {
    return run((int)dtype, family, A, lda, X, bias, Y, M, K, nvec, stream);
}

}  // extern "C"
