// gfx950 GEMV kernels.
//
// Every output y[m] is the dot product of row m of A with x (page "SGEMV
// CUDA代码学习", section "问题定义: 一行一个点积"), plus bias[m] when a bias is
// given, added once after the reduction by the single lane that writes y[m]
// (page "第 3 课：GEMV 与行级并行", sections "C. 点积规约与原子写入解耦" and
// "3. 正确性边界与指针安全性").  Nothing is atomic; each output has exactly
// one writer.
//
// Shared structure:
//   * A is streamed once with coalesced, nontemporal loads: the lanes that share a row
//     read consecutive 16-byte chunks, so one wavefront load instruction
//     covers 1 KiB of A (page "SGEMV CUDA代码学习", section "Kernel 2: k128 +
//     Vec4", carried to 64 lanes);
//   * each lane issues all loads of a batch before it consumes any, so many
//     requests per lane are in flight;
//   * out-of-range chunks in the last batch load a clamped, in-range address
//     and are replaced by zero before use; the row tail shorter than one chunk
//     is read element by element.  Nothing beyond column K-1 of a row is
//     read, so padding between rows (lda > K) never enters a sum;
//   * x is small and read by every row; it stays in the L1/L2 caches (page
//     "第 3 课", section "B. 向量 x 的高速片上缓存复用"); an x too long to stay
//     in a CU's L1 beside the A stream is kept in registers while a workgroup
//     walks several rows, or (longer still) shared by two rows per workgroup;
//   * rows past M in the last wavefront clamp their loads to row M-1, take
//     part in the reduction, and do not write.
#pragma once

#include "gemv_device.hpp"
#include "gemv_plan.hpp"

namespace gemvdev {

// Wavefronts per workgroup of the rows and vector-ALU batched kernels: a
// compile-time constant rather than the launch's block size, so that with
// the kernel arguments preloaded into SGPRs nothing waits on a scalar load
// before the first load of A is issued.
constexpr int kRowsWaves = 4;
// Wavefronts per workgroup of the workgroup-per-row and split-K kernels.
constexpr int kGroupWavesDev = 4;

// A load that stays a vector-memory load even at a wave-uniform address: the
// offset is a zero the compiler cannot see through.  (At a uniform row, as
// in the workgroup-per-row kernel, a plain load of the bias became a scalar
// load that the wavefront waited on before issuing its first A load; a
// vector load is waited on only where its value is used, after the A stream.)
__device__ __forceinline__ float vector_load(const float* p) {
    int zero;
    asm("v_mov_b32 %0, 0" : "=v"(zero));
    return p[zero];
}

// Where row m of the (possibly row-concatenated) problem lives and where its
// result goes.  Passed to the kernels by value, as kernel arguments.
template <class S>
struct OneMatrix {
    static constexpr bool kScaled = false;  // no per-row scale
    const S* A;
    int64_t lda;
    const float* bias;  // or nullptr
    float* y;
    int64_t M;
    __device__ __forceinline__ const S* row(int64_t m) const { return A + m * lda; }
    __device__ __forceinline__ bool any_bias() const { return bias != nullptr; }
    __device__ __forceinline__ float bias_of(int64_t m) const { return vector_load(bias + m); }
    __device__ __forceinline__ void store(int64_t m, float v) const { y[m] = v; }
};

// One int8 weight matrix with a fp32 scale per row: y[m] = scale[m]·(row
// m · x) + bias[m] (the lqnn.cn NPU MatMul essay, section 4.2: int8
// weights with a per-channel scale).
template <class S>
struct ScaledMatrix {
    static constexpr bool kScaled = true;
    const S* A;
    int64_t lda;
    const float* scale;
    const float* bias;  // or nullptr
    float* y;
    int64_t M;
    __device__ __forceinline__ const S* row(int64_t m) const { return A + m * lda; }
    __device__ __forceinline__ float scale_of(int64_t m) const { return vector_load(scale + m); }
    __device__ __forceinline__ bool any_bias() const { return bias != nullptr; }
    __device__ __forceinline__ float bias_of(int64_t m) const { return vector_load(bias + m); }
    __device__ __forceinline__ void store(int64_t m, float v) const { y[m] = v; }
};

// The epilogue of one row: sum·scale + bias (one rounding) for a scaled
// matrix, sum + bias otherwise.
template <class Rows>
__device__ __forceinline__ float row_result(float sum, float scale, float bias) {
    if constexpr (Rows::kScaled)
        return __builtin_fmaf(sum, scale, bias);
    else
        return sum + bias;
}
template <class Rows>
__device__ __forceinline__ float scale_of(const Rows& rows, int64_t m) {
    if constexpr (Rows::kScaled)
        return rows.scale_of(m);
    else
        return 1.f;
}

// Up to kMaxSegments matrices with the same K, stacked row-wise: rows
// seg[i-1].end .. seg[i].end - 1 of the stack are rows of segment i (segment
// 0 starts at row 0).  Every segment multiplies the same x (e.g. the q, k
// and v projections of one token).  A row's segment is found by a select
// chain over the boundaries of the first NSEG entries.  The table is the
// kernel's only argument, read from memory; calls with at most three
// segments of one row pitch use ThreeSegments below instead.
constexpr int kMaxSegments = 8;
constexpr int kFewSegments = 3;

// A wave-uniform value (a kernel argument) passed through readfirstlane.  The
// segment choosers select between such values: a select between two fields
// read from the argument structure would otherwise be turned into one read
// from a selected address, which leaves the structure in scratch memory (or
// makes an indexed memory load of the argument table) ahead of the first
// A load.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A wave-uniform pointer to global memory: its two halves through
// readfirstlane, rebuilt as a pointer into the global address space (rebuilt
// as a generic pointer, every load and store through it was a flat
// instruction: fused q/k/v, 6144 rows, 9.30 -> 9.09 µs).
template <class T>
__device__ __forceinline__ T* uniform_global(T* p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return (T*)(__attribute__((address_space(1))) T*)(((uint64_t)hi << 32) | lo);
}
template <class S>
struct SegEntry {
    const S* A;
    int end;  // one past the segment's last row in the stack
    int lda;
};
static_assert(sizeof(SegEntry<float>) == 16, "four argument dwords per segment");
template <class S, int NSEG>
struct Segments {
    static constexpr bool kScaled = false;
    __device__ __forceinline__ bool any_bias() const { return true; }  // decided per row
    const S* x;
    int K;
    int M;  // rows in all segments
    SegEntry<S> seg[kMaxSegments];
    const float* bias[kMaxSegments];
    float* y[kMaxSegments];
    __device__ __forceinline__ const S* row(int64_t m) const {
        const S* a = seg[0].A;
        int ld = seg[0].lda;
        int64_t s0 = 0;
#pragma unroll
        for (int i = 1; i < NSEG; ++i) {
            const int e = seg[i - 1].end;
            const bool in = m >= e;
            a = in ? seg[i].A : a;
            ld = in ? seg[i].lda : ld;
            s0 = in ? e : s0;
        }
        return a + (m - s0) * (int64_t)ld;
    }
    __device__ __forceinline__ float bias_of(int64_t m) const {
        const float* b = bias[0];
        int64_t s0 = 0;
#pragma unroll
        for (int i = 1; i < NSEG; ++i) {
            const int e = seg[i - 1].end;
            const bool in = m >= e;
            b = in ? bias[i] : b;
            s0 = in ? e : s0;
        }
        return b != nullptr ? b[m - s0] : 0.f;
    }
    __device__ __forceinline__ void store(int64_t m, float v) const {
        float* o = y[0];
        int64_t s0 = 0;
#pragma unroll
        for (int i = 1; i < NSEG; ++i) {
            const int e = seg[i - 1].end;
            const bool in = m >= e;
            o = in ? y[i] : o;
            s0 = in ? e : s0;
        }
        o[m - s0] = v;
    }
};

// Up to three segments with one row pitch, passed as scalar kernel
// arguments: x, the three A pointers, two boundaries, the row pitch, K, the
// row count and whether any segment has a bias are the first 14 argument
// dwords, the ones that arrive preloaded in SGPRs, so the first loads wait on
// no argument load (an aggregate argument is read from memory instead, and
// the select chain over a table in memory became an indexed load ahead of
// the first A load).  Rows below end0 are segment 0, below end1 segment 1,
// the rest segment 2.
template <class S>
struct ThreeSegments {
    static constexpr bool kScaled = false;
    const S* A0;
    const S* A1;
    const S* A2;
    int end0, end1;
    int lda;
    int M;
    int has_bias;  // 0: no segment has a bias (b0..b2 are never read)
    const float* b0;
    const float* b1;
    const float* b2;
    float* y0;
    float* y1;
    float* y2;
    __device__ __forceinline__ const S* row(int64_t m) const {
        const int e0 = uniform(end0), e1 = uniform(end1);
        const bool in1 = m >= e0, in2 = m >= e1;
        const S* a = in2 ? uniform_global(A2) : (in1 ? uniform_global(A1) : uniform_global(A0));
        const int64_t s0 = in2 ? e1 : (in1 ? e0 : 0);
        return a + (m - s0) * (int64_t)lda;
    }
    __device__ __forceinline__ bool any_bias() const { return has_bias != 0; }
    __device__ __forceinline__ float bias_of(int64_t m) const {
        const int e0 = uniform(end0), e1 = uniform(end1);
        const bool in1 = m >= e0, in2 = m >= e1;
        const float* b = in2 ? uniform_global(b2) : (in1 ? uniform_global(b1) : uniform_global(b0));
        const int64_t s0 = in2 ? e1 : (in1 ? e0 : 0);
        return b != nullptr ? b[m - s0] : 0.f;
    }
    __device__ __forceinline__ void store(int64_t m, float v) const {
        const int e0 = uniform(end0), e1 = uniform(end1);
        const bool in1 = m >= e0, in2 = m >= e1;
        float* o = in2 ? uniform_global(y2) : (in1 ? uniform_global(y1) : uniform_global(y0));
        const int64_t s0 = in2 ? e1 : (in1 ? e0 : 0);
        o[m - s0] = v;
    }
};

// One batch of the rows kernels: BATCH chunks per row tile, chunk c + i·L
// for i < BATCH, all loads issued before any is used.  CHECK: chunks at or
// past nfull load chunk nfull-1 instead and are replaced by zero.  The
// batch's products are summed in two fresh accumulators (alternate chunks),
// whose sum is then added to the row tile's running compensated sum: the
// rounding chain of a batch is at most ceil(BATCH/2) chunks of elements,
// whatever the row length.
template <class C, int L, int U, int BATCH, bool CHECK, class S, class XS>
__device__ __forceinline__ void rows_batch(const S* const (&rp)[U], const XS* x, int c, int nfull,
                                           Sum2 (&sum)[U]) {
    using CT = typename C::type;
    using XT = typename C::xtype;
    CT a[U][BATCH];
    XT xv[BATCH];
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
        int cc = c + i * L;
        if constexpr (CHECK) cc = cc < nfull ? cc : nfull - 1;
#pragma unroll
        for (int u = 0; u < U; ++u) a[u][i] = C::stream(rp[u], cc);
        xv[i] = C::load(x, cc);
    }
    // keep every load of the batch ahead of the first use: without this
    // fence the scheduler may interleave each load with its multiply-adds
    // and leave one load in flight at a time
    __builtin_amdgcn_sched_barrier(0);
    float acc[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u][0] = acc[u][1] = 0.f;
#pragma unroll
    for (int i = 0; i < BATCH; ++i) {
        XT xi = xv[i];
        if constexpr (CHECK) xi = C::keep_x(c + i * L < nfull, xi);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            CT ai = a[u][i];
            if constexpr (CHECK) ai = C::keep_a(c + i * L < nfull, ai);
            acc[u][i & 1] = C::dot(ai, xi, acc[u][i & 1]);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u].add(acc[u][0] + acc[u][1]);
}

// Rows-per-wave (L < 64) and wave-per-row (L == 64) kernel.
// A wavefront covers R = 64/L rows per row tile and takes U consecutive row
// tiles; lanes sub = lane % L of one row walk its chunks with stride L, BATCH
// chunks in flight per row tile.  NW wavefronts per workgroup.
template <class D, int L, int U, int BATCH, bool VEC, int NW = kRowsWaves, class Rows>
__device__ __forceinline__ void rows_body(const Rows& rows, const typename D::xstorage* __restrict__ x,
                                          int K) {
    using S = typename D::storage;
    using C = Chunk<D, VEC>;
    constexpr int R = 64 / L;
    constexpr int E = C::elems;

    const int lane = threadIdx.x & 63;
    // the wavefront index is uniform: said so, a wavefront's row tiles, and
    // for one row per wavefront its row and row pointer, are scalars
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int sub = lane & (L - 1);
    const int slot = lane / L;
    const int64_t tile0 = ((int64_t)blockIdx.x * NW + wave) * U;

    const int64_t M = rows.M;
    const S* rp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t row = (tile0 + u) * R + slot;
        rp[u] = rows.row(row < M ? row : M - 1);
    }
    // Epilogue rows: the wavefront's U·R rows are consecutive, and lane
    // (slot, sub) adds the bias to and stores the rows of tiles u = sub,
    // sub + L, ... so that one store covers up to 64 consecutive rows.  The
    // bias loads are issued now, ahead of the A stream.
    constexpr int kOut = U < L ? 1 : U / L;  // rows stored per lane
    float bv[kOut], sv[kOut];
#pragma unroll
    for (int o = 0; o < kOut; ++o) {
        const int u = sub + o * L;
        const int64_t row = (tile0 + u) * R + slot;
        const bool in = u < U && row < M;
        bv[o] = 0.f;
        // a uniform test first, so that a call without a bias reads no bias pointer
        if (rows.any_bias() && in) bv[o] = rows.bias_of(row);
        sv[o] = in ? scale_of(rows, row) : 0.f;
    }

    Sum2 sum[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u] = Sum2{0.f, 0.f};

    const int nfull = K / E;  // whole chunks per row
    // Batches where every lane's chunks are in range need no checks; at most
    // one final batch straddles the end of the row.
    const int nsafe = nfull - nfull % (BATCH * L);
    int c0 = 0;
    for (; c0 < nsafe; c0 += BATCH * L) rows_batch<C, L, U, BATCH, false>(rp, x, c0 + sub, nfull, sum);
    // The checked batch and the element-wise tail are marked unlikely, so
    // the compiler places them after the kernel's end and the batches run
    // straight into the epilogue: every wavefront reaches the epilogue at
    // about the same time, near the end of a launch, and a jump over those
    // blocks there fetched instruction lines no wavefront had run yet (bf16
    // 4096 x 4096 6.643 -> 6.608 us, 1024 x 4096 3.212 -> 3.175).  Skipping
    // an empty tail leaves every sum as it was: adding 0 to a sum that
    // started at +0 changes no bit.
    if (__builtin_expect(c0 < nfull, 0)) rows_batch<C, L, U, BATCH, true>(rp, x, c0 + sub, nfull, sum);
    if constexpr (VEC) {
        if (__builtin_expect(nfull * E < K, 0)) {
            // elements past the last whole chunk (fewer than E of them)
            float tail[U];
#pragma unroll
            for (int u = 0; u < U; ++u) tail[u] = 0.f;
            for (int k = nfull * E + sub; k < K; k += L) {
                const float xe = widen_x(D{}, x[k]);
#pragma unroll
                for (int u = 0; u < U; ++u) tail[u] = __builtin_fmaf(widen_a(D{}, rp[u][k]), xe, tail[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) sum[u].add(tail[u]);
        }
    }

    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = segment_sum<L>(sum[u].value());
#pragma unroll
    for (int o = 0; o < kOut; ++o) {
        const int u = sub + o * L;
        // every lane of a segment holds the segment's sums: pick tile u
        float out = v[0];
#pragma unroll
        for (int t = 1; t < U; ++t) out = (u == t) ? v[t] : out;
        const int64_t row = (tile0 + u) * R + slot;
        if (u < U && row < M) rows.store(row, row_result<Rows>(out, sv[o], bv[o]));
    }
}

// One matrix: the arguments are scalars, so they arrive preloaded in SGPRs.
// (Workgroups of NW = 2 wavefronts spread a wave-per-row grid of a few
// workgroups per compute unit more evenly where 4 would leave some units
// one workgroup more than others.)
template <class D, int L, int U, int BATCH, bool VEC, int NW = kRowsWaves>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_rows_kernel(const typename D::storage* A, int64_t lda, const float* bias, float* y, int64_t M,
                 const typename D::storage* __restrict__ x, int K) {
    rows_body<D, L, U, BATCH, VEC, NW>(OneMatrix<typename D::storage>{A, lda, bias, y, M}, x, K);
}

// Several row-stacked matrices sharing x (the segment table is a kernel
// argument in memory).
template <class D, int L, int U, int BATCH, bool VEC, int NSEG>
__global__ void __launch_bounds__(kRowsWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_rows_multi_kernel(const Segments<typename D::storage, NSEG> rows) {
    rows_body<D, L, U, BATCH, VEC>(rows, rows.x, rows.K);
}

// Up to three matrices: scalar arguments (see ThreeSegments).
#define GEMV_THREE_SEGMENT_PARAMS                                                              \
    const typename D::storage *__restrict__ x, const typename D::storage *A0,                   \
        const typename D::storage *A1, const typename D::storage *A2, int end0, int end1,      \
        int lda, int K, int M, int has_bias, const float *b0, const float *b1,                 \
        const float *b2, float *y0, float *y1, float *y2
#define GEMV_THREE_SEGMENT_ROWS                                                                \
    ThreeSegments<typename D::storage> {                                                       \
        A0, A1, A2, end0, end1, lda, M, has_bias, b0, b1, b2, y0, y1, y2                      \
    }
template <class D, int L, int U, int BATCH, bool VEC>
__global__ void __launch_bounds__(kRowsWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_rows_multi3_kernel(GEMV_THREE_SEGMENT_PARAMS) {
    rows_body<D, L, U, BATCH, VEC>(GEMV_THREE_SEGMENT_ROWS, x, K);
}

// Workgroup-per-row kernel: W wavefronts (64·W lanes) share U consecutive
// rows, rows tile·U .. tile·U + U - 1; lane `sub` walks chunks sub, sub + 64·W,
// ... of every one of the U rows against the same x chunk, so a workgroup
// fetches x once for its U rows.  Each wavefront reduces its lanes, writes one
// partial per row to LDS, and after one barrier thread u adds row u's W
// partials in wavefront order, adds the bias and writes y (page "第 3 课", the
// block-reduction structure of section "C. 点积规约与原子写入解耦" on 64-lane
// wavefronts).  A row's sum does not depend on U.
template <class D, int W, int U, int BATCH, bool VEC, class Rows>
__device__ __forceinline__ void group_body(const Rows& rows, const typename D::xstorage* __restrict__ x,
                                           int K, int64_t tile) {
    using S = typename D::storage;
    using C = Chunk<D, VEC>;
    constexpr int L = W * 64;
    constexpr int E = C::elems;
    __shared__ float partial[W][U];

    const int64_t M = rows.M;
    const int64_t row0 = tile * U;
    if (row0 >= M) return;  // uniform across the workgroup
    const int sub = threadIdx.x;
    const S* rp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) rp[u] = rows.row(row0 + u < M ? row0 + u : M - 1);
    // thread u < U finishes row row0 + u; its bias and scale are read now
    const bool writer = sub < U && row0 + sub < M;
    const float b = (rows.any_bias() && writer) ? rows.bias_of(row0 + sub) : 0.f;
    const float sc = writer ? scale_of(rows, row0 + sub) : 0.f;

    Sum2 sum[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u] = Sum2{0.f, 0.f};
    const int nfull = K / E;
    const int nsafe = nfull - nfull % (BATCH * L);
    int c0 = 0;
    for (; c0 < nsafe; c0 += BATCH * L) rows_batch<C, L, U, BATCH, false>(rp, x, c0 + sub, nfull, sum);
    // (rare paths out of line, as in the rows body: 512 x 4096 2.730 ->
    // 2.687 us, 4096 x 14336 18.01 -> 17.90)
    if (__builtin_expect(c0 < nfull, 0)) rows_batch<C, L, U, BATCH, true>(rp, x, c0 + sub, nfull, sum);
    if (VEC && __builtin_expect(nfull * E < K, 0)) {
        float tail[U];
#pragma unroll
        for (int u = 0; u < U; ++u) tail[u] = 0.f;
        for (int k = nfull * E + sub; k < K; k += L) {
            const float xe = widen_x(D{}, x[k]);
#pragma unroll
            for (int u = 0; u < U; ++u) tail[u] = __builtin_fmaf(widen_a(D{}, rp[u][k]), xe, tail[u]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) sum[u].add(tail[u]);
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float v = segment_sum<64>(sum[u].value());
        if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6][u] = v;
    }
    __syncthreads();
    if (writer) {
        float s = partial[0][sub];
#pragma unroll
        for (int w = 1; w < W; ++w) s += partial[w][sub];
        rows.store(row0 + sub, row_result<Rows>(s, sc, b));
    }
}

template <class D, int W, int U, int BATCH, bool VEC>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_group_kernel(const typename D::storage* A, int64_t lda, const float* bias, float* y, int64_t M,
                  const typename D::storage* __restrict__ x, int K) {
    group_body<D, W, U, BATCH, VEC>(OneMatrix<typename D::storage>{A, lda, bias, y, M}, x, K,
                                    blockIdx.x);
}

// Workgroup-per-row family, x held in registers: for rows whose x is at most
// NX chunks per lane of the W·64 lanes, each lane loads its NX chunks of x
// once and the workgroup walks the R consecutive rows tile·R .. tile·R + R - 1,
// issuing row j+1's loads before row j's multiply-adds.  A workgroup fetches
// x from L2 once for R rows instead of once per row (the block-per-row
// mapping of page "第 3 课" with the x reuse of its section "B. 向量 x 的高速片
// 上缓存复用" moved into registers).  Needs K a whole number of chunks and
// (NX - 1)·64·W < K/E ≤ NX·64·W; the last chunk of a lane may lie past the
// row, and is then a clamped load whose products are dropped.  The per-row
// sums follow the workgroup-per-row body's order for the same W.
template <class D, int W, int NX, int R, class Rows>
__device__ __forceinline__ void group_stream_body(const Rows& rows,
                                                  const typename D::xstorage* __restrict__ x, int K,
                                                  int64_t tile) {
    using S = typename D::storage;
    using C = Chunk<D, true>;
    using CT = typename C::type;
    constexpr int L = W * 64;
    __shared__ float partial[W][R];

    const int64_t M = rows.M;
    const int64_t row0 = tile * R;
    if (row0 >= M) return;  // uniform across the workgroup
    const int sub = threadIdx.x;
    const int nfull = K / C::elems;
    // lane `sub` owns chunks sub + i·L; only the last can lie past the row
    const bool last_ok = sub + (NX - 1) * L < nfull;
    const int clast = last_ok ? sub + (NX - 1) * L : nfull - 1;
    const bool writer = sub < R && row0 + sub < M;
    const float b = (rows.any_bias() && writer) ? rows.bias_of(row0 + sub) : 0.f;
    const float sc = writer ? scale_of(rows, row0 + sub) : 0.f;

    typename C::xtype xv[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) xv[i] = C::load(x, i + 1 < NX ? sub + i * L : clast);

    CT a[2][NX];
    auto fetch = [&](CT (&dst)[NX], int64_t m) {
        const S* p = rows.row(m < M ? m : M - 1);
#pragma unroll
        for (int i = 0; i < NX; ++i) dst[i] = C::stream(p, i + 1 < NX ? sub + i * L : clast);
    };
    fetch(a[0], row0);
    // x and row 0 are the first loads, so that row 0 waits for nothing else
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < R; ++j) {
        if (j + 1 < R) fetch(a[(j + 1) & 1], row0 + j + 1);
        // row j+1's loads stay ahead of row j's multiply-adds
        __builtin_amdgcn_sched_barrier(0);
        // a clamped last chunk contributes nothing (zeroed once x has arrived)
        if (j == 0) xv[NX - 1] = C::keep_x(last_ok, xv[NX - 1]);
        float acc[2] = {0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NX; ++i) acc[i & 1] = C::dot(a[j & 1][i], xv[i], acc[i & 1]);
        const float v = segment_sum<64>(acc[0] + acc[1]);
        if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6][j] = v;
    }
    __syncthreads();
    if (writer) {
        float s = partial[0][sub];
#pragma unroll
        for (int w = 1; w < W; ++w) s += partial[w][sub];
        rows.store(row0 + sub, row_result<Rows>(s, sc, b));
    }
}

template <class D, int W, int NX, int R>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_group_stream_kernel(const typename D::storage* A, int64_t lda, const float* bias, float* y,
                         int64_t M, const typename D::storage* __restrict__ x, int K) {
    group_stream_body<D, W, NX, R>(OneMatrix<typename D::storage>{A, lda, bias, y, M}, x, K,
                                   blockIdx.x);
}

template <class D, int W, int BATCH, bool VEC, int NSEG>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_group_multi_kernel(const Segments<typename D::storage, NSEG> rows) {
    group_body<D, W, 1, BATCH, VEC>(rows, rows.x, rows.K, blockIdx.x);
}

template <class D, int W, int BATCH, bool VEC>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_group_multi3_kernel(GEMV_THREE_SEGMENT_PARAMS) {
    group_body<D, W, 1, BATCH, VEC>(GEMV_THREE_SEGMENT_ROWS, x, K, blockIdx.x);
}

// Weight-only int8: the rows and workgroup-per-row bodies on int8 weights,
// x of type X, and the per-row scale applied after each row's sum.  What the
// first loads need (Q, its pitch, x, M, K, then scale and bias) comes first:
// the first 14 argument dwords arrive preloaded in SGPRs.
template <class X, int L, int U, int BATCH, bool VEC>
__global__ void __launch_bounds__(kRowsWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_rows_q8_kernel(const int8_t* Q, int64_t ldq, const typename X::storage* __restrict__ x,
                    int64_t M, int K, const float* scale, const float* bias, float* y) {
    rows_body<TQ8<X>, L, U, BATCH, VEC>(ScaledMatrix<int8_t>{Q, ldq, scale, bias, y, M}, x, K);
}

// U rows per workgroup: every x chunk a lane loads serves U weight chunks,
// all of them in flight together.  W is 4, or 2 for one row of at most two
// loads per lane.
template <class X, int W, int U, int BATCH, bool VEC>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_group_q8_kernel(const int8_t* Q, int64_t ldq, const typename X::storage* __restrict__ x,
                     int64_t M, int K, const float* scale, const float* bias, float* y) {
    group_body<TQ8<X>, W, U, BATCH, VEC>(ScaledMatrix<int8_t>{Q, ldq, scale, bias, y, M}, x, K,
                                         blockIdx.x);
}

// Int8 weights with x held in registers across R rows: the x-in-registers
// body on int8 rows, whose x chunks (16 elements of the x type) are 32 or 64
// bytes against 16 of weights, so fetching x once per R rows saves more than
// with 2-byte weights.
template <class X, int W, int NX, int R>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_group_stream_q8_kernel(const int8_t* Q, int64_t ldq, const typename X::storage* __restrict__ x,
                            int64_t M, int K, const float* scale, const float* bias, float* y) {
    group_stream_body<TQ8<X>, W, NX, R>(ScaledMatrix<int8_t>{Q, ldq, scale, bias, y, M}, x, K,
                                        blockIdx.x);
}

// Split-K, pass 1: workgroup (t, s) forms the dot products of rows t·U ..
// t·U + U - 1 (U = 1 or 2), slice s (elements s·slice .. s·slice + slice - 1,
// the last slice shorter), with the same slice of x, in the workgroup-per-row
// body (each x chunk serves the U rows), and writes row m's to
// ws[m·splits + s].  The A and x pointers of a slice are offset by a whole
// number of 16-byte loads, so the vector path's alignment holds in every
// slice.  Workgroup id = t·splits + s: consecutive ids, which the dispatcher
// deals round-robin to the 8 XCDs, walk the slices of one row tile, so with
// splits a multiple of 8 every tile's slice s runs on the same XCD and its x
// slice is fetched into that XCD's L2 once, not once per tile.
template <class S>
struct SliceOfRows {
    static constexpr bool kScaled = false;
    const S* A;  // first element of the slice in row 0
    int64_t lda;
    float* ws;   // ws + s: the row-major M × splits partials, column s
    int splits;
    int64_t M;
    __device__ __forceinline__ const S* row(int64_t m) const { return A + m * lda; }
    __device__ __forceinline__ bool any_bias() const { return false; }
    __device__ __forceinline__ float bias_of(int64_t) const { return 0.f; }
    __device__ __forceinline__ void store(int64_t m, float v) const { ws[m * splits] = v; }
};

template <class D, int U, int BATCH, bool VEC>
__global__ void __launch_bounds__(kGroupWavesDev * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_splitk_partial_kernel(const typename D::storage* A, int64_t lda, float* ws, int64_t M,
                           const typename D::storage* __restrict__ x, int K, int slice,
                           int splits) {
    const uint32_t id = blockIdx.x;
    const int s = (int)(id % (uint32_t)splits);
    const int64_t tile = id / (uint32_t)splits;  // rows tile·U .. tile·U + U - 1
    const int64_t k0 = (int64_t)s * slice;
    const int64_t rest = (int64_t)K - k0;
    const int ks = rest < slice ? (int)rest : slice;
    group_body<D, kGroupWavesDev, U, BATCH, VEC>(
        SliceOfRows<typename D::storage>{A + k0, lda, ws + s, splits, M}, x + k0, ks, tile);
}

// Split-K, pass 2: one wavefront per row adds the row's `splits` partials in
// a fixed order (lane l takes partials l, l + 64, ... in turn, then the
// 64-lane tree of segment_sum), adds the bias, and writes y[m].  The order
// depends on nothing but `splits`, so repeated calls give identical results
// (the two-stage reduction of page "第 3 课" with its second stage in a
// kernel of its own, so that no atomics are needed).
__global__ void __launch_bounds__(kRowsWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_splitk_reduce_kernel(const float* __restrict__ ws, int splits, const float* __restrict__ bias,
                          float* __restrict__ y, int64_t M) {
    const int lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * kRowsWaves + (threadIdx.x >> 6);
    if (m >= M) return;  // uniform across the wavefront
    const float* p = ws + m * splits;
    float acc = 0.f;
    for (int s = lane; s < splits; s += 64) acc += p[s];
    acc = segment_sum<64>(acc);
    if (lane == 0) y[m] = acc + (bias != nullptr ? bias[m] : 0.f);
}

// Batched kernel on the vector ALUs: Y = A·X (+ bias) for NV right-hand
// vectors with one pass over A, the wave-per-row mapping with several
// vectors.  A wavefront owns U consecutive rows; its 64 lanes walk the rows'
// chunks with stride 64, B chunks per lane per batch.  Every chunk of X is
// loaded once per wavefront and meets the matching chunk of all U rows
// (X is K×NV column-major: column j at X + j·K, read through the caches).
// With XAHEAD the X chunks of a batch are loaded with its A chunks (all in
// flight together); otherwise (many vectors, whose X chunks would not fit
// the registers) each chunk's X loads follow the batch's A loads.  The
// arithmetic is the single-vector path's: exactly widened elements, IEEE
// fp32 FMA in element order into an accumulator per (row, vector) that runs
// over RUN batches and is then added to a compensated running sum (with
// many vectors the compensated add costs nearly as much as a batch's FMAs
// for one (row, vector), so it is not paid every batch there, and the FMAs
// of all (row, vector) pairs are interleaved).  Then one 64-lane reduction
// per (row, vector) and lane u·NV + j writes Y[j·M + row u] (+ bias).  16-byte
// loads take any row pitch and K (rows and X columns start at
// element-aligned addresses: unaligned global loads).
//
// KS > 1 splits K instead (few rows: one wavefront per row would leave most
// of the chip idle and make the time one wavefront's walk along its row):
// KS consecutive wavefronts share U rows, the k-th of them taking batches
// k, k + KS, ... of each row; the per-wavefront totals meet in LDS and the
// group's first wavefront adds them in wavefront order (the same order
// every call).
template <class D, int NV, int U, int B, bool XAHEAD, bool VEC, int RUN, int KS = 1>
__global__ void __launch_bounds__(kRowsWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
gemv_batched_kernel(const typename D::storage* __restrict__ A, int64_t lda,
                    const typename D::storage* __restrict__ X,
                    const float* __restrict__ bias, float* __restrict__ Y,
                    int64_t M, int K) {
    using S = typename D::storage;
    using C = Chunk<D, VEC>;
    using CT = typename C::type;
    constexpr int E = C::elems;
    static_assert(U * NV <= 64, "one writer lane per (row, vector)");
    static_assert(KS == 1 || KS == 2 || KS == kRowsWaves, "1, 2 or all wavefronts per row group");
    constexpr int kGroups = kRowsWaves / KS;  // row groups per workgroup

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kw = wave % KS;  // this wavefront's share of K
    const int grp = wave / KS;
    const int64_t row0 = ((int64_t)blockIdx.x * kGroups + grp) * U;
    const S* rp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t m = row0 + u;
        rp[u] = A + (m < M ? m : M - 1) * lda;
    }
    const S* xp[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) xp[j] = X + (int64_t)j * K;

    Sum2 sum[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NV; ++j) sum[u][j] = Sum2{0.f, 0.f};

    float acc[U][NV];
    auto clear = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j) acc[u][j] = 0.f;
    };
    auto flush = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j) sum[u][j].add(acc[u][j]);
    };
    clear();

    const int nfull = K / E;
    auto batch = [&](int c0, bool check) {
        CT a[U][B];
        CT xa[XAHEAD ? NV : 1][B];
#pragma unroll
        for (int i = 0; i < B; ++i) {
            int c = c0 + i * 64 + lane;
            c = (check && c >= nfull) ? nfull - 1 : c;
#pragma unroll
            for (int u = 0; u < U; ++u) a[u][i] = C::stream(rp[u], c);
            if constexpr (XAHEAD)
#pragma unroll
                for (int j = 0; j < NV; ++j) xa[j][i] = C::load(xp[j], c);
        }
        __builtin_amdgcn_sched_barrier(0);  // the batch's loads in flight first
#pragma unroll
        for (int i = 0; i < B; ++i) {
            const int c = c0 + i * 64 + lane;
            const bool ok = !check || c < nfull;
            CT ai[U];
#pragma unroll
            for (int u = 0; u < U; ++u) ai[u] = C::keep_a(ok, a[u][i]);
            CT xc[XAHEAD ? 1 : NV];
            if constexpr (!XAHEAD) {
                // X chunk by chunk: the chunk's NV loads in flight together
#pragma unroll
                for (int j = 0; j < NV; ++j) xc[j] = C::load(xp[j], ok ? c : nfull - 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            CT xs[NV];
#pragma unroll
            for (int j = 0; j < NV; ++j) xs[j] = C::keep_x(ok, XAHEAD ? xa[j][i] : xc[j]);
            if constexpr (RUN == 1) {
#pragma unroll
                for (int j = 0; j < NV; ++j)
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[u][j] = C::dot(ai[u], xs[j], acc[u][j]);
            } else {
                // word by word across all (row, vector) accumulators, so that
                // independent multiply-adds follow each other; each
                // accumulator still takes its chunk's elements in order
#pragma unroll
                for (int w = 0; w < C::words; ++w)
#pragma unroll
                    for (int j = 0; j < NV; ++j)
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            acc[u][j] = C::dot_word(ai[u], xs[j], w, acc[u][j]);
            }
            // one chunk's X operands live at a time
            if constexpr (!XAHEAD) __builtin_amdgcn_sched_barrier(0);
        }
    };
    // this wavefront's batches (every KS-th), in runs of at most RUN batches
    // per accumulator (the last, checked batch included)
    int c0 = kw * B * 64, run = 0;
#pragma unroll 1
    for (; c0 + B * 64 <= nfull; c0 += KS * B * 64) {
        batch(c0, false);
        if (++run == RUN) {
            flush();
            clear();
            run = 0;
        }
    }
    if (c0 < nfull) {
        batch(c0, true);
        ++run;
    }
    if (run > 0) flush();
    if (VEC && kw == 0) {
        // elements past the last whole chunk (fewer than E of them)
        float tail[U][NV];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j) tail[u][j] = 0.f;
        for (int k = nfull * E + lane; k < K; k += 64) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const float xe = widen(D{}, xp[j][k]);
#pragma unroll
                for (int u = 0; u < U; ++u) tail[u][j] = __builtin_fmaf(widen(D{}, rp[u][k]), xe, tail[u][j]);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NV; ++j) sum[u][j].add(tail[u][j]);
    }

    // every lane holds every total after the reductions; lane u·NV + j writes
    float out = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const float v = segment_sum<64>(sum[u][j].value());
            out = lane == u * NV + j ? v : out;
        }
    if constexpr (KS > 1) {
        __shared__ float part[kGroups][KS][U * NV];
        if (lane < U * NV) part[grp][kw][lane] = out;
        __syncthreads();
        if (kw != 0) return;
        if (lane < U * NV) {
            out = part[grp][0][lane];
#pragma unroll
            for (int w = 1; w < KS; ++w) out += part[grp][w][lane];
        }
    }
    if (lane < U * NV) {
        const int u = lane / NV, j = lane % NV;
        const int64_t m = row0 + u;
        if (m < M) Y[(int64_t)j * M + m] = out + (bias != nullptr ? bias[m] : 0.f);
    }
}

// Batched kernel on the matrix cores: Y = A·X (+ bias) for up to 16·NT
// vectors.  With 16 vectors every A element takes part in 16 multiply-adds,
// close to the vector ALUs' limit (about 16 FLOP per byte against a ridge of
// about 20), so the contraction runs as 16×16×32 MFMA steps instead.  Past
// 16 vectors (page "第 3 课：GEMV 与行级并行", section "4. 性能与工程权舍" puts
// the switch to matrix-core GEMM at a batch of 16 to 32) each A operand
// meets NT tiles of 16 vectors: A is still read once, and at 64 vectors
// (about 64 FLOP per byte against a matrix-core ridge of about 300) the
// path stays bound by HBM.
//
// Full-line A loads.  A 16×16×32 step takes 16 operand rows with 4 lanes of
// 16 bytes each, so a load in the plain operand layout reads 64 bytes of
// each of 16 rows (half of every 128-byte line; reading A that way took 1 µs
// longer for 32 MiB).  Here each operand row is half of a real row: operand
// row v is real row v/2, elements 64·i + 32·(v % 2) + 8·g of step i, so one
// load reads whole 128-byte lines of 8 real rows.  The contraction index
// must be the same for the two operands, so each A operand meets two X
// operands, one per half (elements 64·i + 8·g and 64·i + 32 + 8·g), in two
// MFMA steps; each step's outputs are right for the operand rows of its half
// and the others are dropped.  Real row R's sum is the even row of the first
// step's tile plus the odd row of the second's.
//
// A workgroup owns Q groups of RG real rows (two groups of 8; one group of 8
// or of 4 where that spreads a small matrix over more compute units; four
// groups of 8 on tall matrices, which halves the X bytes per A byte); its W
// wavefronts split the 64-element steps of K into contiguous slices and walk
// them in chunks of CH steps.  Per chunk a wavefront issues the loads of X
// operands ahead of the loads of A that they meet: loads complete in issue
// order, so the X operands are ready when the A they meet lands and each
// step's MFMAs run as its A arrives (with all A loads first, every MFMA
// waited for the last X load: 16 vectors 9.04 -> 8.76 µs).  X columns are K elements apart, so
// an X operand read straight from memory sends one load to 16 addresses a
// column pitch apart:
//   * with more than kMfmaFewVectors vectors, the K range of every X column
//     is loaded with coalesced 16-byte loads (a load covers whole 128-byte
//     pieces of 8 columns with one step per group, of 2 or 4 columns with a
//     whole chunk), written to the wavefront's own LDS region and read back
//     in operand layout (read straight from memory: 15-20 % slower at 16
//     vectors);
//   * with at most kMfmaFewVectors (FEW) the operands come straight from
//     memory, loaded step by step after the step's A (the lanes of the
//     columns past nvec repeat column nvec-1, so a load touches at most nvec
//     columns; 2 vectors: 7.44 -> 6.99 µs).
// An MFMA output column depends on its own X column only, so the operand
// columns of vectors past nvec are never zeroed (their outputs are never
// stored).  After one barrier wavefront 0 adds the W partial tiles in
// wavefront order and each lane finishes 4 consecutive rows of one column,
// adds the bias and writes them with one 16-byte store where Y allows it
// (four scattered 4-byte stores per lane before: 16 vectors 8.76 -> 8.38
// µs).  Needs 16-byte aligned A, X and row pitch and K % 8 == 0.  The
// ceil(K/64) steps, the partial last one (K % 64 != 0) included, are dealt
// to the wavefronts by gemvplan::mfma_step_range; the steps of a run that do
// not fill a whole chunk, and the partial step, read their operands
// directly, one step at a time.
template <class D, int W, int NT, int CH, bool FEW, int Q = 2, int RG = 8>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(2)))
gemv_batched_mfma_kernel(const typename D::storage* __restrict__ A, int64_t lda,
                         const typename D::storage* __restrict__ X,
                         const float* __restrict__ bias, float* __restrict__ Y,
                         int M, int K, int nvec) {
    using S = typename D::storage;
    constexpr int kCols = 16 * NT;
    // per wavefront: kCols columns × CH steps × 64 elements, each column
    // padded by 16 bytes so that 16 lanes reading 16 columns hit distinct banks
    constexpr int kColQuads = CH * 8 + 1;
    // the partial tiles: one quad per lane per tile and pair of row groups
    constexpr int kPairs = Q == 4 ? 2 : 1;
    static_assert(kCols * kColQuads >= NT * 64 * kPairs, "partials fit in the X region");
    static_assert(!FEW || NT == 1, "few vectors: one tile");
    __shared__ quad xs[W][kCols * kColQuads];

    const int lane = threadIdx.x & 63;
    // uniform: the wavefront's step range, chunk count and folds are scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;  // operand row (A) / column within a tile (X)
    const int g = lane >> 4;  // 8-element group within a 32-element half-step
    const int half = r & 1;
    // Q groups of RG real rows: RG = 8 fills the 16 operand rows with the
    // halves of 8 rows; RG = 4 (one group) gives the operand rows of real
    // rows 4..7 the addresses of rows 0..3, so their loads fetch no bytes of
    // their own and their duplicate outputs are never stored
    static_assert(Q == 1 || Q == 2 || Q == 4, "one, two or four groups of rows");
    static_assert(RG == 8 || (RG == 4 && Q == 1), "groups of 8 rows, or one group of 4");
    const int64_t row0 = (int64_t)blockIdx.x * (RG * Q);
    const S* ap[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t row = row0 + RG * q + ((r >> 1) & (RG - 1));
        ap[q] = A + (row < M ? row : (int64_t)M - 1) * lda + 32 * half + 8 * g;
    }

    // This wavefront's 64-element steps [rg.first, rg.end): whole steps run
    // in chunks of CH; what is left of the run, the partial last step
    // (K % 64 != 0) included, runs one step at a time below.
    const gemvplan::StepRange rg = gemvplan::mfma_step_range(K, W, wave);
    const int whole = K / 64;
    const int s1 = rg.end < whole ? rg.end : whole;
    const quad zero = quad{0u, 0u, 0u, 0u};
    quad* xw = xs[wave];

    // Up to 32 vectors (FRESH) every chunk's steps are summed into fresh
    // accumulators, which are then added into running totals with an
    // error-free two-sum per element (the rounding error of each addition is
    // carried in `cmp`), so a result's rounding chain does not grow with K.
    // With 4 tiles the registers do not allow it: the steps of all chunks
    // are summed into `acc` directly (the planner bounds K for that form).
    constexpr bool FRESH = NT <= 2;
    f32x4 acc[Q][NT][2], tot[Q][NT][2], cmp[Q][NT][2];
    // Every MFMA step starts from a zero accumulator and its outputs are
    // added to `acc` by the vector ALUs.  The matrix core aligns the terms of
    // a step (its 32 products and the accumulator passed in) to the largest
    // and drops the bits more than about 24 places below it (measured on
    // gfx950: 2^k + 1 - 2^k gives 1 for k <= 24 and 0 from k = 25, whether
    // the 1 is a product or the accumulator); with a running sum passed in,
    // every step could lose small products against the whole sum so far.
    // From zero, a step's error is bounded by its own products.
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    auto clear = [](f32x4(&v)[Q][NT][2]) {
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int t = 0; t < NT; ++t) v[q][t][0] = v[q][t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    int folds = 0;  // chunks added to the totals so far (uniform)
    auto fold = [&]() {
        if constexpr (FRESH) {
            if (folds == 0) {  // the first chunk is the total
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        tot[q][t][0] = acc[q][t][0];
                        tot[q][t][1] = acc[q][t][1];
                    }
            } else {
#pragma unroll
                for (int q = 0; q < Q; ++q)
#pragma unroll
                    for (int t = 0; t < NT; ++t)
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const f32x4 a = acc[q][t][h], s = tot[q][t][h];
                            const f32x4 sum = s + a;
                            const f32x4 z = sum - s;
                            cmp[q][t][h] += (s - (sum - z)) + (a - z);
                            tot[q][t][h] = sum;
                        }
            }
            ++folds;
            clear(acc);
        }
    };
    clear(acc);
    if constexpr (FRESH) clear(cmp);  // tot is set by the first fold
    int c = rg.first;
    if constexpr (FEW) {
        // X operands straight from memory: lane (column r, group g)
        const S* xcol = X + (int64_t)(r < nvec ? r : nvec - 1) * K + 8 * g;
        for (; c + CH <= s1; c += CH) {
            // step by step, A then X: step i's MFMAs wait for its own four loads
            // only (all X operands first measured 7.77 against 6.99 µs at 2 vectors)
            quad a[Q][CH], b[2][CH];
#pragma unroll
            for (int i = 0; i < CH; ++i) {
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    a[q][i] = __builtin_nontemporal_load(reinterpret_cast<const quad*>(ap[q] + (int64_t)(c + i) * 64));
                b[0][i] = *reinterpret_cast<const quad*>(xcol + (int64_t)(c + i) * 64);
                b[1][i] = *reinterpret_cast<const quad*>(xcol + (int64_t)(c + i) * 64 + 32);
            }
            __builtin_amdgcn_sched_barrier(0);  // all loads of the chunk in flight first
#pragma unroll
            for (int i = 0; i < CH; ++i)
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    acc[q][0][0] += mma_16x16x32(D{}, a[q][i], b[0][i], zero4);
                    acc[q][0][1] += mma_16x16x32(D{}, a[q][i], b[1][i], zero4);
                }
            fold();
        }
    } else {
        // groups of G steps, X of the group (kCols columns × G steps) before A
        // of the group: with up to two tiles one step per group, so that a
        // step's MFMAs wait for its own X only (fp16 4096 × 4096, µs, whole
        // chunk / 2 steps / 1 step: 16 vectors 8.38 / 8.07 / 7.82, 24
        // vectors 10.12 (2 steps) / 9.52); with four tiles the whole chunk
        // (64 vectors 14.11 against 15.02 one step at a time)
        constexpr int G = NT <= 2 ? 1 : CH;
        constexpr int kGroups = CH / G;
        constexpr int kXLoads = kCols * G / 8;  // 1 KiB loads per group: 64/(8G) columns each
        constexpr int kColsPerLoad = 64 / (8 * G);
        static_assert(CH % G == 0 && kColsPerLoad * 8 * G == 64, "group shape");
        for (; c + CH <= s1; c += CH) {
            quad xv[kGroups][kXLoads], a[Q][CH];
#pragma unroll
            for (int k = 0; k < kGroups; ++k) {
#pragma unroll
                for (int u = 0; u < kXLoads; ++u) {
                    const int col = u * kColsPerLoad + lane / (8 * G);
                    const int qq = lane % (8 * G);
                    const int j = col < nvec ? col : nvec - 1;
                    xv[k][u] = *reinterpret_cast<const quad*>(X + (int64_t)j * K + (int64_t)(c + G * k) * 64 + 8 * qq);
                }
#pragma unroll
                for (int i = G * k; i < G * k + G; ++i)
#pragma unroll
                    for (int q = 0; q < Q; ++q)
                        a[q][i] = __builtin_nontemporal_load(reinterpret_cast<const quad*>(ap[q] + (int64_t)(c + i) * 64));
            }
            __builtin_amdgcn_sched_barrier(0);  // all loads of the chunk in flight first
#pragma unroll
            for (int k = 0; k < kGroups; ++k) {
#pragma unroll
                for (int u = 0; u < kXLoads; ++u) {
                    const int col = u * kColsPerLoad + lane / (8 * G);
                    const int qq = lane % (8 * G);
                    xw[col * kColQuads + 8 * G * k + qq] = xv[k][u];
                }
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int i = G * k; i < G * k + G; ++i) {
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const quad b0 = xw[(16 * t + r) * kColQuads + 8 * i + g];
                        const quad b1 = xw[(16 * t + r) * kColQuads + 8 * i + 4 + g];
#pragma unroll
                        for (int q = 0; q < Q; ++q) {
                            acc[q][t][0] += mma_16x16x32(D{}, a[q][i], b0, zero4);
                            acc[q][t][1] += mma_16x16x32(D{}, a[q][i], b1, zero4);
                        }
                    }
                }
            }
            fold();
            // the next chunk overwrites this wavefront's LDS region
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    }
    // the rest of the run (fewer than CH steps, the partial last step among
    // them when it is this wavefront's) one step at a time, with X read
    // straight from memory; groups of 8 wholly past K are zero (K % 8 == 0)
    const S* xq[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) xq[t] = X + (int64_t)(16 * t + r < nvec ? 16 * t + r : 0) * K + 8 * g;
    const int c_left = c;
#pragma unroll 1
    for (; __builtin_expect(c < rg.end, 0); ++c) {  // (out of line: rare)
        const int e = c * 64;
        const bool ina = e + 32 * half + 8 * g < K;
        quad a[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q)
            a[q] = ina ? *reinterpret_cast<const quad*>(ap[q] + (int64_t)e) : zero;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bool col = 16 * t + r < nvec;
            const quad b0 = (col && e + 8 * g < K) ? *reinterpret_cast<const quad*>(xq[t] + e) : zero;
            const quad b1 = (col && e + 32 + 8 * g < K) ? *reinterpret_cast<const quad*>(xq[t] + e + 32) : zero;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                acc[q][t][0] += mma_16x16x32(D{}, a[q], b0, zero4);
                acc[q][t][1] += mma_16x16x32(D{}, a[q], b1, zero4);
            }
        }
    }

    if (c > c_left) fold();  // the leftover steps, if any ran
    if constexpr (FRESH) {
        if (folds > 1) {
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h) acc[q][t][h] = tot[q][t][h] + cmp[q][t][h];
        } else if (folds == 1) {
#pragma unroll
            for (int q = 0; q < Q; ++q)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    acc[q][t][0] = tot[q][t][0];
                    acc[q][t][1] = tot[q][t][1];
                }
        }  // no steps: acc is zero
    }

    // lane (column j, group g) holds operand rows 4g .. 4g+3, i.e. real rows
    // 2g (halves 0, 1) and 2g+1 of each row group: pair them up, row groups
    // 2p and 2p + 1 in partial quad p
    f32x4* partial = reinterpret_cast<f32x4*>(xw);  // this wavefront's region, now free
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int pp = 0; pp < kPairs; ++pp) {
            f32x4 v;
            v[0] = acc[2 * pp][t][0][0] + acc[2 * pp][t][1][1];
            v[1] = acc[2 * pp][t][0][2] + acc[2 * pp][t][1][3];
            if constexpr (Q >= 2) {
                v[2] = acc[2 * pp + 1][t][0][0] + acc[2 * pp + 1][t][1][1];
                v[3] = acc[2 * pp + 1][t][0][2] + acc[2 * pp + 1][t][1][3];
            } else {
                v[2] = v[3] = 0.f;  // no second row group
            }
            partial[(t * kPairs + pp) * 64 + lane] = v;
        }
    __syncthreads();
    if (wave == 0) {
        // lane (column j0, quad gq) finishes rows 16·p + 4·gq .. 16·p + 4·gq
        // + 3 of column j0 for each pair p of row groups: rows 4·gq, 4·gq + 1
        // of the pair sit in the partials of lane (j0, 2·(gq % 2)), rows
        // 4·gq + 2, 4·gq + 3 in those of lane (j0, 2·(gq % 2) + 1), as
        // components 2·(gq / 2) and 2·(gq / 2) + 1
        const int j0 = lane >> 2;
        const int gq = lane & 3;
        const int srcA = 32 * (gq & 1) + j0;
        const int srcB = srcA + 16;
        const int co = 2 * (gq >> 1);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int pp = 0; pp < kPairs; ++pp) {
            float o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float* P = reinterpret_cast<const float*>(reinterpret_cast<const f32x4*>(xs[w]) +
                                                                (t * kPairs + pp) * 64);
                o[0] += P[srcA * 4 + co];
                o[1] += P[srcA * 4 + co + 1];
                o[2] += P[srcB * 4 + co];
                o[3] += P[srcB * 4 + co + 1];
            }
            const int j = 16 * t + j0;
            const int64_t m0 = row0 + 16 * pp + 4 * gq;
            if (j < nvec && 16 * pp + 4 * gq < RG * Q) {
                float* yp = Y + (int64_t)j * M + m0;
                if (m0 + 3 < M && ((uintptr_t)yp & 15) == 0) {
                    f32x4 out = {o[0], o[1], o[2], o[3]};
                    if (bias != nullptr) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) out[i] += bias[m0 + i];
                    }
                    *reinterpret_cast<f32x4*>(yp) = out;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (m0 + i < M) yp[i] = o[i] + (bias != nullptr ? bias[m0 + i] : 0.f);
                }
            }
        }
    }
}

// Gated pair on one pass over two matrices: h[m] = silu(g[m]) · u[m] with
// g = A_gate·x, u = A_up·x and silu(g) = g / (1 + e^(-g)): the gate and up
// projections of an FFN fused with their activation (the NPU MatMul essay,
// sections 4.2 and 5.1, fuses an FFN's MatMuls with the activation; SiLU is
// the gated activation of the decode shapes here).  W wavefronts share a
// row pair (W = 1: one wavefront, no LDS); both rows' chunks are loaded
// together against the same x chunks, so x is read once for the pair.
template <class D, int W, int BATCH, bool VEC>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_gated_silu_kernel(const typename D::storage* Ag, const typename D::storage* Au, int64_t lda,
                       float* h, int64_t M, const typename D::storage* __restrict__ x, int K) {
    using S = typename D::storage;
    using C = Chunk<D, VEC>;
    constexpr int L = W * 64;
    constexpr int E = C::elems;
    __shared__ float partial[W][2];

    const int64_t row = blockIdx.x;
    if (row >= M) return;  // uniform across the workgroup
    const int sub = threadIdx.x;
    const S* const rps[2] = {Ag + row * lda, Au + row * lda};

    Sum2 sum[2] = {Sum2{0.f, 0.f}, Sum2{0.f, 0.f}};
    const int nfull = K / E;
    const int nsafe = nfull - nfull % (BATCH * L);
    int c0 = 0;
    for (; c0 < nsafe; c0 += BATCH * L) rows_batch<C, L, 2, BATCH, false>(rps, x, c0 + sub, nfull, sum);
    if (c0 < nfull) rows_batch<C, L, 2, BATCH, true>(rps, x, c0 + sub, nfull, sum);
    if constexpr (VEC) {
        float tail[2] = {0.f, 0.f};
        for (int k = nfull * E + sub; k < K; k += L) {
            const float xe = widen(D{}, x[k]);
            tail[0] = __builtin_fmaf(widen(D{}, rps[0][k]), xe, tail[0]);
            tail[1] = __builtin_fmaf(widen(D{}, rps[1][k]), xe, tail[1]);
        }
        sum[0].add(tail[0]);
        sum[1].add(tail[1]);
    }

    float g = segment_sum<64>(sum[0].value());
    float u = segment_sum<64>(sum[1].value());
    if constexpr (W > 1) {
        if ((threadIdx.x & 63) == 0) {
            partial[threadIdx.x >> 6][0] = g;
            partial[threadIdx.x >> 6][1] = u;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            g = partial[0][0];
            u = partial[0][1];
#pragma unroll
            for (int w = 1; w < W; ++w) {
                g += partial[w][0];
                u += partial[w][1];
            }
        }
    }
    if (threadIdx.x == 0) h[row] = g / (1.f + expf(-g)) * u;
}

// Read probe: streams `n16` 16-byte units once, the way the GEMV kernels
// stream A (64-lane wavefronts, 8 nontemporal 1 KiB loads in flight each,
// 4 wavefronts per workgroup, consecutive blocks to consecutive workgroups),
// and writes nothing: the loaded words are folded into one value that is
// stored only if it equals a constant the data cannot be expected to
// produce, so the loads stay live.  It measures what streaming the bytes
// alone costs on this GPU, the practical ceiling for a GEMV of those bytes.
__global__ void __launch_bounds__(kRowsWaves * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_read_probe_kernel(const quad* __restrict__ p, int64_t n16, unsigned* sink) {
    constexpr int kLoads = 8;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * kRowsWaves + (threadIdx.x >> 6);
    const int64_t base = wave * kLoads * 64 + lane;
    quad v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const int64_t q = base + (int64_t)i * 64;
        v[i] = __builtin_nontemporal_load(p + (q < n16 ? q : n16 - 1));
    }
    __builtin_amdgcn_sched_barrier(0);
    unsigned acc = 0;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

// Read-probe variants, for mapping what streaming a buffer costs on this
// GPU against the read pattern (the table of patterns the GEMV families are
// chosen from): LOADS 16-byte loads per lane in flight (LOADS KiB per
// wavefront), W wavefronts per workgroup, CACHED plain instead of
// nontemporal loads, PRIO the wavefront's priority raised while it issues
// its loads.  Each wavefront streams `blocks` blocks of LOADS KiB: with
// `stride` the grid walks the buffer together (block b of wavefront w is
// block w + b·(number of wavefronts)), otherwise each wavefront takes
// `blocks` consecutive blocks.  With `times`, lane 0 of every wavefront
// writes its start and end (the GPU's constant-rate real-time counter) to
// times[2w], times[2w + 1] with ordinary vector stores.  Nothing else is
// written (see gemv_read_probe_kernel).
template <int LOADS, int W, bool CACHED, bool PRIO>
__global__ void __launch_bounds__(W * 64)
gemv_read_probe_variant_kernel(const quad* __restrict__ p, int64_t n16, unsigned* sink, int blocks,
                               int stride, unsigned long long* times) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * W + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * W;
    unsigned long long t0 = 0;
    if (times != nullptr) t0 = __builtin_amdgcn_s_memrealtime();
    unsigned acc = 0;
    for (int b = 0; b < blocks; ++b) {
        const int64_t blk = stride ? wave + (int64_t)b * waves : wave * blocks + b;
        const int64_t base = blk * LOADS * 64 + lane;
        quad v[LOADS];
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(3);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int64_t q = base + (int64_t)i * 64;
            const quad* a = p + (q < n16 ? q : n16 - 1);
            if constexpr (CACHED)
                v[i] = *a;
            else
                v[i] = __builtin_nontemporal_load(a);
        }
        if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < LOADS; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
    if (times != nullptr) {
        // read once every load has arrived (acc needed them all; the fence
        // keeps the counter read after it)
        __builtin_amdgcn_sched_barrier(0);
        const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
        if (lane == 0) {
            times[2 * wave] = t0;
            times[2 * wave + 1] = t1;
        }
    }
}

}  // namespace gemvdev
