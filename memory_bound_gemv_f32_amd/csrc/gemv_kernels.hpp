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
//   * A is streamed once with coalesced loads: the lanes that share a row
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
//     "第 3 课", section "B. 向量 x 的高速片上缓存复用");
//   * rows past M in the last wavefront clamp their loads to row M-1, take
//     part in the reduction, and do not write.
#pragma once

#include "gemv_device.hpp"

namespace gemvdev {

// Rows-per-wave (L < 64) and wave-per-row (L == 64) kernel.
// A wavefront covers R = 64/L rows per row tile and takes U consecutive row
// tiles; lanes sub = lane % L of one row walk its chunks with stride L, BATCH
// chunks in flight per row tile.
template <class D, int L, int U, int BATCH, bool VEC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
gemv_rows_kernel(const typename D::storage* __restrict__ A, int64_t lda,
                 const typename D::storage* __restrict__ x,
                 const float* __restrict__ bias, float* __restrict__ y, int M,
                 int K) {
    using S = typename D::storage;
    using C = Chunk<D, VEC>;
    using CT = typename C::type;
    constexpr int R = 64 / L;
    constexpr int E = C::elems;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane & (L - 1);
    const int slot = lane / L;
    const int64_t tile0 = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * U;

    int64_t row[U];
    const S* rp[U];
    float b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        row[u] = (tile0 + u) * R + slot;
        const int64_t safe = row[u] < M ? row[u] : (int64_t)M - 1;
        rp[u] = A + safe * lda;
        b[u] = 0.f;
        if (bias != nullptr && sub == 0 && row[u] < M) b[u] = bias[row[u]];
    }

    float acc[U][2];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u][0] = acc[u][1] = 0.f;

    const int nfull = K / E;  // whole chunks per row
    for (int c0 = 0; c0 < nfull; c0 += BATCH * L) {
        CT a[U][BATCH];
        CT xv[BATCH];
        bool ok[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int c = c0 + i * L + sub;
            ok[i] = c < nfull;
            const int cc = ok[i] ? c : nfull - 1;
#pragma unroll
            for (int u = 0; u < U; ++u) a[u][i] = C::load(rp[u], cc);
            xv[i] = C::load(x, cc);
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const CT xi = ok[i] ? xv[i] : C::zero();
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const CT ai = ok[i] ? a[u][i] : C::zero();
                acc[u][i & 1] = C::dot(ai, xi, acc[u][i & 1]);
            }
        }
    }
    if constexpr (VEC) {
        // elements past the last whole chunk (fewer than E of them)
        for (int k = nfull * E + sub; k < K; k += L) {
            const float xe = widen(D{}, x[k]);
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u][1] = __builtin_fmaf(widen(D{}, rp[u][k]), xe, acc[u][1]);
        }
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const float v = segment_sum<L>(acc[u][0] + acc[u][1]);
        if (sub == 0 && row[u] < M) y[row[u]] = v + b[u];
    }
}

// Workgroup-per-row kernel: W wavefronts (64·W lanes) share one row; each
// wavefront reduces its lanes, writes one partial to LDS, and after one
// barrier thread 0 adds the W partials in wavefront order, adds the bias and
// writes y[row] (page "第 3 课", the block-reduction structure of section
// "C. 点积规约与原子写入解耦" on 64-lane wavefronts).
template <class D, int W, int BATCH, bool VEC>
__global__ void __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(4)))
gemv_group_kernel(const typename D::storage* __restrict__ A, int64_t lda,
                  const typename D::storage* __restrict__ x,
                  const float* __restrict__ bias, float* __restrict__ y, int M,
                  int K) {
    using S = typename D::storage;
    using C = Chunk<D, VEC>;
    using CT = typename C::type;
    constexpr int L = W * 64;
    constexpr int E = C::elems;
    __shared__ float partial[W];

    const int64_t row = blockIdx.x;
    if (row >= M) return;  // uniform across the workgroup
    const int sub = threadIdx.x;
    const S* rp = A + row * lda;
    float b = 0.f;
    if (bias != nullptr && sub == 0) b = bias[row];

    float acc[2] = {0.f, 0.f};
    const int nfull = K / E;
    for (int c0 = 0; c0 < nfull; c0 += BATCH * L) {
        CT a[BATCH];
        CT xv[BATCH];
        bool ok[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int c = c0 + i * L + sub;
            ok[i] = c < nfull;
            const int cc = ok[i] ? c : nfull - 1;
            a[i] = C::load(rp, cc);
            xv[i] = C::load(x, cc);
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const CT ai = ok[i] ? a[i] : C::zero();
            const CT xi = ok[i] ? xv[i] : C::zero();
            acc[i & 1] = C::dot(ai, xi, acc[i & 1]);
        }
    }
    if constexpr (VEC) {
        for (int k = nfull * E + sub; k < K; k += L)
            acc[1] = __builtin_fmaf(widen(D{}, rp[k]), widen(D{}, x[k]), acc[1]);
    }

    const float v = segment_sum<64>(acc[0] + acc[1]);
    if ((threadIdx.x & 63) == 0) partial[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float s = partial[0];
#pragma unroll
        for (int w = 1; w < W; ++w) s += partial[w];
        y[row] = s + b;
    }
}

// Batched kernel: Y = A·X (+ bias) for NV right-hand vectors with one pass
// over A.  A wavefront owns RB consecutive rows; its lanes walk the chunks of
// those rows with stride 64, and every A chunk is multiplied against the
// same chunk of all NV columns of X (X is K×NV column-major and stays in the
// caches).  RB·NV fp32 accumulators per lane, one 64-lane reduction each, and
// lane 0 writes the RB·NV outputs.
template <class D, int NV, int RB, int BATCH, bool VEC>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
gemv_batched_kernel(const typename D::storage* __restrict__ A, int64_t lda,
                    const typename D::storage* __restrict__ X,
                    const float* __restrict__ bias, float* __restrict__ Y,
                    int M, int K) {
    using S = typename D::storage;
    using C = Chunk<D, VEC>;
    using CT = typename C::type;
    constexpr int E = C::elems;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row0 = ((int64_t)blockIdx.x * (blockDim.x >> 6) + wave) * RB;

    const S* rp[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t m = row0 + r;
        rp[r] = A + (m < M ? m : (int64_t)M - 1) * lda;
    }

    float acc[RB][NV];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int j = 0; j < NV; ++j) acc[r][j] = 0.f;

    const int nfull = K / E;
#pragma unroll 1
    for (int c0 = 0; c0 < nfull; c0 += BATCH * 64) {
        CT a[RB][BATCH];
        bool ok[BATCH];
        int cc[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int c = c0 + i * 64 + lane;
            ok[i] = c < nfull;
            cc[i] = ok[i] ? c : nfull - 1;
#pragma unroll
            for (int r = 0; r < RB; ++r) a[r][i] = C::load(rp[r], cc[i]);
        }
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                CT xv = C::load(X + (int64_t)j * K, cc[i]);
                xv = ok[i] ? xv : C::zero();
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const CT ar = ok[i] ? a[r][i] : C::zero();
                    acc[r][j] = C::dot2(ar, xv, acc[r][j]);
                }
            }
        }
    }
    if constexpr (VEC) {
        for (int k = nfull * E + lane; k < K; k += 64) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const float xe = widen(D{}, X[(int64_t)j * K + k]);
#pragma unroll
                for (int r = 0; r < RB; ++r)
                    acc[r][j] = __builtin_fmaf(widen(D{}, rp[r][k]), xe, acc[r][j]);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int64_t m = row0 + r;
        const float b = (bias != nullptr && m < M) ? bias[m] : 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const float v = segment_sum<64>(acc[r][j]);
            if (lane == 0 && m < M) Y[(int64_t)j * M + m] = v + b;
        }
    }
}

}  // namespace gemvdev
