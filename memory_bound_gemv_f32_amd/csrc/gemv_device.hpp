// Device building blocks for the gfx950 GEMV kernels: element types, loads,
// per-chunk dot products and wavefront segment reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gemvdev {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as four 32-bit words: a native vector type (not HIP's uint4
// struct), so that selects between quads stay in registers
typedef unsigned int quad __attribute__((ext_vector_type(4)));

// Element types.  `storage` is what sits in memory; products are formed and
// summed in fp32 (page "GEMM、GEMV、dtype 与算术强度", section "dtype 改变什么":
// half-precision inputs with a wider accumulator).
struct TF32 {
    using storage = float;
    static constexpr int bytes = 4;
};
struct TF16 {
    using storage = uint16_t;
    static constexpr int bytes = 2;
};
struct TBF16 {
    using storage = uint16_t;
    static constexpr int bytes = 2;
};

// One stored element widened to fp32 (exact for all three types).
__device__ __forceinline__ float widen(TF32, float v) { return v; }
__device__ __forceinline__ float widen(TF16, uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}
__device__ __forceinline__ float widen(TBF16, uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

__device__ __forceinline__ float f32_of(uint32_t w) { return __builtin_bit_cast(float, w); }

// acc + Σ a_i·x_i over one 16-byte chunk (4 fp32 or 8 half-width elements),
// as a chain of IEEE fp32 fused multiply-adds in element order.  Half-width
// elements are widened exactly first (fp16 -> fp32 folds into v_fma_mix_f32;
// bf16 -> fp32 is a 16-bit shift or mask), so the arithmetic is plain fp32
// with round-to-nearest-even: sign-symmetric and the same on every family.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ float lo_f16(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

__device__ __forceinline__ float chunk_dot(TF32, quad a, quad x, float acc) {
    acc = __builtin_fmaf(f32_of(a.x), f32_of(x.x), acc);
    acc = __builtin_fmaf(f32_of(a.y), f32_of(x.y), acc);
    acc = __builtin_fmaf(f32_of(a.z), f32_of(x.z), acc);
    acc = __builtin_fmaf(f32_of(a.w), f32_of(x.w), acc);
    return acc;
}
__device__ __forceinline__ float pair_dot(TF16, uint32_t a, uint32_t x, float acc) {
    acc = __builtin_fmaf(lo_f16(a), lo_f16(x), acc);
    return __builtin_fmaf(hi_f16(a), hi_f16(x), acc);
}
__device__ __forceinline__ float pair_dot(TBF16, uint32_t a, uint32_t x, float acc) {
    acc = __builtin_fmaf(lo_bf16(a), lo_bf16(x), acc);
    return __builtin_fmaf(hi_bf16(a), hi_bf16(x), acc);
}
template <class D>
__device__ __forceinline__ float chunk_dot(D, quad a, quad x, float acc) {
    acc = pair_dot(D{}, a.x, x.x, acc);
    acc = pair_dot(D{}, a.y, x.y, acc);
    acc = pair_dot(D{}, a.z, x.z, acc);
    acc = pair_dot(D{}, a.w, x.w, acc);
    return acc;
}

// The packed two-element dot products with fp32 accumulation
// (v_dot2_f32_f16 / v_dot2_f32_bf16): one instruction per element pair, for
// the batched kernel where every A element meets up to 16 vectors and VALU
// issue, not memory, is the limit.  Their products are exact, but their
// internal rounding is not IEEE round-to-nearest (measured: negating x does
// not exactly negate the result), which the tolerance absorbs.
// (Each 32-bit word is passed by value before it is reinterpreted: a bit
// cast applied directly to an element of a native vector read element 0.)
__device__ __forceinline__ float dot2_word(TF16, uint32_t a, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, x), acc, false);
}
__device__ __forceinline__ float dot2_word(TBF16, uint32_t a, uint32_t x, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, x), acc,
                                           false);
}
template <class D>
__device__ __forceinline__ float chunk_dot2(D, quad a, quad x, float acc) {
    acc = dot2_word(D{}, a.x, x.x, acc);
    acc = dot2_word(D{}, a.y, x.y, acc);
    acc = dot2_word(D{}, a.z, x.z, acc);
    acc = dot2_word(D{}, a.w, x.w, acc);
    return acc;
}
__device__ __forceinline__ float chunk_dot2(TF32, quad a, quad x, float acc) {
    return chunk_dot(TF32{}, a, x, acc);
}

// One 16×16×32 matrix-core step, D = A·B + C with fp32 accumulation:
// A is 16 rows × 32 k, B is 32 k × 16 columns.  Lane l supplies row (or
// column) l % 16 and the 8 consecutive k of group l / 16 as one 16-byte
// register quad; D comes back as rows 4·(l/16) .. 4·(l/16)+3 of column l % 16.
__device__ __forceinline__ f32x4 mma_16x16x32(TF16, quad a, quad b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_16x16x32(TBF16, quad a, quad b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Chunk = one 16-byte load (VEC) or one element.
template <class D, bool VEC>
struct Chunk;
// `load` is for data that is re-read (x, X); `stream` is for A, which every
// call reads exactly once: a nontemporal load, so A streams past the caches
// instead of evicting the re-read vector.
template <class D>
struct Chunk<D, true> {
    using type = quad;
    static constexpr int elems = 16 / D::bytes;
    __device__ __forceinline__ static type load(const typename D::storage* p, int64_t c) {
        return *reinterpret_cast<const quad*>(p + c * elems);
    }
    __device__ __forceinline__ static type stream(const typename D::storage* p, int64_t c) {
        return __builtin_nontemporal_load(reinterpret_cast<const quad*>(p + c * elems));
    }
    __device__ __forceinline__ static type zero() { return quad{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ static float dot(type a, type x, float acc) {
        return chunk_dot(D{}, a, x, acc);
    }
    __device__ __forceinline__ static float dot2(type a, type x, float acc) {
        return chunk_dot2(D{}, a, x, acc);
    }
};
template <class D>
struct Chunk<D, false> {
    using type = typename D::storage;
    static constexpr int elems = 1;
    __device__ __forceinline__ static type load(const typename D::storage* p, int64_t c) {
        return p[c];
    }
    __device__ __forceinline__ static type stream(const typename D::storage* p, int64_t c) {
        return __builtin_nontemporal_load(p + c);
    }
    __device__ __forceinline__ static type zero() { return type(0); }
    __device__ __forceinline__ static float dot(type a, type x, float acc) {
        return __builtin_fmaf(widen(D{}, a), widen(D{}, x), acc);
    }
    __device__ __forceinline__ static float dot2(type a, type x, float acc) {
        return dot(a, x, acc);
    }
};

// DPP lane exchange within 16-lane rows (bound_ctrl: no lane is disabled).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, true));
}
constexpr int kDppSwapAdjacent = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppSwapPairs = 0x4E;      // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfRowMirror = 0x141; // lane i <- 7 - i within 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane i <- 15 - i within 16 lanes

// Sum over each aligned segment of L lanes (L a power of two, 1..64); every
// lane of the segment receives the same, bit-identical total.  Every lane of
// the wavefront must execute this (no lane may be inactive).  After the two
// quad steps all four lanes of a quad hold the quad sum, so the mirrors act
// as the xor-4 and xor-8 butterfly steps; the 32- and 64-lane steps cross DPP
// rows through the LDS crossbar (ds_bpermute), which uses no LDS storage.
template <int L>
__device__ __forceinline__ float segment_sum(float v) {
    if constexpr (L >= 2) v += dpp<kDppSwapAdjacent>(v);
    if constexpr (L >= 4) v += dpp<kDppSwapPairs>(v);
    if constexpr (L >= 8) v += dpp<kDppHalfRowMirror>(v);
    if constexpr (L >= 16) v += dpp<kDppRowMirror>(v);
    if constexpr (L >= 32) v += __shfl_xor(v, 16, 64);
    if constexpr (L >= 64) v += __shfl_xor(v, 32, 64);
    return v;
}

}  // namespace gemvdev
