// Device building blocks for the gfx950 GEMV kernels: element types, loads,
// per-chunk dot products and wavefront segment reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gemvdev {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as four 32-bit words: a native vector type (not HIP's uint4
// struct), so that selects between quads stay in registers
typedef unsigned int quad __attribute__((ext_vector_type(4)));
// The same 16 bytes read from any address (rows whose pitch is not a whole
// number of 16-byte loads): one global_load_dwordx4 all the same, global
// memory being accessed in the GPU's unaligned mode; a load that crosses a
// cache line costs the line it crosses into.
typedef unsigned int quad_any __attribute__((ext_vector_type(4), aligned(1)));

// Element types.  `storage` is what sits in memory; products are formed and
// summed in fp32 (page "GEMM、GEMV、dtype 与算术强度", section "dtype 改变什么":
// half-precision inputs with a wider accumulator).
struct TF32 {
    using storage = float;
    using xstorage = float;  // x has the matrix's type
    static constexpr int bytes = 4;
};
struct TF16 {
    using storage = uint16_t;
    using xstorage = uint16_t;
    static constexpr int bytes = 2;
};
struct TBF16 {
    using storage = uint16_t;
    using xstorage = uint16_t;
    static constexpr int bytes = 2;
};
// Weight-only int8: the matrix holds int8 weights (one fp32 scale per row is
// applied after the row's sum), x stays in the float type X (the lqnn.cn NPU
// MatMul essay, section 1.2: int8 weights, fp16 activations, an fp32
// accumulator).  One 16-byte load carries 16 weights.
template <class X>
struct TQ8 {
    using storage = int8_t;
    using xstorage = typename X::storage;
    using xtype = X;
    static constexpr int bytes = 1;
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

// The tail loops read A and x element by element; for the float types both
// are widened alike, for int8 weights the weight is an integer.
template <class D>
__device__ __forceinline__ float widen_a(D, typename D::storage v) { return widen(D{}, v); }
template <class D>
__device__ __forceinline__ float widen_x(D, typename D::xstorage v) { return widen(D{}, v); }
template <class X>
__device__ __forceinline__ float widen_a(TQ8<X>, int8_t q) { return (float)q; }
template <class X>
__device__ __forceinline__ float widen_x(TQ8<X>, typename X::storage v) { return widen(X{}, v); }

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
        return *reinterpret_cast<const quad_any*>(p + c * elems);
    }
    __device__ __forceinline__ static type stream(const typename D::storage* p, int64_t c) {
        return __builtin_nontemporal_load(reinterpret_cast<const quad_any*>(p + c * elems));
    }
    __device__ __forceinline__ static type zero() { return quad{0u, 0u, 0u, 0u}; }
    using xtype = type;  // x chunks are A chunks
    __device__ __forceinline__ static type keep_a(bool ok, type v) { return ok ? v : zero(); }
    __device__ __forceinline__ static type keep_x(bool ok, type v) { return ok ? v : zero(); }
    __device__ __forceinline__ static float dot(type a, type x, float acc) {
        return chunk_dot(D{}, a, x, acc);
    }
    // the chunk as `words` steps, in element order: dot(a, x, acc) is
    // dot_word(a, x, words - 1, ... dot_word(a, x, 0, acc)) (2-byte elements)
    static constexpr int words = 4;
    __device__ __forceinline__ static float dot_word(type a, type x, int w, float acc) {
        return pair_dot(D{}, a[w], x[w], acc);
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
    using xtype = type;
    __device__ __forceinline__ static type keep_a(bool ok, type v) { return ok ? v : zero(); }
    __device__ __forceinline__ static type keep_x(bool ok, type v) { return ok ? v : zero(); }
    __device__ __forceinline__ static float dot(type a, type x, float acc) {
        return __builtin_fmaf(widen(D{}, a), widen(D{}, x), acc);
    }
    static constexpr int words = 1;
    __device__ __forceinline__ static float dot_word(type a, type x, int, float acc) {
        return dot(a, x, acc);
    }
};

// int8 weights: a chunk is 16 weights (one 16-byte quad, nontemporal) and
// the 16 matching x elements (32 bytes of fp16/bf16 or 64 of fp32, cached),
// held as native vectors so that selects stay in registers.
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x16 __attribute__((ext_vector_type(16)));

// weight i (0..3) of a 32-bit word, sign-extended and converted exactly
__device__ __forceinline__ float q8_at(uint32_t w, int i) {
    return (float)(int)(int8_t)(uint8_t)(w >> (8 * i));
}
// x element e of a chunk: one word holds two half-width or one fp32 element
__device__ __forceinline__ float x_at(TF16, u32x8 x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? hi_f16(w) : lo_f16(w);
}
__device__ __forceinline__ float x_at(TBF16, u32x8 x, int e) {
    const uint32_t w = x[e >> 1];
    return (e & 1) ? hi_bf16(w) : lo_bf16(w);
}
__device__ __forceinline__ float x_at(TF32, u32x16 x, int e) { return f32_of(x[e]); }

template <class X>
struct Chunk<TQ8<X>, true> {
    using type = quad;
    using xtype = typename std::conditional<X::bytes == 4, u32x16, u32x8>::type;
    static constexpr int elems = 16;
    __device__ __forceinline__ static xtype load(const typename X::storage* p, int64_t c) {
        return *reinterpret_cast<const xtype*>(p + c * elems);
    }
    __device__ __forceinline__ static type stream(const int8_t* p, int64_t c) {
        return __builtin_nontemporal_load(reinterpret_cast<const quad_any*>(p + c * elems));
    }
    __device__ __forceinline__ static type zero() { return quad{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ static type keep_a(bool ok, type v) { return ok ? v : zero(); }
    __device__ __forceinline__ static xtype keep_x(bool ok, xtype v) { return ok ? v : xtype(0u); }
    // acc + Σ q_e·x_e over the 16 weights, in weight order, IEEE fp32 FMA
    __device__ __forceinline__ static float dot(type a, xtype x, float acc) {
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc = __builtin_fmaf(q8_at(a[w], i), x_at(X{}, x, 4 * w + i), acc);
        return acc;
    }
};
template <class X>
struct Chunk<TQ8<X>, false> {
    using type = int8_t;
    using xtype = typename X::storage;
    static constexpr int elems = 1;
    __device__ __forceinline__ static xtype load(const xtype* p, int64_t c) { return p[c]; }
    __device__ __forceinline__ static type stream(const int8_t* p, int64_t c) {
        return __builtin_nontemporal_load(p + c);
    }
    __device__ __forceinline__ static type zero() { return type(0); }
    __device__ __forceinline__ static type keep_a(bool ok, type v) { return ok ? v : type(0); }
    __device__ __forceinline__ static xtype keep_x(bool ok, xtype v) { return ok ? v : xtype(0); }
    __device__ __forceinline__ static float dot(type a, xtype x, float acc) {
        return __builtin_fmaf((float)a, widen(X{}, x), acc);
    }
};

// A running fp32 sum that carries the rounding error of every addition
// (Knuth's error-free two-sum: s + a = t + e exactly, with t = fl(s + a)),
// for adding the partial sums of a lane's batches of loads: the error of the
// result is about one rounding of the total plus (n·2^-24)² of the sum of
// |partials| over n additions, instead of growing with n, so the rounding
// chain of a long row stays bounded (page "GEMM、GEMV、dtype 与算术强度",
// section "dtype 改变什么": the accumulator must keep what the inputs carry).
struct Sum2 {
    float s;
    float c;
    __device__ __forceinline__ void add(float a) {
        const float t = s + a;
        const float z = t - s;
        c += (s - (t - z)) + (a - z);
        s = t;
    }
    __device__ __forceinline__ float value() const { return s + c; }
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

// Sums across 16-lane rows with the gfx950 row-swap instructions: swapping
// the odd rows of one copy of v with the even rows of another leaves the
// even row's values in the first copy and the odd row's in the second, in
// both rows of each pair, so their sum is the xor-16 butterfly step (and
// likewise with the two 32-lane halves for xor-32).  Both lanes of a pair add
// the same two values in the same order.
__device__ __forceinline__ float row_pair_sum16(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float half_pair_sum32(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Sum over each aligned segment of L lanes (L a power of two, 1..64); every
// lane of the segment receives the same, bit-identical total.  Every lane of
// the wavefront must execute this (no lane may be inactive).  After the two
// quad steps all four lanes of a quad hold the quad sum, so the mirrors act
// as the xor-4 and xor-8 butterfly steps; the 32- and 64-lane steps swap
// 16-lane rows and 32-lane halves between registers (v_permlane16_swap,
// v_permlane32_swap), without a round trip through the LDS crossbar.
template <int L>
__device__ __forceinline__ float segment_sum(float v) {
    if constexpr (L >= 2) v += dpp<kDppSwapAdjacent>(v);
    if constexpr (L >= 4) v += dpp<kDppSwapPairs>(v);
    if constexpr (L >= 8) v += dpp<kDppHalfRowMirror>(v);
    if constexpr (L >= 16) v += dpp<kDppRowMirror>(v);
    if constexpr (L >= 32) v = row_pair_sum16(v);
    if constexpr (L >= 64) v = half_pair_sum32(v);
    return v;
}

}  // namespace gemvdev
