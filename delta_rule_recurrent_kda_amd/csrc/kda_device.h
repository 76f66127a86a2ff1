// kda_device.h -- device helpers shared by the scan kernels: bf16 conversion,
// MFMA fragment traits and small wave reductions (gfx950).
//
// MFMA fragment convention: a k-block of 32 is held by lane (r = lane%16,
// g = lane/16) as 8 elements with k = 16*t + 4*g + i (t in {0,1}, i in 0..3); a
// k-block of 16 is the t = 0 half. An accumulator tile holds rows 4*g + i,
// column r, so one or two stacked accumulator tiles are directly a B operand (k
// along their rows) and the A operand of their transpose. Both operands of every
// product use the same k map, so the order of k inside a lane does not matter.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ uint16_t f2bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats to a packed bf16 pair (a in the low half), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// gfx950: a matrix instruction that reads, as its A or B operand, a register written by
// v_cvt_pk_bf16_f32 fewer than 8 wait states earlier can read the register's previous
// contents (measured: wrong, run-to-run varying products; 8 wait states give exact
// results). The compiler leaves only the 2-3 wait states of an ordinary VALU result
// there. Every fragment packed from fp32 that a product reads therefore passes through
// mfma_ready() between the packing and the product: the asm takes the fragments as
// read-write operands, so the packing is issued before it and the products after it, with
// s_nop 7 (8 wait states) in between. One call covers up to four fragments.
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4v as_v(const uint4& u) { return __builtin_bit_cast(u32x4v, u); }
__device__ __forceinline__ u32x2v as_v(const uint2& u) { return __builtin_bit_cast(u32x2v, u); }
template <typename T> __device__ __forceinline__ void from_v(T& u, const decltype(as_v(u))& x) {
    u = __builtin_bit_cast(T, x);
}
template <typename A> __device__ __forceinline__ void mfma_ready(A& a) {
    auto x = as_v(a);
    asm volatile("s_nop 7" : "+v"(x));
    from_v(a, x);
}
template <typename A, typename B> __device__ __forceinline__ void mfma_ready(A& a, B& b) {
    auto x = as_v(a);
    auto y = as_v(b);
    asm volatile("s_nop 7" : "+v"(x), "+v"(y));
    from_v(a, x);
    from_v(b, y);
}
template <typename A, typename B, typename C, typename D>
__device__ __forceinline__ void mfma_ready(A& a, B& b, C& c, D& d) {
    auto x = as_v(a);
    auto y = as_v(b);
    auto z = as_v(c);
    auto t = as_v(d);
    asm volatile("s_nop 7" : "+v"(x), "+v"(y), "+v"(z), "+v"(t));
    from_v(a, x);
    from_v(b, y);
    from_v(c, z);
    from_v(d, t);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier for handing LDS data between waves: wait for this wave's LDS
// operations, then s_barrier. Global loads already issued stay in flight (a full
// __syncthreads also waits for them through its workgroup fence, which would
// expose the latency of every prefetch at the next barrier). The memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// element-type traits: storage type E, MFMA fragments and products
// ---------------------------------------------------------------------------
template <typename E> struct Elt;

template <> struct Elt<uint16_t> {            // bf16 data
    struct Frag { uint4 u; };                 // k-block of 32
    struct Frag16 { uint2 u; };               // k-block of 16
    static constexpr int kVec = 8;            // elements per 16-byte vector
    using Vec = uint4;
    __device__ static float to_f(uint16_t x) { return bf2f(x); }
    __device__ static uint16_t from_f(float x) { return f2bf(x); }
    __device__ static Frag load(const uint16_t* row, int g) {
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * g);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 16 + 4 * g);
        return Frag{make_uint4(lo.x, lo.y, hi.x, hi.y)};
    }
    __device__ static Frag16 load16(const uint16_t* row, int g) {
        return Frag16{*reinterpret_cast<const uint2*>(row + 4 * g)};
    }
    __device__ static Frag from_acc(const f32x4& a0, const f32x4& a1) {
        return Frag{make_uint4(pack2(a0[0], a0[1]), pack2(a0[2], a0[3]), pack2(a1[0], a1[1]),
                               pack2(a1[2], a1[3]))};
    }
    __device__ static Frag16 from_acc16(const f32x4& a0) {
        return Frag16{make_uint2(pack2(a0[0], a0[1]), pack2(a0[2], a0[3]))};
    }
    // fragments packed by from_acc / from_acc16 before a product reads them (mfma_ready)
    __device__ static void ready(Frag& a) { mfma_ready(a.u); }
    __device__ static void ready(Frag16& a) { mfma_ready(a.u); }
    __device__ static void ready(Frag& a, Frag& b) { mfma_ready(a.u, b.u); }
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.u),
                                                       __builtin_bit_cast(bf16x8, b.u), c, 0, 0, 0);
    }
    __device__ static f32x4 mma16(const Frag16& a, const Frag16& b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a.u),
                                                         __builtin_bit_cast(s16x4, b.u), c, 0, 0, 0);
    }
    __device__ static void unpack(const Vec& v, float (&f)[8]) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(w[j] << 16);
            f[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
        }
    }
    // 8 values to a row of LDS whose rows are 8-byte aligned
    __device__ static void store_vec(uint16_t* dst, const float (&f)[8]) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(f[0], f[1]), pack2(f[2], f[3]));
        *reinterpret_cast<uint2*>(dst + 4) = make_uint2(pack2(f[4], f[5]), pack2(f[6], f[7]));
    }
    // n consecutive values (n = 2 or 4)
    template <int N> __device__ static void store_run(uint16_t* dst, const float* f) {
        if constexpr (N == 4) *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(f[0], f[1]), pack2(f[2], f[3]));
        else *reinterpret_cast<uint32_t*>(dst) = pack2(f[0], f[1]);
    }
    __device__ static void store4(uint16_t* dst, const f32x4& a) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(a[0], a[1]), pack2(a[2], a[3]));
    }
};

template <> struct Elt<float> {               // fp32 data
    struct Frag { float4 lo, hi; };
    struct Frag16 { float4 lo; };
    static constexpr int kVec = 4;
    using Vec = float4;
    __device__ static float to_f(float x) { return x; }
    __device__ static float from_f(float x) { return x; }
    __device__ static Frag load(const float* row, int g) {
        return Frag{*reinterpret_cast<const float4*>(row + 4 * g),
                    *reinterpret_cast<const float4*>(row + 16 + 4 * g)};
    }
    __device__ static Frag16 load16(const float* row, int g) {
        return Frag16{*reinterpret_cast<const float4*>(row + 4 * g)};
    }
    __device__ static Frag from_acc(const f32x4& a0, const f32x4& a1) {
        return Frag{make_float4(a0[0], a0[1], a0[2], a0[3]), make_float4(a1[0], a1[1], a1[2], a1[3])};
    }
    __device__ static Frag16 from_acc16(const f32x4& a0) {
        return Frag16{make_float4(a0[0], a0[1], a0[2], a0[3])};
    }
    // fp32 fragments are not converted: nothing to wait for
    __device__ static void ready(Frag&) {}
    __device__ static void ready(Frag16&) {}
    __device__ static void ready(Frag&, Frag&) {}
    __device__ static f32x4 mma4(const float4& a, const float4& b, f32x4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, c, 0, 0, 0);
        return c;
    }
    __device__ static f32x4 mma(const Frag& a, const Frag& b, f32x4 c) {
        return mma4(a.hi, b.hi, mma4(a.lo, b.lo, c));
    }
    __device__ static f32x4 mma16(const Frag16& a, const Frag16& b, f32x4 c) { return mma4(a.lo, b.lo, c); }
    __device__ static void unpack(const Vec& v, float (&f)[4]) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
    __device__ static void store_vec(float* dst, const float (&f)[4]) {
        *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
    }
    template <int N> __device__ static void store_run(float* dst, const float* f) {
        if constexpr (N == 4) *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
        else *reinterpret_cast<float2*>(dst) = make_float2(f[0], f[1]);
    }
    __device__ static void store4(float* dst, const f32x4& a) {
        *reinterpret_cast<float4*>(dst) = make_float4(a[0], a[1], a[2], a[3]);
    }
};

// Sum N per-lane values over 2*MASK consecutive lanes (a power of two dividing 64).
// On return every lane holds the total of value index reduce_index<N, 2*MASK>(lane).
template <int N, int MASK>
__device__ __forceinline__ float reduce_scatter(const float* v, int lane)
{
    if constexpr (N == 1) {
        float x = v[0];
#pragma unroll
        for (int m = MASK; m >= 1; m >>= 1) x += __shfl_xor(x, m);
        return x;
    } else {
        const bool up = (lane & MASK) != 0;
        float w[N / 2];
#pragma unroll
        for (int j = 0; j < N / 2; ++j) {
            const float send = up ? v[j] : v[j + N / 2];
            const float keep = up ? v[j + N / 2] : v[j];
            w[j] = keep + __shfl_xor(send, MASK);
        }
        return reduce_scatter<N / 2, MASK / 2>(w, lane);
    }
}
template <int N, int W>
__device__ __forceinline__ int reduce_index(int lane)
{
    int idx = 0;
#pragma unroll
    for (int n = N / 2, m = W / 2; n >= 1; n /= 2, m /= 2)
        if (lane & m) idx += n;
    return idx;
}

}  // namespace dev
}  // namespace kda
