// device_common.h -- gfx950 device helpers shared by the library's kernels:
// bf16 <-> fp32 conversion, 8-element vector loads/stores, dot products and the
// wavefront reduce-scatter used by the BGMV shrink.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace lora {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 is the upper half of an IEEE float: widening is a shift (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> two bf16 (round to nearest even; one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Dot product of two packed bf16 pairs accumulated in fp32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// n / d for 0 <= n, 1 <= d with n * d < 2^24, as one 64-bit multiply and a
// shift: m = floor(2^24 / d) + 1 overshoots 2^24 / d by at most 1, so
// n * m / 2^24 exceeds n / d by less than n / 2^24 < 1 / d, which never
// carries past the next integer.
__device__ __forceinline__ uint32_t div_magic(uint32_t d) { return (1u << 24) / d + 1u; }
__device__ __forceinline__ int div_small(int n, uint32_t m)
{
    return (int)(((uint64_t)(uint32_t)n * m) >> 24);
}

// First 8-element unit of k-split i of n units split d ways, n * i / d, for a
// power-of-two d (every launch's split count is one): a shift.  Division by a
// runtime 64-bit value would expand into a long instruction sequence at the
// start of every workgroup.
__device__ __forceinline__ int64_t split_begin(int64_t n, int i, int d)
{
    return (n * i) >> __builtin_ctz((unsigned)d);
}

// A k-split partial of v as stored: its lowest fraction bit cleared (a
// relative change below 2^-22, far inside the output's rounding).
__device__ __forceinline__ float v_word(float x) { return __uint_as_float(__float_as_uint(x) & ~1u); }

// Workgroups go to the 8 XCDs round-robin (workgroup b runs on XCD b % 8), each
// XCD with its own L2.  xcd_major(b, n) numbers the n workgroups of a 1-D grid
// so that each XCD holds one contiguous range: XCD x gets [x q + min(x, rem),
// + q + (x < rem)) for n = 8 q + rem.  Work handed out in index order then
// keeps neighbouring work items (the chunks of one tile, tiles of one slot)
// in one L2.  A bijection on [0, n) whatever the placement, so only speed
// depends on the round-robin.
__device__ __forceinline__ int xcd_major(int b, int n)
{
    const int x = b & 7, q = n >> 3, rem = n & 7;
    return x * q + min(x, rem) + (b >> 3);
}

// Workgroup barrier that orders LDS only: waits for this wavefront's LDS
// stores (lgkmcnt), not for its global loads, so loads issued ahead of the
// barrier stay in flight across it.  __syncthreads() is a full release fence
// and would drain them.  Not for LDS written by global-to-LDS copies (those
// complete on the vector-memory counter).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// v, or zeros, selected per component.  Used after a load from a clamped,
// in-bounds address: the load needs no branch around it, and a select of the
// whole vector would be compiled as a select of addresses through scratch.
__device__ __forceinline__ float4 keep_if(bool ok, float4 v)
{
    return make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
}

__device__ __forceinline__ uint4 keep_if(bool ok, uint4 v)
{
    return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

// Eight consecutive elements of a row, held in their storage format.
template <int DT> struct Vec8;

template <> struct Vec8<DT_BF16> {
    uint4 w;  // element 2m in the low half of word m, 2m+1 in the high half
    __device__ __forceinline__ void load(const void *base, int64_t idx)
    {
        w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(base) + idx);
    }
    __device__ __forceinline__ void zero() { w = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ uint32_t word(int m) const
    {
        return m == 0 ? w.x : m == 1 ? w.y : m == 2 ? w.z : w.w;
    }
    __device__ __forceinline__ void to_f32(float (&f)[8]) const
    {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f[2 * m] = bf16_lo(word(m));
            f[2 * m + 1] = bf16_hi(word(m));
        }
    }
    // acc += sum_e this[e] * o[e]
    __device__ __forceinline__ float dot(const Vec8 &o, float acc) const
    {
        acc = dot2_bf16(w.x, o.w.x, acc);
        acc = dot2_bf16(w.y, o.w.y, acc);
        acc = dot2_bf16(w.z, o.w.z, acc);
        acc = dot2_bf16(w.w, o.w.w, acc);
        return acc;
    }
    static __device__ __forceinline__ void store(void *base, int64_t idx, const float (&f)[8])
    {
        uint4 o;
        o.x = pack_bf16x2(f[0], f[1]);
        o.y = pack_bf16x2(f[2], f[3]);
        o.z = pack_bf16x2(f[4], f[5]);
        o.w = pack_bf16x2(f[6], f[7]);
        *reinterpret_cast<uint4 *>(reinterpret_cast<uint16_t *>(base) + idx) = o;
    }
};

template <> struct Vec8<DT_F32> {
    float4 a, b;
    __device__ __forceinline__ void load(const void *base, int64_t idx)
    {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + idx);
        a = p[0];
        b = p[1];
    }
    __device__ __forceinline__ void zero()
    {
        a = make_float4(0.f, 0.f, 0.f, 0.f);
        b = a;
    }
    __device__ __forceinline__ void to_f32(float (&f)[8]) const
    {
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
    __device__ __forceinline__ float dot(const Vec8 &o, float acc) const
    {
        acc = fmaf(a.x, o.a.x, acc); acc = fmaf(a.y, o.a.y, acc);
        acc = fmaf(a.z, o.a.z, acc); acc = fmaf(a.w, o.a.w, acc);
        acc = fmaf(b.x, o.b.x, acc); acc = fmaf(b.y, o.b.y, acc);
        acc = fmaf(b.z, o.b.z, acc); acc = fmaf(b.w, o.b.w, acc);
        return acc;
    }
    static __device__ __forceinline__ void store(void *base, int64_t idx, const float (&f)[8])
    {
        float4 *p = reinterpret_cast<float4 *>(reinterpret_cast<float *>(base) + idx);
        p[0] = make_float4(f[0], f[1], f[2], f[3]);
        p[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
};

// Wavefront reduce-scatter of 16 per-lane partial sums.  On return every lane
// holds the sum over all 64 lanes of element j = (lane >> 2) & 15.  Each step
// halves the values a lane keeps and adds its partner's copy of the kept half,
// so the whole reduction costs 17 cross-lane moves instead of 16 x 6.  The
// summation order is fixed by the lane pattern alone.
__device__ __forceinline__ float wave_reduce_scatter16(const float (&v)[16])
{
    const int lane = threadIdx.x & 63;
    float w8[8], w4[4], w2[2];
    bool up = lane & 32;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        float keep = up ? v[8 + m] : v[m];
        float send = up ? v[m] : v[8 + m];
        w8[m] = keep + __shfl_xor(send, 32);
    }
    up = lane & 16;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        float keep = up ? w8[4 + m] : w8[m];
        float send = up ? w8[m] : w8[4 + m];
        w4[m] = keep + __shfl_xor(send, 16);
    }
    up = lane & 8;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        float keep = up ? w4[2 + m] : w4[m];
        float send = up ? w4[m] : w4[2 + m];
        w2[m] = keep + __shfl_xor(send, 8);
    }
    up = lane & 4;
    float w1 = (up ? w2[1] : w2[0]) + __shfl_xor(up ? w2[0] : w2[1], 4);
    w1 += __shfl_xor(w1, 2);
    w1 += __shfl_xor(w1, 1);
    return w1;
}

}  // namespace lora
