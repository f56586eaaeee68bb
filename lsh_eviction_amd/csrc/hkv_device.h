// hkv_device.h -- device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "hkv_kernels.h"

namespace hkv {

typedef uint16_t bf16_t;   // raw bf16 bits

constexpr float kLog2e = 1.4426950408889634f;
// Buffer resources: word 3 = 32-bit data format, no swizzle.  Reads past
// num_records return zero.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

// 16 bytes of a row -> EPL floats
template <typename KT>
struct Vec16;
template <>
struct Vec16<bf16_t> {
    static constexpr int EPL = 8;
    __device__ __forceinline__ static void cvt(const uint4& r, float (&x)[8])
    {
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
};
template <>
struct Vec16<float> {
    static constexpr int EPL = 4;
    __device__ __forceinline__ static void cvt(const uint4& r, float (&x)[4])
    {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
    }
};


// code of `BITS` bits held in the smallest unsigned type
template <int BITS>
struct CodeT;
template <>
struct CodeT<16> { typedef uint16_t T; };
template <>
struct CodeT<32> { typedef uint32_t T; };
template <>
struct CodeT<64> { typedef uint64_t T; };

__device__ __forceinline__ int popc(uint16_t x) { return __popc((uint32_t)x); }
__device__ __forceinline__ int popc(uint32_t x) { return __popc(x); }
__device__ __forceinline__ int popc(uint64_t x) { return __popcll(x); }

// DPP lane exchange inside a row of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16
constexpr int kDppRor8 = 0x128;       // lane i <- lane (i + 8) mod 16 within 16, i.e. i ^ 8

// The lane's value and that of lane ^ X (X = 16 or 32), by the lane-swap
// instructions of gfx950 (VALU, no LDS).  A swap of a register with itself
// hands each lane its own value and its partner's, in an order that depends
// on the lane, so callers combine the two symmetrically.
template <int X>
__device__ __forceinline__ float2 swap_pair(float v)
{
    const unsigned u = __float_as_uint(v);
    if constexpr (X == 32) {
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
}

// Sum over aligned groups of N lanes (N = 1 .. 64, power of two); every lane
// of a group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (N >= 2) x += dpp_f<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp_f<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
    if constexpr (N >= 32) {
        const float2 p = swap_pair<16>(x);
        x = p.x + p.y;
    }
    if constexpr (N >= 64) {
        const float2 p = swap_pair<32>(x);
        x = p.x + p.y;
    }
    return x;
}

// Eight values -> eight int8 codes v / scale, rounded half to even (the
// default rounding of rintf), clamped to +-127; all zero when scale is 0.
__device__ __forceinline__ uint2 quantize8(const float (&f)[8], float scale)
{
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float cq = scale > 0.f ? fminf(fmaxf(rintf(f[e] / scale), -127.f), 127.f) : 0.f;
        w[e >> 2] |= ((uint32_t)(int32_t)cq & 0xFFu) << (8 * (e & 3));
    }
    return make_uint2(w[0], w[1]);
}

// Eight values -> eight 4-bit codes v / scale, rounded half to even, clamped
// to +-7, packed two per byte (element 2i in the low half of byte i); all
// zero when scale is 0.
__device__ __forceinline__ uint32_t quantize4(const float (&f)[8], float scale)
{
    uint32_t w = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float cq = scale > 0.f ? fminf(fmaxf(rintf(f[e] / scale), -7.f), 7.f) : 0.f;
        w |= ((uint32_t)(int32_t)cq & 0xFu) << (4 * e);
    }
    return w;
}

// 64-bit lane exchanges, as two 32-bit halves moved the same way
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v)
{
    const unsigned lo = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)v, CTRL, 0xF, 0xF, false);
    const unsigned hi = (unsigned)__builtin_amdgcn_update_dpp(0, (int)(unsigned)(v >> 32), CTRL, 0xF, 0xF, false);
    return ((unsigned long long)hi << 32) | lo;
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// Largest value over the whole wave (every lane active), joined as in
// wave_max_f.
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v)
{
    v = umax64(v, dpp_u64<kDppXor1>(v));
    v = umax64(v, dpp_u64<kDppXor2>(v));
    v = umax64(v, dpp_u64<kDppHalfMirror>(v));
    v = umax64(v, dpp_u64<kDppMirror>(v));
    {
        const unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
        const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
        v = umax64(((unsigned long long)h[0] << 32) | l[0], ((unsigned long long)h[1] << 32) | l[1]);
    }
    {
        const unsigned lo = (unsigned)v, hi = (unsigned)(v >> 32);
        const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        v = umax64(((unsigned long long)h[0] << 32) | l[0], ((unsigned long long)h[1] << 32) | l[1]);
    }
    return v;
}

// Maximum and sum over the whole wave (every lane active): each step joins a
// lane with one partner lane -- DPP inside rows of 16, then the 16- and
// 32-lane swaps -- under a commutative operation, so every lane ends with
// the same bits.
__device__ __forceinline__ float wave_max_f(float v)
{
    v = fmaxf(v, dpp_f<kDppXor1>(v));
    v = fmaxf(v, dpp_f<kDppXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    float2 p = swap_pair<16>(v);
    v = fmaxf(p.x, p.y);
    p = swap_pair<32>(v);
    return fmaxf(p.x, p.y);
}

__device__ __forceinline__ float wave_sum_f(float v)
{
    v += dpp_f<kDppXor1>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppMirror>(v);
    float2 p = swap_pair<16>(v);
    v = p.x + p.y;
    p = swap_pair<32>(v);
    return p.x + p.y;
}

// Ordering key of a candidate slot: larger score first, then lower slot.
__device__ __forceinline__ unsigned long long cand_key(int score, int slot)
{
    return ((unsigned long long)(unsigned)score << 32) | (unsigned long long)(0xFFFFFFFFu - (unsigned)slot);
}
__device__ __forceinline__ int cand_slot(unsigned long long key)
{
    return (int)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
}


// A code as W little-endian uint32 words.
__device__ __forceinline__ void store_words(uint32_t* dst, int W, unsigned long long code)
{
    dst[0] = (uint32_t)code;
    if (W > 1) dst[1] = (uint32_t)(code >> 32);
}

}  // namespace hkv
