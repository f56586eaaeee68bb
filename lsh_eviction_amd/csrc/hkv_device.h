// hkv_device.h -- device helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "hkv_kernels.h"

namespace hkv {

typedef uint16_t bf16_t;   // raw bf16 bits

constexpr float kLog2e = 1.4426950408889634f;

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

// Sum over aligned groups of N lanes (N = 1 .. 64, power of two); every lane
// of a group ends with the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    if constexpr (N >= 2) x += dpp_f<kDppXor1>(x);
    if constexpr (N >= 4) x += dpp_f<kDppXor2>(x);
    if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
    if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
    if constexpr (N >= 32) x += __shfl_xor(x, 16);
    if constexpr (N >= 64) x += __shfl_xor(x, 32);
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

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        unsigned long long o = __shfl_xor(v, m);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_max_f(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum_f(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
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
