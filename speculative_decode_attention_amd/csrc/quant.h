// quant.h -- the int8 KV quantiser and the stores of one quantised (token, kv
// head) row into the paged pools.  Internal header; not part of the C ABI.
//
// The pages say the decode kernel reads an 8-bit KV cache (Splash community
// summary on discuss.pytorch.kr, section "Metal kernels generated to shape")
// and that KV precision is a setting (localai.co.kr guide to Splash 1.3.0); they
// do not describe the quantiser.  The library's documented one: symmetric int8
// with one fp16 scale per (token, kv head), scale = binary16(amax / 127),
// codes = clamp(rint(x / scale), -127, 127), all in IEEE fp32 so that it is
// bit-exact and reproducible.
#pragma once

#include "device.h"
#include "launch.h"

namespace splash {

template <int D, bool SRC_BF16>
__device__ __forceinline__ void load_row(const void* src, size_t off, float (&x)[D / 64]) {
    constexpr int E = D / 64;
    if constexpr (SRC_BF16) {
        const uint16_t* p = static_cast<const uint16_t*>(src) + off;
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = bit_cast<float>((uint32_t)p[e] << 16);
    } else {
        const float* p = static_cast<const float*>(src) + off;
        if constexpr (E == 4) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
            x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = p[e];
        }
    }
}

// Quantise one row held across the wave; returns this lane's codes packed
// little-endian (code e in byte e) and the binary16 scale bits.
template <int D>
__device__ __forceinline__ uint32_t quantize_row(const float (&x)[D / 64], uint16_t& s16_bits) {
#pragma clang fp contract(off)
    constexpr int E = D / 64;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = wave_max(amax);
    const float s32 = amax / 127.0f;                 // IEEE fp32 division
    const _Float16 s16 = (_Float16)s32;              // round to nearest even
    const float s = (float)s16;                      // exact widening
    s16_bits = bit_cast<uint16_t>(s16);
    // an all-zero row (s = 0) has all-zero codes: divide by 1 and select 0,
    // without a branch
    const bool zero = s == 0.0f;
    const float sd = zero ? 1.0f : s;
    // x / s correctly rounded with one division per row: r = RN(1 / s) (an
    // IEEE division), q0 = RN(x r), the residual x - q0 s is exact on an FMA,
    // and RN(q0 + residual r) is RN(x / s) (Markstein's theorem for division
    // with a correctly rounded reciprocal; no underflow matters here, since
    // |x / s| < 1/2 whenever x is subnormal)
    const float r = 1.0f / sd;
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const float q0 = x[e] * r;
        const float q = __builtin_fmaf(__builtin_fmaf(-q0, sd, x[e]), r, q0);
        float k = __builtin_rintf(q);                 // ties to even
        k = fminf(fmaxf(k, -127.0f), 127.0f);
        const int c = zero ? 0 : (int)k;
        packed |= ((uint32_t)(c & 0xff)) << (8 * e);
    }
    return packed;
}

// Stores of one quantised row: pg is the (page, kv head) block index
// (page * Hkv + g), slot the token's slot in the page, codes this lane's E codes
// (code e in byte e).  K rows are D contiguous bytes (one coalesced store per
// lane); a V page is two d-major tiles of 8 tokens, [P/8][D][8], so each code
// goes to its own byte at a stride of 8.
template <int D>
__device__ __forceinline__ void store_k_row(int8_t* k_pool, uint16_t* k_scale, size_t pg, int slot, int lane,
                                            uint32_t codes, uint16_t s16) {
    constexpr int E = D / 64;
    int8_t* kdst = k_pool + (pg * kPage + slot) * D + (size_t)lane * E;
    if constexpr (E == 4) *reinterpret_cast<uint32_t*>(kdst) = codes;
    else if constexpr (E == 2) *reinterpret_cast<uint16_t*>(kdst) = (uint16_t)codes;
    else *kdst = (int8_t)codes;
    if (lane == 0) k_scale[pg * kPage + slot] = s16;
}

template <int D>
__device__ __forceinline__ void store_v_row(int8_t* v_pool, uint16_t* v_scale, size_t pg, int slot, int lane,
                                            uint32_t codes, uint16_t s16) {
    constexpr int E = D / 64;
    int8_t* vdst = v_pool + ((pg * (kPage / 8) + slot / 8) * D + (size_t)lane * E) * 8 + slot % 8;
#pragma unroll
    for (int e = 0; e < E; ++e) vdst[e * 8] = (int8_t)((codes >> (8 * e)) & 0xff);
    if (lane == 0) v_scale[pg * kPage + slot] = s16;
}

// One wave quantises the K and V rows of one (token, kv head) and stores them;
// src is the row's element offset in k_new / v_new ([..][Hkv][D]).
template <int D, bool SRC_BF16>
__device__ __forceinline__ void append_token_row(const void* k_new, const void* v_new, size_t src,
                                                 int8_t* k_pool, int8_t* v_pool, uint16_t* k_scale,
                                                 uint16_t* v_scale, size_t pg, int slot, int lane) {
    constexpr int E = D / 64;
    const size_t off = src + (size_t)lane * E;
    float x[E];
    uint16_t s16;
    load_row<D, SRC_BF16>(k_new, off, x);
    uint32_t codes = quantize_row<D>(x, s16);
    store_k_row<D>(k_pool, k_scale, pg, slot, lane, codes, s16);
    load_row<D, SRC_BF16>(v_new, off, x);
    codes = quantize_row<D>(x, s16);
    store_v_row<D>(v_pool, v_scale, pg, slot, lane, codes, s16);
}

}  // namespace splash
