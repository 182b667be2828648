// device.h -- types and small helpers shared by the gfx950 kernels of the
// verify-attention library.  Internal header; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splash {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

template <typename To, typename From>
__device__ __forceinline__ To bit_cast(const From& f) {
    static_assert(sizeof(To) == sizeof(From), "bit_cast size");
    return __builtin_bit_cast(To, f);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = bit_cast<uint32_t>(f);
    if ((u & 0x7f800000u) == 0x7f800000u)            // inf / nan: truncate, keep nan quiet
        return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Reduce across the four 16-lane groups (lanes l, l^16, l^32, l^48) with the
// gfx950 lane-swap instructions.  Swapping a register with itself exchanges the
// odd 16-lane rows of one copy with the even rows of the other, so the two
// results hold, in every lane, its own value and its partner's (16 or 32 lanes
// away).  The results are copied to scalars before use: a bit cast applied to a
// vector element in place can read element 0.
__device__ __forceinline__ void lane_swap16(float v, float& own, float& partner) {
    const u32x2_t a = __builtin_amdgcn_permlane16_swap(bit_cast<uint32_t>(v), bit_cast<uint32_t>(v), false, false);
    const uint32_t x = a[0], y = a[1];
    own = bit_cast<float>(x);
    partner = bit_cast<float>(y);
}
__device__ __forceinline__ void lane_swap32(float v, float& own, float& partner) {
    const u32x2_t a = __builtin_amdgcn_permlane32_swap(bit_cast<uint32_t>(v), bit_cast<uint32_t>(v), false, false);
    const uint32_t x = a[0], y = a[1];
    own = bit_cast<float>(x);
    partner = bit_cast<float>(y);
}
__device__ __forceinline__ float group4_max(float v) {
    float a, b;
    lane_swap16(v, a, b);
    lane_swap32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float group4_sum(float v) {
    float a, b;
    lane_swap16(v, a, b);
    lane_swap32(a + b, a, b);
    return a + b;
}

// Maximum over all 64 lanes, in every lane: inside each 16-lane row with DPP
// moves (quad exchanges, then rotations by 4 and 8 lanes), across the rows with
// the lane swaps; all register moves, none through the LDS.  The maximum does
// not depend on the order it is taken in.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float v) {
    return fmaxf(v, bit_cast<float>(__builtin_amdgcn_update_dpp(0u, bit_cast<uint32_t>(v), CTRL, 0xf, 0xf, false)));
}
__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max<0xb1>(v);                            // quad_perm [1, 0, 3, 2]
    v = dpp_max<0x4e>(v);                            // quad_perm [2, 3, 0, 1]
    v = dpp_max<0x124>(v);                           // row_ror 4
    v = dpp_max<0x128>(v);                           // row_ror 8
    return group4_max(v);
}

}  // namespace splash
