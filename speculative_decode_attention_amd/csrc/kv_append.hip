// kv_append.hip -- the write side of the int8 paged KV cache (gfx950).
//
// The pages say the decode kernel reads an 8-bit KV cache (Splash community
// summary on discuss.pytorch.kr, section "Metal kernels generated to shape")
// and that KV precision is a setting (localai.co.kr guide to Splash 1.3.0); they
// do not describe the quantiser.  This kernel implements the library's
// documented one: symmetric int8 with one fp16 scale per (token, kv head),
// scale = binary16(amax / 127), codes = clamp(rint(x / scale), -127, 127), all in
// IEEE fp32 so that it is bit-exact and reproducible.
//
// One wave per (request, token, kv head) row.  Each lane holds D/64 values; the
// row maximum is a wave reduction.  K rows are stored as D contiguous bytes
// (one coalesced store per lane); V pages are two d-major tiles of 8 tokens, so
// each code goes to its own byte at a stride of 8.  The kernel moves a
// few hundred bytes per row and is launch-latency bound for a draft block.
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
    constexpr int E = D / 64;
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(x[e]));
    amax = wave_max(amax);
    const float s32 = amax / 127.0f;                 // IEEE fp32 division
    const _Float16 s16 = (_Float16)s32;              // round to nearest even
    const float s = (float)s16;                      // exact widening
    s16_bits = bit_cast<uint16_t>(s16);
    uint32_t packed = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        int c = 0;
        if (s != 0.0f) {
            float r = __builtin_rintf(x[e] / s);     // IEEE division, ties to even
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            c = (int)r;
        }
        packed |= ((uint32_t)(c & 0xff)) << (8 * e);
    }
    return packed;
}

template <int D, bool SRC_BF16>
__global__ __launch_bounds__(256) void kv_append_int8_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    int8_t* __restrict__ k_pool, int8_t* __restrict__ v_pool,
    uint16_t* __restrict__ k_scale, uint16_t* __restrict__ v_scale,
    const int32_t* __restrict__ block_table, int max_pages_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ draft_lens,
    int B, int T_max, int Hkv) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x & 63;
    const long item = (long)blockIdx.x * 4 + (threadIdx.x >> 6);   // one wave per row
    if (item >= (long)B * T_max * Hkv) return;
    const int g = (int)(item % Hkv);
    const long bt = item / Hkv;
    const int t = (int)(bt % T_max);
    const int b = (int)(bt / T_max);
    const int dl = draft_lens[b];
    if (t >= dl) return;                              // whole wave leaves together
    const int pos = context_lens[b] - dl + t;
    const int page = block_table[(size_t)b * max_pages_per_seq + pos / kPage];
    const int slot = pos % kPage;
    const size_t src = ((size_t)bt * Hkv + g) * D + (size_t)lane * E;
    const size_t pg = (size_t)page * Hkv + g;

    float x[E];
    uint16_t s16;

    // K: the lane's E codes are contiguous in the token row
    load_row<D, SRC_BF16>(k_new, src, x);
    uint32_t codes = quantize_row<D>(x, s16);
    int8_t* kdst = k_pool + (pg * kPage + slot) * D + (size_t)lane * E;
    if constexpr (E == 4) *reinterpret_cast<uint32_t*>(kdst) = codes;
    else if constexpr (E == 2) *reinterpret_cast<uint16_t*>(kdst) = (uint16_t)codes;
    else *kdst = (int8_t)codes;
    if (lane == 0) k_scale[pg * kPage + slot] = s16;

    // V: a page is two d-major tiles of 8 tokens, [P/8][D][8]; one byte per d
    load_row<D, SRC_BF16>(v_new, src, x);
    codes = quantize_row<D>(x, s16);
    int8_t* vdst = v_pool + ((pg * (kPage / 8) + slot / 8) * D + (size_t)lane * E) * 8 + slot % 8;
#pragma unroll
    for (int e = 0; e < E; ++e) vdst[e * 8] = (int8_t)((codes >> (8 * e)) & 0xff);
    if (lane == 0) v_scale[pg * kPage + slot] = s16;
}

template <int D>
static hipError_t launch_append_d(const AppendArgs& a, hipStream_t stream) {
    const long rows = (long)a.B * a.T_max * a.Hkv;
    const long blocks = (rows + 3) / 4;
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (a.src_bf16)
        hipLaunchKernelGGL((kv_append_int8_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, a.k_new, a.v_new, a.k_pool, a.v_pool, a.k_scale, a.v_scale,
                           a.block_table, a.max_pages_per_seq, a.context_lens, a.draft_lens,
                           a.B, a.T_max, a.Hkv);
    else
        hipLaunchKernelGGL((kv_append_int8_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0,
                           stream, a.k_new, a.v_new, a.k_pool, a.v_pool, a.k_scale, a.v_scale,
                           a.block_table, a.max_pages_per_seq, a.context_lens, a.draft_lens,
                           a.B, a.T_max, a.Hkv);
    return hipGetLastError();
}

bool append_supported(int D) { return D == 64 || D == 128 || D == 256; }

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 64: return launch_append_d<64>(a, stream);
        case 128: return launch_append_d<128>(a, stream);
        case 256: return launch_append_d<256>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace splash
