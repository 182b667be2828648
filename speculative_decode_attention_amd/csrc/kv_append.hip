// kv_append.hip -- the write side of the int8 paged KV cache (gfx950).
//
// The quantiser (quant.h) is symmetric int8 with one fp16 scale per (token, kv
// head), in IEEE fp32 so that it is bit-exact and reproducible; the pages fix
// only that the cache is 8-bit (Splash community summary on discuss.pytorch.kr,
// section "Metal kernels generated to shape").
//
// One wave per (request, token, kv head) row.  Each lane holds D/64 values; the
// row maximum is a wave reduction.  K rows are stored as D contiguous bytes
// (one coalesced store per lane); V pages are two d-major tiles of 8 tokens, so
// each code goes to its own byte at a stride of 8.  The kernel moves a
// few hundred bytes per row and is launch-latency bound for a draft block.
#include "device.h"
#include "launch.h"
#include "quant.h"

namespace splash {

template <int D, bool SRC_BF16>
__global__ __launch_bounds__(256) void kv_append_int8_kernel(
    const void* __restrict__ k_new, const void* __restrict__ v_new,
    int8_t* __restrict__ k_pool, int8_t* __restrict__ v_pool,
    uint16_t* __restrict__ k_scale, uint16_t* __restrict__ v_scale,
    const int32_t* __restrict__ block_table, int max_pages_per_seq,
    const int32_t* __restrict__ context_lens, const int32_t* __restrict__ draft_lens,
    int B, int T_max, int Hkv) {
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
    append_token_row<D, SRC_BF16>(k_new, v_new, ((size_t)bt * Hkv + g) * D, k_pool, v_pool, k_scale, v_scale,
                                  (size_t)page * Hkv + g, pos % kPage, lane);
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
