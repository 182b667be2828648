// read_ceiling.hip -- a measurement probe, not part of the attention path: the
// HBM read rate this part sustains for the page stream the partition kernel
// issues (4 KB pages at permuted positions, 16-byte direct-to-LDS loads, no
// compute), so that a kernel's achieved bandwidth can be set against both the
// published peak and what a pure copy of the same pattern reaches.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 512;
constexpr int kPagesPerRound = 16;   // 8 waves x 8 x 1 KB = 64 KB per workgroup per round

__global__ __launch_bounds__(kThreads) void read_pages_kernel(const uint8_t* src, const int32_t* perm,
                                                              int64_t npages, uint32_t* sink) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kPagesPerRound * 4096];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint32_t ldsb = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(lds + w * 8 * 1024));
    for (int64_t p0 = (int64_t)blockIdx.x * kPagesPerRound; p0 + kPagesPerRound <= npages;
         p0 += (int64_t)gridDim.x * kPagesPerRound) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t page = perm[p0 + (w * 8 + i) / 4];
            const uint8_t* a = src + page * 4096 + ((w * 8 + i) % 4) * 1024 + lane * 16;
            asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(a), "{m0}"(ldsb + i * 1024));
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    if (tid == 0) sink[blockIdx.x] = lds[blockIdx.x % sizeof(lds)];
}

}  // namespace

// src: npages * 4096 bytes of device memory; perm: npages page indices in
// [0, npages) (device); sink: `grid` uint32 (device).  Reads every page once,
// in perm order, on `stream`.  Returns 0, or 1 for a bad argument, or 2 if the
// launch failed.
extern "C" int splash_probe_read_pages(const void* src, const int32_t* perm, int64_t npages, uint32_t* sink,
                                       int grid, hipStream_t stream) {
    if (src == nullptr || perm == nullptr || sink == nullptr || npages < kPagesPerRound || grid <= 0) return 1;
    hipLaunchKernelGGL(read_pages_kernel, dim3(grid), dim3(kThreads), 0, stream, static_cast<const uint8_t*>(src),
                       perm, npages, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
