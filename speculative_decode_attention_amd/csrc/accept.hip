// accept.hip -- acceptance of a verified draft block (gfx950).
//
// After the target model checks a drafted block in one forward pass, the step
// keeps the drafts the target agrees with and rolls the cache back past the
// others; the emitted tokens are exactly those of greedy autoregressive
// decoding (Splash community summary on discuss.pytorch.kr, section "DFlash 2
// speculative decoding as the default path": the block is verified in one pass,
// the output is identical to autoregressive decoding, and drafting,
// verification, acceptance and the state update are submitted as one unit, so
// nothing here returns to the host).
//
// Two kernels, no atomics, so every result is the same on every run:
//  * argmax partials: one workgroup of 256 threads per (chunk of kAcceptChunk
//    logits, block position t, request b), for the rows the block has
//    (t < d_b).  Each thread reads 4 x 16 bytes (32 bf16 values) with coalesced
//    loads and keeps the largest value and, among equal values, the lowest
//    token id; the wave and then the workgroup reduce those (value, id) pairs
//    the same way.  This is an HBM stream: the bytes are the logits of the rows
//    read.
//  * finalize: one wave per request folds its rows' chunk partials in chunk
//    order, compares draft t + 1 with the greedy token of row t on lane t, and
//    counts the leading matches with one ballot.
// (A single kernel in which the last workgroup of a request finalises needs a
// device-scope release per workgroup, which writes the L2 back each time: far
// slower than the second launch.)
#include <hip/hip_runtime.h>
#include <math.h>

#include "device.h"
#include "launch.h"

namespace splash {
namespace {

constexpr int kAcceptThreads = 256;
constexpr int kAcceptPerThread = 32;                              // bf16 values per thread
constexpr int kAcceptLoads = kAcceptPerThread / 8;                // 16-byte loads per thread

struct Best {
    float v;
    int i;
};

// (value, id) order: larger value first, then lower id.  Finite or infinite
// values only (NaN logits are outside the contract).
__device__ __forceinline__ Best better(Best a, Best b) {
    return (b.v > a.v || (b.v == a.v && b.i < a.i)) ? b : a;
}

__device__ __forceinline__ Best wave_best(Best x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Best o;
        o.v = __shfl_xor(x.v, m, 64);
        o.i = __shfl_xor(x.i, m, 64);
        x = better(x, o);
    }
    return x;
}

__global__ __launch_bounds__(kAcceptThreads) void accept_argmax_kernel(const AcceptArgs a) {
    const int c = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
    const int d = min(max(a.draft_lens[b], 0), a.T_max);
    if (t >= d) return;                                           // uniform: the block has no row t
    const int tid = threadIdx.x;
    const long row = (long)b * a.T_max + t;
    const uint16_t* src = a.logits + row * a.V;
    const int c0 = c * kAcceptChunk;
    Best best{-INFINITY, 0x7fffffff};
    u32x4_t raw[kAcceptLoads];
#pragma unroll
    for (int k = 0; k < kAcceptLoads; ++k) {
        const int e0 = c0 + (k * kAcceptThreads + tid) * 8;      // first of 8 consecutive ids
        raw[k] = e0 < a.V ? *reinterpret_cast<const u32x4_t*>(src + e0) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kAcceptLoads; ++k) {
        const int e0 = c0 + (k * kAcceptThreads + tid) * 8;
        if (e0 >= a.V) continue;                                  // V is a multiple of 8
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = raw[k][e >> 1];
            const float x = bit_cast<float>((e & 1) ? (w & 0xffff0000u) : (w << 16));   // exact bf16 widening
            if (x > best.v || best.i == 0x7fffffff) best = Best{x, e0 + e};   // ids rise: ties keep the first
        }
    }
    best = wave_best(best);
    __shared__ float sv[kAcceptThreads / 64];
    __shared__ int si[kAcceptThreads / 64];
    const int wv = tid >> 6;
    if ((tid & 63) == 0) {
        sv[wv] = best.v;
        si[wv] = best.i;
    }
    __syncthreads();
    if (tid == 0) {
        Best r{sv[0], si[0]};
#pragma unroll
        for (int w = 1; w < kAcceptThreads / 64; ++w) r = better(r, Best{sv[w], si[w]});
        a.part[row * a.num_chunks + c] = make_int2(__float_as_int(r.v), r.i);
    }
}

__global__ __launch_bounds__(64) void accept_finalize_kernel(const AcceptArgs a) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const int d = min(max(a.draft_lens[b], 0), a.T_max);
    if (d == 0) {                                                 // no block: a no-op
        if (lane == 0) {
            a.accepted[b] = 0;
            a.next_token[b] = -1;
        }
        return;
    }
    // lane t < d: the greedy token of row t, from its chunks in order
    int y = -1;
    if (lane < d) {
        const int2* p = a.part + ((long)b * a.T_max + lane) * a.num_chunks;
        Best r{__int_as_float(p[0].x), p[0].y};
        for (int k = 1; k < a.num_chunks; ++k) r = better(r, Best{__int_as_float(p[k].x), p[k].y});
        y = r.i;
    }
    // draft at block position lane + 1 against row lane's greedy token
    const bool match = lane + 1 < d && a.block_tokens[(long)b * a.T_max + lane + 1] == y;
    const uint64_t m = __builtin_amdgcn_ballot_w64(match);
    const int kept = 1 + (int)__builtin_ctzll(~m);                // 1 + leading matches (<= d)
    const int next = __shfl(y, kept - 1, 64);
    if (lane == 0) {
        a.accepted[b] = kept;
        a.next_token[b] = next;
        a.context_lens[b] -= d - kept;                            // the rejected drafts leave the cache
    }
}

}  // namespace

int accept_num_chunks(int V) { return (V + kAcceptChunk - 1) / kAcceptChunk; }

hipError_t launch_verify_accept(const AcceptArgs& a, hipStream_t stream) {
    if (a.B <= 0) return hipSuccess;
    const dim3 grid((unsigned)a.num_chunks, (unsigned)a.T_max, (unsigned)a.B);
    hipLaunchKernelGGL(accept_argmax_kernel, grid, dim3(kAcceptThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(accept_finalize_kernel, dim3((unsigned)a.B), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace splash
