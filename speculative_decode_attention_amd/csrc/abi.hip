// abi.hip -- the C ABI (include/splash_attn.h): argument checks, the split-K
// preset, workspace sizing and kernel launches.  No call allocates, keeps
// per-call state or synchronises the host; the only state is a per-device
// cache of the compute-unit count used by the preset.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/splash_attn.h"
#include "launch.h"

using namespace splash;

// file scope, one copy per device, held until the process ends
static __device__ __align__(256) uint8_t scratch[SPLASH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
constexpr int kMaxVerifyT = 16;
constexpr int kMaxAcceptT = 64;     // the finalize kernel keeps a block on one wave
constexpr int kMaxAcceptV = 1 << 30;
// smallest number of pages a split is given by the preset: below this the
// fixed cost of a workgroup (loading Q, writing partials) dominates its work.
// Measured on MI355X (verify call, one request, 24 q / 4 kv heads): at D = 256
// one step of 4 pages per split is the fastest up to 64 pages of context
// (256 tokens: 13.5 against 15.9 us with 8 pages a split; 1K tokens: 14.5
// against 16.2 us), 8 pages from 2K tokens on; at D = 64 a single split (no
// merge launch) is the fastest up to 16 pages (256 tokens: 7.4 against 9.4 us).
constexpr int kMinPagesPerSplit = 8;
constexpr int kMinPagesShortD256 = 4, kShortContextPages = 64, kOneSplitPagesD64 = 16;

std::mutex g_cu_mutex;
int g_cu_count[kMaxDevices] = {0};

// Split-partial scratch of splash_verify_attn_noalloc (its largest size is
// SPLASH_NOALLOC_SCRATCH_BYTES).  Host code never uses the array's name as an
// address: the device address comes from hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = (size_t)SPLASH_NOALLOC_SCRATCH_BYTES;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (g_cu_count[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            return -1;
        g_cu_count[dev] = cus;
    }
    return g_cu_count[dev];
}

// The current device's address of `scratch` (nullptr if the query fails).
void* scratch_address() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int pages_per_split(int max_context_len, int P, int num_splits) {
    const int n_pages = ceil_div(max_context_len, P);
    int L = ceil_div(n_pages, num_splits);
    L = ceil_div(L, kPagesPerIter) * kPagesPerIter;
    return L < kPagesPerIter ? kPagesPerIter : L;
}

int check_verify_common(const void* q, const void* k_pool, const void* v_pool, const void* k_scale,
                        const void* v_scale, const void* block_table, const void* context_lens,
                        const void* draft_lens, int max_pages_per_seq, int B, int T_max, int Hq,
                        int Hkv, int D, int P, int num_pages, int max_context_len, float sm_scale) {
    if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !block_table || !context_lens || !draft_lens)
        return SPLASH_ERR_INVALID_ARGUMENT;
    if (B < 0 || T_max < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || num_pages <= 0 ||
        max_context_len < 0 || max_pages_per_seq < 0)
        return SPLASH_ERR_INVALID_ARGUMENT;
    if (Hq % Hkv != 0 || !std::isfinite(sm_scale)) return SPLASH_ERR_INVALID_ARGUMENT;
    if ((long)ceil_div(max_context_len, P) > (long)max_pages_per_seq) return SPLASH_ERR_INVALID_ARGUMENT;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return SPLASH_ERR_INVALID_ARGUMENT;
    if (P != kPage || T_max > kMaxVerifyT || !verify_supported(D, Hq / Hkv)) return SPLASH_ERR_UNSUPPORTED;
    return SPLASH_OK;
}

}  // namespace

extern "C" {

const char* splash_status_string(int status) {
    switch (status) {
        case SPLASH_OK: return "ok";
        case SPLASH_ERR_INVALID_ARGUMENT: return "invalid argument";
        case SPLASH_ERR_UNSUPPORTED: return "shape outside the compiled set";
        case SPLASH_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case SPLASH_ERR_LAUNCH: return "kernel launch failed";
        case SPLASH_ERR_DEVICE: return "device query failed";
        default: return "unknown status";
    }
}

int splash_kv_append_int8(const void* k_new, const void* v_new, int src_dtype, int8_t* k_pool,
                          int8_t* v_pool, uint16_t* k_scale, uint16_t* v_scale,
                          const int32_t* block_table, int max_pages_per_seq,
                          const int32_t* context_lens, const int32_t* draft_lens, int B, int T_max,
                          int Hkv, int D, int P, int num_pages, void* stream) {
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale || !block_table ||
        !context_lens || !draft_lens)
        return SPLASH_ERR_INVALID_ARGUMENT;
    if (B < 0 || T_max < 0 || Hkv <= 0 || D <= 0 || P <= 0 || num_pages <= 0 || max_pages_per_seq <= 0)
        return SPLASH_ERR_INVALID_ARGUMENT;
    if (src_dtype != SPLASH_SRC_F32 && src_dtype != SPLASH_SRC_BF16) return SPLASH_ERR_INVALID_ARGUMENT;
    const size_t elem = src_dtype == SPLASH_SRC_F32 ? 4 : 2;
    if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % (elem * (D / 64 > 0 ? D / 64 : 1)))
        return SPLASH_ERR_INVALID_ARGUMENT;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return SPLASH_ERR_INVALID_ARGUMENT;
    if (P != kPage || !append_supported(D)) return SPLASH_ERR_UNSUPPORTED;
    if (B == 0 || T_max == 0) return SPLASH_OK;
    AppendArgs a{k_new, v_new, src_dtype == SPLASH_SRC_BF16, k_pool, v_pool, k_scale, v_scale,
                 block_table, max_pages_per_seq, context_lens, draft_lens, B, T_max, Hkv, D};
    return launch_kv_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SPLASH_OK
                                                                              : SPLASH_ERR_LAUNCH;
}

int splash_verify_attn_split_pages(int max_context_len, int P, int num_splits) {
    if (max_context_len < 0 || P <= 0 || num_splits <= 0) return -SPLASH_ERR_INVALID_ARGUMENT;
    return pages_per_split(max_context_len, P, num_splits);
}

int splash_verify_attn_default_splits(int B, int Hkv, int max_context_len, int P, int D) {
    if (B <= 0 || Hkv <= 0 || max_context_len < 0 || P <= 0 || D <= 0) return -SPLASH_ERR_INVALID_ARGUMENT;
    const int cus = device_cu_count();
    if (cus <= 0) return -SPLASH_ERR_DEVICE;
    const long items = (long)B * Hkv;
    int S = ceil_div(cus, items);                         // one workgroup per compute unit
    const int n_pages = ceil_div(max_context_len, P);
    const int min_pages = D >= 256 && n_pages <= kShortContextPages ? kMinPagesShortD256 : kMinPagesPerSplit;
    const int cap = D <= 64 && n_pages <= kOneSplitPagesD64 ? 1 : ceil_div(n_pages, min_pages);
    if (S > cap) S = cap;
    return S < 1 ? 1 : S;
}

size_t splash_verify_attn_workspace_bytes(int B, int T_max, int Hq, int D, int num_splits) {
    if (B <= 0 || T_max <= 0 || Hq <= 0 || D <= 0 || num_splits <= 1) return 0;
    // tiled fp16 partials for 16 drafts of every query head (B * Hkv * 16 G rows
    // per split = B * 16 Hq), then fp32 log-sum-exps, then one int32 V exponent
    // per (request, kv head, split) block (B * Hq * S bounds B * Hkv * S)
    const size_t rows = (size_t)B * 16 * Hq * num_splits;
    return align_up(rows * D * 2, 256) + align_up(rows * sizeof(float), 256) +
           align_up((size_t)B * Hq * num_splits * sizeof(int), 256);
}

// the drafted block's source rows (the call that appends and verifies; the
// pools it is stored into are the call's own, writable there)
struct BlockAppend {
    const void* k_new;
    const void* v_new;
    bool src_bf16;
};

static int verify_attn_impl(const uint16_t* q, uint16_t* out, const int8_t* k_pool, const int8_t* v_pool,
                            const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                            int max_pages_per_seq, const int32_t* context_lens, const int32_t* draft_lens,
                            int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                            int max_context_len, float sm_scale, int num_splits, void* workspace,
                            size_t workspace_bytes, void* stream, const uint32_t* block_masks,
                            int window, bool prefill = false, const BlockAppend* app = nullptr) {
    // a prefill chunk runs as ceil(T_max / 16) verify blocks per request
    const int nblk = prefill ? ceil_div(T_max, kMaxVerifyT) : 1;
    if (prefill && (T_max < 0 || (long)B * nblk > 65535)) return SPLASH_ERR_INVALID_ARGUMENT;
    int rc = check_verify_common(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                                 draft_lens, max_pages_per_seq, B, prefill ? (T_max < kMaxVerifyT ? T_max : kMaxVerifyT) : T_max,
                                 Hq, Hkv, D, P, num_pages, max_context_len, sm_scale);
    if (rc != SPLASH_OK) return rc;
    if (!out || !aligned16(out) || num_splits < 0) return SPLASH_ERR_INVALID_ARGUMENT;
    if (B == 0 || T_max == 0 || max_context_len == 0) return SPLASH_OK;   // no draft row can exist
    // the tokens the splits cover: the whole context, or what a window leaves of it
    const int span = window > 0 ? splash_verify_attn_window_tokens(max_context_len, T_max, window, P)
                                : max_context_len;
    const int items = B * nblk;                                  // requests, or 16-token blocks of chunks
    if (num_splits == 0) {
        num_splits = splash_verify_attn_default_splits(items, Hkv, span, P, D);
        if (num_splits < 0) return -num_splits;
    }
    const int L = pages_per_split(span, P, num_splits);
    const int S = ceil_div(ceil_div(span, P), L);                // splits that hold pages
    VerifyArgs a{q, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, k_pool, v_pool, k_scale,
                 v_scale, block_table, max_pages_per_seq, context_lens, draft_lens, items, T_max, Hq, Hkv,
                 D, sm_scale, S, L, num_pages};
    a.block_masks = block_masks;
    a.window = window;
    a.blocks_per_req = nblk;
    if (app != nullptr) {
        a.k_src = app->k_new;
        a.v_src = app->v_new;
        a.src_bf16 = app->src_bf16;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (S == 1) {
        a.out = out;
        return launch_verify_partition(a, st) == hipSuccess ? SPLASH_OK : SPLASH_ERR_LAUNCH;
    }
    // the merge's grid takes requests (or blocks) and kv heads on its 16-bit axes:
    // refuse before anything is launched
    if (items > 65535 || Hkv > 65535) return SPLASH_ERR_UNSUPPORTED;
    const size_t need = splash_verify_attn_workspace_bytes(items, prefill ? kMaxVerifyT : T_max, Hq, D, S);
    if (!workspace || !aligned16(workspace)) return SPLASH_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return SPLASH_ERR_WORKSPACE_TOO_SMALL;
    const size_t rows = (size_t)items * 16 * Hq * S;
    a.part_h = static_cast<uint16_t*>(workspace);
    a.part_hlse = reinterpret_cast<float*>(static_cast<char*>(workspace) + align_up(rows * D * 2, 256));
    a.part_hjv = reinterpret_cast<int*>(static_cast<char*>(workspace) + align_up(rows * D * 2, 256) +
                                        align_up(rows * sizeof(float), 256));
    if (launch_verify_partition(a, st) != hipSuccess) return SPLASH_ERR_LAUNCH;
    TiledMergeArgs m{a.part_h, a.part_hlse, a.part_hjv, out, draft_lens, items, T_max, Hq, Hkv, D, S};
    m.blocks_per_req = nblk;
    return launch_splitk_merge_tiled(m, st) == hipSuccess ? SPLASH_OK : SPLASH_ERR_LAUNCH;
}

int splash_verify_attn(const uint16_t* q, uint16_t* out, const int8_t* k_pool, const int8_t* v_pool,
                       const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                       int max_pages_per_seq, const int32_t* context_lens, const int32_t* draft_lens,
                       int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                       int max_context_len, float sm_scale, int num_splits, void* workspace,
                       size_t workspace_bytes, void* stream) {
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, max_context_len,
                            sm_scale, num_splits, workspace, workspace_bytes, stream, nullptr, 0);
}

int splash_verify_attn_append(const void* k_new, const void* v_new, int src_dtype, const uint16_t* q, uint16_t* out,
                              int8_t* k_pool, int8_t* v_pool, uint16_t* k_scale, uint16_t* v_scale,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* context_lens, const int32_t* draft_lens, int B, int T_max, int Hq,
                              int Hkv, int D, int P, int num_pages, int max_context_len, float sm_scale,
                              int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
    if (!k_new || !v_new) return SPLASH_ERR_INVALID_ARGUMENT;
    if (src_dtype != SPLASH_SRC_F32 && src_dtype != SPLASH_SRC_BF16) return SPLASH_ERR_INVALID_ARGUMENT;
    // a lane reads D / 64 consecutive source values at once (16 bytes of fp32 at
    // D = 256, as the append reads them); a shape outside the compiled set is
    // refused by the verify checks below
    const size_t elem = src_dtype == SPLASH_SRC_F32 ? 4 : 2;
    if (append_supported(D) &&
        (reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) % (elem * (D / 64)))
        return SPLASH_ERR_INVALID_ARGUMENT;
    const BlockAppend app{k_new, v_new, src_dtype == SPLASH_SRC_BF16};
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, max_context_len,
                            sm_scale, num_splits, workspace, workspace_bytes, stream, nullptr, 0, false, &app);
}

int splash_verify_attn_noalloc(const uint16_t* q, uint16_t* out, const int8_t* k_pool, const int8_t* v_pool,
                               const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                               int max_pages_per_seq, const int32_t* context_lens, const int32_t* draft_lens,
                               int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                               int max_context_len, float sm_scale, int num_splits, void* stream) {
    int rc = check_verify_common(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens, draft_lens,
                                 max_pages_per_seq, B, T_max, Hq, Hkv, D, P, num_pages, max_context_len, sm_scale);
    if (rc != SPLASH_OK) return rc;
    if (!out || !aligned16(out) || num_splits < 0) return SPLASH_ERR_INVALID_ARGUMENT;
    if (B == 0 || T_max == 0 || max_context_len == 0) return SPLASH_OK;
    // the split count the call will use, and so the partials it needs
    int S = num_splits;
    if (S == 0) {
        S = splash_verify_attn_default_splits(B, Hkv, max_context_len, P, D);
        if (S < 0) return -S;
    }
    const int L = pages_per_split(max_context_len, P, S);
    S = ceil_div(ceil_div(max_context_len, P), L);
    const size_t need = splash_verify_attn_workspace_bytes(B, T_max, Hq, D, S);
    if (need > kScratchBytes) return SPLASH_ERR_WORKSPACE_TOO_SMALL;
    void* ws = nullptr;
    if (need > 0 && (ws = scratch_address()) == nullptr) return SPLASH_ERR_DEVICE;
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, max_context_len,
                            sm_scale, S, ws, need > 0 ? kScratchBytes : 0, stream, nullptr, 0);
}

int splash_verify_attn_masked(const uint16_t* q, uint16_t* out, const int8_t* k_pool, const int8_t* v_pool,
                              const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                              int max_pages_per_seq, const int32_t* context_lens, const int32_t* draft_lens,
                              const uint32_t* block_masks, int B, int T_max, int Hq, int Hkv, int D, int P,
                              int num_pages, int max_context_len, float sm_scale, int num_splits,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (!block_masks) return SPLASH_ERR_INVALID_ARGUMENT;
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, max_context_len,
                            sm_scale, num_splits, workspace, workspace_bytes, stream, block_masks, 0);
}

size_t splash_prefill_attn_workspace_bytes(int B, int T_max, int Hq, int Hkv, int D, int P,
                                           int max_context_len, int num_splits) {
    if (B < 0 || T_max < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || max_context_len < 0 || num_splits < 0)
        return 0;
    if (B == 0 || T_max == 0 || max_context_len == 0) return 0;
    const int items = B * ceil_div(T_max, kMaxVerifyT);
    if (num_splits == 0) num_splits = splash_verify_attn_default_splits(items, Hkv, max_context_len, P, D);
    if (num_splits <= 0) return 0;
    const int L = pages_per_split(max_context_len, P, num_splits);
    const int S = ceil_div(ceil_div(max_context_len, P), L);
    return S == 1 ? 0 : splash_verify_attn_workspace_bytes(items, kMaxVerifyT, Hq, D, S);
}

int splash_prefill_attn(const uint16_t* q, uint16_t* out, const int8_t* k_pool, const int8_t* v_pool,
                        const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                        int max_pages_per_seq, const int32_t* context_lens, const int32_t* chunk_lens, int B,
                        int T_max, int Hq, int Hkv, int D, int P, int num_pages, int max_context_len,
                        float sm_scale, int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, chunk_lens, B, T_max, Hq, Hkv, D, P, num_pages, max_context_len,
                            sm_scale, num_splits, workspace, workspace_bytes, stream, nullptr, 0, true);
}

int splash_verify_attn_window_tokens(int max_context_len, int T_max, int window, int P) {
    if (max_context_len < 0 || T_max < 0 || window < 1 || P <= 0) return -SPLASH_ERR_INVALID_ARGUMENT;
    // keys the block's drafts can see start at ctx - d + 1 - window, which may sit
    // inside a page: at most ceil((d + window - 1) / P) + 1 pages per request
    const long bound = (long)P * (ceil_div(T_max + window - 1, P) + 1);
    return bound < max_context_len ? (int)bound : max_context_len;
}

int splash_verify_attn_window(const uint16_t* q, uint16_t* out, const int8_t* k_pool, const int8_t* v_pool,
                              const uint16_t* k_scale, const uint16_t* v_scale, const int32_t* block_table,
                              int max_pages_per_seq, const int32_t* context_lens, const int32_t* draft_lens,
                              int window, int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                              int max_context_len, float sm_scale, int num_splits, void* workspace,
                              size_t workspace_bytes, void* stream) {
    if (window < 1) return SPLASH_ERR_INVALID_ARGUMENT;
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, max_context_len,
                            sm_scale, num_splits, workspace, workspace_bytes, stream, nullptr, window);
}

int splash_verify_attn_partition(const uint16_t* q, const int8_t* k_pool, const int8_t* v_pool,
                                 const uint16_t* k_scale, const uint16_t* v_scale,
                                 const int32_t* block_table, int max_pages_per_seq,
                                 const int32_t* context_lens, const int32_t* draft_lens, int B,
                                 int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                                 int max_context_len, float sm_scale, int num_splits, float* part_o,
                                 float* part_lse, void* stream) {
    int rc = check_verify_common(q, k_pool, v_pool, k_scale, v_scale, block_table, context_lens,
                                 draft_lens, max_pages_per_seq, B, T_max, Hq, Hkv, D, P, num_pages,
                                 max_context_len, sm_scale);
    if (rc != SPLASH_OK) return rc;
    if (!part_o || !part_lse || !aligned16(part_o) || num_splits <= 0) return SPLASH_ERR_INVALID_ARGUMENT;
    if (B == 0 || T_max == 0 || max_context_len == 0) return SPLASH_OK;
    const int L = pages_per_split(max_context_len, P, num_splits);
    VerifyArgs a{q, nullptr, nullptr, nullptr, nullptr, part_o, part_lse, k_pool, v_pool, k_scale,
                 v_scale, block_table, max_pages_per_seq, context_lens, draft_lens, B, T_max, Hq, Hkv, D,
                 sm_scale, num_splits, L, num_pages};
    return launch_verify_partition(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SPLASH_OK
                                                                                     : SPLASH_ERR_LAUNCH;
}

int splash_verify_attn_splitk_merge(const float* part_o, const float* part_lse, uint16_t* out,
                                    const int32_t* draft_lens, int B, int T_max, int Hq, int D,
                                    int num_splits, void* stream) {
    if (!part_o || !part_lse || !out || !draft_lens) return SPLASH_ERR_INVALID_ARGUMENT;
    if (B < 0 || T_max < 0 || Hq <= 0 || D <= 0 || num_splits <= 0) return SPLASH_ERR_INVALID_ARGUMENT;
    if (!aligned16(part_o) || (reinterpret_cast<uintptr_t>(out) & 7u)) return SPLASH_ERR_INVALID_ARGUMENT;
    if (!merge_rows_supported(D)) return SPLASH_ERR_UNSUPPORTED;
    if (B == 0 || T_max == 0) return SPLASH_OK;
    RowMergeArgs m{part_o, part_lse, out, draft_lens, B, T_max, Hq, D, num_splits};
    return launch_splitk_merge_rows(m, static_cast<hipStream_t>(stream)) == hipSuccess ? SPLASH_OK
                                                                                     : SPLASH_ERR_LAUNCH;
}

size_t splash_verify_accept_workspace_bytes(int B, int T_max, int V) {
    if (B < 0 || T_max < 0 || V < 8 || V > kMaxAcceptV) return 0;
    return (size_t)B * (size_t)T_max * (size_t)accept_num_chunks(V) * sizeof(int2);
}

int splash_verify_accept(const uint16_t* logits, const int32_t* block_tokens, const int32_t* draft_lens,
                         int32_t* context_lens, int32_t* accepted, int32_t* next_token, int B, int T_max,
                         int V, void* workspace, size_t workspace_bytes, void* stream) {
    if (!logits || !block_tokens || !draft_lens || !context_lens || !accepted || !next_token)
        return SPLASH_ERR_INVALID_ARGUMENT;
    if (B < 0 || B > 65535 || T_max < 0 || V < 8 || V > kMaxAcceptV || V % 8 != 0 || !aligned16(logits))
        return SPLASH_ERR_INVALID_ARGUMENT;
    if (T_max > kMaxAcceptT) return SPLASH_ERR_UNSUPPORTED;
    if (B == 0) return SPLASH_OK;
    if (T_max == 0) return SPLASH_ERR_INVALID_ARGUMENT;      // draft_lens[b] <= T_max leaves no block to accept
    if (!workspace || !aligned16(workspace)) return SPLASH_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < splash_verify_accept_workspace_bytes(B, T_max, V)) return SPLASH_ERR_WORKSPACE_TOO_SMALL;
    AcceptArgs a{logits, block_tokens, draft_lens, context_lens, accepted, next_token,
                 static_cast<int2*>(workspace), B, T_max, V, accept_num_chunks(V)};
    return launch_verify_accept(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SPLASH_OK : SPLASH_ERR_LAUNCH;
}

}  // extern "C"
