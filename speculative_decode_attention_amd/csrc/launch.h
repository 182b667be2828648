// launch.h -- argument bundles and launchers between the C ABI (abi.hip) and
// the kernels.  Internal header; the C ABI is include/splash_attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace splash {

struct AppendArgs {
    const void* k_new;
    const void* v_new;
    bool src_bf16;
    int8_t* k_pool;
    int8_t* v_pool;
    uint16_t* k_scale;
    uint16_t* v_scale;
    const int32_t* block_table;
    int max_pages_per_seq;
    const int32_t* context_lens;
    const int32_t* draft_lens;
    int B, T_max, Hkv, D;
};

struct VerifyArgs {
    const uint16_t* q;
    uint16_t* out;             // final bf16 rows (one split)            or nullptr
    uint16_t* part_h;          // fp16 tiled partial rows (several splits) or nullptr
    float* part_hlse;          // their natural-log log-sum-exps, [B][Hkv][S][16 G]
    int* part_hjv;             // each block's V exponent: the tiles hold the rows times 2^jv, [B][Hkv][S]
    float* part_o32;           // or: fp32 partial rows [B][Hq][T_max][S][D] (the exported layout)
    float* part_lse32;         //     and their natural-log log-sum-exps [B][Hq][T_max][S]
    const int8_t* k_pool;
    const int8_t* v_pool;
    const uint16_t* k_scale;
    const uint16_t* v_scale;
    const int32_t* block_table;
    int max_pages_per_seq;
    const int32_t* context_lens;
    const int32_t* draft_lens;
    int B, T_max, Hq, Hkv, D;
    float sm_scale;
    int num_splits;            // grid size along the context (S used in the layouts)
    int pages_per_split;       // L, a multiple of kPagesPerIter
    int num_pages;             // pool size; page ids are clamped into [0, num_pages)
    const uint32_t* block_masks = nullptr;   // [B][T_max] bit u of row t: draft t sees draft u; null: causal
    int window = 0;                          // > 0: draft at position p sees keys p - window < j <= p
    int blocks_per_req = 1;                  // > 1: a prefill chunk cut into 16-token blocks, B counts blocks
    // non-null: the call appends the drafted block too: its K and V rows come
    // from these source rows ([B][T_max][Hkv][D], fp32 or bf16), quantised as
    // the append quantises them, instead of from the pools' slots of the block,
    // and are stored into the pools (then the caller's writable pools)
    const void* k_src = nullptr;
    const void* v_src = nullptr;
    bool src_bf16 = false;
};

// Merge of fp32 partial rows in the exported layout: part_o [B][Hq][T_max][S][D],
// part_lse [B][Hq][T_max][S] -> out bf16 [B][T_max][Hq][D].
struct RowMergeArgs {
    const float* part_o;
    const float* part_lse;
    uint16_t* out;
    const int32_t* draft_lens;
    int B, T_max, Hq, D, num_splits;
};

struct TiledMergeArgs {
    const uint16_t* part_h;
    const float* part_hlse;
    const int* part_hjv;
    uint16_t* out;
    const int32_t* draft_lens;
    int B, T_max, Hq, Hkv, D, num_splits;
    int blocks_per_req = 1;                  // as in VerifyArgs
};


struct AcceptArgs {
    const uint16_t* logits;    // bf16 [B][T_max][V]
    const int32_t* block_tokens;
    const int32_t* draft_lens;
    int32_t* context_lens;
    int32_t* accepted;
    int32_t* next_token;
    int2* part;                // [B][T_max][num_chunks] (value bits, id) partials
    int B, T_max, V, num_chunks;
};

constexpr int kAcceptChunk = 8192;   // logits per workgroup of the argmax kernel

constexpr int kPage = 16;            // tokens per page (the compiled page size)
constexpr int kPagesPerIter = 4;    // pages a workgroup of the partition kernel takes per step

bool append_supported(int D);
bool verify_supported(int D, int G);
hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_verify_partition(const VerifyArgs& a, hipStream_t stream);
hipError_t launch_splitk_merge_tiled(const TiledMergeArgs& a, hipStream_t stream);
bool merge_rows_supported(int D);
hipError_t launch_splitk_merge_rows(const RowMergeArgs& a, hipStream_t stream);
int accept_num_chunks(int V);
hipError_t launch_verify_accept(const AcceptArgs& a, hipStream_t stream);

}  // namespace splash
