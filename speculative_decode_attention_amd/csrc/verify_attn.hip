// verify_attn.hip -- block-verify decode attention over the int8 paged KV cache
// (gfx950), plus the log-sum-exp merge of context splits.
//
// What is computed: the target model checks a whole drafted block in one pass
// (Splash community summary on discuss.pytorch.kr, section "DFlash 2
// speculative decoding as the default path"), so each drafted row attends
// causally over the cache; the kernel reads the 8-bit cache directly and reuses
// every page across the query heads of its group and all verify tokens (same
// summary, section "Metal kernels generated to shape"; bnskd.com, "Tech core 2").
//
// Work decomposition.  One workgroup of eight waves (two per SIMD) per
// (request b, kv head g, context split s).  Its rows are the R = G * d query
// rows that share kv head g, ordered r = t * G + hh so that a shorter draft
// truncates a prefix of rows, padded to tiles of 16; the tile count in use is a
// compile-time parameter of the body.  The waves take two roles, and wave v and
// wave v + 4 share a SIMD, so every SIMD runs one of each:
//  * score waves 0-3: wave 2 h + pp keeps the queries of row half h in
//    registers, scores pages 2 pp and 2 pp + 1 of every step against them and
//    runs their softmax one step later;
//  * output waves 4-7: wave 4 + c copies page c of every step (K rows, scales,
//    page id, V rows) and owns a quarter of the head dimension of O for P V, so
//    every V code is converted once.
//  * The context is walked in steps of kPagesPerIter = 4 pages (64 tokens).
//    Pages go HBM -> LDS with 16-byte direct-to-LDS loads into rings of four
//    steps: K(i + 3), its scales and the page id of step i + 7 (an LDS ring, so
//    no copy waits on a block-table read), and V(i + 1).  Every step issues the
//    same copy instructions (a copy past the split's pages runs on lane 0 only),
//    so each wait is a constant `s_waitcnt vmcnt(n)`; workgroup barriers wait
//    only on LDS traffic.
//  * One barrier per step.  Between two barriers the score waves run the
//    softmax of step i - 1 (whose flags crossed the barrier) and Q K^T of step
//    i, the output waves P V of step i - 2 (whose P' tiles crossed it).
//  * int8 codes x become fp16 with one byte permute: binary16 0x64uu is
//    1024 + u, and u = x + 128, so the operand holds 1152 + x exactly.  For K the
//    accumulators start at -1152 * sum_d q_d (taken once on the MFMA), so
//    sum_d q_d (1152 + x_d) comes out unbiased; for V the bias is subtracted
//    exactly with a packed fp16 add before the MFMA.
//  * Scores are kept relative to a per-row reference m that moves lazily: only
//    when a step's maximum exceeds it by more than tau = 8 (log2 units), so
//    p = exp2(z - m) <= 2^tau.  Weights are carried as p 2^jv in fp32, with the
//    workgroup's V exponent jv set so that the largest V scale seen times 2^jv
//    lies in [64, 128): P' = p 2^jv s_v is then one fp16 rounding, inside fp16
//    whatever the V scales.  Each score wave publishes one flag per step (a
//    score past its slack, or a V scale in a higher binade than jv allows);
//    without a flag nothing moves and nothing is exchanged.  The first
//    references and jv come from the exact maxima of step 0, exchanged across
//    the barrier that already separates steps 0 and 1.
//  * Q K^T uses v_mfma_f32_16x16x32_f16 (S^T = K Q^T, one 16-key page x 16 rows
//    per tile); P V uses v_mfma_f32_32x32x16_f16 (O^T = V^T P'^T, 32 columns x
//    32 rows x 16 keys).  No AGPR is used: a wave then has 256 VGPRs for the
//    queries (score waves) or the O accumulators (output waves) and the working
//    set.
//  * The epilogue divides by the row sums and writes bf16 rows (one split),
//    fp32 partial rows (the exported partition call) or fp16 partial tiles
//    times 2^jv with jv beside them (several splits inside the verify call),
//    with their natural-log log-sum-exp.
//  * Visibility is a compile-time mode of the kernel, so each variant keeps
//    its own straight-line step: the causal chain; a tree of candidates (bit
//    masks per draft, staged in LDS); a sliding window of the last W keys
//    (splits start at the first visible page); and the causal chain of a
//    prefill chunk cut into 16-token blocks, each a verify block over the cache
//    up to its own last token.  A fifth mode is the causal chain whose call also
//    appends the drafted block (its rows quantised and stored by the workgroup
//    that holds their pages, before it copies them).
#include <math.h>

#include "device.h"
#include "launch.h"
#include "quant.h"

namespace splash {

constexpr int kWaves = 8;      // two waves per SIMD
constexpr int kRing = 4;       // K and V rings, in steps
constexpr int kKAhead = 3;     // K(i + 3) is issued at step i
constexpr int kIdAhead = 7;    // the page id of step i + 7 is copied at step i
constexpr int kIdRing = 8;
// how a draft sees the block and the context: the causal chain, a tree of
// candidates (per-draft bit masks), a sliding window over the keys, or the
// causal chain of a prefill chunk cut into several 16-token blocks per request
constexpr int kMaskCausal = 0, kMaskTree = 1, kMaskWindow = 2, kMaskChunked = 3, kMaskAppend = 4;
// the append mode: a split of at least this many steps stores the block's rows
// into the pools early enough that its own copies of them need no wait
constexpr int kAppendEarlySteps = 6;

// A work item's request.  Verify: request b itself.  A prefill chunk of
// n_b tokens is cut into blocks of 16 (blocks_per_req of them per request):
// item b is block j of request br, its drafts are chunk tokens 16 j + t
// (t < dl) and its context ends after them, so the block is exactly a verify
// block over the cache up to its own last token.
struct BlockReq {
    int req, t_off, dl, ctx;
};
// A draft length past T_max breaks the caller's contract; it is cut to T_max so
// that no q or out row outside the request is touched.
__device__ __forceinline__ BlockReq block_req(const int32_t* draft_lens, const int32_t* context_lens, int b,
                                              int nblk, int T_max) {
    const int br = nblk == 1 ? b : b / nblk;
    const int t_off = 16 * (b - br * nblk);
    const int d_all = min(draft_lens[br], T_max);
    const int ctx_all = context_lens != nullptr ? context_lens[br] : 0;
    const int dl = nblk == 1 ? d_all : min(max(d_all - t_off, 0), 16);
    return BlockReq{br, t_off, dl, ctx_all - (d_all - t_off - dl)};
}

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// 32-bit LDS address of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_void_ptr)(p);
}

// Direct-to-LDS loads: lane i's 16 (or 4) bytes land at LDS address
// m0 + 16 * i (4 * i).  Issued as inline assembly so that the compiler adds no
// wait of its own: these copies are waited for explicitly (wait_vmcnt) before
// the barrier that publishes them.  `lds` must be uniform in the wave.
// Ordering: volatile asm statements keep their order, and the barrier and
// wait statements carry the memory clobber that orders the LDS reads.
__device__ __forceinline__ void dma16_to_lds(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds));
}
__device__ __forceinline__ void dma4_to_lds(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" :: "v"(src), "{m0}"(lds));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most c of this wave's vector-memory loads are outstanding
// (c is wave-uniform).  Counts above the table wait for all.
__device__ __forceinline__ void wait_vmcnt_le(int c) {
    switch (c) {
#define SPLASH_VMCNT_CASE(N) \
    case N: wait_vmcnt<N>(); break;
        SPLASH_VMCNT_CASE(0) SPLASH_VMCNT_CASE(1) SPLASH_VMCNT_CASE(2) SPLASH_VMCNT_CASE(3)
        SPLASH_VMCNT_CASE(4) SPLASH_VMCNT_CASE(5) SPLASH_VMCNT_CASE(6) SPLASH_VMCNT_CASE(7)
        SPLASH_VMCNT_CASE(8) SPLASH_VMCNT_CASE(9) SPLASH_VMCNT_CASE(10) SPLASH_VMCNT_CASE(11)
        SPLASH_VMCNT_CASE(12) SPLASH_VMCNT_CASE(13) SPLASH_VMCNT_CASE(14) SPLASH_VMCNT_CASE(15)
        SPLASH_VMCNT_CASE(16) SPLASH_VMCNT_CASE(17) SPLASH_VMCNT_CASE(18) SPLASH_VMCNT_CASE(19)
        SPLASH_VMCNT_CASE(20) SPLASH_VMCNT_CASE(21) SPLASH_VMCNT_CASE(22) SPLASH_VMCNT_CASE(23)
        SPLASH_VMCNT_CASE(24) SPLASH_VMCNT_CASE(25) SPLASH_VMCNT_CASE(26) SPLASH_VMCNT_CASE(27)
        SPLASH_VMCNT_CASE(28) SPLASH_VMCNT_CASE(29) SPLASH_VMCNT_CASE(30) SPLASH_VMCNT_CASE(31)
#undef SPLASH_VMCNT_CASE
        default: wait_vmcnt<0>(); break;
    }
}

// Workgroup barrier for LDS traffic only: outstanding direct-to-LDS copies stay
// in flight across it (their completion is waited for explicitly).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Codes 0-1 (sel 0) or 2-3 (sel 1) of a dword already XORed with 0x80808080
// -> two fp16 values 1152 + code.
__device__ __forceinline__ uint32_t ucodes2_to_f16(uint32_t u, int sel) {
    return __builtin_amdgcn_perm(0x64646464u, u, sel ? 0x04030402u : 0x04010400u);
}

// 16 codes -> two fp16x8 operands holding 1152 + code.
__device__ __forceinline__ void codes16_to_f16_biased(const u32x4_t raw, f16x8_t& lo, f16x8_t& hi) {
    u32x4_t a, b;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t u0 = raw[k] ^ 0x80808080u, u1 = raw[2 + k] ^ 0x80808080u;
        a[2 * k] = ucodes2_to_f16(u0, 0);
        a[2 * k + 1] = ucodes2_to_f16(u0, 1);
        b[2 * k] = ucodes2_to_f16(u1, 0);
        b[2 * k + 1] = ucodes2_to_f16(u1, 1);
    }
    lo = bit_cast<f16x8_t>(a);
    hi = bit_cast<f16x8_t>(b);
}

// 8 codes -> fp16x8 holding the codes exactly (the 1152 bias subtracted).
__device__ __forceinline__ f16x8_t codes8_to_f16(const u32x2_t raw) {
    const f16x2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    u32x4_t h;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint32_t u = raw[k] ^ 0x80808080u;
        h[2 * k] = bit_cast<uint32_t>(bit_cast<f16x2_t>(ucodes2_to_f16(u, 0)) - bias);
        h[2 * k + 1] = bit_cast<uint32_t>(bit_cast<f16x2_t>(ucodes2_to_f16(u, 1)) - bias);
    }
    return bit_cast<f16x8_t>(h);
}

__device__ __forceinline__ float f16lo(uint32_t b) { return (float)bit_cast<_Float16>((uint16_t)b); }
__device__ __forceinline__ float f16hi(uint32_t b) { return (float)bit_cast<_Float16>((uint16_t)(b >> 16)); }

// fp32 pair -> packed fp16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_f16x2(float x, float y) {
    const f16x2_t h = {(_Float16)x, (_Float16)y};
    return bit_cast<uint32_t>(h);
}

// (x * s.lo, y * s.hi) as a packed binary16 pair: an fp32 weight times a
// binary16 scale, each product rounded to binary16 (two mixed-precision FMAs
// with a zero addend; register operands only).
__device__ __forceinline__ uint32_t mul_f32_f16x2(float x, float y, uint32_t s) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(x), "v"(s));
    asm("v_fma_mixhi_f16 %0, %1, %2, 0 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "+v"(r) : "v"(y), "v"(s));
    return r;
}

// Shapes and the LDS arena of one workgroup.
template <int D, int G>
struct Cfg {
    static constexpr int NT = G;                      // 16-row tiles at 16 drafts
    static constexpr int KB = D / 32;                 // contraction blocks of Q K^T
    static constexpr int CH = D / 16;                 // 16-byte chunks of a K row
    static constexpr int QCH = D / 8;                 // 16-byte chunks of a Q row (bf16, then fp16)
    static constexpr int QSWZ = QCH < 16 ? QCH : 16;  // Q rows are XOR-swizzled over this many chunks
    static constexpr int PAGE = kPage * D;            // bytes of one K or V page (one kv head)
    static constexpr int NI = PAGE / 1024;            // 16-byte copies per lane per page
    static constexpr int PVW = D / 32 < kWaves ? D / 32 : kWaves;   // waves taking part in P V, 32 columns each
    static constexpr int NT32 = (NT + 1) / 2;         // 32-row tiles at 16 drafts
    static constexpr int NSL = D / 32;                // 32-column slices of a partial block
    static constexpr int SLOT = kPagesPerIter * PAGE; // one step of K (or V) pages
    static constexpr int SSLOT = kPagesPerIter * 64;  // one step of scales: per page 16 K then 16 V (fp16)
    static constexpr int K_OFF = 0;
    static constexpr int S_OFF = K_OFF + kRing * SLOT;
    static constexpr int ID_OFF = S_OFF + kRing * SSLOT;            // page ids [kIdRing][page] int32
    static constexpr int F_OFF = ID_OFF + kIdRing * kPagesPerIter * 4;   // two buffers of [wave] step flags
    static constexpr int V_OFF = F_OFF + 2 * kWaves * 4;
    static constexpr int P_OFF = V_OFF + kRing * SLOT;              // two buffers of P'^T operands
    static constexpr int PBUF = kPagesPerIter * NT32 * 64 * 16;     // [page][32-row tile][lane][16 B]
    static constexpr int M_OFF = P_OFF + 2 * PBUF;                  // [row][page] maxima or row sums
    static constexpr int R_OFF = M_OFF + NT * 16 * kPagesPerIter * 4;   // [row] O rescale factors / references
    static constexpr int MASK_OFF = R_OFF + NT * 16 * 4;          // [16] block masks of the request's drafts
    static constexpr int TOTAL = MASK_OFF + 16 * 4;
    // the append mode only: the block's V codes by token, [16][D] bytes, then
    // its K and V scales by token, [16] + [16] fp16
    static constexpr int STG_OFF = TOTAL;
    static constexpr int STG_S_OFF = STG_OFF + kPage * D;
    static constexpr int TOTAL_APPEND = STG_S_OFF + 2 * kPage * 2;
    static constexpr int Q_OFF = V_OFF + SLOT;        // start-up only: Q over the V slots 1.. onwards
    static constexpr int QBYTES = NT * 16 * D * 2;
    static_assert(D % 64 == 0 && PVW >= 1, "head dim must be a multiple of 64");
    static_assert(NT % 2 == 0, "the two row halves hold whole tiles");
    static_assert(PAGE % 1024 == 0, "page must be whole 1 KB copies");
    static_assert(Q_OFF + QBYTES <= TOTAL, "Q staging does not fit");
    static_assert(TOTAL_APPEND <= 160 * 1024, "LDS arena exceeds 160 KB");
};

// XOR swizzle of 16-byte chunks inside a K row, by slot: the 16 lanes reading
// one chunk column of 16 different rows hit different banks.
template <int D>
__device__ __forceinline__ int k_swizzle(int slot) {
    constexpr int CH = D / 16;
    // the LDS serves 16 lanes of a 16-byte read per cycle (64 banks): with 16
    // chunks a row, the 16 rows of a page take 16 different chunk offsets
    return CH >= 16 ? (slot & 15) : CH >= 8 ? (slot & 7) : ((slot / (8 / CH)) % CH);
}

// The body for NTU row tiles in use (NH = ceil(NTU / 2) per row half; a tile
// past NTU is padding with q = 0).  Waves 0-3 score, waves 4-7 accumulate the
// output; wave v and wave v + 4 share a SIMD, so every SIMD runs one of each and
// the score wave's conversion and softmax arithmetic overlap the output wave's
// MFMAs (and the other way round).
//  * Score wave v = 2 h + pp: row half h keeps the queries of tiles
//    [h NH, (h + 1) NH) in registers; each step it scores pages 2 pp and
//    2 pp + 1 against them and runs their softmax one step later.
//  * Output wave c = v - 4: copies page c of every step (K rows, scales, page
//    id, V rows) and owns columns [32 c SPW, 32 (c + 1) SPW) of all rows for
//    P V, so every V code is converted once.
template <int D, int G, int NTU, int MASK>
__device__ __forceinline__ void partition_body(const VerifyArgs& a, uint8_t* lds, const int b, const int br,
                                               const int t_off, const int g, const int s, const int dl,
                                               const int ctx, const int pg_begin, const int pg_end) {
    using C = Cfg<D, G>;
    constexpr int KB = C::KB, NI = C::NI;
    constexpr int NH = (NTU + 1) / 2;                         // 16-row tiles per half
    constexpr int NT32 = NH;                                  // 32-row tiles in use (P V)
    constexpr int SPW = C::NSL >= 4 ? C::NSL / 4 : 1;         // 32-column slices per output wave
    constexpr int QCHUNKS = 2 * NH * 16 * C::QCH;             // 16-byte chunks of Q converted (padding included)
    constexpr int QI = (QCHUNKS + 64 * kWaves - 1) / (64 * kWaves);   // Q chunks per lane
    // Copy instructions an output wave issues per pipeline position, the same
    // for every position: a copy past the wave's pages still runs, on lane 0
    // only (16 bytes from a valid page into a ring slot nobody reads), so every
    // wait below is a constant.  K rows (NI) + scales + the page id, and the V
    // rows (NI).
    constexpr int KC_START = NI + 1, KC_STEP = NI + 2;
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kLn2 = 0.6931471805599453f;
    constexpr float kTau = 8.0f;                              // lazy-reference slack, log2 units

    const int tid = threadIdx.x, lane = tid & 63;
    const int v = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool scorer = v < 4;
    const int gq = lane >> 4, li = lane & 15;
    const int rows = G * dl;
    const int Hq = a.Hq, S = a.num_splits;
    const int n = (pg_end - pg_begin + kPagesPerIter - 1) / kPagesPerIter;   // steps
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(lds));
    // last step holding page p of a step
    auto last_step = [&](int p) -> int { return (pg_end - pg_begin - 1 - p) >> 2; };
    float* const red = reinterpret_cast<float*>(lds + C::M_OFF);     // [row][page pair]
    float* const rowv = reinterpret_cast<float*>(lds + C::R_OFF);
    float* const vxch = reinterpret_cast<float*>(lds + C::F_OFF + 32);   // [score wave] step V-scale maxima
    int* const jv_out = reinterpret_cast<int*>(lds + C::F_OFF + 48);     // after the loop: the V exponent
    // flags of step j: one byte per score wave (bytes 4-7 stay zero)
    auto read_flags = [&](int j) -> uint32_t {
        const u32x2_t fl = *reinterpret_cast<const u32x2_t*>(lds + C::F_OFF + (j & 1) * kWaves);
        uint32_t f = __builtin_amdgcn_readfirstlane(fl[0] | fl[1]);
        f |= f >> 16;
        return (f | (f >> 8)) & 3u;
    };

    // ---- start-up, output waves: page ids of steps 0..kIdAhead-1 of page c
    // through the scalar cache (counted apart from the vector copies, so waiting
    // for them holds no copy back)
    const int c = v & 3;                                      // output wave: page and column quarter
    const int32_t* bt = a.block_table + (size_t)br * a.max_pages_per_seq + pg_begin + c;   // + 4 j
    const int last_c = last_step(c);
    typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
    int idj[kIdAhead];
    if (!scorer) {
        const const_i32_ptr btc = (const_i32_ptr)bt;
#pragma unroll
        for (int j = 0; j < kIdAhead; ++j) idj[j] = j <= last_c ? btc[4 * j] : 0;
    }
    // every wave copies its share of Q into LDS
#pragma unroll
    for (int k = 0; k < QI; ++k) {
        const int ch = 64 * (v + kWaves * k) + lane;          // Q chunk this lane copies
        const int row = ch / C::QCH, pc = ch % C::QCH;
        if (row < rows) {
            const int lc = pc ^ (row % C::QSWZ);
            const int t = row / G, hq = g * G + row % G;
            dma16_to_lds(a.q + (((size_t)br * a.T_max + t_off + t) * Hq + hq) * D + 8 * lc,
                         lds_base + C::Q_OFF + 1024 * (v + kWaves * k));
        }
    }

    // ---- kMaskAppend: the call appends the drafted block too.  The block ends
    // the context, so its pages pA and pB = pA or pA + 1 are the last page or
    // two of the split holding them.  In such a split the score waves, idle
    // while Q and the first pages are in flight, quantise the block's rows
    // exactly as the append does (score wave v: the K and V rows of tokens
    // 4 v .. 4 v + 3) and store them into the pools' slots of the split's
    // pages: K rows directly, V rows through the LDS, each 8-byte word of the
    // [2][D][8] V pages that holds a block slot being read, merged and written
    // back whole after the barrier before the loop.  The stores have
    // completed before the barrier of step 1, and the block's pages are copied
    // after it when the split has kAppendEarlySteps steps or more (they are
    // then in step n - 2 or later, copied from step n - 5 on), so the copies
    // read the appended rows.  A shorter split ("late") issues its first page
    // copies only after one more barrier, which the score waves reach once
    // their stores have completed.  The source rows reach the LDS as direct
    // copies, K rows at the end of the P' buffers, V rows in the K ring slot
    // of step kKAhead, both unused before the loop: copies the compiler does
    // not track, so it adds no wait of its own for them (a tracked load would
    // make it wait for every page copy).
    bool blk = false, late = false;
    int idA = -1, idB = -1;
    // the append mode, score waves: the pool's V words holding block slots
    // (up to three 8-slot groups of D words, VW per lane)
    constexpr int VW = (3 * D + 255) / 256;
    uint64_t vword[VW];
    constexpr int EQ = D / 64;
    constexpr int SRC_STRIDE = 4 * D * 4;                     // one wave's four fp32 rows
    constexpr int SRC_K_OFF = C::P_OFF + 2 * C::PBUF - 4 * SRC_STRIDE;
    static_assert(C::Q_OFF + C::QBYTES <= SRC_K_OFF && SRC_K_OFF >= C::P_OFF && 4 * SRC_STRIDE <= C::SLOT,
                  "source rows do not fit");
    const int tw = v & 3;                                     // this wave's token group
    const uint32_t src_k = SRC_K_OFF + tw * SRC_STRIDE;
    const uint32_t src_v = C::K_OFF + (kKAhead & (kRing - 1)) * C::SLOT + tw * SRC_STRIDE;
    if constexpr (MASK == kMaskAppend) {
        const int pA = (ctx - dl) / kPage, pB = (ctx - 1) / kPage;
        const bool inA = pA >= pg_begin && pA < pg_end, inB = pB >= pg_begin && pB < pg_end;
        blk = inA || inB;
        late = blk && n < kAppendEarlySteps;
        if (blk) {
            if (scorer) {
                const const_i32_ptr row = (const_i32_ptr)(a.block_table + (size_t)br * a.max_pages_per_seq);
                if (inA) idA = row[pA];
                if (inB) idB = row[pB];
            }
            const int row16 = a.src_bf16 ? D / 8 : D / 4;     // 16-byte pieces of a source row
            const int esz = a.src_bf16 ? 2 : 4;
#pragma unroll
            for (int k = 0; k < SRC_STRIDE / 1024; ++k) {
                const int ch = 64 * k + lane, u = ch / row16, t = 4 * tw + u;
                const size_t off = ((((size_t)br * a.T_max + t) * a.Hkv + g) * D) * esz + 16 * (ch % row16);
                if (scorer && u < 4 && t < dl) {
                    dma16_to_lds(static_cast<const uint8_t*>(a.k_src) + off, lds_base + src_k + 1024 * k);
                    dma16_to_lds(static_cast<const uint8_t*>(a.v_src) + off, lds_base + src_v + 1024 * k);
                }
            }
        }
    }
    // per-lane byte offsets of the K copies inside a page (rows XOR-swizzled by chunk)
    auto koff = [&](int i) -> int {
        const int ch = 64 * i + lane;
        const int slot = ch / C::CH, pc = ch % C::CH;
        return slot * D + 16 * (pc ^ k_swizzle<D>(slot));
    };
    const int soff = lane < 8 ? 2 * lane : 2 * (lane - 8);    // scale copy: lanes 0-7 K, 8-15 V
    // page c's K rows and scales of step j, and its V rows.  A step past the
    // page copies on lane 0 only (see above).
    auto issue_k = [&](int j, int page) {
        const bool on = j <= last_c || lane == 0;
        const size_t blk = (size_t)page * a.Hkv + g;
        const int8_t* src = a.k_pool + blk * C::PAGE;
        const uint32_t dst = lds_base + C::K_OFF + (j & (kRing - 1)) * C::SLOT + c * C::PAGE;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (on) dma16_to_lds(src + koff(i), dst + 1024 * i);
        if (lane < 16 && on)
            dma4_to_lds((lane < 8 ? a.k_scale : a.v_scale) + blk * kPage + soff,
                        lds_base + C::S_OFF + (j & (kRing - 1)) * C::SSLOT + c * 64);
    };
    auto issue_v = [&](int j, int page) {
        const bool on = j <= last_c || lane == 0;
        const int8_t* src = a.v_pool + ((size_t)page * a.Hkv + g) * C::PAGE + 16 * lane;
        const uint32_t dst = lds_base + C::V_OFF + (j & (kRing - 1)) * C::SLOT + c * C::PAGE;
#pragma unroll
        for (int i = 0; i < NI; ++i)
            if (on) dma16_to_lds(src + 1024 * i, dst + 1024 * i);
    };
    // page id of step j from the id ring, clamped into the pool so that no copy
    // can leave it
    auto ring_id = [&](int j) -> int {
        return *reinterpret_cast<const int*>(lds + C::ID_OFF + ((j & (kIdRing - 1)) * kPagesPerIter + c) * 4);
    };
    auto clamp_page = [&](int x) -> int { return min(max(__builtin_amdgcn_readfirstlane(x), 0), a.num_pages - 1); };

    if (!scorer) {
        int ids0 = 0;
#pragma unroll
        for (int j = 0; j < kIdAhead; ++j) ids0 = lane == j ? idj[j] : ids0;
        if (lane < kIdAhead) *reinterpret_cast<int*>(lds + C::ID_OFF + (lane * kPagesPerIter + c) * 4) = ids0;
        if (c == 0 && lane < 2 * kWaves / 4)                  // both flag buffers start clear
            *reinterpret_cast<uint32_t*>(lds + C::F_OFF + 4 * lane) = 0u;
        if (MASK == kMaskTree && c == 1 && lane < 16)         // the drafts' block masks
            *reinterpret_cast<uint32_t*>(lds + C::MASK_OFF + 4 * lane) =
                lane < a.T_max ? a.block_masks[(size_t)br * a.T_max + lane] : 0u;
        if (!late) {
#pragma unroll
            for (int j = 0; j < kKAhead; ++j) issue_k(j, clamp_page(idj[j]));
            issue_v(0, clamp_page(idj[0]));
            // this lane's Q chunks (and block source rows) have landed (only
            // the page copies may be in flight)
            wait_vmcnt<3 * KC_START + NI>();
        } else {
            wait_vmcnt<0>();
        }
    } else {
        wait_vmcnt<0>();
        if constexpr (MASK == kMaskAppend) {
            if (blk) {
                // This wave's tokens: K rows and V rows, each read from its
                // LDS copy and quantised as the append quantises it.  K rows
                // (D contiguous bytes) are stored now; V codes and all scales
                // go to the LDS staging area, for the V words to be built
                // after the barrier: a V page is [2][D][8] (8-token groups,
                // d-major), and single-byte stores scattered over it cost
                // hundreds of cycles each, so every 8-byte word holding a
                // block slot is read from the pool, merged and written back
                // whole.  Those words are loaded first, so their latency
                // overlaps the quantisation.  A token of a page outside this
                // split, or a page id outside the pool, is skipped.
                const int sA = (ctx - dl) % kPage;            // the block's first slot in page pA
                const int nvg = (sA + dl - 1) / 8 - sA / 8 + 1;   // 8-slot groups it touches (<= 3)
                uint64_t* const word = vword;
#pragma unroll
                for (int k = 0; k < VW; ++k) {
                    const int i = 64 * (tw + 4 * k) + lane, vg = sA / 8 + i / D, d = i % D;
                    const int id = vg < 2 ? idA : idB;
                    word[k] = 0;
                    if (i / D < nvg && id >= 0 && id < a.num_pages)
                        word[k] = *reinterpret_cast<const uint64_t*>(
                            a.v_pool + ((size_t)id * a.Hkv + g) * C::PAGE + ((vg & 1) * D + d) * 8);
                }
                int8_t* const kp = const_cast<int8_t*>(a.k_pool);         // writable in this mode
                const int pA = (ctx - dl) / kPage;
                float x[8][EQ];
                if (a.src_bf16) {
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const uint16_t* px = reinterpret_cast<const uint16_t*>(lds + (r < 4 ? src_k : src_v) + (r & 3) * D * 2) + lane * EQ;
#pragma unroll
                        for (int e = 0; e < EQ; ++e) x[r][e] = bit_cast<float>((uint32_t)px[e] << 16);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 8; ++r) {
                        const float* px = reinterpret_cast<const float*>(lds + (r < 4 ? src_k : src_v) + (r & 3) * D * 4) + lane * EQ;
#pragma unroll
                        for (int e = 0; e < EQ; ++e) x[r][e] = px[e];
                    }
                }
                uint32_t q8[8];
                uint16_t s8[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const bool in = 4 * tw + (r & 3) < dl;
#pragma unroll
                    for (int e = 0; e < EQ; ++e) x[r][e] = in ? x[r][e] : 0.0f;
                    q8[r] = quantize_row<D>(x[r], s8[r]);
                }
#pragma unroll
                for (int r = 0; r < 8; ++r) {
                    const int u = r & 3, t = 4 * tw + u, pos = ctx - dl + t;
                    if (t >= dl) continue;
                    if (lane == 0)
                        reinterpret_cast<uint16_t*>(lds + C::STG_S_OFF)[(r < 4 ? 0 : kPage) + t] = s8[r];
                    if (r < 4) {
                        const int id = pos / kPage == pA ? idA : idB;
                        if (id >= 0 && id < a.num_pages) {
                            int8_t* const kdst = kp + (((size_t)id * a.Hkv + g) * kPage + pos % kPage) * D + lane * EQ;
                            if constexpr (EQ == 4) *reinterpret_cast<uint32_t*>(kdst) = q8[r];
                            else if constexpr (EQ == 2) *reinterpret_cast<uint16_t*>(kdst) = (uint16_t)q8[r];
                            else *kdst = (int8_t)q8[r];
                        }
                    } else {
                        uint8_t* const row = lds + C::STG_OFF + t * D + lane * EQ;
                        if constexpr (EQ == 4) *reinterpret_cast<uint32_t*>(row) = q8[r];
                        else if constexpr (EQ == 2) *reinterpret_cast<uint16_t*>(row) = (uint16_t)q8[r];
                        else *row = (uint8_t)q8[r];
                    }
                }
            }
        }
    }
    // bf16 -> fp16 in place, each lane its own chunks (exact for 2^-17 <= |q| <= 65504);
    // padded rows become q = 0.  All reads first, then all writes.
    {
        u32x4_t raw[QI];
#pragma unroll
        for (int k = 0; k < QI; ++k) {
            const int ch = 64 * (v + kWaves * k) + lane;
            raw[k] = (QCHUNKS % (64 * kWaves) == 0 || ch < QCHUNKS)
                         ? *reinterpret_cast<const u32x4_t*>(lds + C::Q_OFF + 16 * ch)
                         : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < QI; ++k) {
            const int ch = 64 * (v + kWaves * k) + lane;
            const uint32_t okmask = ch / C::QCH < rows ? 0xffffffffu : 0u;
            u32x4_t hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = raw[k][e] & okmask;
                hv[e] = pack_f16x2(bit_cast<float>(x << 16), bit_cast<float>(x & 0xffff0000u));
            }
            if (QCHUNKS % (64 * kWaves) == 0 || ch < QCHUNKS)
                *reinterpret_cast<u32x4_t*>(lds + C::Q_OFF + 16 * ch) = hv;
        }
    }
    lds_barrier();
    if constexpr (MASK == kMaskAppend) {
        if (scorer && blk) {
            // the V words: the block's codes of each word's slots, from the
            // staging area, over the pool's bytes of the others; then the
            // block's K and V scales (score wave 0, lanes 0-31)
            int8_t* const vp = const_cast<int8_t*>(a.v_pool);             // writable in this mode
            const int sA = (ctx - dl) % kPage;
            const int nvg = (sA + dl - 1) / 8 - sA / 8 + 1;
#pragma unroll
            for (int k = 0; k < VW; ++k) {
                const int i = 64 * (tw + 4 * k) + lane, vg = sA / 8 + i / D, d = i % D;
                const int id = vg < 2 ? idA : idB;
                if (i / D >= nvg || id < 0 || id >= a.num_pages) continue;
                uint64_t w = vword[k];
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    const int t = 8 * vg + b - sA;            // block token of this slot
                    if (t >= 0 && t < dl) {
                        const uint64_t code = lds[C::STG_OFF + t * D + d];
                        w = (w & ~(0xffull << (8 * b))) | (code << (8 * b));
                    }
                }
                *reinterpret_cast<uint64_t*>(vp + ((size_t)id * a.Hkv + g) * C::PAGE + ((vg & 1) * D + d) * 8) = w;
            }
            if (v == 0 && lane < 2 * kPage) {
                const int t = lane & (kPage - 1), pos = ctx - dl + t;
                const int id = pos / kPage == (ctx - dl) / kPage ? idA : idB;
                if (t < dl && id >= 0 && id < a.num_pages) {
                    uint16_t* const sc = const_cast<uint16_t*>(lane < kPage ? a.k_scale : a.v_scale);
                    sc[((size_t)id * a.Hkv + g) * kPage + pos % kPage] =
                        reinterpret_cast<const uint16_t*>(lds + C::STG_S_OFF)[lane];
                }
            }
            if (late) wait_vmcnt<0>();                        // before the barrier the first copies wait on
        }
        if (late) {
            lds_barrier();
            if (!scorer) {                                    // the first copies, now that the block is stored
#pragma unroll
                for (int j = 0; j < kKAhead; ++j) issue_k(j, clamp_page(idj[j]));
                issue_v(0, clamp_page(idj[0]));
            }
        }
    }

    if (scorer) {
        // ================= score waves =================
        const int h = v >> 1, pp = v & 1;
        const int t0 = h * NH;                                // first tile of this half
        const int lv0 = last_step(2 * pp), lv1 = last_step(2 * pp + 1);
        // this half's Q as fp16 B operands, resident in VGPRs, and the per-row
        // K-code bias -1152 * sum_d q_d, taken on the MFMA; it is the starting
        // value of every Q K^T accumulator, so the scores come out unbiased.
        // Lane (gq, li) holds d in [8 lc, 8 lc + 8) of row 16 (t0 + i) + li for
        // contraction block kb, the same d as the K codes it meets.
        f16x8_t qf[KB][NH];
        f32x4_t nqb[NH];
        {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const int row = 16 * (t0 + i) + li;
                    const int lc = 8 * (kb >> 1) + 2 * gq + (kb & 1);
                    qf[kb][i] = *reinterpret_cast<const f16x8_t*>(lds + C::Q_OFF + row * (2 * D) + 16 * (lc ^ (row % C::QSWZ)));
                }
            }
            f16x8_t k1152;
#pragma unroll
            for (int e = 0; e < 8; ++e) k1152[e] = (_Float16)-1152.0f;
#pragma unroll
            for (int i = 0; i < NH; ++i) nqb[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int i = 0; i < NH; ++i) nqb[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1152, qf[kb][i], nqb[i], 0, 0, 0);
        }
        // per-row state of this half's tiles (row 16 (t0 + i) + li, the same in all lanes of a row)
        // nmr = jv minus the row's reference m (the reference is 0 until the row
        // has one), so that scores come out as z - m + jv and exp2 of them is the
        // weight p 2^jv the softmax carries.  hasref: bit
        // 16 i + li is set once row 16 (t0 + i) + li has a reference (a scalar
        // mask: every lane of a row agrees on it, and it costs no VGPR)
        float nmr[NH], l_run[NH];
        uint64_t hasref = 0;
        auto has_ref = [&](int i) -> bool {
            const uint32_t f = __builtin_amdgcn_readfirstlane((uint32_t)(hasref >> (16 * i)) & 0xffffu);
            return ((f >> li) & 1u) != 0;
        };
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            nmr[i] = 0.0f;
            l_run[i] = 0.0f;
        }
        f32x4_t zs[2][NH];                                    // scores of the previous step, relative to m
        f16x2_t vsh[2][2];                                    // V scales of the previous step's keys (fp16 pairs)
        // V exponent: the softmax weights are carried as p 2^jv (fp32), and
        // P' = p 2^jv s_v is rounded to binary16 once, with jv chosen so that the
        // largest V scale seen so far, times 2^jv, lies in [64, 128): with
        // p <= 2^tau, P' stays below 2^15, and P' of small V scales or small p
        // stays normal.  The row sums carry the same 2^jv, so O / l is the row.
        // A step holding a scale at or above vlim = 2^(7 - jv) (the next binade)
        // raises the wave's flag, and the exchange lowers jv for every wave (the
        // row sums and O are rescaled by the same power of two).  Until a nonzero
        // scale is seen, jv = 0 and vlim is the least positive normal float.
        // Identical in every score wave: set only from maxima all of them read.
        int jv = 0;
        float jvf = 0.0f, vlim = 1.17549435e-38f, vrun = 0.0f;   // vrun: largest V scale seen
        // this lane's largest V scale among the keys of the last scored step (its
        // pages' scales stay in vsh until the next step is scored; 0 past the context)
        auto vscale_max = [&]() -> float {
            const f16x2_t m2 = __builtin_elementwise_max(__builtin_elementwise_max(vsh[0][0], vsh[0][1]),
                                                         __builtin_elementwise_max(vsh[1][0], vsh[1][1]));
            return fmaxf((float)m2[0], (float)m2[1]);
        };
        auto set_jv = [&](float m) {                          // m > 0, uniform: the largest V scale
            const uint32_t mb = __builtin_amdgcn_readfirstlane(bit_cast<uint32_t>(m));
            vrun = bit_cast<float>(mb);
            const int e = (int)((mb >> 23) & 0xffu) - 127;    // floor(log2 m), m normal in fp32
            jv = 6 - e;
            jvf = (float)jv;
            vlim = bit_cast<float>((uint32_t)(e + 1 + 127) << 23);   // 2^(e + 1)
        };
#pragma unroll
        for (int k = 0; k < 2; ++k) {
#pragma unroll
            for (int i = 0; i < NH; ++i) zs[k][i] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int j = 0; j < 2; ++j) vsh[k][j] = f16x2_t{(_Float16)0.0f, (_Float16)0.0f};
        }
        const float zscale = a.sm_scale * kLog2e;

        for (int it = 0; it < n + 2; ++it) {
            // the append mode: this wave's pool stores have completed before
            // the barrier of step 1, after which the block's pages may be copied
            if (MASK == kMaskAppend && it == 1) wait_vmcnt<0>();
            // the K pages of step it, the flags of step it - 1 and (for the
            // output waves) the P' tiles of step it - 2 are published
            lds_barrier();
            const bool do_sm = it >= 1 && it <= n;
            const uint32_t flags = do_sm ? read_flags(it - 1) : 0u;
            // ---- references.  A flag says some score of the wave's pages
            // exceeded the row's reference by more than the slack, or a V scale
            // reached vlim.  Without a flag anywhere nothing moves: every
            // p <= 2^slack and P' stays inside binary16.  Otherwise the exact step
            // maxima (scores per row, V scales per wave) are exchanged, the rows
            // beyond the slack move to their maxima, jv follows the V scales, and
            // the output waves rescale O.
            if (flags & 1u) {                                 // rare after the first step
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const f32x4_t z0 = zs[0][i], z1 = zs[1][i];
                    const float m4 = fmaxf(fmaxf(fmaxf(z0[0], z0[1]), fmaxf(z0[2], z0[3])),
                                           fmaxf(fmaxf(z1[0], z1[1]), fmaxf(z1[2], z1[3])));
                    const float mx = group4_max(m4);
                    if (gq == 0) red[(16 * (t0 + i) + li) * 2 + pp] = mx;
                }
                {
                    const float vw = wave_max(vscale_max());
                    if (lane == 0) vxch[v] = vw;
                }
                lds_barrier();
                // the O factor of a V-exponent change is an exact power of two (a
                // rise of jv only happens while every scale seen was 0, so O = 0);
                // the scores held carry the old jv
                float vscale = 1.0f, dj = 0.0f;
                const float jv_old = jvf;
                {
                    const float vnew = bit_cast<float>(__builtin_amdgcn_readfirstlane(
                        bit_cast<uint32_t>(fmaxf(fmaxf(vxch[0], vxch[1]), fmaxf(vxch[2], vxch[3])))));
                    if (vnew >= vlim) {
                        const int old = jv;
                        set_jv(fmaxf(vrun, vnew));
                        vscale = __builtin_ldexpf(1.0f, jv - old);
                        dj = (float)(jv - old);
                    }
                }
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const u32x2_t mw = *reinterpret_cast<const u32x2_t*>(red + (16 * (t0 + i) + li) * 2);
                    // the step's maximum above the row's reference
                    const float mstep = fmaxf(bit_cast<float>(mw[0]), bit_cast<float>(mw[1])) - jv_old;
                    const bool fresh = !has_ref(i);
                    const bool move = fresh ? mstep > -INFINITY : mstep > kTau;
                    float alpha = 1.0f;
                    if (move) {
                        alpha = fresh ? 0.0f : __builtin_amdgcn_exp2f(-mstep);
                        nmr[i] -= mstep;                      // a fresh row has nmr = 0
                        l_run[i] *= alpha;                    // (the V factor below as well)
#pragma unroll
                        for (int k = 0; k < 2; ++k)
#pragma unroll
                            for (int j = 0; j < 4; ++j) zs[k][i][j] -= mstep;
                    }
                    nmr[i] += dj;
#pragma unroll
                    for (int k = 0; k < 2; ++k)
#pragma unroll
                        for (int j = 0; j < 4; ++j) zs[k][i][j] += dj;
                    l_run[i] *= vscale;
                    if (pp == 0 && gq == 0) rowv[16 * (t0 + i) + li] = alpha * vscale;
                    hasref |= (__builtin_amdgcn_ballot_w64(move) & 0xffffull) << (16 * i);   // lanes gq = 0
                }
                lds_barrier();                                // factors written, maxima read
            }
            if (it == 1) {                                    // first references and V exponent (O is still zero)
                {
                    const float v0 = bit_cast<float>(__builtin_amdgcn_readfirstlane(
                        bit_cast<uint32_t>(fmaxf(fmaxf(vxch[0], vxch[1]), fmaxf(vxch[2], vxch[3])))));
                    if (v0 > 0.0f) set_jv(v0);
                }
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const u32x2_t mw = *reinterpret_cast<const u32x2_t*>(red + (16 * (t0 + i) + li) * 2);
                    const float mstep = fmaxf(bit_cast<float>(mw[0]), bit_cast<float>(mw[1]));   // step 0 scored with jv = 0
                    hasref |= (__builtin_amdgcn_ballot_w64(mstep > -INFINITY) & 0xffffull) << (16 * i);
                    nmr[i] = jvf;
#pragma unroll
                    for (int k = 0; k < 2; ++k)
#pragma unroll
                        for (int j = 0; j < 4; ++j) zs[k][i][j] += jvf;
                    if (mstep > -INFINITY) {
                        nmr[i] = jvf - mstep;
#pragma unroll
                        for (int k = 0; k < 2; ++k)
#pragma unroll
                            for (int j = 0; j < 4; ++j) zs[k][i][j] -= mstep;
                    }
                }
            }

            // ---- softmax of step it - 1: p = exp2(z - m), P' = p * s_v, tile by
            // tile.  A page the split lacks left z = -inf: its P' tiles are zero,
            // so P V runs over every page of a step without a branch.
            auto softmax_page = [&](int k) {
                _Float16* pb = reinterpret_cast<_Float16*>(lds + C::P_OFF + ((it - 1) & 1) * C::PBUF);
                const int p = 2 * pp + k;
#pragma unroll
                for (int i = 0; i < NH; ++i) {
                    const int t = t0 + i;
                    // p 2^jv in fp32 (exp2(-inf) = 0): the row sum adds it in fp32,
                    // and P' = p 2^jv s_v is rounded to binary16 once (the keys' V
                    // scales are 0 past the context)
                    float e[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) e[j] = __builtin_amdgcn_exp2f(zs[k][i][j]);
                    l_run[i] += (e[0] + e[1]) + (e[2] + e[3]);
                    u32x2_t packed;
                    packed[0] = mul_f32_f16x2(e[0], e[1], bit_cast<uint32_t>(vsh[k][0]));
                    packed[1] = mul_f32_f16x2(e[2], e[3], bit_cast<uint32_t>(vsh[k][1]));
                    // reader lane of the 32-row tile t/2: rows 16 (t&1) + li, keys 8 (gq>>1) + 4 (gq&1) + j
                    *reinterpret_cast<u32x2_t*>(pb + ((p * NT32 + (t >> 1)) * 64 + 32 * (gq >> 1) + 16 * (t & 1) + li) * 8 +
                                                4 * (gq & 1)) = packed;
                }
            };
            // ---- Q K^T of step it, page 2 pp + k: K rows of the page from LDS
            // (lane (gq, li) reads chunks 4 cc + gq of key row li), then the
            // scores z = (q . (1152 + x) - 1152 sum q) * s_k * scale * log2(e) - m
            const int slot = it & (kRing - 1);
            auto read_k = [&](int k, u32x4_t (&kraw)[KB / 2], u32x2_t& ks, u32x2_t& vs) {
                const int p = 2 * pp + k;
                const uint8_t* kpage = lds + C::K_OFF + slot * C::SLOT + p * C::PAGE + li * D;
                const int swz = k_swizzle<D>(li);
#pragma unroll
                for (int cc = 0; cc < KB / 2; ++cc)
                    kraw[cc] = *reinterpret_cast<const u32x4_t*>(kpage + 16 * ((4 * cc + gq) ^ swz));
                const uint8_t* sc = lds + C::S_OFF + slot * C::SSLOT + p * 64;
                ks = *reinterpret_cast<const u32x2_t*>(sc + 8 * gq);
                vs = *reinterpret_cast<const u32x2_t*>(sc + 32 + 8 * gq);
            };
            auto qk_chunk = [&](const u32x4_t kr, int cc, f32x4_t (&acc)[NH]) {
                f16x8_t k0, k1;
                codes16_to_f16_biased(kr, k0, k1);
#pragma unroll
                for (int i = 0; i < NH; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[2 * cc][i], acc[i], 0, 0, 0);
#pragma unroll
                for (int i = 0; i < NH; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[2 * cc + 1][i], acc[i], 0, 0, 0);
            };
            // lane (gq, li) holds keys 4 gq + j of the page, row 16 (t0 + i) + li;
            // returns whether a score exceeded its row's threshold
            auto finish_page = [&](int k, const f32x4_t (&acc)[NH], const u32x2_t ks, const u32x2_t vs,
                                   const bool may_mask) -> bool {
                const int p = 2 * pp + k;
                const float thr_ref = kTau + jvf;             // a row with a reference: its slack above m - jv
                float kc[4];
                kc[0] = f16lo(ks[0]) * zscale;
                kc[1] = f16hi(ks[0]) * zscale;
                kc[2] = f16lo(ks[1]) * zscale;
                kc[3] = f16hi(ks[1]) * zscale;
                vsh[k][0] = bit_cast<f16x2_t>(vs[0]);
                vsh[k][1] = bit_cast<f16x2_t>(vs[1]);
                const int key0 = (pg_begin + kPagesPerIter * it + p) * kPage;
                // every key of the page is visible to every row (padded rows see q = 0)
                bool masked = may_mask && !(key0 + kPage - 1 <= ctx - dl);
                if constexpr (MASK == kMaskWindow) masked = may_mask && !(key0 + kPage - 1 <= ctx - dl && key0 >= ctx - a.window);
                const int kl = key0 + 4 * gq;
                if (masked) {                                 // keys past the context carry no V weight
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const uint32_t keep = (kl + 2 * j < ctx ? 0xffffu : 0u) | (kl + 2 * j + 1 < ctx ? 0xffff0000u : 0u);
                        vsh[k][j] = bit_cast<f16x2_t>(bit_cast<uint32_t>(vsh[k][j]) & keep);
                    }
                }
                // a V scale in a higher binade than jv allows flags the step
                const f16x2_t vm2 = __builtin_elementwise_max(vsh[k][0], vsh[k][1]);
                const float vmx = fmaxf((float)vm2[0], (float)vm2[1]);
                bool exceed = vmx >= vlim;
#pragma unroll
                for (int i = 0; i < NH; ++i) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) zs[k][i][j] = __builtin_fmaf(acc[i][j], kc[j], nmr[i]);
                    if (masked) {
                        // a row sees the keys before the block and the block key of
                        // draft u when bit u of its mask is set (the causal chain:
                        // bits 0..t); a padded row sees nothing here
                        const int row = 16 * (t0 + i) + li;
                        if constexpr (MASK == kMaskTree) {
                            const int blk0 = ctx - dl;
                            const uint32_t mrow = row < rows ? *reinterpret_cast<const uint32_t*>(lds + C::MASK_OFF + 4 * (row / G)) : 0u;
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                const int key = kl + j, u = key - blk0;
                                const bool inblk = (unsigned)u < (unsigned)dl;
                                const bool vis = (row < rows) & ((key < blk0) | (inblk & (((mrow >> (u & 31)) & 1u) != 0u)));
                                zs[k][i][j] = vis ? zs[k][i][j] : -INFINITY;
                            }
                        } else if constexpr (MASK == kMaskWindow) {
                            // keys pos - W < key <= pos of the row's own position pos
                            const int pos = row < rows ? ctx - dl + row / G : -1;   // -1: padded row
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                zs[k][i][j] = (kl + j <= pos) & (kl + j > pos - a.window) ? zs[k][i][j] : -INFINITY;
                        } else {
                            const int last_key = row < rows ? ctx - dl + row / G : -1;   // -1: padded row
#pragma unroll
                            for (int j = 0; j < 4; ++j) zs[k][i][j] = kl + j <= last_key ? zs[k][i][j] : -INFINITY;
                        }
                    }
                    const float mx = fmaxf(fmaxf(zs[k][i][0], zs[k][i][1]), fmaxf(zs[k][i][2], zs[k][i][3]));
                    exceed |= mx > (has_ref(i) ? thr_ref : -INFINITY);
                }
                return exceed;
            };
            auto write_flag = [&](bool exceed) {
                const uint32_t flag = __builtin_amdgcn_ballot_w64(exceed) != 0 ? 1u : 0u;
                if (lane == 0)
                    *reinterpret_cast<uint8_t*>(lds + C::F_OFF + (it & 1) * kWaves + v) = (uint8_t)flag;
            };

            // Steady steps (both pages present, no key past any row's view) run
            // as one block: the K reads go first, so their latency overlaps the
            // softmax, and the two pages' MFMA chains interleave.
            const int key_end = (pg_begin + kPagesPerIter * it + 2 * pp + 2) * kPage;   // one past page 2 pp + 1
            bool steady = do_sm && it < n && it <= lv1 && key_end - 1 <= ctx - dl;
            if constexpr (MASK == kMaskWindow)              // every row sees the step's first key
                steady = steady && (pg_begin + kPagesPerIter * it + 2 * pp) * kPage >= ctx - a.window;
            if (steady) {
                u32x4_t kraw[2][KB / 2];
                u32x2_t ks[2], vs[2];
                read_k(0, kraw[0], ks[0], vs[0]);
                read_k(1, kraw[1], ks[1], vs[1]);
                softmax_page(0);
                softmax_page(1);
                f32x4_t acc[2][NH];
#pragma unroll
                for (int k = 0; k < 2; ++k)
#pragma unroll
                    for (int i = 0; i < NH; ++i) acc[k][i] = nqb[i];
#pragma unroll
                for (int cc = 0; cc < KB / 2; ++cc) {
                    qk_chunk(kraw[0][cc], cc, acc[0]);
                    qk_chunk(kraw[1][cc], cc, acc[1]);
                }
                const bool e0 = finish_page(0, acc[0], ks[0], vs[0], false);
                const bool e1 = finish_page(1, acc[1], ks[1], vs[1], false);
                write_flag(e0 || e1);
            } else {
                if (do_sm) {
                    softmax_page(0);
                    softmax_page(1);
                }
                if (it < n) {
                    bool exceed = false;
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        if (it <= (k == 0 ? lv0 : lv1)) {
                            u32x4_t kraw[KB / 2];
                            u32x2_t ks, vs;
                            read_k(k, kraw, ks, vs);
                            f32x4_t acc[NH];
#pragma unroll
                            for (int i = 0; i < NH; ++i) acc[i] = nqb[i];
#pragma unroll
                            for (int cc = 0; cc < KB / 2; ++cc) qk_chunk(kraw[cc], cc, acc);
                            exceed |= finish_page(k, acc, ks, vs, true);
                        } else {
#pragma unroll
                            for (int i = 0; i < NH; ++i) zs[k][i] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
                            for (int j = 0; j < 2; ++j) vsh[k][j] = f16x2_t{(_Float16)0.0f, (_Float16)0.0f};
                        }
                    }
                    if (it == 0) {
                        // the first references are the exact maxima of step 0,
                        // set at step 1 after the barrier: no flag, no exchange
#pragma unroll
                        for (int i = 0; i < NH; ++i) {
                            const f32x4_t z0 = zs[0][i], z1 = zs[1][i];
                            const float m4 = fmaxf(fmaxf(fmaxf(z0[0], z0[1]), fmaxf(z0[2], z0[3])),
                                                   fmaxf(fmaxf(z1[0], z1[1]), fmaxf(z1[2], z1[3])));
                            const float mx = group4_max(m4);
                            if (gq == 0) red[(16 * (t0 + i) + li) * 2 + pp] = mx;
                        }
                        const float vw = wave_max(vscale_max());  // and the V-scale maxima of step 0
                        if (lane == 0) vxch[v] = vw;
                        exceed = false;
                    }
                    write_flag(exceed);
                }
            }
        }

        // ---- epilogue, score side: row sums across lane groups, the references
        // and the largest V scale
#pragma unroll
        for (int i = 0; i < NH; ++i) {
            const float l = group4_sum(l_run[i]);
            if (gq == 0) red[(16 * (t0 + i) + li) * 2 + pp] = l;
            if (pp == 0 && gq == 0) rowv[16 * (t0 + i) + li] = jvf - nmr[i];   // the reference (any value when l = 0)
        }
        if (v == 0 && lane == 0) *jv_out = jv;
        lds_barrier();
        return;
    }

    // ================= output waves =================
    const bool owns = c * SPW < C::NSL;                       // D = 64: two waves own the columns
    f32x16_t o[SPW][NT32];                                    // O^T, columns [32 (c SPW + sl), +32) of all rows
#pragma unroll
    for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
        for (int r = 0; r < NT32; ++r)
#pragma unroll
            for (int e = 0; e < 16; ++e) o[sl][r][e] = 0.0f;
    int id_k = clamp_page(idj[kKAhead]);                      // K page of the next copies
    int id_v = clamp_page(idj[1]);                            // V page of the next copies
    // From iteration last_c on, every copy this wave would issue (K(it + 3),
    // V(it + 1), the page id of step it + 7) is past the split's pages of
    // column c: from iteration E on the wave issues none (positions before 2
    // keep the start-up's fixed counts), and the tail's waits count what
    // actually went out, so no copy is left to wait for after the loop.
    const int E = max(2, last_c);

    for (int it = 0; it < n + 2; ++it) {
        // this wave's copies of K(it) and V(it - 2) (position it - 3) have
        // landed: at most the copies of positions it - 2 and it - 1 are in flight
        if (it >= 2) {
            if (it - 1 < E) wait_vmcnt<2 * (KC_STEP + NI)>();
            else if (it - 2 < E) wait_vmcnt<KC_STEP + NI>();
            else wait_vmcnt<0>();
        } else if (it == 1) wait_vmcnt<KC_START + KC_STEP + 2 * NI>();
        else wait_vmcnt<2 * KC_START + NI>();
        lds_barrier();
        const bool do_sm = it >= 1 && it <= n;
        const uint32_t flags = do_sm ? read_flags(it - 1) : 0u;
        // ---- copies for later steps; a page id past the split's pages is read
        // from the split's first entry of page c's column, which always exists
        if (it < E) {
            issue_k(it + kKAhead, id_k);
            issue_v(it + 1, id_v);
            if (lane == 0)
                dma4_to_lds(it + kIdAhead <= last_c ? bt + 4 * (it + kIdAhead) : bt - c,
                            lds_base + C::ID_OFF + (((it + kIdAhead) & (kIdRing - 1)) * kPagesPerIter + c) * 4);
        }

        // ---- P V of step it - 2: O^T += V^T P'^T for this wave's columns.
        // Every operand is read first, so the LDS round trips overlap.
        if (it >= 2 && owns) {
            const int pstep = it - 2;
            const uint8_t* vst = lds + C::V_OFF + (pstep & (kRing - 1)) * C::SLOT + (lane >> 5) * (D * 8) +
                                 (32 * c * SPW + (lane & 31)) * 8;
            const uint8_t* pbr = lds + C::P_OFF + (pstep & 1) * C::PBUF + lane * 16;
            f16x8_t pf[kPagesPerIter][NT32];
            u32x2_t vr[kPagesPerIter][SPW];
#pragma unroll
            for (int p = 0; p < kPagesPerIter; ++p) {
#pragma unroll
                for (int sl = 0; sl < SPW; ++sl) vr[p][sl] = *reinterpret_cast<const u32x2_t*>(vst + p * C::PAGE + 256 * sl);
#pragma unroll
                for (int r = 0; r < NT32; ++r) pf[p][r] = *reinterpret_cast<const f16x8_t*>(pbr + (p * NT32 + r) * 1024);
            }
#pragma unroll
            for (int p = 0; p < kPagesPerIter; ++p) {
#pragma unroll
                for (int sl = 0; sl < SPW; ++sl) {
                    const f16x8_t vf = codes8_to_f16(vr[p][sl]);
#pragma unroll
                    for (int r = 0; r < NT32; ++r)
                        o[sl][r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[p][r], o[sl][r], 0, 0, 0);
                }
            }
        }

        if (flags & 1u) {                                     // the score waves move references
            lds_barrier();
            lds_barrier();                                    // factors written
            // O holds P V up to step it - 2, made with the old references
            if (owns) {
#pragma unroll
                for (int r = 0; r < NT32; ++r) {
                    const int row = 32 * r + (lane & 31);
                    const float al = row < 2 * NH * 16 ? rowv[row] : 1.0f;
#pragma unroll
                    for (int sl = 0; sl < SPW; ++sl)
#pragma unroll
                        for (int e = 0; e < 16; ++e) o[sl][r][e] *= al;
                }
            }
        }
        // page ids of this wave's next copies: their ring entries were copied at
        // least three steps ago, so the wait at the top of this step covered them
        id_k = clamp_page(ring_id(it + 1 + kKAhead));
        id_v = clamp_page(ring_id(it + 2));
    }

    wait_vmcnt<0>();                                          // the lane-0 copies past the pages
    lds_barrier();                                            // row sums, references, V scale maxima
    if (!owns) return;
    // ---- epilogue, output side.  O and l both carry 2^jv, so O / l is the row
    // and log2 l is jv above the row's log-sum-exp.  The fp16 partial tiles hold
    // the rows times 2^jv (at most 127 * 128 in magnitude, whatever V's scale)
    // with the block's jv beside them for the merge.
    const int jv = *jv_out;
    if (a.out == nullptr && a.part_o32 == nullptr && c == 0 && lane == 0)
        a.part_hjv[((size_t)b * a.Hkv + g) * S + s] = jv;
#pragma unroll
    for (int r = 0; r < NT32; ++r) {
        const int row = 32 * r + (lane & 31);
        if (row >= rows) continue;
        const u32x2_t lw = *reinterpret_cast<const u32x2_t*>(red + row * 2);
        const float l = bit_cast<float>(lw[0]) + bit_cast<float>(lw[1]);
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        const int t = row / G, hq = g * G + row % G;
#pragma unroll
        for (int sl = 0; sl < SPW; ++sl) {
            const int vs = c * SPW + sl;                      // 32-column slice
            if (a.out != nullptr) {
                uint16_t* orow = a.out + (((size_t)br * a.T_max + t_off + t) * Hq + hq) * D;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d = 32 * vs + 8 * q4 + 4 * (lane >> 5);
                    u32x2_t x;
                    x[0] = (uint32_t)f32_to_bf16_rne(o[sl][r][4 * q4] * inv) |
                           ((uint32_t)f32_to_bf16_rne(o[sl][r][4 * q4 + 1] * inv) << 16);
                    x[1] = (uint32_t)f32_to_bf16_rne(o[sl][r][4 * q4 + 2] * inv) |
                           ((uint32_t)f32_to_bf16_rne(o[sl][r][4 * q4 + 3] * inv) << 16);
                    *reinterpret_cast<u32x2_t*>(orow + d) = x;
                }
            } else if (a.part_o32 != nullptr) {
                // exported layout: fp32 rows [B][Hq][T_max][S][D], 16 bytes a lane
                float* orow = a.part_o32 + ((((size_t)br * Hq + hq) * a.T_max + t_off + t) * S + s) * D;
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    const int d = 32 * vs + 8 * q4 + 4 * (lane >> 5);
                    f32x4_t x;
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[e] = o[sl][r][4 * q4 + e] * inv;
                    *reinterpret_cast<f32x4_t*>(orow + d) = x;
                }
            } else {
                // tile order [slice][32-row tile r][q4][lane][4]: every store of
                // the wave writes 512 contiguous bytes
                const size_t blk = ((size_t)b * a.Hkv + g) * S + s;
                uint16_t* dst = a.part_h + blk * (16 * G * D) + (size_t)(((vs * C::NT32 + r) * 4) * 64 + lane) * 4;
                const float sc = __builtin_ldexpf(inv, jv);
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    u32x2_t x;
                    x[0] = pack_f16x2(o[sl][r][4 * q4] * sc, o[sl][r][4 * q4 + 1] * sc);
                    x[1] = pack_f16x2(o[sl][r][4 * q4 + 2] * sc, o[sl][r][4 * q4 + 3] * sc);
                    __builtin_nontemporal_store(x, reinterpret_cast<u32x2_t*>(dst + q4 * 256));
                }
            }
        }
        if (a.out == nullptr && c == 0 && lane < 32) {
            const float m = rowv[row];
            const float lg = m + __builtin_log2f(l) - (float)jv;
            if (a.part_o32 != nullptr) {
                a.part_lse32[(((size_t)br * Hq + hq) * a.T_max + t_off + t) * S + s] = l > 0.0f ? lg * kLn2 : -INFINITY;
            } else {
                const size_t blk = ((size_t)b * a.Hkv + g) * S + s;
                a.part_hlse[blk * (16 * G) + row] = l > 0.0f ? lg * kLn2 : -INFINITY;
            }
        }
    }
}

// run the body with the number of row tiles in use as a compile-time constant
template <int D, int G, int NTU, int MASK>
__device__ __forceinline__ void dispatch_tiles(int nt_used, const VerifyArgs& a, uint8_t* lds, int b, int br,
                                               int t_off, int g, int s, int dl, int ctx, int pg_begin, int pg_end) {
    if constexpr (NTU > 1) {
        if (nt_used < NTU) {
            dispatch_tiles<D, G, NTU - 1, MASK>(nt_used, a, lds, b, br, t_off, g, s, dl, ctx, pg_begin, pg_end);
            return;
        }
    }
    partition_body<D, G, NTU, MASK>(a, lds, b, br, t_off, g, s, dl, ctx, pg_begin, pg_end);
}

template <int D, int G, int MASK>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void verify_partition_kernel(const VerifyArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[MASK == kMaskAppend ? Cfg<D, G>::TOTAL_APPEND
                                                                               : Cfg<D, G>::TOTAL];

    // work item: blockIdx.x = (b * Hkv + g) * S + s  (equal (g, s) of different
    // requests sit S * Hkv apart, so they share an XCD when that is a multiple of 8)
    const int S = a.num_splits;
    const int s = blockIdx.x % S;
    const int bg = blockIdx.x / S;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;

    const BlockReq rq = block_req(a.draft_lens, a.context_lens, b, MASK == kMaskChunked ? a.blocks_per_req : 1,
                                  a.T_max);
    const int dl = rq.dl, ctx = rq.ctx;
    if (dl <= 0) return;                                      // request (or block) is a no-op
    const int n_pages = (ctx + kPage - 1) / kPage;
    // a window hides every key before the first one the block's first draft sees
    const int lo_page = MASK == kMaskWindow ? max(0, ctx - dl + 1 - a.window) / kPage : 0;
    const int pg_begin = lo_page + s * a.pages_per_split;
    const int pg_end = min(pg_begin + a.pages_per_split, n_pages);
    const int rows = G * dl;
    if (pg_begin >= pg_end) {                                 // empty split: lse = -inf
        if (a.part_o32 != nullptr) {
            // exported layout: the rows are written too (zero), as the definition gives
            for (int i = threadIdx.x; i < rows * (D / 4); i += kWaves * 64) {
                const int r = i / (D / 4), t = r / G, hq = g * G + r % G;
                const size_t prow = (((size_t)rq.req * a.Hq + hq) * a.T_max + rq.t_off + t) * S + s;
                reinterpret_cast<f32x4_t*>(a.part_o32 + prow * D)[i % (D / 4)] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if (i % (D / 4) == 0) a.part_lse32[prow] = -INFINITY;
            }
        } else {
            for (int r = threadIdx.x; r < rows; r += kWaves * 64)
                a.part_hlse[(((size_t)b * a.Hkv + g) * S + s) * (16 * G) + r] = -INFINITY;
            if (threadIdx.x == 0) a.part_hjv[((size_t)b * a.Hkv + g) * S + s] = 0;
        }
        return;
    }
    dispatch_tiles<D, G, G, MASK>((rows + 15) >> 4, a, lds, b, rq.req, rq.t_off, g, s, dl, ctx, pg_begin, pg_end);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of the tiled fp16 partials the partition writes.  One
// workgroup of kMergeWaves waves per (request, kv head, 32-row tile, 32-column
// slice, q4 group): lane l holds row 32 r + l % 32 and 4 columns, so every load
// of a split is 512 contiguous bytes across a wave.  The waves take contiguous
// quarters of the splits; each issues the loads of up to kMergeBatch splits
// before using any (one memory latency for S <= 64) and folds them into a
// running (M, W, acc) in split order; the quarters are then combined in wave
// order through LDS.  The result depends only on S.  A split whose lse is -inf
// is selected away, never multiplied.
// ---------------------------------------------------------------------------
constexpr int kMergeWaves = 4;
constexpr int kMergeBatch = 16;

struct MergeState {
    float M, W;
    f32x4_t acc;
};

// One split into the running state (mn finite): an empty split's weight is
// exp2(-inf) = 0 and its rows, which may hold anything, are zeroed bitwise.
// The split's tiles hold its rows times 2^jv: the rows' weight carries 2^-jv,
// the weight sum does not.
__device__ __forceinline__ void merge_fold(MergeState& st, float l, int jv, u32x2_t x, float mn) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float lw = (l - mn) * kLog2e;
    const float wt = __builtin_amdgcn_exp2f(lw);
    const float wo = __builtin_amdgcn_exp2f(lw - (float)jv);
    const uint32_t keep = l != -INFINITY ? 0xffffffffu : 0u;
    x[0] &= keep;
    x[1] &= keep;
    st.W += wt;
    st.acc[0] = __builtin_fmaf(wo, f16lo(x[0]), st.acc[0]);
    st.acc[1] = __builtin_fmaf(wo, f16hi(x[0]), st.acc[1]);
    st.acc[2] = __builtin_fmaf(wo, f16lo(x[1]), st.acc[2]);
    st.acc[3] = __builtin_fmaf(wo, f16hi(x[1]), st.acc[3]);
}

__device__ __forceinline__ void merge_rescale(MergeState& st, float mn) {
    constexpr float kLog2e = 1.4426950408889634f;
    const float c = st.M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((st.M - mn) * kLog2e);
    st.W *= c;
    st.acc *= c;
    st.M = mn;
}

// ALL_SPLITS (S <= kMergeBatch): each wave takes one group of four columns
// (q4 = its index) and every split, so no wave waits for another; the grid is
// a quarter of the size.
template <int D, int G, bool CHUNKED, bool ALL_SPLITS>
__global__ __launch_bounds__(kMergeWaves * 64) void splitk_merge_tiled_kernel(const TiledMergeArgs a) {
    constexpr int NSL = Cfg<D, G>::NSL, NT32 = Cfg<D, G>::NT32, ROWS = 16 * G;
    __shared__ float xch[kMergeWaves - 1][6][64];
    // blockIdx.x = (r * NSL + v) * 4 + q4 (ALL_SPLITS: r * NSL + v, q4 = wave),
    // blockIdx.y = kv head, blockIdx.z = request
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int q4 = ALL_SPLITS ? wv : (int)(blockIdx.x % 4);
    const int rv = ALL_SPLITS ? (int)blockIdx.x : (int)(blockIdx.x / 4);
    const int v = rv % NSL;
    const int r = rv / NSL;
    const int g = blockIdx.y, b = blockIdx.z;
    const BlockReq rq = block_req(a.draft_lens, nullptr, b, CHUNKED ? a.blocks_per_req : 1, a.T_max);
    const int lim = G * rq.dl;
    if (32 * r >= lim) return;                                // uniform: no row of this tile is a draft row
    const int row = 32 * r + (lane & 31);
    const int S = a.num_splits;
    const int per = (S + kMergeWaves - 1) / kMergeWaves;
    const int s_begin = ALL_SPLITS ? 0 : min(S, wv * per), s_end = ALL_SPLITS ? S : min(S, s_begin + per);
    const size_t blk0 = ((size_t)b * a.Hkv + g) * S;
    const uint16_t* src = a.part_h + blk0 * (ROWS * D) + (size_t)(((v * NT32 + r) * 4 + q4) * 64 + lane) * 4;
    const float* lse = a.part_hlse + blk0 * ROWS + row;
    const int* jvs = a.part_hjv + blk0;

    MergeState st{-INFINITY, 0.0f, f32x4_t{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = s_begin; s0 < s_end; s0 += kMergeBatch) {
        u32x2_t x[kMergeBatch];
        float l[kMergeBatch];
        int jw[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            // every load is issued (a split past the range re-reads the last
            // one, in bounds) and then selected away: no branch per load
            const uint32_t sp = (uint32_t)min(s0 + u, s_end - 1);
            x[u] = *reinterpret_cast<const u32x2_t*>(src + sp * (uint32_t)(ROWS * D));
            l[u] = lse[sp * (uint32_t)ROWS];
            jw[u] = jvs[sp];
        }
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) l[u] = s0 + u < s_end ? l[u] : -INFINITY;
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) mb = fmaxf(mb, l[u]);
        const float mn = fmaxf(st.M, mb);
        if (mn == -INFINITY) continue;                        // no split with a visible key yet
        merge_rescale(st, mn);
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
            merge_fold(st, l[u], jw[u], x[u], mn);
    }
    if constexpr (!ALL_SPLITS) {
        if (wv > 0) {
            xch[wv - 1][0][lane] = st.M;
            xch[wv - 1][1][lane] = st.W;
#pragma unroll
            for (int e = 0; e < 4; ++e) xch[wv - 1][2 + e][lane] = st.acc[e];
        }
        __syncthreads();
        if (wv > 0) return;
#pragma unroll
        for (int k = 0; k < kMergeWaves - 1; ++k) {
            const float Mk = xch[k][0][lane];
            const float mn = fmaxf(st.M, Mk);
            if (mn == -INFINITY) continue;
            merge_rescale(st, mn);
            // a wave without a live split holds W = 0 and acc = 0, and gets c = 0
            const float c = __builtin_amdgcn_exp2f((Mk - mn) * 1.4426950408889634f);
            st.W = __builtin_fmaf(c, xch[k][1][lane], st.W);
#pragma unroll
            for (int e = 0; e < 4; ++e) st.acc[e] = __builtin_fmaf(c, xch[k][2 + e][lane], st.acc[e]);
        }
    }
    if (row >= lim) return;
    const float inv = st.W > 0.0f ? 1.0f / st.W : 0.0f;
    const int t = row / G, hq = g * G + row % G;
    const int d = 32 * v + 8 * q4 + 4 * (lane >> 5);
    u32x2_t o;
    o[0] = (uint32_t)f32_to_bf16_rne(st.acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(st.acc[1] * inv) << 16);
    o[1] = (uint32_t)f32_to_bf16_rne(st.acc[2] * inv) | ((uint32_t)f32_to_bf16_rne(st.acc[3] * inv) << 16);
    *reinterpret_cast<u32x2_t*>(a.out + (((size_t)rq.req * a.T_max + rq.t_off + t) * a.Hq + hq) * D + d) = o;
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of fp32 partial rows in the exported layout
// (part_o [B][Hq][T_max][S][D], part_lse [B][Hq][T_max][S]).  D / 4 threads per
// output row, 4 consecutive columns each (16-byte loads); a thread issues the
// loads of kMergeBatch splits before folding them in split order, so the
// result depends only on S.  Rows are numbered in the output's order
// (b, t, h), so neighbouring threads of a workgroup write neighbouring rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void splitk_merge_rows_kernel(const RowMergeArgs a) {
    constexpr int TPR = D / 4;                                // threads per output row
    constexpr int RPB = 256 / TPR;                            // rows per workgroup
    constexpr float kLog2e = 1.4426950408889634f;
    const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c4 = threadIdx.x % TPR;
    if (row >= (long)a.B * a.T_max * a.Hq) return;
    const int h = (int)(row % a.Hq);
    const long bt = row / a.Hq;
    const int t = (int)(bt % a.T_max), b = (int)(bt / a.T_max);
    if (t >= min(a.draft_lens[b], a.T_max)) return;           // not a draft row: untouched
    const int S = a.num_splits;
    const size_t prow = (((size_t)b * a.Hq + h) * a.T_max + t) * (size_t)S;
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.part_o + prow * D) + c4;
    const float* lse = a.part_lse + prow;
    float M = -INFINITY, W = 0.0f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
        f32x4_t x[kMergeBatch];
        float l[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const int sp = min(s0 + u, S - 1);                // past the end: re-read, selected away
            x[u] = src[(size_t)sp * TPR];
            l[u] = lse[sp];
        }
        float mb = -INFINITY;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            l[u] = s0 + u < S ? l[u] : -INFINITY;
            mb = fmaxf(mb, l[u]);
        }
        const float mn = fmaxf(M, mb);
        if (mn == -INFINITY) continue;                        // no split with a visible key yet
        const float cr = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((M - mn) * kLog2e);
        W *= cr;
        acc *= cr;
        M = mn;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            // an empty split weighs exp2(-inf) = 0 and its row, which may hold
            // anything, is zeroed bitwise
            const float wt = __builtin_amdgcn_exp2f((l[u] - mn) * kLog2e);
            const uint32_t keep = l[u] != -INFINITY ? 0xffffffffu : 0u;
            W += wt;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                acc[e] = __builtin_fmaf(wt, bit_cast<float>(bit_cast<uint32_t>(x[u][e]) & keep), acc[e]);
        }
    }
    const float inv = W > 0.0f ? 1.0f / W : 0.0f;
    u32x2_t o;
    o[0] = (uint32_t)f32_to_bf16_rne(acc[0] * inv) | ((uint32_t)f32_to_bf16_rne(acc[1] * inv) << 16);
    o[1] = (uint32_t)f32_to_bf16_rne(acc[2] * inv) | ((uint32_t)f32_to_bf16_rne(acc[3] * inv) << 16);
    *reinterpret_cast<u32x2_t*>(a.out + (((size_t)b * a.T_max + t) * a.Hq + h) * D + 4 * c4) = o;
}

bool merge_rows_supported(int D) { return D == 64 || D == 128 || D == 256; }

template <int D>
static hipError_t launch_merge_rows_d(const RowMergeArgs& a, hipStream_t stream) {
    constexpr int RPB = 256 / (D / 4);
    const long rows = (long)a.B * a.T_max * a.Hq;
    if (rows <= 0) return hipSuccess;
    const long blocks = (rows + RPB - 1) / RPB;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((splitk_merge_rows_kernel<D>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_splitk_merge_rows(const RowMergeArgs& a, hipStream_t stream) {
    if (a.D == 64) return launch_merge_rows_d<64>(a, stream);
    if (a.D == 128) return launch_merge_rows_d<128>(a, stream);
    if (a.D == 256) return launch_merge_rows_d<256>(a, stream);
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
bool verify_supported(int D, int G) {
    return (D == 64 && G == 4) || (D == 128 && G == 8) || (D == 256 && G == 6);
}

template <int D, int G>
static hipError_t launch_partition_dg(const VerifyArgs& a, hipStream_t stream) {
    const long blocks = (long)a.B * a.Hkv * a.num_splits;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (a.blocks_per_req > 1)
        hipLaunchKernelGGL((verify_partition_kernel<D, G, kMaskChunked>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
    else if (a.block_masks != nullptr)
        hipLaunchKernelGGL((verify_partition_kernel<D, G, kMaskTree>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
    else if (a.window > 0)
        hipLaunchKernelGGL((verify_partition_kernel<D, G, kMaskWindow>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
    else if (a.k_src != nullptr)
        hipLaunchKernelGGL((verify_partition_kernel<D, G, kMaskAppend>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
    else
        hipLaunchKernelGGL((verify_partition_kernel<D, G, kMaskCausal>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_verify_partition(const VerifyArgs& a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (a.D == 64 && G == 4) return launch_partition_dg<64, 4>(a, stream);
    if (a.D == 128 && G == 8) return launch_partition_dg<128, 8>(a, stream);
    if (a.D == 256 && G == 6) return launch_partition_dg<256, 6>(a, stream);
    return hipErrorInvalidValue;
}

template <int D, int G>
static hipError_t launch_merge_tiled_dg(const TiledMergeArgs& a, hipStream_t stream) {
    if (a.B <= 0 || a.Hkv <= 0) return hipSuccess;
    if (a.B > 65535 || a.Hkv > 65535) return hipErrorInvalidConfiguration;
    const bool all = a.num_splits <= kMergeBatch;
    const dim3 grid(Cfg<D, G>::NT32 * Cfg<D, G>::NSL * (all ? 1 : 4), (unsigned)a.Hkv, (unsigned)a.B);
    const dim3 block(kMergeWaves * 64);
    if (a.blocks_per_req > 1) {
        if (all) hipLaunchKernelGGL((splitk_merge_tiled_kernel<D, G, true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((splitk_merge_tiled_kernel<D, G, true, false>), grid, block, 0, stream, a);
    } else {
        if (all) hipLaunchKernelGGL((splitk_merge_tiled_kernel<D, G, false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((splitk_merge_tiled_kernel<D, G, false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_splitk_merge_tiled(const TiledMergeArgs& a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (a.D == 64 && G == 4) return launch_merge_tiled_dg<64, 4>(a, stream);
    if (a.D == 128 && G == 8) return launch_merge_tiled_dg<128, 8>(a, stream);
    if (a.D == 256 && G == 6) return launch_merge_tiled_dg<256, 6>(a, stream);
    return hipErrorInvalidValue;
}


}  // namespace splash
