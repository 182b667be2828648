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
// Work decomposition.  One workgroup of 8 waves (two per SIMD, so that each
// SIMD always has a second wave to issue from) per (request b, kv head g,
// context split s).  Its rows are the R = G * d query rows that share kv head
// g, ordered r = t * G + hh so that a shorter draft truncates a prefix of rows,
// padded to tiles of 16; the tile count in use is a compile-time parameter of
// the body.  The 8 waves are two row halves (half h owns tiles h, h+2, h+4)
// times four: wave (h, w) computes scores for page w of each step and owns
// head-dim quarter w of the output, for the rows of half h.
//  * Q is loaded once, converted bf16 -> fp16 (exact for 2^-17 <= |q| <= 65504)
//    and kept in registers as the B operand of 16x16x32 fp16 MFMAs.
//  * The context is walked in steps of kPagesPerIter = 4 pages (64 tokens).
//    Pages are copied HBM -> LDS with 16-byte direct-to-LDS loads into a ring
//    of kStages steps, two steps ahead of their use; half 0 copies the K pages
//    and the scales, half 1 the V pages.  K rows are XOR-swizzled by 16-byte
//    chunk through the per-lane source address, which keeps the MFMA operand
//    reads free of bank conflicts; V pages are stored as two d-major tiles of 8
//    tokens, which gives the same property with a verbatim copy.
//  * int8 codes x become fp16 with one byte permute: binary16 0x64uu is
//    1024 + u, and u = x + 128, so the operand holds 1152 + x exactly.  For K the
//    bias is removed per row after the MFMA (sum_d q_d (1152 + x_d) - 1152 *
//    sum_d q_d); for V it is subtracted exactly with a packed fp16 add.
//  * Per step: S^T = K Q^T for the wave's page; scaled scores (K scale and
//    softmax scale in log2 units, fp32); row maxima exchanged in LDS among the
//    half's four waves; p = exp2(z - m) against a lazily moved reference m;
//    P' = p * s_v written as fp16 to LDS; then O^T += V^T P'^T for the wave's
//    head-dim quarter over the step's 64 keys.  The P V product of a step runs
//    after the next step's Q K^T, inside the same barrier interval, so each
//    step needs two workgroup barriers.
//  * The epilogue divides by the row sums and writes bf16 rows (one split) or
//    fp32 partial rows plus their natural-log log-sum-exp (several splits).
#include <math.h>

#include "device.h"
#include "launch.h"

namespace splash {

constexpr int kStages = 4;     // LDS ring of page steps (two ahead, one in Q K^T, one in P V)
constexpr int kWaves = 8;      // two row halves x four

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// 32-bit LDS address of a pointer into the workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(lds_void_ptr)(p);
}

// Direct-to-LDS loads: lane i's 16 (or 4) bytes land at LDS address
// m0 + 16 * i (4 * i).  Issued as inline assembly so that the compiler adds no
// wait of its own: these copies are waited for explicitly (wait_vmcnt) before
// the barrier that publishes a stage.  `lds` must be uniform in the wave.
// Ordering: volatile asm statements keep their order, and the barrier and
// wait statements carry the memory clobber that orders the LDS reads.
__device__ __forceinline__ void dma16_to_lds(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dwordx4 %0, off" :: "v"(src), "{m0}"(lds));
}
__device__ __forceinline__ void dma4_to_lds(const void* src, uint32_t lds) {
    asm volatile("global_load_lds_dword %0, off" :: "v"(src), "{m0}"(lds));
}

// Block-table entry through the scalar cache (the table is read-only here).
// As a plain C++ load the compiler would use a vector load whose wait also
// drains the in-flight page copies.
__device__ __forceinline__ int load_page_id(const int32_t* p) {
    int v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
    return v;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS traffic only: outstanding direct-to-LDS copies stay
// in flight across it (their completion is waited for explicitly).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Codes 0-1 (sel 0) or 2-3 (sel 1) of a dword -> two fp16 values 1152 + code.
__device__ __forceinline__ uint32_t codes2_to_f16_biased(uint32_t raw, int sel) {
    const uint32_t u = raw ^ 0x80808080u;
    return __builtin_amdgcn_perm(0x64646464u, u, sel ? 0x04030402u : 0x04010400u);
}

// 16 codes -> two fp16x8 operands holding 1152 + code.
__device__ __forceinline__ void codes16_to_f16_biased(const u32x4_t raw, f16x8_t& lo, f16x8_t& hi) {
    const u32x4_t a = {codes2_to_f16_biased(raw[0], 0), codes2_to_f16_biased(raw[0], 1),
                       codes2_to_f16_biased(raw[1], 0), codes2_to_f16_biased(raw[1], 1)};
    const u32x4_t b = {codes2_to_f16_biased(raw[2], 0), codes2_to_f16_biased(raw[2], 1),
                       codes2_to_f16_biased(raw[3], 0), codes2_to_f16_biased(raw[3], 1)};
    lo = bit_cast<f16x8_t>(a);
    hi = bit_cast<f16x8_t>(b);
}

// 8 codes -> fp16x8 holding the codes exactly (the 1152 bias subtracted).
__device__ __forceinline__ f16x8_t codes8_to_f16(const u32x2_t raw) {
    const f16x2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    u32x4_t h;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        h[k] = bit_cast<uint32_t>(bit_cast<f16x2_t>(codes2_to_f16_biased(raw[k >> 1], k & 1)) - bias);
    return bit_cast<f16x8_t>(h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) { return (float)bit_cast<_Float16>((uint16_t)b); }

// LDS arena of one workgroup.
template <int D, int G>
struct Arena {
    static constexpr int PAGE = kPage * D;                    // bytes of one K or V page (one kv head)
    static constexpr int SCALES = 2 * kPage * 2;              // 16 fp16 K scales then 16 fp16 V scales
    static constexpr int STAGE = kPagesPerIter * (2 * PAGE + SCALES);
    static constexpr int k_off(int j) { return j * PAGE; }
    static constexpr int v_off(int j) { return kPagesPerIter * PAGE + j * PAGE; }
    static constexpr int s_off(int j) { return 2 * kPagesPerIter * PAGE + j * SCALES; }
    static constexpr int NT = G;                              // row tiles for up to 16 drafts
    static constexpr int NTH = (NT + 1) / 2;                  // row tiles per half
    static constexpr int P_OFF = kStages * STAGE;             // two buffers of P'^T operand tiles, fp16
    static constexpr int P_BUF = 2 * (kPagesPerIter / 2) * NTH * 64 * 16;   // [half][kb2][tile][lane][16 B]
    static constexpr int RED_OFF = P_OFF + 2 * P_BUF;         // [row][page] fp32 maxima / sums,
    static constexpr int TOTAL = RED_OFF + (NT * 16 + 1) * 4 * 4;   // then [page] V-scale maxima
    static_assert(TOTAL <= 160 * 1024, "LDS arena exceeds 160 KB");
};

template <int D>
struct Tiles {
    static constexpr int KB = D / 32;         // contraction blocks of Q K^T
    static constexpr int CH = D / 16;         // 16-byte chunks in a K row
    static constexpr int DW = D / 4;          // head-dim columns each wave owns in P V
    static constexpr int MT = DW / 16;        // V^T tiles of 16 columns per wave
    static constexpr int NI = kPage * D / 1024;   // 16-byte copies per lane per page
    static constexpr int SWZ_DIV = CH >= 8 ? 1 : 8 / CH;
    static constexpr int SWZ_MOD = CH >= 8 ? 8 : CH;
    static_assert(D % 64 == 0 && MT >= 1, "head dim must be a multiple of 64");
};

// XOR swizzle of 16-byte chunks inside a K row, by slot.
template <int D>
__device__ __forceinline__ int k_swizzle(int slot) {
    return (slot / Tiles<D>::SWZ_DIV) % Tiles<D>::SWZ_MOD;
}

// Half 0 wave w copies the K page and the scales of page w of a step into the
// stage at LDS address `stage`; half 1 wave w copies its V page.
template <int D, int G>
__device__ __forceinline__ void stage_page(uint32_t stage, int half, int w, int lane, const VerifyArgs& a,
                                           int page, int g) {
    using A = Arena<D, G>;
    using T = Tiles<D>;
    const size_t blk = (size_t)page * a.Hkv + g;
    if (half == 0) {
        const int8_t* kp = a.k_pool + blk * A::PAGE;
#pragma unroll
        for (int i = 0; i < T::NI; ++i) {
            const int c = 64 * i + lane;                      // LDS chunk of this lane
            const int slot = c / T::CH, pc = c % T::CH;
            const int lc = pc ^ k_swizzle<D>(slot);           // logical chunk stored there
            dma16_to_lds(kp + slot * D + 16 * lc, stage + A::k_off(w) + 1024 * i);
        }
        if (lane < 16) {
            const uint16_t* src = lane < 8 ? a.k_scale + blk * kPage + 2 * lane
                                           : a.v_scale + blk * kPage + 2 * (lane - 8);
            dma4_to_lds(src, stage + A::s_off(w));
        }
    } else {
        const int8_t* vp = a.v_pool + blk * A::PAGE;
#pragma unroll
        for (int i = 0; i < T::NI; ++i) dma16_to_lds(vp + 1024 * i + 16 * lane, stage + A::v_off(w) + 1024 * i);
    }
}

template <int D, int G, int NTU>
__device__ __forceinline__ void partition_body(const VerifyArgs& a, uint8_t* lds, const int b, const int g,
                                               const int s, const int dl, const int ctx, const int pg_begin,
                                               const int pg_end) {
    using A = Arena<D, G>;
    using T = Tiles<D>;
    constexpr int KB = T::KB, DW = T::DW, MT = T::MT;
    constexpr int NTH = (NTU + 1) / 2;                        // tiles of this body per half
    constexpr int LOADS_H0 = T::NI + 1, LOADS_H1 = T::NI;     // copies per wave per step
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kLn2 = 0.6931471805599453f;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int half = wave >> 2, w = wave & 3;
    const int gq = lane >> 4, li = lane & 15;
    const int rows = G * dl;
    const int Hq = a.Hq, S = a.num_splits;
    const int32_t* bt = a.block_table + (size_t)b * a.max_pages_per_seq;
    const int n_steps = (pg_end - pg_begin + kPagesPerIter - 1) / kPagesPerIter;
    // half 1 has one tile fewer when the tile count is odd
    const bool last_tile = (half == 0) || (NTU % 2 == 0);
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane(lds_addr(lds));

    auto issue_step = [&](int step) {
        int pg = pg_begin + step * kPagesPerIter + w;
        if (pg >= pg_end) pg = pg_end - 1;                    // past the split: copy a valid page, masked later
        stage_page<D, G>(lds_base + (step % kStages) * A::STAGE, half, w, lane, a, load_page_id(bt + pg), g);
    };
    issue_step(0);
    if (n_steps > 1) issue_step(1);

    // ---- Q for this half's tiles (tile i of the half is row tile half + 2 i), fp16,
    // as the B operand of S^T = K Q^T; the per-row code bias 1152 * sum_d q_d
    f16x8_t qf[NTH][KB];
    float qbias[NTH];
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        const int row = (half + 2 * i) * 16 + li;
        const bool ok = row < rows && (i + 1 < NTH || last_tile);
        const int t = ok ? row / G : 0, h = g * G + (ok ? row % G : 0);
        const uint16_t* qrow = a.q + (((size_t)b * a.T_max + t) * Hq + h) * D;
        float acc = 0.0f;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int d0 = 64 * (kb >> 1) + 16 * gq + 8 * (kb & 1);
            u32x4_t raw = u32x4_t{0u, 0u, 0u, 0u};
            if (ok) raw = *reinterpret_cast<const u32x4_t*>(qrow + d0);
            f16x8_t hv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = bit_cast<float>(e & 1 ? raw[e >> 1] & 0xffff0000u : raw[e >> 1] << 16);
                hv[e] = (_Float16)f;
                acc += (float)hv[e];
            }
            qf[i][kb] = hv;
        }
        qbias[i] = group4_sum(acc) * 1152.0f;
    }

    float m_run[NTH], l_run[NTH];
    f32x4_t o[MT][NTH];
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float zscale = a.sm_scale * kLog2e;
    float* red = reinterpret_cast<float*>(lds + A::RED_OFF);
    // P' tiles of this half: [buf][half][kb2][tile][lane][8 fp16]
    auto pbuf = [&](int buf, int kb2, int i) {
        return reinterpret_cast<_Float16*>(lds + A::P_OFF + buf * A::P_BUF) +
               (((half * (kPagesPerIter / 2) + kb2) * NTH + i) * 64) * 8;
    };

    for (int it = 0; it <= n_steps; ++it) {
        // stage `it` copied (this wave's part) and visible to all after the barrier;
        // also publishes P'(it - 1)
        if (it < n_steps) {
            if (it + 1 < n_steps) {
                if (half == 0) wait_vmcnt<LOADS_H0>(); else wait_vmcnt<LOADS_H1>();
            } else {
                wait_vmcnt<0>();
            }
        }
        lds_barrier();
        if (it + 2 < n_steps) issue_step(it + 2);             // into the slot of step it - 2

        // ---- P V for the previous step: O^T += V^T P'^T (this wave's head-dim quarter)
        if (it >= 1) {
            const int pstep = it - 1;
            const uint8_t* pst = lds + (pstep % kStages) * A::STAGE;
            const int ppg0 = pg_begin + pstep * kPagesPerIter;
#pragma unroll
            for (int kb2 = 0; kb2 < kPagesPerIter / 2; ++kb2) {
                if (ppg0 + 2 * kb2 < pg_end) {                // uniform
                    f16x8_t pf[NTH];
#pragma unroll
                    for (int i = 0; i < NTH; ++i)
                        pf[i] = *reinterpret_cast<const f16x8_t*>(pbuf(pstep & 1, kb2, i) + lane * 8);
                    // lane group gq holds keys of page 2*kb2 + gq/2, tile gq&1 (slots 8*(gq&1)..+7)
                    const uint8_t* vt = pst + A::v_off(2 * kb2 + (gq >> 1)) + (gq & 1) * (D * 8);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int d = w * DW + mt * 16 + li;
                        const f16x8_t vf = codes8_to_f16(*reinterpret_cast<const u32x2_t*>(vt + d * 8));
#pragma unroll
                        for (int i = 0; i < NTH; ++i)
                            o[mt][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[i], o[mt][i], 0, 0, 0);
                    }
                }
            }
        }

        // ---- Q K^T for this step's page w and this half's tiles
        f32x4_t sacc[NTH];
        float kc[4], vsc[4];
        bool all_visible = false;
        const int pg0 = pg_begin + it * kPagesPerIter;
        const int my_page = pg0 + w;
        const bool page_ok = my_page < pg_end;               // uniform in the wave
        if (it < n_steps) {
            const uint8_t* stage = lds + (it % kStages) * A::STAGE;
            const uint8_t* kpage = stage + A::k_off(w) + li * D;
            const int swz = k_swizzle<D>(li);
            u32x4_t kraw[KB / 2];
#pragma unroll
            for (int c = 0; c < KB / 2; ++c)
                kraw[c] = *reinterpret_cast<const u32x4_t*>(kpage + 16 * ((4 * c + gq) ^ swz));
#pragma unroll
            for (int i = 0; i < NTH; ++i) sacc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < KB / 2; ++c) {
                f16x8_t k0, k1;
                codes16_to_f16_biased(kraw[c], k0, k1);
#pragma unroll
                for (int i = 0; i < NTH; ++i) {
                    sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, qf[i][2 * c], sacc[i], 0, 0, 0);
                    sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, qf[i][2 * c + 1], sacc[i], 0, 0, 0);
                }
            }
            // lane (gq, li) holds keys at slots 4*gq + j of page my_page, for row 16*tile + li
            const u32x2_t ks_raw = *reinterpret_cast<const u32x2_t*>(stage + A::s_off(w) + 8 * gq);
            const u32x2_t vs_raw = *reinterpret_cast<const u32x2_t*>(stage + A::s_off(w) + 32 + 8 * gq);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                kc[j] = f16_bits_to_f32(ks_raw[j >> 1] >> (16 * (j & 1))) * zscale;
                vsc[j] = f16_bits_to_f32(vs_raw[j >> 1] >> (16 * (j & 1)));
            }
            // every key of the page is visible to every row (padded rows see q = 0)
            all_visible = page_ok && my_page * kPage + kPage - 1 <= ctx - dl;
            float rmax[NTH];
            if (all_visible) {
#pragma unroll
                for (int i = 0; i < NTH; ++i) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        sacc[i][j] = (sacc[i][j] - qbias[i]) * kc[j];
                        mx = fmaxf(mx, sacc[i][j]);
                    }
                    rmax[i] = group4_max(mx);
                }
            } else {
                const int key0 = my_page * kPage + 4 * gq;
#pragma unroll
                for (int i = 0; i < NTH; ++i) {
                    const int row = (half + 2 * i) * 16 + li;
                    const int pos_t = ctx - dl + row / G;     // last key this row may see
                    const bool row_ok = page_ok && row < rows;
                    float mx = -INFINITY;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float zz = (sacc[i][j] - qbias[i]) * kc[j];
                        sacc[i][j] = (row_ok && key0 + j <= pos_t) ? zz : -INFINITY;
                        mx = fmaxf(mx, sacc[i][j]);
                    }
                    rmax[i] = group4_max(mx);
                }
            }
            // largest V scale of the page (masked slots included: a non-finite or
            // huge value only makes the rescaling below exact)
            const float vmax = group4_max(fmaxf(fmaxf(vsc[0], vsc[1]), fmaxf(vsc[2], vsc[3])));
            if (gq == 0) {
#pragma unroll
                for (int i = 0; i < NTH; ++i) red[((half + 2 * i) * 16 + li) * 4 + w] = rmax[i];
                if (li == 0 && half == 0) red[A::NT * 16 * 4 + w] = vmax;
            }
        }
        lds_barrier();

        // ---- online softmax with a lazily moved reference.  A row's reference m
        // only moves when the step's maximum exceeds it by more than tau (log2
        // units), so p = exp2(z - m) <= 2^tau; tau = 8 unless a V scale of the
        // step exceeds 255, where P' = p * s_v could leave the fp16 range, and then
        // tau = 0 (the reference follows the maximum exactly).
        if (it < n_steps) {
            const f32x4_t vsm = *reinterpret_cast<const f32x4_t*>(red + A::NT * 16 * 4);
            const float tau = (fmaxf(fmaxf(vsm[0], vsm[1]), fmaxf(vsm[2], vsm[3])) <= 255.0f) ? 8.0f : 0.0f;
#pragma unroll
            for (int i = 0; i < NTH; ++i) {
                const int row = (half + 2 * i) * 16 + li;
                const f32x4_t mw = *reinterpret_cast<const f32x4_t*>(red + row * 4);
                const float mstep = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
                const bool move = mstep > m_run[i] + tau;     // -inf + tau stays -inf
                const float alpha = move ? __builtin_amdgcn_exp2f(m_run[i] - mstep) : 1.0f;
                if (move) m_run[i] = mstep;
                if (__builtin_amdgcn_ballot_w64(move) != 0) { // some row of the tile moved
                    l_run[i] *= alpha;
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) o[mt][i] *= alpha;
                }
                // rows that have seen no key yet keep m = -inf; their scores are all -inf
                const float mref = m_run[i] == -INFINITY ? 0.0f : m_run[i];
                float psum = 0.0f;
                _Float16 ph[4];
                if (all_visible) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float p = __builtin_amdgcn_exp2f(sacc[i][j] - mref);
                        psum += p;
                        ph[j] = (_Float16)(p * vsc[j]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float p = __builtin_amdgcn_exp2f(sacc[i][j] - mref);   // exp2(-inf) = 0
                        psum += p;
                        ph[j] = (_Float16)(sacc[i][j] != -INFINITY ? p * vsc[j] : 0.0f);
                    }
                }
                l_run[i] += psum;                             // this lane's share of the row sum
                // reader lane (group 2*(w&1) + gq/2, li) of block kb2 = w/2 holds 8 keys;
                // these 4 are its elements 4*(gq&1)..+3
                u32x2_t packed;
                packed[0] = (uint32_t)bit_cast<uint16_t>(ph[0]) | ((uint32_t)bit_cast<uint16_t>(ph[1]) << 16);
                packed[1] = (uint32_t)bit_cast<uint16_t>(ph[2]) | ((uint32_t)bit_cast<uint16_t>(ph[3]) << 16);
                *reinterpret_cast<u32x2_t*>(pbuf(it & 1, w >> 1, i) + ((2 * (w & 1) + (gq >> 1)) * 16 + li) * 8 +
                                            4 * (gq & 1)) = packed;
            }
        }
    }

    // ---- epilogue: row sums across lane groups and the half's four waves, then normalise
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        const float l = group4_sum(l_run[i]);
        if (gq == 0) red[((half + 2 * i) * 16 + li) * 4 + w] = l;
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NTH; ++i) {
        const int row = (half + 2 * i) * 16 + li;
        if (row >= rows || !(i + 1 < NTH || last_tile)) continue;
        const f32x4_t lw = *reinterpret_cast<const f32x4_t*>(red + row * 4);
        const float l = (lw[0] + lw[1]) + (lw[2] + lw[3]);
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        const int t = row / G, h = g * G + row % G;
        if (a.out != nullptr) {
            uint16_t* orow = a.out + (((size_t)b * a.T_max + t) * Hq + h) * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int d = w * DW + mt * 16 + 4 * gq;
                u32x2_t v;
                v[0] = (uint32_t)f32_to_bf16_rne(o[mt][i][0] * inv) |
                       ((uint32_t)f32_to_bf16_rne(o[mt][i][1] * inv) << 16);
                v[1] = (uint32_t)f32_to_bf16_rne(o[mt][i][2] * inv) |
                       ((uint32_t)f32_to_bf16_rne(o[mt][i][3] * inv) << 16);
                *reinterpret_cast<u32x2_t*>(orow + d) = v;
            }
        } else {
            const size_t prow = (((size_t)b * Hq + h) * a.T_max + t) * S + s;
            float* po = a.part_o + prow * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int d = w * DW + mt * 16 + 4 * gq;
                *reinterpret_cast<f32x4_t*>(po + d) = o[mt][i] * inv;
            }
            if (w == 0 && gq == 0)
                a.part_lse[prow] = l > 0.0f ? (m_run[i] + log2f(l)) * kLn2 : -INFINITY;
        }
    }
}

// run the body with the number of row tiles in use as a compile-time constant
template <int D, int G, int NTU>
__device__ __forceinline__ void dispatch_tiles(int nt_used, const VerifyArgs& a, uint8_t* lds, int b, int g,
                                               int s, int dl, int ctx, int pg_begin, int pg_end) {
    if constexpr (NTU > 1) {
        if (nt_used < NTU) {
            dispatch_tiles<D, G, NTU - 1>(nt_used, a, lds, b, g, s, dl, ctx, pg_begin, pg_end);
            return;
        }
    }
    partition_body<D, G, NTU>(a, lds, b, g, s, dl, ctx, pg_begin, pg_end);
}

template <int D, int G>
__global__ __launch_bounds__(kWaves * 64) void verify_partition_kernel(const VerifyArgs a) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[Arena<D, G>::TOTAL];

    // work item: blockIdx.x = (b * Hkv + g) * S + s  (equal (g, s) of different
    // requests sit S * Hkv apart, so they share an XCD when that is a multiple of 8)
    const int S = a.num_splits;
    const int s = blockIdx.x % S;
    const int bg = blockIdx.x / S;
    const int g = bg % a.Hkv;
    const int b = bg / a.Hkv;

    const int dl = a.draft_lens[b];
    if (dl <= 0) return;                                      // request is a no-op
    const int ctx = a.context_lens[b];
    const int n_pages = (ctx + kPage - 1) / kPage;
    const int pg_begin = s * a.pages_per_split;
    const int pg_end = min(pg_begin + a.pages_per_split, n_pages);
    const int rows = G * dl;
    if (pg_begin >= pg_end) {                                 // empty split: mark it, write no row
        for (int r = threadIdx.x; r < rows; r += kWaves * 64) {
            const int t = r / G, h = g * G + r % G;
            a.part_lse[(((size_t)b * a.Hq + h) * a.T_max + t) * S + s] = -INFINITY;
        }
        return;
    }
    dispatch_tiles<D, G, G>((rows + 15) >> 4, a, lds, b, g, s, dl, ctx, pg_begin, pg_end);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of S context splits.  One workgroup per output row.  The
// row's D columns are read as 16-byte groups; the 256 threads are NG groups of
// D/4 threads, and group sg takes splits sg, sg + NG, ...  Every load of a
// round (partial rows and log-sum-exps) is issued before any is used, so a
// round costs one memory latency; S <= NG * kMergeUnroll takes one round.
// M = max_s lse_s and W = sum_s e^(lse_s - M) are computed by every wave in the
// same order; the groups' sums are added in group order.  Fixed orders
// throughout, so the result is deterministic.  A split whose lse is -inf gets
// weight 0 through a select, so its row (which may hold anything) never
// reaches the sum.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
constexpr int kMergeUnroll = 16;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void splitk_merge_kernel(const MergeArgs a) {
    constexpr int C4 = D / 4;                                 // 16-byte column groups
    constexpr int NG = kMergeThreads / C4;                    // split groups
    constexpr float kLog2e = 1.4426950408889634f;
    __shared__ f32x4_t red[NG][C4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int c4 = tid % C4, sg = tid / C4;
    const int h = blockIdx.x % a.Hq;
    const int bt = blockIdx.x / a.Hq;
    const int t = bt % a.T_max;
    const int b = bt / a.T_max;
    if (t >= a.draft_lens[b]) return;
    const int S = a.num_splits;
    const size_t prow = (((size_t)b * a.Hq + h) * a.T_max + t) * S;
    const float* lse = a.part_lse + prow;
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(a.part_o + prow * D) + c4;

    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float M = -INFINITY, W = 0.0f;
    for (int s0 = 0; s0 < S; s0 += NG * kMergeUnroll) {
        f32x4_t v[kMergeUnroll];
        float l[kMergeUnroll];
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const int s = s0 + sg + u * NG;
            v[u] = s < S ? src[(size_t)s * C4] : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const int s = s0 + sg + u * NG;
            l[u] = s < S ? lse[s] : -INFINITY;
        }
        if (s0 == 0) {                                        // M and W over all splits, per wave
            float mx = -INFINITY;
            for (int s = lane; s < S; s += 64) mx = fmaxf(mx, lse[s]);
            M = wave_max(mx);
            float ws = 0.0f;
            if (M != -INFINITY)
                for (int s = lane; s < S; s += 64) {
                    const float x = lse[s];
                    ws += x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((x - M) * kLog2e);
                }
            W = wave_sum(ws);
        }
#pragma unroll
        for (int u = 0; u < kMergeUnroll; ++u) {
            const bool live = l[u] != -INFINITY;
            const float w = live ? __builtin_amdgcn_exp2f((l[u] - M) * kLog2e) : 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += live ? w * v[u][e] : 0.0f;
        }
    }
    red[sg][c4] = acc;
    __syncthreads();
    if (sg == 0) {
        f32x4_t x = red[0][c4];
#pragma unroll
        for (int g2 = 1; g2 < NG; ++g2) x += red[g2][c4];
        const float inv = W > 0.0f ? 1.0f / W : 0.0f;
        u32x2_t o;
        o[0] = (uint32_t)f32_to_bf16_rne(x[0] * inv) | ((uint32_t)f32_to_bf16_rne(x[1] * inv) << 16);
        o[1] = (uint32_t)f32_to_bf16_rne(x[2] * inv) | ((uint32_t)f32_to_bf16_rne(x[3] * inv) << 16);
        *reinterpret_cast<u32x2_t*>(a.out + (((size_t)b * a.T_max + t) * a.Hq + h) * D + 4 * c4) = o;
    }
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
    hipLaunchKernelGGL((verify_partition_kernel<D, G>), dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_verify_partition(const VerifyArgs& a, hipStream_t stream) {
    const int G = a.Hq / a.Hkv;
    if (a.D == 64 && G == 4) return launch_partition_dg<64, 4>(a, stream);
    if (a.D == 128 && G == 8) return launch_partition_dg<128, 8>(a, stream);
    if (a.D == 256 && G == 6) return launch_partition_dg<256, 6>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_splitk_merge(const MergeArgs& a, hipStream_t stream) {
    const long blocks = (long)a.B * a.T_max * a.Hq;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    switch (a.D) {
        case 64: hipLaunchKernelGGL((splitk_merge_kernel<64>), dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream, a); break;
        case 128: hipLaunchKernelGGL((splitk_merge_kernel<128>), dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream, a); break;
        case 256: hipLaunchKernelGGL((splitk_merge_kernel<256>), dim3((unsigned)blocks), dim3(kMergeThreads), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace splash
