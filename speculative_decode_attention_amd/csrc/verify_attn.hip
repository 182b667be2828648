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
// Work decomposition.  One workgroup (4 waves, one per SIMD) per (request b,
// kv head g, context split s).  Its rows are the R = G * d query rows that
// share kv head g (G = Hq / Hkv heads times d drafts), ordered r = t * G + hh so
// that a shorter draft truncates a prefix of rows; rows are padded to tiles of
// 16 and the number of tiles in use is a compile-time parameter of the body.
//  * Q is loaded once and kept in accumulation registers (AGPRs) of every wave,
//    laid out as the B operand of 16x16x32 bf16 MFMAs (6 tiles x 8 blocks = 192
//    registers at D = 256, G = 6, 16 drafts).
//  * The context is walked in steps of kPagesPerIter = 4 pages (64 tokens).
//    Wave w copies page w of a step -- K (4 KB), V (4 KB) and its 32 scales --
//    from HBM straight into LDS with 16-byte direct-to-LDS loads, kStages - 1
//    steps ahead of the step being computed, so the copies for two future steps
//    are in flight while one is consumed.  K rows are XOR-swizzled by 16-byte
//    chunk through the per-lane source address, which makes the MFMA operand
//    reads free of bank conflicts; V pages are already stored as two d-major
//    tiles of 8 tokens, which gives the same property with a verbatim copy.
//  * Wave w computes S^T = K Q^T for page w (16 keys x R rows).  int8 codes x
//    are converted exactly: byte u = x + 128 becomes fp32 then bf16 (exact for
//    0..255), and the bias is removed per row after the MFMA:
//        sum_d q_d x_d = sum_d q_d u_d - 128 * sum_d q_d.
//    The K scale and the softmax scale (in log2 units) are applied in fp32.
//  * The per-row maximum over the step's 64 keys is exchanged through LDS; each
//    wave computes p = exp2(z - m) for its keys, folds the V scale in fp32
//    (P' = p * s_v) and writes P' as fp16 to LDS in the B-operand layout.
//  * Each wave then owns a quarter of the head dimension and accumulates
//    O^T += V^T P'^T over all 64 keys with 16x16x32 fp16 MFMAs; V codes are
//    exact in fp16 (binary16 0x64uu is 1024 + u; subtracting 1152 leaves x).
//  * The epilogue divides by the row sums and writes bf16 rows (one split) or
//    fp32 partial rows plus their natural-log log-sum-exp (several splits).
#include <math.h>

#include "device.h"
#include "launch.h"

namespace splash {

constexpr int kStages = 3;     // LDS ring of page steps: one consumed, two in flight

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) const void* global_cvoid_ptr;

// Direct-to-LDS loads: lane i's 16 (or 4) bytes land at lds + 16 * i (4 * i).
__device__ __forceinline__ void dma16_to_lds(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds((global_cvoid_ptr)src, (lds_void_ptr)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4_to_lds(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds((global_cvoid_ptr)src, (lds_void_ptr)lds, 4, 0, 0);
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

// 16 int8 codes (4 dwords) -> two bf16x8 operands holding code + 128 exactly.
__device__ __forceinline__ uint32_t pack_bf16_bytes(uint32_t u, int hi) {
    const float f0 = (float)((u >> (16 * hi)) & 0xffu);
    const float f1 = (float)((u >> (16 * hi + 8)) & 0xffu);
    // upper halves of the two fp32 values: exact bf16 because the integers fit 8 bits
    return __builtin_amdgcn_perm(bit_cast<uint32_t>(f1), bit_cast<uint32_t>(f0), 0x07060302u);
}

__device__ __forceinline__ void codes16_to_bf16_biased(const u32x4_t raw, bf16x8_t& lo, bf16x8_t& hi) {
    u32x4_t a, b;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t u = raw[w] ^ 0x80808080u;
        a[2 * w] = pack_bf16_bytes(u, 0);
        a[2 * w + 1] = pack_bf16_bytes(u, 1);
        const uint32_t v = raw[w + 2] ^ 0x80808080u;
        b[2 * w] = pack_bf16_bytes(v, 0);
        b[2 * w + 1] = pack_bf16_bytes(v, 1);
    }
    lo = bit_cast<bf16x8_t>(a);
    hi = bit_cast<bf16x8_t>(b);
}

// 8 int8 codes -> fp16x8 holding the codes exactly.
__device__ __forceinline__ f16x8_t codes8_to_f16(const u32x2_t raw) {
    const uint32_t magic = 0x64646464u;
    const f16x2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    u32x4_t h;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const uint32_t u = raw[w] ^ 0x80808080u;
        const f16x2_t e0 = bit_cast<f16x2_t>(__builtin_amdgcn_perm(magic, u, 0x04010400u)) - bias;
        const f16x2_t e1 = bit_cast<f16x2_t>(__builtin_amdgcn_perm(magic, u, 0x04030402u)) - bias;
        h[2 * w] = bit_cast<uint32_t>(e0);
        h[2 * w + 1] = bit_cast<uint32_t>(e1);
    }
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
    static constexpr int P_OFF = kStages * STAGE;             // P'^T operand tiles, fp16
    static constexpr int P_BYTES = (kPagesPerIter / 2) * NT * 64 * 16;
    static constexpr int RED_OFF = P_OFF + P_BYTES;           // [row][wave] fp32 row maxima / sums,
    static constexpr int TOTAL = RED_OFF + (NT * 16 + 1) * 4 * 4;   // then [wave] page V-scale maxima
};

template <int D, int NTU>
struct Tiles {
    static constexpr int KB = D / 32;         // contraction blocks of Q K^T
    static constexpr int CH = D / 16;         // 16-byte chunks in a K row
    static constexpr int DW = D / 4;          // head-dim columns each wave owns in P V
    static constexpr int MT = DW / 16;        // V^T tiles of 16 columns per wave
    static constexpr int SWZ_DIV = CH >= 8 ? 1 : 8 / CH;
    static constexpr int SWZ_MOD = CH >= 8 ? 8 : CH;
    static_assert(D % 64 == 0 && MT >= 1, "head dim must be a multiple of 64");
};

// XOR swizzle of 16-byte chunks inside a K row, by slot.
template <int D>
__device__ __forceinline__ int k_swizzle(int slot) {
    using T = Tiles<D, 1>;
    return (slot / T::SWZ_DIV) % T::SWZ_MOD;
}

// Wave `wave` copies page `pg` of kv head g into stage slot `wave`.
template <int D, int G>
__device__ __forceinline__ void stage_page(uint8_t* stage, int wave, int lane, const VerifyArgs& a,
                                           int page, int g) {
    using A = Arena<D, G>;
    constexpr int CH = D / 16;
    constexpr int NI = A::PAGE / 1024;                        // 16-byte copies per lane per page
    const size_t blk = (size_t)page * a.Hkv + g;
    const int8_t* kp = a.k_pool + blk * A::PAGE;
    const int8_t* vp = a.v_pool + blk * A::PAGE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int c = 64 * i + lane;                          // LDS chunk of this lane
        const int slot = c / CH, pc = c % CH;
        const int lc = pc ^ k_swizzle<D>(slot);               // logical chunk stored there
        dma16_to_lds(kp + slot * D + 16 * lc, stage + A::k_off(wave) + 1024 * i);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16_to_lds(vp + 1024 * i + 16 * lane, stage + A::v_off(wave) + 1024 * i);
    if (lane < 16) {
        const uint16_t* src = lane < 8 ? a.k_scale + blk * kPage + 2 * lane : a.v_scale + blk * kPage + 2 * (lane - 8);
        dma4_to_lds(src, stage + A::s_off(wave));
    }
}

template <int D, int G, int NTU>
__device__ __forceinline__ void partition_body(const VerifyArgs& a, uint8_t* lds, const int b, const int g,
                                               const int s, const int dl, const int ctx, const int pg_begin,
                                               const int pg_end) {
    using A = Arena<D, G>;
    using T = Tiles<D, NTU>;
    constexpr int KB = T::KB, DW = T::DW, MT = T::MT;
    constexpr int NI = A::PAGE / 1024;
    constexpr int LOADS_PER_STEP = 2 * NI + 1;                // DMA instructions per wave per step
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kLn2 = 0.6931471805599453f;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gq = lane >> 4, li = lane & 15;
    const int rows = G * dl;
    const int Hq = a.Hq, S = a.num_splits;
    const int32_t* bt = a.block_table + (size_t)b * a.max_pages_per_seq;
    const int n_steps = (pg_end - pg_begin + kPagesPerIter - 1) / kPagesPerIter;

    // start the copies of the first kStages - 1 steps before touching Q
    auto issue_step = [&](int step) {
        int pg = pg_begin + step * kPagesPerIter + wave;
        if (pg >= pg_end) pg = pg_end - 1;                    // past the split: copy a valid page, masked later
        stage_page<D, G>(lds + (step % kStages) * A::STAGE, wave, lane, a, bt[pg], g);
    };
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
        if (st < n_steps) issue_step(st);

    // ---- Q: B operand of S^T = K Q^T, plus the per-row sum that removes the code bias
    bf16x8_t qf[NTU][KB];
    float qsum[NTU];
#pragma unroll
    for (int nt = 0; nt < NTU; ++nt) {
        const int row = nt * 16 + li;
        float acc = 0.0f;
        const bool ok = row < rows;
        const int t = ok ? row / G : 0, h = g * G + (ok ? row % G : 0);
        const uint16_t* qrow = a.q + (((size_t)b * a.T_max + t) * Hq + h) * D;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int d0 = 64 * (kb >> 1) + 16 * gq + 8 * (kb & 1);
            u32x4_t raw = u32x4_t{0u, 0u, 0u, 0u};
            if (ok) raw = *reinterpret_cast<const u32x4_t*>(qrow + d0);
            qf[nt][kb] = bit_cast<bf16x8_t>(raw);
#pragma unroll
            for (int w = 0; w < 4; ++w)
                acc += bit_cast<float>(raw[w] << 16) + bit_cast<float>(raw[w] & 0xffff0000u);
        }
        qsum[nt] = group4_sum(acc) * 128.0f;
    }
#pragma unroll
    for (int nt = 0; nt < NTU; ++nt)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+a"(qf[nt][kb]));

    float m_run[NTU], l_run[NTU];
    f32x4_t o[MT][NTU];
#pragma unroll
    for (int nt = 0; nt < NTU; ++nt) {
        m_run[nt] = -INFINITY;
        l_run[nt] = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float zscale = a.sm_scale * kLog2e;
    float* red = reinterpret_cast<float*>(lds + A::RED_OFF);
    _Float16* pbuf = reinterpret_cast<_Float16*>(lds + A::P_OFF);

    for (int step = 0; step < n_steps; ++step) {
        // this wave's copies for `step` are done once at most the next step's remain
        if (step + 1 < n_steps) wait_vmcnt<LOADS_PER_STEP>();
        else wait_vmcnt<0>();
        lds_barrier();                                        // every wave's copies visible; step-1 finished
        if (step + kStages - 1 < n_steps) issue_step(step + kStages - 1);
#pragma unroll
        for (int nt = 0; nt < NTU; ++nt) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) asm volatile("" : "+a"(qf[nt][kb]));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) asm volatile("" : "+v"(o[mt][nt]));
        }

        const uint8_t* stage = lds + (step % kStages) * A::STAGE;
        const int pg0 = pg_begin + step * kPagesPerIter;
        const int my_page = pg0 + wave;
        const bool page_ok = my_page < pg_end;               // uniform in the wave

        // ---- S^T = K Q^T for this wave's page
        f32x4_t sacc[NTU];
#pragma unroll
        for (int nt = 0; nt < NTU; ++nt) sacc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const uint8_t* kpage = stage + A::k_off(wave) + li * D;
        const int swz = k_swizzle<D>(li);
#pragma unroll
        for (int c = 0; c < KB / 2; ++c) {
            const u32x4_t raw = *reinterpret_cast<const u32x4_t*>(kpage + 16 * ((4 * c + gq) ^ swz));
            bf16x8_t k0, k1;
            codes16_to_bf16_biased(raw, k0, k1);
#pragma unroll
            for (int nt = 0; nt < NTU; ++nt) {
                sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[nt][2 * c], sacc[nt], 0, 0, 0);
                sacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[nt][2 * c + 1], sacc[nt], 0, 0, 0);
            }
        }

        // ---- scaled scores (masked only on pages that are not fully visible)
        // lane (gq, li) holds keys at slots 4*gq + j of page my_page, for row 16*nt + li
        const u32x2_t ks_raw = *reinterpret_cast<const u32x2_t*>(stage + A::s_off(wave) + 8 * gq);
        const u32x2_t vs_raw = *reinterpret_cast<const u32x2_t*>(stage + A::s_off(wave) + 32 + 8 * gq);
        float kc[4], vsc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kc[j] = f16_bits_to_f32(ks_raw[j >> 1] >> (16 * (j & 1))) * zscale;
            vsc[j] = f16_bits_to_f32(vs_raw[j >> 1] >> (16 * (j & 1)));
        }
        // every key of the page is visible to every row (padded rows see q = 0)
        const bool all_visible = page_ok && my_page * kPage + kPage - 1 <= ctx - dl;
        if (all_visible) {
#pragma unroll
            for (int nt = 0; nt < NTU; ++nt) {
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sacc[nt][j] = (sacc[nt][j] - qsum[nt]) * kc[j];
                    mx = fmaxf(mx, sacc[nt][j]);
                }
                mx = group4_max(mx);
                if (gq == 0) red[(nt * 16 + li) * 4 + wave] = mx;
            }
        } else {
            const int key0 = my_page * kPage + 4 * gq;
#pragma unroll
            for (int nt = 0; nt < NTU; ++nt) {
                const int row = nt * 16 + li;
                const int pos_t = ctx - dl + row / G;         // last key this row may see
                const bool row_ok = page_ok && row < rows;
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float zz = (sacc[nt][j] - qsum[nt]) * kc[j];
                    sacc[nt][j] = (row_ok && key0 + j <= pos_t) ? zz : -INFINITY;
                    mx = fmaxf(mx, sacc[nt][j]);
                }
                mx = group4_max(mx);
                if (gq == 0) red[row * 4 + wave] = mx;
            }
        }
        // largest V scale of this page (masked slots included: a non-finite or
        // huge value only makes the rescaling below exact)
        {
            float vm = fmaxf(fmaxf(vsc[0], vsc[1]), fmaxf(vsc[2], vsc[3]));
            vm = group4_max(vm);
            if (lane == 0) red[A::NT * 16 * 4 + wave] = vm;
        }
        lds_barrier();

        // ---- online softmax with a lazily moved reference.  The reference m of a
        // row only moves when the step's maximum exceeds it by more than tau (log2
        // units), so p = exp2(z - m) <= 2^tau; tau = 8 unless a V scale of the
        // step exceeds 255, where P' = p * s_v could leave the fp16 range, and then
        // tau = 0 (the reference follows the maximum exactly).
        const f32x4_t vsm = *reinterpret_cast<const f32x4_t*>(red + A::NT * 16 * 4);
        const float tau = (fmaxf(fmaxf(vsm[0], vsm[1]), fmaxf(vsm[2], vsm[3])) <= 255.0f) ? 8.0f : 0.0f;
        _Float16* p_dst = pbuf + (((wave >> 1) * NTU) * 64 + (2 * (wave & 1) + (gq >> 1)) * 16 + li) * 8
                          + 4 * (gq & 1);
#pragma unroll
        for (int nt = 0; nt < NTU; ++nt) {
            const int row = nt * 16 + li;
            const f32x4_t mw = *reinterpret_cast<const f32x4_t*>(red + row * 4);
            const float mstep = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
            const bool move = mstep > m_run[nt] + tau;       // -inf + tau stays -inf
            const float alpha = move ? __builtin_amdgcn_exp2f(m_run[nt] - mstep) : 1.0f;
            if (move) m_run[nt] = mstep;
            if (__builtin_amdgcn_ballot_w64(move) != 0) {     // some row of the tile moved
                l_run[nt] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) o[mt][nt] *= alpha;
            }
            // rows that have seen no key yet keep m = -inf; their scores are all -inf
            const float mref = m_run[nt] == -INFINITY ? 0.0f : m_run[nt];
            float psum = 0.0f;
            _Float16 ph[4];
            if (all_visible) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = __builtin_amdgcn_exp2f(sacc[nt][j] - mref);
                    psum += p;
                    ph[j] = (_Float16)(p * vsc[j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p = __builtin_amdgcn_exp2f(sacc[nt][j] - mref);   // exp2(-inf) = 0
                    psum += p;
                    ph[j] = (_Float16)(sacc[nt][j] != -INFINITY ? p * vsc[j] : 0.0f);
                }
            }
            l_run[nt] += psum;                                // this lane's share of the row sum
            u32x2_t packed;
            packed[0] = (uint32_t)bit_cast<uint16_t>(ph[0]) | ((uint32_t)bit_cast<uint16_t>(ph[1]) << 16);
            packed[1] = (uint32_t)bit_cast<uint16_t>(ph[2]) | ((uint32_t)bit_cast<uint16_t>(ph[3]) << 16);
            *reinterpret_cast<u32x2_t*>(p_dst + nt * 64 * 8) = packed;
        }
        lds_barrier();

        // ---- O^T += V^T P'^T over the step's keys, for this wave's head-dim quarter
#pragma unroll
        for (int kb2 = 0; kb2 < kPagesPerIter / 2; ++kb2) {
            if (pg0 + 2 * kb2 < pg_end) {                    // uniform
                f16x8_t pf[NTU];
#pragma unroll
                for (int nt = 0; nt < NTU; ++nt)
                    pf[nt] = *reinterpret_cast<const f16x8_t*>(pbuf + ((kb2 * NTU + nt) * 64 + lane) * 8);
                // lane group gq holds keys of page 2*kb2 + gq/2, tile (slots 8*(gq&1)..+7)
                const uint8_t* vt = stage + A::v_off(2 * kb2 + (gq >> 1)) + (gq & 1) * (D * 8);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int d = wave * DW + mt * 16 + li;
                    const f16x8_t vf = codes8_to_f16(*reinterpret_cast<const u32x2_t*>(vt + d * 8));
#pragma unroll
                    for (int nt = 0; nt < NTU; ++nt)
                        o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[nt], o[mt][nt], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: row sums across lane groups and waves, then normalise
    lds_barrier();
#pragma unroll
    for (int nt = 0; nt < NTU; ++nt) {
        const float l = group4_sum(l_run[nt]);
        if (gq == 0) red[(nt * 16 + li) * 4 + wave] = l;
    }
    lds_barrier();
#pragma unroll
    for (int nt = 0; nt < NTU; ++nt) {
        const int row = nt * 16 + li;
        if (row >= rows) continue;
        const f32x4_t lw = *reinterpret_cast<const f32x4_t*>(red + row * 4);
        const float l = (lw[0] + lw[1]) + (lw[2] + lw[3]);
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        const int t = row / G, h = g * G + row % G;
        if (a.out != nullptr) {
            uint16_t* orow = a.out + (((size_t)b * a.T_max + t) * Hq + h) * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int d = wave * DW + mt * 16 + 4 * gq;
                u32x2_t w;
                w[0] = (uint32_t)f32_to_bf16_rne(o[mt][nt][0] * inv) |
                       ((uint32_t)f32_to_bf16_rne(o[mt][nt][1] * inv) << 16);
                w[1] = (uint32_t)f32_to_bf16_rne(o[mt][nt][2] * inv) |
                       ((uint32_t)f32_to_bf16_rne(o[mt][nt][3] * inv) << 16);
                *reinterpret_cast<u32x2_t*>(orow + d) = w;
            }
        } else {
            const size_t prow = (((size_t)b * Hq + h) * a.T_max + t) * S + s;
            float* po = a.part_o + prow * D;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int d = wave * DW + mt * 16 + 4 * gq;
                *reinterpret_cast<f32x4_t*>(po + d) = o[mt][nt] * inv;
            }
            if (wave == 0 && gq == 0)
                a.part_lse[prow] = l > 0.0f ? (m_run[nt] + log2f(l)) * kLn2 : -INFINITY;
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
__global__ __launch_bounds__(256, 1) void verify_partition_kernel(const VerifyArgs a) {
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
        for (int r = threadIdx.x; r < rows; r += 256) {
            const int t = r / G, h = g * G + r % G;
            a.part_lse[(((size_t)b * a.Hq + h) * a.T_max + t) * S + s] = -INFINITY;
        }
        return;
    }
    dispatch_tiles<D, G, G>((rows + 15) >> 4, a, lds, b, g, s, dl, ctx, pg_begin, pg_end);
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of S context splits: one wave per output row.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void splitk_merge_kernel(const MergeArgs a) {
    constexpr int E = D / 64;
    const int lane = threadIdx.x;
    const int h = blockIdx.x % a.Hq;
    const int bt = blockIdx.x / a.Hq;
    const int t = bt % a.T_max;
    const int b = bt / a.T_max;
    if (t >= a.draft_lens[b]) return;
    const int S = a.num_splits;
    const size_t prow = (((size_t)b * a.Hq + h) * a.T_max + t) * S;
    const float* lse = a.part_lse + prow;
    float M = -INFINITY;
    for (int s = lane; s < S; s += 64) M = fmaxf(M, lse[s]);
    M = wave_max(M);
    float acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0f;
    float W = 0.0f;
    for (int s = 0; s < S; ++s) {                             // ascending s: deterministic
        const float l = lse[s];
        if (l == -INFINITY) continue;                         // empty split: its row is never read
        const float w = expf(l - M);
        W += w;
        const float* src = a.part_o + (prow + s) * D + lane * E;
        if constexpr (E == 4) {
            const f32x4_t v = *reinterpret_cast<const f32x4_t*>(src);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += w * v[e];
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] += w * src[e];
        }
    }
    uint16_t* dst = a.out + (((size_t)b * a.T_max + t) * a.Hq + h) * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = f32_to_bf16_rne(acc[e] / W);
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
    hipLaunchKernelGGL((verify_partition_kernel<D, G>), dim3((unsigned)blocks), dim3(256), 0, stream, a);
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
        case 64: hipLaunchKernelGGL((splitk_merge_kernel<64>), dim3((unsigned)blocks), dim3(64), 0, stream, a); break;
        case 128: hipLaunchKernelGGL((splitk_merge_kernel<128>), dim3((unsigned)blocks), dim3(64), 0, stream, a); break;
        case 256: hipLaunchKernelGGL((splitk_merge_kernel<256>), dim3((unsigned)blocks), dim3(64), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace splash
