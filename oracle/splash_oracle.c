/*
 * splash_oracle.c -- CPU oracle for speculative block-verify decode attention
 * over an int8 paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  The parity tests, the smoke check and the
 * benchmark's CPU-baseline leg load this file's shared library; the product
 * path (the HIP library and its Python binding) never does, and the two share
 * no code, header, table or helper.
 *
 * What is computed, and where the pages fix it:
 *  - The target model checks a whole drafted block in one forward pass
 *    (Splash community summary on discuss.pytorch.kr, section "DFlash 2
 *    speculative decoding as the default path"; bnskd.com article, "Tech core
 *    1").  For attention this means: every draft row t of a request attends
 *    causally over the cached context plus drafts 0..t.
 *  - The decode kernel reads the KV cache stored as 8-bit values and reuses
 *    each page across the query heads of its group and across the verify
 *    tokens (discuss.pytorch.kr summary, section "Metal kernels generated to
 *    shape"; bnskd.com, "Tech core 2").  Reuse is an evaluation strategy; the
 *    value computed is ordinary grouped-query softmax attention over the
 *    dequantised cache.
 *  - The cache is paged and indexed by prefix, so requests sharing a prefix
 *    share its pages (discuss.pytorch.kr summary, section "Batch scheduling
 *    and a memory budget fixed at start-up").  Here: identical block_table
 *    entries.
 *  - Output of speculative decoding equals plain autoregressive decoding
 *    (discuss.pytorch.kr summary, DFlash 2 section).  At the attention level:
 *    row t of a block equals a one-token decode at context position t.
 *  - Beside the causal block: tree-shaped block masks and sliding windows
 *    (same section; see the functions below), greedy acceptance of the drafts
 *    with the rollback of context_lens (same section), and prefill, whose
 *    attention is this same definition with a block of any length (the
 *    summary's Metal-kernels section keeps prefill and verify kernels apart).
 *
 * The pages give no formula, layout or precision.  Readings taken where they
 * are silent (all stated again in the design notes):
 *  - int8, symmetric, no zero point, one fp16 scale per (token, kv head),
 *    scale = fp16_rne(fp32(amax / 127)), codes = clamp(rne(x / scale), -127,
 *    127) computed with the stored fp16 scale, all in IEEE fp32 (this step is
 *    a bit-exact contract, so it is NOT done in fp64);
 *  - context_lens[b] counts the tokens after the draft block was appended;
 *    draft t sits at position context_lens[b] - draft_lens[b] + t;
 *  - query head h belongs to kv head h / (Hq / Hkv);
 *  - K pool layout [num_pages][Hkv][P][D]; V pool layout
 *    [num_pages][Hkv][P/8][D][8] (a V page is two d-major tiles of 8 tokens);
 *    scales [num_pages][Hkv][P]; P must be a multiple of 8;
 *  - q and out are [B][T_max][Hq][D]; rows t >= draft_lens[b] are neither
 *    read nor written.
 *
 * Floating point: attention runs in fp64 throughout and the result stays
 * fp64 (the comparison rounds nothing).  Build with -O2, no -ffast-math.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_OK 0
#define REF_ERR_ARG 1

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32, written from the format's definition.        */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.       */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Exact widening of a binary16 value to binary32. */
float ref_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) << 31;
    uint32_t expo = (h >> 10) & 0x1f;
    uint32_t frac = h & 0x3ff;
    if (expo == 0x1f)                       /* inf / nan */
        return bits_f32(sign | 0x7f800000u | (frac << 13));
    if (expo == 0) {
        /* zero or subnormal: value = frac * 2^-24, exact in binary32 */
        float v = (float)frac * 0x1p-24f;
        return sign ? -v : v;
    }
    return bits_f32(sign | ((expo - 15 + 127) << 23) | (frac << 13));
}

/* Round a binary32 value to the nearest binary16, ties to even. */
uint16_t ref_f32_to_f16_rne(float f)
{
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t expo = (u >> 23) & 0xff;
    uint32_t mant = u & 0x7fffffu;
    if (expo == 0xff)                       /* inf / nan (keep a quiet nan) */
        return (uint16_t)(sign | 0x7c00u | (mant ? 0x200u | (mant >> 13) : 0));
    int e = (int)expo - 127;                /* unbiased exponent            */
    if (e > 15)                             /* |f| >= 2^16: overflow to inf */
        return (uint16_t)(sign | 0x7c00u);
    if (e >= -14) {
        /* normal binary16 candidate: keep 10 of the 23 fraction bits */
        uint32_t h = ((uint32_t)(e + 15) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1fffu;      /* 13 dropped bits             */
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u)))
            h += 1;                          /* may carry into the exponent */
        if (h >= 0x7c00u) return (uint16_t)(sign | 0x7c00u);
        return (uint16_t)(sign | h);
    }
    /* subnormal binary16 (or zero): value = n * 2^-24 with n in [0, 1024] */
    if (e < -25) return sign;               /* below half the smallest step */
    uint32_t sig = mant | 0x800000u;        /* 24-bit significand, 1.f      */
    int shift = -e - 1;                     /* f = sig * 2^(e-23); n = f*2^24 */
    /* n = sig * 2^(e+1) = sig >> (-(e+1)); shift in [14, 24]              */
    uint32_t n = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (n & 1u))) n += 1;
    return (uint16_t)(sign | n);            /* n == 1024 is the smallest normal */
}

/* bf16 is the top half of a binary32, so widening is exact. */
static float bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* ------------------------------------------------------------------------ */
/* Quantiser: one row of D source values -> D int8 codes + one fp16 scale.  */
/* fp32 arithmetic, correctly rounded division, rint() in the default       */
/* round-to-nearest-even mode.                                              */
/* ------------------------------------------------------------------------ */
void ref_quantize_row(const float* x, int D, int8_t* q, uint16_t* scale16)
{
    float amax = 0.0f;
    for (int d = 0; d < D; ++d) {
        float a = fabsf(x[d]);
        if (a > amax) amax = a;
    }
    float s32 = amax / 127.0f;
    uint16_t s16 = ref_f32_to_f16_rne(s32);
    float s = ref_f16_to_f32(s16);
    for (int d = 0; d < D; ++d) {
        if (s == 0.0f) { q[d] = 0; continue; }
        float r = rintf(x[d] / s);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[d] = (int8_t)r;
    }
    *scale16 = s16;
}

/* ------------------------------------------------------------------------ */
/* Pool addressing (the layouts the library documents).                    */
/* ------------------------------------------------------------------------ */
static size_t k_index(int page, int g, int slot, int d, int Hkv, int P, int D)
{ return (((size_t)page * Hkv + g) * P + slot) * D + d; }
static size_t v_index(int page, int g, int slot, int d, int Hkv, int P, int D)
{ return ((((size_t)page * Hkv + g) * (P / 8) + slot / 8) * D + d) * 8 + slot % 8; }
static size_t s_index(int page, int g, int slot, int Hkv, int P)
{ return ((size_t)page * Hkv + g) * P + slot; }

/*
 * splash_ref_kv_append_int8: quantise the K and V rows of each request's new
 * tokens and store them at their cache positions.  Source layout
 * [B][T_max][Hkv][D], fp32 (src_dtype 0) or bf16 bits (src_dtype 1).
 * Token t < draft_lens[b] of request b lands at position
 * context_lens[b] - draft_lens[b] + t.  Nothing else in the pools changes.
 */
int splash_ref_kv_append_int8(const void* k_new, const void* v_new, int src_dtype,
                              int8_t* k_pool, int8_t* v_pool,
                              uint16_t* k_scale, uint16_t* v_scale,
                              const int32_t* block_table, int max_pages_per_seq,
                              const int32_t* context_lens, const int32_t* draft_lens,
                              int B, int T_max, int Hkv, int D, int P, int num_pages)
{
    if (!k_new || !v_new || !k_pool || !v_pool || !k_scale || !v_scale ||
        !block_table || !context_lens || !draft_lens) return REF_ERR_ARG;
    if (B < 0 || T_max < 0 || Hkv <= 0 || D <= 0 || P <= 0 || P % 8 != 0 || num_pages <= 0 ||
        (src_dtype != 0 && src_dtype != 1)) return REF_ERR_ARG;
    float row[1024];
    int8_t codes[1024];
    if (D > 1024) return REF_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        int n = context_lens[b], dl = draft_lens[b];
        if (dl < 0 || dl > T_max || dl > n) return REF_ERR_ARG;
        for (int t = 0; t < dl; ++t) {
            int pos = n - dl + t;
            int pi = pos / P;
            if (pi >= max_pages_per_seq) return REF_ERR_ARG;
            int page = block_table[(size_t)b * max_pages_per_seq + pi];
            int slot = pos % P;
            if (page < 0 || page >= num_pages) return REF_ERR_ARG;
            for (int g = 0; g < Hkv; ++g) {
                size_t src = (((size_t)b * T_max + t) * Hkv + g) * D;
                for (int which = 0; which < 2; ++which) {
                    const void* base = which == 0 ? k_new : v_new;
                    for (int d = 0; d < D; ++d)
                        row[d] = src_dtype == 0 ? ((const float*)base)[src + d]
                                                : bf16_to_f32(((const uint16_t*)base)[src + d]);
                    uint16_t s16;
                    ref_quantize_row(row, D, codes, &s16);
                    if (which == 0) {
                        for (int d = 0; d < D; ++d)
                            k_pool[k_index(page, g, slot, d, Hkv, P, D)] = codes[d];
                        k_scale[s_index(page, g, slot, Hkv, P)] = s16;
                    } else {
                        for (int d = 0; d < D; ++d)
                            v_pool[v_index(page, g, slot, d, Hkv, P, D)] = codes[d];
                        v_scale[s_index(page, g, slot, Hkv, P)] = s16;
                    }
                }
            }
        }
    }
    return REF_OK;
}

/* ------------------------------------------------------------------------ */
/* Attention.                                                               */
/* ------------------------------------------------------------------------ */

/*
 * One output row: draft t of request b, query head h, attending over the
 * keys j in [j_lo, j_hi) that it sees.  Causally (mask == NULL) that is
 * j <= pos_t, pos_t = n - d + t.  With a block mask (the tree of candidates
 * that verification checks at once, DFlash 2 section of the summary: several
 * candidate tokens per position), draft t sees every key before the block and
 * the block key of draft u exactly when bit u of *mask is set.
 * With a window W > 0 (sliding-window attention, which the draft model uses
 * so that its memory stays bounded at long context: summary, DFlash 2
 * section), draft t sees only keys j > pos_t - W, on top of the rule above.
 * Writes the normalised row to out_row (D doubles) and returns the natural
 * log-sum-exp of the scaled scores; no visible key gives -inf and a zero row.
 */
static int key_visible(int j, int blk0, int n, const uint32_t* mask)
{
    if (!mask) return 1;                        /* causal: the range end bounds the keys */
    if (j < blk0) return 1;
    if (j >= n) return 0;
    return (int)((*mask >> (j - blk0)) & 1u);
}

static double attend_row(const uint16_t* q_row,
                         const int8_t* k_pool, const int8_t* v_pool,
                         const uint16_t* k_scale, const uint16_t* v_scale,
                         const int32_t* bt_row, int b_ctx, int b_draft, int t, int g,
                         int Hkv, int D, int P, double sm_scale,
                         int j_lo, int j_hi, const uint32_t* mask, int window, double* z, double* out_row)
{
    int blk0 = b_ctx - b_draft;                 /* first key of the block     */
    int pos = blk0 + t;                         /* this draft's own position */
    int j_base = j_lo;                          /* z is indexed from the range start */
    if (window > 0 && pos - window + 1 > j_lo) j_lo = pos - window + 1;   /* keys j > pos - W */
    int end = mask ? (b_ctx < j_hi ? b_ctx : j_hi)
                   : (pos + 1 < j_hi ? pos + 1 : j_hi);   /* causal: keys 0..pos */
    for (int d = 0; d < D; ++d) out_row[d] = 0.0;
    int seen = 0;
    for (int j = j_lo; j < end; ++j) seen += key_visible(j, blk0, b_ctx, mask);
    if (!seen) return -INFINITY;

    /* scores z_j = sm_scale * <q, K_hat_j>, K_hat_j = scale_j * codes_j */
    double zmax = -INFINITY;
    for (int j = j_lo; j < end; ++j) {
        if (!key_visible(j, blk0, b_ctx, mask)) continue;
        int page = bt_row[j / P], slot = j % P;
        double ks = (double)ref_f16_to_f32(k_scale[s_index(page, g, slot, Hkv, P)]);
        double dot = 0.0;
        for (int d = 0; d < D; ++d) {
            double kh = ks * (double)k_pool[k_index(page, g, slot, d, Hkv, P, D)];
            dot += (double)bf16_to_f32(q_row[d]) * kh;
        }
        z[j - j_base] = sm_scale * dot;
        if (z[j - j_base] > zmax) zmax = z[j - j_base];
    }
    /* softmax weights relative to the max, then the weighted sum of V_hat */
    double wsum = 0.0;
    for (int j = j_lo; j < end; ++j) {
        if (!key_visible(j, blk0, b_ctx, mask)) continue;
        int page = bt_row[j / P], slot = j % P;
        double w = exp(z[j - j_base] - zmax);
        double vs = (double)ref_f16_to_f32(v_scale[s_index(page, g, slot, Hkv, P)]);
        for (int d = 0; d < D; ++d)
            out_row[d] += w * (vs * (double)v_pool[v_index(page, g, slot, d, Hkv, P, D)]);
        wsum += w;
    }
    for (int d = 0; d < D; ++d) out_row[d] /= wsum;
    return zmax + log(wsum);
}

static int check_attn_args(const void* q, const void* out, const void* k_pool, const void* v_pool,
                           const void* k_scale, const void* v_scale, const void* bt,
                           const int32_t* context_lens, const int32_t* draft_lens,
                           int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                           int max_pages_per_seq)
{
    if (!q || !out || !k_pool || !v_pool || !k_scale || !v_scale || !bt ||
        !context_lens || !draft_lens) return REF_ERR_ARG;
    if (B < 0 || T_max < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || P <= 0 ||
        P % 8 != 0 || num_pages <= 0 || max_pages_per_seq < 0) return REF_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        int n = context_lens[b], dl = draft_lens[b];
        if (dl < 0 || dl > T_max || dl > n) return REF_ERR_ARG;
        if ((n + P - 1) / P > max_pages_per_seq) return REF_ERR_ARG;
    }
    return REF_OK;
}

/*
 * splash_ref_verify_attn: fp64 block-verify attention.  out is fp64
 * [B][T_max][Hq][D]; rows t >= draft_lens[b] are left untouched.
 * splash_ref_verify_attn_masked: the same with block_masks uint32 [B][T_max]
 * (bit u of block_masks[b][t]: draft t sees draft u) in place of the causal
 * chain inside the block.
 */
static int verify_attn_impl(const uint16_t* q, double* out,
                            const int8_t* k_pool, const int8_t* v_pool,
                            const uint16_t* k_scale, const uint16_t* v_scale,
                            const int32_t* block_table, int max_pages_per_seq,
                            const int32_t* context_lens, const int32_t* draft_lens,
                            int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                            double sm_scale, const uint32_t* block_masks, int window)
{
    int rc = check_attn_args(q, out, k_pool, v_pool, k_scale, v_scale, block_table,
                             context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages,
                             max_pages_per_seq);
    if (rc) return rc;
    (void)num_pages;
    int group = Hq / Hkv;
    long nrows = (long)B * T_max * Hq;
    int maxn = 0;
    for (int b = 0; b < B; ++b) if (context_lens[b] > maxn) maxn = context_lens[b];
    int fail = 0;
    #pragma omp parallel reduction(|:fail)
    {
    double* z = (double*)malloc(sizeof(double) * (size_t)(maxn + 1));
    if (!z) fail = 1;
    #pragma omp for schedule(dynamic, 1)
    for (long r = 0; r < nrows; ++r) {
        int h = (int)(r % Hq);
        int t = (int)((r / Hq) % T_max);
        int b = (int)(r / ((long)Hq * T_max));
        if (!z || t >= draft_lens[b]) continue;
        size_t row = (((size_t)b * T_max + t) * Hq + h) * D;
        attend_row(q + row, k_pool, v_pool, k_scale, v_scale,
                   block_table + (size_t)b * max_pages_per_seq,
                   context_lens[b], draft_lens[b], t, h / group, Hkv, D, P, sm_scale,
                   0, context_lens[b], block_masks ? block_masks + (size_t)b * T_max + t : NULL,
                   window, z, out + row);
    }
    free(z);
    }
    return fail ? REF_ERR_ARG : REF_OK;
}

int splash_ref_verify_attn(const uint16_t* q, double* out,
                           const int8_t* k_pool, const int8_t* v_pool,
                           const uint16_t* k_scale, const uint16_t* v_scale,
                           const int32_t* block_table, int max_pages_per_seq,
                           const int32_t* context_lens, const int32_t* draft_lens,
                           int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                           double sm_scale)
{
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, sm_scale, NULL, 0);
}

/* splash_ref_verify_attn_masked: block attention where draft t sees every key
 * before the block and the block key of draft u only if bit u of
 * block_masks[b][t] is set: a tree of candidate tokens per position, which the
 * path selector of DFlash 2 chooses among (discuss.pytorch.kr summary, DFlash 2
 * section); the chain mask (bits 0..t) is the causal block. */
int splash_ref_verify_attn_masked(const uint16_t* q, double* out,
                                  const int8_t* k_pool, const int8_t* v_pool,
                                  const uint16_t* k_scale, const uint16_t* v_scale,
                                  const int32_t* block_table, int max_pages_per_seq,
                                  const int32_t* context_lens, const int32_t* draft_lens,
                                  int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                                  double sm_scale, const uint32_t* block_masks)
{
    if (!block_masks || T_max > 32) return REF_ERR_ARG;
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, sm_scale,
                            block_masks, 0);
}

/* splash_ref_verify_attn_window: causal block attention where draft t at
 * position pos_t sees only keys pos_t - window < j <= pos_t (window >= 1): the
 * draft model's sliding-window attention that bounds its memory
 * (discuss.pytorch.kr summary, DFlash 2 section). */
int splash_ref_verify_attn_window(const uint16_t* q, double* out,
                                  const int8_t* k_pool, const int8_t* v_pool,
                                  const uint16_t* k_scale, const uint16_t* v_scale,
                                  const int32_t* block_table, int max_pages_per_seq,
                                  const int32_t* context_lens, const int32_t* draft_lens,
                                  int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                                  double sm_scale, int window)
{
    if (window < 1) return REF_ERR_ARG;
    return verify_attn_impl(q, out, k_pool, v_pool, k_scale, v_scale, block_table, max_pages_per_seq,
                            context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages, sm_scale,
                            NULL, window);
}

/*
 * splash_ref_verify_attn_rows: the same definition for a chosen list of output
 * rows (b, t, h), so that very long contexts can be checked on a sample.
 * out_rows is fp64 [n_rows][D].
 */
int splash_ref_verify_attn_rows(const uint16_t* q,
                                const int8_t* k_pool, const int8_t* v_pool,
                                const uint16_t* k_scale, const uint16_t* v_scale,
                                const int32_t* block_table, int max_pages_per_seq,
                                const int32_t* context_lens, const int32_t* draft_lens,
                                int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                                double sm_scale,
                                const int32_t* rows_b, const int32_t* rows_t, const int32_t* rows_h,
                                int n_rows, double* out_rows)
{
    int rc = check_attn_args(q, out_rows, k_pool, v_pool, k_scale, v_scale, block_table,
                             context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages,
                             max_pages_per_seq);
    if (rc) return rc;
    int group = Hq / Hkv;
    int maxn = 0;
    for (int b = 0; b < B; ++b) if (context_lens[b] > maxn) maxn = context_lens[b];
    for (int i = 0; i < n_rows; ++i) {
        int b = rows_b[i], t = rows_t[i], h = rows_h[i];
        if (b < 0 || b >= B || h < 0 || h >= Hq || t < 0 || t >= draft_lens[b]) return REF_ERR_ARG;
    }
    int fail = 0;
    #pragma omp parallel reduction(|:fail)
    {
    double* z = (double*)malloc(sizeof(double) * (size_t)(maxn + 1));
    if (!z) fail = 1;
    #pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < n_rows; ++i) {
        int b = rows_b[i], t = rows_t[i], h = rows_h[i];
        if (!z) continue;
        size_t row = (((size_t)b * T_max + t) * Hq + h) * D;
        attend_row(q + row, k_pool, v_pool, k_scale, v_scale,
                   block_table + (size_t)b * max_pages_per_seq,
                   context_lens[b], draft_lens[b], t, h / group, Hkv, D, P, sm_scale,
                   0, context_lens[b], NULL, 0, z, out_rows + (size_t)i * D);
    }
    free(z);
    }
    return fail ? REF_ERR_ARG : REF_OK;
}

/*
 * splash_ref_verify_attn_split: the same attention evaluated through explicit
 * context splits [s*L*P, (s+1)*L*P) of L = pages_per_split pages each,
 * giving per split the normalised partial row o_s and its natural-log
 * log-sum-exp lse_s (-inf and a zero row for a split with no visible key).
 * part_o is fp64 [B][Hq][T_max][S][D], part_lse fp64 [B][Hq][T_max][S].
 */
int splash_ref_verify_attn_split(const uint16_t* q,
                                 const int8_t* k_pool, const int8_t* v_pool,
                                 const uint16_t* k_scale, const uint16_t* v_scale,
                                 const int32_t* block_table, int max_pages_per_seq,
                                 const int32_t* context_lens, const int32_t* draft_lens,
                                 int B, int T_max, int Hq, int Hkv, int D, int P, int num_pages,
                                 double sm_scale, int num_splits, int pages_per_split,
                                 double* part_o, double* part_lse)
{
    int rc = check_attn_args(q, part_o, k_pool, v_pool, k_scale, v_scale, block_table,
                             context_lens, draft_lens, B, T_max, Hq, Hkv, D, P, num_pages,
                             max_pages_per_seq);
    if (rc) return rc;
    if (num_splits <= 0 || pages_per_split <= 0 || !part_lse) return REF_ERR_ARG;
    int S = num_splits;
    int L = pages_per_split;
    int group = Hq / Hkv;
    int maxn = 0;
    for (int b = 0; b < B; ++b) if (context_lens[b] > maxn) maxn = context_lens[b];
    long nunits = (long)B * Hq * T_max * S;
    int fail = 0;
    #pragma omp parallel reduction(|:fail)
    {
    double* z = (double*)malloc(sizeof(double) * (size_t)(maxn + 1));
    if (!z) fail = 1;
    #pragma omp for schedule(dynamic, 1)
    for (long u = 0; u < nunits; ++u) {
        int s = (int)(u % S);
        int t = (int)((u / S) % T_max);
        int h = (int)((u / ((long)S * T_max)) % Hq);
        int b = (int)(u / ((long)S * T_max * Hq));
        if (!z || t >= draft_lens[b]) continue;
        size_t qrow = (((size_t)b * T_max + t) * Hq + h) * D;
        size_t prow = (((size_t)b * Hq + h) * T_max + t) * S + s;
        long lo = (long)s * L * P, hi = (long)(s + 1) * L * P;
        if (lo > context_lens[b]) lo = context_lens[b];
        if (hi > context_lens[b]) hi = context_lens[b];
        part_lse[prow] = attend_row(q + qrow, k_pool, v_pool, k_scale, v_scale,
                                    block_table + (size_t)b * max_pages_per_seq,
                                    context_lens[b], draft_lens[b], t, h / group, Hkv, D, P,
                                    sm_scale, (int)lo, (int)hi, NULL, 0, z, part_o + prow * D);
    }
    free(z);
    }
    return fail ? REF_ERR_ARG : REF_OK;
}

/*
 * splash_ref_splitk_merge: combine S normalised partial rows with their
 * natural-log log-sum-exps: out = sum_s e^(lse_s - M) o_s / sum_s e^(lse_s - M),
 * M = max_s lse_s, splits with lse = -inf weigh nothing.  Inputs are fp32 as
 * the library's workspace holds them ([B][Hq][T_max][S][D] and
 * [B][Hq][T_max][S]); arithmetic and out ([B][T_max][Hq][D]) are fp64.
 * Rows t >= draft_lens[b] are left untouched.
 */
/* Threads the OpenMP loops of this library use (1 when built without OpenMP). */
int splash_ref_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int splash_ref_splitk_merge(const float* part_o, const float* part_lse, double* out,
                            const int32_t* draft_lens, int B, int T_max, int Hq, int D,
                            int num_splits)
{
    if (!part_o || !part_lse || !out || !draft_lens || B < 0 || T_max < 0 || Hq <= 0 ||
        D <= 0 || num_splits <= 0) return REF_ERR_ARG;
    int S = num_splits;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h)
            for (int t = 0; t < draft_lens[b] && t < T_max; ++t) {
                size_t prow = (((size_t)b * Hq + h) * T_max + t) * S;
                double M = -INFINITY;
                for (int s = 0; s < S; ++s)
                    if ((double)part_lse[prow + s] > M) M = (double)part_lse[prow + s];
                double* o = out + (((size_t)b * T_max + t) * Hq + h) * D;
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                double wsum = 0.0;
                for (int s = 0; s < S; ++s) {
                    double l = (double)part_lse[prow + s];
                    if (l == -INFINITY) continue;
                    double w = exp(l - M);
                    wsum += w;
                    for (int d = 0; d < D; ++d) o[d] += w * (double)part_o[(prow + s) * D + d];
                }
                for (int d = 0; d < D; ++d) o[d] /= wsum;
            }
    return REF_OK;
}

/* ------------------------------------------------------------------------
 * Acceptance of a verified draft block (discuss.pytorch.kr summary, section
 * "DFlash 2 speculative decoding as the default path": the draft model
 * proposes a block, the target checks the whole block in one forward pass, the
 * final output is identical to autoregressive decoding, and drafting,
 * verification, acceptance and the state update run as one unit).
 *
 * Written as that definition: the target's greedy choice after block position
 * t is y_t = argmax_v logits[b][t][v] (the largest value, compared as the exact
 * value of the bf16 number; among equal values the lowest token id).  Greedy
 * autoregressive decoding emits y_0 first; it keeps emitting the drafts for as
 * long as each draft equals the token greedy decoding would have chosen at its
 * position, and the first disagreement (or the end of the block) ends the
 * step with the target's own choice at that position.  So
 *   accepted   = 1 + number of leading i with block[i + 1] == y_i (i < d - 1)
 *   next_token = y_{accepted - 1}
 *   context_lens[b] -= d - accepted   (the rejected drafts leave the cache)
 * d = draft_lens[b] = 0 is a no-op: accepted = 0, next_token = -1.
 * logits: bf16 bits [B][T_max][V]; rows t >= d are not read.
 * ------------------------------------------------------------------------ */
static int ref_argmax_bf16(const uint16_t* row, int V)
{
    int best = 0;
    float bv = bf16_to_f32(row[0]);
    for (int v = 1; v < V; ++v) {
        float x = bf16_to_f32(row[v]);
        if (x > bv) { bv = x; best = v; }          /* strictly larger: ties keep the lowest id */
    }
    return best;
}

int splash_ref_verify_accept(const uint16_t* logits, const int32_t* block_tokens,
                             const int32_t* draft_lens, int32_t* context_lens,
                             int32_t* accepted, int32_t* next_token,
                             int B, int T_max, int V)
{
    if (!logits || !block_tokens || !draft_lens || !context_lens || !accepted || !next_token ||
        B < 0 || T_max < 0 || V <= 0) return REF_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        int d = draft_lens[b];
        if (d < 0 || d > T_max) return REF_ERR_ARG;
        if (d == 0) { accepted[b] = 0; next_token[b] = -1; continue; }
        const int32_t* blk = block_tokens + (size_t)b * T_max;
        int a = 1;
        int y = ref_argmax_bf16(logits + ((size_t)b * T_max + 0) * V, V);
        while (a < d && blk[a] == y) {             /* draft a matches the greedy token: keep it */
            y = ref_argmax_bf16(logits + ((size_t)b * T_max + a) * V, V);
            ++a;
        }
        accepted[b] = a;
        next_token[b] = y;
        context_lens[b] -= d - a;
    }
    return REF_OK;
}
