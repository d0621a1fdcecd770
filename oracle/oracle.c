/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the DSA
 * sparse absorbed-MLA attention path over a paged FP8 KV pool.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header, table or constant with the
 * HIP kernels.
 *
 * Sources (the three SGLang pull-request pages this library follows):
 *   [RAW]    "extend CUDA TileLang raw FP8 KV path" (sglang PR #44012)
 *   [SCALED] "[DSA] Support group-scaled FP8 NoPE KV reads for CUDA TileLang"
 *            (sglang PR #39349)
 *   [Q8]     "[DSA] Support flashmla_sparse_q8 prefill backend on CUDA"
 *            (sglang PR #44217)
 * and, for the 8-bit float format, the OCP "OFP8 Formats for Deep Learning"
 * specification (E4M3 with no infinities, one NaN mantissa pattern).
 *
 * Precision: FP8 encoding and the writer's scale arithmetic are done in fp32
 * exactly as a device would do them (they produce bytes that must match bit
 * for bit); everything about attention is FP64 on exactly-dequantised values.
 *
 * Readings taken where the pages are silent are listed next to each function.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_D 512          /* latent width, kv_lora_rank = 512 [Q8, Modifications] */
#define ORC_GROUP 128      /* elements per scale group in the 528-byte row        */
#define ORC_RAW_BYTES 512  /* raw row: 512 unscaled FP8 values [RAW, Speed Tests]  */
#define ORC_SCALED_BYTES 528 /* 512 FP8 + 4 fp32 scales [SCALED, Motivation]      */
/* RoPE row [SCALED, Motivation: the existing helpers require a 656-byte    */
/* RoPE layout].  Reading (the pages give only the size): the 528-byte      */
/* scaled row followed by 64 bf16 RoPE values, little-endian; the query is  */
/* then 512 + 64 wide and the RoPE part adds q_rope . k_rope to the score.  */
#define ORC_ROPE 64
#define ORC_ROPE_BYTES 656
/* BF16 row: the 512 latent values as bf16, 1024 bytes [RAW, Speed Tests and */
/* Profiling: the BF16 pool the FP8 rows are compared against].              */
#define ORC_BF16_BYTES 1024

/* ------------------------------------------------------------------------ */
/* FP8 E4M3FN (OCP): sign | 4 exponent bits (bias 7) | 3 mantissa bits.      */
/* Exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity.     */
/* ------------------------------------------------------------------------ */

double orc_fp8_decode(uint8_t b)
{
    int s = b >> 7;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return s ? -NAN : NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round to nearest, ties to even mantissa; finite overflow and +-inf
 * saturate to +-448 (the largest finite E4M3FN value); NaN keeps its sign
 * as S.1111.111; -0 encodes as 0x80.  The pages do not state the encoder's
 * rounding or overflow rule; this is the plainest reading and the one the
 * rest of the library fixes. */
uint8_t orc_fp8_encode(float x)
{
    uint8_t s = signbit(x) ? 0x80 : 0x00;
    double a;
    int E, k;
    double f, mant;

    if (isnan(x))
        return s | 0x7F;
    a = fabs((double)x);
    if (a >= 448.0)
        return s | 0x7E;
    if (a < ldexp(1.0, -6)) {
        /* subnormal band: integer multiples of 2^-9; 8 * 2^-9 is the smallest
           normal, whose code is 0x08, so the integer is the code itself. */
        mant = nearbyint(a * 512.0);
        return s | (uint8_t)mant;
    }
    f = frexp(a, &E);          /* a = f * 2^E, f in [0.5, 1)   */
    k = E - 1;                 /* a = (2f) * 2^k, 2f in [1, 2) */
    mant = nearbyint((2.0 * f - 1.0) * 8.0);
    if (mant == 8.0) {
        mant = 0.0;
        k += 1;
    }
    return s | (uint8_t)(((k + 7) << 3) | (int)mant);
}

void orc_fp8_encode_array(const float *x, int64_t n, uint8_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_fp8_encode(x[i]);
}

void orc_fp8_decode_array(const uint8_t *b, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = orc_fp8_decode(b[i]);
}

static float bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Fused cast-to-FP8 paged KV writer [RAW, Modifications: one fused kernel  */
/* casts and scatters, chosen by raw or scaled layout; SCALED, Motivation].  */
/*                                                                          */
/* Row i of kv (bf16, 512 values, rows kv_row_stride elements apart) goes to */
/* pool slot slot_mapping[i].  A negative slot skips the row silently; a     */
/* slot >= num_slots skips it and counts one error.  Returns the number of   */
/* counted errors.                                                          */
/*   raw (layout 0):    byte[d] = E4M3(x[d]), no scale.                     */
/*   scaled (layout 1): group g = elements [128g, 128g+128);                */
/*       s_g = fp32(amax_g / 448) (1.0 if amax_g == 0),                    */
/*       byte[d] = E4M3(fp32(x[d] / s_g)), scales stored little-endian fp32 */
/*       at row bytes 512 + 4g.                                             */
/*   RoPE (layout 2): input rows of 512 + 64 values; the first 512 as the   */
/*       scaled layout, the 64 RoPE values copied as bf16 to bytes 528..655. */
/*   BF16 (layout 3): the 512 bf16 values copied unchanged (no cast).       */
/* ------------------------------------------------------------------------ */
int64_t orc_kv_write(const uint16_t *kv, int64_t n, int64_t kv_row_stride,
                     const int64_t *slot_mapping, uint8_t *pool,
                     int64_t num_slots, int layout)
{
    int64_t errors = 0;
    int64_t row_bytes = layout == 0 ? ORC_RAW_BYTES
                        : layout == 1 ? ORC_SCALED_BYTES
                        : layout == 2 ? ORC_ROPE_BYTES : ORC_BF16_BYTES;

    for (int64_t i = 0; i < n; i++) {
        int64_t slot = slot_mapping[i];
        const uint16_t *src = kv + i * kv_row_stride;
        uint8_t *dst;

        if (slot < 0)
            continue;
        if (slot >= num_slots) {
            errors++;
            continue;
        }
        dst = pool + slot * row_bytes;
        if (layout == 3) {
            for (int d = 0; d < ORC_D; d++) {
                dst[2 * d] = (uint8_t)(src[d] & 0xff);
                dst[2 * d + 1] = (uint8_t)(src[d] >> 8);
            }
        } else if (layout == 0) {
            for (int d = 0; d < ORC_D; d++)
                dst[d] = orc_fp8_encode(bf16_to_f32(src[d]));
        } else {
            for (int g = 0; g < ORC_D / ORC_GROUP; g++) {
                float amax = 0.0f, scale;
                for (int j = 0; j < ORC_GROUP; j++) {
                    float v = fabsf(bf16_to_f32(src[g * ORC_GROUP + j]));
                    if (v > amax)
                        amax = v;
                }
                scale = amax == 0.0f ? 1.0f : amax / 448.0f;
                for (int j = 0; j < ORC_GROUP; j++) {
                    float v = bf16_to_f32(src[g * ORC_GROUP + j]);
                    dst[g * ORC_GROUP + j] = orc_fp8_encode(v / scale);
                }
                memcpy(dst + ORC_D + 4 * g, &scale, 4);
            }
            if (layout == 2)
                for (int r = 0; r < ORC_ROPE; r++) {
                    dst[ORC_SCALED_BYTES + 2 * r] = (uint8_t)(src[ORC_D + r] & 0xff);
                    dst[ORC_SCALED_BYTES + 2 * r + 1] = (uint8_t)(src[ORC_D + r] >> 8);
                }
        }
    }
    return errors;
}

/* ------------------------------------------------------------------------ */
/* Query FP8 quantisation with one per-tensor scale [Q8, review thread:      */
/* concat_and_cast_q_fp8_pad handles a zero-width RoPE part, so with NoPE    */
/* the query is only cast].  The scale rule is not on the pages; reading:    */
/* q_scale = fp32(amax(|q|) / 448) (1.0 when amax == 0); q8 = E4M3(q/scale). */
/* ------------------------------------------------------------------------ */
float orc_q_scale(const uint16_t *q, int64_t n)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; i++) {
        float v = fabsf(bf16_to_f32(q[i]));
        if (v > amax)
            amax = v;
    }
    return amax == 0.0f ? 1.0f : amax / 448.0f;
}

void orc_q_quantize(const uint16_t *q, int64_t n, float scale, uint8_t *q8)
{
    for (int64_t i = 0; i < n; i++)
        q8[i] = orc_fp8_encode(bf16_to_f32(q[i]) / scale);
}

/* ------------------------------------------------------------------------ */
/* Index resolution [Q8, Modifications: top-k holds KV-pool indices padded   */
/* with -1 to a multiple of 128; SCALED, Modifications: invalid entries stay */
/* masked; Q8 review thread: page_table_1_flattened maps positions to slots].*/
/*                                                                          */
/* Entry value i of token t (sequence seq):                                 */
/*   i == -1                       -> masked (padding, not an error)        */
/*   i < -1                        -> masked, error                         */
/*   seq_lens given, i >= len      -> masked, error                         */
/*   page table given: page = i / P; page >= max_pages or table entry < 0   */
/*                                 -> masked, error;                        */
/*                     slot = table[seq][page] * P + i % P                   */
/*   no page table:    slot = i                                             */
/*   slot >= num_slots             -> masked, error                         */
/* Returns the slot, or -1 (masked); *err is incremented on errors.         */
/* ------------------------------------------------------------------------ */
static int64_t resolve_slot(int32_t i, int seq, const int32_t *page_table,
                            int page_size, int max_pages,
                            const int32_t *seq_lens, int64_t num_slots,
                            int64_t *err)
{
    int64_t slot;
    if (i == -1)
        return -1;
    if (i < 0) {
        (*err)++;
        return -1;
    }
    if (seq_lens && i >= seq_lens[seq]) {
        (*err)++;
        return -1;
    }
    if (page_table) {
        int page = i / page_size;
        int32_t phys;
        if (page >= max_pages) {
            (*err)++;
            return -1;
        }
        phys = page_table[(int64_t)seq * max_pages + page];
        if (phys < 0) {
            (*err)++;
            return -1;
        }
        slot = (int64_t)phys * page_size + (i % page_size);
    } else {
        slot = i;
    }
    if (slot >= num_slots) {
        (*err)++;
        return -1;
    }
    return slot;
}

int64_t orc_resolve(const int32_t *topk, int T, int K, const int32_t *token_seq,
                    const int32_t *page_table, int page_size, int max_pages,
                    const int32_t *seq_lens, int64_t num_slots, int64_t *slots)
{
    int64_t err = 0;
    for (int t = 0; t < T; t++) {
        int seq = token_seq ? token_seq[t] : t;
        for (int j = 0; j < K; j++)
            slots[(int64_t)t * K + j] =
                resolve_slot(topk[(int64_t)t * K + j], seq, page_table,
                             page_size, max_pages, seq_lens, num_slots, &err);
    }
    return err;
}

/* ------------------------------------------------------------------------ */
/* Index transform ahead of the attention [SCALED, the draft notes: the     */
/* variable-width page-table transform; Q8, review discussion: prefix       */
/* requests gather only the referenced context slots through the flattened  */
/* page-size-1 table, the RAGGED path].                                      */
/* Readings: every entry is resolved exactly as resolve_slot does for the   */
/* attention; the row's valid slots are written first, in their input      */
/* order, then -1 up to the output width k_out (>= k_in); counts[t] is the  */
/* number of valid slots of row t.  Returns the number of masked entries    */
/* other than -1 (the attention's error count for the same input).         */
/* ------------------------------------------------------------------------ */
int64_t orc_topk_transform(const int32_t *topk, int T, int k_in,
                           const int32_t *token_seq, const int32_t *page_table,
                           int page_size, int max_pages,
                           const int32_t *seq_lens, int64_t num_slots,
                           int k_out, int32_t *out, int32_t *counts)
{
    int64_t err = 0;
    for (int t = 0; t < T; t++) {
        int seq = token_seq ? token_seq[t] : t;
        int32_t *row = out + (int64_t)t * k_out;
        int n = 0;
        for (int j = 0; j < k_in; j++) {
            int64_t slot = resolve_slot(topk[(int64_t)t * k_in + j], seq,
                                        page_table, page_size, max_pages,
                                        seq_lens, num_slots, &err);
            if (slot >= 0)
                row[n++] = (int32_t)slot;
        }
        if (counts)
            counts[t] = n;
        for (int j = n; j < k_out; j++)
            row[j] = -1;
    }
    return err;
}

/* Exact dequantised row value in FP64 [RAW, Modifications: the raw layout  */
/* is unscaled; SCALED, Motivation: four fp32 scales, one per 128 values].   */
/* Reading: a scale multiplies its group's decoded values.  The RoPE part   */
/* of a 656-byte row (its bf16 values, exact in FP64) goes to xr.           */
static void rope_row(const uint8_t *row, double *xr)
{
    for (int r = 0; r < ORC_ROPE; r++)
        xr[r] = bf16_to_f32((uint16_t)(row[ORC_SCALED_BYTES + 2 * r] |
                                       (row[ORC_SCALED_BYTES + 2 * r + 1] << 8)));
}

static void dequant_row(const uint8_t *row, int layout, double *x)
{
    if (layout == 3) {
        for (int d = 0; d < ORC_D; d++)
            x[d] = bf16_to_f32((uint16_t)(row[2 * d] | (row[2 * d + 1] << 8)));
    } else if (layout == 0) {
        for (int d = 0; d < ORC_D; d++)
            x[d] = orc_fp8_decode(row[d]);
    } else {
        float scale[4];
        memcpy(scale, row + ORC_D, 16);
        for (int d = 0; d < ORC_D; d++)
            x[d] = orc_fp8_decode(row[d]) * (double)scale[d / ORC_GROUP];
    }
}

/* ------------------------------------------------------------------------ */
/* Sparse attention in absorbed-MLA form with no RoPE part                   */
/* [Q8, Modifications: NoPE, kv_lora_rank = 512; SCALED, Modifications: BF16 */
/* latent-512 / RoPE-0 queries].  The 512-wide latent row is both key and   */
/* value.  For token t, head h, over the multiset of valid entries j:       */
/*   s_j   = softmax_scale * sum_d qhat[h][d] * x_j[d]                      */
/*           (656-byte rows: + softmax_scale * sum_r qhat[h][512+r] * xr_j[r]) */
/*   o     = sum_j exp(s_j - M) x_j / sum_j exp(s_j - M),  M = max_j s_j   */
/*   lse   = M + log(sum_j exp(s_j - M))                                    */
/* Two passes (max, then weights): deliberately not an online softmax.     */
/* A duplicated entry is one more term: the scaled reader keeps duplicates */
/* and never de-duplicates [SCALED, Modifications].  No valid entry:        */
/* o = 0 exactly and lse = -inf (the pages leave the all-masked row open). */
/* qhat = bf16 value, or decode(q8) * q_scale for an FP8 query.            */
/* ------------------------------------------------------------------------ */
struct attn_job {
    const void *q;
    int q_is_fp8;
    float q_scale;
    int T, H;
    const uint8_t *pool;
    int64_t num_slots;
    int layout;
    const int32_t *topk;
    int K;
    const int32_t *page_table;
    int page_size, max_pages;
    const int32_t *token_seq, *seq_lens;
    float softmax_scale;
    double *out, *lse;
    int t_begin, t_end;
    int64_t err;
};

static void attn_tokens(struct attn_job *jb)
{
    int64_t row_bytes = jb->layout == 0 ? ORC_RAW_BYTES
                        : jb->layout == 1 ? ORC_SCALED_BYTES
                        : jb->layout == 2 ? ORC_ROPE_BYTES : ORC_BF16_BYTES;
    int rope = jb->layout == 2 ? ORC_ROPE : 0;   /* query row: ORC_D + rope */
    double *x = malloc(sizeof(double) * (size_t)jb->K * ORC_D);
    double *xr = malloc(sizeof(double) * (size_t)jb->K * ORC_ROPE);
    double *qh = malloc(sizeof(double) * (ORC_D + ORC_ROPE));
    double *s = malloc(sizeof(double) * (size_t)jb->K);

    for (int t = jb->t_begin; t < jb->t_end; t++) {
        int seq = jb->token_seq ? jb->token_seq[t] : t;
        int nv = 0;

        /* gather + dequantise every valid entry once, in index order */
        for (int j = 0; j < jb->K; j++) {
            int64_t sl = resolve_slot(jb->topk[(int64_t)t * jb->K + j], seq,
                                      jb->page_table, jb->page_size,
                                      jb->max_pages, jb->seq_lens,
                                      jb->num_slots, &jb->err);
            if (sl < 0)
                continue;
            dequant_row(jb->pool + sl * row_bytes, jb->layout,
                        x + (int64_t)nv * ORC_D);
            if (rope)
                rope_row(jb->pool + sl * row_bytes, xr + (int64_t)nv * ORC_ROPE);
            nv++;
        }

        for (int h = 0; h < jb->H; h++) {
            int64_t qoff = ((int64_t)t * jb->H + h) * (ORC_D + rope);
            double *o = jb->out + ((int64_t)t * jb->H + h) * ORC_D;
            double M = -INFINITY, L = 0.0;

            for (int d = 0; d < ORC_D + rope; d++) {
                if (jb->q_is_fp8)
                    qh[d] = orc_fp8_decode(((const uint8_t *)jb->q)[qoff + d]) *
                            (double)jb->q_scale;
                else
                    qh[d] = bf16_to_f32(((const uint16_t *)jb->q)[qoff + d]);
            }
            for (int j = 0; j < nv; j++) {
                double dot = 0.0;
                for (int d = 0; d < ORC_D; d++)
                    dot += qh[d] * x[(int64_t)j * ORC_D + d];
                for (int r = 0; r < rope; r++)
                    dot += qh[ORC_D + r] * xr[(int64_t)j * ORC_ROPE + r];
                s[j] = (double)jb->softmax_scale * dot;
                if (s[j] > M)
                    M = s[j];
            }
            for (int d = 0; d < ORC_D; d++)
                o[d] = 0.0;
            if (nv == 0) {
                if (jb->lse)
                    jb->lse[(int64_t)t * jb->H + h] = -INFINITY;
                continue;
            }
            for (int j = 0; j < nv; j++) {
                double w = exp(s[j] - M);
                L += w;
                for (int d = 0; d < ORC_D; d++)
                    o[d] += w * x[(int64_t)j * ORC_D + d];
            }
            for (int d = 0; d < ORC_D; d++)
                o[d] /= L;
            if (jb->lse)
                jb->lse[(int64_t)t * jb->H + h] = M + log(L);
        }
    }
    free(x);
    free(xr);
    free(qh);
    free(s);
}

static void *attn_thread(void *arg)
{
    attn_tokens((struct attn_job *)arg);
    return NULL;
}

/* out: [T][H][512] doubles, lse: [T][H] doubles or NULL.
 * Returns the number of invalid (non -1) index entries met. */
int64_t orc_sparse_attn(const void *q, int q_is_fp8, float q_scale, int T,
                        int H, const uint8_t *pool, int64_t num_slots,
                        int layout, const int32_t *topk, int K,
                        const int32_t *page_table, int page_size,
                        int max_pages, const int32_t *token_seq,
                        const int32_t *seq_lens, float softmax_scale,
                        double *out, double *lse, int nthreads)
{
    struct attn_job *jobs;
    pthread_t *tid;
    int64_t err = 0;

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > T)
        nthreads = T > 0 ? T : 1;
    jobs = calloc((size_t)nthreads, sizeof(*jobs));
    tid = calloc((size_t)nthreads, sizeof(*tid));
    for (int i = 0; i < nthreads; i++) {
        struct attn_job *jb = &jobs[i];
        jb->q = q;
        jb->q_is_fp8 = q_is_fp8;
        jb->q_scale = q_scale;
        jb->T = T;
        jb->H = H;
        jb->pool = pool;
        jb->num_slots = num_slots;
        jb->layout = layout;
        jb->topk = topk;
        jb->K = K;
        jb->page_table = page_table;
        jb->page_size = page_size;
        jb->max_pages = max_pages;
        jb->token_seq = token_seq;
        jb->seq_lens = seq_lens;
        jb->softmax_scale = softmax_scale;
        jb->out = out;
        jb->lse = lse;
        jb->t_begin = (int)((int64_t)T * i / nthreads);
        jb->t_end = (int)((int64_t)T * (i + 1) / nthreads);
    }
    for (int i = 1; i < nthreads; i++)
        pthread_create(&tid[i], NULL, attn_thread, &jobs[i]);
    attn_tokens(&jobs[0]);
    for (int i = 1; i < nthreads; i++)
        pthread_join(tid[i], NULL);
    for (int i = 0; i < nthreads; i++)
        err += jobs[i].err;
    free(jobs);
    free(tid);
    return err;
}
