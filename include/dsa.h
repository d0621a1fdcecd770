/*
 * dsa.h -- C ABI of a gfx950 (MI355X) library for DeepSeek-style sparse
 * attention (DSA) in absorbed-MLA form over a paged FP8 KV pool.
 *
 * Sources (pages of the SGLang project this library follows):
 *   [RAW]    "extend CUDA TileLang raw FP8 KV path" (sglang PR #44012)
 *   [SCALED] "[DSA] Support group-scaled FP8 NoPE KV reads for CUDA TileLang"
 *            (sglang PR #39349)
 *   [Q8]     "[DSA] Support flashmla_sparse_q8 prefill backend on CUDA"
 *            (sglang PR #44217)
 *
 * What is computed.  Each query token t has H heads; each head is a 512-wide
 * latent query (absorbed MLA, no RoPE part: kv_lora_rank 512,
 * qk_rope_head_dim 0 [Q8, Modifications]).  The token attends only to the
 * pool rows its top-k list names [Q8, Modifications: physical KV-pool indices,
 * -1 padding to a multiple of 128].  Each pool row is one 512-wide latent that
 * serves as both key and value.  For the multiset J of valid entries:
 *     s_j = softmax_scale * q_scale * <q[t,h,:], x_j>
 *     out[t,h,:] = sum_j exp(s_j - m) x_j / sum_j exp(s_j - m)
 *     lse[t,h]   = m + log(sum_j exp(s_j - m))            (natural log)
 * With 656-byte RoPE rows the query is 512 + 64 wide and the score adds the
 * RoPE part: s_j += softmax_scale * <q[t,h,512:576], r_j> over the row's 64
 * RoPE values r_j; the value (and out) stays the 512-wide latent.
 * A duplicated entry counts once per occurrence (no de-duplication [SCALED,
 * Modifications]).  A token with no valid entry gets out = 0 exactly and
 * lse = -inf (the pages leave this contract open [SCALED, Accuracy Tests]).
 *
 * Row formats (bytes of one pool slot):
 *   DSA_KV_RAW_FP8_512     512 OCP E4M3FN codes, no scale [RAW, Modifications;
 *                          Speed Tests: 512 B against 1024 B for BF16].
 *   DSA_KV_SCALED_FP8_528  512 E4M3FN codes, then four little-endian fp32
 *                          scales; scale g multiplies elements [128g,128g+128)
 *                          [SCALED, Motivation].
 *   DSA_KV_SCALED_FP8_656  the RoPE variant the readers keep [SCALED,
 *                          Motivation]; the pages give only its size.  Read
 *                          here as the 528-byte row followed by 64
 *                          little-endian bf16 RoPE values (bytes 528..655).
 *   DSA_KV_BF16_1024       the 512 latent values as little-endian bf16, no
 *                          cast: the pool the FP8 rows halve [RAW, Speed
 *                          Tests: 512 B against 1024 B].  bf16 queries only.
 * E4M3FNUZ is rejected before any launch [RAW, Modifications].
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless stated otherwise.  The caller owns
 *     every buffer; the library allocates nothing and keeps no state beyond a
 *     once-per-device architecture and compute-unit query.
 *   - All argument checks run on the host before any launch and return a
 *     status; nothing is launched unless the status is DSA_OK (the pages
 *     reject unsupported formats and widths "before kernel dispatch" [RAW,
 *     Modifications]).  The only device query is the once-per-device
 *     architecture and compute-unit lookup.  Values stored
 *     in device memory (indices, slots, sequence ids) are data: invalid ones
 *     are masked on the device and counted into *err_count (optional int32
 *     device counter that is only ever incremented; the caller zeroes it).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     the call returns without waiting for it.  Calls never synchronise the
 *     host with the device, never allocate, and take their scales through
 *     device pointers, so they can be captured in a HIP graph and replayed
 *     with changed indices, queries and scales [SCALED, Accuracy Tests].
 *   - A writer followed by attention on the same stream sees the rows just
 *     written (live-tail entries [Q8, Modifications]).
 *   - `out` must not overlap q, the pool or the workspace.
 *   - DSA_ERR_DEVICE is returned when the current device is not gfx950.
 */
#ifndef DSA_MI355X_H
#define DSA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_kv_layout {
    DSA_KV_RAW_FP8_512 = 0,
    DSA_KV_SCALED_FP8_528 = 1,
    DSA_KV_SCALED_FP8_656 = 2,
    DSA_KV_BF16_1024 = 3
} dsa_kv_layout;

typedef enum dsa_dtype {
    DSA_BF16 = 0,
    DSA_FP32 = 1,
    DSA_FP8_E4M3FN = 2,
    DSA_FP8_E4M3FNUZ = 3
} dsa_dtype;

/* Status codes.  Each rejection is returned before anything is launched:
 * the pages require unsupported FP8 flavours (E4M3FNUZ), latent widths other
 * than the rows' and unknown layouts to be refused before kernel dispatch
 * [RAW, Modifications], and the geometry to be checked as required integers
 * against the layout [Q8, review thread]. */
typedef enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_NULL = 1,           /* a required pointer is NULL                 */
    DSA_ERR_SHAPE = 2,          /* a size is negative, zero where it may not  */
                                /* be, too large, or not a multiple of 128    */
    DSA_ERR_WIDTH_MISMATCH = 3, /* latent width is not the 512 of the rows    */
    DSA_ERR_LAYOUT = 4,         /* unknown or unsupported row layout / RoPE   */
    DSA_ERR_DTYPE = 5,          /* unsupported element type (incl. FNUZ)      */
    DSA_ERR_ALIGN = 6,          /* pointer or stride not 16-byte aligned (or
                                   an attention pool reaching 2^55)           */
    DSA_ERR_WORKSPACE = 7,      /* workspace missing or too small             */
    DSA_ERR_DEVICE = 8,         /* current device is not gfx950               */
    DSA_ERR_LAUNCH = 9          /* the HIP runtime refused a launch           */
} dsa_status;

/* Bytes of one pool row for `layout`: 512, 528, 656 or 1024; -1 for unknown
 * values.  [RAW, Accuracy Tests: exported buffer lengths are part of the
 * tested surface.] */
int32_t dsa_kv_row_bytes(int32_t layout);

/* Static, NUL-terminated name of a status code ("DSA_OK", ...;
 * "DSA_ERR_UNKNOWN" for a value outside the enum): the message of the
 * before-dispatch rejections [RAW, Modifications]. */
const char *dsa_status_string(int32_t status);

/*
 * dsa_kv_write -- fused cast-to-FP8 paged KV writer [RAW, Modifications: one
 * kernel casts and scatters, chosen by raw or scaled layout, and accepts
 * NoPE-only input with no RoPE tensor; SCALED, Motivation: the writer produces
 * the 528-byte rows].
 *
 *   kv            [n, kv_row_stride] elements of kv_dtype (DSA_BF16 only);
 *                 the first 512 of each row are written (656-byte layout:
 *                 the first 576, the latent then the RoPE values).  16-byte
 *                 aligned, kv_row_stride * 2 a multiple of 16.
 *   kv_dim        latent width of kv; must be 512 (DSA_ERR_WIDTH_MISMATCH).
 *   rope_dim      64 for DSA_KV_SCALED_FP8_656, else 0 (DSA_ERR_LAYOUT).
 *   fp8_format    DSA_FP8_E4M3FN for every layout (DSA_KV_BF16_1024 stores
 *                 no FP8 but the argument is checked the same way).
 *   slot_mapping  [n] int64 physical slot of each row; a negative slot skips
 *                 the row; a slot >= num_slots skips it and is counted.
 *   pool          [num_slots, dsa_kv_row_bytes(layout)] bytes, 16-byte
 *                 aligned.  Only the named slots are written.
 *   fp8_format    DSA_FP8_E4M3FN (FNUZ and others: DSA_ERR_DTYPE).
 * Encoding: round to nearest even, saturating to +-448, NaN kept as NaN.
 * Scaled rows: per 128-group s = fp32(amax / 448) (1 when amax = 0), codes
 * E4M3(fp32(x / s)), scales stored after the codes; 656-byte rows then take
 * the 64 RoPE values as bf16, unchanged.  DSA_KV_BF16_1024 rows are the
 * input's 512 bf16 values, unchanged.  n == 0 is a no-op.
 */
int32_t dsa_kv_write(const void *kv, int64_t n, int64_t kv_row_stride,
                     int32_t kv_dtype, int32_t kv_dim, int32_t rope_dim,
                     const int64_t *slot_mapping, void *pool,
                     int64_t num_slots, int32_t layout, int32_t fp8_format,
                     int32_t *err_count, void *stream);

/*
 * dsa_quantize_q_fp8 -- cast the query to E4M3FN with one per-tensor scale
 * (the NoPE case of the query concat-and-cast step: with a zero-width RoPE
 * part there is nothing to concatenate [Q8, review thread]).
 *
 *   q         n_elems values of q_dtype (DSA_BF16), 16-byte aligned.
 *   q8        n_elems output codes, 16-byte aligned.
 *   q_scale   one fp32 in device memory.  scale_given == 0: written with
 *             fp32(amax|q| / 448) (1 when amax = 0).  scale_given != 0: read.
 *   workspace dsa_quantize_q_workspace_bytes(n_elems) bytes (partial maxima);
 *             NULL allowed when that is 0 or scale_given != 0.  The caller
 *             provides this bounded scratch, so the call neither allocates
 *             nor synchronises [SCALED, Modifications: bounded workspace, no
 *             host sync].
 * Codes are E4M3(fp32(q / q_scale)), round to nearest even, saturating.
 * n_elems must be a multiple of 8.  n_elems == 0 is a no-op.
 */
int32_t dsa_quantize_q_fp8(const void *q, int64_t n_elems, int32_t q_dtype,
                           void *q8, float *q_scale, int32_t scale_given,
                           int32_t fp8_format, void *workspace,
                           size_t workspace_bytes, void *stream);
/* Bytes of the quantize workspace for n_elems values: 4 per block of the
 * amax pass (a pure function of n_elems; 0 for n_elems <= 0) [SCALED,
 * Modifications: a bounded workspace sized from the shape]. */
size_t dsa_quantize_q_workspace_bytes(int64_t n_elems);

/*
 * dsa_sparse_attn_decode / dsa_sparse_attn_prefill -- the attention itself.
 * Both compute exactly the function stated at the top of this file over the
 * same arguments; they differ only in how work is spread over the GPU:
 * decode splits each token's top-k list over several workgroups and merges
 * the partial softmax states in a second kernel (few tokens, each reading a
 * lot); prefill gives each (token, head block) one workgroup (many tokens).
 * The FP8-query path reads q as E4M3FN codes times *q_scale [Q8, Motivation
 * and Modifications: FP8 query against FP8 KV].
 *
 *   q           [T, H, D + rope_dim] contiguous, q_dtype DSA_BF16 or
 *               DSA_FP8_E4M3FN (656-byte rows: DSA_BF16 only, else
 *               DSA_ERR_DTYPE -- the FP8 query path is NoPE-only [Q8,
 *               Modifications]; bf16 rows: DSA_BF16 only); 16-byte aligned.
 *   q_scale     one fp32 (device) for an FP8 query, else ignored (may be NULL).
 *   D           must be 512 (DSA_ERR_WIDTH_MISMATCH); rope_dim must be 64
 *               for DSA_KV_SCALED_FP8_656 and 0 otherwise (DSA_ERR_LAYOUT).
 *               1 <= H <= 128.  T == 0 is a no-op.
 *   pool        [num_slots, row bytes of `layout`], 16-byte aligned, below
 *               address 2^55 (DSA_ERR_ALIGN otherwise; device allocations are).
 *   topk        [T, K] int32; K a positive multiple of 128, at most 65536.
 *               Entry i: -1 is padding; other values are positions resolved
 *               through page_table (or pool slots when page_table is NULL).
 *   page_table  [num_seqs, max_pages] int32 physical page numbers or NULL.
 *               slot = page_table[seq][i / page_size] * page_size
 *                      + i % page_size, page_size a power of two.
 *   token_seq   [T] int32 sequence of each token, or NULL for token t ->
 *               sequence t (then T <= num_seqs is required when page_table or
 *               seq_lens is given).
 *   seq_lens    [num_seqs] int32 or NULL; entries i >= seq_lens[seq] are
 *               masked.
 *   Masked and counted into *err_count: i < -1, i >= seq_lens[seq],
 *   i / page_size >= max_pages, a negative page-table entry, a resolved slot
 *   >= num_slots, a token whose sequence id is outside [0, num_seqs).
 *   softmax_scale  fp32 factor on the dot product (e.g. 1/sqrt(512)).
 *   out         [T, H, 512] of out_dtype (DSA_BF16 or DSA_FP32), fully
 *               overwritten; 16-byte aligned.
 *   lse         [T, H] fp32 natural-log sum-exp, or NULL.
 *   workspace   dsa_attn_workspace_bytes(T, H, K, phase) bytes, 256-byte
 *               aligned (phase 0 = decode, 1 = prefill); may be NULL when
 *               that size is 0.
 */
int32_t dsa_sparse_attn_decode(
    const void *q, int32_t q_dtype, const float *q_scale, int32_t T, int32_t H,
    int32_t D, int32_t rope_dim, const void *pool, int64_t num_slots,
    int32_t layout, int32_t fp8_format, const int32_t *topk, int32_t K,
    const int32_t *page_table, int32_t page_size, int32_t max_pages,
    int32_t num_seqs, const int32_t *token_seq, const int32_t *seq_lens,
    float softmax_scale, void *out, int32_t out_dtype, float *lse,
    void *workspace, size_t workspace_bytes, int32_t *err_count, void *stream);

/*
 * dsa_sparse_attn_decode_noalloc -- dsa_sparse_attn_decode for callers that
 * cannot allocate device memory (work captured in a graph that must not
 * allocate, serving loops held to a fixed memory footprint, harnesses that
 * forbid allocation): the same computation, kernels and arguments, without
 * the workspace.  The split partials go to a scratch array the library owns
 * on each GPU it runs on: DSA_DECODE_SCRATCH_BYTES (32 MiB) per GPU,
 * resident from the first call on that GPU until the process ends.  A call
 * whose dsa_attn_workspace_bytes(T, H, K, 0) exceeds that returns
 * DSA_ERR_WORKSPACE before anything is launched (every top-k width up to
 * 2048 fits on a 256-CU MI355X).  The call allocates nothing.  Every call on
 * one GPU shares that GPU's scratch, which keeps the last call's contents
 * (each split overwrites all of its state, so nothing needs clearing): calls
 * that overlap on one GPU, on different streams, race.  Other arguments and
 * errors as for dsa_sparse_attn_decode.
 */
#define DSA_DECODE_SCRATCH_BYTES (32u << 20)
int32_t dsa_sparse_attn_decode_noalloc(
    const void *q, int32_t q_dtype, const float *q_scale, int32_t T, int32_t H,
    int32_t D, int32_t rope_dim, const void *pool, int64_t num_slots,
    int32_t layout, int32_t fp8_format, const int32_t *topk, int32_t K,
    const int32_t *page_table, int32_t page_size, int32_t max_pages,
    int32_t num_seqs, const int32_t *token_seq, const int32_t *seq_lens,
    float softmax_scale, void *out, int32_t out_dtype, float *lse,
    int32_t *err_count, void *stream);

int32_t dsa_sparse_attn_prefill(
    const void *q, int32_t q_dtype, const float *q_scale, int32_t T, int32_t H,
    int32_t D, int32_t rope_dim, const void *pool, int64_t num_slots,
    int32_t layout, int32_t fp8_format, const int32_t *topk, int32_t K,
    const int32_t *page_table, int32_t page_size, int32_t max_pages,
    int32_t num_seqs, const int32_t *token_seq, const int32_t *seq_lens,
    float softmax_scale, void *out, int32_t out_dtype, float *lse,
    void *workspace, size_t workspace_bytes, int32_t *err_count, void *stream);

/* Workspace bytes the attention call needs for this shape and phase
 * (0 = decode, 1 = prefill): the fp32 split partials of the decode, whose
 * split count fills the current device's compute units (256 are assumed when
 * no device can be queried); 0 when the call needs none.  The caller owns
 * this bounded scratch, so the attention neither allocates nor synchronises
 * [SCALED, Modifications: selected rows go through a bounded workspace, with
 * no host sync]. */
size_t dsa_attn_workspace_bytes(int32_t T, int32_t H, int32_t K, int32_t phase);

/*
 * dsa_topk_transform -- the index transform ahead of the attention: top-k
 * positions of any width resolved to physical pool slots and compacted
 * ["[DSA] Support group-scaled FP8 NoPE KV reads for CUDA TileLang", the
 * draft notes: the page-table transform over non-2048 top-k widths; Q8,
 * review thread: prefix requests read only the referenced context slots
 * through the flattened page table (the RAGGED path)].
 *
 * Every entry of row t is resolved with exactly the attention's rule (see
 * dsa_sparse_attn_decode: -1 is padding; the same invalid values are masked
 * and counted into *err_count).  Row t of out_slots then holds the valid
 * slots in their input order, followed by -1 up to k_out, and valid_count[t]
 * their number.  out_slots is what the attention takes with page_table ==
 * NULL (its width k_out already a multiple of 128), and the attention skips
 * the tiles after a row's last valid entry.
 *
 *   topk        [T, k_in] int32, 1 <= k_in <= 65536 (any width).
 *   page_table, page_size, max_pages, num_seqs, token_seq, seq_lens,
 *   num_slots   as for the attention.
 *   out_slots   [T, k_out] int32, fully overwritten; k_out a multiple of 128
 *               with k_in <= k_out <= 65536; must not overlap topk.
 *   valid_count [T] int32 or NULL.
 *   err_count   one int32 (device) that masked entries are added to, or NULL.
 *   T == 0 is a no-op.  Asynchronous on `stream` (NULL = the default stream);
 *   argument errors are returned before anything is launched.
 */
int32_t dsa_topk_transform(const int32_t *topk, int32_t T, int32_t k_in,
                           const int32_t *page_table, int32_t page_size,
                           int32_t max_pages, int32_t num_seqs,
                           const int32_t *token_seq, const int32_t *seq_lens,
                           int64_t num_slots, int32_t *out_slots, int32_t k_out,
                           int32_t *valid_count, int32_t *err_count, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_MI355X_H */
