// launch.h -- internal launchers behind the C ABI (argument checks are done
// by the callers in api.hip; these only size grids and enqueue kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

hipError_t launch_kv_write(const uint16_t *kv, int64_t n, int64_t row_stride,
                           const int64_t *slot_mapping, uint8_t *pool,
                           int64_t num_slots, int layout, int32_t *err_count,
                           hipStream_t stream);

int quantize_q_blocks(int64_t n_elems);
hipError_t launch_quantize_q(const uint16_t *q, int64_t n_elems, uint8_t *q8,
                             float *q_scale, bool scale_given, float *partials,
                             hipStream_t stream);

struct AttnArgs {
    const void *q;              // [T, H, 512] bf16 or e4m3 codes
    const float *q_scale;       // device scalar (fp8 query) or null
    int T, H;
    const uint8_t *pool;
    int64_t num_slots;
    const int32_t *topk;        // [T, K]
    int K;
    const int32_t *page_table;  // [num_seqs, max_pages] or null
    int page_shift;             // log2(page_size)
    int max_pages, num_seqs;
    const int32_t *token_seq;   // [T] or null
    const int32_t *seq_lens;    // [num_seqs] or null
    float softmax_scale;
    void *out;                  // [T, H, 512] bf16 or fp32
    float *lse;                 // [T, H] or null
    float *ws;                  // split partials (decode)
    int n_splits;               // splits of the top-k list per (token, head block)
    int split_len;              // entries per split, a multiple of 64
    int32_t *err_count;
    int grid_cap = 0;           // 32-head blocks: at most this many workgroups,
                                // each taking several units (0 = one unit each)
};

// Number of top-k splits for this shape and phase (1 = none) on a device
// with `cus` compute units.
int attn_decode_splits(int T, int H, int K, int layout, int cus);
int attn_splits(int T, int H, int K, int phase, int layout, int cus);
size_t attn_workspace_bytes(int T, int H, int K, int phase, int cus);

hipError_t launch_attn(const AttnArgs &a, int layout, bool q_fp8, bool out_bf16,
                       hipStream_t stream);

struct TransformArgs {
    const int32_t *topk;        // [T, k_in]
    int T, k_in, k_out;
    const int32_t *page_table;  // [num_seqs, max_pages] or null
    int page_shift;             // log2(page_size)
    int max_pages, num_seqs;
    const int32_t *token_seq;   // [T] or null
    const int32_t *seq_lens;    // [num_seqs] or null
    int64_t num_slots;
    int32_t *out;               // [T, k_out]
    int32_t *counts;            // [T] or null
    int32_t *err_count;         // or null
};

hipError_t launch_topk_transform(const TransformArgs &a, hipStream_t stream);

}  // namespace dsa
