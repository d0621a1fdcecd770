// api.hip -- the C ABI declared in include/dsa.h: argument validation (all of
// it on the host, before any launch), the once-per-device architecture and
// compute-unit query, and dispatch to the launchers.
//
// Rejections follow the SGLang pages: a latent width other than the rows'
// 512 and E4M3FNUZ are refused before any kernel is dispatched ("extend CUDA
// TileLang raw FP8 KV path", Modifications); the geometry is passed as
// required integers and checked against the row layout, not inferred from a
// model name ("[DSA] Support flashmla_sparse_q8 prefill backend on CUDA",
// review thread): the RoPE width must be the layout's own (64 for the
// 656-byte rows, 0 for every other layout).
#include <atomic>
#include <cstring>

#include "../../include/dsa.h"
#include "launch.h"

namespace {

constexpr int kMaxDevices = 64;
constexpr int kDefaultCus = 256;             // MI355X: 8 XCDs x 32 compute units
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_cus[kMaxDevices];         // compute units (set with the state)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Architecture and compute-unit count of device `dev`, queried once.
int device_state(int dev) {
    int st = g_arch_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
        g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : kDefaultCus,
                         std::memory_order_relaxed);
        st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_arch_state[dev].store(st, std::memory_order_release);
    }
    return st;
}

int32_t check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return DSA_ERR_DEVICE;
    return device_state(dev) == 1 ? DSA_OK : DSA_ERR_DEVICE;
}

// Compute units the decode split count is sized for: those of the current
// device, or 256 (an MI355X) when no device can be queried, so that the
// workspace size is defined on a host without a GPU as well.
int split_target_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return kDefaultCus;
    if (device_state(dev) == 0) return kDefaultCus;
    return g_cus[dev].load(std::memory_order_relaxed);
}

// Scratch of the allocation-free decode entry point: the split partials of
// one call in a device array the library owns (one copy on every GPU the
// library runs on, resident until the process ends).  Host code never uses
// the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[DSA_DECODE_SCRATCH_BYTES];
std::atomic<void *> g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (NULL on failure).
void *scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    return p;
}

int32_t check_fp8_format(int32_t f) {
    return f == DSA_FP8_E4M3FN ? DSA_OK : DSA_ERR_DTYPE;
}

int32_t check_layout(int32_t layout) {
    return (layout == DSA_KV_RAW_FP8_512 || layout == DSA_KV_SCALED_FP8_528 ||
            layout == DSA_KV_SCALED_FP8_656 || layout == DSA_KV_BF16_1024)
               ? DSA_OK
               : DSA_ERR_LAYOUT;
}

// The RoPE width a layout carries: 64 for the 656-byte rows, else 0.
int32_t rope_of(int32_t layout) { return layout == DSA_KV_SCALED_FP8_656 ? 64 : 0; }

// Shared validation of the two attention entry points.
int32_t validate_attn(const void *q, int32_t q_dtype, const float *q_scale,
                      int32_t T, int32_t H, int32_t D, int32_t rope_dim,
                      const void *pool, int64_t num_slots, int32_t layout,
                      int32_t fp8_format, const int32_t *topk, int32_t K,
                      const int32_t *page_table, int32_t page_size,
                      int32_t max_pages, int32_t num_seqs,
                      const int32_t *token_seq, const int32_t *seq_lens,
                      void *out, int32_t out_dtype, void *workspace,
                      size_t workspace_bytes, int32_t phase) {
    if (D != 512) return DSA_ERR_WIDTH_MISMATCH;
    int32_t st = check_layout(layout);
    if (st) return st;
    if (rope_dim != rope_of(layout)) return DSA_ERR_LAYOUT;
    if ((st = check_fp8_format(fp8_format))) return st;
    if (q_dtype != DSA_BF16 && q_dtype != DSA_FP8_E4M3FN) return DSA_ERR_DTYPE;
    // the FP8 query path is NoPE-only [Q8, Modifications], and FP8 codes
    // meet FP8 rows only
    if ((rope_dim != 0 || layout == DSA_KV_BF16_1024) && q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (out_dtype != DSA_BF16 && out_dtype != DSA_FP32) return DSA_ERR_DTYPE;
    if (T < 0 || H < 1 || H > 128) return DSA_ERR_SHAPE;
    if (K <= 0 || K % 128 != 0 || K > 65536) return DSA_ERR_SHAPE;
    if (num_slots < 0 || num_slots >= ((int64_t)1 << 31)) return DSA_ERR_SHAPE;
    if (page_table) {
        if (page_size < 1 || (page_size & (page_size - 1)) != 0 || page_size > (1 << 20))
            return DSA_ERR_SHAPE;
        if (max_pages < 1) return DSA_ERR_SHAPE;
    }
    if ((page_table || seq_lens) && num_seqs < 1) return DSA_ERR_SHAPE;
    if ((page_table || seq_lens) && !token_seq && T > num_seqs) return DSA_ERR_SHAPE;
    if (T == 0) return DSA_OK;
    if (!q || !pool || !topk || !out) return DSA_ERR_NULL;
    if (q_dtype == DSA_FP8_E4M3FN && !q_scale) return DSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(pool) || !aligned16(out)) return DSA_ERR_ALIGN;
    // the kernels mark a masked entry's row source with the bits of -inf in
    // its high word (0xff800000 << 32): every pool row must lie below 2^55
    const uint64_t pool_end = reinterpret_cast<uint64_t>(pool) +
                              static_cast<uint64_t>(num_slots) * static_cast<uint64_t>(dsa_kv_row_bytes(layout));
    if ((pool_end >> 55) != 0 || pool_end < reinterpret_cast<uint64_t>(pool)) return DSA_ERR_ALIGN;
    const size_t need = dsa::attn_workspace_bytes(T, H, K, phase, split_target_cus());
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return DSA_ERR_WORKSPACE;
        if (!aligned256(workspace)) return DSA_ERR_ALIGN;
    }
    return DSA_OK;
}

int32_t run_attn(int32_t phase, const void *q, int32_t q_dtype,
                 const float *q_scale, int32_t T, int32_t H, int32_t D,
                 int32_t rope_dim, const void *pool, int64_t num_slots,
                 int32_t layout, int32_t fp8_format, const int32_t *topk,
                 int32_t K, const int32_t *page_table, int32_t page_size,
                 int32_t max_pages, int32_t num_seqs, const int32_t *token_seq,
                 const int32_t *seq_lens, float softmax_scale, void *out,
                 int32_t out_dtype, float *lse, void *workspace,
                 size_t workspace_bytes, int32_t *err_count, void *stream) {
    int32_t st = validate_attn(q, q_dtype, q_scale, T, H, D, rope_dim, pool,
                               num_slots, layout, fp8_format, topk, K,
                               page_table, page_size, max_pages, num_seqs,
                               token_seq, seq_lens, out, out_dtype, workspace,
                               workspace_bytes, phase);
    if (st != DSA_OK || T == 0) return st;
    if ((st = check_device())) return st;

    dsa::AttnArgs a;
    a.q = q;
    a.q_scale = q_scale;
    a.T = T;
    a.H = H;
    a.pool = static_cast<const uint8_t *>(pool);
    a.num_slots = num_slots;
    a.topk = topk;
    a.K = K;
    a.page_table = page_table;
    int shift = 0;
    if (page_table)
        while ((1 << shift) < page_size) shift++;
    a.page_shift = shift;
    a.max_pages = max_pages;
    a.num_seqs = num_seqs;
    a.token_seq = token_seq;
    a.seq_lens = seq_lens;
    a.softmax_scale = softmax_scale;
    a.out = out;
    a.lse = lse;
    a.ws = static_cast<float *>(workspace);
    a.n_splits = dsa::attn_splits(T, H, K, phase, layout, split_target_cus());
    a.split_len = 0;
    a.err_count = err_count;
    // prefill: one 32-head workgroup per compute unit (a multiple of 8, so
    // that a workgroup's units keep their XCD), each taking its share of
    // the units with the next unit's entries resolved ahead
    a.grid_cap = phase == 1 ? std::max(8, split_target_cus() / 8 * 8) : 0;
    hipError_t e = dsa::launch_attn(a, layout, q_dtype == DSA_FP8_E4M3FN,
                                    out_dtype == DSA_BF16,
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int32_t dsa_kv_row_bytes(int32_t layout) {
    if (layout == DSA_KV_RAW_FP8_512) return 512;
    if (layout == DSA_KV_SCALED_FP8_528) return 528;
    if (layout == DSA_KV_SCALED_FP8_656) return 656;
    if (layout == DSA_KV_BF16_1024) return 1024;
    return -1;
}

const char *dsa_status_string(int32_t status) {
    switch (status) {
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_NULL: return "DSA_ERR_NULL";
    case DSA_ERR_SHAPE: return "DSA_ERR_SHAPE";
    case DSA_ERR_WIDTH_MISMATCH: return "DSA_ERR_WIDTH_MISMATCH";
    case DSA_ERR_LAYOUT: return "DSA_ERR_LAYOUT";
    case DSA_ERR_DTYPE: return "DSA_ERR_DTYPE";
    case DSA_ERR_ALIGN: return "DSA_ERR_ALIGN";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_DEVICE: return "DSA_ERR_DEVICE";
    case DSA_ERR_LAUNCH: return "DSA_ERR_LAUNCH";
    default: return "DSA_ERR_UNKNOWN";
    }
}

int32_t dsa_kv_write(const void *kv, int64_t n, int64_t kv_row_stride,
                     int32_t kv_dtype, int32_t kv_dim, int32_t rope_dim,
                     const int64_t *slot_mapping, void *pool,
                     int64_t num_slots, int32_t layout, int32_t fp8_format,
                     int32_t *err_count, void *stream) {
    if (kv_dim != 512) return DSA_ERR_WIDTH_MISMATCH;
    int32_t st = check_layout(layout);
    if (st) return st;
    if (rope_dim != rope_of(layout)) return DSA_ERR_LAYOUT;
    if ((st = check_fp8_format(fp8_format))) return st;
    if (kv_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (n < 0 || num_slots < 0 || kv_row_stride < 512 + rope_dim) return DSA_ERR_SHAPE;
    if (n > ((int64_t)1 << 33)) return DSA_ERR_SHAPE;
    if (n == 0) return DSA_OK;
    if (!kv || !slot_mapping || !pool) return DSA_ERR_NULL;
    if (!aligned16(kv) || !aligned16(pool) || (kv_row_stride * 2) % 16 != 0)
        return DSA_ERR_ALIGN;
    if ((st = check_device())) return st;
    hipError_t e = dsa::launch_kv_write(
        static_cast<const uint16_t *>(kv), n, kv_row_stride, slot_mapping,
        static_cast<uint8_t *>(pool), num_slots, layout, err_count,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

size_t dsa_quantize_q_workspace_bytes(int64_t n_elems) {
    if (n_elems <= 0) return 0;
    return (size_t)dsa::quantize_q_blocks(n_elems) * sizeof(float);
}

int32_t dsa_quantize_q_fp8(const void *q, int64_t n_elems, int32_t q_dtype,
                           void *q8, float *q_scale, int32_t scale_given,
                           int32_t fp8_format, void *workspace,
                           size_t workspace_bytes, void *stream) {
    int32_t st = check_fp8_format(fp8_format);
    if (st) return st;
    if (q_dtype != DSA_BF16) return DSA_ERR_DTYPE;
    if (n_elems < 0 || n_elems % 8 != 0) return DSA_ERR_SHAPE;
    if (n_elems == 0) return DSA_OK;
    if (!q || !q8 || !q_scale) return DSA_ERR_NULL;
    if (!aligned16(q) || !aligned16(q8)) return DSA_ERR_ALIGN;
    if (!scale_given) {
        if (!workspace || workspace_bytes < dsa_quantize_q_workspace_bytes(n_elems))
            return DSA_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return DSA_ERR_ALIGN;
    }
    if ((st = check_device())) return st;
    hipError_t e = dsa::launch_quantize_q(
        static_cast<const uint16_t *>(q), n_elems, static_cast<uint8_t *>(q8),
        q_scale, scale_given != 0, static_cast<float *>(workspace),
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

int32_t dsa_topk_transform(const int32_t *topk, int32_t T, int32_t k_in,
                           const int32_t *page_table, int32_t page_size,
                           int32_t max_pages, int32_t num_seqs,
                           const int32_t *token_seq, const int32_t *seq_lens,
                           int64_t num_slots, int32_t *out_slots, int32_t k_out,
                           int32_t *valid_count, int32_t *err_count, void *stream) {
    if (T < 0 || k_in < 1 || k_in > 65536) return DSA_ERR_SHAPE;
    if (k_out < k_in || k_out % 128 != 0 || k_out > 65536) return DSA_ERR_SHAPE;
    if (num_slots < 0 || num_slots >= ((int64_t)1 << 31)) return DSA_ERR_SHAPE;
    if (page_table) {
        if (page_size < 1 || (page_size & (page_size - 1)) != 0 || page_size > (1 << 20))
            return DSA_ERR_SHAPE;
        if (max_pages < 1) return DSA_ERR_SHAPE;
    }
    if ((page_table || seq_lens) && num_seqs < 1) return DSA_ERR_SHAPE;
    if ((page_table || seq_lens) && !token_seq && T > num_seqs) return DSA_ERR_SHAPE;
    if (T == 0) return DSA_OK;
    if (!topk || !out_slots) return DSA_ERR_NULL;
    int32_t st = check_device();
    if (st) return st;
    dsa::TransformArgs a;
    a.topk = topk;
    a.T = T;
    a.k_in = k_in;
    a.k_out = k_out;
    a.page_table = page_table;
    int shift = 0;
    if (page_table)
        while ((1 << shift) < page_size) shift++;
    a.page_shift = shift;
    a.max_pages = max_pages;
    a.num_seqs = num_seqs;
    a.token_seq = token_seq;
    a.seq_lens = seq_lens;
    a.num_slots = num_slots;
    a.out = out_slots;
    a.counts = valid_count;
    a.err_count = err_count;
    hipError_t e = dsa::launch_topk_transform(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

size_t dsa_attn_workspace_bytes(int32_t T, int32_t H, int32_t K, int32_t phase) {
    if (T <= 0 || H <= 0 || K <= 0 || K % 128 != 0) return 0;
    return dsa::attn_workspace_bytes(T, H, K, phase, split_target_cus());
}

int32_t dsa_sparse_attn_decode(
    const void *q, int32_t q_dtype, const float *q_scale, int32_t T, int32_t H,
    int32_t D, int32_t rope_dim, const void *pool, int64_t num_slots,
    int32_t layout, int32_t fp8_format, const int32_t *topk, int32_t K,
    const int32_t *page_table, int32_t page_size, int32_t max_pages,
    int32_t num_seqs, const int32_t *token_seq, const int32_t *seq_lens,
    float softmax_scale, void *out, int32_t out_dtype, float *lse,
    void *workspace, size_t workspace_bytes, int32_t *err_count, void *stream) {
    return run_attn(0, q, q_dtype, q_scale, T, H, D, rope_dim, pool, num_slots,
                    layout, fp8_format, topk, K, page_table, page_size,
                    max_pages, num_seqs, token_seq, seq_lens, softmax_scale,
                    out, out_dtype, lse, workspace, workspace_bytes, err_count,
                    stream);
}

int32_t dsa_sparse_attn_decode_noalloc(
    const void *q, int32_t q_dtype, const float *q_scale, int32_t T, int32_t H,
    int32_t D, int32_t rope_dim, const void *pool, int64_t num_slots,
    int32_t layout, int32_t fp8_format, const int32_t *topk, int32_t K,
    const int32_t *page_table, int32_t page_size, int32_t max_pages,
    int32_t num_seqs, const int32_t *token_seq, const int32_t *seq_lens,
    float softmax_scale, void *out, int32_t out_dtype, float *lse,
    int32_t *err_count, void *stream) {
    // every argument check first, against a stand-in for the scratch (an
    // aligned address that is never dereferenced), then the scratch's own
    // size limit
    void *const stand_in = reinterpret_cast<void *>(uintptr_t(256));
    int32_t st = validate_attn(q, q_dtype, q_scale, T, H, D, rope_dim, pool, num_slots,
                               layout, fp8_format, topk, K, page_table, page_size,
                               max_pages, num_seqs, token_seq, seq_lens, out, out_dtype,
                               stand_in, DSA_DECODE_SCRATCH_BYTES, 0);
    if (st != DSA_OK || T == 0) return st;
    if (dsa::attn_workspace_bytes(T, H, K, 0, split_target_cus()) > DSA_DECODE_SCRATCH_BYTES)
        return DSA_ERR_WORKSPACE;
    if ((st = check_device())) return st;
    void *ws = scratch_ptr();
    if (!ws) return DSA_ERR_DEVICE;
    return run_attn(0, q, q_dtype, q_scale, T, H, D, rope_dim, pool, num_slots,
                    layout, fp8_format, topk, K, page_table, page_size,
                    max_pages, num_seqs, token_seq, seq_lens, softmax_scale,
                    out, out_dtype, lse, ws, DSA_DECODE_SCRATCH_BYTES, err_count,
                    stream);
}

int32_t dsa_sparse_attn_prefill(
    const void *q, int32_t q_dtype, const float *q_scale, int32_t T, int32_t H,
    int32_t D, int32_t rope_dim, const void *pool, int64_t num_slots,
    int32_t layout, int32_t fp8_format, const int32_t *topk, int32_t K,
    const int32_t *page_table, int32_t page_size, int32_t max_pages,
    int32_t num_seqs, const int32_t *token_seq, const int32_t *seq_lens,
    float softmax_scale, void *out, int32_t out_dtype, float *lse,
    void *workspace, size_t workspace_bytes, int32_t *err_count, void *stream) {
    return run_attn(1, q, q_dtype, q_scale, T, H, D, rope_dim, pool, num_slots,
                    layout, fp8_format, topk, K, page_table, page_size,
                    max_pages, num_seqs, token_seq, seq_lens, softmax_scale,
                    out, out_dtype, lse, workspace, workspace_bytes, err_count,
                    stream);
}

}  // extern "C"
