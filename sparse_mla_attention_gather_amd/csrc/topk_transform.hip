// topk_transform.hip -- the index transform that runs ahead of the attention
// ("[DSA] Support group-scaled FP8 NoPE KV reads for CUDA TileLang", the
// draft notes: the page-table transform over top-k lists of any width;
// "[DSA] Support flashmla_sparse_q8 prefill backend on CUDA", review thread:
// prefix requests read only the referenced context slots, through the
// flattened page table, on the RAGGED path).
//
// Each row of top-k positions is resolved with the attention's own rule
// (TokenIndexRule) and written compacted: the valid physical slots first, in
// their input order, then -1 up to the output width.  The result is the
// slot list the attention takes with no page table, and its trailing -1
// tiles are the ones the attention skips.
#include "common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kTWaves = 4;                  // one workgroup per row
constexpr int kTThreads = 64 * kTWaves;
constexpr int kTU = 4;                      // 256-entry blocks per pass

// One row per workgroup.  A pass loads kTU blocks of 256 entries (wave w
// takes entries 64w .. 64w+63 of each block, so a block's entries are in
// lane order within a wave and in wave order across waves), resolves them,
// and counts each wave's valid entries with a ballot; one barrier makes the
// counts of the pass visible (double-buffered by pass parity), and each lane
// then writes its slot at the row's running count plus the valid entries
// before it (lower blocks, lower waves, lower lanes).
__global__ __launch_bounds__(kTThreads) void topk_transform_kernel(TransformArgs a) {
    __shared__ __attribute__((aligned(16))) int cnt[2][kTU][kTWaves];
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int64_t t = blockIdx.x;
    const int seq = a.token_seq ? a.token_seq[t] : (int)t;
    const bool seq_ok = (a.page_table == nullptr && a.seq_lens == nullptr) ||
                        (seq >= 0 && seq < a.num_seqs);
    const int seq_len = (a.seq_lens && seq_ok) ? a.seq_lens[seq] : INT_MAX;
    const int32_t *row = a.topk + t * a.k_in;
    const int32_t *pt = a.page_table
                            ? a.page_table + (int64_t)(seq_ok ? seq : 0) * a.max_pages
                            : nullptr;
    int32_t *out = a.out + t * a.k_out;
    const TokenIndexRule rule(seq_ok, seq_len, pt != nullptr, a.page_shift, a.max_pages, a.num_slots);

    int n = 0, n_err = 0, par = 0;
    for (int j0 = 0; j0 < a.k_in; j0 += kTU * kTThreads, par ^= 1) {
        // every load unconditional and in range (clamped), results selected
        int32_t v[kTU], ph[kTU], s[kTU];
#pragma unroll
        for (int u = 0; u < kTU; u++) {
            const int j = j0 + u * kTThreads + threadIdx.x;
            const int32_t x = row[min(j, a.k_in - 1)];
            v[u] = j < a.k_in ? x : -1;
        }
#pragma unroll
        for (int u = 0; u < kTU; u++)
            ph[u] = pt ? pt[min(max(v[u], 0) >> a.page_shift, a.max_pages - 1)] : 0;
        uint64_t vm[kTU];
#pragma unroll
        for (int u = 0; u < kTU; u++) {
            bool err;
            s[u] = rule(v[u], ph[u], err);
            vm[u] = __builtin_amdgcn_ballot_w64(s[u] >= 0);
            n_err += __builtin_popcountll(__builtin_amdgcn_ballot_w64(err));
            if (lane == 0) cnt[par][u][w] = __builtin_popcountll(vm[u]);
        }
        __syncthreads();
        int base = n;
#pragma unroll
        for (int u = 0; u < kTU; u++) {
            const int4 c4 = *reinterpret_cast<const int4 *>(cnt[par][u]);
            const int below = (w > 0 ? c4.x : 0) + (w > 1 ? c4.y : 0) + (w > 2 ? c4.z : 0);
            const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(vm[u] >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)vm[u], 0));
            if (s[u] >= 0) out[base + below + rank] = s[u];
            base += c4.x + c4.y + c4.z + c4.w;
        }
        n = base;
    }
    for (int j = n + threadIdx.x; j < a.k_out; j += kTThreads) out[j] = -1;
    if (threadIdx.x == 0 && a.counts) a.counts[t] = n;
    if (lane == 0 && n_err && a.err_count) atomicAdd(a.err_count, n_err);
}

}  // namespace

hipError_t launch_topk_transform(const TransformArgs &a, hipStream_t stream) {
    topk_transform_kernel<<<dim3((unsigned)a.T), dim3(kTThreads), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace dsa
