// attn.hip -- sparse absorbed-MLA attention over gathered FP8 pool rows.
//
// Method ("[DSA] Support flashmla_sparse_q8 prefill backend on CUDA",
// Modifications; "extend CUDA TileLang raw FP8 KV path", Motivation): every
// query token t has H heads of 512-wide latent queries and a top-k list of
// pool entries (-1 = padding); each selected 512-wide latent row is both key
// and value.  out[t,h] = softmax_j(scale * <q[t,h], x_j>) . x_j over the
// multiset of valid entries; all-masked tokens give 0 (lse = -inf).
//
// Work decomposition: one workgroup (8 wavefronts) owns one unit = (token t,
// block of 16 NT heads, NT = 1 or 2) and one split of t's top-k list (at most
// 2048 entries).  All heads of the block share every gathered row, so Q.X^T
// is a real [16NT x 512] x [512 x entries] contraction for the matrix cores,
// and a row is gathered once per block of up to 32 heads.
//
//   prologue: the split's indices are resolved once (top-k value -> page
//     table -> slot; -1 for padding and for invalid values, which are also
//     counted) into LDS, every phase's loads issued before one wait;
//   gather:   rows move HBM -> LDS with global_load_lds_dwordx4 (16 bytes per
//     lane, no registers), 64-row tiles in 4 LDS buffers, 3 tiles in flight
//     while one is computed, every wave issuing a share of each tile; the
//     16-byte chunks of row r are stored XOR-swizzled by (r & 7) so that the
//     matrix-operand reads below spread over the LDS banks; masked entries
//     read zero rows;
//   QK^T:     wave w forms the partial S^T of entries 16(w%4) .. +16 over the
//     dims half w/4; bf16 query: v_mfma_f32_16x16x32_bf16 on rows converted
//     FP8 -> bf16 exactly; FP8 query: v_mfma_scale_f32_16x16x128_f8f6f4 on
//     the codes themselves (unit block scales), the query scale folded into
//     the score scale.  The two halves are summed through LDS;
//   softmax:  the waves agree on the tile max per head through LDS (online
//     softmax, log2e folded into the scale) and publish P;
//   PV:       wave w accumulates O^T for dims [64w, 64w+64) over the 64
//     entries with v_mfma_f32_16x16x32_f16; its A operand (8 entries x 1 dim
//     per lane) comes straight from the row-major tile through the gfx950
//     LDS transpose read ds_read_b64_tr_b8 and serves every head tile; P is
//     rounded to f16.  528-byte rows: group scales multiply the QK partial
//     sums per 128-wide group and, in PV, multiply P (normalised per tile by
//     the largest scale, the factor applied to the tile's f32 product);
//   epilogue: normalised output + lse, or (several splits) unnormalised
//     partial (o, m, l) states that a second kernel merges.
//
// All workgroups of one token are numbered b = 8k + (t mod 8), so with the
// round-robin workgroup-to-XCD dispatch they share one XCD's L2.
//
// MFMA operand layouts (c = lane % 16, g = lane / 16): A (16 x K): lane (c, g)
// holds row c; B (K x 16): lane (c, g) holds column c; for a given g and
// register slot both hold the same reduction index, which is all a
// contraction needs, so the reduction index is assigned freely (dims for
// QK, entries ks*32 + g*8 + r for PV).  The 16x16 result: lane (c, g) holds
// rows 4g..4g+3 of column c.
//
// ds_read_b64_tr_b8 (measured on gfx950): within each 16-lane group, byte b
// of lane l is byte (l & 7) of the 8 bytes addressed by lane 2b + (l >> 3).
#include <limits.h>

#include "common.h"
#include "launch.h"

#ifndef DSA_DECODE_TARGET_BLOCKS
#define DSA_DECODE_TARGET_BLOCKS 256
#endif

namespace dsa {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;          // entries per tile
constexpr int kNBuf = 4;           // LDS tile buffers
constexpr int kMaxSplit = 2048;    // entries per workgroup at most
constexpr int kRowsPerWave = kTile / kWaves;        // DMA share of a tile
constexpr int kLoadsRaw = kRowsPerWave / 2;         // DMA instructions per wave per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;     // log2 headroom of the running max (P <= 256)
// "No maximum yet": finite, so that 2^(-inf - kNoMax) = 0 for masked scores
// without a select, and far below any real score.
constexpr float kNoMax = -1.0e30f;

// LDS map (bytes) for NT head tiles of 16
template <int NT>
struct Lds {
    static constexpr int kHB = 16 * NT;
    static constexpr int kBufBytes = kTile * 512;                // 32 KB payload
    static constexpr int kScBytes = kTile * 16;                  // 1 KB scales
    static constexpr int kOffScales = kNBuf * kBufBytes;
    static constexpr int kOffSlots = kOffScales + kNBuf * kScBytes;
    static constexpr int kOffP = kOffSlots + kMaxSplit * 4;      // P, aliased with partial S
    static constexpr int kPBytes = kWaves * kHB * 16 * 4;        // partial S of 8 waves
    static constexpr int kOffRedM = kOffP + kPBytes;
    static constexpr int kOffRedL = kOffRedM + kWaves * kHB * 4;
    static constexpr int kBytes = kOffRedL + kWaves * kHB * 4;
    static_assert(kBytes <= 160 * 1024, "LDS budget");
    static_assert(kHB * kTile * 4 <= kPBytes, "P fits in the partial-S area");
};

// Masked entries read zeros (P = 0 must never meet a NaN of an unreferenced
// slot).  64 distinct zero rows, picked by the tile row, keep these reads off
// a single set of L2 lines.
constexpr int kZeroRows = 64;
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[kZeroRows * kScaledBytes] = {};

#define LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

// Workgroup barrier without the workgroup memory fence that __syncthreads()
// implies: that fence would also wait for every outstanding LDS-DMA load and
// so serialise the gather pipeline.  Callers wait for what they need first.
__device__ __forceinline__ void barrier_raw() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt with vmcnt <= N (N <= 63) and lgkmcnt == 0; expcnt not waited.
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// Index resolution of one entry value i, given the page-table word `phys`
// already fetched for it (see the prologue): -1 -> padding; other invalid
// values -> masked and counted.
__device__ __forceinline__ int32_t resolve_entry(const AttnArgs &a, int32_t i,
                                                 int32_t phys, bool seq_ok,
                                                 int seq_len, bool &err) {
    err = false;
    if (i == -1) return -1;
    err = true;
    if (i < 0 || !seq_ok || i >= seq_len) return -1;
    int64_t slot = i;
    if (a.page_table) {
        if ((i >> a.page_shift) >= a.max_pages || phys < 0) return -1;
        slot = ((int64_t)phys << a.page_shift) | (int64_t)(i & ((1 << a.page_shift) - 1));
    }
    if (slot >= a.num_slots) return -1;
    err = false;
    return (int32_t)slot;
}

__device__ __forceinline__ int swz(int row) { return row & 7; }

// LDS slot swizzles that keep eight consecutive lanes c of a 16-byte access
// on distinct banks: the partial-score rows ([head][4 entry groups]) rotate
// their groups by (c & 7) >> 1, the P rows ([head][16 groups of 4 entries])
// XOR their group index with c & 7.
__device__ __forceinline__ int sp_slot(int grp, int c) { return (grp + ((c & 7) >> 1)) & 3; }
__device__ __forceinline__ int p_slot(int grp, int c) { return grp ^ (c & 7); }

// 32-bit LDS address of a pointer into dynamic shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)LDS_PTR(p);
}

// One 16-byte-per-lane HBM -> LDS copy: lane l's 16 bytes land at
// lds_base + 16 l.  Issued through inline assembly so that the compiler does
// not see pending LDS writes: it would otherwise guard every later LDS read
// with a wait for all outstanding loads.  Completion is tracked explicitly
// with s_waitcnt vmcnt before the barrier that publishes a tile.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved; only this asm writes it
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// Issue the DMA of one 64-row tile: wave w moves rows [8w, 8w+8), two rows
// per instruction (lane l -> row 8w + 2k + (l >> 5), LDS chunk position
// l & 31, holding global chunk (l & 31) ^ swz(row)); scaled rows add one
// 8-lane instruction for the rows' 16-byte scale words.
template <int LAYOUT, int NT>
__device__ __forceinline__ void issue_tile(const AttnArgs &a, uint32_t lds0,
                                           const int32_t *slots, int tile_base,
                                           int buf, int w, int lane) {
    using L = Lds<NT>;
    constexpr int64_t kRow = LAYOUT == 0 ? kRawBytes : kScaledBytes;
    const int r0 = kRowsPerWave * w;
    const uint32_t dst = lds0 + buf * L::kBufBytes + r0 * 512;
    const int pos = lane & 31;
    int32_t sl[kLoadsRaw];
#pragma unroll
    for (int k = 0; k < kLoadsRaw; k++) sl[k] = slots[tile_base + r0 + 2 * k + (lane >> 5)];
#pragma unroll
    for (int k = 0; k < kLoadsRaw; k++) {
        const int r = r0 + 2 * k + (lane >> 5);
        const int chunk = pos ^ swz(r);
        const uint8_t *src = sl[k] >= 0 ? a.pool + (int64_t)sl[k] * kRow + chunk * 16
                                        : kZeroRow + r * kRow + chunk * 16;
        dma16(src, dst + k * 1024);
    }
    if (LAYOUT == 1) {
        if (lane < kRowsPerWave) {
            const int r = r0 + lane;
            const int32_t slot = slots[tile_base + r];
            const uint8_t *src = slot >= 0 ? a.pool + (int64_t)slot * kRow + kD
                                           : kZeroRow + r * kRow + kD;
            dma16(src, lds0 + L::kOffScales + buf * L::kScBytes + r0 * 16);
        }
    }
}

template <int LAYOUT, bool QFP8, bool OUT_BF16, bool SPLIT, int NT>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
    using L = Lds<NT>;
    constexpr int kHB = L::kHB;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int kLoads = kLoadsRaw + (LAYOUT == 1 ? 1 : 0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int wq = w & 3;           // QK: entries 16 wq .. +16 of the tile
    const int hq = w >> 2;          // QK: dims half hq (256 dims)
    const int n_hb = (a.H + kHB - 1) / kHB;

    // XCD-aware numbering: all of token t's workgroups are 8k + (t % 8)
    const int per_tok = n_hb * a.n_splits;
    const int x = blockIdx.x & 7;
    const int kq = blockIdx.x >> 3;
    const int t = (kq / per_tok) * 8 + x;
    if (t >= a.T) return;
    const int hb = (kq % per_tok) / a.n_splits;
    const int split = kq % a.n_splits;

    int32_t *slots = reinterpret_cast<int32_t *>(lds + L::kOffSlots);
    float *p_lds = reinterpret_cast<float *>(lds + L::kOffP);    // [kHB heads][64 entries]
    float *sp_lds = reinterpret_cast<float *>(lds + L::kOffP);   // [8 waves][kHB heads][16]
    float *red_m = reinterpret_cast<float *>(lds + L::kOffRedM);
    float *red_l = reinterpret_cast<float *>(lds + L::kOffRedL);

    const int seq = a.token_seq ? a.token_seq[t] : t;
    const bool seq_ok = (a.page_table == nullptr && a.seq_lens == nullptr) ||
                        (seq >= 0 && seq < a.num_seqs);
    const int seq_len = (a.seq_lens && seq_ok) ? a.seq_lens[seq] : INT_MAX;
    const int begin = split * a.split_len;
    const int n_ent = min(a.K - begin, a.split_len);   // a multiple of 64
    const int n_tiles = n_ent / kTile;

    // Query of head nt*16 + c as the B operand.  bf16: bq[nt][kk] = q[h][d ..
    // d+8] with d = (hq*16 + (kk>>1)*4 + g)*16 + (kk&1)*8, so that a lane's
    // two steps 2m, 2m+1 use one 16-byte chunk of the row; FP8: bq8[nt][k2] =
    // q8[h][hq*256 + k2*128 + g*32 .. +32].  Heads beyond H read head 0 and
    // are not stored.
    bf16x8 bq[QFP8 ? 1 : NT][8];
    i32x8 bq8[QFP8 ? NT : 1][2];
    float sscale = a.softmax_scale * kLog2e;
    if constexpr (QFP8) {
        sscale *= *a.q_scale;
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const int h = hb * kHB + nt * 16 + c;
            const uint8_t *qp = reinterpret_cast<const uint8_t *>(a.q) +
                                ((int64_t)t * a.H + (h < a.H ? h : 0)) * kD + hq * 256 + g * 32;
#pragma unroll
            for (int k2 = 0; k2 < 2; k2++)
                bq8[nt][k2] = *reinterpret_cast<const i32x8 *>(qp + k2 * 128);
        }
    } else {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const int h = hb * kHB + nt * 16 + c;
            const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) +
                               ((int64_t)t * a.H + (h < a.H ? h : 0)) * kD;
#pragma unroll
            for (int kk = 0; kk < 8; kk++)
                bq[nt][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                    qp + (hq * 16 + (kk >> 1) * 4 + g) * 16 + (kk & 1) * 8));
        }
    }

    // ---- prologue: resolve this split's indices into LDS.  Every load is
    // unconditional (addresses clamped into range, results selected after),
    // so each phase issues all its loads before a single wait.  When the
    // token's page-table row fits in the (still unused) P area it is staged
    // there together with the top-k loads, so resolution costs one global
    // latency instead of two.
    {
        constexpr int kPer = kMaxSplit / kThreads;
        constexpr int kPtCap = L::kPBytes / 4;
        constexpr int kPtPer = kPtCap / kThreads;
        const int32_t *tk = a.topk + (int64_t)t * a.K + begin;
        const int32_t *row = a.page_table + (int64_t)(seq_ok ? seq : 0) * a.max_pages;
        int32_t *pt_lds = reinterpret_cast<int32_t *>(lds + L::kOffP);
        const bool pt_staged = a.page_table != nullptr && a.max_pages <= kPtCap;
        int32_t v[kPer], phys[kPer];
        if (pt_staged) {
            int32_t pw[kPtPer];
#pragma unroll
            for (int k = 0; k < kPtPer; k++) pw[k] = row[min(tid + k * kThreads, a.max_pages - 1)];
#pragma unroll
            for (int i = 0; i < kPer; i++) {
                const int j = tid + i * kThreads;
                const int32_t xv = tk[min(j, n_ent - 1)];
                v[i] = j < n_ent ? xv : -1;
            }
#pragma unroll
            for (int k = 0; k < kPtPer; k++)
                if (tid + k * kThreads < a.max_pages) pt_lds[tid + k * kThreads] = pw[k];
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kPer; i++)
                phys[i] = pt_lds[min(max(v[i], 0) >> a.page_shift, a.max_pages - 1)];
        } else {
#pragma unroll
            for (int i = 0; i < kPer; i++) {
                const int j = tid + i * kThreads;
                const int32_t xv = tk[min(j, n_ent - 1)];
                v[i] = j < n_ent ? xv : -1;
            }
            if (a.page_table) {
#pragma unroll
                for (int i = 0; i < kPer; i++)
                    phys[i] = row[min(max(v[i], 0) >> a.page_shift, a.max_pages - 1)];
            } else {
#pragma unroll
                for (int i = 0; i < kPer; i++) phys[i] = 0;
            }
        }
        int n_err = 0;
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            const int j = tid + i * kThreads;
            bool err;
            const int32_t s = resolve_entry(a, v[i], phys[i], seq_ok, seq_len, err);
            n_err += err;
            if (j < n_ent) slots[j] = s;
        }
        if (a.err_count && hb == 0) {
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) n_err += __shfl_xor(n_err, s);
            if (lane == 0 && n_err) atomicAdd(a.err_count, n_err);
        }
    }
    // slots visible; also drains the query and index loads, so that inside
    // the loop the only outstanding vector-memory operations are tile DMAs
    __syncthreads();
    const uint32_t lds0 = lds_addr(lds);

    // ---- fill the pipeline
#pragma unroll
    for (int i = 0; i < kNBuf - 1; i++)
        if (i < n_tiles) issue_tile<LAYOUT, NT>(a, lds0, slots, i * kTile, i, w, lane);

    float m_run[NT], l_part[NT];
    f32x4 acc[4][NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        m_run[nt] = kNoMax;
        l_part[nt] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) acc[dt][nt] = f32x4{0, 0, 0, 0};
    }

    for (int it = 0; it < n_tiles; it++) {
        const int buf = it % kNBuf;
        const uint8_t *xb = lds + buf * L::kBufBytes;
        const f32x4 *scb = reinterpret_cast<const f32x4 *>(lds + L::kOffScales + buf * L::kScBytes);
        const int32_t *ts = slots + it * kTile;

        // (A) this tile's rows have landed (for this wave), then for all
        const int ahead = min(kNBuf - 2, n_tiles - 1 - it);
        if (ahead >= 2) wait_vm_lgkm0<2 * kLoads>();
        else if (ahead == 1) wait_vm_lgkm0<kLoads>();
        else wait_vm_lgkm0<0>();
        barrier_raw();
        if (it + kNBuf - 1 < n_tiles)
            issue_tile<LAYOUT, NT>(a, lds0, slots, (it + kNBuf - 1) * kTile,
                                   (it + kNBuf - 1) % kNBuf, w, lane);

        // (B) partial S^T for entries 16 wq .. +16 over dims half hq
        {
            const int r = 16 * wq + c;
            const uint8_t *xr = xb + r * 512;
            const int sw = swz(r);
            f32x4 sc4[4];
            if constexpr (LAYOUT == 1) {
#pragma unroll
                for (int i = 0; i < 4; i++) sc4[i] = scb[16 * wq + 4 * g + i];
            }
            f32x4 part[NT];
            if constexpr (QFP8) {
                // 2 steps of K = 128: dims hq*256 + k2*128 + g*32 .. +32 (two
                // 16-byte chunks); each step is exactly one scale group
                u32x4 xa[2][2];
#pragma unroll
                for (int k2 = 0; k2 < 2; k2++)
#pragma unroll
                    for (int hf = 0; hf < 2; hf++)
                        xa[k2][hf] = *reinterpret_cast<const u32x4 *>(
                            xr + (((hq * 16 + k2 * 8 + g * 2 + hf) ^ sw) * 16));
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    f32x4 accg[2];
#pragma unroll
                    for (int k2 = 0; k2 < 2; k2++) {
                        const i32x8 av = {(int)xa[k2][0][0], (int)xa[k2][0][1], (int)xa[k2][0][2],
                                          (int)xa[k2][0][3], (int)xa[k2][1][0], (int)xa[k2][1][1],
                                          (int)xa[k2][1][2], (int)xa[k2][1][3]};
                        accg[k2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            av, bq8[nt][k2], f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
                    }
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        if constexpr (LAYOUT == 0)
                            part[nt][i] = accg[0][i] + accg[1][i];
                        else
                            part[nt][i] = accg[0][i] * sc4[i][2 * hq] + accg[1][i] * sc4[i][2 * hq + 1];
                    }
                }
            } else {
                // 8 steps of K = 32; steps 2m, 2m+1 take the two halves of
                // chunk hq*16 + 4m + g (so a step's 32 dims stay inside one
                // 128-wide scale group: group 2hq + m/2)
                u32x4 xc[4];
#pragma unroll
                for (int m = 0; m < 4; m++)
                    xc[m] = *reinterpret_cast<const u32x4 *>(xr + (((hq * 16 + m * 4 + g) ^ sw) * 16));
                f32x4 accg[NT][2];
#pragma unroll
                for (int nt = 0; nt < NT; nt++) accg[nt][0] = accg[nt][1] = f32x4{0, 0, 0, 0};
#pragma unroll
                for (int kk = 0; kk < 8; kk++) {
                    const u32x4 &ch = xc[kk >> 1];
                    const bf16x8 av = (kk & 1) ? e4m3x8_to_bf16(ch[2], ch[3])
                                               : e4m3x8_to_bf16(ch[0], ch[1]);
                    // raw rows: two independent chains (even / odd kk); scaled
                    // rows: one chain per 128-wide scale group of this half
                    const int q = LAYOUT == 0 ? (kk & 1) : (kk >> 2);
#pragma unroll
                    for (int nt = 0; nt < NT; nt++)
                        accg[nt][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[nt][kk],
                                                                              accg[nt][q], 0, 0, 0);
                }
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        if constexpr (LAYOUT == 0)
                            part[nt][i] = accg[nt][0][i] + accg[nt][1][i];
                        else
                            part[nt][i] = accg[nt][0][i] * sc4[i][2 * hq] +
                                          accg[nt][1][i] * sc4[i][2 * hq + 1];
                    }
            }
#pragma unroll
            for (int nt = 0; nt < NT; nt++)
                *reinterpret_cast<f32x4 *>(sp_lds + (w * kHB + nt * 16 + c) * 16 +
                                           4 * sp_slot(g, c)) = part[nt];
        }
        wait_lgkm0();
        barrier_raw();

        // (C) full scores of entries 16 wq + 4g + i, heads nt*16 + c; tile max
        float sv[NT][4];
        {
            const int4 sl4 = *reinterpret_cast<const int4 *>(ts + 16 * wq + 4 * g);
            const int slv[4] = {sl4.x, sl4.y, sl4.z, sl4.w};
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                const int hh = nt * 16 + c;
                const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sp_lds + (wq * kHB + hh) * 16 + 4 * sp_slot(g, c));
                const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sp_lds + ((wq + 4) * kHB + hh) * 16 + 4 * sp_slot(g, c));
                float mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    sv[nt][i] = slv[i] >= 0 ? (s0[i] + s1[i]) * sscale : -INFINITY;
                    mx = fmaxf(mx, sv[nt][i]);
                }
                mx = fmaxf(mx, __shfl_xor(mx, 16));
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                if (g == 0 && w < 4) red_m[w * kHB + hh] = mx;
            }
        }
        wait_lgkm0();
        barrier_raw();

        // (D) shared tile max and probabilities.  The running reference max
        // only moves when the tile max exceeds it by more than kSlack (log2
        // units), so the O rescale is rare; P = 2^(s - m_ref) <= 2^kSlack.
        // All waves see the same maxima and so make the same choice.  Waves
        // 0-3 own the entries' P and their share of the denominator.
        {
            bool any_resc = false;
            float alpha[NT];
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                const int hh = nt * 16 + c;
                const float tmax = fmaxf(fmaxf(red_m[hh], red_m[kHB + hh]),
                                         fmaxf(red_m[2 * kHB + hh], red_m[3 * kHB + hh]));
                const bool resc = tmax - m_run[nt] > kSlack;   // false for an all-masked tile
                alpha[nt] = resc ? __builtin_amdgcn_exp2f(m_run[nt] - tmax) : 1.0f;
                if (resc) m_run[nt] = tmax;
                any_resc |= resc;
                if (w < 4) {
                    f32x4 p;
                    float ps = 0.0f;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        p[i] = __builtin_amdgcn_exp2f(sv[nt][i] - m_run[nt]);   // masked: 2^-inf = 0
                        ps += p[i];
                    }
                    l_part[nt] = l_part[nt] * alpha[nt] + ps;
                    *reinterpret_cast<f32x4 *>(p_lds + hh * kTile + 4 * p_slot(4 * w + g, c)) = p;
                }
            }
            if (__ballot(any_resc)) {
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
#pragma unroll
                    for (int dt = 0; dt < 4; dt++) acc[dt][nt] *= alpha[nt];
            }
        }
        wait_lgkm0();
        barrier_raw();

        // (E) O^T[dims 64w.., heads] += X^T . P^T over the 64 entries.
        {
            // A operand X^T via transpose reads: lane (c, g) addresses entry
            // e0 + (c >> 1), half (c & 1) of the chunk of dims 64w + 16dt ..
            u32x2 tv[2][4];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const int row = ks * 32 + g * 8 + (c >> 1);
                const uint8_t *rp = xb + row * 512 + (c & 1) * 8;
                const int sw = swz(row);
#pragma unroll
                for (int dt = 0; dt < 4; dt++)
                    tv[ks][dt] = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2 *>(
                                   LDS_PTR(rp + (((4 * w + dt) ^ sw) * 16)))));
            }
            // B operand P^T: entries ks*32 + g*8 + r of head nt*16 + c
            float pv[NT][2][8];
#pragma unroll
            for (int nt = 0; nt < NT; nt++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    const float *pp = p_lds + (nt * 16 + c) * kTile;
                    const f32x4 p0 = *reinterpret_cast<const f32x4 *>(pp + 4 * p_slot(ks * 8 + g * 2, c));
                    const f32x4 p1 = *reinterpret_cast<const f32x4 *>(pp + 4 * p_slot(ks * 8 + g * 2 + 1, c));
#pragma unroll
                    for (int r = 0; r < 4; r++) {
                        pv[nt][ks][r] = p0[r];
                        pv[nt][ks][4 + r] = p1[r];
                    }
                }
            float smax = 1.0f;
            if constexpr (LAYOUT == 1) {
                // scale group w/2 of each entry, normalised by the tile's
                // largest so that the f16 operand stays in range; the factor
                // is put back when the tile's product is added to O
                const float *scf = reinterpret_cast<const float *>(scb);
                const int grp = w >> 1;
                float sc[2][8];
                smax = 0.0f;
#pragma unroll
                for (int ks = 0; ks < 2; ks++)
#pragma unroll
                    for (int r = 0; r < 8; r++) {
                        sc[ks][r] = scf[(ks * 32 + g * 8 + r) * 4 + grp];
                        smax = fmaxf(smax, sc[ks][r]);
                    }
                smax = fmaxf(smax, __shfl_xor(smax, 16));
                smax = fmaxf(smax, __shfl_xor(smax, 32));
                const float inv = smax > 0.0f ? 1.0f / smax : 0.0f;
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
#pragma unroll
                    for (int ks = 0; ks < 2; ks++)
#pragma unroll
                        for (int r = 0; r < 8; r++) pv[nt][ks][r] *= sc[ks][r] * inv;
            }
            f16x8 bp[NT][2];
#pragma unroll
            for (int nt = 0; nt < NT; nt++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++)
#pragma unroll
                    for (int r = 0; r < 8; r++) bp[nt][ks][r] = (_Float16)pv[nt][ks][r];
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                const f16x8 av0 = e4m3x8_to_f16(tv[0][dt][0], tv[0][dt][1]);
                const f16x8 av1 = e4m3x8_to_f16(tv[1][dt][0], tv[1][dt][1]);
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    if constexpr (LAYOUT == 0) {
                        acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av0, bp[nt][0], acc[dt][nt], 0, 0, 0);
                        acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av1, bp[nt][1], acc[dt][nt], 0, 0, 0);
                    } else {
                        f32x4 prt = __builtin_amdgcn_mfma_f32_16x16x32_f16(av0, bp[nt][0], f32x4{0, 0, 0, 0}, 0, 0, 0);
                        prt = __builtin_amdgcn_mfma_f32_16x16x32_f16(av1, bp[nt][1], prt, 0, 0, 0);
                        acc[dt][nt] += prt * smax;
                    }
                }
            }
        }
    }

    // total softmax denominator per head: lanes of this wave, then waves 0-3
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        l_part[nt] += __shfl_xor(l_part[nt], 16);
        l_part[nt] += __shfl_xor(l_part[nt], 32);
        if (g == 0 && w < 4) red_l[w * kHB + nt * 16 + c] = l_part[nt];
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        const int hh = nt * 16 + c;
        const int h = hb * kHB + hh;
        if (h >= a.H) continue;
        const float l_tot = red_l[hh] + red_l[kHB + hh] + red_l[2 * kHB + hh] + red_l[3 * kHB + hh];
        const int64_t th = (int64_t)t * a.H + h;
        if (SPLIT) {
            float *wo = a.ws + (th * a.n_splits + split) * kD + 64 * w + 4 * g;
#pragma unroll
            for (int dt = 0; dt < 4; dt++) *reinterpret_cast<f32x4 *>(wo + dt * 16) = acc[dt][nt];
            if (w == 0 && g == 0) {
                float *ml = a.ws + (int64_t)a.T * a.H * a.n_splits * kD +
                            (th * a.n_splits + split) * 2;
                ml[0] = m_run[nt];
                ml[1] = l_tot;
            }
        } else {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            const int64_t base = th * kD + 64 * w + 4 * g;
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                const f32x4 o = acc[dt][nt] * inv;
                if (OUT_BF16) {
                    u32x2 pk = {f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16),
                                f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16)};
                    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + base + dt * 16) = pk;
                } else {
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + base + dt * 16) = o;
                }
            }
            if (a.lse && w == 0 && g == 0)
                a.lse[th] = l_tot > 0.0f ? (m_run[nt] + log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

// Merge of the split partial states: one wavefront per (token, head), each
// lane owning 8 of the 512 dims.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (th >= (int64_t)a.T * a.H) return;
    const int S = a.n_splits;
    const float *ml = a.ws + (int64_t)a.T * a.H * S * kD + th * S * 2;
    float M = -INFINITY;
    for (int s = 0; s < S; s++) M = fmaxf(M, ml[2 * s]);
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float Lsum = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < S; s++) {
            const float ms = ml[2 * s];
            if (ms == -INFINITY) continue;
            const float wgt = exp2f(ms - M);
            Lsum += wgt * ml[2 * s + 1];
            const float *src = a.ws + (th * S + s) * kD + lane * 8;
            const f32x4 v0 = *reinterpret_cast<const f32x4 *>(src);
            const f32x4 v1 = *reinterpret_cast<const f32x4 *>(src + 4);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                o[i] += wgt * v0[i];
                o[4 + i] += wgt * v1[i];
            }
        }
    }
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    if (OUT_BF16) {
        u32x4 pk;
#pragma unroll
        for (int i = 0; i < 4; i++)
            pk[i] = f32_to_bf16_bits(o[2 * i] * inv) | (f32_to_bf16_bits(o[2 * i + 1] * inv) << 16);
        *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(a.out) + th * kD + lane * 8) = pk;
    } else {
        float *dst = reinterpret_cast<float *>(a.out) + th * kD + lane * 8;
        *reinterpret_cast<f32x4 *>(dst) = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
    }
    if (a.lse && lane == 0) a.lse[th] = Lsum > 0.0f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// Heads per workgroup: 32 when there are more than 16 heads (a row is then
// gathered once per 32 heads), else 16.
static int head_tiles(int H) { return H > 16 ? 2 : 1; }

// Splits per (token, head block): enough workgroups to cover the CUs for
// small batches, and never more than kMaxSplit entries per workgroup.
int attn_decode_splits(int T, int H, int K) {
    const int hbw = 16 * head_tiles(H);
    const int64_t units = (int64_t)T * ((H + hbw - 1) / hbw);
    const int tiles = K / kTile;
    if (units <= 0 || tiles <= 0) return 1;
    int64_t s = (DSA_DECODE_TARGET_BLOCKS + units - 1) / units;
    const int64_t s_min = (K + kMaxSplit - 1) / kMaxSplit;
    if (s < s_min) s = s_min;
    if (s > tiles) s = tiles;
    const int tps = (int)((tiles + s - 1) / s);
    return (tiles + tps - 1) / tps;
}

static int prefill_splits(int K) { return (K + kMaxSplit - 1) / kMaxSplit; }

static int split_len_for(int K, int splits) {
    const int tiles = K / kTile;
    return ((tiles + splits - 1) / splits) * kTile;
}

int attn_splits(int T, int H, int K, int phase) {
    return phase == 0 ? attn_decode_splits(T, H, K) : prefill_splits(K);
}

size_t attn_workspace_bytes(int T, int H, int K, int phase) {
    const int s = attn_splits(T, H, K, phase);
    if (s <= 1) return 0;
    size_t b = (size_t)T * H * s * (kD + 2) * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

template <typename Kern>
static void allow_big_lds(Kern kern, int bytes) {
    // once per instantiation; not a stream operation, so capture-safe
    static const hipError_t e = hipFuncSetAttribute(
        (const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    (void)e;
}

template <int LAYOUT, bool QFP8, bool OUT_BF16, int NT>
static hipError_t launch_one(const AttnArgs &a, hipStream_t stream) {
    constexpr int kHB = 16 * NT;
    const int n_hb = (a.H + kHB - 1) / kHB;
    const dim3 grid((unsigned)(((int64_t)a.T + 7) / 8 * 8 * n_hb * a.n_splits));
    constexpr int bytes = Lds<NT>::kBytes;
    if (a.n_splits > 1) {
        auto kern = attn_kernel<LAYOUT, QFP8, OUT_BF16, true, NT>;
        allow_big_lds(kern, bytes);
        kern<<<grid, dim3(kThreads), bytes, stream>>>(a);
        const dim3 cgrid((unsigned)(((int64_t)a.T * a.H + 3) / 4));
        attn_combine_kernel<OUT_BF16><<<cgrid, dim3(256), 0, stream>>>(a);
    } else {
        auto kern = attn_kernel<LAYOUT, QFP8, OUT_BF16, false, NT>;
        allow_big_lds(kern, bytes);
        kern<<<grid, dim3(kThreads), bytes, stream>>>(a);
    }
    return hipGetLastError();
}

template <int LAYOUT, bool QFP8, bool OUT_BF16>
static hipError_t launch_nt(const AttnArgs &a, hipStream_t stream) {
    return head_tiles(a.H) == 2 ? launch_one<LAYOUT, QFP8, OUT_BF16, 2>(a, stream)
                                : launch_one<LAYOUT, QFP8, OUT_BF16, 1>(a, stream);
}

hipError_t launch_attn(const AttnArgs &a_in, int layout, bool q_fp8, bool out_bf16,
                       hipStream_t stream) {
    AttnArgs a = a_in;
    if (a.n_splits < 1) a.n_splits = 1;
    a.split_len = split_len_for(a.K, a.n_splits);
#define DSA_DISPATCH(L, Q, O) \
    if (layout == L && q_fp8 == Q && out_bf16 == O) return launch_nt<L, Q, O>(a, stream);
    DSA_DISPATCH(0, false, false)
    DSA_DISPATCH(0, false, true)
    DSA_DISPATCH(0, true, false)
    DSA_DISPATCH(0, true, true)
    DSA_DISPATCH(1, false, false)
    DSA_DISPATCH(1, false, true)
    DSA_DISPATCH(1, true, false)
    DSA_DISPATCH(1, true, true)
#undef DSA_DISPATCH
    return hipErrorInvalidValue;
}

}  // namespace dsa
