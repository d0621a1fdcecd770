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
// block of 16 heads) and one split of t's top-k list (at most 2048 entries).
// All 16 heads share every gathered row, so Q.X^T is a real
// [16 x 512] x [512 x entries] contraction for the matrix cores.
//
//   prologue: the split's indices are resolved once (top-k value -> page
//     table -> slot; -1 for padding and for invalid values, which are also
//     counted) into LDS;
//   gather:   rows move HBM -> LDS with global_load_lds_dwordx4 (16 bytes per
//     lane, no registers), 64-row tiles in 4 LDS buffers, 3 tiles in flight
//     while one is computed, every wave issuing a share of each tile; the
//     16-byte chunks of row r are stored XOR-swizzled by (r & 7) so that the
//     matrix-operand reads below spread over the LDS banks; masked entries
//     read a static zero row;
//   QK^T:     wave w forms the partial S^T of entries 16(w%4) .. +16 over the
//     dims half w/4 with v_mfma_f32_16x16x32_bf16 (rows FP8 -> bf16 exactly;
//     an FP8 query is converted exactly too and its scale folded into the
//     score scale); the two halves are summed through LDS;
//   softmax:  the waves agree on the tile max per head through LDS (online
//     softmax, log2e folded into the scale) and publish P;
//   PV:       wave w accumulates O^T for dims [64w, 64w+64) over the 64
//     entries with v_mfma_f32_16x16x32_f16; its A operand (8 entries x 1 dim
//     per lane) comes straight from the row-major tile through the gfx950
//     LDS transpose read ds_read_b64_tr_b8; P is rounded to f16.  528-byte
//     rows: group scales multiply the QK partial sums per 128-wide group
//     and, in PV, multiply P (normalised per tile by the largest scale, the
//     factor applied to the tile's f32 product);
//   epilogue: normalised output + lse, or (several splits) unnormalised
//     partial (o, m, l) states that a second kernel merges.
//
// Workgroups of one unit are numbered b = 8k + x with the same x, so with the
// round-robin workgroup-to-XCD dispatch they share one XCD's L2.
//
// MFMA operand layouts (c = lane % 16, g = lane / 16): A (16 x K): lane (c, g)
// holds row c; B (K x 16): lane (c, g) holds column c; for a given g and
// register slot both hold the same reduction index, which is all a
// contraction needs, so the reduction index is assigned freely: dims
// kk*32 + g*8 + r for QK, entries ks*32 + g*8 + r for PV.  The 16x16 result:
// lane (c, g) holds rows 4g..4g+3 of column c.
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

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHB = 16;            // heads per workgroup
constexpr int kTile = 64;          // entries per tile
constexpr int kNBuf = 4;           // LDS tile buffers
constexpr int kMaxSplit = 2048;    // entries per workgroup at most
constexpr int kRowsPerWave = kTile / kWaves;        // DMA share of a tile
constexpr int kLoadsRaw = kRowsPerWave / 2;         // DMA instructions per wave per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;     // log2 headroom of the running max (P <= 256)

// LDS map (bytes)
constexpr int kBufBytes = kTile * 512;                  // 32 KB payload
constexpr int kScBytes = kTile * 16;                    // 1 KB scales
constexpr int kOffScales = kNBuf * kBufBytes;
constexpr int kOffSlots = kOffScales + kNBuf * kScBytes;
constexpr int kOffP = kOffSlots + kMaxSplit * 4;        // P, aliased with partial S
constexpr int kPBytes = kWaves * kHB * 16 * 4;          // 8 KB
constexpr int kOffRedM = kOffP + kPBytes;
constexpr int kOffRedL = kOffRedM + kWaves * kHB * 4;
constexpr int kLdsBytes = kOffRedL + kWaves * kHB * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kHB * kTile * 4 <= kPBytes, "P fits in the partial-S area");

__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[kScaledBytes] = {};

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
template <int LAYOUT>
__device__ __forceinline__ void issue_tile(const AttnArgs &a, uint32_t lds0,
                                           const int32_t *slots, int tile_base,
                                           int buf, int w, int lane) {
    constexpr int64_t kRow = LAYOUT == 0 ? kRawBytes : kScaledBytes;
    const int r0 = kRowsPerWave * w;
    const uint32_t dst = lds0 + buf * kBufBytes + r0 * 512;
    const int pos = lane & 31;
    int32_t sl[kLoadsRaw];
#pragma unroll
    for (int k = 0; k < kLoadsRaw; k++) sl[k] = slots[tile_base + r0 + 2 * k + (lane >> 5)];
#pragma unroll
    for (int k = 0; k < kLoadsRaw; k++) {
        const int r = r0 + 2 * k + (lane >> 5);
        const int chunk = pos ^ swz(r);
        const uint8_t *src = sl[k] >= 0 ? a.pool + (int64_t)sl[k] * kRow + chunk * 16
                                        : kZeroRow + chunk * 16;
        dma16(src, dst + k * 1024);
    }
    if (LAYOUT == 1) {
        if (lane < kRowsPerWave) {
            const int r = r0 + lane;
            const int32_t slot = slots[tile_base + r];
            const uint8_t *src = slot >= 0 ? a.pool + (int64_t)slot * kRow + kD : kZeroRow;
            dma16(src, lds0 + kOffScales + buf * kScBytes + r0 * 16);
        }
    }
}

template <int LAYOUT, bool QFP8, bool OUT_BF16, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int kLoads = kLoadsRaw + (LAYOUT == 1 ? 1 : 0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const int wq = w & 3;           // QK: entries 16 wq .. +16 of the tile
    const int hq = w >> 2;          // QK: dims half hq (256 dims)
    const int n_hb = (a.H + kHB - 1) / kHB;
    const int units = a.T * n_hb;

    // XCD-aware numbering: unit u's splits are blocks 8k + (u % 8)
    const int x = blockIdx.x & 7;
    const int kq = blockIdx.x >> 3;
    const int split = kq % a.n_splits;
    const int unit = (kq / a.n_splits) * 8 + x;
    if (unit >= units) return;
    const int hb = unit % n_hb;
    const int t = unit / n_hb;
    const int h = hb * kHB + c;
    const bool h_ok = h < a.H;

    int32_t *slots = reinterpret_cast<int32_t *>(lds + kOffSlots);
    float *p_lds = reinterpret_cast<float *>(lds + kOffP);    // [16 heads][64 entries]
    float *sp_lds = reinterpret_cast<float *>(lds + kOffP);   // [8 waves][16 heads][16 entries]
    float *red_m = reinterpret_cast<float *>(lds + kOffRedM);
    float *red_l = reinterpret_cast<float *>(lds + kOffRedL);

    const int seq = a.token_seq ? a.token_seq[t] : t;
    const bool seq_ok = (a.page_table == nullptr && a.seq_lens == nullptr) ||
                        (seq >= 0 && seq < a.num_seqs);
    const int seq_len = (a.seq_lens && seq_ok) ? a.seq_lens[seq] : INT_MAX;
    const int begin = split * a.split_len;
    const int n_ent = min(a.K - begin, a.split_len);   // a multiple of 64
    const int n_tiles = n_ent / kTile;

    // Query of head c, dims half hq, as the B operand:
    // bq[kk] = q[h][(8 hq + kk)*32 + g*8 .. +8].
    bf16x8 bq[8];
    float sscale = a.softmax_scale * kLog2e;
    if (QFP8) {
        sscale *= *a.q_scale;
        const uint8_t *qp = reinterpret_cast<const uint8_t *>(a.q) +
                            ((int64_t)t * a.H + (h_ok ? h : 0)) * kD + hq * 256 + g * 8;
#pragma unroll
        for (int kk = 0; kk < 8; kk++) {
            u32x2 v = h_ok ? *reinterpret_cast<const u32x2 *>(qp + kk * 32) : u32x2{0, 0};
            bq[kk] = e4m3x8_to_bf16(v[0], v[1]);
        }
    } else {
        const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) +
                           ((int64_t)t * a.H + (h_ok ? h : 0)) * kD + hq * 256 + g * 8;
#pragma unroll
        for (int kk = 0; kk < 8; kk++) {
            u32x4 v = h_ok ? *reinterpret_cast<const u32x4 *>(qp + kk * 32)
                           : u32x4{0, 0, 0, 0};
            bq[kk] = __builtin_bit_cast(bf16x8, v);
        }
    }
    // ---- prologue: resolve this split's indices into LDS.  Every load is
    // unconditional (addresses clamped into range, results selected after),
    // so each phase issues all its loads before a single wait.
    {
        constexpr int kPer = kMaxSplit / kThreads;
        const int32_t *tk = a.topk + (int64_t)t * a.K + begin;
        int32_t v[kPer], phys[kPer];
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            const int j = tid + i * kThreads;
            const int32_t x = tk[min(j, n_ent - 1)];
            v[i] = j < n_ent ? x : -1;
        }
        if (a.page_table) {
            const int32_t *row = a.page_table + (int64_t)(seq_ok ? seq : 0) * a.max_pages;
#pragma unroll
            for (int i = 0; i < kPer; i++)
                phys[i] = row[min(max(v[i], 0) >> a.page_shift, a.max_pages - 1)];
        } else {
#pragma unroll
            for (int i = 0; i < kPer; i++) phys[i] = 0;
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
        if (i < n_tiles) issue_tile<LAYOUT>(a, lds0, slots, i * kTile, i, w, lane);

    float m_run = -INFINITY, l_part = 0.0f;
    f32x4 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; dt++) acc[dt] = f32x4{0, 0, 0, 0};

    for (int it = 0; it < n_tiles; it++) {
        const int buf = it % kNBuf;
        const uint8_t *xb = lds + buf * kBufBytes;
        const f32x4 *scb = reinterpret_cast<const f32x4 *>(lds + kOffScales + buf * kScBytes);
        const int32_t *ts = slots + it * kTile;

        // (A) this tile's rows have landed (for this wave), then for all
        const int ahead = min(kNBuf - 2, n_tiles - 1 - it);
        if (ahead >= 2) wait_vm_lgkm0<2 * kLoads>();
        else if (ahead == 1) wait_vm_lgkm0<kLoads>();
        else wait_vm_lgkm0<0>();
        barrier_raw();
        if (it + kNBuf - 1 < n_tiles)
            issue_tile<LAYOUT>(a, lds0, slots, (it + kNBuf - 1) * kTile,
                               (it + kNBuf - 1) % kNBuf, w, lane);

        // (B) partial S^T for entries 16 wq .. +16 over dims half hq
        {
            const int r = 16 * wq + c;
            const uint8_t *xr = xb + r * 512 + (g & 1) * 8;
            const int sw = swz(r);
            u32x2 xa[8];
#pragma unroll
            for (int kk = 0; kk < 8; kk++)
                xa[kk] = *reinterpret_cast<const u32x2 *>(
                    xr + ((((8 * hq + kk) * 2 + (g >> 1)) ^ sw) * 16));
            f32x4 sc4[4];
            if constexpr (LAYOUT == 1) {
#pragma unroll
                for (int i = 0; i < 4; i++) sc4[i] = scb[16 * wq + 4 * g + i];
            }
            f32x4 accg[2];
            accg[0] = accg[1] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < 8; kk++) {
                const bf16x8 av = e4m3x8_to_bf16(xa[kk][0], xa[kk][1]);
                // raw rows: two independent chains (even / odd kk); scaled
                // rows: one chain per 128-wide scale group of this half
                const int q = LAYOUT == 0 ? (kk & 1) : (kk >> 2);
                accg[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[kk], accg[q], 0, 0, 0);
            }
            f32x4 part;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if constexpr (LAYOUT == 0)
                    part[i] = accg[0][i] + accg[1][i];
                else
                    part[i] = accg[0][i] * sc4[i][2 * hq] + accg[1][i] * sc4[i][2 * hq + 1];
            }
            *reinterpret_cast<f32x4 *>(sp_lds + (w * kHB + c) * 16 + 4 * g) = part;
        }
        wait_lgkm0();
        barrier_raw();

        // (C) full scores of entries 16 wq + 4g + i, head c; tile max
        float sv[4];
        {
            const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sp_lds + (wq * kHB + c) * 16 + 4 * g);
            const f32x4 s1 = *reinterpret_cast<const f32x4 *>(sp_lds + ((wq + 4) * kHB + c) * 16 + 4 * g);
            const int4 sl4 = *reinterpret_cast<const int4 *>(ts + 16 * wq + 4 * g);
            const int slv[4] = {sl4.x, sl4.y, sl4.z, sl4.w};
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                sv[i] = slv[i] >= 0 ? (s0[i] + s1[i]) * sscale : -INFINITY;
                mx = fmaxf(mx, sv[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (g == 0 && w < 4) red_m[w * kHB + c] = mx;
        }
        wait_lgkm0();
        barrier_raw();

        // (D) shared tile max and probabilities.  The running reference max
        // only moves when the tile max exceeds it by more than kSlack (log2
        // units), so the O rescale is rare; P = 2^(s - m_ref) <= 2^kSlack.
        // All waves see the same maxima and so make the same choice.  Waves
        // 0-3 own the entries' P and their share of the denominator.
        {
            const float tmax = fmaxf(fmaxf(red_m[c], red_m[kHB + c]),
                                     fmaxf(red_m[2 * kHB + c], red_m[3 * kHB + c]));
            const bool resc = tmax - m_run > kSlack;   // false when both are -inf
            const float alpha = resc ? exp2f(m_run - tmax) : 1.0f;
            if (resc) m_run = tmax;
            if (w < 4) {
                f32x4 p;
                float ps = 0.0f;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    p[i] = sv[i] == -INFINITY ? 0.0f : exp2f(sv[i] - m_run);
                    ps += p[i];
                }
                l_part = l_part * alpha + ps;
                *reinterpret_cast<f32x4 *>(p_lds + c * kTile + 16 * w + 4 * g) = p;
            }
            if (__ballot(resc)) {
#pragma unroll
                for (int dt = 0; dt < 4; dt++) acc[dt] *= alpha;
            }
        }
        wait_lgkm0();
        barrier_raw();

        // (E) O^T[dims 64w.., heads] += X^T . P^T over the 64 entries.
        {
            // B operand P^T: entries ks*32 + g*8 + r of head c
            f32x4 pr[4];
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                pr[2 * ks] = *reinterpret_cast<const f32x4 *>(p_lds + c * kTile + ks * 32 + g * 8);
                pr[2 * ks + 1] = *reinterpret_cast<const f32x4 *>(p_lds + c * kTile + ks * 32 + g * 8 + 4);
            }
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
            float pv[2][8];
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    pv[ks][r] = pr[2 * ks][r];
                    pv[ks][4 + r] = pr[2 * ks + 1][r];
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
                for (int ks = 0; ks < 2; ks++)
#pragma unroll
                    for (int r = 0; r < 8; r++) pv[ks][r] *= sc[ks][r] * inv;
            }
            f16x8 bp[2];
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int r = 0; r < 8; r++) bp[ks][r] = (_Float16)pv[ks][r];
#pragma unroll
            for (int dt = 0; dt < 4; dt++) {
                if constexpr (LAYOUT == 0) {
#pragma unroll
                    for (int ks = 0; ks < 2; ks++)
                        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            e4m3x8_to_f16(tv[ks][dt][0], tv[ks][dt][1]), bp[ks], acc[dt], 0, 0, 0);
                } else {
                    f32x4 part = {0, 0, 0, 0};
#pragma unroll
                    for (int ks = 0; ks < 2; ks++)
                        part = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            e4m3x8_to_f16(tv[ks][dt][0], tv[ks][dt][1]), bp[ks], part, 0, 0, 0);
                    acc[dt] += part * smax;
                }
            }
        }
    }

    // total softmax denominator per head: lanes of this wave, then waves 0-3
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
    if (g == 0 && w < 4) red_l[w * kHB + c] = l_part;
    __syncthreads();
    const float l_tot = red_l[c] + red_l[kHB + c] + red_l[2 * kHB + c] + red_l[3 * kHB + c];
    if (!h_ok) return;

    const int64_t th = (int64_t)t * a.H + h;
    if (SPLIT) {
        float *wo = a.ws + (th * a.n_splits + split) * kD + 64 * w + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) *reinterpret_cast<f32x4 *>(wo + dt * 16) = acc[dt];
        if (w == 0 && g == 0) {
            float *ml = a.ws + (int64_t)a.T * a.H * a.n_splits * kD +
                        (th * a.n_splits + split) * 2;
            ml[0] = m_run;
            ml[1] = l_tot;
        }
    } else {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int64_t base = th * kD + 64 * w + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 4; dt++) {
            const f32x4 o = acc[dt] * inv;
            if (OUT_BF16) {
                u32x2 pk = {f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16),
                            f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16)};
                *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + base + dt * 16) = pk;
            } else {
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + base + dt * 16) = o;
            }
        }
        if (a.lse && w == 0 && g == 0)
            a.lse[th] = l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
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
    float L = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < S; s++) {
            const float ms = ml[2 * s];
            if (ms == -INFINITY) continue;
            const float wgt = exp2f(ms - M);
            L += wgt * ml[2 * s + 1];
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
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
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
    if (a.lse && lane == 0) a.lse[th] = L > 0.0f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

// Splits per (token, head block): enough workgroups to cover the CUs for
// small batches, and never more than kMaxSplit entries per workgroup.
int attn_decode_splits(int T, int H, int K) {
    const int64_t units = (int64_t)T * ((H + kHB - 1) / kHB);
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

template <typename K>
static void allow_big_lds(K kern) {
    // once per instantiation; not a stream operation, so capture-safe
    static const hipError_t e = hipFuncSetAttribute(
        (const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    (void)e;
}

template <int LAYOUT, bool QFP8, bool OUT_BF16>
static hipError_t launch_one(const AttnArgs &a, hipStream_t stream) {
    const int n_hb = (a.H + kHB - 1) / kHB;
    const int64_t units = (int64_t)a.T * n_hb;
    const dim3 grid((unsigned)(((units + 7) / 8) * 8 * a.n_splits));
    if (a.n_splits > 1) {
        auto kern = attn_kernel<LAYOUT, QFP8, OUT_BF16, true>;
        allow_big_lds(kern);
        kern<<<grid, dim3(kThreads), kLdsBytes, stream>>>(a);
        const dim3 cgrid((unsigned)(((int64_t)a.T * a.H + 3) / 4));
        attn_combine_kernel<OUT_BF16><<<cgrid, dim3(256), 0, stream>>>(a);
    } else {
        auto kern = attn_kernel<LAYOUT, QFP8, OUT_BF16, false>;
        allow_big_lds(kern);
        kern<<<grid, dim3(kThreads), kLdsBytes, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs &a_in, int layout, bool q_fp8, bool out_bf16,
                       hipStream_t stream) {
    AttnArgs a = a_in;
    if (a.n_splits < 1) a.n_splits = 1;
    a.split_len = split_len_for(a.K, a.n_splits);
#define DSA_DISPATCH(L, Q, O) \
    if (layout == L && q_fp8 == Q && out_bf16 == O) return launch_one<L, Q, O>(a, stream);
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
