// attn.hip -- sparse absorbed-MLA attention over gathered FP8 pool rows.
//
// Method ("[DSA] Support flashmla_sparse_q8 prefill backend on CUDA",
// Modifications; "extend CUDA TileLang raw FP8 KV path", Motivation): every
// query token t has H heads of 512-wide latent queries and a top-k list of
// pool entries (-1 = padding); each selected 512-wide latent row is both key
// and value.  out[t,h] = softmax_j(scale * <q[t,h], x_j>) . x_j over the
// multiset of valid entries; all-masked tokens give 0 (lse = -inf).
//
// Work decomposition (one workgroup = 4 wavefronts):
//   * a workgroup owns (token t, block of 16 heads, one split of the list);
//     all 16 heads share every gathered row, so Q.X^T is a real
//     [16 x 512] x [512 x entries] contraction for the matrix cores;
//   * per tile of 64 entries: resolve indices -> byte offsets (int64), gather
//     the 64 rows (512 or 528 B each) with 16-byte loads into LDS, then
//       - wave w computes S^T for entries [16w, 16w+16) with
//         v_mfma_f32_16x16x32_bf16 (rows converted FP8 -> bf16 exactly,
//         bf16 query; an FP8 query is converted exactly as well and its
//         scale folded into the score scale);
//       - the four waves agree on the tile's max per head through LDS, form
//         p = 2^(s - m) (log2e folded into the scale) and publish P;
//       - wave w accumulates O^T for dims [128w, 128w+128) over all 64
//         entries with v_mfma_f32_16x16x32_f16 (FP8 -> f16 exact; P rounded
//         to f16).  For 528-byte rows the per-row group scale is applied to
//         the QK partial sums of each 128-wide group and, in PV, to P
//         (wave w's 128 dims are exactly scale group w).
//   * decode splits the list over several workgroups and writes unnormalised
//     partial (o, m, l) states that a second kernel merges; prefill writes
//     the normalised output directly.
//
// MFMA operand layouts used (64 lanes; c = lane % 16, g = lane / 16):
//   A (16 x K): lane (c, g) holds row c, B (K x 16): lane (c, g) holds
//   column c; both hold the same 8 reduction indices for a given g and
//   register slot, which is all a contraction needs, so the reduction index
//   is assigned freely: dims kk*32 + g*8 + r for QK, entries ks*32 + g*8 + r
//   for PV.  The 16x16 result: lane (c, g) holds rows 4g..4g+3 of column c.
#include <limits.h>

#include "common.h"
#include "launch.h"

#ifndef DSA_DECODE_TARGET_BLOCKS
#define DSA_DECODE_TARGET_BLOCKS 1024
#endif

namespace dsa {

constexpr int kThreads = 256;
constexpr int kHB = 16;         // heads per workgroup
constexpr int kTile = 64;       // entries per tile
constexpr int kXStride = 528;   // LDS bytes between staged rows
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Smem {
    uint8_t x[kTile * kXStride];
    float p[kHB][kTile];
    f32x4 scales[kTile];
    int64_t off[kTile];
    float red_m[4][kHB];
    float red_l[4][kHB];
};

// Index resolution: -1 -> padding; other invalid values -> masked + error.
__device__ __forceinline__ int64_t resolve_entry(const AttnArgs &a, int32_t i,
                                                 int seq, bool seq_ok,
                                                 int seq_len, bool &err) {
    err = false;
    if (i == -1) return -1;
    if (i < 0 || !seq_ok || i >= seq_len) {
        err = true;
        return -1;
    }
    int64_t slot;
    if (a.page_table) {
        const int page = i >> a.page_shift;
        if (page >= a.max_pages) {
            err = true;
            return -1;
        }
        const int32_t phys = a.page_table[(int64_t)seq * a.max_pages + page];
        if (phys < 0) {
            err = true;
            return -1;
        }
        slot = ((int64_t)phys << a.page_shift) | (int64_t)(i & ((1 << a.page_shift) - 1));
    } else {
        slot = i;
    }
    if (slot >= a.num_slots) {
        err = true;
        return -1;
    }
    return slot;
}

template <int LAYOUT, bool QFP8, bool OUT_BF16, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
    __shared__ Smem sm;
    constexpr int64_t kRow = LAYOUT == 0 ? kRawBytes : kScaledBytes;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int c = lane & 15, g = lane >> 4;
    const int n_hb = (a.H + kHB - 1) / kHB;

    int bid = blockIdx.x;
    const int split = bid % a.n_splits;
    bid /= a.n_splits;
    const int hb = bid % n_hb;
    const int t = bid / n_hb;
    const int h = hb * kHB + c;
    const bool h_ok = h < a.H;

    const int seq = a.token_seq ? a.token_seq[t] : t;
    const bool seq_ok = (a.page_table == nullptr && a.seq_lens == nullptr) ||
                        (seq >= 0 && seq < a.num_seqs);
    const int seq_len = (a.seq_lens && seq_ok) ? a.seq_lens[seq] : INT_MAX;

    // Query of head c as the B operand: bq[kk] = q[h][kk*32 + g*8 .. +8].
    bf16x8 bq[16];
    float sscale = a.softmax_scale * kLog2e;
    if (QFP8) {
        sscale *= *a.q_scale;
        const uint8_t *qp = reinterpret_cast<const uint8_t *>(a.q) +
                            ((int64_t)t * a.H + (h_ok ? h : 0)) * kD + g * 8;
#pragma unroll
        for (int kk = 0; kk < 16; kk++) {
            u32x2 v = h_ok ? *reinterpret_cast<const u32x2 *>(qp + kk * 32) : u32x2{0, 0};
            bq[kk] = e4m3x8_to_bf16(v[0], v[1]);
        }
    } else {
        const __bf16 *qp = reinterpret_cast<const __bf16 *>(a.q) +
                           ((int64_t)t * a.H + (h_ok ? h : 0)) * kD + g * 8;
#pragma unroll
        for (int kk = 0; kk < 16; kk++) {
            u32x4 v = h_ok ? *reinterpret_cast<const u32x4 *>(qp + kk * 32)
                           : u32x4{0, 0, 0, 0};
            bq[kk] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const int begin = split * a.split_len;
    const int end = min(a.K, begin + a.split_len);
    float m_run = -INFINITY, l_part = 0.0f;
    f32x4 acc[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++) acc[dt] = f32x4{0, 0, 0, 0};

    for (int tb = begin; tb < end; tb += kTile) {
        // (1) resolve the tile's indices to row byte offsets
        if (tid < kTile) {
            const int j = tb + tid;
            int64_t slot = -1;
            bool err = false;
            if (j < end)
                slot = resolve_entry(a, a.topk[(int64_t)t * a.K + j], seq, seq_ok,
                                     seq_len, err);
            sm.off[tid] = slot < 0 ? (int64_t)-1 : slot * kRow;
            if (a.err_count && hb == 0) {
                const uint64_t bal = __ballot(err);
                if (lane == 0 && bal) atomicAdd(a.err_count, (int)__popcll(bal));
            }
        }
        __syncthreads();

        // (2) gather 64 rows into LDS; masked rows are zero so that P = 0
        // never meets a NaN from an unreferenced slot.
        {
            const int cch = tid & 31, r0 = tid >> 5;
            u32x4 v[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int64_t off = sm.off[r0 + 8 * i];
                v[i] = off >= 0 ? *reinterpret_cast<const u32x4 *>(a.pool + off + cch * 16)
                                : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < 8; i++)
                *reinterpret_cast<u32x4 *>(sm.x + (r0 + 8 * i) * kXStride + cch * 16) = v[i];
            if (LAYOUT == 1 && tid < kTile) {
                const int64_t off = sm.off[tid];
                sm.scales[tid] = off >= 0 ? *reinterpret_cast<const f32x4 *>(a.pool + off + kD)
                                          : f32x4{0, 0, 0, 0};
            }
        }
        __syncthreads();

        // (3) S^T for this wave's 16 entries
        float sv[4];
        {
            const uint8_t *xr = sm.x + (16 * w + c) * kXStride + g * 8;
            f32x4 accg[4];
#pragma unroll
            for (int q = 0; q < 4; q++) accg[q] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < 16; kk++) {
                const u32x2 wv = *reinterpret_cast<const u32x2 *>(xr + kk * 32);
                const bf16x8 av = e4m3x8_to_bf16(wv[0], wv[1]);
                const int q = LAYOUT == 0 ? 0 : (kk >> 2);
                accg[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[kk], accg[q], 0, 0, 0);
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int e = 16 * w + 4 * g + i;
                float s;
                if constexpr (LAYOUT == 0) {
                    s = accg[0][i];
                } else {
                    const f32x4 sc = sm.scales[e];
                    s = accg[0][i] * sc[0] + accg[1][i] * sc[1] + accg[2][i] * sc[2] +
                        accg[3][i] * sc[3];
                }
                sv[i] = sm.off[e] >= 0 ? s * sscale : -INFINITY;
                mx = fmaxf(mx, sv[i]);
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (g == 0) sm.red_m[w][c] = mx;
        }
        __syncthreads();

        // (4) shared tile max, probabilities, rescale
        {
            const float tmax = fmaxf(fmaxf(sm.red_m[0][c], sm.red_m[1][c]),
                                     fmaxf(sm.red_m[2][c], sm.red_m[3][c]));
            const float m_new = fmaxf(m_run, tmax);
            const float alpha = m_new == -INFINITY ? 1.0f : exp2f(m_run - m_new);
            f32x4 p;
            float ps = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p[i] = sv[i] == -INFINITY ? 0.0f : exp2f(sv[i] - m_new);
                ps += p[i];
            }
            l_part = l_part * alpha + ps;
            m_run = m_new;
            *reinterpret_cast<f32x4 *>(&sm.p[c][16 * w + 4 * g]) = p;
#pragma unroll
            for (int dt = 0; dt < 8; dt++) acc[dt] *= alpha;
        }
        __syncthreads();

        // (5) O^T[dims 128w.., heads] += X^T . P^T over the 64 entries
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
            const int e0 = ks * 32 + g * 8;
            const f32x4 p0 = *reinterpret_cast<const f32x4 *>(&sm.p[c][e0]);
            const f32x4 p1 = *reinterpret_cast<const f32x4 *>(&sm.p[c][e0 + 4]);
            float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            if (LAYOUT == 1) {
#pragma unroll
                for (int r = 0; r < 8; r++) pv[r] *= sm.scales[e0 + r][w];
            }
            f16x8 bp;
#pragma unroll
            for (int r = 0; r < 8; r++) bp[r] = (_Float16)pv[r];
            const uint8_t *col = sm.x + e0 * kXStride + 128 * w + c;
#pragma unroll
            for (int dt = 0; dt < 8; dt++) {
                const uint8_t *cp = col + dt * 16;
                const uint32_t b0 = (uint32_t)cp[0] | ((uint32_t)cp[kXStride] << 8) |
                                    ((uint32_t)cp[2 * kXStride] << 16) |
                                    ((uint32_t)cp[3 * kXStride] << 24);
                const uint32_t b1 = (uint32_t)cp[4 * kXStride] |
                                    ((uint32_t)cp[5 * kXStride] << 8) |
                                    ((uint32_t)cp[6 * kXStride] << 16) |
                                    ((uint32_t)cp[7 * kXStride] << 24);
                const f16x8 av = e4m3x8_to_f16(b0, b1);
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bp, acc[dt], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // total softmax denominator per head: lanes of this wave, then waves
    l_part += __shfl_xor(l_part, 16);
    l_part += __shfl_xor(l_part, 32);
    if (g == 0) sm.red_l[w][c] = l_part;
    __syncthreads();
    const float l_tot = sm.red_l[0][c] + sm.red_l[1][c] + sm.red_l[2][c] + sm.red_l[3][c];
    if (!h_ok) return;

    const int64_t th = (int64_t)t * a.H + h;
    if (SPLIT) {
        float *wo = a.ws + (th * a.n_splits + split) * kD + 128 * w + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) *reinterpret_cast<f32x4 *>(wo + dt * 16) = acc[dt];
        if (w == 0 && g == 0) {
            float *ml = a.ws + (int64_t)a.T * a.H * a.n_splits * kD +
                        (th * a.n_splits + split) * 2;
            ml[0] = m_run;
            ml[1] = l_tot;
        }
    } else {
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        const int64_t base = th * kD + 128 * w + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
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

int attn_decode_splits(int T, int H, int K) {
    const int64_t units = (int64_t)T * ((H + kHB - 1) / kHB);
    const int tiles = K / kTile;
    if (units <= 0 || tiles <= 0) return 1;
    int64_t s = (DSA_DECODE_TARGET_BLOCKS + units - 1) / units;
    if (s < 1) s = 1;
    if (s > tiles) s = tiles;
    const int tps = (int)((tiles + s - 1) / s);
    return (tiles + tps - 1) / tps;
}

static int split_len_for(int K, int splits) {
    const int tiles = K / kTile;
    return ((tiles + splits - 1) / splits) * kTile;
}

size_t attn_workspace_bytes(int T, int H, int K, int phase) {
    if (phase != 0) return 0;
    const int s = attn_decode_splits(T, H, K);
    if (s <= 1) return 0;
    size_t b = (size_t)T * H * s * (kD + 2) * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

template <int LAYOUT, bool QFP8, bool OUT_BF16>
static void launch_one(const AttnArgs &a, hipStream_t stream) {
    const int n_hb = (a.H + kHB - 1) / kHB;
    const dim3 grid((unsigned)((int64_t)a.T * n_hb * a.n_splits));
    if (a.n_splits > 1) {
        attn_kernel<LAYOUT, QFP8, OUT_BF16, true><<<grid, dim3(kThreads), 0, stream>>>(a);
        const dim3 cgrid((unsigned)(((int64_t)a.T * a.H + 3) / 4));
        attn_combine_kernel<OUT_BF16><<<cgrid, dim3(256), 0, stream>>>(a);
    } else {
        attn_kernel<LAYOUT, QFP8, OUT_BF16, false><<<grid, dim3(kThreads), 0, stream>>>(a);
    }
}

hipError_t launch_attn(const AttnArgs &a_in, int layout, bool q_fp8, bool out_bf16,
                       hipStream_t stream) {
    AttnArgs a = a_in;
    if (a.n_splits < 1) a.n_splits = 1;
    a.split_len = split_len_for(a.K, a.n_splits);
#define DSA_DISPATCH(L, Q, O) \
    if (layout == L && q_fp8 == Q && out_bf16 == O) launch_one<L, Q, O>(a, stream);
    DSA_DISPATCH(0, false, false)
    DSA_DISPATCH(0, false, true)
    DSA_DISPATCH(0, true, false)
    DSA_DISPATCH(0, true, true)
    DSA_DISPATCH(1, false, false)
    DSA_DISPATCH(1, false, true)
    DSA_DISPATCH(1, true, false)
    DSA_DISPATCH(1, true, true)
#undef DSA_DISPATCH
    return hipGetLastError();
}

}  // namespace dsa
