// attn.hip -- sparse absorbed-MLA attention over gathered FP8 pool rows.
//
// Method ("[DSA] Support flashmla_sparse_q8 prefill backend on CUDA",
// Modifications; "extend CUDA TileLang raw FP8 KV path", Motivation): every
// query token t has H heads of 512-wide latent queries and a top-k list of
// pool entries (-1 = padding); each selected 512-wide latent row is both key
// and value.  out[t,h] = softmax_j(scale * <q[t,h], x_j>) . x_j over the
// multiset of valid entries; all-masked tokens give 0 (lse = -inf).
//
// Work decomposition: one workgroup owns one unit = (token t, block of heads)
// and one split of t's top-k list (at most 2048 entries).  All heads of the
// block share every gathered row, so Q.X^T is a real [heads x 512] x
// [512 x entries] contraction for the matrix cores, and a row is gathered
// once per block.  attn_kernel (16 wavefronts, 4 per SIMD, 128 registers)
// takes blocks of 16 heads, for every row layout; attn_w8_kernel further
// down (8 wavefronts, 256 registers) takes blocks of 32 heads over raw rows,
// the form used when there are more than 16 heads.  The outline below is
// attn_kernel's.
//
//   prologue: the split's indices are resolved once (top-k value -> page
//     table -> slot; -1 for padding and for invalid values, which are also
//     counted) into LDS, as each entry's 64-bit row address (a zero row for
//     a masked entry); the token's page-table row is staged in LDS next to
//     the top-k loads when it fits;
//   gather:   rows move HBM -> LDS with global_load_lds_dwordx4 (16 bytes per
//     lane, no registers) in 64-row tiles through up to 4 LDS buffers.
//     Every wave copies the operands it needs from a landed tile into
//     registers at once, so a buffer is refilled as soon as all waves hold
//     their copy.  The 16-byte chunks of row r are stored XOR-swizzled by
//     (r & 15) so that the matrix-operand reads spread over the LDS banks;
//     masked entries read zero rows;
//   QK^T:     waves 0-7 form 16 x 16 partial S^T blocks: 16 entries, one head
//     tile, one 256-dim half of the dims.  bf16 query:
//     v_mfma_f32_16x16x32_bf16 on rows converted FP8 -> bf16 exactly (exact
//     products, fp32 sums); FP8 query: v_mfma_scale_f32_16x16x128_f8f6f4 on
//     the codes themselves (unit block scales), the query scale folded into
//     the score scale;
//   softmax:  the owner of an (entry quarter, head tile) adds the other
//     half's partial (through LDS), keeps its own running maximum per head
//     (log2 domain, moved only when exceeded by more than kSlack, so
//     P <= 2^kSlack) and publishes P (f16; bf16 for bf16 rows) and its
//     maximum;
//   PV:       waves 8-15 accumulate O^T for 64 dims each over the 64 entries
//     with v_mfma_f32_16x16x32_f16, against a per-head reference maximum
//     that tracks the largest quarter maximum; P of quarter q is weighted by
//     2^(m_q - m_ref) <= 1 on the way into the f16 operand.  The A operand
//     (8 entries x 1 dim per lane) comes from the row-major tile through the
//     gfx950 LDS transpose read ds_read_b64_tr_b8.  Group-scaled rows scale
//     the QK partial sums per 128-wide group and multiply P by each entry's
//     scale over the running largest scale of its group;
//   schedule: PV runs one tile behind QK, the next tile's operands are read
//     from LDS while the owners' softmax and the PV run; two barriers per
//     tile;
//   epilogue: normalised output + lse, or (several splits) the normalised
//     fp32 output and (m, l) of each split, which a second kernel merges.
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

#include <type_traits>

// This file is compiled without NaN semantics (-fno-honor-nans): its scores
// are finite, -inf for masked entries, and the running maxima start at the
// finite kNoMax, so maxima need no NaN quieting.  The encoders in common.h,
// which test for NaN, are not used here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wnan-infinity-disabled"
#include "common.h"
#pragma clang diagnostic pop
#include "launch.h"

namespace dsa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;          // entries per tile
constexpr int kNBuf = 4;           // LDS tile buffers (all four in flight)
constexpr int kNScale = 6;         // scale-word buffers (outlive their tile's rows)
constexpr int kMaxSplit = 2048;    // entries per workgroup at most
constexpr int kRowsPerWave = kTile / kWaves;        // DMA share of a tile (4 rows)
constexpr int kLoadsRaw = kRowsPerWave / 2;         // DMA instructions per wave per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;     // log2 headroom of a running max (P <= 256)
// "No maximum yet": finite, so that 2^(-inf - kNoMax) = 0 for masked scores
// without a select, and far below any real score.
constexpr float kNoMax = -1.0e30f;

// LDS map (bytes) for NT head tiles of 16 and a row layout.  656-byte rows
// add a ring of RoPE parts (64 rows x 128 B per tile) and, to stay within the
// 160 KB of a CU, keep three tile buffers instead of four; 1024-byte bf16
// rows keep two buffers of 64 KB.
template <int LAYOUT>
struct Lds {
    static constexpr int kHB = 16;
    static constexpr int kNB = LAYOUT == 2 ? 3 : LAYOUT == 3 ? 2 : kNBuf;   // tile buffers
    static constexpr int kParts = 2;                             // QK dim parts
    static constexpr int kRowPitch = LAYOUT == 3 ? 1024 : 512;   // LDS bytes per row
    static constexpr int kBufBytes = kTile * kRowPitch;          // 32 KB (bf16 rows: 64 KB)
    static constexpr bool kHasScales = LAYOUT == 1 || LAYOUT == 2;
    // raw FP8 rows carry P to the PV product as two f16 terms (hi + lo),
    // see the softmax
    static constexpr bool kLo = LAYOUT == 0;
    static constexpr int kScBytes = kTile * 16;                  // 1 KB scales
    static constexpr int kRopeTile = kTile * 2 * kRopeDim;       // 8 KB RoPE parts
    static constexpr int kOffScales = kNB * kBufBytes;
    // the entries' row sources (64-bit addresses, see kMaskBits)
    static constexpr int kOffSlots = kOffScales + (kHasScales ? kNScale * kScBytes : 0);
    // partial S^T of the waves holding dim parts 1.. (16 x 16 fp32 each)
    static constexpr int kOffSp = kOffSlots + kMaxSplit * 8;
    static constexpr int kSpBytes = (kParts - 1) * 4 * 1024;
    // P ([kHB][64] 16-bit, swizzled; the lo terms follow the hi terms): one
    // buffer, since the PV waves hold tile k's P in registers before the
    // barrier after which the owners write tile k+1's; then the quarter
    // maxima ([kHB][4] fp32), two (by tile parity: each owner reads the
    // previous tile's while it writes its own)
    static constexpr int kOffP = kOffSp + kSpBytes;
    static constexpr int kPBytes = kHB * kTile * 2;
    static constexpr int kPArea = (kLo ? 2 : 1) * kPBytes;
    static constexpr int kOffMq = kOffP + kPArea;
    static constexpr int kMqBytes = kHB * 16;
    static constexpr int kOffRedL = kOffMq + 2 * kMqBytes;       // [kHB][4] fp32
    // group-scaled rows: running largest scale of each 128-wide group (the
    // PV operand's reference), two tiles (by parity)
    static constexpr int kOffSmax = kOffRedL + kHB * 16;
    // per head and quarter: 1 when the quarter's maximum did not move this
    // tile (then it equals the reference maximum), two tiles (by parity)
    static constexpr int kOffFlags = kOffSmax + 2 * 16;
    // group-scaled rows: f16 factor scale / reference of each entry and
    // group ([4][64]), two tiles (by parity)
    static constexpr int kOffFac = kOffFlags + 2 * kHB * 4;
    static constexpr int kFacBytes = 4 * kTile * 2;
    static constexpr int kOffRope = kOffFac + (LAYOUT == 1 || LAYOUT == 2 ? 2 * kFacBytes : 0);
    static constexpr int kBytes = kOffRope + (LAYOUT == 2 ? kNB * kRopeTile : 0);
    // the token's page-table row is staged over the sp and P areas
    static constexpr int kPtPer = (kSpBytes + kPArea) / 4 / kThreads;
    static_assert(kBytes <= 160 * 1024, "LDS budget");
    static_assert(kOffRope % 16 == 0 && kOffScales % 16 == 0, "16-byte DMA destinations");
    static_assert(kPtPer >= 1, "page-table staging");
};

// Masked entries read zeros (P = 0 must never meet a NaN of an unreferenced
// slot).  64 distinct zero rows, picked by the tile row, keep these reads off
// a single set of L2 lines.
constexpr int kZeroRows = 64;
__device__ __attribute__((aligned(16))) const uint8_t kZeroRow[kZeroRows * kBf16RowBytes] = {};

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

// Reductions over the four lanes c, c+16, c+32, c+48 (the 16-lane groups g)
// with the gfx950 cross-half lane swaps (no LDS traffic): v_permlane32_swap
// exchanges the upper half of its first operand with the lower half of its
// second, v_permlane16_swap the odd 16-lane rows of the first with the even
// rows of the second; with both operands equal, the two results hold lanes l
// and l ^ 32 (resp. l ^ 16).
// Maximum over all 64 lanes: within each 16-lane row through DPP (quad
// permutations, then the half-row and row mirrors), then across rows.
__device__ __forceinline__ float dpp_max16(float v) {
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));  // quad [1,0,3,2]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));  // quad [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true))); // half-row mirror
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true))); // row mirror
    return v;
}

__device__ __forceinline__ float max_over_g(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Two fp32 values as packed bf16 (low half first), rounded to nearest even
// by gfx950's v_cvt_pk_bf16_f32: bit for bit the rounding of
// f32_to_bf16_bits (a device probe compared them over every exponent and
// sign with ties and near-ties in the low half), NaN staying NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// The maxima over g of two values at once: the first swap pairs the lanes
// l, l ^ 32 of a in lanes 0-31 and those of b in lanes 32-63, the second the
// 16-lane rows, the third hands every lane both results.
__device__ __forceinline__ void max_over_g2(float &a, float &b) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    float v = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
    const auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
    const auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    a = __uint_as_float(u[0]);
    b = __uint_as_float(u[1]);
}
__device__ __forceinline__ float sum_over_g(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// LDS bank spreading.  A 16-byte-per-lane access serves 16 lanes at a time
// over the 64 four-byte banks (256 bytes), so the 16 rows c = 0..15 that
// such an access touches must land on 16 distinct 16-byte positions of a
// 256-byte period: the chunks of a row (512-byte pitch) are XOR-swizzled by
// row & 15 (measured against row & 7: half the bank-conflict cycles, Q8
// prefill -2.5 %).  1024-byte bf16 rows keep row & 7 (their 2-byte PV reads
// would otherwise not fit the registers), and so does the 8-chunk ring of
// RoPE parts.
template <int LAYOUT>
__device__ __forceinline__ int swz(int row) { return LAYOUT == 3 ? row & 7 : row & 15; }
__device__ __forceinline__ int swz8(int row) { return row & 7; }

// The partial-score rows ([head][4 entry groups of 4], 64 bytes) rotate
// their groups by c >> 2, so that the 16 lanes c of a 16-byte access fall on
// distinct banks.
__device__ __forceinline__ int sp_slot(int grp, int c) { return (grp + (c >> 2)) & 3; }

// Byte offset of the 16-byte P chunk k (entries 8k .. 8k+7) of head row hh:
// rows of 128 bytes, chunks XOR-swizzled by (hh >> 1) & 7 (rows hh and hh + 2
// share banks; 16 consecutive rows cover them once).
__device__ __forceinline__ int p_off(int hh, int k) { return hh * 128 + ((k ^ ((hh >> 1) & 7)) << 4); }

// 32-bit LDS address of a pointer into dynamic shared memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)LDS_PTR(p);
}

// One 16-byte-per-lane HBM -> LDS copy: lane l's 16 bytes land at
// lds_base + 16 l.  Issued through inline assembly so that the compiler does
// not see pending LDS writes: it would otherwise guard every later LDS read
// with a wait for all outstanding loads.  Completion is tracked explicitly
// with s_waitcnt vmcnt before the barrier that publishes a tile.  The
// compiler's hazard checks do not look inside an asm block, so the block
// carries the wait state that an LDS DMA needs after a scalar write of M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // m0 is reserved; only this asm writes it
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gptr), "s"(lds_base) : "memory", "m0");
}
// The same with 4 bytes per lane (lane l's word lands at lds_base + 4 l).
__device__ __forceinline__ void dma4(const void *gptr, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(gptr), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// bf16 outputs of a head tile's row segment.  Lane (c, g) holds, for each
// 16-dim tile dt, dims 16 dt + 4g .. +4 of head row c (o(dt), fp32).  For
// each pair of dim tiles, lanes of even g take dim tile 2m (their own 4 dims
// and those of lane g + 1), lanes of odd g dim tile 2m + 1 (those of lane
// g - 1 and their own), exchanged with one 16-lane row swap per word; a
// 16-byte store then covers 64 contiguous bytes of each of the 16 rows
// (8-byte stores of each lane's own dims: 32 bytes per row and twice the
// instructions).  row: the head row's first dim of this segment.
template <int kDT, typename F>
__device__ __forceinline__ void store_bf16_tiles(uint16_t *row, int g, F &&o) {
    static_assert(kDT % 2 == 0, "dim tiles in pairs");
#pragma unroll
    for (int m = 0; m < kDT / 2; m++) {
        const f32x4 o0 = o(2 * m), o1 = o(2 * m + 1);
        uint32_t p0[2] = {pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3])};
        uint32_t p1[2] = {pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const auto sw = __builtin_amdgcn_permlane16_swap(p0[k], p1[k], false, false);
            p0[k] = sw[0];
            p1[k] = sw[1];
        }
        const int d0 = (2 * m + (g & 1)) * 16 + 4 * (g & 2);
        *reinterpret_cast<u32x4 *>(row + d0) = u32x4{p0[0], p0[1], p1[0], p1[1]};
    }
}

// A 16- or 8-byte global store written through to device scope (sc1), so
// that the line is not left dirty in this XCD's L2 for the write-back that
// ends the kernel; the decode's split partials otherwise put that write-back
// between the attention kernel and the merge.  A cache policy only: the
// kernel boundary still orders the data for its reader.  The trailing s_nop
// is the wait state a vector store of more than 8 bytes needs before a
// vector instruction may overwrite its data registers (the compiler's hazard
// checks do not see a store inside an asm block).
template <typename V>
__device__ __forceinline__ void store_through(V *p, V v) {
    static_assert(sizeof(V) == 16 || sizeof(V) == 8, "dwordx4 or dwordx2");
    if constexpr (sizeof(V) == 16)
        asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
    else
        asm volatile("global_store_dwordx2 %0, %1, off sc1\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}

// Bytes of one pool row of a layout.
template <int LAYOUT>
constexpr int64_t row_bytes() {
    return LAYOUT == 0 ? kRawBytes : LAYOUT == 1 ? kScaledBytes : LAYOUT == 2 ? kRopeRowBytes : kBf16RowBytes;
}

// An entry's row source, resolved once in the prologue: the row's address in
// the pool, or for a masked entry the address of zero row (entry mod 64) of
// kZeroRow with the bits of an fp32 -inf (0xff800000) or-ed into its high
// word (cleared before use; the launcher checks that no pool address has any
// of them set).  The tile DMA then forms each lane's address with two
// instructions, and the softmax takes the mask term of a score (0 or -inf)
// as the high word of the source with one AND.
constexpr uint64_t kMaskBits = 0xff800000ull << 32;
__device__ __forceinline__ float mask_term(int32_t src_hi) { return __int_as_float(src_hi & (int32_t)0xff800000u); }

// Row sources of the rows this wave copies for one tile (see issue_tile).
struct TileSlots {
    uint64_t row[kLoadsRaw];
    uint64_t sc;     // the scale words' row (lanes 0-3)
    uint64_t rp;     // the RoPE part's row (lanes 0-31)
    uint64_t r4[kRowsPerWave];   // bf16 rows: the wave's rows, one per instruction
};

template <int LAYOUT>
__device__ __forceinline__ TileSlots read_slots(const uint64_t *slots, int tile_base, int w, int lane) {
    TileSlots s;
    const int r0 = kRowsPerWave * w;
#pragma unroll
    for (int k = 0; k < kLoadsRaw; k++) s.row[k] = slots[tile_base + r0 + 2 * k + (lane >> 5)];
    s.sc = (LAYOUT == 1 || LAYOUT == 2) ? slots[tile_base + r0 + (lane & (kRowsPerWave - 1))] : 0;
    s.rp = LAYOUT == 2 ? slots[tile_base + r0 + ((lane >> 3) & (kRowsPerWave - 1))] : 0;
#pragma unroll
    for (int k = 0; k < kRowsPerWave; k++) s.r4[k] = LAYOUT == 3 ? slots[tile_base + r0 + k] : 0;
    return s;
}

// Issue the DMA of one 64-row tile into data buffer `buf` and scale buffer
// `sbuf`: wave w moves rows [4w, 4w+4), two rows per instruction (lane l ->
// row 4w + 2k + (l >> 5), LDS chunk position l & 31, holding global chunk
// (l & 31) ^ swz<LAYOUT>(row)); scaled rows add one 4-lane instruction for the rows'
// 16-byte scale words; 656-byte rows one 32-lane instruction for their RoPE
// parts (lane l -> row 4w + (l >> 3), position l & 7 of the row's 128 bytes
// in ring slot `buf`, holding chunk (l & 7) ^ swz<LAYOUT>(row)).
template <int LAYOUT>
__device__ __forceinline__ void issue_tile(uint32_t lds0, const TileSlots &s,
                                           int buf, int sbuf, int w, int lane) {
    using L = Lds<LAYOUT>;
    const int r0 = kRowsPerWave * w;
    const uint32_t dst = lds0 + buf * L::kBufBytes + r0 * L::kRowPitch;
    // (a masked entry's source is its zero row of kZeroRow)
    auto src_of = [](uint64_t src, int byte) {
        return reinterpret_cast<const uint8_t *>((src & ~kMaskBits) + (uint64_t)byte);
    };
    if constexpr (LAYOUT == 3) {
        // one 1024-byte row per instruction: lane l -> position l, holding
        // chunk l ^ swz<LAYOUT>(row)
#pragma unroll
        for (int k = 0; k < kRowsPerWave; k++) {
            const int r = r0 + k;
            dma16(src_of(s.r4[k], (lane ^ swz<LAYOUT>(r)) * 16), dst + k * 1024);
        }
        return;
    }
    const int pos = lane & 31;
#pragma unroll
    for (int k = 0; k < kLoadsRaw; k++) {
        const int r = r0 + 2 * k + (lane >> 5);
        dma16(src_of(s.row[k], (pos ^ swz<LAYOUT>(r)) * 16), dst + k * 1024);
    }
    if (LAYOUT == 1 || LAYOUT == 2) {
        if (lane < kRowsPerWave)
            dma16(src_of(s.sc, kD), lds0 + L::kOffScales + sbuf * L::kScBytes + r0 * 16);
    }
    if (LAYOUT == 2) {
        if (lane < 8 * kRowsPerWave) {
            const int r = r0 + (lane >> 3);
            dma16(src_of(s.rp, kScaledBytes + ((lane & 7) ^ swz8(r)) * 16),
                  lds0 + L::kOffRope + buf * L::kRopeTile + r0 * 2 * kRopeDim);
        }
    }
}

template <int LAYOUT, bool QFP8, bool OUT_BF16, bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_kernel(AttnArgs a) {
    using L = Lds<LAYOUT>;
    constexpr int NT = 1;                        // head tiles of 16 per block
    constexpr int kNB = L::kNB;                  // tile buffers
    constexpr int kHB = L::kHB;
    constexpr int kParts = L::kParts;            // dim parts of the QK reduction
    constexpr int kDP = kD / kParts;             // dims per part: 128 or 256
    constexpr int kSteps = kDP / 32;             // bf16 K = 32 steps per part
    constexpr int kSteps8 = kDP / 128;           // FP8 K = 128 steps per part
    constexpr int kGpp = kDP / 128;              // scale groups per part
    constexpr int kChunks = kDP / 16;            // 16-byte row chunks per part
    constexpr int kXc = LAYOUT == 3 ? kDP / 32 : kDP / 64;   // of which one lane holds (4 lane groups)
    // Schedule: waves 0-7 score (QK and the owners' softmax), waves 8-15
    // accumulate PV one tile behind, so the owners' softmax of tile k
    // overlaps the PV of tile k-1 and each tile's operand reads overlap the
    // phase before.
    static_assert(kParts == 2, "one publishing wave per quarter");
    // PV operands read in their own step (one register set; a tile's buffer
    // is refilled right after its step): 656-byte and bf16 rows, whose extra
    // operands would not fit otherwise
    constexpr bool kLate = LAYOUT >= 2;
    constexpr bool kScaled = LAYOUT == 1 || LAYOUT == 2;   // rows carry group scales
    constexpr int kDT = 4;                       // PV: 16-dim tiles per wave
    // tiles requested before the first lands (1 to 4 measured the same)
    constexpr int kFill0 = 2;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr int kLoads = LAYOUT == 3 ? kRowsPerWave
                                       : kLoadsRaw + (kScaled ? 1 : 0) + (LAYOUT == 2 ? 1 : 0);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const bool is_v = w >= 8;                    // a PV-only wave
    // Scoring (partials of 16 entries x 16 heads x one 256-dim part dp):
    // wave (q = w & 3, dp = w >> 2) scores entry quarter q; the dp = 0 waves
    // own their quarter (add the other part, form P), the dp = 1 waves only
    // publish their partial, through LDS slot q.  (32-head blocks run
    // attn_w8_kernel.)
    // scoring waves read a tile's row chunks in the tile's own step rather
    // than during the softmax before (possible with kLate's buffer rotation)
    constexpr bool kOwnStep = LAYOUT >= 2;
    constexpr int kRT = 1;                       // entry quarters a scoring wave scores
    constexpr int kQT = NT;                      // head tiles it scores
    const int dp = (w >> 2) % kParts;            // QK: dims part
    const int wq = w & 3;                        // entry quarter owned (and scored)
    const int ht = 0;
    const bool owns = dp == 0;
    const bool owner = !is_v && owns;
    const int dbase = 64 * (w - 8);              // PV: first of this wave's dims
    const int n_hb = (a.H + kHB - 1) / kHB;

    // XCD-aware numbering: all of token t's workgroups are 8k + (t % 8)
    const int per_tok = n_hb * a.n_splits;
    const int x = blockIdx.x & 7;
    const int kq = blockIdx.x >> 3;
    const int t = (kq / per_tok) * 8 + x;
    if (t >= a.T) return;
    const int hb = (kq % per_tok) / a.n_splits;
    const int split = kq % a.n_splits;

    uint64_t *slots = reinterpret_cast<uint64_t *>(lds + L::kOffSlots);   // row sources
    float *sp_lds = reinterpret_cast<float *>(lds + L::kOffSp);     // [waves][16 heads][16]
    float *rl_lds = reinterpret_cast<float *>(lds + L::kOffRedL);   // [kHB][4 quarters]

    const int seq = a.token_seq ? a.token_seq[t] : t;
    const bool seq_ok = (a.page_table == nullptr && a.seq_lens == nullptr) ||
                        (seq >= 0 && seq < a.num_seqs);
    const int seq_len = (a.seq_lens && seq_ok) ? a.seq_lens[seq] : INT_MAX;
    const int begin = split * a.split_len;
    const int n_ent = min(a.K - begin, a.split_len);   // a multiple of 64

    // Query of head (ht or nt)*16 + c of each scored head tile, dims part dp,
    // as the B operand.  bf16: bq[nt][kk] = q[h][d .. d+8] with d = (dp*kChunks
    // + (kk>>1)*4 + g)*16 + (kk&1)*8, so that a lane's steps 2m, 2m+1 use one
    // 16-byte chunk of the row; FP8: bq8[nt][k2] = q8[h][dp*kDP + k2*128 +
    // g*32 .. +32].  Heads beyond H read head 0 and are not stored.
    // 656-byte rows: query rows of 512 + 64, and bqr = the RoPE part of head
    // c, dims dp*32 + g*8 .. +8 (B operand of one bf16 MFMA step per part).
    constexpr int kQRow = kD + (LAYOUT == 2 ? kRopeDim : 0);
    constexpr int kQRowBytes = kQRow * (QFP8 ? 1 : 2);
    constexpr int kQChunks = kQRowBytes / 16;        // 16-byte chunks per head row
    bf16x8 bq[QFP8 ? 1 : kQT][QFP8 ? 1 : kSteps];
    i32x8 bq8[QFP8 ? kQT : 1][QFP8 ? kSteps8 : 1];
    bf16x8 bqr;
    float sscale = a.softmax_scale * kLog2e;
    if constexpr (QFP8) sscale *= *a.q_scale;
    // The query registers from `at(hl, byte)`: the address of byte `byte` of
    // the row of head hb*kHB + hl, in global memory or in the LDS copy.
    auto load_q = [&](auto at) {
#pragma unroll
        for (int nt = 0; nt < kQT; nt++) {
            const int hl = nt * 16 + c;
            if constexpr (LAYOUT == 2)
                bqr = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(at(hl, (kD + dp * 32 + g * 8) * 2)));
            if constexpr (QFP8) {
#pragma unroll
                for (int k2 = 0; k2 < kSteps8; k2++) {
                    const int b = dp * kDP + k2 * 128 + g * 32;
                    const u32x4 lo = *reinterpret_cast<const u32x4 *>(at(hl, b));
                    const u32x4 hi = *reinterpret_cast<const u32x4 *>(at(hl, b + 16));
                    bq8[nt][k2] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < kSteps; kk++)
                    bq[nt][kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                        at(hl, ((dp * kChunks + (kk >> 1) * 4 + g) * 16 + (kk & 1) * 8) * 2)));
            }
        }
    };
    auto q_global = [&](int hl, int byte) {
        const int h = hb * kHB + hl;
        return reinterpret_cast<const uint8_t *>(a.q) +
               ((int64_t)t * a.H + (h < a.H ? h : 0)) * kQRowBytes + byte;
    };
    // With a tile buffer that the pipeline fills only after the first tile
    // has landed (kStageQ), the query goes to LDS by DMA right behind the
    // prologue, ahead of the first tiles (so the wait for tile 0 covers it),
    // instead of into registers at the start: loaded at the start, its
    // latency would be part of the prologue's (every load waited for there
    // is older).  In the LDS copy, chunk k < 64 of head hl's row sits at
    // position k ^ (hl & 7), so that the 16 heads' reads spread over the
    // banks.
    constexpr bool kStageQ = kNB > kFill0;
    uint8_t *const qst = lds + (kNB - 1) * L::kBufBytes;
    static_assert(!kStageQ || kHB * kQRowBytes <= L::kBufBytes, "query copy fits a tile buffer");
    static_assert((kHB * kQChunks) % 64 == 0, "whole waves of query chunks");
    auto q_lds = [&](int hl, int byte) {
        const int k = byte >> 4;
        return qst + hl * kQRowBytes + ((k < 64 ? k ^ (hl & 7) : k) << 4) + (byte & 15);
    };
    if constexpr (!kStageQ) {
        if (!is_v) load_q(q_global);
    }

    // ---- prologue: resolve this split's indices into LDS.  Every load is
    // unconditional (addresses clamped into range, results selected after),
    // so each phase issues all its loads before a single wait.  When the
    // token's page-table row fits in the (still unused) sp/P areas it is
    // staged there together with the top-k loads, so resolution costs one
    // global latency instead of two.
    {
        constexpr int kPer = kMaxSplit / kThreads;
        constexpr int kPtPer = L::kPtPer;
        constexpr int kPtCap = kPtPer * kThreads;
        // lane l of wave w resolves entry i of the rows it copies in every
        // tile: row kRowsPerWave w + (l mod kRowsPerWave) of tile
        // l / kRowsPerWave + (64 / kRowsPerWave) i, so that its first tiles'
        // copies read only its own slot stores and go out before the barrier
        constexpr int kTilesPerI = 64 / kRowsPerWave;
        static_assert(kPer * kTilesPerI * kTile == kMaxSplit, "every entry once");
        auto entry_of = [&](int i) {
            return (lane / kRowsPerWave + kTilesPerI * i) * kTile + kRowsPerWave * w + lane % kRowsPerWave;
        };
        const int32_t *tk = a.topk + (int64_t)t * a.K + begin;
        const int32_t *row = a.page_table + (int64_t)(seq_ok ? seq : 0) * a.max_pages;
        int32_t *pt_lds = reinterpret_cast<int32_t *>(lds + L::kOffSp);
        const bool pt_staged = a.page_table != nullptr && a.max_pages <= kPtCap;
        int32_t v[kPer], phys[kPer];
        if (pt_staged) {
            int32_t pw[kPtPer];
#pragma unroll
            for (int k = 0; k < kPtPer; k++) pw[k] = row[min(tid + k * kThreads, a.max_pages - 1)];
#pragma unroll
            for (int i = 0; i < kPer; i++) {
                const int j = entry_of(i);
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
                const int j = entry_of(i);
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
        // the highest tile of each wave holding a valid entry (ballot of the
        // resolved slots; the tile grows with the lane): the tiles after the
        // split's last valid entry hold only masked entries, which
        // contribute nothing, and are skipped
        const TokenIndexRule rule(seq_ok, seq_len, a.page_table != nullptr, a.page_shift, a.max_pages,
                                  a.num_slots);
        int n_err = 0, last = -1;
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            const int j = entry_of(i);
            // (tiles past the split's end hold padding only)
            if (kTilesPerI * i * kTile >= n_ent) continue;
            bool err;
            const int32_t s = rule(v[i], phys[i], err);
            n_err += __builtin_popcountll(__builtin_amdgcn_ballot_w64(err));   // the wave's
            if (j < n_ent)
                slots[j] = s >= 0 ? reinterpret_cast<uint64_t>(a.pool + (int64_t)s * row_bytes<LAYOUT>())
                                  : reinterpret_cast<uint64_t>(kZeroRow + (j & (kTile - 1)) * row_bytes<LAYOUT>()) | kMaskBits;
            const uint64_t vb = __builtin_amdgcn_ballot_w64(j < n_ent && s >= 0);
            if (vb) last = max(last, (kTilesPerI * i + (63 - (int)__builtin_clzll(vb)) / kRowsPerWave) * kTile);
        }
        if (lane == 0) reinterpret_cast<int *>(rl_lds)[w] = last;
        if (a.err_count && hb == 0 && lane == 0 && n_err) atomicAdd(a.err_count, n_err);
    }
    const uint32_t lds0 = lds_addr(lds);
    // Every load issued so far (the index loads, already used, and the
    // query's register loads) has landed after the wait below, and the
    // compiler knows it: it then puts no wait of its own behind the copies,
    // which it does not see.  Then the query copy (kStageQ:
    // chunk i of the block's kHB rows to LDS position i, holding the row's
    // chunk (i % kQChunks) unswizzled) and this wave's rows of the first
    // kFill0 tiles, before the barrier: they read only this wave's slot
    // stores (the tiles past the last valid entry read masked rows).
    wait_vm_lgkm0<0>();
    if constexpr (kStageQ) {
        const uint32_t qbase = lds_addr(qst);
#pragma unroll
        for (int i0 = 0; i0 < kHB * kQChunks; i0 += kThreads) {
            if (i0 + w * 64 < kHB * kQChunks) {
                const int i = i0 + w * 64 + lane;
                const int hl = i / kQChunks, kp = i % kQChunks;
                dma16(q_global(hl, (kp < 64 ? kp ^ (hl & 7) : kp) << 4), qbase + (i0 + w * 64) * 16);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kFill0; i++)
        if (i * kTile < n_ent)
            issue_tile<LAYOUT>(lds0, read_slots<LAYOUT>(slots, i * kTile, w, lane), i,
                                   i, w, lane);
    // slots and last entries visible (the copies stay in flight)
    wait_lgkm0();
    barrier_raw();
    // tiles up to the one holding the last valid entry (at least one: an
    // all-masked split still runs one tile and leaves l = 0)
    int n_tiles;
    {
        const int4 *lw = reinterpret_cast<const int4 *>(rl_lds);
        int last = -1;
#pragma unroll
        for (int i = 0; i < kWaves / 4; i++) {
            const int4 v4 = lw[i];
            last = max(max(last, max(v4.x, v4.y)), max(v4.z, v4.w));
        }
        n_tiles = __builtin_amdgcn_readfirstlane(max(1, (last + kTile) / kTile));
    }

    // ---- fill the pipeline: the first kFill0 tiles went out before the
    // barrier, the other buffers once tile 0 has landed (requested all at
    // once, every workgroup's first tile would come back only with the rest
    // of the burst); the buffer holding the query copy once every wave has
    // its query
    auto fill_rest = [&](auto last) {
        constexpr bool LAST = decltype(last)::value;
#pragma unroll
        for (int i = kFill0; i < kNB; i++)
            if (i < n_tiles && (i == kNB - 1) == LAST)
                issue_tile<LAYOUT>(lds0, read_slots<LAYOUT>(slots, i * kTile, w, lane), i,
                                       i, w, lane);
    };

    // Running state.  Owner lanes: the running maximum m_own of head ht*16+c
    // over their quarter's entries and the lane's share l_part of the
    // denominator (relative to m_own).  Every wave: the reference maximum
    // m_ref[nt] of head nt*16+c that O is accumulated against.
    // Group-scaled rows: the owners of head tile 0 keep the running largest
    // scale of group wq (s_run); the PV operand of an entry is P times
    // scale / s_run, and O is accumulated in units of the reference s_ref
    // (the wave's group's s_run, rescaled when it grows).
    float m_own = kNoMax, l_part = 0.0f;
    float m_ref[NT];
    float s_run = 0.0f, s_ref = 0.0f;
    f32x4 acc[kDT][NT];
    // One-term f16 P (group-scaled rows): PV wave 8 accumulates the
    // denominator itself, as the product of a ones
    // operand with the very P operand of the numerator (same roundings,
    // same rescales), so that the rounding of an entry's weight moves
    // numerator and denominator alike.  (bf16 rows, whose kernel has no
    // register to spare for it, sum the rounded P in the owners.)
    constexpr bool kLacc = !L::kLo && LAYOUT != 3;
    f32x4 lacc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        m_ref[nt] = kNoMax;
        lacc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int dt = 0; dt < kDT; dt++) acc[dt][nt] = f32x4{0, 0, 0, 0};
    }
    // Operands of a tile in registers: the QK row chunks (xc) of the tile
    // being scored, the PV transpose reads (tv) of the last two tiles (by
    // tile parity; one set when not pipelined or with kLate).
    u32x4 xc[kRT][kXc];
    u32x4 xcr;                  // 656-byte rows: this lane's RoPE chunk
    // (bf16 rows: eight 16-bit values per operand, u32x4)
    std::conditional_t<LAYOUT == 3, u32x4, u32x2> tv[kLate ? 1 : 2][2][kDT];
    f32x4 part[kRT * kQT];      // [entry quarter][head tile]

    // Wait until this wave's DMA of tile j has landed: `issued` is the last
    // tile issued so far, later tiles may still be in flight.
    auto wait_tile = [&](int j, int issued) {
        const int ahead = min(issued, n_tiles - 1) - j;
        if (ahead >= 3) wait_vm_lgkm0<3 * kLoads>();
        else if (ahead == 2) wait_vm_lgkm0<2 * kLoads>();
        else if (ahead == 1) wait_vm_lgkm0<kLoads>();
        else wait_vm_lgkm0<0>();
    };

    // Row chunks of tile j for QK: entry 16 wq + c; bf16 steps 2m, 2m+1 take
    // the halves of chunk dp*kChunks + 4m + g, FP8 steps k2 the chunk pair
    // dp*kChunks + 8 k2 + 2g, +1 (a step never leaves a 128-wide scale group).
    auto read_xc = [&](int j) {
#pragma unroll
        for (int rt = 0; rt < kRT; rt++) {
            const int r = 16 * wq + c;
            const uint8_t *xr = lds + (j % kNB) * L::kBufBytes + r * L::kRowPitch;
            const int sw = swz<LAYOUT>(r);
#pragma unroll
            for (int m = 0; m < kXc; m++) {
                // bf16 rows: step m's 8 dims (the query's d of step m) are the
                // 16-byte chunk d / 8
                const int ch = LAYOUT == 3 ? dp * 32 + (m >> 1) * 8 + 2 * g + (m & 1)
                               : QFP8 ? dp * kChunks + (m >> 1) * 8 + g * 2 + (m & 1)
                                      : dp * kChunks + m * 4 + g;
                xc[rt][m] = *reinterpret_cast<const u32x4 *>(xr + ((ch ^ sw) * 16));
            }
            if constexpr (LAYOUT == 2) {
                // RoPE dims dp*32 + g*8 .. +8 of the same row: chunk dp*4 + g
                const uint8_t *rr = lds + L::kOffRope + (j % kNB) * L::kRopeTile + r * (2 * kRopeDim);
                xcr = *reinterpret_cast<const u32x4 *>(rr + (((dp * 4 + g) ^ swz8(r)) * 16));
            }
        }
    };
    // PV operand X^T of tile j via transpose reads: lane (c, g) addresses
    // entry ks*32 + g*8 + (c >> 1), half (c & 1) of the chunk of dims
    // dbase + 16dt ..
    auto read_tv = [&](int j, auto par) {
        constexpr int PAR = decltype(par)::value;
        const uint8_t *xb = lds + (j % kNB) * L::kBufBytes;
        if constexpr (LAYOUT == 3) {
            // bf16 rows: the operand's 8 entries ks*32 + g*8 + i of dim
            // dbase + 16dt + c, one 16-bit read each (chunk dim / 8 of each
            // entry's row, swizzled by that row)
#pragma unroll
            for (int ks = 0; ks < 2; ks++)
#pragma unroll
                for (int dt = 0; dt < kDT; dt++) {
                    const int dim = dbase + 16 * dt + c;
                    uint32_t hw[8];
#pragma unroll
                    for (int i = 0; i < 8; i++) {
                        const int e = ks * 32 + g * 8 + i;
                        hw[i] = *reinterpret_cast<const uint16_t *>(
                            xb + e * 1024 + (((dim >> 3) ^ swz<LAYOUT>(e)) * 16) + (dim & 7) * 2);
                    }
                    tv[PAR][ks][dt] = u32x4{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16),
                                            hw[4] | (hw[5] << 16), hw[6] | (hw[7] << 16)};
                    // at most two operands' reads in flight (all 64 at once
                    // would not fit the registers)
                    if (dt & 1) __builtin_amdgcn_sched_barrier(0);
                }
        } else {
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const int row = ks * 32 + g * 8 + (c >> 1);
                const uint8_t *rp = xb + row * 512 + (c & 1) * 8;
                const int sw = swz<LAYOUT>(row);
#pragma unroll
                for (int dt = 0; dt < kDT; dt++)
                    tv[PAR][ks][dt] = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2 *>(
                                   LDS_PTR(rp + (((dbase / 16 + dt) ^ sw) * 16)))));
            }
        }
    };

    // Partial S^T of tile j from xc: entries 16 wq .. +16, dims part dp, of
    // each scored head tile (part[nt]; each converted operand feeds every
    // head tile).  The partial of a head tile the wave does not own goes to
    // LDS slot (head tile)*4 + wq, for its owner.
    auto qk = [&](int j) {
        const float *scf = reinterpret_cast<const float *>(lds + L::kOffScales + (j % kNScale) * L::kScBytes);
        float scv[4][kGpp];
        if constexpr (kScaled) {
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int jj = 0; jj < kGpp; jj++)
                    scv[i][jj] = scf[(16 * wq + 4 * g + i) * 4 + dp * kGpp + jj];
        }
        if constexpr (QFP8 && !kScaled) {
            // raw rows: one chain through the accumulator input (exact fp32
            // addition of C, as in attn_w8_kernel)
#pragma unroll
            for (int nt = 0; nt < kQT; nt++) {
                f32x4 acc8 = {0, 0, 0, 0};
#pragma unroll
                for (int k2 = 0; k2 < kSteps8; k2++) {
                    const u32x4 &lo = xc[0][2 * k2], &hi = xc[0][2 * k2 + 1];
                    const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    acc8 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bq8[nt][k2], acc8, 0, 0, 0, 127, 0, 127);
                }
                part[nt] = acc8;
            }
        } else if constexpr (QFP8) {
            // group-scaled rows: each 128-wide step is scaled by its group's
            // scale, so the steps are summed apart
#pragma unroll
            for (int nt = 0; nt < kQT; nt++) {
                f32x4 accg[kSteps8];
#pragma unroll
                for (int k2 = 0; k2 < kSteps8; k2++) {
                    const u32x4 &lo = xc[0][2 * k2], &hi = xc[0][2 * k2 + 1];
                    const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    accg[k2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        av, bq8[nt][k2], f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    float s = accg[0][i] * scv[i][0];
#pragma unroll
                    for (int k2 = 1; k2 < kSteps8; k2++) s += accg[k2][i] * scv[i][k2];
                    part[nt][i] = s;
                }
            }
        } else {
            // raw rows: two independent chains (even / odd kk) for a single
            // (quarter, head tile) product, else one per product; scaled
            // rows (one of each): one chain per 128-wide scale group
            constexpr int kCh = (!kScaled && kQT > 1) ? 1 : 2;
            f32x4 accg[kRT][kQT][2];
#pragma unroll
            for (int rt = 0; rt < kRT; rt++)
#pragma unroll
                for (int nt = 0; nt < kQT; nt++) accg[rt][nt][0] = accg[rt][nt][1] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int rt = 0; rt < kRT; rt++)
#pragma unroll
                for (int kk = 0; kk < kSteps; kk++) {
                    const int q = !kScaled ? (kCh == 2 ? (kk & 1) : 0)
                                           : (kGpp == 1 ? (kk & 1) : (kk >> 2));
                    bf16x8 av;
                    if constexpr (LAYOUT == 3) {
                        av = __builtin_bit_cast(bf16x8, xc[rt][kk]);   // bf16 rows: as read
                    } else {
                        const u32x4 &ch = xc[rt][kk >> 1];
                        av = (kk & 1) ? e4m3x8_to_bf16(ch[2], ch[3]) : e4m3x8_to_bf16(ch[0], ch[1]);
                    }
#pragma unroll
                    for (int nt = 0; nt < kQT; nt++)
                        accg[rt][nt][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av, bq[nt][kk], accg[rt][nt][q], 0, 0, 0);
                    // two quarters: each step's converts stay next to its
                    // MFMAs (hoisted ahead, the converted operands would not
                    // fit the registers beside both quarters' rows)
                    if constexpr (kRT > 1) __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
            for (int rt = 0; rt < kRT; rt++)
#pragma unroll
                for (int nt = 0; nt < kQT; nt++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const f32x4 *ag = accg[rt][nt];
                        if constexpr (!kScaled || kGpp == 1) {
                            const float s = kCh == 2 ? ag[0][i] + ag[1][i] : ag[0][i];
                            part[rt * kQT + nt][i] = !kScaled ? s : s * scv[i][0];
                        } else {
                            part[rt * kQT + nt][i] = ag[0][i] * scv[i][0] + ag[1][i] * scv[i][kGpp - 1];
                        }
                    }
            if constexpr (LAYOUT == 2) {
                // this part's 32 RoPE dims: exact bf16 products, no scale
                const f32x4 accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, xcr), bqr, f32x4{0, 0, 0, 0}, 0, 0, 0);
                part[0] += accr;
            }
        }
        // publish every partial this wave does not own
#pragma unroll
        for (int rt = 0; rt < kRT; rt++)
#pragma unroll
            for (int nt = 0; nt < kQT; nt++) {
                const int qt = nt;                         // its head tile
                const int qq = wq;                         // its entry quarter
                if (!(owner && qt == ht && qq == wq)) {
                    const int slot = qt * 4 + qq;
                    *reinterpret_cast<f32x4 *>(sp_lds + (slot * 16 + c) * 16 + 4 * sp_slot(g, c)) =
                        part[rt * kQT + nt];
                }
            }
    };

    // Owner waves, tile j: full scores of entries 16 wq + 4g + i, head ht*16
    // + c; running maximum of the quarter (moved only when the tile maximum
    // exceeds it by more than kSlack, so P <= 2^kSlack); P as f16 into the P
    // buffer of parity PAR.
    // `then` runs after the softmax's own LDS reads are issued (the
    // pipelined schedule issues the next tile's operand reads there, so that
    // they queue behind the softmax's and not in front of them).
    auto softmax = [&](int j, auto then) {
        const int par = j & 1;
        float *mq_w = reinterpret_cast<float *>(lds + L::kOffMq + par * L::kMqBytes);
        uint8_t *p_w = lds + L::kOffP;
        const int hh = ht * 16 + c;
        // (the high words of the entries' row sources, see kMaskBits)
        const int32_t *slh = reinterpret_cast<const int32_t *>(slots + j * kTile + 16 * wq + 4 * g) + 1;
        const int4 sl4 = {slh[0], slh[2], slh[4], slh[6]};
        // own part of the owned (quarter, head tile) plus the other part's,
        // published
        f32x4 s;
        s = part[0];
        {
            const int slot = ht * 4 + wq;
            s += *reinterpret_cast<const f32x4 *>(sp_lds + (slot * 16 + c) * 16 + 4 * sp_slot(g, c));
        }
        const f32x4 mp = *reinterpret_cast<const f32x4 *>(
            lds + L::kOffMq + (par ^ 1) * L::kMqBytes + hh * 16);
        float sc_own = 0.0f;
        if constexpr (kScaled)
            sc_own = reinterpret_cast<const float *>(lds + L::kOffScales + (j % kNScale) * L::kScBytes)[lane * 4 + wq];
        then();
        // a masked entry reads a zero row: its score is exactly 0, and the
        // mask term (-inf) masks it
        const float madd[4] = {mask_term(sl4.x), mask_term(sl4.y), mask_term(sl4.z), mask_term(sl4.w)};
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) sv[i] = __builtin_fmaf(s[i], sscale, madd[i]);
        const float mx = max_over_g(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
        if (j > 0) {
            // adopt the largest quarter maximum of the previous tile, so that
            // the quarters keep a common reference (their P then needs no
            // reweighting in PV) until one of them moves
            const float r = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
            if (r > m_own) {
                l_part *= __builtin_amdgcn_exp2f(m_own - r);
                m_own = r;
            }
        }
        const bool moved = mx - m_own > kSlack;   // false for an all-masked tile
        if (moved) {
            l_part *= __builtin_amdgcn_exp2f(m_own - mx);
            m_own = mx;
        }
        if (g == 0) lds[L::kOffFlags + par * kHB * 4 + hh * 4 + wq] = j > 0 && !moved;
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(sv[i] - m_own);   // masked: 2^-inf = 0
        // P goes to the PV product as 16-bit values.  Raw FP8 rows (whose
        // values reach +-448) carry it as two f16 terms, hi = f16(P) and
        // lo = f16(P - hi): one f16 rounding alone (2^-11 relative) moves a
        // weighted sum of such values by up to 2^-10 of its spread; the
        // owners' shares of the denominator are then sums of P itself.
        // Group-scaled rows carry one f16 term (the entry's scale factor
        // multiplies it in the PV waves), whose denominator is formed from
        // the operand itself in the PV waves (lacc); bf16 rows carry one
        // bf16 term (their PV product takes bf16) and sum it here as
        // rounded.  (32-head blocks: attn_w8_kernel, one f16 term.)
        const int poff = p_off(hh, 2 * wq + (g >> 1)) + (g & 1) * 8;
        if constexpr (LAYOUT == 3) {
            const uint32_t b01 = pack_bf16x2(p[0], p[1]), b23 = pack_bf16x2(p[2], p[3]);
            l_part += bf16_bits_to_f32(b01 & 0xffffu);
            l_part += bf16_bits_to_f32(b01 >> 16);
            l_part += bf16_bits_to_f32(b23 & 0xffffu);
            l_part += bf16_bits_to_f32(b23 >> 16);
            *reinterpret_cast<u32x2 *>(p_w + poff) = u32x2{b01, b23};
        } else {
            const f16x2 p01 = {(_Float16)p[0], (_Float16)p[1]};
            const f16x2 p23 = {(_Float16)p[2], (_Float16)p[3]};
            *reinterpret_cast<u32x2 *>(p_w + poff) =
                u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
            if constexpr (L::kLo) {
                const f16x2 l01 = {(_Float16)(p[0] - (float)p01[0]), (_Float16)(p[1] - (float)p01[1])};
                const f16x2 l23 = {(_Float16)(p[2] - (float)p23[0]), (_Float16)(p[3] - (float)p23[1])};
                *reinterpret_cast<u32x2 *>(p_w + L::kPBytes + poff) =
                    u32x2{__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23)};
                l_part += (p[0] + p[1]) + (p[2] + p[3]);
            }
        }
        if (g == 0) mq_w[hh * 4 + wq] = m_own;
        if constexpr (kScaled) {
            // running largest scale of group wq (this tile's 64 entries one
            // per lane), then each entry's factor scale / s_run (at most 1,
            // so that P times it stays within f16); one owner per group
            s_run = fmaxf(s_run, max_over_g(dpp_max16(sc_own)));
            if (ht == 0) {
                const float inv = s_run > 0.0f ? __builtin_amdgcn_rcpf(s_run) : 0.0f;
                reinterpret_cast<_Float16 *>(lds + L::kOffFac + par * L::kFacBytes)[wq * kTile + lane] =
                    (_Float16)fminf(sc_own * inv, 1.0f);
                if (lane == 0) reinterpret_cast<float *>(lds + L::kOffSmax)[par * 4 + wq] = s_run;
            }
        }
    };

    // O^T[dims dbase.., heads] += X^T . P^T over tile j's 64 entries from
    // tv[TPAR] and the P buffer of parity j & 1; P of quarter q weighted by
    // 2^(m_q - m_ref) (m_ref = running max of the quarter maxima; O rescaled
    // when it moves).
    // PV in two steps: pv_prep(j) fixes the reference maximum, rescales O
    // and loads tile j's P operand (pv_bp, with the weights applied);
    // pv_mma(TPAR, DT0, DT1) then accumulates dim tiles [DT0, DT1) from
    // tv[TPAR].  The pipelined schedule splits the dim tiles over its two
    // phases.
    // P times a weight factor, formed in fp32 and rounded to f16 once
    auto reweight_f16 = [](f16x8 &b, float f) {
#pragma unroll
        for (int e = 0; e < 8; e++) b[e] = (_Float16)((float)b[e] * f);
    };
    f16x8 pv_bp[NT][2];
    f16x8 pv_bl[L::kLo ? NT : 1][2];     // the lo terms (raw rows)
    auto pv_prep = [&](int j) {
        const int ppar = j & 1;
        const float *mq_lds = reinterpret_cast<const float *>(lds + L::kOffMq + ppar * L::kMqBytes);
        const uint8_t *p_lds = lds + L::kOffP;
        // While every quarter kept the previous reference (all four flags
        // set) the reference, O and P stay as they are.  Otherwise: m_ref
        // takes the largest quarter maximum (O rescaled when it moves) and
        // fq[nt][ks] weights this lane's quarter 2ks + g/2 (read by address:
        // a register-array select on g would go to scratch).
        // B operand P^T: entries ks*32 + g*8 + r of head nt*16 + c (one
        // 16-byte chunk, quarter 2ks + g/2); read together with the flags
        auto &bp = pv_bp;
        auto &bl = pv_bl;
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                bp[nt][ks] = *reinterpret_cast<const f16x8 *>(p_lds + p_off(nt * 16 + c, 4 * ks + g));
                if constexpr (L::kLo)
                    bl[nt][ks] = *reinterpret_cast<const f16x8 *>(p_lds + L::kPBytes +
                                                                 p_off(nt * 16 + c, 4 * ks + g));
            }
        bool uneven = false;
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
            uneven |= *reinterpret_cast<const uint32_t *>(
                          lds + L::kOffFlags + ppar * kHB * 4 + (nt * 16 + c) * 4) != 0x01010101u;
        const bool reweight = __ballot(uneven) != 0;
        float fq[NT][2];
#pragma unroll
        for (int nt = 0; nt < NT; nt++) fq[nt][0] = fq[nt][1] = 1.0f;
        if (reweight) {
            bool any_resc = false;
            float alpha[NT];
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                const float *mrow = mq_lds + (nt * 16 + c) * 4;
                const f32x4 mq = *reinterpret_cast<const f32x4 *>(mrow);
                const float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
                const bool resc = mx > m_ref[nt];
                alpha[nt] = resc ? __builtin_amdgcn_exp2f(m_ref[nt] - mx) : 1.0f;
                if (resc) m_ref[nt] = mx;
                any_resc |= resc;
                fq[nt][0] = __builtin_amdgcn_exp2f(mrow[g >> 1] - m_ref[nt]);
                fq[nt][1] = __builtin_amdgcn_exp2f(mrow[2 + (g >> 1)] - m_ref[nt]);
            }
            if (__ballot(any_resc)) {
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
#pragma unroll
                    for (int dt = 0; dt < kDT; dt++) acc[dt][nt] *= alpha[nt];
                    if constexpr (kLacc) lacc[nt] *= alpha[nt];
                }
            }
        }
        // the denominator of one-term P from the operand as weighted
        auto add_lacc = [&]() {
            if constexpr (kLacc) {
                if (w == 8) {
#pragma unroll
                    for (int nt = 0; nt < NT; nt++)
#pragma unroll
                        for (int ks = 0; ks < 2; ks++) {
                            const f16x8 one = {1, 1, 1, 1, 1, 1, 1, 1};
                            lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(one, bp[nt][ks], lacc[nt], 0, 0, 0);
                        }
                }
            }
        };
        if constexpr (kScaled) {
            // the group's running largest scale (uniform): O moves to the
            // new reference when it grows; then P times each entry's factor
            // scale / s_run, published by the group's owner
            const int grp = dbase >> 7;
            const float sr = reinterpret_cast<const float *>(lds + L::kOffSmax)[ppar * 4 + grp];
            const f16x8 *fac = reinterpret_cast<const f16x8 *>(lds + L::kOffFac + ppar * L::kFacBytes +
                                                                (grp * kTile + g * 8) * 2);
            const f16x8 fk[2] = {fac[0], fac[32 / 8]};
            if (sr > s_ref) {
                const float beta = s_ref * __builtin_amdgcn_rcpf(sr);
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
#pragma unroll
                    for (int dt = 0; dt < kDT; dt++) acc[dt][nt] *= beta;
                s_ref = sr;
            }
            if (reweight) {
#pragma unroll
                for (int nt = 0; nt < NT; nt++)
#pragma unroll
                    for (int ks = 0; ks < 2; ks++) reweight_f16(bp[nt][ks], fq[nt][ks]);
            }
            add_lacc();
#pragma unroll
            for (int nt = 0; nt < NT; nt++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++) bp[nt][ks] *= fk[ks];
            return;
        } else if (reweight) {
#pragma unroll
            for (int nt = 0; nt < NT; nt++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++) {
                    if constexpr (LAYOUT == 3) {
                        // bf16 P: widen, weight in fp32, round back
                        u32x4 b = __builtin_bit_cast(u32x4, bp[nt][ks]);
#pragma unroll
                        for (int e = 0; e < 4; e++) {
                            const float lo = bf16_bits_to_f32(b[e] & 0xffffu) * fq[nt][ks];
                            const float hi = bf16_bits_to_f32(b[e] >> 16) * fq[nt][ks];
                            b[e] = pack_bf16x2(lo, hi);
                        }
                        bp[nt][ks] = __builtin_bit_cast(f16x8, b);
                    } else if constexpr (L::kLo) {
                        // hi + lo weighted in fp32 and split again
#pragma unroll
                        for (int e = 0; e < 8; e++) {
                            const float v = ((float)bp[nt][ks][e] + (float)bl[nt][ks][e]) * fq[nt][ks];
                            bp[nt][ks][e] = (_Float16)v;
                            bl[nt][ks][e] = (_Float16)(v - (float)bp[nt][ks][e]);
                        }
                        __builtin_amdgcn_sched_barrier(0);
                    } else {
                        reweight_f16(bp[nt][ks], fq[nt][ks]);
                    }
                }
        }
        add_lacc();
    };
    auto pv_mma = [&](auto tpar, auto dt0, auto dt1) {
        constexpr int TPAR = decltype(tpar)::value;
#pragma unroll
        for (int dt = decltype(dt0)::value; dt < decltype(dt1)::value; dt++) {
            if constexpr (LAYOUT == 3) {
                // bf16 rows: the gathered operands as they are, bf16 P
                const bf16x8 bv0 = __builtin_bit_cast(bf16x8, tv[TPAR][0][dt]);
                const bf16x8 bv1 = __builtin_bit_cast(bf16x8, tv[TPAR][1][dt]);
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        bv0, __builtin_bit_cast(bf16x8, pv_bp[nt][0]), acc[dt][nt], 0, 0, 0);
                    acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        bv1, __builtin_bit_cast(bf16x8, pv_bp[nt][1]), acc[dt][nt], 0, 0, 0);
                }
            } else {
                const f16x8 av0 = e4m3x8_to_f16(tv[TPAR][0][dt][0], tv[TPAR][0][dt][1]);
                const f16x8 av1 = e4m3x8_to_f16(tv[TPAR][1][dt][0], tv[TPAR][1][dt][1]);
#pragma unroll
                for (int nt = 0; nt < NT; nt++) {
                    acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av0, pv_bp[nt][0], acc[dt][nt], 0, 0, 0);
                    acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av1, pv_bp[nt][1], acc[dt][nt], 0, 0, 0);
                    if constexpr (L::kLo) {
                        acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av0, pv_bl[nt][0], acc[dt][nt], 0, 0, 0);
                        acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av1, pv_bl[nt][1], acc[dt][nt], 0, 0, 0);
                    }
                }
            }
        }
    };
    using DT0 = std::integral_constant<int, 0>;
    using DTH = std::integral_constant<int, 1>;
    using DTN = std::integral_constant<int, kDT>;
    auto pv = [&](int j, auto tpar) {
        pv_prep(j);
        pv_mma(tpar, DT0{}, DTN{});
    };

    // denominators: the owner lanes' shares, then the four quarters weighted
    // by 2^(m_q - m_ref); the quarter maxima are the last tile's.  Output or
    // partial state from the waves that hold O.
    // SCORING (compile-time): called by the pipelined scoring waves, which
    // only publish their denominators (O, which they never touch, is then
    // not live in their code).
    auto epilogue = [&](auto scoring) {
        const float *mq_fin = reinterpret_cast<const float *>(
            lds + L::kOffMq + ((n_tiles - 1) & 1) * L::kMqBytes);
        if constexpr (!kLacc) {
            if (owner) {
                l_part = sum_over_g(l_part);
                if (g == 0) rl_lds[(ht * 16 + c) * 4 + wq] = l_part;
            }
        } else if (!decltype(scoring)::value) {
            if (w == 8 && g == 0) {
#pragma unroll
                for (int nt = 0; nt < NT; nt++) rl_lds[nt * 16 + c] = lacc[nt][0];
            }
        }
        __syncthreads();
        if constexpr (decltype(scoring)::value) return;   // the PV waves hold O
        const int w_first = 8;                // writes m, l and lse
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            const int hh = nt * 16 + c;
            const int h = hb * kHB + hh;
            if (h >= a.H) continue;
            float l_tot = 0.0f;
            if constexpr (kLacc) {
                l_tot = rl_lds[hh];
            } else {
                const f32x4 mq = *reinterpret_cast<const f32x4 *>(mq_fin + hh * 4);
                const f32x4 lq = *reinterpret_cast<const f32x4 *>(rl_lds + hh * 4);
#pragma unroll
                for (int q = 0; q < 4; q++) l_tot += lq[q] * __builtin_amdgcn_exp2f(mq[q] - m_ref[nt]);
            }
            const int64_t th = (int64_t)t * a.H + h;
            if (SPLIT) {
                // the split's normalised output o / l in fp32 (a raw row's
                // values reach +-448, where f16 would round by up to 0.125),
                // then (m, l)
                const float inv = (l_tot > 0.0f ? 1.0f / l_tot : 0.0f) * (kScaled ? s_ref : 1.0f);
                const int64_t po = (th * a.n_splits + split) * kD + dbase + 4 * g;
#pragma unroll
                for (int dt = 0; dt < kDT; dt++)
                    store_through(reinterpret_cast<f32x4 *>(a.ws + po + dt * 16), acc[dt][nt] * inv);
                if (w == w_first && g == 0) {
                    float *ml = a.ws + (int64_t)a.T * a.H * a.n_splits * kD +
                                (th * a.n_splits + split) * 2;
                    ml[0] = m_ref[nt];
                    ml[1] = l_tot;
                }
            } else {
                const float inv = (l_tot > 0.0f ? 1.0f / l_tot : 0.0f) * (kScaled ? s_ref : 1.0f);
                if (OUT_BF16) {
                    store_bf16_tiles<kDT>(reinterpret_cast<uint16_t *>(a.out) + th * kD + dbase, g,
                                          [&](int dt) { return acc[dt][nt] * inv; });
                } else {
                    const int64_t base = th * kD + dbase + 4 * g;
#pragma unroll
                    for (int dt = 0; dt < kDT; dt++)
                        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + base + dt * 16) = acc[dt][nt] * inv;
                }
                if (a.lse && w == w_first && g == 0)
                    a.lse[th] = l_tot > 0.0f ? (m_ref[nt] + log2f(l_tot)) * kLn2 : -INFINITY;
            }
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    {
        // Tile k (parity PAR = k & 1), its operands already in registers:
        //   scoring waves: QK(k) -> partials; PV waves: P of tile k-1 (P
        //   buffer PAR^1) and the first of their four dim tiles (tv[PAR^1]);
        //   [tile k+1 landed]  barrier;  scoring waves read tile k+1's row
        //   chunks, owners turn tile k's scores into P (buffer PAR); PV
        //   waves: the other three dim tiles (after the barrier, where they
        //   overlap the softmax rather than hold up the scoring waves; one
        //   or none before it measured alike, two or three slower), then read tile
        //   k+1's transpose operands into tv[PAR^1];  barrier;
        //   tile k+1's buffer takes tile k+1+kNBuf.
        // Both roles pass the same barriers in the same order.
        // 656-byte and bf16 rows (kLate): the PV waves read tile k's
        // transpose operands in step k itself, into a single register set,
        // and tile k's buffer (not tile k+1's) takes the next tile after
        // step k, so that one tile fewer is in flight beyond the one being
        // scored.
        constexpr int kAhead = kLate ? kNB - 1 : kNB;
        auto refill = [&](int k, const TileSlots &nsl) {
            const int nx = k + 1 + kAhead;
            if (nx < n_tiles)
                issue_tile<LAYOUT>(lds0, nsl, nx % kNB, nx % kNScale, w, lane);
        };
        // tile 0's operands, then (16 heads) its buffer takes tile kNBuf
        // (each role keeps its own registers: nothing flows from one role's
        // code into the other's)
        auto first_tile = [&](auto read_ops) {
            // tile 0 (and the query copy, issued before it) landed
            wait_tile(0, kFill0 - 1);
            barrier_raw();
            if constexpr (kStageQ) {
                fill_rest(std::false_type{});
                if (!is_v) load_q(q_lds);
            } else {
                fill_rest(std::false_type{});
                fill_rest(std::true_type{});
            }
            read_ops();
            const TileSlots nsl = read_slots<LAYOUT>(slots, min(kNB, n_tiles - 1) * kTile, w, lane);
            wait_lgkm0();
            barrier_raw();
            // every wave holds its query: its buffer takes its tile
            if constexpr (kStageQ) fill_rest(std::true_type{});
            if (!kLate && kNB < n_tiles) issue_tile<LAYOUT>(lds0, nsl, 0, kNB % kNScale, w, lane);
        };
        // (the role test goes through readfirstlane so that the compiler
        // sees a uniform branch and gives each role its own registers)
        if (__builtin_amdgcn_readfirstlane((int)is_v)) {
            first_tile([&] { if constexpr (!kLate) read_tv(0, I0{}); });
            auto vstep = [&](int k, auto par) {
                constexpr int PAR = decltype(par)::value;
                // tv set of tiles k-1 and k+1 (kLate: the one set, tiles
                // k-1 then k)
                using TP = std::integral_constant<int, kLate ? 0 : PAR ^ 1>;
                if (k > 0) {
                    pv_prep(k - 1);
                    pv_mma(TP{}, DT0{}, DTH{});
                }
                wait_tile(k + 1, k + kAhead);
                barrier_raw();
                if (k > 0) pv_mma(TP{}, DTH{}, DTN{});
                if constexpr (kLate) read_tv(k, TP{});
                else if (k + 1 < n_tiles) read_tv(k + 1, TP{});
                wait_lgkm0();
                barrier_raw();
                refill(k, read_slots<LAYOUT>(slots, min(k + 1 + kAhead, n_tiles - 1) * kTile, w, lane));
            };
            for (int k = 0; k < n_tiles; k += 2) {
                vstep(k, I0{});
                if (k + 1 < n_tiles) vstep(k + 1, I1{});
            }
            if constexpr (kLate) {
                pv(n_tiles - 1, I0{});
            } else {
                if ((n_tiles - 1) & 1) pv(n_tiles - 1, I1{});
                else pv(n_tiles - 1, I0{});
            }
            epilogue(std::false_type{});
        } else {
            // (kOwnStep: a tile's row chunks are read in its own step, not
            // prefetched during the softmax before, so that they are not live
            // beside the softmax; with kLate the tile's buffer outlives the
            // step)
            first_tile([&] { if constexpr (!kOwnStep) read_xc(0); });
            for (int k = 0; k < n_tiles; k++) {
                const TileSlots nsl = read_slots<LAYOUT>(slots, min(k + 1 + kAhead, n_tiles - 1) * kTile, w, lane);
                if constexpr (kOwnStep) read_xc(k);
                qk(k);
                wait_tile(k + 1, k + kAhead);
                barrier_raw();
                // The next tile's chunks are read on every step (past the
                // last tile from a stale buffer, unused), and an owner is
                // told apart by `owns` rather than `owner`, whose role test
                // the compiler does not see as settled here: each way, the
                // chunks have a single definition per step and keep their
                // registers across the loop instead of being copied.
                if (owns) softmax(k, [&] { if constexpr (!kOwnStep) read_xc(k + 1); });
                else if constexpr (!kOwnStep) read_xc(k + 1);
                wait_lgkm0();
                barrier_raw();
                refill(k, nsl);
            }
            epilogue(std::true_type{});
        }
    }
}
// ===========================================================================
// Raw rows in 32-head blocks: eight wavefronts of 256 registers (two per
// SIMD) instead of sixteen of 128.
//
// Sixteen waves of 128 registers cannot hold a 32-head block's query over
// all dims: their scoring splits QK^T over two 256-dim halves, whose partial
// scores cross waves through LDS, and each of their eight PV waves reads all
// of P; about 150 KB of LDS traffic per 64-entry tile set the pace of that
// form.  With 256 registers a lane:
//   waves 0-3 (scoring, entry quarter q = w) hold the query of both head
//     tiles over all 512 dims and score their quarter completely (FP8
//     query: eight FP8 MFMAs per tile; bf16 query: each row chunk converted
//     once and fed to both head tiles' bf16 MFMAs), then run the softmax of
//     both head tiles.  They also copy their own quarter's 16 rows of every
//     tile, so that each waits for its rows with vmcnt alone and reads the
//     next tile's row chunks during the softmax, with no barrier in between;
//   waves 4-7 (PV, dims 128 (w - 4) .. +128) accumulate both head tiles one
//     tile behind: P of tile k-1 and the transpose operands read in step
//     k-1, then tile k's operands.
// One barrier per tile: every scoring wave has waited for its rows of tile
// k+1 before barrier k, so the PV waves read that tile after it; P, the
// quarter maxima and the flags are double-buffered by tile parity.  LDS
// traffic per tile: DMA 32 KB, row chunks 32 KB, P 4 + 16 KB, transpose
// operands 32 KB.  Numerics: attn_kernel's products and lazy maximum; P as
// one f16 term (a second would double the PV waves' matrix work, which sets
// their pace), with the denominator formed from that operand itself, so
// that the rounding of an entry's weight moves numerator and denominator
// alike.
struct W8 {
    static constexpr int kWaves = 8;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kNB = 4;                              // tile buffers
    static constexpr int kHB = 32;                             // heads per block
    static constexpr int kBufBytes = kTile * kRawBytes;        // 32 KB
    static constexpr int kOffSlots = kNB * kBufBytes;          // row sources (16 KB)
    static constexpr int kOffP = kOffSlots + kMaxSplit * 8;    // P ([32][64] f16), two
    static constexpr int kPBytes = kHB * kTile * 2;
    static constexpr int kOffMq = kOffP + 2 * kPBytes;         // quarter maxima [32][4], two
    static constexpr int kMqBytes = kHB * 16;
    static constexpr int kOffRedL = kOffMq + 2 * kMqBytes;     // the denominators [32]
    static constexpr int kOffFlags = kOffRedL + kHB * 16;      // [32][4] bytes, two
    // per wave, the first entry of the unit's last tile holding a valid
    // entry of that wave (-1: none) [8]
    static constexpr int kOffLast = kOffFlags + 2 * kHB * 4;
    // persistent workgroups: the next unit's page-table row (when it fits),
    // its sequence length (64 copies) and its sequence
    static constexpr int kOffPtN = kOffLast + 8 * 4;
    static constexpr int kPtNCap = 1472;
    static constexpr int kOffSeqN = kOffPtN + kPtNCap * 4;
    static constexpr int kBytes = kOffSeqN + 64 * 4 + 16;
    static constexpr int kDT = 8;                              // PV: 16-dim tiles per wave
    static constexpr int kLoads = 8;                           // DMA instructions per scoring wave and tile
    // the page-table row is staged in tile buffer 2 (free until after the prologue)
    static constexpr int kPtPer = kBufBytes / 4 / kThreads;
    static_assert(kBytes <= 160 * 1024, "LDS budget");
};

template <bool QFP8, bool OUT_BF16, bool SPLIT>
__global__ __launch_bounds__(W8::kThreads) void attn_w8_kernel(AttnArgs a) {
    using L = W8;
    constexpr int kQRowBytes = QFP8 ? kD : 2 * kD;       // query row bytes
    constexpr int kQChunks = kQRowBytes / 16;            // 16-byte chunks per head row
    constexpr int kNB = L::kNB, kHB = L::kHB, kDT = L::kDT;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 15, g = lane >> 4;
    const bool is_v = w >= 4;                    // a PV wave
    const int q = w & 3;                         // scoring: the entry quarter
    const int dbase = 128 * (w - 4);             // PV: first of this wave's dims
    const int n_hb = (a.H + kHB - 1) / kHB;

    // Units in XCD-aware numbering, as in attn_kernel: virtual block v is
    // token (v >> 3) / per_tok * 8 + (v & 7), head block and split.  A
    // workgroup takes the virtual blocks blockIdx.x, + gridDim.x, ... (the
    // Q8 prefill launches one workgroup per compute unit, gridDim.x a
    // multiple of 8, so that a workgroup's units keep its XCD); from its
    // second unit on, a unit's entries were resolved into LDS at the end of
    // the previous one (resolve_next), so that its start needs no prologue.
    const int per_tok = n_hb * a.n_splits;
    const int n_virt = (a.T + 7) / 8 * 8 * per_tok;
    struct Unit { int t, hb, split, begin, n_ent; bool valid; };
    auto unit_at = [&](int v) {
        Unit u;
        const int kqv = v >> 3;
        u.t = (kqv / per_tok) * 8 + (v & 7);
        u.hb = (kqv % per_tok) / a.n_splits;
        u.split = kqv % a.n_splits;
        u.begin = u.split * a.split_len;
        u.n_ent = min(a.K - u.begin, a.split_len);   // a multiple of 64
        u.valid = v < n_virt && u.t < a.T;          // (past the last token, so is every later one)
        return u;
    };
    int t = 0, hb = 0, split = 0, begin = 0, n_ent = 0;   // the current unit
    auto set_unit = [&](const Unit &u) {
        t = u.t;
        hb = u.hb;
        split = u.split;
        begin = u.begin;
        n_ent = u.n_ent;
        return u.valid;
    };
    if (!set_unit(unit_at(blockIdx.x))) return;
    // (several units per workgroup with an FP8 query only: with a bf16 query
    // the scoring waves' registers leave no room for the unit loop)
    constexpr bool kPersist = QFP8;

    uint64_t *slots = reinterpret_cast<uint64_t *>(lds + L::kOffSlots);   // row sources
    float *rl_lds = reinterpret_cast<float *>(lds + L::kOffRedL);
    int *last_lds = reinterpret_cast<int *>(lds + L::kOffLast);
    const float sscale = a.softmax_scale * kLog2e * (QFP8 ? *a.q_scale : 1.0f);

    // ---- prologue of the workgroup's first unit: its entries resolved to
    // row sources in LDS (as
    // in attn_kernel: unconditional loads, the page-table row staged when it
    // fits, the last valid entry found by ballots)
    {
        const int seq = a.token_seq ? a.token_seq[t] : t;
        const bool seq_ok = (a.page_table == nullptr && a.seq_lens == nullptr) ||
                            (seq >= 0 && seq < a.num_seqs);
        const int seq_len = (a.seq_lens && seq_ok) ? a.seq_lens[seq] : INT_MAX;
        constexpr int kPer = kMaxSplit / L::kThreads;
        constexpr int kPtCap = L::kPtPer * L::kThreads;
        const int32_t *tk = a.topk + (int64_t)t * a.K + begin;
        const int32_t *row = a.page_table + (int64_t)(seq_ok ? seq : 0) * a.max_pages;
        int32_t *pt_lds = reinterpret_cast<int32_t *>(lds + 2 * L::kBufBytes);
        const bool pt_staged = a.page_table != nullptr && a.max_pages <= kPtCap;
        int32_t v[kPer], phys[kPer];
        if (pt_staged) {
            const int npt = (a.max_pages + L::kThreads - 1) / L::kThreads;   // uniform
            int32_t pw[L::kPtPer];
#pragma unroll
            for (int k = 0; k < L::kPtPer; k++)
                pw[k] = k < npt ? row[min(tid + k * L::kThreads, a.max_pages - 1)] : 0;
#pragma unroll
            for (int i = 0; i < kPer; i++) {
                const int j = tid + i * L::kThreads;
                const int32_t xv = tk[min(j, n_ent - 1)];
                v[i] = j < n_ent ? xv : -1;
            }
#pragma unroll
            for (int k = 0; k < L::kPtPer; k++)
                if (k < npt && tid + k * L::kThreads < a.max_pages) pt_lds[tid + k * L::kThreads] = pw[k];
            __syncthreads();
#pragma unroll
            for (int i = 0; i < kPer; i++)
                phys[i] = pt_lds[min(max(v[i], 0) >> a.page_shift, a.max_pages - 1)];
        } else {
#pragma unroll
            for (int i = 0; i < kPer; i++) {
                const int j = tid + i * L::kThreads;
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
        const TokenIndexRule rule(seq_ok, seq_len, a.page_table != nullptr, a.page_shift, a.max_pages,
                                  a.num_slots);
        int n_err = 0, last = -1;
#pragma unroll
        for (int i = 0; i < kPer; i++) {
            const int j = tid + i * L::kThreads;
            // (a wave past the split's end holds padding only)
            if (w * 64 + i * L::kThreads >= n_ent) continue;
            bool err;
            const int32_t s = rule(v[i], phys[i], err);
            n_err += __builtin_popcountll(__builtin_amdgcn_ballot_w64(err));   // the wave's
            if (j < n_ent)
                slots[j] = s >= 0 ? reinterpret_cast<uint64_t>(a.pool + (int64_t)s * kRawBytes)
                                  : reinterpret_cast<uint64_t>(kZeroRow + (j & (kTile - 1)) * kRawBytes) | kMaskBits;
            const uint64_t vb = __builtin_amdgcn_ballot_w64(j < n_ent && s >= 0);
            if (vb) last = max(last, w * 64 + 63 - (int)__builtin_clzll(vb) + i * L::kThreads);
        }
        if (lane == 0) last_lds[w] = last;
        if (a.err_count && hb == 0 && lane == 0 && n_err) atomicAdd(a.err_count, n_err);
    }
    __syncthreads();
    const uint32_t lds0 = lds_addr(lds);
    int n_tiles = 1;
    auto read_n_tiles = [&] {
        const int4 *lw = reinterpret_cast<const int4 *>(last_lds);
        const int4 v0 = lw[0], v1 = lw[1];
        const int last = max(max(max(v0.x, v0.y), max(v0.z, v0.w)), max(max(v1.x, v1.y), max(v1.z, v1.w)));
        n_tiles = __builtin_amdgcn_readfirstlane(max(1, (last + kTile) / kTile));
    };

    // ---- scoring waves: the tile DMA of their quarter's rows (two rows per
    // instruction: lane l -> row 16q + 2k + (l >> 5), position l & 31
    // holding chunk (l & 31) ^ swz(row)), and the wait for their own rows
    auto row_src = [&](int j, int k) { return slots[j * kTile + 16 * q + 2 * k + (lane >> 5)]; };
    auto issue = [&](int j, const uint64_t (&src)[L::kLoads]) {
        const uint32_t dst = lds0 + (j % kNB) * L::kBufBytes + 16 * q * kRawBytes;
        const int pos = lane & 31;
#pragma unroll
        for (int k = 0; k < L::kLoads; k++) {
            const int r = 16 * q + 2 * k + (lane >> 5);
            dma16(reinterpret_cast<const uint8_t *>((src[k] & ~kMaskBits) + (uint64_t)((pos ^ swz<0>(r)) * 16)),
                  dst + k * 1024);
        }
    };
    auto issue_tile8 = [&](int j) {
        uint64_t src[L::kLoads];
#pragma unroll
        for (int k = 0; k < L::kLoads; k++) src[k] = row_src(j, k);
        issue(j, src);
    };
    // this wave's rows of tile j landed; `issued` is the last tile issued
    auto wait_own = [&](int j, int issued) {
        const int ahead = min(issued, n_tiles - 1) - j;
        if (ahead >= 3) wait_vm_lgkm0<3 * L::kLoads>();
        else if (ahead == 2) wait_vm_lgkm0<2 * L::kLoads>();
        else if (ahead == 1) wait_vm_lgkm0<L::kLoads>();
        else wait_vm_lgkm0<0>();
    };

    // ---- the query copy (tile buffer 3, chunk k of head row hl at
    // position k ^ (hl & 7)), issued by the scoring waves before their first
    // tiles, so that the wait for tile 0 covers it
    uint8_t *const qst = lds + 3 * L::kBufBytes;
    static_assert(kHB * kQRowBytes <= L::kBufBytes, "query copy fits a tile buffer");
    auto q_global = [&](int tq, int hbq, int hl, int byte) {
        const int h = hbq * kHB + hl;
        return reinterpret_cast<const uint8_t *>(a.q) + ((int64_t)tq * a.H + (h < a.H ? h : 0)) * kQRowBytes + byte;
    };
    // this scoring wave's share of the query copy of (token tq, head block hbq)
    auto issue_q = [&](int tq, int hbq) {
        constexpr int kPerWave = kHB * kQChunks / 4;   // chunks copied by each scoring wave
        const uint32_t qbase = lds_addr(qst);
#pragma unroll
        for (int i0 = 0; i0 < kPerWave; i0 += 64) {
            const int i = q * kPerWave + i0 + lane;
            const int hl = i / kQChunks, kp = i % kQChunks;
            dma16(q_global(tq, hbq, hl, (kp ^ (hl & 7)) << 4), qbase + (q * kPerWave + i0) * 16);
        }
    };
    auto q_lds = [&](int hl, int chunk) {
        return reinterpret_cast<const u32x4 *>(qst + hl * kQRowBytes + ((chunk ^ (hl & 7)) << 4));
    };

    // The next unit (virtual block vn) is started while the current one
    // ends: its token's sequence is read at the unit's start, and once the
    // query is taken that sequence's length and page-table row (when it
    // fits) are copied into LDS, where they wait through the unit with no
    // register held; its top-k words are loaded during each role's last
    // step (fetch_next) and resolved into the slot array after it
    // (resolve_next), half by each role; the scoring waves then issue their
    // shares of the next query copy and their rows of the next unit's first
    // two tiles.  After the last step no wave reads a tile buffer or the
    // slot array any more, so all four buffers are free.  Lane (c, g) of
    // scoring wave q (and of PV wave 4 + q) resolves entries
    // (4 i + g) * 64 + 16 q + c: the rows that scoring wave q copies in
    // every tile, so that its copies read only slots it wrote itself.
    constexpr int kPf = kMaxSplit / (4 * kTile);
    const int32_t *const seq_n_lds = reinterpret_cast<const int32_t *>(lds + L::kOffSeqN);
    auto seq_ok_of = [&](int sq) {
        return (a.page_table == nullptr && a.seq_lens == nullptr) || (sq >= 0 && sq < a.num_seqs);
    };
    const bool pt_n_fits = a.page_table != nullptr && a.max_pages <= L::kPtNCap;
    // the next unit's sequence length and page-table row into LDS (scoring
    // waves, once the query is taken; landed, like every copy, by the
    // next-to-last step's wait, or the last step's in a one-tile unit)
    auto stage_next = [&](int sq) {
        const bool sq_ok = seq_ok_of(sq);
        if (pt_n_fits) {
            const int32_t *row = a.page_table + (int64_t)(sq_ok ? sq : 0) * a.max_pages;
            for (int m = q; m * 64 < a.max_pages; m += 4)
                dma4(row + min(m * 64 + lane, a.max_pages - 1), lds0 + L::kOffPtN + m * 256);
        }
        if (q == 0) {
            if (a.seq_lens && sq_ok) dma4(a.seq_lens + sq, lds0 + L::kOffSeqN);
            if (lane == 0) reinterpret_cast<int32_t *>(lds + L::kOffSeqN)[64] = sq;
        }
    };
    // The next unit's entries in two halves: chunks 0-3 (tiles 0-15) by the
    // scoring waves, whose copies of tiles 0 and 1 follow, and chunks 4-7
    // (tiles 16-31) by the PV waves once their last tile is done; wave 4 + q
    // takes quarter q like scoring wave q.  Words are loaded during the
    // role's last step (fetch_next) and resolved after it (resolve_next).
    constexpr int kHalf = kPf / 2;
    // (nu: the next unit, computed once at the unit's start)
    auto fetch_next = [&](const Unit &nu, int qq, int i0, int32_t (&v)[kHalf]) {
        const int n_ent_n = nu.n_ent;
        const int32_t *tk = a.topk + (int64_t)nu.t * a.K + nu.begin;
#pragma unroll
        for (int ii = 0; ii < kHalf; ii++) {
            const int e = (4 * (i0 + ii) + g) * kTile + 16 * qq + c;
            const int32_t xv = tk[min(e, n_ent_n - 1)];
            v[ii] = e < n_ent_n ? xv : -1;
        }
    };
    auto resolve_next = [&](const Unit &nu, int qq, int i0, const int32_t (&v)[kHalf]) {
        const int n_ent_n = nu.n_ent;
        const int sq = __builtin_amdgcn_readfirstlane(seq_n_lds[64]);
        const bool sq_ok = seq_ok_of(sq);
        const int sq_len = (a.seq_lens && sq_ok) ? __builtin_amdgcn_readfirstlane(seq_n_lds[0]) : INT_MAX;
        int32_t phys[kHalf];
        if (pt_n_fits) {
            const int32_t *pt_n = reinterpret_cast<const int32_t *>(lds + L::kOffPtN);
#pragma unroll
            for (int ii = 0; ii < kHalf; ii++) phys[ii] = pt_n[min(max(v[ii], 0) >> a.page_shift, a.max_pages - 1)];
        } else {
            const int32_t *row = a.page_table + (int64_t)(sq_ok ? sq : 0) * a.max_pages;
#pragma unroll
            for (int ii = 0; ii < kHalf; ii++)
                phys[ii] = a.page_table ? row[min(max(v[ii], 0) >> a.page_shift, a.max_pages - 1)] : 0;
        }
        const TokenIndexRule rule(sq_ok, sq_len, a.page_table != nullptr, a.page_shift, a.max_pages,
                                  a.num_slots);
        const uint64_t zero_src = reinterpret_cast<uint64_t>(kZeroRow + (16 * qq + c) * kRawBytes) | kMaskBits;
        int n_err = 0, last = -1;
#pragma unroll
        for (int ii = 0; ii < kHalf; ii++) {
            const int i = i0 + ii;
            // (a chunk past the split's end holds padding only; past it
            // within a chunk, v is -1 and the slot a zero row, never read)
            if (4 * i * kTile >= n_ent_n) continue;
            const int e = (4 * i + g) * kTile + 16 * qq + c;
            bool err;
            const int32_t sl = rule(v[ii], phys[ii], err);
            n_err += __builtin_popcountll(__builtin_amdgcn_ballot_w64(err));
            slots[e] = sl >= 0 ? reinterpret_cast<uint64_t>(a.pool + (int64_t)sl * kRawBytes) : zero_src;
            // the highest tile of chunk i holding a valid entry
            const uint64_t bal = __builtin_amdgcn_ballot_w64(sl >= 0);
            if (bal) last = (4 * i + ((63 - (int)__builtin_clzll(bal)) >> 4)) * kTile;
        }
        if (lane == 0) last_lds[w] = last;
        if (a.err_count && nu.hb == 0 && lane == 0 && n_err) atomicAdd(a.err_count, n_err);
    };
    // scoring waves, after their half: the next query copy and this wave's
    // rows of tiles 0 and 1 (reading its own slot stores, in order)
    auto issue_next = [&](const Unit &nu) {
        asm volatile("" ::: "memory");
        issue_q(nu.t, nu.hb);
#pragma unroll
        for (int j = 0; j < 2; j++)
            if (j * kTile < nu.n_ent) issue_tile8(j);
    };

    if (__builtin_amdgcn_readfirstlane((int)is_v) == 0) {
        // ================= scoring waves =================
        // (from the second unit on, the query copy and tiles 0-1 were issued
        // at the end of the previous one)
        for (int vb = blockIdx.x, pref = 0;; pref = 1) {
            read_n_tiles();
            // the next unit and its token's sequence (a scalar load, waited
            // for with tile 0)
            const int vn = vb + (int)gridDim.x;
            const Unit nu = kPersist ? unit_at(vn) : Unit{0, 0, 0, 0, 0, false};
            const bool has_next = kPersist && nu.valid;
            int sq_n = 0;
            if (has_next) sq_n = a.token_seq ? a.token_seq[nu.t] : nu.t;
            if (!pref) {
                issue_q(t, hb);
                issue_tile8(0);
                if (n_tiles > 1) issue_tile8(1);
            }
            wait_own(0, 1);
            barrier_raw();                       // tile 0 and the query copy landed
            // The query of both head tiles as the B operand.  FP8:
            // bq8[nt][k2] = q8[h][128 k2 + 32 g .. +32] (chunks 8 k2 + 2g, +1);
            // bf16: bq[nt][kk] = q[h][d .. d+8] with d = (4 (kk >> 1) + g) * 16 +
            // 8 (kk & 1), so that a lane's steps 2m, 2m+1 use the two halves of
            // one 16-byte row chunk (the reduction index is free: A and B agree).
            i32x8 bq8[QFP8 ? 2 : 1][QFP8 ? 4 : 1];
            bf16x8 bq[QFP8 ? 1 : 2][QFP8 ? 1 : 16];
#pragma unroll
            for (int nt = 0; nt < 2; nt++) {
                const int hl = nt * 16 + c;
                if constexpr (QFP8) {
#pragma unroll
                    for (int k2 = 0; k2 < 4; k2++) {
                        const u32x4 lo = *q_lds(hl, 8 * k2 + 2 * g), hi = *q_lds(hl, 8 * k2 + 2 * g + 1);
                        bq8[nt][k2] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    }
                } else {
#pragma unroll
                    for (int kk = 0; kk < 16; kk++)
                        // (bf16 row bytes: chunk 2 d / 16)
                        bq[nt][kk] = __builtin_bit_cast(bf16x8, *q_lds(hl, ((4 * (kk >> 1) + g) * 16 + 8 * (kk & 1)) / 8));
                }
            }
            // row chunks of the quarter's row 16q + c: FP8 step k2 takes chunks
            // 8 k2 + 2g and 8 k2 + 2g + 1, bf16 steps 2m, 2m+1 the halves of
            // chunk 4m + g
            u32x4 xc[8];
            auto read_xc = [&](int j) {
                const int r = 16 * q + c;
                const uint8_t *xr = lds + (j % kNB) * L::kBufBytes + r * kRawBytes;
                const int sw = swz<0>(r);
                // chunk ch(m + 4) = ch(m) + 16, and the swizzle (< 16) leaves bit
                // 4 of a chunk index alone: steps m and m + 4 share an address,
                // 256 bytes apart
#pragma unroll
                for (int m = 0; m < 4; m++) {
                    const int ch = QFP8 ? (m >> 1) * 8 + g * 2 + (m & 1) : 4 * m + g;
                    const uint8_t *xa = xr + ((ch ^ sw) * 16);
                    xc[m] = *reinterpret_cast<const u32x4 *>(xa);
                    xc[m + 4] = *reinterpret_cast<const u32x4 *>(xa + 256);
                }
            };
            read_xc(0);
            if (n_tiles > 2) issue_tile8(2);
            wait_lgkm0();
            barrier_raw();                       // every scoring wave holds the query
            if (n_tiles > 3) issue_tile8(3);
            if (has_next) stage_next(sq_n);

            float m_own[2] = {kNoMax, kNoMax};
            // this lane's LDS addresses in the step, less their per-tile parts
            // (head tile nt adds 16 heads: 64 bytes of flags and maxima, 2 KB of
            // P, since the P swizzle (hh >> 1) & 7 does not see nt)
            const uint64_t *const src_l = slots + 16 * q + (lane >> 5);          // + j kTile + 2 i
            const int32_t *const mask_l = reinterpret_cast<const int32_t *>(slots + 16 * q + 4 * g) + 1;
            uint8_t *const flag_l = lds + L::kOffFlags + c * 4 + q;
            float *const mq_l = reinterpret_cast<float *>(lds + L::kOffMq) + c * 4 + q;
            const f32x4 *const mp_l = reinterpret_cast<const f32x4 *>(lds + L::kOffMq) + c;
            uint8_t *const p_l = lds + L::kOffP + p_off(c, 2 * q + (g >> 1)) + (g & 1) * 8;
            int32_t nwords[kHalf];
            // one step: the last one apart (last_step), so that the next
            // unit's words are live only from there on
            auto step = [&](const int k, const bool last_step) {
                if (last_step && has_next) fetch_next(nu, q, 0, nwords);
                // row sources of the tile that refills this step's buffer
                const int nx = k + kNB;
                uint64_t nsrc[L::kLoads];
#pragma unroll
                for (int i = 0; i < L::kLoads; i++) nsrc[i] = src_l[min(nx, n_tiles - 1) * kTile + 2 * i];
                // QK^T of both head tiles over the quarter's 16 entries
                f32x4 part[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
                if constexpr (QFP8) {
                    // one chain per head tile through the accumulator input, the
                    // two chains interleaved: the MFMA adds its C input at full
                    // fp32 precision (only its own 128 products are summed with
                    // fewer bits), so the chain equals fp32 sums of the steps
#pragma unroll
                    for (int k2 = 0; k2 < 4; k2++) {
                        const u32x4 &lo = xc[2 * k2], &hi = xc[2 * k2 + 1];
                        const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
                        for (int nt = 0; nt < 2; nt++)
                            part[nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                av, bq8[nt][k2], part[nt], 0, 0, 0, 127, 0, 127);
                    }
                } else {
                    // bf16 products of the rows converted FP8 -> bf16 exactly
                    // (each converted operand feeds both head tiles), fp32 sums
                    // in two chains per head tile
                    f32x4 accg[2][2];
#pragma unroll
                    for (int nt = 0; nt < 2; nt++) accg[nt][0] = accg[nt][1] = f32x4{0, 0, 0, 0};
#pragma unroll
                    for (int kk = 0; kk < 16; kk++) {
                        const u32x4 &ch = xc[kk >> 1];
                        const bf16x8 av = (kk & 1) ? e4m3x8_to_bf16(ch[2], ch[3]) : e4m3x8_to_bf16(ch[0], ch[1]);
#pragma unroll
                        for (int nt = 0; nt < 2; nt++)
                            accg[nt][kk & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bq[nt][kk], accg[nt][kk & 1], 0, 0, 0);
                    }
#pragma unroll
                    for (int nt = 0; nt < 2; nt++) part[nt] = accg[nt][0] + accg[nt][1];
                }
                // softmax of both head tiles (as attn_kernel's owners): entries
                // 16q + 4g + i of head nt*16 + c.  A masked entry's row is a zero
                // row, so its product is exactly 0 and adding -inf masks it.
                const int par = k & 1;
                float madd[4];
#pragma unroll
                for (int i = 0; i < 4; i++) madd[i] = mask_term(mask_l[2 * (k * kTile + i)]);
                f32x4 mp[2];
#pragma unroll
                for (int nt = 0; nt < 2; nt++) mp[nt] = mp_l[(par ^ 1) * (L::kMqBytes / 16) + nt * 16];
                // the next tile's row chunks, once this wave's rows of it landed
                // (none after the last: every copy has landed then)
                if (!last_step) {
                    wait_own(k + 1, k + 3);
                    read_xc(k + 1);
                }
                float sv[2][4], mx[2];
#pragma unroll
                for (int nt = 0; nt < 2; nt++) {
#pragma unroll
                    for (int i = 0; i < 4; i++) sv[nt][i] = __builtin_fmaf(part[nt][i], sscale, madd[i]);
                    mx[nt] = fmaxf(fmaxf(sv[nt][0], sv[nt][1]), fmaxf(sv[nt][2], sv[nt][3]));
                }
                max_over_g2(mx[0], mx[1]);
#pragma unroll
                for (int nt = 0; nt < 2; nt++) {
                    if (k > 0) {
                        const float r = fmaxf(fmaxf(mp[nt][0], mp[nt][1]), fmaxf(mp[nt][2], mp[nt][3]));
                        m_own[nt] = fmaxf(m_own[nt], r);
                    }
                    const bool moved = mx[nt] - m_own[nt] > kSlack;   // false for an all-masked tile
                    if (moved) m_own[nt] = mx[nt];
                    if (g == 0) flag_l[par * kHB * 4 + nt * 64] = k > 0 && !moved;
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; i++) p[i] = __builtin_amdgcn_exp2f(sv[nt][i] - m_own[nt]);
                    const f16x2 p01 = {(_Float16)p[0], (_Float16)p[1]};
                    const f16x2 p23 = {(_Float16)p[2], (_Float16)p[3]};
                    *reinterpret_cast<u32x2 *>(p_l + par * L::kPBytes + nt * 2048) =
                        u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
                    if (g == 0) mq_l[par * (L::kMqBytes / 4) + nt * 64] = m_own[nt];
                }
                // (in a one-tile unit the next unit's staging copies, issued
                // after the query was taken, have had no wait yet)
                if (last_step && n_tiles == 1) wait_vm_lgkm0<0>();
                else wait_lgkm0();
                barrier_raw();
                if (!last_step && nx < n_tiles) issue(nx, nsrc);
            };
            for (int k = 0; k < n_tiles - 1; k++) step(k, false);
            step(n_tiles - 1, true);
            if (has_next) {
                resolve_next(nu, q, 0, nwords);
                issue_next(nu);
            }
            __syncthreads();                 // the PV waves' epilogue barrier
            vb = vn;
            if (!has_next) break;
            set_unit(nu);
        }
        return;
    }

    // ================= PV waves =================
    for (int vb = blockIdx.x;;) {
        read_n_tiles();
        const int vn = vb + (int)gridDim.x;
        const Unit nu = kPersist ? unit_at(vn) : Unit{0, 0, 0, 0, 0, false};
        const bool has_next = kPersist && nu.valid;
        int32_t nwords[kHalf];
        f32x4 acc[kDT][2], lacc[2];
        float m_ref[2] = {kNoMax, kNoMax};
#pragma unroll
        for (int nt = 0; nt < 2; nt++) {
            lacc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
            for (int dt = 0; dt < kDT; dt++) acc[dt][nt] = f32x4{0, 0, 0, 0};
        }
        // transpose operands of a tile: lane (c, g) addresses entry
        // ks*32 + g*8 + (c >> 1), half (c & 1) of the chunk of dims dbase + 16 dt
        u32x2 tv[2][kDT];
        auto read_tv = [&](int j) {
            const uint8_t *xb = lds + (j % kNB) * L::kBufBytes;
#pragma unroll
            for (int ks = 0; ks < 2; ks++) {
                const int row = ks * 32 + g * 8 + (c >> 1);
                const uint8_t *rp = xb + row * kRawBytes + (c & 1) * 8;
                const int sw = swz<0>(row);
#pragma unroll
                for (int dt = 0; dt < kDT; dt++)
                    tv[ks][dt] = __builtin_bit_cast(
                        u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32(reinterpret_cast<lds_i32x2 *>(
                                   LDS_PTR(rp + (((dbase / 16 + dt) ^ sw) * 16)))));
            }
        };
        // P of tile j (weighted by 2^(m_q - m_ref) while a quarter's maximum
        // differs from the reference, O rescaled when the reference moves), the
        // denominator from the operand (wave 4), then the product over the
        // wave's dims
        // (next >= 0: then the transpose reads of tile next)
        auto pv = [&](int j, int next) {
            const int ppar = j & 1;
            const float *mq_lds = reinterpret_cast<const float *>(lds + L::kOffMq + ppar * L::kMqBytes);
            const uint8_t *p_lds = lds + L::kOffP + ppar * L::kPBytes;
            f16x8 bp[2][2];
#pragma unroll
            for (int nt = 0; nt < 2; nt++)
#pragma unroll
                for (int ks = 0; ks < 2; ks++)
                    bp[nt][ks] = *reinterpret_cast<const f16x8 *>(p_lds + p_off(nt * 16 + c, 4 * ks + g));
            bool uneven = false;
#pragma unroll
            for (int nt = 0; nt < 2; nt++)
                uneven |= *reinterpret_cast<const uint32_t *>(
                              lds + L::kOffFlags + ppar * kHB * 4 + (nt * 16 + c) * 4) != 0x01010101u;
            if (__ballot(uneven) != 0) {
                bool any_resc = false;
                float alpha[2], fq[2][2];
#pragma unroll
                for (int nt = 0; nt < 2; nt++) {
                    const float *mrow = mq_lds + (nt * 16 + c) * 4;
                    const f32x4 mq = *reinterpret_cast<const f32x4 *>(mrow);
                    const float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
                    const bool resc = mx > m_ref[nt];
                    alpha[nt] = resc ? __builtin_amdgcn_exp2f(m_ref[nt] - mx) : 1.0f;
                    if (resc) m_ref[nt] = mx;
                    any_resc |= resc;
                    fq[nt][0] = __builtin_amdgcn_exp2f(mrow[g >> 1] - m_ref[nt]);
                    fq[nt][1] = __builtin_amdgcn_exp2f(mrow[2 + (g >> 1)] - m_ref[nt]);
                }
                if (__ballot(any_resc)) {
#pragma unroll
                    for (int nt = 0; nt < 2; nt++) {
#pragma unroll
                        for (int dt = 0; dt < kDT; dt++) acc[dt][nt] *= alpha[nt];
                        lacc[nt] *= alpha[nt];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
#pragma unroll
                    for (int ks = 0; ks < 2; ks++)
#pragma unroll
                        for (int e = 0; e < 8; e++)
                            bp[nt][ks][e] = (_Float16)((float)bp[nt][ks][e] * fq[nt][ks]);
            }
            if (w == 4) {
                const f16x8 one = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
                for (int nt = 0; nt < 2; nt++)
#pragma unroll
                    for (int ks = 0; ks < 2; ks++)
                        lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(one, bp[nt][ks], lacc[nt], 0, 0, 0);
            }
#pragma unroll
            for (int dt = 0; dt < kDT; dt++) {
                const f16x8 av0 = e4m3x8_to_f16(tv[0][dt][0], tv[0][dt][1]);
                const f16x8 av1 = e4m3x8_to_f16(tv[1][dt][0], tv[1][dt][1]);
#pragma unroll
                for (int nt = 0; nt < 2; nt++) {
                    acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av0, bp[nt][0], acc[dt][nt], 0, 0, 0);
                    acc[dt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av1, bp[nt][1], acc[dt][nt], 0, 0, 0);
                }
            }
            if (next >= 0) read_tv(next);
        };

        barrier_raw();                           // tile 0 and the query copy landed
        read_tv(0);
        wait_lgkm0();
        barrier_raw();                           // (the scoring waves hold the query)
        // step k: the product of tile k - 1, then tile k's transpose reads
        for (int k = 0; k < n_tiles; k++) {
            if (k > 0) pv(k - 1, k);
            if (has_next && k == n_tiles - 1) fetch_next(nu, w - 4, kHalf, nwords);
            wait_lgkm0();
            barrier_raw();
        }
        pv(n_tiles - 1, -1);
        if (has_next) resolve_next(nu, w - 4, kHalf, nwords);

        // epilogue: wave 4's denominators through LDS, then O / l
        if (w == 4 && g == 0) {
#pragma unroll
            for (int nt = 0; nt < 2; nt++) rl_lds[nt * 16 + c] = lacc[nt][0];
        }
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < 2; nt++) {
            const int hh = nt * 16 + c;
            const int h = hb * kHB + hh;
            if (h >= a.H) continue;
            const float l_tot = rl_lds[hh];
            const int64_t th = (int64_t)t * a.H + h;
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            if (SPLIT) {
                const int64_t po = (th * a.n_splits + split) * kD + dbase + 4 * g;
#pragma unroll
                for (int dt = 0; dt < kDT; dt++)
                    store_through(reinterpret_cast<f32x4 *>(a.ws + po + dt * 16), acc[dt][nt] * inv);
                if (w == 4 && g == 0) {
                    float *ml = a.ws + (int64_t)a.T * a.H * a.n_splits * kD + (th * a.n_splits + split) * 2;
                    ml[0] = m_ref[nt];
                    ml[1] = l_tot;
                }
            } else {
                if (OUT_BF16) {
                    store_bf16_tiles<kDT>(reinterpret_cast<uint16_t *>(a.out) + th * kD + dbase, g,
                                          [&](int dt) { return acc[dt][nt] * inv; });
                } else {
                    const int64_t base = th * kD + dbase + 4 * g;
#pragma unroll
                    for (int dt = 0; dt < kDT; dt++)
                        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + base + dt * 16) = acc[dt][nt] * inv;
                }
                if (a.lse && w == 4 && g == 0)
                    a.lse[th] = l_tot > 0.0f ? (m_ref[nt] + log2f(l_tot)) * kLn2 : -INFINITY;
            }
        }
        vb = vn;
        if (!has_next) break;
        set_unit(nu);
    }
}

// Merge of the split partial states: one wavefront per (token, head), each
// lane owning 8 of the 512 dims.  A split holds its normalised output o_s
// (fp32) and (m_s, l_s); the merge is
// sum_s 2^(m_s - M) l_s o_s / sum_s 2^(m_s - M) l_s.  Splits are taken CH at
// a time (CH <= 8, the whole merge for up to eight splits): every split's
// state in a chunk is loaded before any of it is used, so a chunk costs one
// memory latency; chunks are merged online.
template <bool OUT_BF16, int CH>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (th >= (int64_t)a.T * a.H) return;
    const int ns = a.n_splits;
    const float *ml = a.ws + (int64_t)a.T * a.H * ns * kD + th * ns * 2;
    const int64_t ob = th * ns * kD + lane * 8;
    float M = kNoMax, Lsum = 0.0f;
    f32x4 o0 = {0, 0, 0, 0}, o1 = {0, 0, 0, 0};
    for (int s0 = 0; s0 < ns; s0 += CH) {
        float m[CH], l[CH];
        f32x4 v0[CH], v1[CH];
#pragma unroll
        for (int k = 0; k < CH; k++) {
            // splits beyond the last read split 0 and carry no weight
            const int s = s0 + k < ns ? s0 + k : 0;
            m[k] = ml[2 * s];
            l[k] = ml[2 * s + 1];
            v0[k] = *reinterpret_cast<const f32x4 *>(a.ws + ob + (int64_t)s * kD);
            v1[k] = *reinterpret_cast<const f32x4 *>(a.ws + ob + (int64_t)s * kD + 4);
        }
        float Mn = M;
#pragma unroll
        for (int k = 0; k < CH; k++)
            if (s0 + k < ns) Mn = fmaxf(Mn, m[k]);
        // splits with no valid entry carry m = kNoMax, l = 0 and o = 0
        const float r = __builtin_amdgcn_exp2f(M - Mn);
        Lsum *= r;
        o0 *= r;
        o1 *= r;
#pragma unroll
        for (int k = 0; k < CH; k++) {
            const float wgt = s0 + k < ns ? __builtin_amdgcn_exp2f(m[k] - Mn) * l[k] : 0.0f;
            Lsum += wgt;
            o0 += wgt * v0[k];
            o1 += wgt * v1[k];
        }
        M = Mn;
    }
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    o0 *= inv;
    o1 *= inv;
    if (OUT_BF16) {
        u32x4 pk = {pack_bf16x2(o0[0], o0[1]), pack_bf16x2(o0[2], o0[3]),
                    pack_bf16x2(o1[0], o1[1]), pack_bf16x2(o1[2], o1[3])};
        *reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(a.out) + th * kD + lane * 8) = pk;
    } else {
        float *dst = reinterpret_cast<float *>(a.out) + th * kD + lane * 8;
        *reinterpret_cast<f32x4 *>(dst) = o0;
        *reinterpret_cast<f32x4 *>(dst + 4) = o1;
    }
    if (a.lse && lane == 0) a.lse[th] = Lsum > 0.0f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// Heads per workgroup: 32 for raw rows when there are more than 16 heads (a
// row is then gathered once per 32 heads), else 16 (528-byte rows at 32
// heads would need more than the 128 registers a lane has at 16 waves per
// CU).
static int head_tiles(int H, int layout) { return H > 16 && layout == 0 ? 2 : 1; }

constexpr int kMaxSplits = 32;     // K <= 65536 with 2048 entries per split

// Splits per (token, head block): enough workgroups to give each of the
// device's `cus` compute units one (a workgroup fills a CU), and never more
// than kMaxSplit entries per workgroup.
int attn_decode_splits(int T, int H, int K, int layout, int cus) {
    const int hbw = 16 * head_tiles(H, layout);
    const int64_t units = (int64_t)T * ((H + hbw - 1) / hbw);
    const int tiles = K / kTile;
    if (units <= 0 || tiles <= 0) return 1;
    int64_t s = (max(cus, 1) + units - 1) / units;
    const int64_t s_min = (K + kMaxSplit - 1) / kMaxSplit;
    if (s < s_min) s = s_min;
    if (s > tiles) s = tiles;
    if (s > kMaxSplits) s = kMaxSplits;
    const int tps = (int)((tiles + s - 1) / s);
    return (tiles + tps - 1) / tps;
}

static int prefill_splits(int K) { return (K + kMaxSplit - 1) / kMaxSplit; }

static int split_len_for(int K, int splits) {
    const int tiles = K / kTile;
    return ((tiles + splits - 1) / splits) * kTile;
}

int attn_splits(int T, int H, int K, int phase, int layout, int cus) {
    return phase == 0 ? attn_decode_splits(T, H, K, layout, cus) : prefill_splits(K);
}

// Layout 0 has the fewest head blocks and so the most splits: its size
// covers every layout.
size_t attn_workspace_bytes(int T, int H, int K, int phase, int cus) {
    const int s = attn_splits(T, H, K, phase, 0, cus);
    if (s <= 1) return 0;
    size_t b = (size_t)T * H * s * (kD + 2) * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

// Dynamic LDS above the default limit, set once per kernel instantiation (a
// function attribute, not a stream operation, so graph capture is unaffected).
template <auto Kern>
static void allow_big_lds(int bytes) {
    static const hipError_t e = hipFuncSetAttribute(
        (const void *)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    (void)e;
}

template <bool OUT_BF16, int CH>
static void launch_combine(const AttnArgs &a, hipStream_t stream) {
    const dim3 cgrid((unsigned)(((int64_t)a.T * a.H + 3) / 4));
    attn_combine_kernel<OUT_BF16, CH><<<cgrid, dim3(256), 0, stream>>>(a);
}

template <bool OUT_BF16>
static void launch_combine_s(const AttnArgs &a, hipStream_t stream) {
    if (a.n_splits <= 2) return launch_combine<OUT_BF16, 2>(a, stream);
    if (a.n_splits <= 4) return launch_combine<OUT_BF16, 4>(a, stream);
    return launch_combine<OUT_BF16, 8>(a, stream);
}

template <int LAYOUT, bool QFP8, bool OUT_BF16, int NT>
static hipError_t launch_one(const AttnArgs &a, hipStream_t stream) {
    constexpr int kHB = 16 * NT;
    const int n_hb = (a.H + kHB - 1) / kHB;
    const dim3 grid((unsigned)(((int64_t)a.T + 7) / 8 * 8 * n_hb * a.n_splits));
    if constexpr (LAYOUT == 0 && NT == 2) {
        // raw rows in 32-head blocks: the eight-wave kernel, whose
        // workgroups may each take several units (grid_cap)
        const dim3 grid8(a.grid_cap > 0 && (unsigned)a.grid_cap < grid.x ? (unsigned)a.grid_cap : grid.x);
        if (a.n_splits > 1) {
            constexpr auto kern = attn_w8_kernel<QFP8, OUT_BF16, true>;
            allow_big_lds<kern>(W8::kBytes);
            kern<<<grid8, dim3(W8::kThreads), W8::kBytes, stream>>>(a);
            launch_combine_s<OUT_BF16>(a, stream);
        } else {
            constexpr auto kern = attn_w8_kernel<QFP8, OUT_BF16, false>;
            allow_big_lds<kern>(W8::kBytes);
            kern<<<grid8, dim3(W8::kThreads), W8::kBytes, stream>>>(a);
        }
    } else {
        static_assert(NT == 1, "16-head blocks");
        constexpr int bytes = Lds<LAYOUT>::kBytes;
        if (a.n_splits > 1) {
            constexpr auto kern = attn_kernel<LAYOUT, QFP8, OUT_BF16, true>;
            allow_big_lds<kern>(bytes);
            kern<<<grid, dim3(kThreads), bytes, stream>>>(a);
            launch_combine_s<OUT_BF16>(a, stream);
        } else {
            constexpr auto kern = attn_kernel<LAYOUT, QFP8, OUT_BF16, false>;
            allow_big_lds<kern>(bytes);
            kern<<<grid, dim3(kThreads), bytes, stream>>>(a);
        }
    }
    return hipGetLastError();
}

template <int LAYOUT, bool QFP8, bool OUT_BF16>
static hipError_t launch_nt(const AttnArgs &a, hipStream_t stream) {
    if constexpr (LAYOUT == 0) {
        if (head_tiles(a.H, LAYOUT) == 2) return launch_one<LAYOUT, QFP8, OUT_BF16, 2>(a, stream);
    }
    return launch_one<LAYOUT, QFP8, OUT_BF16, 1>(a, stream);
}

hipError_t launch_attn(const AttnArgs &a_in, int layout, bool q_fp8, bool out_bf16,
                       hipStream_t stream) {
    AttnArgs a = a_in;
    // masked entries are marked by kMaskBits in their row source: no pool
    // address may carry any of those bits
    const uint64_t pool_lo = reinterpret_cast<uint64_t>(a.pool);
    const uint64_t pool_hi = pool_lo + (uint64_t)a.num_slots * (uint64_t)kBf16RowBytes;
    if (((pool_lo | pool_hi) & kMaskBits) != 0 || pool_hi < pool_lo) return hipErrorInvalidValue;
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
    DSA_DISPATCH(2, false, false)
    DSA_DISPATCH(2, false, true)
    DSA_DISPATCH(3, false, false)
    DSA_DISPATCH(3, false, true)
#undef DSA_DISPATCH
    return hipErrorInvalidValue;
}

}  // namespace dsa
