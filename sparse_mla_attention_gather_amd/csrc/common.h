// common.h -- device-side types and helpers shared by the gfx950 kernels.
//
// FP8 here is the OCP E4M3FN format (bias 7, no infinities, S.1111.111 is
// NaN), the flavour the SGLang pages require on this path ("extend CUDA
// TileLang raw FP8 KV path", Modifications: E4M3FNUZ is rejected).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 512;          // latent width (kv_lora_rank)
constexpr int kGroup = 128;      // elements per scale group (528-byte rows)
constexpr int kRawBytes = 512;
constexpr int kScaledBytes = 528;
// 656-byte RoPE rows: the 528-byte scaled row, then 64 little-endian bf16
// RoPE values (the pages give only the size; this split is the reading)
constexpr int kRopeDim = 64;
constexpr int kRopeRowBytes = 656;
constexpr int kBf16RowBytes = 1024;   // 512 bf16 values, no cast

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// fp32 -> E4M3FN code: round to nearest even, +-inf and finite values whose
// magnitude is at least 448 saturate to +-448 (0x7E), NaN -> 0x7F with the
// input's sign, -0 -> 0x80.  Written on the fp32 bit pattern:
//   |x| <  2^-6  : subnormal band, code = rint(|x| * 2^9)  (0..8; 8 is the
//                  smallest normal's code 0x08);
//   2^-6 <= |x| < 448 : add half an ulp of a 3-bit mantissa (ties to even) at
//                  bit 20 and re-bias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
    uint32_t u = __float_as_uint(x);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return sign | 0x7fu;          // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;         // >= 448 (and inf)
    if (a < 0x3c800000u) {                             // < 2^-6
        float t = __uint_as_float(a) * 512.0f;         // exact scaling
        return sign | (uint32_t)__builtin_rintf(t);
    }
    uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
    uint32_t e = (r >> 23) - 120u;                     // 127 -> 7
    uint32_t m = (r >> 20) & 7u;
    return sign | (e << 3) | m;
}

// Four fp32 -> four E4M3FN codes packed little-endian in a uint32 (f32_to_e4m3
// on each).
__device__ __forceinline__ uint32_t pack4_e4m3_sw(float a, float b, float c, float d) {
    return f32_to_e4m3(a) | (f32_to_e4m3(b) << 8) | (f32_to_e4m3(c) << 16) |
           (f32_to_e4m3(d) << 24);
}

// The same codes by the gfx950 converter, for inputs that are not NaN.
// v_cvt_pk_fp8_f32 rounds to nearest even exactly as f32_to_e4m3 does but
// turns magnitudes above 464 into NaN; clamping to +-448 first (v_med3) makes
// it saturate like f32_to_e4m3 for every finite value and +-inf (compared on
// the device over all 2^32 fp32 patterns).  The clamp does not return NaN.
__device__ __forceinline__ uint32_t pack4_e4m3_hw(float a, float b, float c, float d) {
    const auto clamp = [](float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(a), clamp(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(clamp(c), clamp(d), w, true);
    return (uint32_t)w;
}

// Eight fp32 -> eight E4M3FN codes: the converter, or f32_to_e4m3 on the
// (normally never taken) branch for a group holding a NaN.
__device__ __forceinline__ u32x2 encode8(const float (&x)[8]) {
    bool nan = false;
#pragma unroll
    for (int i = 0; i < 8; i++) nan |= __builtin_isnan(x[i]);
    // wave-uniform branch (a ballot): kept as a branch, not blended per lane
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(nan) != 0, 0))
        return u32x2{pack4_e4m3_sw(x[0], x[1], x[2], x[3]), pack4_e4m3_sw(x[4], x[5], x[6], x[7])};
    return u32x2{pack4_e4m3_hw(x[0], x[1], x[2], x[3]), pack4_e4m3_hw(x[4], x[5], x[6], x[7])};
}

// Codes of the IEEE quotients fp32(x[i] / s) for a divisor used many times,
// with r = 1/s (IEEE, computed once; r_ok: s and r normal).  q = x * r is
// within two fp32 ulps of the IEEE quotient (relative error <= 2^-23 for
// normal s and q), so both have the same code unless q lies within a few
// ulps of a point halfway between two codes (fp32 mantissa bits 19..0 near
// 0x80000 in the normal band) or in the subnormal band (0 < |q| < 2^-6).  A
// wave holding such a value, a NaN, or a divisor without a usable 1/s takes
// the IEEE division and f32_to_e4m3 for all its values instead (a
// wave-uniform branch; about 1.5e-4 of normally distributed values trigger
// it, so under a tenth of the 512-value waves).
__device__ __forceinline__ u32x2 encode8_div(const float (&x)[8], float s, float r, bool r_ok) {
    float q[8];
    bool slow = !r_ok;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        q[i] = x[i] * r;
        const float m = fabsf(q[i]);
        const uint32_t lo = (__float_as_uint(q[i]) - 0x7fff8u) & 0xfffffu;
        slow |= (m < 0x1p-6f && m != 0.0f) | (lo < 16u) | (m != m);
    }
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(slow) != 0, 0)) {
#pragma unroll
        for (int i = 0; i < 8; i++) q[i] = x[i] / s;
        return u32x2{pack4_e4m3_sw(q[0], q[1], q[2], q[3]), pack4_e4m3_sw(q[4], q[5], q[6], q[7])};
    }
    return u32x2{pack4_e4m3_hw(q[0], q[1], q[2], q[3]), pack4_e4m3_hw(q[4], q[5], q[6], q[7])};
}

// 1/s is usable by encode8_div: s and 1/s normal and finite.
__device__ __forceinline__ bool recip_ok(float s) {
    const float m = fabsf(s);
    return m >= 0x1p-120f && m <= 0x1p120f;
}

// Exact E4M3FN -> bf16 / f16 conversions of the two codes in the low (hi =
// false) or high half of a 32-bit word, through gfx950's OCP FP8 converts
// with a unit scale.
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_to_bf16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
}
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w, 1.0f, HI);
}

// Eight codes (two little-endian words) -> bf16x8 / f16x8, element order kept.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
    bf16x2 a = e4m3x2_to_bf16<false>(w0), b = e4m3x2_to_bf16<true>(w0);
    bf16x2 c = e4m3x2_to_bf16<false>(w1), d = e4m3x2_to_bf16<true>(w1);
    bf16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}
__device__ __forceinline__ f16x8 e4m3x8_to_f16(uint32_t w0, uint32_t w1) {
    f16x2 a = e4m3x2_to_f16<false>(w0), b = e4m3x2_to_f16<true>(w0);
    f16x2 c = e4m3x2_to_f16<false>(w1), d = e4m3x2_to_f16<true>(w1);
    f16x8 r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
}

// Resolution of a token's top-k entry values i (the attention's prologues
// and the index transform apply the same rule), each given the page-table
// word `phys` already fetched for it: -1 -> padding (not an error); a
// negative value, a token whose sequence is invalid, i >= seq_len, a page
// beyond max_pages or a negative page-table word, or a slot >= num_slots ->
// masked and counted (`err`).  page_shift = log2(page_size); has_pt false:
// i is the slot.
struct TokenIndexRule {
    uint32_t lim;        // valid positions are below it (0: none)
    int shift;
    uint32_t pmask;
    bool has_pt;
    int64_t num_slots;
    // the token's checks folded into one bound: a valid position is below
    // the sequence length and below the page table's reach, so one unsigned
    // compare covers i < 0, an invalid sequence, i >= seq_len and a page
    // beyond max_pages
    __device__ __forceinline__ TokenIndexRule(bool seq_ok, int seq_len, bool has_pt_, int page_shift,
                                              int max_pages, int64_t num_slots_)
        : lim(!seq_ok ? 0u
                      : (uint32_t)max((int64_t)0, has_pt_ ? min((int64_t)seq_len, (int64_t)max_pages << page_shift)
                                                          : (int64_t)seq_len)),
          shift(page_shift), pmask((1u << page_shift) - 1u), has_pt(has_pt_), num_slots(num_slots_) {}
    // the slot of entry i (phys: its page-table word, unused without a page
    // table), or -1; err: masked other than as padding.  Nothing is branched
    // on per entry: callers resolve several entries per lane, where a lane's
    // branches cost more than the selects.
    __device__ __forceinline__ int32_t operator()(int32_t i, int32_t phys, bool &err) const {
        const int64_t slot = has_pt ? (int64_t)(((uint64_t)(uint32_t)phys << shift) | ((uint32_t)i & pmask))
                                    : (int64_t)i;
        const bool ok = (uint32_t)i < lim && (!has_pt || phys >= 0) && slot < num_slots;
        err = !ok && i != -1;
        return ok ? (int32_t)slot : -1;
    }
};

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace dsa
