// kv_write.hip -- fused cast-to-FP8 paged KV writer.
//
// One kernel both casts a bf16 latent row to FP8 and scatters it into its
// pool slot, for the raw 512-byte and the group-scaled 528-byte layouts
// ("extend CUDA TileLang raw FP8 KV path", Modifications; "[DSA] Support
// group-scaled FP8 NoPE KV reads for CUDA TileLang", Motivation: 512 FP8
// values followed by four fp32 scales, one per 128 values), and the 656-byte
// RoPE layout the same page says the readers keep (the scaled row followed by
// the row's 64 RoPE values, copied as bf16); bf16 rows are stored as given
// (the 1024-byte pool the raw page compares against).
//
// Mapping: one 64-lane wavefront per row; lane l owns elements [8l, 8l+8)
// (one 16-byte load of bf16, one 8-byte store of codes), so a 128-element
// scale group is 16 adjacent lanes and its max is a 4-step lane reduction.
// Memory-bound: 1024 B read + 512/528 B written per row.
#include "common.h"
#include "launch.h"

namespace dsa {

template <int LAYOUT>
__global__ __launch_bounds__(256) void kv_write_kernel(
    const uint16_t *__restrict__ kv, int64_t n, int64_t row_stride,
    const int64_t *__restrict__ slot_mapping, uint8_t *__restrict__ pool,
    int64_t num_slots, int32_t *__restrict__ err_count) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= n) return;
    const int64_t slot = slot_mapping[row];
    if (slot < 0) return;
    if (slot >= num_slots) {
        if (lane == 0 && err_count) atomicAdd(err_count, 1);
        return;
    }
    const u32x4 raw = *reinterpret_cast<const u32x4 *>(kv + row * row_stride + lane * 8);
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        x[2 * i] = bf16_bits_to_f32(raw[i] & 0xffffu);
        x[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
    }
    constexpr int64_t kRow = LAYOUT == 0 ? kRawBytes : LAYOUT == 1 ? kScaledBytes
                             : LAYOUT == 2 ? kRopeRowBytes : kBf16RowBytes;
    uint8_t *dst = pool + slot * kRow;
    if (LAYOUT == 3) {
        // bf16 rows: the 16 input bytes as they are
        *reinterpret_cast<u32x4 *>(dst + lane * 16) = raw;
    } else if (LAYOUT == 0) {
        *reinterpret_cast<u32x2 *>(dst + lane * 8) = encode8(x);
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++) amax = fmaxf(amax, fabsf(x[i]));
        // max over the 16 lanes of this 128-element group
#pragma unroll
        for (int s = 1; s < 16; s <<= 1) amax = fmaxf(amax, __shfl_xor(amax, s));
        const float scale = amax == 0.0f ? 1.0f : amax / 448.0f;   // IEEE division
        // codes of fp32(x / scale), the IEEE quotient
        *reinterpret_cast<u32x2 *>(dst + lane * 8) =
            encode8_div(x, scale, 1.0f / scale, recip_ok(scale));
        if ((lane & 15) == 0)
            *reinterpret_cast<float *>(dst + kD + 4 * (lane >> 4)) = scale;
        if (LAYOUT == 2 && lane < kRopeDim / 8) {
            // the RoPE values after the latent: 16 bytes per lane
            const u32x4 r = *reinterpret_cast<const u32x4 *>(kv + row * row_stride + kD + lane * 8);
            *reinterpret_cast<u32x4 *>(dst + kScaledBytes + lane * 16) = r;
        }
    }
}

hipError_t launch_kv_write(const uint16_t *kv, int64_t n, int64_t row_stride,
                           const int64_t *slot_mapping, uint8_t *pool,
                           int64_t num_slots, int layout, int32_t *err_count,
                           hipStream_t stream) {
    const int64_t blocks = (n + 3) / 4;
    if (layout == 0)
        kv_write_kernel<0><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            kv, n, row_stride, slot_mapping, pool, num_slots, err_count);
    else if (layout == 1)
        kv_write_kernel<1><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            kv, n, row_stride, slot_mapping, pool, num_slots, err_count);
    else if (layout == 2)
        kv_write_kernel<2><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            kv, n, row_stride, slot_mapping, pool, num_slots, err_count);
    else
        kv_write_kernel<3><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
            kv, n, row_stride, slot_mapping, pool, num_slots, err_count);
    return hipGetLastError();
}

}  // namespace dsa
