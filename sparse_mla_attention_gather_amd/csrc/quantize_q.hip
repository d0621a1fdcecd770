// quantize_q.hip -- query cast to E4M3FN with one per-tensor scale.
//
// With no RoPE part the query concat-and-cast step of the FP8-query prefill
// reduces to this cast ("[DSA] Support flashmla_sparse_q8 prefill backend on
// CUDA", review thread).  Two kernels, no atomics and no memset (so the pair
// can be captured in a graph): (1) per-block max |q| into `partials`;
// (2) every block reduces the partials to the same scale (block 0 also
// stores it), then encodes its share.  Given a scale, only (2) runs and reads
// it from device memory.
#include "common.h"
#include "launch.h"

namespace dsa {

constexpr int kQThreads = 256;
// 8 blocks of 4 waves per compute unit: for a 128 MiB query, 2048 blocks of
// 2 loads in flight per thread measured 59 us per cast against 66 us for 1024
// blocks of 4 (4096 blocks: 62; 8192: 80, where the encode's reduction of
// the partial maxima grows with the block count)
constexpr int kQMaxBlocks = 2048;

int quantize_q_blocks(int64_t n_elems) {
    int64_t vecs = n_elems / 8;
    int64_t b = (vecs + kQThreads - 1) / kQThreads;
    if (b > kQMaxBlocks) b = kQMaxBlocks;
    if (b < 1) b = 1;
    return (int)b;
}

__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) v = fmaxf(v, __shfl_xor(v, s));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    v = red[0];
#pragma unroll
    for (int i = 1; i < kQThreads / 64; i++) v = fmaxf(v, red[i]);
    __syncthreads();
    return v;
}

// Each thread keeps kQUnroll 16-byte loads in flight per pass (grid-stride
// over 8-element vectors), so the stream is bandwidth- rather than
// latency-bound.
constexpr int kQUnroll = 2;

__device__ __forceinline__ float amax8(u32x4 raw) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        m = fmaxf(m, fabsf(bf16_bits_to_f32(raw[i] & 0xffffu)));
        m = fmaxf(m, fabsf(bf16_bits_to_f32(raw[i] >> 16)));
    }
    return m;
}

__global__ __launch_bounds__(kQThreads) void q_amax_kernel(
    const uint16_t *__restrict__ q, int64_t n_vec, float *__restrict__ partials) {
    __shared__ float red[kQThreads / 64];
    const u32x4 *qv = reinterpret_cast<const u32x4 *>(q);
    const int64_t stride = (int64_t)gridDim.x * kQThreads;
    float m = 0.0f;
    for (int64_t v = (int64_t)blockIdx.x * kQThreads + threadIdx.x; v < n_vec;
         v += kQUnroll * stride) {
        u32x4 raw[kQUnroll];
#pragma unroll
        for (int u = 0; u < kQUnroll; u++)
            raw[u] = v + u * stride < n_vec ? qv[v + u * stride] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kQUnroll; u++) m = fmaxf(m, amax8(raw[u]));
    }
    m = block_max(m, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

__device__ __forceinline__ u32x2 encode_vec(u32x4 raw, float scale, float rs, bool rs_ok) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        x[2 * i] = bf16_bits_to_f32(raw[i] & 0xffffu);
        x[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
    }
    return encode8_div(x, scale, rs, rs_ok);
}

__global__ __launch_bounds__(kQThreads) void q_encode_kernel(
    const uint16_t *__restrict__ q, int64_t n_vec, uint8_t *__restrict__ q8,
    float *__restrict__ q_scale, const float *__restrict__ partials,
    int n_partials, int scale_given) {
    __shared__ float red[kQThreads / 64];
    float scale;
    if (scale_given) {
        scale = *q_scale;
    } else {
        float m = 0.0f;
        for (int i = threadIdx.x; i < n_partials; i += kQThreads)
            m = fmaxf(m, partials[i]);
        m = block_max(m, red);
        scale = m == 0.0f ? 1.0f : m / 448.0f;               // IEEE division
        if (blockIdx.x == 0 && threadIdx.x == 0) *q_scale = scale;
    }
    // codes of fp32(q / scale), the IEEE quotient (encode8_div)
    const float rs = 1.0f / scale;
    const bool rs_ok = recip_ok(scale);
    const u32x4 *qv = reinterpret_cast<const u32x4 *>(q);
    u32x2 *ov = reinterpret_cast<u32x2 *>(q8);
    const int64_t stride = (int64_t)gridDim.x * kQThreads;
    for (int64_t v = (int64_t)blockIdx.x * kQThreads + threadIdx.x; v < n_vec;
         v += kQUnroll * stride) {
        u32x4 raw[kQUnroll];
#pragma unroll
        for (int u = 0; u < kQUnroll; u++)
            raw[u] = v + u * stride < n_vec ? qv[v + u * stride] : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kQUnroll; u++)
            if (v + u * stride < n_vec) ov[v + u * stride] = encode_vec(raw[u], scale, rs, rs_ok);
    }
}

hipError_t launch_quantize_q(const uint16_t *q, int64_t n_elems, uint8_t *q8,
                             float *q_scale, bool scale_given, float *partials,
                             hipStream_t stream) {
    const int64_t n_vec = n_elems / 8;
    const int blocks = quantize_q_blocks(n_elems);
    if (!scale_given)
        q_amax_kernel<<<dim3(blocks), dim3(kQThreads), 0, stream>>>(q, n_vec, partials);
    q_encode_kernel<<<dim3(blocks), dim3(kQThreads), 0, stream>>>(
        q, n_vec, q8, q_scale, partials, blocks, scale_given ? 1 : 0);
    return hipGetLastError();
}

}  // namespace dsa
