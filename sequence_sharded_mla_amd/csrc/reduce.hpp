// LSE-merge kernels (intra-shard chunk combine, cross-shard merge), index
// localisation and the device-error reset.
//
// The merge of parts (O_s, LSE_s) follows "GLM-5.2 vLLM Decode Context
// Parallelism", sections "See why vLLM 0.26.0 fails" and "Separate the
// backend merge from stable": M = max LSE_s, w_s = exp(LSE_s - M),
// O = sum w_s O_s / sum w_s, LSE = M + log sum w_s; parts with LSE -inf carry
// weight 0 and a row whose parts are all -inf is (0, -inf).  Parts are summed
// in index order, so the result is reproducible bit for bit.
#pragma once

#include "common.hpp"
#include "params.hpp"

namespace mla {

template <typename T>
__device__ __forceinline__ void load4(const T* base, size_t i, float (&v)[4]);

template <>
__device__ __forceinline__ void load4<float>(const float* base, size_t i, float (&v)[4]) {
    const float4 x = *reinterpret_cast<const float4*>(base + i);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}

template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* base, size_t i, float (&v)[4]) {
    const uint2 x = *reinterpret_cast<const uint2*>(base + i);
    v[0] = bf16_to_f32(uint16_t(x.x)); v[1] = bf16_to_f32(uint16_t(x.x >> 16));
    v[2] = bf16_to_f32(uint16_t(x.y)); v[3] = bf16_to_f32(uint16_t(x.y >> 16));
}

__device__ __forceinline__ void store4(void* base, int dtype, size_t i, const float (&v)[4]) {
    if (dtype == MLA_F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(base) + i) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        uint2 x;
        x.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
        x.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + i) = x;
    }
}

// Merge n parts of one row of width 512; 128 threads, 4 dims each.
// part_stride / lse_stride: element distance between consecutive parts.
template <typename T>
__device__ __forceinline__ void merge_row(int n, const T* o, size_t part_stride,
                                          const float* lse, size_t lse_stride, void* out,
                                          int out_dtype, size_t out_off, float* lse_out,
                                          int lane128) {
    float M = -INFINITY;
    for (int s = 0; s < n; ++s) M = fmaxf(M, lse[s * lse_stride]);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    const int d = lane128 * 4;
    if (M != -INFINITY) {
        for (int s = 0; s < n; ++s) {
            const float ls = lse[s * lse_stride];
            if (ls == -INFINITY) continue;
            const float w = expf(ls - M);
            W += w;
            float v[4];
            load4<T>(o, s * part_stride + d, v);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = fmaf(w, v[k], acc[k]);
        }
        const float inv = 1.f / W;
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] *= inv;
    }
    store4(out, out_dtype, out_off + d, acc);
    if (lse_out && lane128 == 0) lse_out[0] = (M == -INFINITY) ? -INFINITY : M + logf(W);
}

// Chunk partials of each (shard, request, query token) row -> that shard's
// O_partial / LSE.  grid = (rows, H / 2), 256 threads = 2 heads.
__global__ void __launch_bounds__(256) chunk_combine_kernel(DecodeParams p) {
    const int row = blockIdx.x;
    const int h = blockIdx.y * 2 + (threadIdx.x >> 7);
    const size_t slot0 = size_t(row) * p.n_chunks * p.H + h;
    const size_t head = size_t(row) * p.H + h;
    merge_row<float>(p.n_chunks, p.ws_o + slot0 * kLatent, size_t(p.H) * kLatent,
                     p.ws_lse + slot0, size_t(p.H), p.o_out, p.out_dtype, head * kLatent,
                     p.lse_out + head, threadIdx.x & 127);
}

// Cross-part merge: grid = ceil(rows / 2), 256 threads = 2 rows.
template <typename T>
__global__ void __launch_bounds__(256) lse_merge_kernel(int n, int64_t rows, const T* o,
                                                         const float* lse, int out_dtype,
                                                         void* out, float* lse_out) {
    const int64_t row = int64_t(blockIdx.x) * 2 + (threadIdx.x >> 7);
    if (row >= rows) return;
    merge_row<T>(n, o + size_t(row) * kLatent, size_t(rows) * kLatent, lse + row, size_t(rows),
                 out, out_dtype, size_t(row) * kLatent, lse_out ? lse_out + row : nullptr,
                 threadIdx.x & 127);
}

__global__ void localize_kernel(const int32_t* g, int64_t count, int32_t shard, int32_t n,
                                int32_t* out) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int32_t v = g[i];
        out[i] = (v >= 0 && v % n == shard) ? v / n : -1;
    }
}

__global__ void clear_word_kernel(uint32_t* w) {
    if (threadIdx.x == 0) w[0] = 0u;
}

}  // namespace mla
