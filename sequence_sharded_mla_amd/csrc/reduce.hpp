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

// 8 consecutive elements of a part row as float.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}

__device__ __forceinline__ void store8(void* base, int dtype, size_t i, const float (&v)[8]) {
    if (dtype == MLA_F32) {
        float* o = static_cast<float*>(base) + i;
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint4 x;
        x.x = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
        x.y = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
        x.z = uint32_t(f32_to_bf16(v[4])) | (uint32_t(f32_to_bf16(v[5])) << 16);
        x.w = uint32_t(f32_to_bf16(v[6])) | (uint32_t(f32_to_bf16(v[7])) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + i) = x;
    }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Merge n parts of one row of width 512 with one wave: lane i accumulates
// dims 8 i .. 8 i + 7; the weights of 64 parts at a time live one per lane.
// part_stride / lse_stride: element distance between consecutive parts.
// Parts are added in index order, so the result is reproducible bit for bit.
template <typename T>
__device__ __forceinline__ void merge_wave(int n, const T* o, size_t part_stride, const float* lse,
                                           size_t lse_stride, void* out, int out_dtype,
                                           size_t out_off, float* lse_out, int lane) {
    float M = -INFINITY;
    for (int s0 = 0; s0 < n; s0 += 64)
        M = fmaxf(M, s0 + lane < n ? lse[size_t(s0 + lane) * lse_stride] : -INFINITY);
    M = wave_max(M);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    const T* base = o + lane * 8;
    constexpr int kBatch = 8;  // parts whose loads are in flight together
    for (int s0 = 0; s0 < n; s0 += 64) {
        const float ls = s0 + lane < n ? lse[size_t(s0 + lane) * lse_stride] : -INFINITY;
        const float w = (ls == -INFINITY) ? 0.f : expf(ls - M);  // M = -inf: every w is 0
        W += w;
        const int cnt = min(64, n - s0);
        for (int k0 = 0; k0 < cnt; k0 += kBatch) {
            float v[kBatch][8];
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if (k0 + k < cnt) load8<T>(base + size_t(s0 + k0 + k) * part_stride, v[k]);
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (k0 + k >= cnt) break;
                const float ws = __shfl(w, k0 + k);
                // a part of weight 0 (LSE -inf) contributes nothing, whatever
                // its values; the test is uniform over the wave
                if (ws != 0.f) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[k][e], acc[e]);
                }
            }
        }
    }
    W = wave_sum(W);
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    store8(out, out_dtype, out_off + lane * 8, acc);
    if (lse_out && lane == 0) lse_out[0] = (M == -INFINITY) ? -INFINITY : M + logf(W);
}

// Chunk partials of each (shard, request, query token) row -> that shard's
// O_partial / LSE.  grid = (rows, H / 4), 256 threads = 4 heads.
__global__ void __launch_bounds__(256) chunk_combine_kernel(DecodeParams p) {
    const int row = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    const size_t slot0 = size_t(row) * p.n_chunks * p.H + h;
    const size_t head = size_t(row) * p.H + h;
    merge_wave<float>(p.n_chunks, p.ws_o + slot0 * kLatent, size_t(p.H) * kLatent,
                      p.ws_lse + slot0, size_t(p.H), p.o_out, p.out_dtype, head * kLatent,
                      p.lse_out + head, threadIdx.x & 63);
}

// Cross-part merge: grid = ceil(rows / 4), 256 threads = 4 rows.
template <typename T>
__global__ void __launch_bounds__(256) lse_merge_kernel(int n, int64_t rows, const T* o,
                                                         const float* lse, int out_dtype,
                                                         void* out, float* lse_out) {
    const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    merge_wave<T>(n, o + size_t(row) * kLatent, size_t(rows) * kLatent, lse + row, size_t(rows),
                  out, out_dtype, size_t(row) * kLatent, lse_out ? lse_out + row : nullptr,
                  threadIdx.x & 63);
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
