// Writing new tokens into the sequence-sharded paged cache (gfx950).
//
// Two steps ahead of decode attention:
//
// * slot_mapping_kernel: the cache slot each new token takes on the shards
//   this call serves.  Global position p of request b belongs to shard
//   p mod N as its local token j = p div N ("How vLLM Serves GLM-5.3 with
//   Million-Token Contexts on 16 H200s", section "The core design"); the
//   slot is row j mod 64 of block block_table[b][j div 64].  Tokens owned by
//   other shards get -1.
// * kv_write_kernel: stores each token whose slot is >= 0 in the cache's row
//   format.  A negative slot means another rank owns the token's KV (or the
//   token is padding): the write is skipped, which is the only thing KV
//   ownership suppresses ("GLM-5.2 vLLM Decode Context Parallelism", section
//   "Keep the current-main correctness blocker visible").  For the packed
//   fp8 row the 512 latent values are quantised per 128-dimension group:
//   scale = max |x| / 448 (1 for an all-zero group), code = x / scale
//   rounded to the nearest E4M3FN value (ties to even), saturating at +-448;
//   both divisions are IEEE float32.  The rope part is stored as bf16.
//
// One wave per token: a 576-value row is at most 2.3 KB, so a wave moves it
// with one or two 16-byte accesses per lane; the per-group maximum is a
// 16-lane DPP reduction (one DPP row per 128-dim group).  Tokens whose slot
// is negative are skipped before their source row is read, so a rank reads
// only its own share of the new tokens.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_dcp.h"
#include "common.hpp"

namespace mla {
namespace kvw {

constexpr int kWaves = 4;  // tokens in flight per 256-thread workgroup

struct SlotParams {
    const int32_t* req_idx;
    const int32_t* positions;
    const int32_t* block_tables;  // [shard_count][B][max_blocks]
    int64_t* slots;
    uint32_t* err;                // may be null
    int64_t n;
    int64_t pool_blocks;
    int32_t B, max_blocks, shard_begin, shard_count, n_shards;
};

__global__ __launch_bounds__(256) void slot_mapping_kernel(SlotParams p) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < p.n;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int32_t b = p.req_idx[i];
        const int32_t pos = p.positions[i];
        int64_t slot = -1;
        if (pos >= 0 && b >= 0 && b < p.B) {
            const int32_t s = pos % p.n_shards;
            const int32_t j = pos / p.n_shards;
            const int32_t rel = s - p.shard_begin;
            if (rel >= 0 && rel < p.shard_count) {
                const int32_t col = j >> 6;
                bool bad = col >= p.max_blocks;
                if (!bad) {
                    const int32_t blk =
                        p.block_tables[(int64_t(rel) * p.B + b) * p.max_blocks + col];
                    bad = blk < 0 || int64_t(blk) >= p.pool_blocks;
                    if (!bad) slot = int64_t(blk) * kBlock + (j & (kBlock - 1));
                }
                if (bad && p.err) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
            }
        }
        p.slots[i] = slot;
    }
}

struct WriteParams {
    const uint8_t* src;    // [n][576] f32 or bf16
    const int64_t* slots;  // [n]
    uint8_t* pool;
    uint32_t* err;         // may be null
    int64_t n;
    int64_t pool_rows;
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Maximum over the 16 lanes of this lane's DPP row (row_ror by 8, 4, 2, 1).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dpp_f<0x128>(v));
    v = fmaxf(v, dpp_f<0x124>(v));
    v = fmaxf(v, dpp_f<0x122>(v));
    v = fmaxf(v, dpp_f<0x121>(v));
    return v;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
}

// Four float32 quotients -> four E4M3FN codes (RNE), packed little-endian.
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return uint32_t(w);
}

template <int SRC, int KV>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteParams p) {
    constexpr int kSrcRow = SRC == MLA_F32 ? kDk * 4 : kDk * 2;
    constexpr int kRow = KV == MLA_F32 ? kDk * 4 : KV == MLA_BF16 ? kDk * 2 : kLatent + 16 + kRope * 2;
    const int lane = threadIdx.x & 63;
    const int64_t first = int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6);
    const int64_t step = int64_t(gridDim.x) * kWaves;
    for (int64_t t = first; t < p.n; t += step) {
        const int64_t slot = p.slots[t];
        if (slot < 0) continue;
        if (slot >= p.pool_rows) {
            if (lane == 0 && p.err) raise_error(p.err, MLA_DEVERR_SLOT);
            continue;
        }
        const uint8_t* s = p.src + t * kSrcRow;
        uint8_t* row = p.pool + slot * kRow;

        // latent dims 8*lane .. 8*lane+7 as float32 (and the raw bf16 bits)
        float x[8];
        uint4 raw_lat{};
        if constexpr (SRC == MLA_BF16) {
            raw_lat = *reinterpret_cast<const uint4*>(s + lane * 16);
            const uint32_t w[4] = {raw_lat.x, raw_lat.y, raw_lat.z, raw_lat.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[2 * k] = __uint_as_float(w[k] << 16);
                x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
            }
        } else {
            const float4 a = *reinterpret_cast<const float4*>(s + lane * 32);
            const float4 b = *reinterpret_cast<const float4*>(s + lane * 32 + 16);
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        }
        // rope: bf16 source, lanes 0..7 hold 8 values; f32 source, lanes
        // 0..15 hold 4 values
        uint4 raw_rope{};
        float4 f_rope{};
        if constexpr (SRC == MLA_BF16) {
            if (lane < 8) raw_rope = *reinterpret_cast<const uint4*>(s + kLatent * 2 + lane * 16);
        } else {
            if (lane < 16) f_rope = *reinterpret_cast<const float4*>(s + kLatent * 4 + lane * 16);
        }

        if constexpr (KV == MLA_F32) {
            float4* dst = reinterpret_cast<float4*>(row + lane * 32);
            dst[0] = make_float4(x[0], x[1], x[2], x[3]);
            dst[1] = make_float4(x[4], x[5], x[6], x[7]);
            if constexpr (SRC == MLA_BF16) {
                if (lane < 8) {
                    const uint32_t w[4] = {raw_rope.x, raw_rope.y, raw_rope.z, raw_rope.w};
                    float4* r = reinterpret_cast<float4*>(row + kLatent * 4 + lane * 32);
                    r[0] = make_float4(__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                       __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u));
                    r[1] = make_float4(__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                       __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u));
                }
            } else {
                if (lane < 16) *reinterpret_cast<float4*>(row + kLatent * 4 + lane * 16) = f_rope;
            }
        } else {
            // bf16 cache row, or the bf16 rope tail of the packed fp8 row
            constexpr int kRopeOff = KV == MLA_BF16 ? kLatent * 2 : kLatent + 16;
            if constexpr (KV == MLA_BF16) {
                uint4 out = raw_lat;
                if constexpr (SRC == MLA_F32)
                    out = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                     pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7]));
                *reinterpret_cast<uint4*>(row + lane * 16) = out;
            } else {
                float amax = 0.f;
#pragma unroll
                for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(x[k]));
                amax = row16_max(amax);
                const float scale = amax > 0.f ? amax / 448.f : 1.f;
                float q[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) q[k] = fminf(fmaxf(x[k] / scale, -448.f), 448.f);
                *reinterpret_cast<uint2*>(row + lane * 8) =
                    make_uint2(cvt_e4m3x4(q[0], q[1], q[2], q[3]), cvt_e4m3x4(q[4], q[5], q[6], q[7]));
                const int b0 = __builtin_amdgcn_readlane(__float_as_int(scale), 0);
                const int b1 = __builtin_amdgcn_readlane(__float_as_int(scale), 16);
                const int b2 = __builtin_amdgcn_readlane(__float_as_int(scale), 32);
                const int b3 = __builtin_amdgcn_readlane(__float_as_int(scale), 48);
                if (lane == 0)
                    *reinterpret_cast<int4*>(row + kLatent) = make_int4(b0, b1, b2, b3);
            }
            if constexpr (SRC == MLA_BF16) {
                if (lane < 8) *reinterpret_cast<uint4*>(row + kRopeOff + lane * 16) = raw_rope;
            } else {
                if (lane < 16)
                    *reinterpret_cast<uint2*>(row + kRopeOff + lane * 8) =
                        make_uint2(pack_bf16x2(f_rope.x, f_rope.y), pack_bf16x2(f_rope.z, f_rope.w));
            }
        }
    }
}

}  // namespace kvw
}  // namespace mla
