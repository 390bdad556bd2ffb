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
// One wave per token row: a 576-value row is at most 2.3 KB, so a wave moves
// it with one or two 16-byte accesses per lane; the per-group maximum is a
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

constexpr int kWaves = 4;  // waves per 256-thread workgroup
constexpr int kTok = 8;    // source rows a wave keeps in flight

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

// Slot of the token at global position `pos` of request `b` on the shards
// p serves, or -1 (another shard's token, or padding).  `bad` is set for a
// table row too narrow for the token or a block id outside the pool.
__device__ __forceinline__ int64_t owner_slot(const SlotParams& p, int32_t b, int32_t pos, bool& bad) {
    bad = false;
    if (pos < 0 || b < 0 || b >= p.B) return -1;
    const int32_t s = pos % p.n_shards;
    const int32_t j = pos / p.n_shards;
    const int32_t rel = s - p.shard_begin;
    if (rel < 0 || rel >= p.shard_count) return -1;
    const int32_t col = j >> 6;
    if (col >= p.max_blocks) {
        bad = true;
        return -1;
    }
    const int32_t blk = p.block_tables[(int64_t(rel) * p.B + b) * p.max_blocks + col];
    if (blk < 0 || int64_t(blk) >= p.pool_blocks) {
        bad = true;
        return -1;
    }
    return int64_t(blk) * kBlock + (j & (kBlock - 1));
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(SlotParams p) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < p.n;
         i += int64_t(gridDim.x) * blockDim.x) {
        bool bad;
        p.slots[i] = owner_slot(p, p.req_idx[i], p.positions[i], bad);
        if (bad && p.err) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
    }
}

struct WriteParams {
    const uint8_t* src;    // [n][576] f32 or bf16
    const int64_t* slots;  // [n], or null when the slots are computed from `map`
    uint8_t* pool;
    uint32_t* err;         // may be null
    int64_t n;
    int64_t pool_rows;
    SlotParams map;        // positions, requests and tables of the fused form
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xf, 0xf, false));
}

// Maximum over the 16 lanes of this lane's DPP row (row_ror by 8, 4, 2, 1).
// The values are bit patterns of non-negative floats, which order as
// unsigned integers.
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
    v = max(v, dpp_u<0x128>(v));
    v = max(v, dpp_u<0x124>(v));
    v = max(v, dpp_u<0x122>(v));
    v = max(v, dpp_u<0x121>(v));
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

// One token's source values in a lane: bf16 source, `a` = latent dims
// 8*lane .. 8*lane+7 and, in lanes 0..7, `r` = rope dims 8*lane ..; f32
// source, `a`, `b` = latent dims 8*lane .. 8*lane+7 and, in lanes 0..15, `r`
// = rope dims 4*lane ...
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct SrcRegs {
    u32x4 a, b, r;
};

template <typename T>
__device__ __forceinline__ T ld(const uint8_t* p) {
    return *reinterpret_cast<const T*>(p);
}

template <typename T>
__device__ __forceinline__ void st(uint8_t* p, T v) {
    *reinterpret_cast<T*>(p) = v;
}

// Every lane loads (the rope of lanes past the rope's width repeats lower
// lanes' addresses, which coalesce), so no load sits in a divergent branch.
template <int SRC>
__device__ __forceinline__ void load_src(SrcRegs& v, const uint8_t* s, int lane) {
    if constexpr (SRC == MLA_BF16) {
        v.a = ld<u32x4>(s + lane * 16);
        v.r = ld<u32x4>(s + kLatent * 2 + (lane & 7) * 16);
    } else {
        v.a = ld<u32x4>(s + lane * 32);
        v.b = ld<u32x4>(s + lane * 32 + 16);
        v.r = ld<u32x4>(s + kLatent * 4 + (lane & 15) * 16);
    }
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int SRC, int KV>
__device__ __forceinline__ void store_row(const SrcRegs& v, uint8_t* row, int lane) {
    float x[8];
    if constexpr (SRC == MLA_BF16) {
        const uint32_t w[4] = {v.a.x, v.a.y, v.a.z, v.a.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            x[2 * k] = lo_bf16(w[k]);
            x[2 * k + 1] = hi_bf16(w[k]);
        }
    } else {
        x[0] = __uint_as_float(v.a.x); x[1] = __uint_as_float(v.a.y);
        x[2] = __uint_as_float(v.a.z); x[3] = __uint_as_float(v.a.w);
        x[4] = __uint_as_float(v.b.x); x[5] = __uint_as_float(v.b.y);
        x[6] = __uint_as_float(v.b.z); x[7] = __uint_as_float(v.b.w);
    }
    if constexpr (KV == MLA_F32) {
        st(row + lane * 32, u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                                  __float_as_uint(x[3])});
        st(row + lane * 32 + 16, u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]),
                                       __float_as_uint(x[6]), __float_as_uint(x[7])});
        if constexpr (SRC == MLA_BF16) {
            if (lane < 8) {
                uint8_t* r = row + kLatent * 4 + lane * 32;
                st(r, u32x4{v.r.x << 16, v.r.x & 0xffff0000u, v.r.y << 16, v.r.y & 0xffff0000u});
                st(r + 16, u32x4{v.r.z << 16, v.r.z & 0xffff0000u, v.r.w << 16, v.r.w & 0xffff0000u});
            }
        } else {
            if (lane < 16) st(row + kLatent * 4 + lane * 16, v.r);
        }
        return;
    }
    // bf16 cache row, or the bf16 rope tail of the packed fp8 row
    constexpr int kRopeOff = KV == MLA_BF16 ? kLatent * 2 : kLatent + 16;
    if constexpr (KV == MLA_BF16) {
        u32x4 out = v.a;
        if constexpr (SRC == MLA_F32)
            out = u32x4{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                        pack_bf16x2(x[6], x[7])};
        st(row + lane * 16, out);
    } else {
        uint32_t abits = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) abits = max(abits, __float_as_uint(x[k]) & 0x7fffffffu);
        const float amax = __uint_as_float(row16_max(abits));
        const float scale = amax > 0.f ? amax / 448.f : 1.f;
        float q[8];
        if (!__ballot(scale < 0x1p-80f || scale > 0x1p100f)) {
            // x / scale, correctly rounded, from a refined reciprocal shared
            // by the group: two residual corrections per element (the same
            // arithmetic as the IEEE division sequence, whose pre- and
            // post-scaling steps are identities while every operand and
            // intermediate stays normal).  With scale in [2^-80, 2^100],
            // elements small enough to make a residual subnormal have
            // |x / scale| < 2^-20 and encode to a signed zero either way;
            // the sign is taken from x.
            float r = __builtin_amdgcn_rcpf(scale);
            r = fmaf(fmaf(-scale, r, 1.f), r, r);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float m = x[k] * r;
                const float f3 = fmaf(fmaf(-scale, m, x[k]), r, m);
                const float f5 = fmaf(fmaf(-scale, f3, x[k]), r, f3);
                q[k] = copysignf(f5, x[k]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = x[k] / scale;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) q[k] = __builtin_amdgcn_fmed3f(q[k], -448.f, 448.f);
        st(row + lane * 8, u32x2{cvt_e4m3x4(q[0], q[1], q[2], q[3]), cvt_e4m3x4(q[4], q[5], q[6], q[7])});
        const int b0 = __builtin_amdgcn_readlane(__float_as_int(scale), 0);
        const int b1 = __builtin_amdgcn_readlane(__float_as_int(scale), 16);
        const int b2 = __builtin_amdgcn_readlane(__float_as_int(scale), 32);
        const int b3 = __builtin_amdgcn_readlane(__float_as_int(scale), 48);
        if (lane == 0) st(row + kLatent, u32x4{uint32_t(b0), uint32_t(b1), uint32_t(b2), uint32_t(b3)});
    }
    if constexpr (SRC == MLA_BF16) {
        if (lane < 8) st(row + kRopeOff + lane * 16, v.r);
    } else {
        if (lane < 16)
            st(row + kRopeOff + lane * 8, u32x2{pack_bf16x2(__uint_as_float(v.r.x), __uint_as_float(v.r.y)),
                                                pack_bf16x2(__uint_as_float(v.r.z), __uint_as_float(v.r.w))});
    }
}

__device__ __forceinline__ int64_t read_slot(int64_t v, int k) {
    const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), k);
    const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(uint64_t(v) >> 32), k);
    return int64_t((uint64_t(hi) << 32) | lo);
}

// Token held by lane `l` of a wave scanning chunks c0, c0 + W, ...
__device__ __forceinline__ int64_t token_of(int64_t c0, int64_t waves, int l) {
    return (c0 + int64_t(l >> 3) * waves) * 8 + (l & 7);
}

// Pops up to kTok tokens from the wave's to-do mask into idx; when the mask
// runs out, the remaining entries repeat the last one (or the previous
// group's last token when nothing is left at all).  Returns the number of
// tokens popped.
__device__ __forceinline__ int take_group(uint64_t& todo, int (&idx)[kTok], int fallback) {
    int cnt = 0;
#pragma unroll
    for (int k = 0; k < kTok; ++k) {
        if (todo) {
            idx[k] = __builtin_ctzll(todo);
            todo &= todo - 1;
            cnt = k + 1;
        } else {
            idx[k] = k ? idx[k - 1] : fallback;
        }
    }
    return cnt;
}

template <int SRC>
__device__ __forceinline__ void load_group(SrcRegs (&v)[kTok], const int (&idx)[kTok], const uint8_t* src,
                                           int64_t c0, int64_t waves, int lane) {
    constexpr int kSrcRow = SRC == MLA_F32 ? kDk * 4 : kDk * 2;
#pragma unroll
    for (int k = 0; k < kTok; ++k)
        load_src<SRC>(v[k], src + token_of(c0, waves, idx[k]) * kSrcRow, lane);
}

template <int SRC, int KV>
__device__ __forceinline__ void store_group(const SrcRegs (&v)[kTok], const int (&idx)[kTok], int cnt,
                                            int64_t mine, uint8_t* pool, int lane) {
    constexpr int kRow = KV == MLA_F32 ? kDk * 4 : KV == MLA_BF16 ? kDk * 2 : kLatent + 16 + kRope * 2;
#pragma unroll
    for (int k = 0; k < kTok; ++k)
        if (k < cnt) store_row<SRC, KV>(v[k], pool + read_slot(mine, idx[k]) * kRow, lane);
}

// Tokens are taken in chunks of 8 consecutive tokens.  With W waves in the
// grid, wave w scans the chunks w, w + W, ..., w + 7W together (lane 8i + j
// holds the slot of token j of its i-th chunk), keeps the tokens this call
// writes (a ballot; rows of the other tokens are never read) and walks them
// kTok at a time, requesting all kTok source rows before converting the
// first.  The grid decides how many chunks a wave scans: waves that write
// several groups in a row measured slower than waves that write one, so
// when every token is written the grid gives one chunk per wave (and waves
// side by side write neighbouring rows of each block), and when one shard of
// N writes, N chunks per wave gather about one group.  Short
// groups repeat a token's load (a cache hit) and store each row once.
// FUSED: the slot of each token comes from its position and request through
// the shards' block tables (owner_slot) instead of a slot array.
template <int SRC, int KV, bool FUSED>
__global__ __launch_bounds__(256) void kv_write_kernel(WriteParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t waves = int64_t(gridDim.x) * kWaves;
    const int64_t n_chunks = (p.n + 7) >> 3;
    for (int64_t c0 = int64_t(blockIdx.x) * kWaves + wave; c0 < n_chunks; c0 += waves * 8) {
        const int64_t t = token_of(c0, waves, lane);
        const bool live = (c0 + (lane >> 3) * waves) < n_chunks && t < p.n;
        int64_t mine = -1;
        bool bad_map = false;
        if (live) {
            if constexpr (FUSED)
                mine = owner_slot(p.map, p.map.req_idx[t], p.map.positions[t], bad_map);
            else
                mine = p.slots[t];
        }
        const uint64_t bad = __ballot(mine >= p.pool_rows);
        if (p.err && lane == 0) {
            if (bad) raise_error(p.err, MLA_DEVERR_SLOT);
        }
        if constexpr (FUSED) {
            if (__ballot(bad_map) && p.err && lane == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
        }
        uint64_t todo = __ballot(mine >= 0 && mine < p.pool_rows);
        while (todo) {
            SrcRegs v[kTok];
            int idx[kTok];
            const int cnt = take_group(todo, idx, 0);
            load_group<SRC>(v, idx, p.src, c0, waves, lane);
            store_group<SRC, KV>(v, idx, cnt, mine, p.pool, lane);
        }
    }
}

}  // namespace kvw
}  // namespace mla
