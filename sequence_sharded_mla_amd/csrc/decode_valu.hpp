// Vector-ALU partial decode: the float32 path, and the reference-shaped GPU
// path for every cache format.
//
// One workgroup of 256 threads handles one (shard, request, query token,
// chunk) row for a group of 16 query heads.  It walks the shard's local tokens
// in tiles of 32: the tile is decoded to float32 in LDS, each thread forms two
// of the 16 x 32 scores, the 16 threads of a head update that head's running
// max / sum (online softmax), and each thread accumulates 32 of the head's 512
// output dimensions.  Sparse rows first compact the top-K entries this shard
// owns (in entry order, so results are reproducible bit for bit).
#pragma once

#include "common.hpp"
#include "params.hpp"

namespace mla {

namespace valu {

constexpr int kHeads = 16;     // heads per workgroup
constexpr int kTile = 32;      // tokens per tile
constexpr int kKStride = kDk + 1;
constexpr int kThreads = 256;
constexpr int kListCap = 256;  // sparse entries scanned per batch

template <int KV>
__device__ __forceinline__ void load_quad(const uint8_t* row, int d, float* dst) {
    if (KV == MLA_F32) {
        const float4 v = *reinterpret_cast<const float4*>(row + size_t(d) * 4);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    } else if (KV == MLA_BF16) {
        const uint2 v = *reinterpret_cast<const uint2*>(row + size_t(d) * 2);
        dst[0] = bf16_to_f32(uint16_t(v.x)); dst[1] = bf16_to_f32(uint16_t(v.x >> 16));
        dst[2] = bf16_to_f32(uint16_t(v.y)); dst[3] = bf16_to_f32(uint16_t(v.y >> 16));
    } else {
        if (d < kLatent) {
            const uint32_t c = *reinterpret_cast<const uint32_t*>(row + d);
            const float sc = *reinterpret_cast<const float*>(row + kLatent + 4 * (d / kFp8Group));
            dst[0] = e4m3fn_to_f32(c & 0xffu) * sc;
            dst[1] = e4m3fn_to_f32((c >> 8) & 0xffu) * sc;
            dst[2] = e4m3fn_to_f32((c >> 16) & 0xffu) * sc;
            dst[3] = e4m3fn_to_f32(c >> 24) * sc;
        } else {
            const uint2 v = *reinterpret_cast<const uint2*>(row + kLatent + 16 + size_t(d - kLatent) * 2);
            dst[0] = bf16_to_f32(uint16_t(v.x)); dst[1] = bf16_to_f32(uint16_t(v.x >> 16));
            dst[2] = bf16_to_f32(uint16_t(v.y)); dst[3] = bf16_to_f32(uint16_t(v.y >> 16));
        }
    }
}

struct Smem {
    float q[kHeads][kDk];
    float k[kTile][kKStride];
    float p[kHeads][kTile];
    int64_t rowoff[kTile];
    int64_t list[kListCap];
    int32_t wave_cnt[kThreads / 64];
};

// Process one tile of `cnt` rows whose byte offsets are in sm.rowoff.
template <int KV>
__device__ __forceinline__ void tile_step(const DecodeParams& p, Smem& sm, int cnt, float& m,
                                          float& l, float (&acc)[32]) {
    const int tid = threadIdx.x;
    // decode the tile into LDS (rows >= cnt are zero)
    for (int i = tid; i < kTile * (kDk / 4); i += kThreads) {
        const int r = i / (kDk / 4);
        const int d = (i % (kDk / 4)) * 4;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (r < cnt) load_quad<KV>(p.kv + sm.rowoff[r], d, v);
        float* dst = &sm.k[r][d];
        dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
    }
    __syncthreads();

    const int h = tid >> 4;
    const int tl = tid & 15;
    float s[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int t = tl + 16 * u;
        float dot = 0.f;
        for (int d = 0; d < kDk; ++d) dot = fmaf(sm.q[h][d], sm.k[t][d], dot);
        s[u] = t < cnt ? dot * p.scale : -INFINITY;
    }
    const float tmax = group_max<16>(fmaxf(s[0], s[1]));
    const float m_new = fmaxf(m, tmax);
    // rescale of the running state; with no earlier token (m = -inf) the
    // state is zero and the factor is irrelevant
    const float a = (m == -INFINITY) ? 0.f : expf(m - m_new);
    const float e0 = (s[0] == -INFINITY) ? 0.f : expf(s[0] - m_new);
    const float e1 = (s[1] == -INFINITY) ? 0.f : expf(s[1] - m_new);
    l = l * a + group_sum<16>(e0 + e1);
    m = m_new;
    sm.p[h][tl] = e0;
    sm.p[h][tl + 16] = e1;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= a;
    for (int t = 0; t < kTile; ++t) {
        const float pt = sm.p[h][t];
#pragma unroll
        for (int i = 0; i < 32; ++i) acc[i] = fmaf(pt, sm.k[t][tl + 16 * i], acc[i]);
    }
    __syncthreads();
}

template <int KV>
__global__ void __launch_bounds__(kThreads) decode_valu_kernel(DecodeParams p) {
    __shared__ Smem sm;
    RowId id;
    if (!work_item(p, blockIdx.x, id)) return;  // past the last planned item
    const int h0 = blockIdx.y * kHeads;
    const int tid = threadIdx.x;
    const int s = p.shard_begin + id.s_rel;
    const int32_t* bt = p.block_tables + (size_t(id.s_rel) * p.B + id.b) * p.max_blocks;

    // query heads h0 .. h0+15 of (b, t) as float32
    {
        const size_t qbase = (size_t(id.qi) * p.H + h0) * kDk;
        for (int i = tid; i < kHeads * kDk; i += kThreads) {
            float v;
            if (KV == MLA_F32) v = static_cast<const float*>(p.q)[qbase + i];
            else v = bf16_to_f32(static_cast<const uint16_t*>(p.q)[qbase + i]);
            sm.q[i / kDk][i % kDk] = v;
        }
    }
    __syncthreads();

    float m = -INFINITY, l = 0.f;
    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;

    const int32_t L = p.context_lens[id.b];
    int32_t visible = L - id.qlen + id.t + 1;  // positions this query token sees
    if (visible < 0) visible = 0;

    if (p.topk == 0) {
        int32_t local = dev_local_len(visible, s, p.n_shards);
        if ((local + kBlock - 1) / kBlock > p.max_blocks) {
            if (tid == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
            local = p.max_blocks * kBlock;
        }
        const int32_t tok0 = id.chunk * id.chunk_tok;
        int32_t tok1 = id.chunk_tok ? tok0 + id.chunk_tok : local;
        if (tok1 > local) tok1 = local;
        for (int32_t j0 = tok0; j0 < tok1; j0 += kTile) {
            const int cnt = min(kTile, tok1 - j0);
            if (tid < kTile) {
                int64_t off = -1;
                if (tid < cnt) {
                    const int32_t j = j0 + tid;
                    const int32_t blk = bt[j / kBlock];
                    if (blk >= 0 && blk < p.pool_blocks)
                        off = (int64_t(blk) * kBlock + (j % kBlock)) * p.row_bytes;
                    else
                        raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
                }
                sm.rowoff[tid] = off;
            }
            __syncthreads();
            // compact away rows with a bad block id (keeps the order)
            int c = 0;
            if (tid == 0) {
                for (int r = 0; r < cnt; ++r)
                    if (sm.rowoff[r] >= 0) sm.rowoff[c++] = sm.rowoff[r];
                sm.wave_cnt[0] = c;
            }
            __syncthreads();
            c = sm.wave_cnt[0];
            __syncthreads();
            if (c > 0) tile_step<KV>(p, sm, c, m, l, acc);
        }
    } else {
        const int32_t* idx = p.topk_idx + size_t(id.qi) * p.topk;
        const int lane = tid & 63, wave = tid >> 6;
        for (int32_t e0 = 0; e0 < p.topk; e0 += kListCap) {
            const int32_t e = e0 + tid;
            int64_t off = -1;
            if (e < p.topk) {
                const int32_t g = idx[e];
                if (g >= 0) {
                    if (g >= visible) {
                        raise_error(p.err, MLA_DEVERR_INDEX);
                    } else if (g % p.n_shards == s) {
                        const int32_t j = g / p.n_shards;
                        if (j / kBlock >= p.max_blocks) {
                            raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
                        } else {
                            const int32_t blk = bt[j / kBlock];
                            if (blk >= 0 && blk < p.pool_blocks)
                                off = (int64_t(blk) * kBlock + (j % kBlock)) * p.row_bytes;
                            else
                                raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
                        }
                    }
                }
            }
            const uint64_t mask = __ballot(off >= 0);
            const int before = __popcll(mask & ((uint64_t(1) << lane) - 1));
            if (lane == 0) sm.wave_cnt[wave] = __popcll(mask);
            __syncthreads();
            int base = 0, total = 0;
            for (int w = 0; w < kThreads / 64; ++w) {
                if (w < wave) base += sm.wave_cnt[w];
                total += sm.wave_cnt[w];
            }
            if (off >= 0) sm.list[base + before] = off;
            __syncthreads();
            for (int r0 = 0; r0 < total; r0 += kTile) {
                const int cnt = min(kTile, total - r0);
                if (tid < kTile) sm.rowoff[tid] = tid < cnt ? sm.list[r0 + tid] : -1;
                __syncthreads();
                tile_step<KV>(p, sm, cnt, m, l, acc);
            }
        }
    }

    // finalise: O = acc / l, LSE = m + log l; an empty row is (0, -inf)
    const int h = tid >> 4, tl = tid & 15;
    const bool empty = l == 0.f;  // NaN stays visible
    const float inv = empty ? 0.f : 1.f / l;
    const float lse = empty ? -INFINITY : m + logf(l);
    // whole row: the shard's output; a chunk of a split row: its partial slot
    const bool direct = id.slot < 0;
    const size_t head = (direct ? size_t(id.row) : size_t(id.slot)) * p.H + h0 + h;
    // chunk partials stay float32 whatever the output dtype
    if (p.out_dtype == MLA_F32 || !direct) {
        float* o = static_cast<float*>(direct ? p.o_out : p.ws_o) + head * kLatent;
#pragma unroll
        for (int i = 0; i < 32; ++i) o[tl + 16 * i] = acc[i] * inv;
    } else {
        uint16_t* o = static_cast<uint16_t*>(p.o_out) + head * kLatent;
#pragma unroll
        for (int i = 0; i < 32; ++i) o[tl + 16 * i] = uint16_t(bf16x2_rne(acc[i] * inv, 0.f));
    }
    if (tl == 0) (direct ? p.lse_out : p.ws_lse)[head] = lse;
}

}  // namespace valu
}  // namespace mla
