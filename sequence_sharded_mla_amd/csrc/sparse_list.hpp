// Pool rows of the top-K entries each shard owns, for the bf16 matrix-core
// kernel's top-K steps (gfx950).
//
// A top-K list holds global context positions (-1 = padding).  Shard s owns
// position g when g mod N = s, at local index j = g div N, which sits in row
// j mod 64 of block table[s][b][j div 64] ("GLM-5.2 vLLM Decode Context
// Parallelism", sections "Separate the backend merge from stable" and
// "Understand the cache-copy opportunity": indices are localised per shard
// before the shard's attention, with the paged latent cache behind them).
// This pass turns one (shard, query token) row's list into the pool rows of
// the entries that shard owns, in entry order (a repeated position stays one
// entry per repeat), so that the decode kernel can gather them without any
// per-entry arithmetic.
#pragma once

#include "common.hpp"
#include "params.hpp"

namespace mla {

constexpr int kListThreads = 256;

// Entries per row of the list buffer: the list itself rounded up to whole
// 32-entry sub-tiles, so a sub-tile read never leaves the row.
__host__ __device__ constexpr int64_t sparse_list_stride(int32_t topk) { return (int64_t(topk) + 31) / 32 * 32; }

// One workgroup per row (row = s_rel * n_q + qi, as the decode kernels number
// them).  list[row][0 .. count) = pool rows (block id * 64 + row in block) of
// the owned entries in entry order, list[row][count .. stride) = -1,
// count[row] = number of owned entries.  An entry at or past its token's
// visible prefix sets MLA_DEVERR_INDEX and is dropped; an owned entry whose
// local index is past the table or whose block id is outside the pool sets
// MLA_DEVERR_BLOCK_TABLE and is dropped.  Every read is inside the top-K row,
// the block-table row and context_lens; every write inside list[row] and
// count[row].
__global__ void __launch_bounds__(kListThreads) sparse_list_kernel(DecodeParams p, int32_t* list,
                                                                  int32_t* count) {
    __shared__ int32_t wave_cnt[kListThreads / 64];
    RowId id;
    id.row = blockIdx.x;
    split_row(p, id);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t s = p.shard_begin + id.s_rel;
    int32_t visible = p.context_lens[id.b] - id.qlen + id.t + 1;
    if (visible < 0) visible = 0;
    const int32_t* idx = p.topk_idx + size_t(id.qi) * p.topk;
    const int32_t* bt = p.block_tables + (size_t(id.s_rel) * p.B + id.b) * p.max_blocks;
    const int64_t stride = sparse_list_stride(p.topk);
    int32_t* out = list + size_t(id.row) * stride;
    const uint64_t below = (uint64_t(1) << lane) - 1;
    bool bad_index = false, bad_table = false;
    int32_t base = 0;  // owned entries before this pass of kListThreads entries
    for (int32_t e0 = 0; e0 < p.topk; e0 += kListThreads) {
        const int32_t e = e0 + int32_t(threadIdx.x);
        const int32_t g = e < p.topk ? idx[e] : -1;
        bad_index |= g >= visible;
        int32_t row = -1;
        if (g >= 0 && g < visible && g % p.n_shards == s) {
            const int32_t j = g / p.n_shards;
            const int32_t blk = j / kBlock < p.max_blocks ? bt[j / kBlock] : -1;
            if (blk >= 0 && blk < p.pool_blocks) row = blk * kBlock + j % kBlock;
            else bad_table = true;
        }
        const uint64_t mask = __ballot(row >= 0);
        if (lane == 0) wave_cnt[wave] = __popcll(mask);
        __syncthreads();
        int32_t before = base, total = base;
        for (int w = 0; w < kListThreads / 64; ++w) {
            const int32_t c = wave_cnt[w];
            if (w < wave) before += c;
            total += c;
        }
        if (row >= 0) out[before + __popcll(mask & below)] = row;
        base = total;
        __syncthreads();  // wave_cnt is rewritten by the next pass
    }
    for (int64_t i = base + int32_t(threadIdx.x); i < stride; i += kListThreads) out[i] = -1;
    if (threadIdx.x == 0) count[id.row] = base;
    if (__syncthreads_or(bad_index) && threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_INDEX);
    if (__syncthreads_or(bad_table) && threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
}

}  // namespace mla
