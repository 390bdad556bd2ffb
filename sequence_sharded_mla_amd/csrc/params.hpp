// Kernel parameter block for one decode step over a range of shards.
#pragma once

#include <stdint.h>

namespace mla {

struct DecodeParams {
    const void* q;               // [B][Tq][H][576] f32 or bf16
    const uint8_t* kv;           // [pool_blocks][64][row_bytes]
    const int32_t* block_tables; // [shard_count][B][max_blocks]
    const int32_t* context_lens; // [B]
    const int32_t* topk_idx;     // [B][Tq][topk] or null
    void* o_out;                 // [shard_count][B*Tq][H][512] out dtype
    float* lse_out;              // [shard_count][B*Tq][H]
    float* ws_o;                 // [rows][n_chunks][H][512] (n_chunks > 1)
    float* ws_lse;               // [rows][n_chunks][H]
    uint32_t* ws_cnt;            // [rows]
    uint32_t* err;               // device error word
    int64_t pool_blocks;
    int32_t row_bytes;
    int32_t B, Tq, H, max_blocks, topk;
    int32_t shard_begin, shard_count, n_shards;
    int32_t n_chunks, tiles_per_chunk;
    int32_t out_dtype;
    float scale;
};

// (shard, request, query token, chunk) of a flat work index.
struct RowId {
    int32_t s_rel, b, t, chunk, row;
};

__device__ __forceinline__ RowId decode_row(const DecodeParams& p, int32_t idx) {
    RowId r;
    r.chunk = idx % p.n_chunks;
    r.row = idx / p.n_chunks;
    r.t = r.row % p.Tq;
    const int32_t bt = r.row / p.Tq;
    r.b = bt % p.B;
    r.s_rel = bt / p.B;
    return r;
}

}  // namespace mla
