// Kernel parameter block for one decode step over a range of shards, and the
// mapping from a workgroup to its unit of work.
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
    void* ws_o;                  // partials of split rows: [slots][H][512] out dtype
    float* ws_lse;               // [slots][H]
    const int32_t* items;        // [n][4] row, chunk, partial slot (-1: whole row), 0;
                                 // null: one item per row, covering all of it
    const int32_t* row_info;     // [rows][2] first partial slot (-1: none), items of the row
    const int32_t* plan_hdr;     // [0] error word, [1] item count, [2] tokens per chunk
    uint32_t* err;               // device error word
    int64_t pool_blocks;
    int32_t row_bytes;
    int32_t B, Tq, H, max_blocks, topk;
    int32_t shard_begin, shard_count, n_shards;
    int32_t rows;
    int32_t out_dtype;
    float scale;
};

// One unit of work: a (shard, request, query token) row, or a chunk of the
// row's local tokens.
struct RowId {
    int32_t s_rel, b, t, row;
    int32_t chunk;      // chunk index within the row
    int32_t slot;       // partial slot, or -1 when the item covers the whole row
    int32_t chunk_tok;  // tokens per chunk (0: the whole row)
};

__device__ __forceinline__ void split_row(const DecodeParams& p, RowId& r) {
    r.t = r.row % p.Tq;
    const int32_t bt = r.row / p.Tq;
    r.b = bt % p.B;
    r.s_rel = bt / p.B;
}

// Work item of workgroup `idx`; false for a workgroup past the last item (the
// grid is sized for the most items a plan can make).  Reads are uniform over
// the workgroup and go through the scalar cache.
__device__ __forceinline__ bool work_item(const DecodeParams& p, int32_t idx, RowId& r) {
    if (!p.items) {
        r.row = idx;
        r.chunk = 0;
        r.slot = -1;
        r.chunk_tok = 0;
    } else {
        const __attribute__((address_space(4))) int32_t* hdr =
            (const __attribute__((address_space(4))) int32_t*)p.plan_hdr;
        if (idx >= hdr[1]) return false;
        const __attribute__((address_space(4))) int32_t* it =
            (const __attribute__((address_space(4))) int32_t*)p.items + 4 * size_t(idx);
        r.row = it[0];
        r.chunk = it[1];
        r.slot = it[2];
        r.chunk_tok = hdr[2];
    }
    split_row(p, r);
    return true;
}

}  // namespace mla
