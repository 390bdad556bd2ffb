// Kernel parameter block for one decode step over a range of shards, and the
// mapping from a workgroup to its unit of work.
#pragma once

#include <stdint.h>

namespace mla {

struct DecodeParams {
    const void* q;               // [n_q][H][576] f32 or bf16 (n_q = B*Tq, or the varlen count)
    const uint8_t* kv;           // [pool_blocks][64][row_bytes]
    const int32_t* block_tables; // [shard_count][B][max_blocks]
    const int32_t* context_lens; // [B]
    const int32_t* topk_idx;     // [n_q][topk] or null
    const int32_t* qmap;         // varlen: [n_q][4] request, token index in it, its query count, 0;
                                 // null: Tq tokens per request
    void* o_out;                 // [shard_count][n_q][H][512] out dtype
    float* lse_out;              // [shard_count][n_q][H]
    float* ws_o;                 // partials of split rows: [slots][H][512] float32
    float* ws_lse;               // [slots][H]
    const int32_t* items;        // [n][4] row, chunk, partial slot (-1: whole row), 0;
                                 // null: one item per row, covering all of it
    const int32_t* row_info;     // [rows][2] first partial slot (-1: none), items of the row
    const int32_t* plan_hdr;     // [0] error word, [1] item count, [2] tokens per chunk
    uint32_t* err;               // device error word
    const int32_t* sp_list;      // bf16 top-K steps: [rows][stride] pool rows each shard owns, -1 after
    const int32_t* sp_count;     // [rows] owned entries of each row
    int64_t pool_blocks;
    int32_t row_bytes;
    int32_t B, Tq, H, max_blocks, topk;
    int32_t n_q;                 // query tokens per shard: B * Tq, or the varlen count
    int32_t shard_begin, shard_count, n_shards;
    int32_t rows;
    int32_t out_dtype;
    float scale;
};

// One unit of work: a (shard, request, query token) row, or a chunk of the
// row's local tokens.  qi indexes the query token in q, topk_idx and the
// outputs; qlen is its request's query count (query token t of a request
// with context L sits at position L - qlen + t).
struct RowId {
    int32_t s_rel, b, t, row;
    int32_t qi, qlen;
    int32_t chunk;      // chunk index within the row
    int32_t slot;       // partial slot, or -1 when the item covers the whole row
    int32_t chunk_tok;  // tokens per chunk (0: the whole row)
};

__device__ __forceinline__ void split_row(const DecodeParams& p, RowId& r) {
    r.s_rel = r.row / p.n_q;
    r.qi = r.row - r.s_rel * p.n_q;
    if (!p.qmap) {
        r.t = r.qi % p.Tq;
        r.b = r.qi / p.Tq;
        r.qlen = p.Tq;
    } else {
        const __attribute__((address_space(4))) int32_t* m =
            (const __attribute__((address_space(4))) int32_t*)p.qmap + 4 * size_t(r.qi);
        r.b = m[0];
        r.t = m[1];
        r.qlen = m[2];
    }
}

// Work item of workgroup `idx`; false for a workgroup past the last item (the
// grid is sized for the most items a plan can make).  Reads are uniform over
// the workgroup and go through the scalar cache.
__device__ __forceinline__ bool work_item(const DecodeParams& p, int32_t idx, RowId& r) {
    if (!p.items) {
        // Workgroups are dealt to the eight XCDs round robin (workgroup i on
        // XCD i mod 8), each with its own L2.  Rows are numbered shard-major
        // (row = s_rel * n_q + qi); XCD x instead takes the rows of a block
        // of query tokens in token-major order, so the shards of one token
        // run together on one XCD and read its query (and index list) from
        // that L2.
        r.row = idx;
        if (p.rows % 8 == 0) {
            const int32_t u = (idx % 8) * (p.rows / 8) + idx / 8;  // token-major row
            const int32_t qi = u / p.shard_count;
            r.row = (u - qi * p.shard_count) * p.n_q + qi;
        }
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
