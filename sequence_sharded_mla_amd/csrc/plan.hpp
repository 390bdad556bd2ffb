// Host-side validation and workspace sizing for one decode step.
//
// Pure C++ (no HIP): the same code is compiled into the library and can be
// exercised without a GPU.  Sparse steps run one workgroup per (shard,
// request, query token) row.  Dense steps whose rows may exceed one chunk
// are planned on the device: a plan kernel reads the real context lengths,
// picks a chunk size from the total work (about two chunks per resident
// workgroup, never fewer than the plan's floor), and lists (row, chunk)
// items; rows of one chunk write their result directly, split rows write
// partials into the workspace and a combine pass merges them with the same
// LSE rule as the cross-shard merge.
#pragma once

#include <cstdint>

#include "../../include/mla_dcp.h"

namespace mla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDk = kLatent + kRope;
constexpr int kBlock = 64;
constexpr int kFp8Group = 128;
constexpr int64_t kWsHeader = 256;  // int32 [0] device error word, [1] item count, [2] chunk tokens

// Fewest local tokens per chunk of a split row.  A call with at least as
// many rows as the chip holds workgroups splits only long rows (kChunkMin);
// one with fewer rows (one DCP rank's share of a small batch) aims for one
// chunk per resident workgroup, down to kChunkSmall tokens, so that every
// compute unit gets work, at the cost of more partials for the combine.
constexpr int32_t kChunkMin = 4096;
constexpr int32_t kChunkSmall = 512;

struct Plan {
    int32_t n_q = 0;            // query tokens per shard (B * Tq, or the varlen count)
    int32_t rows = 0;           // shard_count * n_q
    bool planned = false;       // dense rows that may split: device plan + combine
    int32_t target = 0;         // items the device plan aims for
    int32_t chunk_min = 0;      // the device plan's floor on the chunk size
    int32_t items_max = 0;      // workgroups to launch (an upper bound on items)
    int32_t slots = 0;          // partial slots of split rows
    int64_t ws_bytes = kWsHeader; // workspace the call needs
    int64_t qmap_off = 0;       // int32 [n_q][4]
    int64_t items_off = 0;      // int32 [items_max][4]
    int64_t row_info_off = 0;   // int32 [rows][2]
    int64_t ws_o_off = 0;       // float [slots][H][512]
    int64_t ws_lse_off = 0;     // float [slots][H]
    bool sp_list = false;       // top-K step on a bf16 cache: a list pass, then the matrix-core kernel
    int64_t sp_list_off = 0;    // int32 [rows][topk rounded up to 32] pool rows each row owns
    int64_t sp_count_off = 0;   // int32 [rows]
};

int64_t row_bytes(int32_t kv_dtype);
int32_t local_len(int32_t context_len, int32_t shard_id, int32_t n_shards);

// Validates desc (and shard_count >= 1) and fills the plan.  Returns MLA_OK or
// the status code of the first failed check.
int32_t validate_desc(const mla_decode_desc* d);
// n_q: query tokens per shard, at most batch * q_len (-1: batch * q_len).
// ws_cap > 0: the workspace may not exceed ws_cap bytes; a planned step then
// aims for fewer, longer chunks until its partials fit, and the call fails
// with MLA_ERR_WORKSPACE when even that does not fit.
int32_t make_plan(const mla_decode_desc* d, int32_t shard_count, Plan* plan, int32_t n_q = -1,
                  int64_t ws_cap = -1);

bool aligned16(const void* p);

}  // namespace mla
