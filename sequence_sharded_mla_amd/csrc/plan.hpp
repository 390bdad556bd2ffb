// Host-side validation and work planning for one decode step.
//
// Pure C++ (no HIP): the same code is compiled into the library and can be
// exercised without a GPU.  A plan splits every (shard, request, query token)
// row of a dense decode into `n_chunks` chunks of `tiles_per_chunk` 64-token
// tiles of that shard's local cache; each chunk is one workgroup.  When a row
// has more than one chunk, the chunks write float32 (O, LSE) partials into the
// workspace and a combine pass merges them with the same LSE rule as the
// cross-shard merge.
#pragma once

#include <cstdint>

#include "../../include/mla_dcp.h"

namespace mla {

constexpr int kLatent = 512;
constexpr int kRope = 64;
constexpr int kDk = kLatent + kRope;
constexpr int kBlock = 64;
constexpr int kFp8Group = 128;
constexpr int64_t kWsHeader = 256;  // device error word + reserved

struct Plan {
    int32_t rows = 0;             // shard_count * B * Tq
    int32_t n_chunks = 1;         // chunks per row
    int32_t tiles_per_chunk = 0;  // 64-token tiles per chunk (dense)
    int64_t ws_bytes = kWsHeader; // workspace the call needs
    int64_t ws_o_off = 0;         // float [rows][n_chunks][H][512]
    int64_t ws_lse_off = 0;       // float [rows][n_chunks][H]
    int64_t ws_cnt_off = 0;       // uint32 [rows] completion counters
};

int64_t row_bytes(int32_t kv_dtype);
int32_t local_len(int32_t context_len, int32_t shard_id, int32_t n_shards);

// Validates desc (and shard_count >= 1) and fills the plan.  Returns MLA_OK or
// the status code of the first failed check.
int32_t validate_desc(const mla_decode_desc* d);
int32_t make_plan(const mla_decode_desc* d, int32_t shard_count, Plan* plan);

bool aligned16(const void* p);

}  // namespace mla
