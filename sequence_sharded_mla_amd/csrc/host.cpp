// Host-only part of the library: status strings, argument validation, sizes
// and the chunk plan.  No HIP dependency.
#include <cmath>
#include <cstdint>

#include "plan.hpp"

namespace mla {

int64_t row_bytes(int32_t kv_dtype) {
    switch (kv_dtype) {
        case MLA_F32: return int64_t(kDk) * 4;
        case MLA_BF16: return int64_t(kDk) * 2;
        case MLA_FP8_DS: return int64_t(kLatent) + 4 * (kLatent / kFp8Group) + 2 * kRope;
        default: return -1;
    }
}

int32_t local_len(int32_t L, int32_t s, int32_t n) {
    if (n < 1 || s < 0 || s >= n || L < 0) return -1;
    return L > s ? (L - s + n - 1) / n : 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static bool heads_supported(int32_t h) { return h == 16 || h == 32 || h == 64 || h == 128; }

int32_t validate_desc(const mla_decode_desc* d) {
    if (!d) return MLA_ERR_NULL;
    if (d->batch < 0 || d->q_len < 1 || d->max_blocks < 1 || d->topk < 0 || d->topk > 65536 ||
        d->pool_blocks < 1)
        return MLA_ERR_SHAPE;
    if (d->kv_lora_rank != kLatent || d->rope_dim != kRope || d->block_size != kBlock)
        return MLA_ERR_UNSUPPORTED;
    if (!heads_supported(d->num_heads)) return MLA_ERR_UNSUPPORTED;
    const bool f32_pair = d->q_dtype == MLA_F32 && d->kv_dtype == MLA_F32;
    const bool bf16_q = d->q_dtype == MLA_BF16 && (d->kv_dtype == MLA_BF16 || d->kv_dtype == MLA_FP8_DS);
    if (!f32_pair && !bf16_q) return MLA_ERR_UNSUPPORTED;
    if (d->out_dtype != MLA_F32 && d->out_dtype != MLA_BF16) return MLA_ERR_UNSUPPORTED;
    if (!std::isfinite(d->softmax_scale) || !(d->softmax_scale > 0.f)) return MLA_ERR_SHAPE;
    // element offsets are 64-bit in the kernels; bound the per-call rows
    if (int64_t(d->batch) * d->q_len > (int64_t(1) << 24)) return MLA_ERR_SHAPE;
    return MLA_OK;
}

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Items the device plan aims for: about two per workgroup that fits on the
// chip at once (256 compute units; the fp8 kernel for 64 heads fits two
// workgroups per unit).
static int32_t plan_target(const mla_decode_desc* d) {
    if (d->kv_dtype == MLA_FP8_DS && d->num_heads == 64) return 1024;
    if (d->kv_dtype == MLA_F32 || (d->kv_dtype == MLA_BF16 && d->num_heads != 128)) return 1024;
    return 512;
}

// Item, row and partial-slot bounds of a planned step with p->target items
// (and the workspace offsets after `off`); returns the workspace end.
static int64_t size_planned(const mla_decode_desc* d, Plan* p, int64_t off) {
    // items per row <= local / chunk + 1 and sum(local) / chunk <= target
    p->items_max = p->rows + p->target;
    // a row splits only when local > chunk >= chunk_min, into at most
    // 2 local / chunk items: at most 2 target and 2 total / chunk_min
    const int64_t total_bound = int64_t(p->rows) * d->max_blocks * kBlock;
    int64_t slots = 2 * int64_t(p->target);
    const int64_t by_len = 2 * ((total_bound + p->chunk_min - 1) / p->chunk_min);
    if (by_len < slots) slots = by_len;
    if (p->items_max < slots) slots = p->items_max;
    p->slots = int32_t(slots);
    p->items_off = off;
    off = align_up(off + int64_t(p->items_max) * 16, 256);
    p->row_info_off = off;
    off = align_up(off + int64_t(p->rows) * 8, 256);
    p->ws_o_off = off;
    off = align_up(off + slots * d->num_heads * kLatent * 4, 256);  // float32 partials
    p->ws_lse_off = off;
    off = align_up(off + slots * d->num_heads * 4, 256);
    return off;
}

static int64_t planned_bytes(const mla_decode_desc* d, Plan p, int64_t off) { return size_planned(d, &p, off); }

int32_t make_plan(const mla_decode_desc* d, int32_t shard_count, Plan* plan, int32_t n_q, int64_t ws_cap) {
    int32_t st = validate_desc(d);
    if (st != MLA_OK) return st;
    if (shard_count < 1 || shard_count > 4096) return MLA_ERR_SHARD;
    const int64_t bound = int64_t(d->batch) * d->q_len;  // the most query tokens a call can have
    if (n_q < 0) n_q = int32_t(bound);
    if (n_q > bound) return MLA_ERR_SHAPE;
    Plan p;
    p.n_q = n_q;
    p.rows = int32_t(int64_t(shard_count) * n_q);
    // a row holds at most max_blocks * 64 local tokens; when that fits in one
    // chunk of the smallest size, every row is one item and no plan is needed.
    // plan_target is about two items per workgroup the chip holds at once; a
    // call with fewer rows than that many workgroups aims for one item per
    // workgroup, with the smaller floor.
    const bool few_rows = p.rows < plan_target(d) / 2;
    p.chunk_min = few_rows ? kChunkSmall : kChunkMin;
    p.planned = d->topk == 0 && int64_t(d->max_blocks) * kBlock > p.chunk_min;
    p.items_max = p.rows;
    int64_t off = kWsHeader;
    // per query token (request, index in it, its query count, 0), filled for
    // calls with a query count per request
    p.qmap_off = off;
    off = align_up(off + int64_t(n_q) * 16, 256);
    if (p.planned) {
        p.target = few_rows ? plan_target(d) / 2 : plan_target(d);
        // a capped workspace plans fewer, longer chunks until the partials fit
        if (ws_cap > 0)
            while (p.target > 1 && planned_bytes(d, p, off) > ws_cap) p.target /= 2;
        off = size_planned(d, &p, off);
    }
    // A top-K step on a bf16 cache runs on the matrix-core kernel behind a
    // list pass whose output (each row's owned pool rows) lives in the
    // workspace.  A capped workspace too small for the lists keeps the step
    // on the VALU kernel, which needs none.
    if (d->topk > 0 && d->kv_dtype == MLA_BF16) {
        const int64_t stride = (int64_t(d->topk) + 31) / 32 * 32;
        int64_t o2 = off;
        const int64_t list_off = o2;
        o2 = align_up(o2 + int64_t(p.rows) * stride * 4, 256);
        const int64_t count_off = o2;
        o2 = align_up(o2 + int64_t(p.rows) * 4, 256);
        if (ws_cap <= 0 || o2 <= ws_cap) {
            p.sp_list = true;
            p.sp_list_off = list_off;
            p.sp_count_off = count_off;
            off = o2;
        }
    }
    p.ws_bytes = off;
    if (ws_cap > 0 && p.ws_bytes > ws_cap) return MLA_ERR_WORKSPACE;
    *plan = p;
    return MLA_OK;
}

}  // namespace mla

extern "C" {

const char* mla_status_string(int32_t status) {
    switch (status) {
        case MLA_OK: return "ok";
        case MLA_ERR_NULL: return "a required pointer is NULL";
        case MLA_ERR_SHAPE: return "a size is out of range or inconsistent";
        case MLA_ERR_SHARD: return "shard id, shard range or shard count is invalid";
        case MLA_ERR_UNSUPPORTED: return "head count, dimension or dtype combination is not supported";
        case MLA_ERR_WORKSPACE: return "workspace is smaller than mla_decode_workspace_size";
        case MLA_ERR_DEVICE: return "a HIP runtime call failed";
        case MLA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        default: return "unknown status";
    }
}

int32_t mla_shard_local_len(int32_t context_len, int32_t shard_id, int32_t n_shards) {
    return mla::local_len(context_len, shard_id, n_shards);
}

int64_t mla_kv_row_bytes(int32_t kv_dtype) { return mla::row_bytes(kv_dtype); }

int32_t mla_decode_workspace_size(const mla_decode_desc* desc, int32_t shard_count,
                                  int64_t* bytes_out) {
    if (!bytes_out) return MLA_ERR_NULL;
    mla::Plan p;
    int32_t st = mla::make_plan(desc, shard_count, &p);
    if (st != MLA_OK) return st;
    *bytes_out = p.ws_bytes;
    return MLA_OK;
}

}  // extern "C"
