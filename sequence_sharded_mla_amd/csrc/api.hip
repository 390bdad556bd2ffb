// extern "C" entry points of libmla_dcp: argument checks, plan, launches.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/mla_dcp.h"
#include "common.hpp"
#include "decode_fp8.hpp"
#include "decode_mfma.hpp"
#include "decode_valu.hpp"
#include "kv_write.hpp"
#include "topk.hpp"
#include "params.hpp"
#include "plan.hpp"
#include "reduce.hpp"

namespace mla {
namespace {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int32_t launch_status() {
    return hipGetLastError() == hipSuccess ? MLA_OK : MLA_ERR_DEVICE;
}

// qsl: null (q_len query tokens per request), or the varlen query offsets
// [batch + 1] with n_q query tokens in all.  ws_cap > 0: the plan must fit in
// ws_cap bytes of workspace (the allocation-free call's scratch).  err_word:
// the device error word, or null for the workspace's first word.
int32_t decode_impl(const mla_decode_desc* d, const void* q, const void* kv_pool,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* topk_idx, int32_t shard_begin, int32_t shard_count,
                    int32_t n_shards, void* o, float* lse, void* ws, int64_t ws_bytes,
                    void* stream, const int32_t* qsl = nullptr, int32_t n_q = -1,
                    int64_t ws_cap = -1, uint32_t* err_word = nullptr) {
    Plan plan;
    int32_t st = make_plan(d, shard_count, &plan, n_q, ws_cap);
    if (st != MLA_OK) return st;
    if (qsl && (reinterpret_cast<uintptr_t>(qsl) & 3u)) return MLA_ERR_ALIGN;
    if (n_shards < 1 || n_shards > 4096 || shard_begin < 0 || shard_begin + shard_count > n_shards)
        return MLA_ERR_SHARD;
    if (!q || !kv_pool || !block_tables || !context_lens || !o || !lse || !ws) return MLA_ERR_NULL;
    if (d->topk > 0 && !topk_idx) return MLA_ERR_NULL;
    if (d->topk == 0 && topk_idx) return MLA_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(o) || !aligned16(ws) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(err_word) & 3u))
        return MLA_ERR_ALIGN;
    if (ws_bytes < plan.ws_bytes) return MLA_ERR_WORKSPACE;
    if (d->batch == 0 || plan.n_q == 0) return MLA_OK;

    DecodeParams p{};
    p.q = q;
    p.kv = static_cast<const uint8_t*>(kv_pool);
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.topk_idx = topk_idx;
    p.o_out = o;
    p.lse_out = lse;
    uint8_t* w = static_cast<uint8_t*>(ws);
    p.err = err_word ? err_word : reinterpret_cast<uint32_t*>(w);
    p.plan_hdr = reinterpret_cast<const int32_t*>(w);
    if (plan.sp_list) {
        p.sp_list = reinterpret_cast<const int32_t*>(w + plan.sp_list_off);
        p.sp_count = reinterpret_cast<const int32_t*>(w + plan.sp_count_off);
    }
    if (plan.planned) {
        p.items = reinterpret_cast<const int32_t*>(w + plan.items_off);
        p.row_info = reinterpret_cast<const int32_t*>(w + plan.row_info_off);
        p.ws_o = reinterpret_cast<float*>(w + plan.ws_o_off);
        p.ws_lse = reinterpret_cast<float*>(w + plan.ws_lse_off);
    }
    p.pool_blocks = d->pool_blocks;
    p.row_bytes = int32_t(row_bytes(d->kv_dtype));
    p.B = d->batch;
    p.Tq = d->q_len;
    p.n_q = plan.n_q;
    if (qsl) p.qmap = reinterpret_cast<const int32_t*>(w + plan.qmap_off);
    p.H = d->num_heads;
    p.max_blocks = d->max_blocks;
    p.topk = d->topk;
    p.shard_begin = shard_begin;
    p.shard_count = shard_count;
    p.n_shards = n_shards;
    p.rows = plan.rows;
    p.out_dtype = d->out_dtype;
    p.scale = d->softmax_scale;

    hipStream_t s = as_stream(stream);
    if (qsl) {
        int64_t blocks = (plan.n_q + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(qmap_kernel, dim3(uint32_t(blocks)), dim3(256), 0, s, qsl, d->batch, plan.n_q,
                           reinterpret_cast<int32_t*>(w + plan.qmap_off), p.err);
        if ((st = launch_status()) != MLA_OK) return st;
    }
    if (plan.planned) {
        hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, p, plan.target, plan.chunk_min,
                           reinterpret_cast<int32_t*>(w), reinterpret_cast<int32_t*>(w + plan.items_off),
                           reinterpret_cast<int32_t*>(w + plan.row_info_off));
        if ((st = launch_status()) != MLA_OK) return st;
    }
    const uint32_t n_items = uint32_t(plan.items_max);
    // bf16 dense: every supported head count (16 pads to 32); 128 / H' output
    // dimension parts per head group keep all four waves busy
    // bf16 top-K: when the workspace holds the list pass's output
    const bool mfma_bf16 = d->kv_dtype == MLA_BF16 && (d->topk == 0 || plan.sp_list) &&
                           (d->num_heads == 16 || d->num_heads == 32 || d->num_heads == 64 || d->num_heads == 128);
    const bool mfma_fp8 = d->kv_dtype == MLA_FP8_DS && (d->num_heads == 64 || d->num_heads == 128) &&
                          d->topk <= mfma::kMaxTopk;
    if (mfma_bf16 && d->topk > 0) {
        hipLaunchKernelGGL(sparse_list_kernel, dim3(uint32_t(plan.rows)), dim3(kListThreads), 0, s, p,
                           reinterpret_cast<int32_t*>(w + plan.sp_list_off),
                           reinterpret_cast<int32_t*>(w + plan.sp_count_off));
        if ((st = launch_status()) != MLA_OK) return st;
        if (d->num_heads == 128)
            hipLaunchKernelGGL((mfma::decode_mfma_bf16_kernel<1, true>), dim3(n_items), dim3(256), 0, s, p);
        else if (d->num_heads == 64)
            hipLaunchKernelGGL((mfma::decode_mfma_bf16_kernel<2, true>), dim3(n_items), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((mfma::decode_mfma_bf16_kernel<4, true>), dim3(n_items), dim3(256), 0, s, p);
    } else if (mfma_bf16) {
        if (d->num_heads == 128)
            hipLaunchKernelGGL(mfma::decode_mfma_bf16_kernel<1>, dim3(n_items), dim3(256), 0, s, p);
        else if (d->num_heads == 64)
            hipLaunchKernelGGL(mfma::decode_mfma_bf16_kernel<2>, dim3(n_items), dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL(mfma::decode_mfma_bf16_kernel<4>, dim3(n_items), dim3(256), 0, s, p);
    } else if (mfma_fp8) {
        const bool sparse = d->topk > 0;
        if (d->num_heads == 64) {
            if (sparse)
                hipLaunchKernelGGL((mfma::decode_mfma_fp8_kernel<2, true>), dim3(n_items), dim3(128), 0, s, p);
            else
                hipLaunchKernelGGL((mfma::decode_mfma_fp8_kernel<2, false>), dim3(n_items), dim3(128), 0, s, p);
        } else {
            if (sparse)
                hipLaunchKernelGGL((mfma::decode_mfma_fp8_kernel<4, true>), dim3(n_items), dim3(256), 0, s, p);
            else
                hipLaunchKernelGGL((mfma::decode_mfma_fp8_kernel<4, false>), dim3(n_items), dim3(256), 0, s, p);
        }
    } else {
        const dim3 grid(n_items, uint32_t(d->num_heads / valu::kHeads));
        switch (d->kv_dtype) {
            case MLA_F32:
                hipLaunchKernelGGL(valu::decode_valu_kernel<MLA_F32>, grid, dim3(valu::kThreads), 0, s, p);
                break;
            case MLA_BF16:
                hipLaunchKernelGGL(valu::decode_valu_kernel<MLA_BF16>, grid, dim3(valu::kThreads), 0, s, p);
                break;
            default:
                hipLaunchKernelGGL(valu::decode_valu_kernel<MLA_FP8_DS>, grid, dim3(valu::kThreads), 0, s, p);
                break;
        }
    }
    if ((st = launch_status()) != MLA_OK) return st;
    if (plan.planned) {
        // chunks of a row <= its local tokens / the smallest chunk size: when no
        // row can pass 64 partials, a wave per head and four heads per
        // workgroup; else one head per workgroup for the four-wave split
        const int64_t max_chunks = (int64_t(d->max_blocks) * mla::kBlock + plan.chunk_min - 1) / plan.chunk_min;
        const int hpw = max_chunks <= 64 ? 4 : 1;
        hipLaunchKernelGGL(chunk_combine_kernel, dim3(uint32_t(plan.rows), uint32_t((d->num_heads + hpw - 1) / hpw)),
                           dim3(256), 0, s, p, hpw);
        if ((st = launch_status()) != MLA_OK) return st;
    }
    return MLA_OK;
}


// ---- scratch of the allocation-free decode call ---------------------------
// A file-scope device array, one copy per GPU, allocated with the code object
// and held until the process ends.  In host code its name is a host-side
// stand-in, never a device address: the address used everywhere is the one
// hipGetSymbolAddress returns, looked up once per device (with that device
// current) on the call's first use of the device.
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int32_t scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MLA_ERR_DEVICE;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return MLA_OK;
}

int32_t make_slot_params(const int32_t* req_idx, const int32_t* positions, int64_t n_tokens,
                         const int32_t* block_tables, int32_t batch, int32_t max_blocks,
                         int64_t pool_blocks, int32_t shard_begin, int32_t shard_count, int32_t n_shards,
                         void* workspace, kvw::SlotParams* p) {
    if (n_tokens < 0 || n_tokens > INT32_MAX || batch < 1 || max_blocks < 1 || pool_blocks < 1 ||
        pool_blocks > (int64_t(1) << 40))
        return MLA_ERR_SHAPE;
    if (n_shards < 1 || shard_begin < 0 || shard_count < 1 || shard_begin + shard_count > n_shards)
        return MLA_ERR_SHARD;
    if (n_tokens == 0) return MLA_OK;
    if (!req_idx || !positions || !block_tables) return MLA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(req_idx) & 3u) || (reinterpret_cast<uintptr_t>(positions) & 3u) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) || (reinterpret_cast<uintptr_t>(workspace) & 3u))
        return MLA_ERR_ALIGN;
    p->req_idx = req_idx;
    p->positions = positions;
    p->block_tables = block_tables;
    p->err = static_cast<uint32_t*>(workspace);
    p->n = n_tokens;
    p->pool_blocks = pool_blocks;
    p->B = batch;
    p->max_blocks = max_blocks;
    p->shard_begin = shard_begin;
    p->shard_count = shard_count;
    p->n_shards = n_shards;
    return MLA_OK;
}

int32_t check_write(const void* kv_new, int32_t src_dtype, int64_t n_tokens, int32_t kv_dtype,
                    const void* kv_pool, int64_t pool_blocks, const void* workspace) {
    if (n_tokens < 0 || n_tokens > INT32_MAX || pool_blocks < 1 || pool_blocks > (int64_t(1) << 40))
        return MLA_ERR_SHAPE;
    if ((src_dtype != MLA_F32 && src_dtype != MLA_BF16) ||
        (kv_dtype != MLA_F32 && kv_dtype != MLA_BF16 && kv_dtype != MLA_FP8_DS))
        return MLA_ERR_UNSUPPORTED;
    if (n_tokens == 0) return MLA_OK;
    if (!kv_new || !kv_pool) return MLA_ERR_NULL;
    if (!aligned16(kv_new) || !aligned16(kv_pool) || (reinterpret_cast<uintptr_t>(workspace) & 3u))
        return MLA_ERR_ALIGN;
    return MLA_OK;
}

// chunks_per_wave: how many 8-token chunks one wave scans (1..8).
int32_t launch_write(kvw::WriteParams p, const void* kv_new, int32_t src_dtype, int64_t n_tokens,
                     int32_t kv_dtype, void* kv_pool, int64_t pool_blocks, void* workspace,
                     int32_t chunks_per_wave, bool fused, void* stream) {
    p.src = static_cast<const uint8_t*>(kv_new);
    p.pool = static_cast<uint8_t*>(kv_pool);
    p.err = static_cast<uint32_t*>(workspace);
    p.n = n_tokens;
    p.pool_rows = pool_blocks * kBlock;
    const int64_t chunks = (n_tokens + 7) / 8;
    const int64_t waves = (chunks + chunks_per_wave - 1) / chunks_per_wave;
    int64_t blocks = (waves + kvw::kWaves - 1) / kvw::kWaves;
    if (blocks > (int64_t(1) << 22)) blocks = int64_t(1) << 22;
    const dim3 grid(static_cast<uint32_t>(blocks));
    hipStream_t s = as_stream(stream);
    using kvw::kv_write_kernel;
#define MLA_KVW_LAUNCH(S, K)                                                                  \
    do {                                                                                      \
        if (fused)                                                                            \
            hipLaunchKernelGGL((kv_write_kernel<S, K, true>), grid, dim3(256), 0, s, p);      \
        else                                                                                  \
            hipLaunchKernelGGL((kv_write_kernel<S, K, false>), grid, dim3(256), 0, s, p);     \
    } while (0)
    if (src_dtype == MLA_BF16) {
        if (kv_dtype == MLA_FP8_DS) MLA_KVW_LAUNCH(MLA_BF16, MLA_FP8_DS);
        else if (kv_dtype == MLA_BF16) MLA_KVW_LAUNCH(MLA_BF16, MLA_BF16);
        else MLA_KVW_LAUNCH(MLA_BF16, MLA_F32);
    } else {
        if (kv_dtype == MLA_FP8_DS) MLA_KVW_LAUNCH(MLA_F32, MLA_FP8_DS);
        else if (kv_dtype == MLA_BF16) MLA_KVW_LAUNCH(MLA_F32, MLA_BF16);
        else MLA_KVW_LAUNCH(MLA_F32, MLA_F32);
    }
#undef MLA_KVW_LAUNCH
    return launch_status();
}

}  // namespace
}  // namespace mla

extern "C" {

int32_t mla_decode_partial(const mla_decode_desc* desc, const void* q, const void* kv_pool,
                           const int32_t* block_table, const int32_t* context_lens,
                           const int32_t* topk_idx, int32_t shard_id, int32_t n_shards,
                           void* o_partial, float* lse, void* workspace,
                           int64_t workspace_bytes, void* stream) {
    if (n_shards < 1 || shard_id < 0 || shard_id >= n_shards) {
        if (!desc) return MLA_ERR_NULL;
        int32_t st = mla::validate_desc(desc);
        return st != MLA_OK ? st : MLA_ERR_SHARD;
    }
    return mla::decode_impl(desc, q, kv_pool, block_table, context_lens, topk_idx, shard_id, 1,
                            n_shards, o_partial, lse, workspace, workspace_bytes, stream);
}

int32_t mla_decode_partial_noalloc(const mla_decode_desc* desc, const void* q, const void* kv_pool,
                                   const int32_t* block_table, const int32_t* context_lens,
                                   const int32_t* topk_idx, int32_t shard_id, int32_t n_shards,
                                   void* o_partial, float* lse, uint32_t* err_word, void* stream) {
    if (n_shards < 1 || shard_id < 0 || shard_id >= n_shards) {
        if (!desc) return MLA_ERR_NULL;
        int32_t st = mla::validate_desc(desc);
        return st != MLA_OK ? st : MLA_ERR_SHARD;
    }
    void* ws = nullptr;
    int32_t st = mla::scratch_ptr(&ws);
    if (st != MLA_OK) return st;
    return mla::decode_impl(desc, q, kv_pool, block_table, context_lens, topk_idx, shard_id, 1, n_shards,
                            o_partial, lse, ws, mla::kNoAllocScratchBytes, stream, nullptr, -1,
                            mla::kNoAllocScratchBytes, err_word);
}

int32_t mla_decode_partial_shards(const mla_decode_desc* desc, const void* q,
                                  const void* kv_pool, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* topk_idx,
                                  int32_t shard_begin, int32_t shard_count, int32_t n_shards,
                                  void* o_partials, float* lses, void* workspace,
                                  int64_t workspace_bytes, void* stream) {
    return mla::decode_impl(desc, q, kv_pool, block_tables, context_lens, topk_idx, shard_begin,
                            shard_count, n_shards, o_partials, lses, workspace, workspace_bytes,
                            stream);
}

int32_t mla_decode_partial_shards_varlen(const mla_decode_desc* desc, const void* q,
                                         const void* kv_pool, const int32_t* block_tables,
                                         const int32_t* context_lens,
                                         const int32_t* query_start_loc, int32_t n_query_tokens,
                                         const int32_t* topk_idx, int32_t shard_begin,
                                         int32_t shard_count, int32_t n_shards, void* o_partials,
                                         float* lses, void* workspace, int64_t workspace_bytes,
                                         void* stream) {
    if (!desc) return MLA_ERR_NULL;
    if (n_query_tokens < 0) return MLA_ERR_SHAPE;
    if (!query_start_loc && desc->batch > 0 && n_query_tokens > 0) return MLA_ERR_NULL;
    return mla::decode_impl(desc, q, kv_pool, block_tables, context_lens, topk_idx, shard_begin,
                            shard_count, n_shards, o_partials, lses, workspace, workspace_bytes,
                            stream, query_start_loc, n_query_tokens);
}

int32_t mla_lse_merge(int32_t n_parts, int64_t rows, int32_t dv, int32_t part_dtype,
                      const void* o_parts, const float* lse_parts, int32_t out_dtype,
                      void* o_out, float* lse_out, void* stream) {
    if (n_parts < 1 || n_parts > 64 || rows < 0) return MLA_ERR_SHAPE;
    if (dv != mla::kLatent) return MLA_ERR_UNSUPPORTED;
    if ((part_dtype != MLA_F32 && part_dtype != MLA_BF16) ||
        (out_dtype != MLA_F32 && out_dtype != MLA_BF16))
        return MLA_ERR_UNSUPPORTED;
    if (!o_parts || !lse_parts || !o_out) return MLA_ERR_NULL;
    if (!mla::aligned16(o_parts) || !mla::aligned16(o_out) ||
        (reinterpret_cast<uintptr_t>(lse_parts) & 3u) ||
        (reinterpret_cast<uintptr_t>(lse_out) & 3u))
        return MLA_ERR_ALIGN;
    if (rows == 0) return MLA_OK;
    if (rows > (int64_t(1) << 31)) return MLA_ERR_SHAPE;
    const dim3 grid(uint32_t((rows + 3) / 4));
    hipStream_t s = mla::as_stream(stream);
    if (part_dtype == MLA_F32)
        hipLaunchKernelGGL(mla::lse_merge_kernel<float>, grid, dim3(256), 0, s, n_parts, rows,
                           static_cast<const float*>(o_parts), lse_parts, out_dtype, o_out, lse_out);
    else
        hipLaunchKernelGGL(mla::lse_merge_kernel<uint16_t>, grid, dim3(256), 0, s, n_parts, rows,
                           static_cast<const uint16_t*>(o_parts), lse_parts, out_dtype, o_out,
                           lse_out);
    return mla::launch_status();
}

int32_t mla_localize_indices(const int32_t* global_idx, int64_t count, int32_t shard_id,
                             int32_t n_shards, int32_t* local_idx, void* stream) {
    if (count < 0) return MLA_ERR_SHAPE;
    if (n_shards < 1 || shard_id < 0 || shard_id >= n_shards) return MLA_ERR_SHARD;
    if (count == 0) return MLA_OK;
    if (!global_idx || !local_idx) return MLA_ERR_NULL;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(mla::localize_kernel, dim3(uint32_t(blocks)), dim3(256), 0,
                       mla::as_stream(stream), global_idx, count, shard_id, n_shards, local_idx);
    return mla::launch_status();
}

int32_t mla_dcp_slot_mapping(const int32_t* req_idx, const int32_t* positions, int64_t n_tokens,
                             const int32_t* block_tables, int32_t batch, int32_t max_blocks,
                             int64_t pool_blocks, int32_t shard_begin, int32_t shard_count,
                             int32_t n_shards, int64_t* slot_mapping, void* workspace,
                             void* stream) {
    mla::kvw::SlotParams p{};
    int32_t st = mla::make_slot_params(req_idx, positions, n_tokens, block_tables, batch, max_blocks,
                                       pool_blocks, shard_begin, shard_count, n_shards, workspace, &p);
    if (st != MLA_OK || n_tokens == 0) return st;
    if (!slot_mapping) return MLA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(slot_mapping) & 7u) return MLA_ERR_ALIGN;
    p.slots = slot_mapping;
    int64_t blocks = (n_tokens + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(mla::kvw::slot_mapping_kernel, dim3(uint32_t(blocks)), dim3(256), 0,
                       mla::as_stream(stream), p);
    return mla::launch_status();
}

int32_t mla_kv_write(const void* kv_new, int32_t src_dtype, int64_t n_tokens,
                     const int64_t* slot_mapping, int32_t kv_dtype, void* kv_pool,
                     int64_t pool_blocks, void* workspace, void* stream) {
    int32_t st = mla::check_write(kv_new, src_dtype, n_tokens, kv_dtype, kv_pool, pool_blocks, workspace);
    if (st != MLA_OK || n_tokens == 0) return st;
    if (!slot_mapping) return MLA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(slot_mapping) & 7u) return MLA_ERR_ALIGN;
    mla::kvw::WriteParams p{};
    p.slots = slot_mapping;
    // any slot may be written: one chunk of 8 tokens per wave
    return mla::launch_write(p, kv_new, src_dtype, n_tokens, kv_dtype, kv_pool, pool_blocks, workspace,
                             1, false, stream);
}

int32_t mla_dcp_kv_write(const void* kv_new, int32_t src_dtype, const int32_t* req_idx,
                         const int32_t* positions, int64_t n_tokens, const int32_t* block_tables,
                         int32_t batch, int32_t max_blocks, int32_t shard_begin, int32_t shard_count,
                         int32_t n_shards, int32_t kv_dtype, void* kv_pool, int64_t pool_blocks,
                         void* workspace, void* stream) {
    int32_t st = mla::check_write(kv_new, src_dtype, n_tokens, kv_dtype, kv_pool, pool_blocks, workspace);
    if (st != MLA_OK) return st;
    mla::kvw::WriteParams p{};
    st = mla::make_slot_params(req_idx, positions, n_tokens, block_tables, batch, max_blocks, pool_blocks,
                               shard_begin, shard_count, n_shards, workspace, &p.map);
    if (st != MLA_OK || n_tokens == 0) return st;
    // about one group of written tokens per wave: shards own 1/N of
    // consecutive positions each
    const int32_t per_wave = (n_shards + shard_count - 1) / shard_count;
    return mla::launch_write(p, kv_new, src_dtype, n_tokens, kv_dtype, kv_pool, pool_blocks, workspace,
                             per_wave > 8 ? 8 : per_wave, true, stream);
}

namespace {

int32_t topk_local_impl(const float* scores, int64_t row_stride, const int32_t* context_lens,
                        const int32_t* qsl, int32_t batch, int32_t q_len, int32_t n_q, int32_t topk,
                        int32_t shard_begin, int32_t shard_count, int32_t n_shards, int32_t* cand_idx,
                        float* cand_score, void* workspace, void* stream) {
    using namespace mla::topk;
    if (batch < 0 || n_q < 0 || topk < 1 || row_stride < 1 || row_stride > kMaxLocal)
        return MLA_ERR_SHAPE;
    if (n_shards < 1 || shard_begin < 0 || shard_count < 1 || shard_begin + shard_count > n_shards)
        return MLA_ERR_SHARD;
    const int64_t rows = int64_t(shard_count) * n_q;
    if (rows > INT32_MAX || rows * int64_t(topk) > (int64_t(1) << 40)) return MLA_ERR_SHAPE;
    if (rows == 0) return MLA_OK;
    if (!scores || !context_lens || !cand_idx || !cand_score) return MLA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(scores) & 3u) || (reinterpret_cast<uintptr_t>(cand_idx) & 3u) ||
        (reinterpret_cast<uintptr_t>(cand_score) & 3u) || (reinterpret_cast<uintptr_t>(workspace) & 3u) ||
        (reinterpret_cast<uintptr_t>(qsl) & 3u))
        return MLA_ERR_ALIGN;
    LocalParams p{};
    p.scores = scores;
    p.context_lens = context_lens;
    p.qsl = qsl;
    p.out_idx = cand_idx;
    p.out_score = cand_score;
    p.err = static_cast<uint32_t*>(workspace);
    p.stride = row_stride;
    p.B = batch;
    p.Tq = q_len;
    p.n_q = n_q;
    p.K = topk;
    p.shard_begin = shard_begin;
    p.n_shards = n_shards;
    const int32_t words = int32_t((row_stride + 31) / 32);
    hipLaunchKernelGGL(local_topk_kernel, dim3(uint32_t(rows)), dim3(kThreads), size_t(words) * 8,
                       mla::as_stream(stream), p, words);
    return mla::launch_status();
}

}  // namespace

int32_t mla_topk_local(const float* scores, int64_t row_stride, const int32_t* context_lens,
                       int32_t batch, int32_t q_len, int32_t topk, int32_t shard_begin,
                       int32_t shard_count, int32_t n_shards, int32_t* cand_idx, float* cand_score,
                       void* workspace, void* stream) {
    if (batch < 0 || q_len < 1 || int64_t(batch) * q_len > INT32_MAX) return MLA_ERR_SHAPE;
    return topk_local_impl(scores, row_stride, context_lens, nullptr, batch, q_len, batch * q_len, topk,
                           shard_begin, shard_count, n_shards, cand_idx, cand_score, workspace, stream);
}

int32_t mla_topk_local_varlen(const float* scores, int64_t row_stride, const int32_t* context_lens,
                              const int32_t* query_start_loc, int32_t batch, int32_t n_q, int32_t topk,
                              int32_t shard_begin, int32_t shard_count, int32_t n_shards,
                              int32_t* cand_idx, float* cand_score, void* workspace, void* stream) {
    if (batch < 0 || n_q < 0 || (batch == 0 && n_q != 0)) return MLA_ERR_SHAPE;
    if (n_q > 0 && !query_start_loc) return MLA_ERR_NULL;
    return topk_local_impl(scores, row_stride, context_lens, query_start_loc, batch, 1, n_q, topk,
                           shard_begin, shard_count, n_shards, cand_idx, cand_score, workspace, stream);
}

int32_t mla_topk_merge(const int32_t* cand_idx, const float* cand_score, int32_t n_lists, int64_t rows,
                       int32_t cand_k, int32_t topk, int32_t* topk_idx, void* stream) {
    using namespace mla::topk;
    if (n_lists < 1 || rows < 0 || cand_k < 1 || topk < 1 || topk > kMaxMergeK ||
        int64_t(n_lists) * cand_k > kMaxCand || rows > INT32_MAX)
        return MLA_ERR_SHAPE;
    if (rows == 0) return MLA_OK;
    if (!cand_idx || !cand_score || !topk_idx) return MLA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cand_idx) & 3u) || (reinterpret_cast<uintptr_t>(cand_score) & 3u) ||
        (reinterpret_cast<uintptr_t>(topk_idx) & 3u))
        return MLA_ERR_ALIGN;
    MergeParams p{};
    p.cand_idx = cand_idx;
    p.cand_score = cand_score;
    p.out_idx = topk_idx;
    p.rows = rows;
    p.n_lists = n_lists;
    p.k_in = cand_k;
    p.K = topk;
    const int32_t words = int32_t((int64_t(n_lists) * cand_k + 31) / 32);
    int32_t pw = 1;
    while (pw < topk) pw <<= 1;
    if (int64_t(n_lists) * cand_k <= kStage / 2 && topk <= kStageK)
        hipLaunchKernelGGL(merge_topk_staged_kernel, dim3(uint32_t(rows)), dim3(kThreads), 0,
                           mla::as_stream(stream), p);
    else
        hipLaunchKernelGGL(merge_topk_kernel, dim3(uint32_t(rows)), dim3(kThreads),
                           size_t(words) * 4 + size_t(pw) * 4, mla::as_stream(stream), p, words);
    return mla::launch_status();
}

int32_t mla_get_device_error(const void* workspace, int32_t* code_out, void* stream) {
    if (!workspace || !code_out) return MLA_ERR_NULL;
    uint32_t word = 0;
    hipStream_t s = mla::as_stream(stream);
    if (hipMemcpyAsync(&word, workspace, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess)
        return MLA_ERR_DEVICE;
    if (hipStreamSynchronize(s) != hipSuccess) return MLA_ERR_DEVICE;
    *code_out = int32_t(word);
    return MLA_OK;
}

int32_t mla_clear_device_error(void* workspace, void* stream) {
    if (!workspace) return MLA_ERR_NULL;
    hipLaunchKernelGGL(mla::clear_word_kernel, dim3(1), dim3(64), 0, mla::as_stream(stream),
                       static_cast<uint32_t*>(workspace));
    return mla::launch_status();
}

}  // extern "C"
