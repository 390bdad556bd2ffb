// LSE-merge kernels (intra-shard chunk combine, cross-shard merge), index
// localisation and the device-error reset.
//
// The merge of parts (O_s, LSE_s) follows "GLM-5.2 vLLM Decode Context
// Parallelism", sections "See why vLLM 0.26.0 fails" and "Separate the
// backend merge from stable": M = max LSE_s, w_s = exp(LSE_s - M),
// O = sum w_s O_s / sum w_s, LSE = M + log sum w_s; parts with LSE -inf carry
// weight 0 and a row whose parts are all -inf is (0, -inf).  Parts are summed
// in index order, so the result is reproducible bit for bit.
#pragma once

#include "common.hpp"
#include "params.hpp"

namespace mla {

// 8 consecutive elements of a part row as float.
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        v[2 * k] = __uint_as_float(w[k] << 16);
        v[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
}

__device__ __forceinline__ void store8(void* base, int dtype, size_t i, const float (&v)[8]) {
    if (dtype == MLA_F32) {
        float* o = static_cast<float*>(base) + i;
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
    } else {
        uint4 x;
        x.x = bf16x2_rne(v[0], v[1]);
        x.y = bf16x2_rne(v[2], v[3]);
        x.z = bf16x2_rne(v[4], v[5]);
        x.w = bf16x2_rne(v[6], v[7]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + i) = x;
    }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Merge n parts of one row of width 512 with one wave: lane i accumulates
// dims 8 i .. 8 i + 7; the weights of 64 parts at a time live one per lane.
// part_stride / lse_stride: element distance between consecutive parts.
// Parts are added in index order, so the result is reproducible bit for bit.
template <typename T>
__device__ __forceinline__ void merge_wave(int n, const T* o, size_t part_stride, const float* lse,
                                           size_t lse_stride, void* out, int out_dtype,
                                           size_t out_off, float* lse_out, int lane) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    float M = -INFINITY;
    const T* base = o + lane * 8;
    constexpr int kBatch = 8;  // parts whose loads are in flight together
    if (n <= 64) {
        // one LSE per lane, and the first batch of parts requested together
        // with it: the data does not wait for the weights
        const float ls = lane < n ? lse[size_t(lane) * lse_stride] : -INFINITY;
        float v[kBatch][8];
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (k < n) load8<T>(base + size_t(k) * part_stride, v[k]);
        M = wave_max(ls);
        const float w = (ls == -INFINITY) ? 0.f : expf(ls - M);  // M = -inf: every w is 0
        W = w;
        for (int k0 = 0; k0 < n; k0 += kBatch) {
            if (k0 > 0) {
#pragma unroll
                for (int k = 0; k < kBatch; ++k)
                    if (k0 + k < n) load8<T>(base + size_t(k0 + k) * part_stride, v[k]);
            }
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (k0 + k >= n) break;
                const float ws = __shfl(w, k0 + k);
                if (ws != 0.f) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[k][e], acc[e]);
                }
            }
        }
        n = 0;  // done: skip the general loop below
    }
    for (int s0 = 0; s0 < n; s0 += 64)
        M = fmaxf(M, s0 + lane < n ? lse[size_t(s0 + lane) * lse_stride] : -INFINITY);
    if (n > 0) M = wave_max(M);
    for (int s0 = 0; s0 < n; s0 += 64) {
        const float ls = s0 + lane < n ? lse[size_t(s0 + lane) * lse_stride] : -INFINITY;
        const float w = (ls == -INFINITY) ? 0.f : expf(ls - M);  // M = -inf: every w is 0
        W += w;
        const int cnt = min(64, n - s0);
        for (int k0 = 0; k0 < cnt; k0 += kBatch) {
            float v[kBatch][8];
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if (k0 + k < cnt) load8<T>(base + size_t(s0 + k0 + k) * part_stride, v[k]);
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (k0 + k >= cnt) break;
                const float ws = __shfl(w, k0 + k);
                // a part of weight 0 (LSE -inf) contributes nothing, whatever
                // its values; the test is uniform over the wave
                if (ws != 0.f) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[k][e], acc[e]);
                }
            }
        }
    }
    W = wave_sum(W);
    const float inv = W > 0.f ? 1.f / W : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    store8(out, out_dtype, out_off + lane * 8, acc);
    if (lse_out && lane == 0) lse_out[0] = (M == -INFINITY) ? -INFINITY : M + logf(W);
}

// Weighted sum of parts j0 .. j1 - 1 of one row (weights exp(lse - M)), in
// part order, into acc / W: lane i holds dims 8 i .. 8 i + 7; eight parts'
// loads are in flight together.
template <typename T>
__device__ __forceinline__ void accumulate_parts(const T* base, size_t part_stride, const float* lse,
                                                 size_t lse_stride, int j0, int j1, float M,
                                                 float (&acc)[8], float& W, int lane) {
    constexpr int kBatch = 8;
    for (int s0 = j0; s0 < j1; s0 += 64) {
        const float ls = s0 + lane < j1 ? lse[size_t(s0 + lane) * lse_stride] : -INFINITY;
        const float w = (ls == -INFINITY) ? 0.f : expf(ls - M);
        W += w;
        const int cnt = min(64, j1 - s0);
        for (int k0 = 0; k0 < cnt; k0 += kBatch) {
            float v[kBatch][8];
#pragma unroll
            for (int k = 0; k < kBatch; ++k)
                if (k0 + k < cnt) load8<T>(base + size_t(s0 + k0 + k) * part_stride, v[k]);
#pragma unroll
            for (int k = 0; k < kBatch; ++k) {
                if (k0 + k >= cnt) break;
                const float ws = __shfl(w, k0 + k);
                if (ws != 0.f) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] = fmaf(ws, v[k][e], acc[e]);
                }
            }
        }
    }
}

// One head of a row with more than 64 partials (a few very long rows split
// into many chunks): its parts are dealt to the four waves in contiguous
// quarters; the waves' sums meet in LDS and are added in wave order, so the
// result is reproducible bit for bit.  Every thread of the workgroup calls it.
template <typename T>
__device__ __forceinline__ void combine_head(const DecodeParams& p, int row, int h, int32_t slot0,
                                             int32_t k) {
    __shared__ float part_acc[4][64][8];
    __shared__ float part_w[4];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const size_t head = size_t(row) * p.H + h;
    const size_t s0 = size_t(slot0) * p.H + h;
    const T* o = static_cast<const T*>(p.ws_o) + s0 * kLatent;
    const float* lse = p.ws_lse + s0;
    const size_t stride = size_t(p.H);
    float M = -INFINITY;  // every wave finds the same maximum
    for (int j = lane; j < k; j += 64) M = fmaxf(M, lse[size_t(j) * stride]);
    M = wave_max(M);
    const int per = (k + 3) / 4;
    const int j0 = min(k, wave * per), j1 = min(k, j0 + per);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float W = 0.f;
    if (M != -INFINITY) accumulate_parts<T>(o + lane * 8, stride * kLatent, lse, stride, j0, j1, M, acc, W, lane);
    W = wave_sum(W);
#pragma unroll
    for (int e = 0; e < 8; ++e) part_acc[wave][lane][e] = acc[e];
    if (lane == 0) part_w[wave] = W;
    __syncthreads();
    if (wave == 0) {
        float sum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float Wt = 0.f;
        for (int w = 0; w < 4; ++w) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sum[e] += part_acc[w][lane][e];
            Wt += part_w[w];
        }
        const float inv = Wt > 0.f ? 1.f / Wt : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] *= inv;
        store8(p.o_out, p.out_dtype, head * kLatent + lane * 8, sum);
        if (lane == 0) p.lse_out[head] = (M == -INFINITY) ? -INFINITY : M + logf(Wt);
    }
    __syncthreads();  // part_acc is free for the next head
}

// Chunk combine of a planned step (partials of split rows -> that shard's
// O_partial / LSE; rows of one item were written directly): grid = (rows,
// ceil(H / hpw)), 256 threads; workgroup (row, y) owns heads hpw * y ..
// hpw * y + hpw - 1, hpw = 4 when no row can have more than 64 partials,
// else 1.  Up to 64 partials per row, wave w merges head hpw * y + w on its
// own; more than that, the four waves split each head's partials in turn.
template <typename T>
__device__ __forceinline__ void combine_heads(const DecodeParams& p, int row, int32_t slot0, int32_t k,
                                              int hpw) {
    const int h0 = hpw * int(blockIdx.y);
    const int h_end = min(h0 + hpw, p.H);
    if (k <= 64) {
        const int h = h0 + int(threadIdx.x >> 6);
        if (h >= h_end) return;
        const size_t head = size_t(row) * p.H + h;
        const size_t s0 = size_t(slot0) * p.H + h;
        merge_wave<T>(k, static_cast<const T*>(p.ws_o) + s0 * kLatent, size_t(p.H) * kLatent, p.ws_lse + s0,
                      size_t(p.H), p.o_out, p.out_dtype, head * kLatent, p.lse_out + head, threadIdx.x & 63);
        return;
    }
    for (int h = h0; h < h_end; ++h) combine_head<T>(p, row, h, slot0, k);
}

__global__ void __launch_bounds__(256) chunk_combine_kernel(DecodeParams p, int hpw) {
    const int row = blockIdx.x;
    const int32_t slot0 = p.row_info[2 * size_t(row)];  // a row's slots are consecutive
    const int32_t k = p.row_info[2 * size_t(row) + 1];
    if (k <= 1) return;
    combine_heads<float>(p, row, slot0, k, hpw);  // partials are float32
}

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;

// Exclusive prefix sum of 64-bit values over the plan's workgroup; `total`
// receives the workgroup sum.  Every thread must call it.
__device__ __forceinline__ uint64_t block_excl_scan(uint64_t x, uint64_t* wave_tot, uint64_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint64_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint64_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kPlanWaves; ++w) {
        const uint64_t t = wave_tot[w];
        if (w < wave) before += t;
        total += t;
    }
    __syncthreads();
    return before + inc - x;
}

__device__ __forceinline__ uint64_t block_total(uint64_t x, uint64_t* wave_tot) {
    uint64_t total;
    block_excl_scan(x, wave_tot, total);
    return total;
}

// Device plan of a dense step (one workgroup of kPlanThreads threads).
//
// The chunk size T comes from the real total of local tokens (about
// `target` items, never below chunk_min).  Row r becomes floor(local / T)
// full chunks plus one remainder chunk when local is not a multiple of T
// (a row with no token still gets one item, which writes (0, -inf)).  Items
// are listed longest first, so the dispatcher ends on short work: all full
// chunks, then the remainder chunks in eight size classes, largest first.
// row_info[r] = (first partial slot, items of the row); the slots of a split
// row are consecutive and follow its chunk order.
//
// Counts travel packed: per pass of kPlanThreads rows, (full chunks, chunks
// of split rows) share one 64-bit scan as two 32-bit fields and the eight
// size classes share two scans as 16-bit fields (at most kPlanThreads per
// field); over all rows the class counts take 32-bit fields.
__global__ void __launch_bounds__(kPlanThreads) plan_kernel(DecodeParams p, int32_t target,
                                                            int32_t chunk_min, int32_t* hdr, int32_t* items,
                                                            int32_t* row_info) {
    constexpr int kBuckets = 8;
    __shared__ uint64_t wave_tot[kPlanWaves];
    const int tid = threadIdx.x;
    const int32_t cap = int32_t(int64_t(p.max_blocks) * kBlock > INT32_MAX ? INT32_MAX
                                                                          : int64_t(p.max_blocks) * kBlock);
    auto local_of = [&](int32_t row) -> int32_t {
        RowId r;
        r.row = row;
        split_row(p, r);
        int32_t visible = p.context_lens[r.b] - r.qlen + r.t + 1;
        if (visible < 0) visible = 0;
        const int32_t local = dev_local_len(visible, p.shard_begin + r.s_rel, p.n_shards);
        return local > cap ? cap : local;
    };
    uint64_t tot = 0;
    for (int32_t r = tid; r < p.rows; r += kPlanThreads) tot += uint64_t(local_of(r));
    tot = block_total(tot, wave_tot);
    uint64_t chunk = (tot + uint64_t(target) - 1) / uint64_t(target);
    chunk = (chunk + kBlock - 1) / kBlock * kBlock;
    if (chunk < uint64_t(chunk_min)) chunk = uint64_t(chunk_min);
    if (chunk > (uint64_t(1) << 30)) chunk = uint64_t(1) << 30;
    const int32_t T = int32_t(chunk);

    // shape of row r: full chunks, remainder chunk (0/1), its size class
    auto shape = [&](int32_t r, int32_t& full, int32_t& rem, int32_t& bucket) {
        full = 0;
        rem = 0;
        bucket = -1;
        if (r >= p.rows) return;
        const int32_t local = local_of(r);
        full = local / T;
        const int32_t left = local - full * T;
        if (left > 0 || local == 0) {
            rem = 1;
            bucket = left / (T / kBuckets);  // T is a multiple of 64: floor(8 * left / T)
        }
    };
    // totals: full chunks, and remainder chunks per size class (32-bit fields)
    uint64_t n_full = 0, n_b01 = 0, n_b23 = 0, n_b45 = 0, n_b67 = 0;
    for (int32_t r = tid; r < p.rows; r += kPlanThreads) {
        int32_t full, rem, bucket;
        shape(r, full, rem, bucket);
        n_full += uint64_t(full);
        if (rem) {
            const uint64_t one = uint64_t(1) << (32 * (bucket & 1));
            if (bucket < 2) n_b01 += one;
            else if (bucket < 4) n_b23 += one;
            else if (bucket < 6) n_b45 += one;
            else n_b67 += one;
        }
    }
    n_full = block_total(n_full, wave_tot);
    n_b01 = block_total(n_b01, wave_tot);
    n_b23 = block_total(n_b23, wave_tot);
    n_b45 = block_total(n_b45, wave_tot);
    n_b67 = block_total(n_b67, wave_tot);
    const uint64_t packs[4] = {n_b01, n_b23, n_b45, n_b67};
    uint64_t off_b[kBuckets];
    uint64_t next = n_full;
#pragma unroll
    for (int b = kBuckets - 1; b >= 0; --b) {
        off_b[b] = next;
        next += (packs[b >> 1] >> (32 * (b & 1))) & 0xffffffffu;
    }
    const uint64_t n_items = next;

    uint64_t base_full = 0, base_split = 0;
    uint64_t base_b[kBuckets] = {};
    for (int32_t r0 = 0; r0 < p.rows; r0 += kPlanThreads) {
        const int32_t r = r0 + tid;
        int32_t full, rem, bucket;
        shape(r, full, rem, bucket);
        const int32_t k = full + rem;
        const int32_t ks = k > 1 ? k : 0;
        uint64_t tot_fk;
        const uint64_t ex_fk = block_excl_scan(uint64_t(uint32_t(full)) | (uint64_t(uint32_t(ks)) << 32),
                                               wave_tot, tot_fk);
        const uint64_t onehot = rem ? uint64_t(1) << (16 * (bucket & 3)) : 0;
        uint64_t tot_lo, tot_hi;
        const uint64_t ex_lo = block_excl_scan(bucket < 4 ? onehot : 0, wave_tot, tot_lo);
        const uint64_t ex_hi = block_excl_scan(bucket >= 4 ? onehot : 0, wave_tot, tot_hi);
        if (r < p.rows) {
            const uint64_t ex_full = ex_fk & 0xffffffffu, ex_ks = ex_fk >> 32;
            uint64_t ex_b = 0;
#pragma unroll
            for (int b = 0; b < kBuckets; ++b) {
                const uint64_t field = ((b < 4 ? ex_lo : ex_hi) >> (16 * (b & 3))) & 0xffffu;
                if (bucket == b) ex_b = off_b[b] + base_b[b] + field;
            }
            const int64_t slot0 = k > 1 ? int64_t(base_split + ex_ks) : -1;
            row_info[2 * size_t(r)] = int32_t(slot0);
            row_info[2 * size_t(r) + 1] = k;
            for (int32_t c = 0; c < k; ++c) {
                const uint64_t pos = c < full ? base_full + ex_full + uint64_t(c) : ex_b;
                int32_t* it = items + 4 * size_t(pos);
                it[0] = r;
                it[1] = c;
                it[2] = k > 1 ? int32_t(slot0 + c) : -1;
                it[3] = 0;
            }
        }
        base_full += tot_fk & 0xffffffffu;
        base_split += tot_fk >> 32;
#pragma unroll
        for (int b = 0; b < kBuckets; ++b)
            base_b[b] += ((b < 4 ? tot_lo : tot_hi) >> (16 * (b & 3))) & 0xffffu;
    }
    if (tid == 0) {
        hdr[1] = int32_t(n_items);
        hdr[2] = T;
    }
}

// Cross-part merge: grid = ceil(rows / 4), 256 threads = 4 rows.
template <typename T>
__global__ void __launch_bounds__(256) lse_merge_kernel(int n, int64_t rows, const T* o,
                                                         const float* lse, int out_dtype,
                                                         void* out, float* lse_out) {
    const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    merge_wave<T>(n, o + size_t(row) * kLatent, size_t(rows) * kLatent, lse + row, size_t(rows),
                  out, out_dtype, size_t(row) * kLatent, lse_out ? lse_out + row : nullptr,
                  threadIdx.x & 63);
}

// Varlen query map: query token i of a call whose request b holds tokens
// qsl[b] .. qsl[b + 1] - 1 -> (b, index t in the request, the request's
// query count, 0).  Offsets that are not a partition of [0, n_q) set
// MLA_DEVERR_QUERY; a token the search cannot place inside its request then
// gets a query count so large that it sees no position.  Every read stays in
// qsl[0 .. B] and every write in qmap[0 .. 4 n_q).
__global__ void qmap_kernel(const int32_t* qsl, int32_t B, int32_t n_q, int32_t* qmap, uint32_t* err) {
    const int32_t stride = gridDim.x * blockDim.x;
    const int32_t first = blockIdx.x * blockDim.x + threadIdx.x;
    if (first == 0 && (qsl[0] != 0 || qsl[B] != n_q)) raise_error(err, MLA_DEVERR_QUERY);
    for (int32_t b = first; b < B; b += stride)
        if (qsl[b] > qsl[b + 1]) raise_error(err, MLA_DEVERR_QUERY);
    for (int32_t i = first; i < n_q; i += stride) {
        int32_t lo = 0, hi = B - 1;  // largest b with qsl[b] <= i, for sorted offsets
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (qsl[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        const int64_t start = qsl[lo], end = qsl[lo + 1];
        int32_t* m = qmap + 4 * size_t(i);
        if (start < 0 || end > n_q || i < start || i >= end) {
            raise_error(err, MLA_DEVERR_QUERY);
            m[0] = 0;
            m[1] = 0;
            m[2] = INT32_MAX / 2;
        } else {
            m[0] = lo;
            m[1] = int32_t(i - start);
            m[2] = int32_t(end - start);
        }
        m[3] = 0;
    }
}

__global__ void localize_kernel(const int32_t* g, int64_t count, int32_t shard, int32_t n,
                                int32_t* out) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
         i += int64_t(gridDim.x) * blockDim.x) {
        const int32_t v = g[i];
        out[i] = (v >= 0 && v % n == shard) ? v / n : -1;
    }
}

__global__ void clear_word_kernel(uint32_t* w) {
    if (threadIdx.x == 0) w[0] = 0u;
}

}  // namespace mla
