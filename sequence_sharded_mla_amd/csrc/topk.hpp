// Top-K selection of sparse-attention indices, per shard and merged (gfx950).
//
// A query token attends the K best positions of its causal prefix by
// indexer score ("GLM-5.2 vLLM Decode Context Parallelism", section
// "Understand the cache-copy opportunity": top-K of 2,048; "How vLLM Serves
// GLM-5.3 with Million-Token Contexts on 16 H200s", section "Why
// conventional TP and DP fall short": the indexer scores earlier tokens and
// sparse attention selects a fixed set).  With the cache sharded
// round-robin, a shard holds the scores of its own positions: it selects its
// local top-K, and the top-K of the union of the shards' lists is the global
// top-K.
//
// Order: larger score first; equal scores (+0 and -0 are one value) by lower
// position.  Every element therefore has a distinct 64-bit key
//   key = order-preserving bits of the score << 32 | ~id
// (id = local index or global position, both increasing with position), and
// the K elements with the largest keys are the selection.  Lists are written
// as ascending positions padded with -1 (scores of padded entries -inf).
//
// One workgroup per row.  The K-th key is found digit by digit from the top
// (12, 12, 8, 12, 12, 8 bits): a histogram of the elements still tied with
// the prefix found so far (LDS atomics), then a suffix scan picks the digit
// holding the K-th key.  As soon as the tied group is small enough
// (<= kCand), one more pass over the row sets a bit for every element above
// the group and copies the group into LDS, where 8-bit digits settle it.  The set bits, read in index order, give the output; a row
// usually needs two passes over its scores (one from HBM, one from cache).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_dcp.h"
#include "common.hpp"

namespace mla {
namespace topk {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kWavesT = kThreads / 64;
constexpr int kBins = 4096;       // 12-bit digits
constexpr int kCand = 2048;       // tied group resolved in LDS (a power of two)
constexpr int kSel = 2048;        // local rows with K <= kSel list their selection in LDS
constexpr int kMaxMergeK = 8192;  // output list sorted in LDS by the merge
// Local positions per row: the row's bitmap (32 positions in two 32-bit
// words: bits and a running count) is 8 B per 32 positions of dynamic LDS
// beside the kernel's static state (about 58 KB), inside the 160 KB a
// workgroup may hold.
constexpr int64_t kMaxLocal = 393216;
constexpr int64_t kMaxCand = int64_t(1) << 18;    // candidates per merged row (32 KB bitmap)
constexpr int kStage = 32768;     // merge rows of up to kStage / 2 candidates are read once into LDS
constexpr int kStageK = kCand;    // largest K the staged merge sorts in the tied-group space

struct LocalParams {
    const float* scores;     // [shard_count][n_q][stride], n_q = B * Tq unless varlen
    const int32_t* context_lens;
    const int32_t* qsl;      // varlen: [B + 1] query offsets per request; null: Tq each
    int32_t* out_idx;        // [shard_count][n_q][K]
    float* out_score;        // [shard_count][n_q][K]
    uint32_t* err;           // may be null
    int64_t stride;
    int32_t B, Tq, n_q, K, shard_begin, n_shards;
};

struct MergeParams {
    const int32_t* cand_idx;  // [n_lists][rows][k_in]
    const float* cand_score;
    int32_t* out_idx;         // [rows][K]
    int64_t rows;
    int32_t n_lists, k_in, K;
};

// Order-preserving bits of a float (larger float -> larger unsigned value);
// -0 and +0 map to the same value.
__device__ __forceinline__ uint32_t score_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u = (u << 1) == 0 ? 0u : u;                              // -0 -> +0
    return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);  // negative: ~u; else set the sign
}

__device__ __forceinline__ uint64_t make_key(float score, uint32_t id) {
    return (uint64_t(score_bits(score)) << 32) | uint64_t(~id);
}

// Digits from the top of the 64-bit key: (shift, width).
__device__ __forceinline__ int digit_shift(int pass) {
    constexpr int kShift[6] = {52, 40, 32, 20, 8, 0};
    return kShift[pass];
}
__device__ __forceinline__ int digit_width(int pass) { return (pass % 3 == 2) ? 8 : 12; }

// Elements of a row kept in LDS: the score bits of the key (its high 32
// bits; the low 32 are the complement of the index) and the index.
constexpr int kBuf = 4096;
struct SelList {
    uint32_t sb[kBuf];
    uint32_t idx[kBuf];
    uint32_t n;
};

__device__ __forceinline__ uint64_t key_of(uint32_t sb, uint32_t idx) {
    return (uint64_t(sb) << 32) | uint64_t(~idx);
}

struct SelectShared {
    // the histogram serves the digit passes over the row, the tied group
    // the last pass and its settling in LDS
    union {
        uint32_t hist[kBins];
        struct {
            uint64_t cand_key[kCand];
            uint32_t cand_idx[kCand];
        };
    };
    uint32_t hist8[256];     // 8-bit digits of the tied group in LDS
    uint64_t prefix;         // fixed top bits of the K-th key
    uint64_t mask;           // which bits are fixed
    uint32_t need;           // elements still to take from the tied group
    uint32_t tied;           // size of the tied group
    uint32_t n_cand;
    uint32_t scan[kWavesT];
};

// Inclusive scan helpers over the workgroup (kThreads threads).
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t x, uint32_t* wave_tot, uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o);
        if (lane >= o) inc += y;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint32_t before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kWavesT; ++w) {
        const uint32_t t = wave_tot[w];
        if (w < wave) before += t;
        total += t;
    }
    __syncthreads();
    return before + inc - x;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, uint32_t(__shfl_xor(int(x), o)));
    return x;
}

// Finds the digit holding the need-th largest key among the histogram's
// bins (nbins <= kBins), updates prefix/mask/need/tied.  All threads call.
__device__ __forceinline__ void pick_digit(SelectShared& sh, const uint32_t* hist, int nbins, int shift) {
    // each thread sums a contiguous run of bins, counted from the top bin down
    constexpr int kPer = kBins / kThreads;  // 8
    const int per = nbins / kThreads > 0 ? nbins / kThreads : 1;
    const int active = nbins / per;  // threads holding bins
    uint32_t mine = 0;
    const int t = threadIdx.x;
    if (t < active) {
        for (int j = 0; j < per && j < kPer; ++j) mine += hist[nbins - 1 - (t * per + j)];
    }
    const uint32_t need = sh.need;  // read before the scan's barriers: one thread rewrites it
    uint32_t total;
    const uint32_t before = block_excl_scan_u32(mine, sh.scan, total);  // count of larger bins
    if (t < active && before < need && need <= before + mine) {
        uint32_t above = before;
        for (int j = 0; j < per; ++j) {
            const int bin = nbins - 1 - (t * per + j);
            const uint32_t c = hist[bin];
            if (need <= above + c) {
                sh.prefix |= uint64_t(bin) << shift;
                sh.mask |= uint64_t(nbins - 1) << shift;
                sh.need = need - above;
                sh.tied = c;
                break;
            }
            above += c;
        }
    }
    __syncthreads();
}

// Calls f(i, key) for every element i < n whose key is not 0 (0 marks an
// invalid element; every real key is larger).  A source loads Src::V
// consecutive elements at once; each thread requests U such loads before
// using the first, so U loads per lane are in flight.
template <int U, typename Src, typename F>
__device__ __forceinline__ void for_each_key(const Src& src, int64_t n, F f) {
    constexpr int V = Src::V;
    const int64_t groups = (n + V - 1) / V;
    for (int64_t g0 = threadIdx.x; g0 < groups; g0 += int64_t(kThreads) * U) {
        uint64_t k[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + int64_t(u) * kThreads;
            if (g < groups) src.keys(g, n, k[u]);
            else {
#pragma unroll
                for (int v = 0; v < V; ++v) k[u][v] = 0;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int v = 0; v < V; ++v)
                if (k[u][v]) f((g0 + int64_t(u) * kThreads) * V + v, k[u][v]);
    }
}

// COLLECT: also list the selected elements in *sel (K <= kSel).
template <int U, bool COLLECT, typename Src>
__device__ void select_into_bitmap(SelectShared& sh, const Src& src, int64_t n, uint32_t K,
                                   uint32_t* bits, SelList* sel = nullptr) {
    if (threadIdx.x == 0) {
        sh.prefix = 0;
        sh.mask = 0;
        sh.need = K;
        sh.tied = uint32_t(n);
        sh.n_cand = 0;
        if (COLLECT) sel->n = 0;
    }
    __syncthreads();
    for (int pass = 0; pass < 6; ++pass) {
        if (sh.tied <= uint32_t(kCand) || sh.tied == sh.need) break;
        const int shift = digit_shift(pass);
        const int nbins = 1 << digit_width(pass);
        for (int i = threadIdx.x; i < nbins; i += kThreads) sh.hist[i] = 0;
        __syncthreads();
        const uint64_t prefix = sh.prefix, mask = sh.mask;
        for_each_key<U>(src, n, [&](int64_t, uint64_t k) {
            if ((k & mask) == prefix) atomicAdd(&sh.hist[uint32_t(k >> shift) & uint32_t(nbins - 1)], 1u);
        });
        __syncthreads();
        pick_digit(sh, sh.hist, nbins, shift);
    }
    // one pass: elements above the tied group are selected; the group goes
    // to LDS unless all of it is taken
    const uint64_t prefix = sh.prefix, mask = sh.mask;
    const bool take_all = sh.tied == sh.need;
    // Appends go through one wave-wide scan and one LDS atomic per list per
    // batch: each lane counts its selected and tied elements, a wave scan
    // turns the counts into slots.  The loop runs the same number of
    // batches in every lane, so the wave is whole for the scan.
    constexpr int V = Src::V;
    const int64_t groups = (n + V - 1) / V;
    const int lane = threadIdx.x & 63;
    for (int64_t base = 0; base < groups; base += int64_t(kThreads) * U) {
        const int64_t g0 = base + threadIdx.x;
        uint64_t k[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t g = g0 + int64_t(u) * kThreads;
            if (g < groups) src.keys(g, n, k[u]);
            else {
#pragma unroll
                for (int v = 0; v < V; ++v) k[u][v] = 0;
            }
        }
        uint32_t counts = 0;  // selected in the low 16 bits, tied in the high 16
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int64_t i = (g0 + int64_t(u) * kThreads) * V + v;
                const uint64_t kk = k[u][v];
                const uint64_t top = kk & mask;
                const bool is_sel = kk && (top > prefix || (top == prefix && take_all));
                const bool tie = kk && top == prefix && !take_all;
                if (is_sel) atomicOr(&bits[i >> 5], 1u << (i & 31));
                counts += (COLLECT && is_sel ? 1u : 0u) + (tie ? 0x10000u : 0u);
            }
        }
        uint32_t incl = counts;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const uint32_t y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        const uint32_t tot = __shfl(incl, 63);
        if (tot == 0) continue;
        uint32_t bases = 0;
        if (lane == 0) {
            const uint32_t bs = (COLLECT && (tot & 0xffffu)) ? atomicAdd(&sel->n, tot & 0xffffu) : 0u;
            const uint32_t bt = (tot >> 16) ? atomicAdd(&sh.n_cand, tot >> 16) : 0u;
            bases = bs | (bt << 16);  // both below 2^16
        }
        bases = __shfl(bases, 0);
        const uint32_t excl = incl - counts;
        uint32_t at_sel = (bases & 0xffffu) + (excl & 0xffffu);
        uint32_t at_tie = (bases >> 16) + (excl >> 16);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int64_t i = (g0 + int64_t(u) * kThreads) * V + v;
                const uint64_t kk = k[u][v];
                const uint64_t top = kk & mask;
                const bool is_sel = kk && (top > prefix || (top == prefix && take_all));
                const bool tie = kk && top == prefix && !take_all;
                // the bounds hold by construction (at most K selected, the
                // tied group fits); the checks keep a broken invariant in LDS
                if (COLLECT && is_sel) {
                    if (at_sel < uint32_t(kBuf)) {
                        sel->sb[at_sel] = uint32_t(kk >> 32);
                        sel->idx[at_sel] = uint32_t(i);
                    }
                    ++at_sel;
                }
                if (tie) {
                    if (at_tie < uint32_t(kCand)) {
                        sh.cand_key[at_tie] = kk;
                        sh.cand_idx[at_tie] = uint32_t(i);
                    }
                    ++at_tie;
                }
            }
        }
    }
    __syncthreads();
    if (!take_all) {
        // the tied group is in LDS: settle it with 8-bit digits of the
        // bits not fixed yet, down to a group taken whole (keys are distinct)
        const uint32_t nc = sh.n_cand < uint32_t(kCand) ? sh.n_cand : uint32_t(kCand);
        int shift = 64;
        while (shift > 0 && ((sh.mask >> (shift - 1)) & 1u)) --shift;  // highest free bit + 1
        shift = shift > 8 ? shift - 8 : 0;
        while (sh.tied != sh.need) {
            for (int i = threadIdx.x; i < 256; i += kThreads) sh.hist8[i] = 0;
            __syncthreads();
            const uint64_t pre = sh.prefix, msk = sh.mask;
            for (uint32_t j = threadIdx.x; j < nc; j += kThreads) {
                const uint64_t kk = sh.cand_key[j];
                if ((kk & msk) == pre) atomicAdd(&sh.hist8[uint32_t(kk >> shift) & 255u], 1u);
            }
            __syncthreads();
            pick_digit(sh, sh.hist8, 256, shift);
            shift = shift > 8 ? shift - 8 : 0;
        }
        const uint64_t pre = sh.prefix, msk = sh.mask;
        const uint32_t ns = COLLECT ? sel->n : 0;
        uint32_t mine = 0;
        for (uint32_t j = threadIdx.x; j < nc; j += kThreads) mine += (sh.cand_key[j] & msk) >= pre ? 1u : 0u;
        uint32_t total;
        uint32_t at = ns + block_excl_scan_u32(mine, sh.scan, total);
        for (uint32_t j = threadIdx.x; j < nc; j += kThreads) {
            const uint64_t kk = sh.cand_key[j];
            if ((kk & msk) >= pre) {
                const uint32_t i = sh.cand_idx[j];
                atomicOr(&bits[i >> 5], 1u << (i & 31));
                if (COLLECT && at < uint32_t(kBuf)) {
                    sel->sb[at] = uint32_t(kk >> 32);
                    sel->idx[at] = i;
                }
                ++at;
            }
        }
    }
    __syncthreads();
}

struct LocalSrc {
    static constexpr int V = 1;
    const float* row;
    __device__ void keys(int64_t g, int64_t, uint64_t (&k)[V]) const { k[0] = make_key(row[g], uint32_t(g)); }
    __device__ void load(int64_t g, float (&x)[V]) const { x[0] = row[g]; }
};

// A score row read 16 bytes (four elements) per load; the row is 16-byte
// aligned and readable up to n rounded up to four.
struct LocalSrc4 {
    static constexpr int V = 4;
    const float* row;
    __device__ void keys(int64_t g, int64_t n, uint64_t (&k)[V]) const {
        const f32x4_t x = reinterpret_cast<const f32x4_t*>(row)[g];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int64_t i = g * V + v;
            k[v] = i < n ? make_key(x[v], uint32_t(i)) : 0;
        }
    }
    __device__ void load(int64_t g, float (&x)[V]) const {
        const f32x4_t y = reinterpret_cast<const f32x4_t*>(row)[g];
        x[0] = y[0];
        x[1] = y[1];
        x[2] = y[2];
        x[3] = y[3];
    }
};

// A candidate score as returned: the stored score, with -0 written as +0
// (the two are one value for the selection).
__device__ __forceinline__ float canon(float x) { return x == 0.f ? 0.f : x; }

// The score given its order-preserving bits (canonical: -0 comes back as +0).
__device__ __forceinline__ float score_of(uint32_t b) {
    return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}

// Settles a tied group held in LDS: `count` entries of `buf`, those whose
// key matches sh.prefix under sh.mask are tied, sh.need of them are taken.
// Adds 8-bit digits below the fixed bits until the group is taken whole.
__device__ void settle_in_lds(SelectShared& sh, const SelList& buf, uint32_t count) {
    int shift = 64;
    while (shift > 0 && ((sh.mask >> (shift - 1)) & 1u)) --shift;
    shift = shift > 8 ? shift - 8 : 0;
    while (sh.tied != sh.need) {
        for (int i = threadIdx.x; i < 256; i += kThreads) sh.hist8[i] = 0;
        __syncthreads();
        const uint64_t pre = sh.prefix, msk = sh.mask;
        for (uint32_t j = threadIdx.x; j < count; j += kThreads) {
            const uint64_t kk = key_of(buf.sb[j], buf.idx[j]);
            if ((kk & msk) == pre) atomicAdd(&sh.hist8[uint32_t(kk >> shift) & 255u], 1u);
        }
        __syncthreads();
        pick_digit(sh, sh.hist8, 256, shift);
        shift = shift > 8 ? shift - 8 : 0;
    }
}

// One read of the row: a 512-element sample places a first digit D a little
// below the K-th key's; the pass over the row counts the 12-bit digits of,
// and keeps in LDS, every element whose digit is at least D.  When the K-th key's digit turns
// out to be at least D (and the kept set fit), the whole selection is among
// the kept elements and settles in LDS; `buf` then holds them and the ones
// chosen satisfy (key & sh.mask) >= sh.prefix.  Returns false otherwise (no
// bit set; the caller runs the general selection).
template <int U, typename Src>
__device__ bool select_one_pass(SelectShared& sh, SelList& buf, const Src& src, const float* row,
                                int64_t n, uint32_t K, uint32_t* bits) {
    for (int i = threadIdx.x; i < kBins; i += kThreads) sh.hist[i] = 0;
    if (threadIdx.x == 0) {
        sh.prefix = 0;
        sh.mask = 0;
        sh.need = K;
        sh.tied = uint32_t(n);
        buf.n = 0;
    }
    __syncthreads();
    // raw scores stay in registers (4 bytes each) until they are used
    uint32_t d_min = 0;
    constexpr int V = Src::V;
    // local rows hold at most kMaxLocal positions: 32-bit indices
    const int32_t n32 = int32_t(n);
    const int32_t groups = (n32 + V - 1) / V;
    const int lane = threadIdx.x & 63;
    for (int32_t base = 0; base < groups; base += kThreads * U) {
        const int32_t g0 = base + int32_t(threadIdx.x);
        float x[U][V];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t g = g0 + u * kThreads;
            if (g < groups) src.load(g, x[u]);
        }
        if (base == 0 && n > kBuf) {
            // the sample's load goes out behind the first batch's, so the
            // wait for it costs no extra round trip
            const int32_t i = int32_t(threadIdx.x) * (n32 / kThreads);
            atomicAdd(&sh.hist[uint32_t(make_key(row[i], uint32_t(i)) >> 52)], 1u);
            __syncthreads();
            // the kept share of the sample plus a few: the digit's bins are
            // coarse (about 1.5% of a normal row near the top 6%), so the
            // kept set already has slack; a row whose estimate misses takes
            // the general path
            uint32_t need_s = uint32_t((uint64_t(K) * kThreads + n - 1) / uint64_t(n)) + 8;
            if (need_s > uint32_t(kThreads)) need_s = kThreads;
            if (threadIdx.x == 0) sh.need = need_s;
            __syncthreads();
            pick_digit(sh, sh.hist, kBins, 52);
            d_min = uint32_t(sh.prefix >> 52);
            __syncthreads();  // every thread has read the sample's digit
            for (int j = threadIdx.x; j < kBins; j += kThreads) sh.hist[j] = 0;
            if (threadIdx.x == 0) {
                sh.prefix = 0;
                sh.mask = 0;
                sh.need = K;
                sh.tied = uint32_t(n);
            }
            __syncthreads();
        }
        // Only elements whose digit is at least D are counted and kept: the
        // K-th key's digit is found among them or the row takes the general
        // path.  A batch wholly inside the row skips the per-element test
        // against the row's end.
        auto run = [&](auto check_c) {
            constexpr bool CHECK = decltype(check_c)::value;
            auto keep = [&](int u, int v, uint32_t b) {
                return (!CHECK || (g0 + u * kThreads) * V + v < n32) && (b >> 20) >= d_min;
            };
            uint32_t cnt = 0;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const uint32_t b = score_bits(x[u][v]);
                    if (keep(u, v, b)) {
                        atomicAdd(&sh.hist[b >> 20], 1u);
                        ++cnt;
                    }
                }
            uint32_t incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(incl, o);
                if (lane >= o) incl += y;
            }
            const uint32_t tot = __shfl(incl, 63);
            if (tot == 0) return;
            uint32_t at = 0;
            if (lane == 0) at = atomicAdd(&buf.n, tot);
            at = __shfl(at, 0) + incl - cnt;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const uint32_t b = score_bits(x[u][v]);
                    if (!keep(u, v, b)) continue;
                    if (at < uint32_t(kBuf)) {
                        buf.sb[at] = b;
                        buf.idx[at] = uint32_t((g0 + u * kThreads) * V + v);
                    }
                    ++at;
                }
        };
        if ((base + kThreads * U) * V <= n32)
            run(std::false_type{});
        else
            run(std::true_type{});
    }
    __syncthreads();
    pick_digit(sh, sh.hist, kBins, 52);
    const uint32_t kept = buf.n;
    const bool fits = kept <= uint32_t(kBuf) && uint32_t(sh.prefix >> 52) >= d_min;
    __syncthreads();  // the caller may reset the state next
    if (!fits) return false;
    settle_in_lds(sh, buf, kept);
    const uint64_t pre = sh.prefix, msk = sh.mask;
    for (uint32_t j = threadIdx.x; j < kept; j += kThreads) {
        const uint32_t i = buf.idx[j];
        if ((key_of(buf.sb[j], i) & msk) >= pre) atomicOr(&bits[i >> 5], 1u << (i & 31));
    }
    __syncthreads();
    return true;
}

// Request b, index t in it and its token count c of query token qi when
// request b holds tokens qsl[b] .. qsl[b + 1] - 1.  The workgroup reads the
// offsets together and counts those after qsl[0] that are <= qi; false when
// the offsets are not a partition of 0 .. n_q (first 0, last n_q, none
// decreasing).  Every thread of the workgroup must call it.
__device__ bool varlen_token(const int32_t* qsl, int32_t B, int32_t n_q, int32_t qi, int32_t& b,
                             int32_t& t, int32_t& c) {
    int32_t below = 0;
    int bad = threadIdx.x == 0 && (qsl[0] != 0 || qsl[B] != n_q);
    for (int32_t j0 = 1; j0 <= B; j0 += kThreads) {  // the same trip count in every thread
        const int32_t j = j0 + int32_t(threadIdx.x);
        int le = 0;
        if (j <= B) {
            const int32_t v = qsl[j];
            le = v <= qi;
            bad |= v < qsl[j - 1];
        }
        below += __syncthreads_count(le);
    }
    if (__syncthreads_or(bad) || below >= B) return false;
    b = below;
    const int32_t start = qsl[b];
    t = qi - start;
    c = qsl[b + 1] - start;
    return true;
}

// Local top-K of one (shard, request, query token) row.  Dynamic LDS: the
// bitmap (one bit per local position of the longest row of the launch) and
// the running count of set bits before each bitmap word.
// Two workgroups per CU (LDS allows it): at most 128 VGPRs.
static_assert(sizeof(SelectShared) + sizeof(SelList) + kMaxLocal / 32 * 8 + 1024 <= 160 * 1024,
              "the longest local row's bitmap fits beside the selection's static LDS");
__global__ void __launch_bounds__(kThreads, 4) local_topk_kernel(LocalParams p, int32_t bitmap_words) {
    __shared__ SelectShared sh;
    __shared__ SelList sel;
    extern __shared__ uint32_t dyn[];
    uint32_t* bits = dyn;
    uint32_t* wprefix = dyn + bitmap_words;
    const int32_t row = blockIdx.x;  // (s_rel, query token)
    const int32_t s_rel = row / p.n_q;
    const int32_t qi = row - s_rel * p.n_q;
    const int32_t s = p.shard_begin + s_rel;
    int32_t vis;
    if (!p.qsl) {
        const int32_t t = qi % p.Tq;
        vis = p.context_lens[qi / p.Tq] - p.Tq + t + 1;
    } else {
        int32_t b, t, c;
        vis = 0;  // a token that cannot be placed selects nothing
        if (varlen_token(p.qsl, p.B, p.n_q, qi, b, t, c)) vis = p.context_lens[b] - c + t + 1;
        else if (threadIdx.x == 0 && p.err) raise_error(p.err, MLA_DEVERR_QUERY);
    }
    if (vis < 0) vis = 0;
    int64_t n = dev_local_len(vis, s, p.n_shards);
    if (n > p.stride) {  // the score row is shorter than the shard's visible prefix
        if (threadIdx.x == 0 && p.err) raise_error(p.err, MLA_DEVERR_SCORES);
        n = p.stride;
    }
    const float* scores = p.scores + size_t(row) * p.stride;
    int32_t* out_i = p.out_idx + size_t(row) * p.K;
    float* out_s = p.out_score + size_t(row) * p.K;
    if (n <= p.K) {  // every owned position is kept, in order
        for (int64_t j = threadIdx.x; j < p.K; j += kThreads) {
            out_i[j] = j < n ? int32_t(j * p.n_shards + s) : -1;
            out_s[j] = j < n ? canon(scores[j]) : -INFINITY;
        }
        return;
    }
    const int32_t words = int32_t((n + 31) >> 5);
    for (int i = threadIdx.x; i < words; i += kThreads) bits[i] = 0;
    __syncthreads();
    const int per = (words + kThreads - 1) / kThreads;
    const int w0 = threadIdx.x * per;
    const bool vec = (reinterpret_cast<uintptr_t>(scores) & 15u) == 0 && (p.stride & 3) == 0;
    if (p.K <= kSel) {
        // one read of the row when the sample's estimate holds; else the
        // digit passes, listing the kept elements as they are marked
        const bool one = vec ? select_one_pass<8>(sh, sel, LocalSrc4{scores}, scores, n, uint32_t(p.K), bits)
                             : select_one_pass<16>(sh, sel, LocalSrc{scores}, scores, n, uint32_t(p.K), bits);
        uint32_t listed = uint32_t(p.K);
        uint64_t pre = 0, msk = 0;
        if (one) {
            listed = sel.n;
            pre = sh.prefix;
            msk = sh.mask;
        } else if (vec) {
            select_into_bitmap<2, true>(sh, LocalSrc4{scores}, n, uint32_t(p.K), bits, &sel);
        } else {
            select_into_bitmap<8, true>(sh, LocalSrc{scores}, n, uint32_t(p.K), bits, &sel);
        }
        // output slot of a kept element = kept elements before it
        uint32_t cnt = 0;
        for (int w = w0; w < w0 + per && w < words; ++w) cnt += __popc(bits[w]);
        uint32_t total;
        uint32_t run = block_excl_scan_u32(cnt, sh.scan, total);
        for (int w = w0; w < w0 + per && w < words; ++w) {
            wprefix[w] = run;
            run += __popc(bits[w]);
        }
        __syncthreads();
        for (uint32_t j = threadIdx.x; j < listed && j < uint32_t(kBuf); j += kThreads) {
            const uint32_t i = sel.idx[j];
            if (one && (key_of(sel.sb[j], i) & msk) < pre) continue;  // kept in LDS, not chosen
            const uint32_t rank = wprefix[i >> 5] + __popc(bits[i >> 5] & ((1u << (i & 31)) - 1u));
            if (rank < uint32_t(p.K)) {  // exactly K are chosen; the check guards the output row
                out_i[rank] = int32_t(int64_t(i) * p.n_shards + s);
                out_s[rank] = score_of(sel.sb[j]);
            }
        }
        return;
    }
    if (vec)
        select_into_bitmap<2, false>(sh, LocalSrc4{scores}, n, uint32_t(p.K), bits);
    else
        select_into_bitmap<8, false>(sh, LocalSrc{scores}, n, uint32_t(p.K), bits);
    // set bits in index order -> ascending positions
    uint32_t cnt = 0;
    for (int w = w0; w < w0 + per && w < words; ++w) cnt += __popc(bits[w]);
    uint32_t total;
    uint32_t pos = block_excl_scan_u32(cnt, sh.scan, total);
    for (int w = w0; w < w0 + per && w < words; ++w) {
        uint32_t m = bits[w];
        while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1;
            const int64_t j = int64_t(w) * 32 + bit;
            out_i[pos] = int32_t(j * p.n_shards + s);
            out_s[pos] = canon(scores[j]);
            ++pos;
        }
    }
    for (int32_t i = int32_t(total) + threadIdx.x; i < p.K; i += kThreads) {
        out_i[i] = -1;
        out_s[i] = -INFINITY;
    }
}

struct MergeSrc {
    const int32_t* idx;
    const float* score;
    size_t list_stride;
    int32_t k_in;
    __device__ size_t at(int64_t i) const {
        const uint32_t l = uint32_t(i) / uint32_t(k_in);
        return size_t(l) * list_stride + (uint32_t(i) - l * uint32_t(k_in));
    }
    static constexpr int V = 1;
    __device__ void keys(int64_t g, int64_t, uint64_t (&k)[V]) const {
        const size_t a = at(g);
        const int32_t id = idx[a];
        k[0] = id >= 0 ? make_key(score[a], uint32_t(id)) : 0;
    }
};

// Global top-K of one row from the shards' candidate lists.  Dynamic LDS:
// a bitmap over the n_lists * k_in candidates, then the K chosen positions.
__global__ void __launch_bounds__(kThreads, 4) merge_topk_kernel(MergeParams p, int32_t bitmap_words) {
    __shared__ SelectShared sh;
    extern __shared__ uint32_t dyn[];
    uint32_t* bits = dyn;
    int32_t* chosen = reinterpret_cast<int32_t*>(dyn + bitmap_words);
    const int64_t row = blockIdx.x;
    const size_t list_stride = size_t(p.rows) * p.k_in;
    const int32_t* idx = p.cand_idx + size_t(row) * p.k_in;
    const float* sc = p.cand_score + size_t(row) * p.k_in;
    const MergeSrc src{idx, sc, list_stride, p.k_in};
    const int64_t n = int64_t(p.n_lists) * p.k_in;
    for (int i = threadIdx.x; i < bitmap_words; i += kThreads) bits[i] = 0;
    // valid candidates
    uint32_t nv = 0;
    for_each_key<16>(src, n, [&](int64_t, uint64_t) { ++nv; });
    uint32_t n_valid;
    block_excl_scan_u32(nv, sh.scan, n_valid);  // also orders the clearing above
    if (n_valid <= uint32_t(p.K)) {
        for_each_key<16>(src, n, [&](int64_t i, uint64_t) { atomicOr(&bits[i >> 5], 1u << (i & 31)); });
        __syncthreads();
    } else {
        select_into_bitmap<16, false>(sh, src, n, uint32_t(p.K), bits);
    }
    // gather the chosen positions (bitmap order), then sort them ascending
    const int per = (bitmap_words + kThreads - 1) / kThreads;
    const int w0 = threadIdx.x * per;
    uint32_t cnt = 0;
    for (int w = w0; w < w0 + per && w < bitmap_words; ++w) cnt += __popc(bits[w]);
    uint32_t total;
    uint32_t pos = block_excl_scan_u32(cnt, sh.scan, total);
    for (int w = w0; w < w0 + per && w < bitmap_words; ++w) {
        uint32_t m = bits[w];
        while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1;
            chosen[pos++] = idx[src.at(int64_t(w) * 32 + bit)];
        }
    }
    uint32_t pw = 1;
    while (pw < total) pw <<= 1;
    for (uint32_t i = total + threadIdx.x; i < pw; i += kThreads) chosen[i] = INT32_MAX;
    __syncthreads();
    for (uint32_t size = 2; size <= pw; size <<= 1) {
        for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
            for (uint32_t i = threadIdx.x; i < pw / 2; i += kThreads) {
                const uint32_t lo = 2 * i - (i & (stride - 1));
                const uint32_t hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const int32_t a = chosen[lo], c = chosen[hi];
                if ((a > c) == asc) {
                    chosen[lo] = c;
                    chosen[hi] = a;
                }
            }
            __syncthreads();
        }
    }
    int32_t* out = p.out_idx + size_t(row) * p.K;
    for (int32_t i = threadIdx.x; i < p.K; i += kThreads) out[i] = uint32_t(i) < total ? chosen[i] : -1;
}

// ---- rows read once into LDS --------------------------------------------
//
// A row of at most kStage elements is loaded into LDS in one sweep (16-byte
// loads, all of a thread's loads in flight at once) and every later pass
// reads LDS, so the scores cross HBM once.  128 KB of staging plus the
// selection state fills one CU's LDS: one workgroup per CU.

struct StagedMergeSrc {
    static constexpr int V = 1;
    const int32_t* idx;
    const float* score;
    __device__ void keys(int64_t g, int64_t, uint64_t (&k)[V]) const {
        const int32_t id = idx[g];
        k[0] = id >= 0 ? make_key(score[g], uint32_t(id)) : 0;
    }
};

// n_lists * k_in <= kStage / 2 candidates, K <= kStageK.
__global__ void __launch_bounds__(kThreads) merge_topk_staged_kernel(MergeParams p) {
    constexpr int kN = kStage / 2;
    __shared__ SelectShared sh;
    __shared__ int32_t idx_s[kN];
    __shared__ float sc_s[kN];
    __shared__ uint32_t bits[kN / 32];
    const int64_t row = blockIdx.x;
    const size_t list_stride = size_t(p.rows) * p.k_in;
    const int64_t n = int64_t(p.n_lists) * p.k_in;
    {
        // all of a thread's loads in flight before the first LDS store
        constexpr int kPer = kN / kThreads;  // 32
        int32_t vi[kPer];
        float vs[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = int64_t(j) * kThreads + threadIdx.x;
            if (i < n) {
                const uint32_t l = uint32_t(i) / uint32_t(p.k_in);
                const size_t a = size_t(l) * list_stride + size_t(row) * p.k_in + (uint32_t(i) - l * uint32_t(p.k_in));
                vi[j] = p.cand_idx[a];
                vs[j] = p.cand_score[a];
            }
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int64_t i = int64_t(j) * kThreads + threadIdx.x;
            if (i < n) {
                idx_s[i] = vi[j];
                sc_s[i] = vs[j];
            }
        }
    }
    const int32_t words = int32_t((n + 31) / 32);
    for (int i = threadIdx.x; i < words; i += kThreads) bits[i] = 0;
    __syncthreads();
    const StagedMergeSrc src{idx_s, sc_s};
    uint32_t nv = 0;
    for_each_key<8>(src, n, [&](int64_t, uint64_t) { ++nv; });
    uint32_t n_valid;
    block_excl_scan_u32(nv, sh.scan, n_valid);
    if (n_valid <= uint32_t(p.K)) {
        for_each_key<8>(src, n, [&](int64_t i, uint64_t) { atomicOr(&bits[i >> 5], 1u << (i & 31)); });
        __syncthreads();
    } else {
        select_into_bitmap<8, false>(sh, src, n, uint32_t(p.K), bits);
    }
    // The chosen positions, compacted in candidate order (the tied-group
    // space holds two lists of kCand); wpre[w] = chosen before word w.
    int32_t* chosen = reinterpret_cast<int32_t*>(sh.cand_key);
    int32_t* merged = chosen + kCand;
    __shared__ uint32_t wpre[kN / 32];
    __shared__ uint32_t unsorted, max_pos;
    const int per = (words + kThreads - 1) / kThreads;
    const int w0 = threadIdx.x * per;
    uint32_t cnt = 0;
    for (int w = w0; w < w0 + per && w < words; ++w) cnt += __popc(bits[w]);
    uint32_t total;
    uint32_t pos = block_excl_scan_u32(cnt, sh.scan, total);
    if (threadIdx.x == 0) {
        unsorted = 0;
        max_pos = 0;
    }
    for (int w = w0; w < w0 + per && w < words; ++w) {
        wpre[w] = pos;
        uint32_t m = bits[w];
        while (m) {
            const int bit = __builtin_ctz(m);
            m &= m - 1;
            chosen[pos++] = idx_s[w * 32 + bit];
        }
    }
    __syncthreads();
    // Ascending order.  When every chosen position is below 2^19, the
    // staging arrays (free now) hold a bitmap over positions: an entry's
    // output index is the number of set bits before its own.  Otherwise the
    // lists' sorted runs are merged, or sorted when a list is not ascending.
    constexpr int kPerT = kCand / kThreads;
    constexpr uint32_t kPosBits = uint32_t(kN) * 32;  // idx_s as a bitmap
    {
        uint32_t mx = 0;
#pragma unroll
        for (int k = 0; k < kPerT; ++k) {
            const uint32_t c = threadIdx.x + k * kThreads;
            if (c < total) mx = max(mx, uint32_t(chosen[c]));
        }
        mx = uint32_t(wave_max_u32(mx));
        if ((threadIdx.x & 63) == 0) atomicMax(&max_pos, mx);
    }
    __syncthreads();
    if (total > 0 && max_pos < kPosBits) {
        uint32_t* pbits = reinterpret_cast<uint32_t*>(idx_s);
        uint32_t* pre = reinterpret_cast<uint32_t*>(sc_s);  // set bits before each word
        const uint32_t nw = max_pos / 32 + 1;
        for (uint32_t w = threadIdx.x; w < nw; w += kThreads) pbits[w] = 0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPerT; ++k) {
            const uint32_t c = threadIdx.x + k * kThreads;
            if (c < total) atomicOr(&pbits[uint32_t(chosen[c]) >> 5], 1u << (uint32_t(chosen[c]) & 31u));
        }
        __syncthreads();
        const uint32_t per_w = (nw + kThreads - 1) / kThreads;
        const uint32_t wb = threadIdx.x * per_w;
        uint32_t mine = 0;
        for (uint32_t w = wb; w < wb + per_w && w < nw; ++w) mine += __popc(pbits[w]);
        uint32_t all;
        uint32_t run_b = block_excl_scan_u32(mine, sh.scan, all);
        for (uint32_t w = wb; w < wb + per_w && w < nw; ++w) {
            pre[w] = run_b;
            run_b += __popc(pbits[w]);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPerT; ++k) {
            const uint32_t c = threadIdx.x + k * kThreads;
            if (c >= total) continue;
            const uint32_t v = uint32_t(chosen[c]);
            merged[pre[v >> 5] + __popc(pbits[v >> 5] & ((1u << (v & 31u)) - 1u))] = int32_t(v);
        }
        __syncthreads();
        int32_t* out = p.out_idx + size_t(row) * p.K;
        for (int32_t i = threadIdx.x; i < p.K; i += kThreads) out[i] = uint32_t(i) < total ? merged[i] : -1;
        return;
    }
    // chosen entries of list l start at rs[l] (rs[n_lists] = total); a list
    // of mla_topk_local is ascending, so its chosen entries form a sorted run
    const bool tree = p.n_lists <= 64;
    __shared__ uint32_t rs[65];
    if (tree && int(threadIdx.x) <= p.n_lists) {
        const uint32_t c = uint32_t(threadIdx.x) * uint32_t(p.k_in);
        const uint32_t w = c >> 5, b = c & 31u;
        rs[threadIdx.x] = (int(threadIdx.x) == p.n_lists || w >= uint32_t(words))
                              ? total : wpre[w] + __popc(bits[w] & ((1u << b) - 1u));
    }
    __syncthreads();
    // a thread's entries c = tid + k * kThreads; their searches advance in
    // step, so the LDS reads of one step are in flight together
    int lrun[kPerT];  // list (run) of each entry
#pragma unroll
    for (int k = 0; k < kPerT; ++k) lrun[k] = 0;
    if (tree) {
        for (int step = 32; step > 0; step >>= 1) {
#pragma unroll
            for (int k = 0; k < kPerT; ++k) {
                const uint32_t c = threadIdx.x + k * kThreads;
                const int t = lrun[k] + step;
                const uint32_t r = rs[t < p.n_lists ? t : p.n_lists];  // rs[n_lists] = total
                lrun[k] = (t < p.n_lists && r <= c) ? t : lrun[k];
            }
        }
#pragma unroll
        for (int k = 0; k < kPerT; ++k) {
            const uint32_t c = threadIdx.x + k * kThreads;
            if (c < total && c > rs[lrun[k]] && chosen[c - 1] > chosen[c]) unsorted = 1;
        }
        __syncthreads();
    }
    const int32_t* result = chosen;
    if (tree && !unsorted) {
        // Pairwise merges of sorted runs, log2(n_lists) levels: an entry's
        // place in the merged run is its index in its own run plus the
        // entries of the partner run below it (positions are distinct).
        int32_t* src_b = chosen;
        int32_t* dst_b = merged;
        const int nl = p.n_lists;
        auto start = [&](int l) { return rs[l < nl ? l : nl]; };
        for (int span = 1; span < nl; span <<= 1) {
            uint32_t lo[kPerT], len[kPerT], b0[kPerT];
            int32_t v[kPerT];
#pragma unroll
            for (int k = 0; k < kPerT; ++k) {
                const uint32_t c = threadIdx.x + k * kThreads;
                const int l = lrun[k] / span, mate = l ^ 1;
                b0[k] = start(mate * span);
                lo[k] = b0[k];
                len[k] = start((mate + 1) * span) - b0[k];
                v[k] = src_b[c < total ? c : 0];
            }
            // first partner entry >= v: a fixed number of halving steps with
            // no branch, so the four searches' reads go out together
            const uint32_t last = total > 0 ? total - 1 : 0;
            for (int it = 0; it < 12; ++it) {
#pragma unroll
                for (int k = 0; k < kPerT; ++k) {
                    const uint32_t half = len[k] >> 1;
                    const uint32_t probe = lo[k] + half;
                    const int32_t x = src_b[probe < last ? probe : last];
                    const bool go = len[k] > 0 && x < v[k];
                    lo[k] = go ? probe + 1 : lo[k];
                    len[k] = len[k] == 0 ? 0u : (go ? len[k] - half - 1 : half);
                }
            }
#pragma unroll
            for (int k = 0; k < kPerT; ++k) {
                const uint32_t c = threadIdx.x + k * kThreads;
                if (c >= total) continue;
                const int l = lrun[k] / span;
                dst_b[start((l & ~1) * span) + (c - start(l * span)) + (lo[k] - b0[k])] = v[k];
            }
            __syncthreads();
            int32_t* t = src_b;
            src_b = dst_b;
            dst_b = t;
        }
        result = src_b;
    } else {
        // candidate lists in no particular order: bitonic sort in LDS
        uint32_t pw = 1;
        while (pw < total) pw <<= 1;
        for (uint32_t i = total + threadIdx.x; i < pw; i += kThreads) chosen[i] = INT32_MAX;
        __syncthreads();
        for (uint32_t size = 2; size <= pw; size <<= 1) {
            for (uint32_t stride = size >> 1; stride > 0; stride >>= 1) {
                for (uint32_t i = threadIdx.x; i < pw / 2; i += kThreads) {
                    const uint32_t lo = 2 * i - (i & (stride - 1));
                    const uint32_t hi = lo + stride;
                    const bool asc = (lo & size) == 0;
                    const int32_t a = chosen[lo], c = chosen[hi];
                    if ((a > c) == asc) {
                        chosen[lo] = c;
                        chosen[hi] = a;
                    }
                }
                __syncthreads();
            }
        }
    }
    int32_t* out = p.out_idx + size_t(row) * p.K;
    for (int32_t i = threadIdx.x; i < p.K; i += kThreads) out[i] = uint32_t(i) < total ? result[i] : -1;
}

}  // namespace topk
}  // namespace mla
