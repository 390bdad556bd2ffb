// Matrix-core partial decode for the packed fp8 latent cache (gfx950), dense
// and sparse.
//
// Row format (656 B): 512 E4M3FN codes, 4 float32 scales (one per 128-dim
// group), 64 bf16 rope values.  Latent value d of token t is
// code[t][d] * scale[t][d / 128].
//
// One workgroup of NW waves handles one (shard, request, query token, chunk)
// row; wave w owns query heads [32w, 32w + 32).  Rows stream through a ring
// of three 32-token sub-tiles in LDS (direct global->LDS loads), with codes,
// rope parts and scales in separate regions.  Codes are widened to bf16
// exactly in registers (v_cvt_scalef32_pk_bf16_fp8 with scale 1) right before
// their MFMA, and the group scales are applied in float32 outside the
// products, so the scores are exact bf16 x fp8 products accumulated in
// float32:
//
//   S^T  = K_rope . Q_rope^T + sum_g scale_g (.) (C_g . Q_g^T)      MFMA 32x32x16
//   O^T += sum_g C_g^T . (P (.) scale_g)^T                          MFMA 32x32x16
//
// C_g are the codes of group g, (.) scales token rows.  The convert
// instructions of each MFMA's operand are issued while the previous MFMA
// runs; loads stay two sub-tiles ahead of compute.
//
// Score steps pair up: one 16-byte read of a code row feeds two MFMAs, so
// K-step 2s + e covers dims 32 s + 16 half + 8 e .. + 8 of lane half `half`,
// and the query fragments are loaded in the same order.  V^T fragments come
// from ds_read_b64_tr_b8: in each 16-lane group, output lane i receives byte
// i % 8 of source lanes 2r + i / 8 (r = 0..7), so source lane 2r + b loads 8
// codes of one token, which gives each lane 8 tokens of one latent dimension.
//
// Sparse rows (top-K) first compact the entries this shard owns, in entry
// order, into an LDS list of pool rows; the ring then gathers 32 listed rows
// per sub-tile.
#pragma once

#include "common.hpp"
#include "mfma_common.hpp"
#include "params.hpp"

namespace mla {
namespace mfma {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kRowF = 656;            // bytes per fp8 row in the cache
constexpr int kScaleOff = kLatent;    // byte offset of the scales in a row
constexpr int kRopeOff = kLatent + 16;  // byte offset of the rope part
constexpr int kMaxTopk = 2048;        // longest top-K list kept in LDS
constexpr int kRingF = 3;             // sub-tiles resident in LDS

// LDS regions of one ring slot.  Code row t (512 B) keeps its 16-byte chunk c
// at (c & 16) | ((c & 15) ^ f8(t)); rope chunk c of row t at c ^ ((t >> 1) & 7).
// With 64 four-byte banks, the 16-lane passes of the K code reads (16 rows,
// one chunk each) and the 32-lane passes of the transposing V^T reads (8 rows
// x 2 chunks) then hit every bank once.
constexpr int kCodesB = kSub * kLatent;  // 16 KB
constexpr int kRopeSB = kSub * kRope * 2;  // 4 KB
constexpr int kSclB = kSub * 16;         // 512 B: 4 f32 per row
__device__ __forceinline__ int f8swz(int t) {
    return ((t & 3) << 2) | (((t >> 3) & 1) << 1) | ((t >> 2) & 1);
}
__device__ __forceinline__ int code_pos(int c, int t) { return (c & 16) | ((c & 15) ^ f8swz(t)); }
__device__ __forceinline__ int rope_swz(int t) { return (t >> 1) & 7; }

template <int NW, bool SPARSE>
struct alignas(16) SmemFp8 {
    uint8_t codes[kRingF][kCodesB];
    uint8_t rope[kRingF][kRopeSB];
    uint8_t scl[kRingF][kSclB];
    // scales of a slot as [group][token].  Every wave writes all of it (the
    // same values) before reading it, and a slot is rewritten only three
    // barriers after its last read, so the shared copy needs no extra sync.
    float sct[kRingF][4][kSub];
    uint8_t qrope[NW * 32 * kRope * 2];   // [head][8 chunks], chunk c at c ^ ((head >> 1) & 7)
    int32_t rows[SPARSE ? kMaxTopk : 1];  // sparse: pool rows this shard owns, entry order
    int32_t wave_cnt[NW];
};

// 8 E4M3FN codes (two dwords, byte e = token/dim e) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(int lo, int hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = d[0]; r[5] = d[1]; r[6] = e[0]; r[7] = e[1];
    return r;
}

template <int NW, bool SPARSE>
__global__ void __launch_bounds__(NW * 64, 1) decode_mfma_fp8_kernel(DecodeParams p) {
    __shared__ SmemFp8<NW, SPARSE> sm;
    constexpr int kCodeLoads = kSub / 2 / NW;   // code loads per wave (2 rows each)
    constexpr int kRopeLoads = kSub / 8 / NW;   // rope loads per wave (8 rows each)
    constexpr int kSclRows = kSub / NW;         // scale rows per wave (one load)
    constexpr int kLoads = kCodeLoads + kRopeLoads + 1;
    RowId id;
    if (!work_item(p, blockIdx.x, id)) return;  // past the last planned item
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int half = lane >> 5;
    const int col = lane & 31;
    const int head = wave * 32 + col;
    const int s = p.shard_begin + id.s_rel;
    const int32_t* bt = p.block_tables + (size_t(id.s_rel) * p.B + id.b) * p.max_blocks;
    const __attribute__((address_space(4))) int32_t* btc =
        (const __attribute__((address_space(4))) int32_t*)bt;

    const int32_t L = p.context_lens[id.b];
    int32_t visible = L - id.qlen + id.t + 1;
    if (visible < 0) visible = 0;

    // ---- query fragments: latent in registers (paired-step order), rope
    // part through LDS.  Issued first, so that their latency overlaps the
    // sparse compaction's loads.
    bf16x8 qf[kQLatSteps];
    bf16x8 qrope_r[4];
    const int qr_off = head * (kRope * 2);
    const int qr_sw = (head >> 1) & 7;
    {
        const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
            static_cast<const uint16_t*>(p.q) + (size_t(id.qi) * p.H + head) * kDk);
#pragma unroll
        for (int ks = 0; ks < kQLatSteps; ++ks) qf[ks] = qrow[4 * (ks >> 1) + 2 * half + (ks & 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) qrope_r[u] = qrow[2 * (kQLatSteps + u) + half];
    }

    // ---- the tokens this workgroup attends ---------------------------------
    int32_t tok0 = 0, tok1 = 0;  // dense: local token range; sparse: list range
    int total_owned = 0;
    if (!SPARSE) {
        int32_t local = dev_local_len(visible, s, p.n_shards);
        if ((local + kBlock - 1) / kBlock > p.max_blocks) {
            if (threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
            local = p.max_blocks * kBlock;
        }
        tok0 = id.chunk * id.chunk_tok;
        tok1 = id.chunk_tok ? min(tok0 + id.chunk_tok, local) : local;
        if (tok1 < tok0) tok1 = tok0;
    } else {
        // Compact the entries this shard owns, in entry order: wave w scans
        // its own slice of the list (ballot + popcount, no barrier), then
        // moves its owned entries down to their final position.
        // The block-table row goes to LDS (the third ring slot is free until
        // the ring starts) with direct loads issued beside the index loads,
        // so one memory round trip covers the query, the indices and the
        // table; a row wider than the slot is looked up in memory instead.
        const bool bt_lds = p.max_blocks <= kCodesB / 4;
        const uint32_t bt_stage = lds_addr(sm.codes[kRingF - 1]);
        if (bt_lds) {
            const int nk = (p.max_blocks + NW * 64 - 1) / (NW * 64);
            const uint32_t m_bt = __builtin_amdgcn_readfirstlane(bt_stage + wv * 256);
            for (int k = 0; k < nk; ++k) {
                const int e = k * NW * 64 + wave * 64 + lane;
                dma4_at<0>(bt, 4 * (e < p.max_blocks ? e : p.max_blocks - 1),
                           __builtin_amdgcn_readfirstlane(m_bt + k * NW * 256));
            }
        }
        const MLA_LDS int32_t* bt_l = (const MLA_LDS int32_t*)sm.codes[kRingF - 1];
        const int32_t* idx = p.topk_idx + size_t(id.qi) * p.topk;
        const int32_t slice = (p.topk + NW - 1) / NW;
        const int32_t e_begin = wave * slice;
        const int32_t e_end = min(p.topk, e_begin + slice);
        const uint64_t below = (uint64_t(1) << lane) - 1;
        // all index loads of the slice in flight at once, then all block-table
        // lookups, then the ballots (slice <= kMaxTopk / NW entries)
        constexpr int kSteps = kMaxTopk / (NW * 64);
        int32_t gv[kSteps];
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            const int32_t e = e_begin + k * 64 + lane;
            gv[k] = e < e_end ? idx[e] : -1;
        }
        if (bt_lds) {
            wait_vm<0>();  // this wave's table loads (and the query and index loads)
            __syncthreads();
        }
        const double inv_n = 1.0 / double(p.n_shards);
        int32_t row[kSteps];
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            const int32_t g = gv[k];
            const int32_t j = div_by(g < 0 ? 0 : g, inv_n);  // local index if owned
            row[k] = -1;
            if (g >= visible) {
                raise_error(p.err, MLA_DEVERR_INDEX);
            } else if (g >= 0 && g - j * p.n_shards == s) {
                // block id for now
                row[k] = j / kBlock >= p.max_blocks ? -1 : bt_lds ? bt_l[j / kBlock] : bt[j / kBlock];
                row[k] = row[k] >= 0 && row[k] < p.pool_blocks ? row[k] * kBlock + (j % kBlock) : -2;
            }
        }
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            if (row[k] == -2) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
            const uint64_t mask = __ballot(row[k] >= 0);
            if (row[k] >= 0) sm.rows[e_begin + cnt + __popcll(mask & below)] = row[k];
            cnt += __popcll(mask);
        }
        if (lane == 0) sm.wave_cnt[wave] = cnt;
        __syncthreads();
        int base = 0;
        total_owned = 0;
        for (int w = 0; w < NW; ++w) {
            const int c = sm.wave_cnt[w];
            if (w < wave) base += c;
            total_owned += c;
        }
        // Move every wave's entries to their final position.  A later wave's
        // destination can overlap an earlier wave's source, so all waves
        // read first, then all write.
        constexpr int kPerLane = kMaxTopk / (NW * 64);  // slice <= kMaxTopk / NW
        int32_t mine[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int i = k * 64 + lane;
            mine[k] = i < cnt ? sm.rows[e_begin + i] : 0;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int i = k * 64 + lane;
            if (i < cnt) sm.rows[base + i] = mine[k];
        }
        __syncthreads();
        tok1 = total_owned;
    }
    const int n_sub = tok1 > tok0 ? (tok1 - tok0 + kSub - 1) / kSub : 0;
    // the pipelined loop is unrolled by the ring size and always runs whole
    // rounds: padding sub-tiles are zero rows with every score masked
    const int n_pad = (n_sub + kRingF - 1) / kRingF * kRingF;

    // rope part in LDS; each wave writes and later reads only its own heads
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int c = 2 * u + half;
        *(MLA_LDS bf16x8*)((MLA_LDS uint8_t*)sm.qrope + qr_off + ((c ^ qr_sw) << 4)) = qrope_r[u];
    }
    auto qread = [&](int u) -> bf16x8 {
        return *(const MLA_LDS bf16x8*)((const MLA_LDS uint8_t*)sm.qrope + qr_off +
                                        (((2 * u + half) ^ qr_sw) << 4));
    };

    // ---- sub-tile loads ------------------------------------------------------
    // wave w: code loads k = 0..kCodeLoads-1 cover rows 2i, 2i + 1 with
    // i = w * kCodeLoads + k (lane half picks the row, lane % 32 the stored
    // chunk position); rope loads cover rows 8i .. 8i + 7 with
    // i = w * kRopeLoads + k; one scale load covers rows w * kSclRows + lane.
    // Byte offsets (in a sub-tile's rows) of the chunks a lane loads.  Code
    // load k of wave w covers rows 2i, 2i + 1 (i = w * kCodeLoads + k; lane
    // half h picks the row), rope load k rows 8i' .. 8i' + 7 (i' = w *
    // kRopeLoads + k), the scale load rows w * kSclRows + lane.  The swizzle of
    // row 2i + h is (h << 2) ^ U(i) with U linear in the bits of i, so every
    // offset is a per-lane part XOR a compile-time constant, plus a row term.
    auto u_bits = [](int i) { return ((2 * (i & 1)) << 2) | (((i >> 2) & 1) << 1) | ((i >> 1) & 1); };
    const int h = lane >> 5;
    const int c_x0 = ((((lane & 16) | ((lane & 15) ^ (h << 2)))) ^ u_bits(wave * kCodeLoads)) << 4;
    const int c_h0 = (h + 2 * wave * kCodeLoads) * kRowF;
    const int rr = lane >> 3;
    const int r_x0 = (((lane & 7) ^ (rr >> 1)) ^ (4 * ((wave * kRopeLoads) & 1))) << 4;
    const int r_h0 = (rr + 8 * wave * kRopeLoads) * kRowF + kRopeOff;
    const int s_row0 = wave * kSclRows + lane;  // scale load (lanes < kSclRows)
    const uint32_t lc0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.codes) + wv * kCodeLoads * 1024);
    const uint32_t lr0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.rope) + wv * kRopeLoads * 1024);
    const uint32_t ls0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.scl) + wv * kSclRows * 16);

    bool bad_slot[kRingF] = {false, false, false};
    auto issue = [&](int j, auto slot_c) {
        constexpr int slot = decltype(slot_c)::value;
        // opaque copies: the per-load offsets below are then computed here,
        // not hoisted out of the loop into a dozen live registers
        int c_x = c_x0, c_h = c_h0, r_x = r_x0, r_h = r_h0, s_row = s_row0;
        asm volatile("" : "+v"(c_x), "+v"(c_h), "+v"(r_x), "+v"(r_h), "+v"(s_row));
        const int32_t j0 = tok0 + j * kSub;
        const int v = min(kSub, tok1 - j0);  // <= 0: padding
        if (!SPARSE) {
            const uint8_t* src = kZeroRow;
            bool bad = false;
            int last = 0;
            if (v > 0) {
                const int32_t blk = btc[uint32_t(j0) / kBlock];
                if (blk >= 0 && blk < p.pool_blocks) {
                    src = p.kv + (int64_t(blk) * kBlock + (uint32_t(j0) % kBlock)) * kRowF;
                    last = v - 1;
                } else {
                    bad = true;
                }
            }
            bad_slot[slot] = bad;
            if (v == kSub && !bad) {
                static_for<0, kCodeLoads>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    dma16_at<slot * kCodesB + k * 1024>(src, (c_x ^ (u_bits(k) << 4)) + c_h + 2 * k * kRowF,
                                                        lc0);
                });
                static_for<0, kRopeLoads>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    dma16_at<slot * kRopeSB + k * 1024>(src, (r_x ^ ((4 * (k & 1)) << 4)) + r_h + 8 * k * kRowF,
                                                        lr0);
                });
                if (lane < kSclRows) dma16_at<slot * kSclB>(src, s_row * kRowF + kScaleOff, ls0);
            } else {
                // rows past `last` re-read row `last`
                static_for<0, kCodeLoads>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    const int t = 2 * (wv * kCodeLoads + k) + h;
                    dma16_at<slot * kCodesB + k * 1024>(
                        src, (c_x ^ (u_bits(k) << 4)) + (t < last ? t : last) * kRowF, lc0);
                });
                static_for<0, kRopeLoads>([&](auto kc) {
                    constexpr int k = decltype(kc)::value;
                    const int t = 8 * (wv * kRopeLoads + k) + rr;
                    dma16_at<slot * kRopeSB + k * 1024>(
                        src, (r_x ^ ((4 * (k & 1)) << 4)) + kRopeOff + (t < last ? t : last) * kRowF, lr0);
                });
                const int t = s_row < last ? s_row : last;
                if (lane < kSclRows) dma16_at<slot * kSclB>(src, t * kRowF + kScaleOff, ls0);
            }
        } else {
            // gathered rows: each lane addresses its own row of the list
            const int last = (v > 0 ? v : 1) - 1;
            auto rowp = [&](int t) -> const uint8_t* {
                if (v <= 0) return kZeroRow;
                return p.kv + int64_t(sm.rows[j0 + (t < last ? t : last)]) * kRowF;
            };
            static_for<0, kCodeLoads>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const int t = 2 * (wv * kCodeLoads + k) + h;
                dma16_v_at<slot * kCodesB + k * 1024>(rowp(t) + (c_x ^ (u_bits(k) << 4)), lc0);
            });
            static_for<0, kRopeLoads>([&](auto kc) {
                constexpr int k = decltype(kc)::value;
                const int t = 8 * (wv * kRopeLoads + k) + rr;
                dma16_v_at<slot * kRopeSB + k * 1024>(rowp(t) + (r_x ^ ((4 * (k & 1)) << 4)) + kRopeOff, lr0);
            });
            if (lane < kSclRows) dma16_v_at<slot * kSclB>(rowp(s_row) + kScaleOff, ls0);
        }
    };
    // real rows of sub-tile j (0 for padding); its scores past that are masked
    auto sub_count = [&](int j) { return max(0, min(kSub, tok1 - tok0 - j * kSub)); };

    __builtin_amdgcn_s_waitcnt(0);  // query fragments, before the ring starts
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    if (n_pad > 0) {
        issue(0, S0{});
        issue(1, S1{});
    }

    f32x16 acc[kDvTiles];
#pragma unroll
    for (int i = 0; i < kDvTiles; ++i) acc[i] = f32x16{};
    float m = -INFINITY;  // reference max of this head, log2 domain
    float l = 0.f;        // sum of 2^(s - m)
    const float sl2 = p.scale * 1.4426950408889634f;
    bool bad_block = false;

    // per-lane operand addresses inside slot 0 (plus compile-time offsets)
    const MLA_LDS uint8_t* lds_codes = (const MLA_LDS uint8_t*)sm.codes;
    const MLA_LDS uint8_t* lds_rope = (const MLA_LDS uint8_t*)sm.rope;
    int kb[8];  // code pair s (chunk 2 s + half): kb[s & 7] + 256 (s >> 3)
#pragma unroll
    for (int u = 0; u < 8; ++u) kb[u] = col * kLatent + (((2 * u + half) ^ f8swz(col)) << 4);
    int kr[4];  // rope chunk 2 u + half
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = col * kRope * 2 + (((2 * u + half) ^ rope_swz(col)) << 4);
    int vb[2][4];  // V^T reads of tile mt = 4 g + q: vb[g & 1][q] + 256 (g >> 1) + 8 KB jj
    {
        const int g16 = lane >> 4, s16 = lane & 15;
        const int r = s16 >> 1, b = s16 & 1;
        const int t = 8 * (r >> 2) + 4 * (g16 >> 1) + (r & 3);
#pragma unroll
        for (int g1 = 0; g1 < 2; ++g1)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                vb[g1][q] = t * kLatent + (((8 * g1 + 2 * q + (g16 & 1)) ^ f8swz(t)) << 4) + 8 * b;
    }
    // scales of the 16 tokens this lane holds in S^T, tokens
    // (i >> 2) * 8 + 4 half + (i & 3), for group g of the sub-tile in `slot`
    auto load_scales = [&](int slot, int g, float (&sc)[16]) {
        const MLA_LDS float* rowp =
            (const MLA_LDS float*)((const MLA_LDS uint8_t*)&sm.sct[slot][g][0] + 16 * half);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 v = *(const MLA_LDS f32x4*)(rowp + 8 * q);
            sc[4 * q] = v[0]; sc[4 * q + 1] = v[1]; sc[4 * q + 2] = v[2]; sc[4 * q + 3] = v[3];
        }
    };

    auto iteration = [&](int j, auto slot_c) {
        constexpr int sc = decltype(slot_c)::value;  // slot of sub-tile j
        // own loads of sub-tile j are complete once at most one later
        // sub-tile (j+1) remains in flight; the barrier makes all waves'
        // loads visible and frees the slot of sub-tile j-1 for j+2
        if (j + 1 < n_pad) wait_vm<kLoads>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (j + 2 < n_pad) issue(j + 2, std::integral_constant<int, (sc + 2) % kRingF>{});
        const int cnt = bad_slot[sc] ? 0 : sub_count(j);
        bad_block |= bad_slot[sc];
        // group scales of sub-tile j, transposed to [group][token]
        {
            const f32x2 v = *(const MLA_LDS f32x2*)((const MLA_LDS uint8_t*)sm.scl[sc] +
                                                    (lane >> 1) * 16 + 8 * (lane & 1));
            MLA_LDS float* w = (MLA_LDS float*)&sm.sct[sc][0][0];
            w[(2 * (lane & 1)) * kSub + (lane >> 1)] = v[0];
            w[(2 * (lane & 1) + 1) * kSub + (lane >> 1)] = v[1];
        }

        // ---- scores ------------------------------------------------------------
        const MLA_LDS uint8_t* lc = lds_codes + sc * kCodesB;
        f32x16 st;
        {
            const MLA_LDS uint8_t* lr = lds_rope + sc * kRopeSB;
            bf16x8 k0 = *(const MLA_LDS bf16x8*)(lr + kr[0]);
            bf16x8 q0 = qread(0);
            bf16x8 k1 = *(const MLA_LDS bf16x8*)(lr + kr[1]);
            bf16x8 q1 = qread(1);
            mfma32_v_first(st, k0, q0);
            k0 = *(const MLA_LDS bf16x8*)(lr + kr[2]);
            q0 = qread(2);
            mfma32_v(st, k1, q1);
            k1 = *(const MLA_LDS bf16x8*)(lr + kr[3]);
            q1 = qread(3);
            mfma32_v(st, k0, q0);
            mfma32_v(st, k1, q1);
        }
        __builtin_amdgcn_sched_barrier(0);
        auto cread = [&](int s2) -> i32x4 {
            return *(const MLA_LDS i32x4*)(lc + kb[s2 & 7] + 256 * (s2 >> 3));
        };
        i32x4 cw[2];
        cw[0] = cread(0);
        f32x16 ag;
        static_for<0, 4>([&](auto gc) {
            constexpr int g = decltype(gc)::value;
            float scg[16];
            load_scales(sc, g, scg);
            static_for<0, 4>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                constexpr int s2 = 4 * g + u;  // code pair: steps 2 s2, 2 s2 + 1
                if (s2 + 1 < 16) cw[(s2 + 1) & 1] = cread(s2 + 1);
                const i32x4 w = cw[s2 & 1];
                const bf16x8 a0 = fp8x8_to_bf16(w[0], w[1]);
                const bf16x8 a1 = fp8x8_to_bf16(w[2], w[3]);
                if (u == 0) mfma32_v_first<true>(ag, a0, qf[2 * s2]);
                else mfma32_v<true>(ag, a0, qf[2 * s2]);
                mfma32_v<true>(ag, a1, qf[2 * s2 + 1]);
                __builtin_amdgcn_sched_barrier(0);
            });
            mfma_result_wait(ag);  // before the VALU reads the group product
#pragma unroll
            for (int i = 0; i < 16; ++i) st[i] = fmaf(scg[i], ag[i], st[i]);
            __builtin_amdgcn_sched_barrier(0);
        });

        // ---- online softmax (log2 domain, lagging reference max) ----------
        if (cnt < kSub) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tok = (i >> 2) * 8 + half * 4 + (i & 3);
                if (tok >= cnt) st[i] = -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(st[0], st[1]), st[2]);
#pragma unroll
        for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, st[i]), st[i + 1]);
        mx = fmaxf(mx, st[15]);
        mx = xhalf_max(mx) * sl2;
        // a head whose max grew by more than kLag moves its reference;
        // accumulators of heads that had one rescale
        const bool grow = mx > m + kLag;
        if (__any(grow && m != -INFINITY)) {
            const float alpha = grow ? exp2f(m - mx) : 1.f;
#pragma unroll
            for (int i = 0; i < kDvTiles; ++i) scale_acc(acc[i], alpha);
            l *= alpha;
        }
        if (grow) m = mx;
        const float nm = (m == -INFINITY) ? 0.f : -m;
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float e = __builtin_amdgcn_exp2f(fmaf(st[i], sl2, nm));
            st[i] = e;
            ps += e;
        }
        ps = xhalf_sum(ps);
        l += ps;

        // ---- O^T += sum_g C_g^T . (P (.) scale_g)^T ----------------------------
        static_for<0, 4>([&](auto gc) {
            constexpr int g = decltype(gc)::value;
            float scg[16];
            load_scales(sc, g, scg);
            bf16x8 pf[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[jj][e] = (__bf16)(st[8 * jj + e] * scg[8 * jj + e]);
            i32x2 vr[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    vr[q][jj] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (MLA_LDS i32x2*)(lc + vb[g & 1][q] + 256 * (g >> 1) + 8192 * jj));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int mt = 4 * g + q;
                mfma32_acc<true>(acc[mt], fp8x8_to_bf16(vr[q][0][0], vr[q][0][1]), pf[0]);
                mfma32_acc<true>(acc[mt], fp8x8_to_bf16(vr[q][1][0], vr[q][1][1]), pf[1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    for (int j = 0; j < n_pad; j += kRingF) {
        iteration(j, S0{});
        iteration(j + 1, S1{});
        iteration(j + 2, S2{});
    }
    mfma_drain();
    if (bad_block && threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);

    // ---- finalise: O = acc / l, LSE = ln 2 * (m + log2 l) --------------------
    const bool empty = l == 0.f;  // NaN stays visible
    const float inv = empty ? 0.f : 1.f / l;
    const float lse = empty ? -INFINITY : (m + log2f(l)) * 0.6931471805599453f;
    // whole row: the shard's output; a chunk of a split row: its partial slot
    const bool direct = id.slot < 0;
    const size_t orow = direct ? size_t(id.row) * p.H + head : size_t(id.slot) * p.H + head;
    if (p.out_dtype == MLA_BF16) {
        // staged through the ring's LDS once every wave is past its last read
        constexpr int kPasses = NW == 2 ? 1 : 2;
        constexpr int kWaveB = 32 * 1024 / kPasses;
        static_assert(sizeof(sm) >= NW * kWaveB, "staging fits the LDS of the ring");
        __syncthreads();
        store_rows_bf16<kPasses>(acc, inv, (MLA_LDS uint8_t*)&sm + wave * kWaveB,
                                    static_cast<uint16_t*>(direct ? p.o_out : p.ws_o) +
                                        (orow - col) * kLatent,
                                    lane);
    } else {
        float* o = static_cast<float*>(direct ? p.o_out : p.ws_o) + orow * kLatent;
#pragma unroll
        for (int mt = 0; mt < kDvTiles; ++mt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * mt + 8 * q4 + 4 * half;
                *reinterpret_cast<float4*>(o + d) =
                    make_float4(acc[mt][4 * q4] * inv, acc[mt][4 * q4 + 1] * inv,
                                acc[mt][4 * q4 + 2] * inv, acc[mt][4 * q4 + 3] * inv);
            }
    }
    if (half == 0) (direct ? p.lse_out : p.ws_lse)[orow] = lse;
}

}  // namespace mfma
}  // namespace mla
