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
    int32_t rows[SPARSE ? kMaxTopk + 1 : 1];  // sparse: pool rows this shard owns, entry order; a spare slot
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
    // part through LDS.  A dense row requests them first; a sparse row right
    // after its index and block-table loads, so that the compaction waits
    // for those alone while the query is still in flight.
    bf16x8 qf[kQLatSteps];
    bf16x8 qrope_r[4];
    const int qr_off = head * (kRope * 2);
    const int qr_sw = (head >> 1) & 7;
    auto load_query = [&] {
        const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
            static_cast<const uint16_t*>(p.q) + (size_t(id.qi) * p.H + head) * kDk);
#pragma unroll
        for (int ks = 0; ks < kQLatSteps; ++ks) qf[ks] = qrow[4 * (ks >> 1) + 2 * half + (ks & 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) qrope_r[u] = qrow[2 * (kQLatSteps + u) + half];
    };
    if constexpr (!SPARSE) load_query();

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
        __builtin_amdgcn_sched_barrier(0);
        load_query();
        __builtin_amdgcn_sched_barrier(0);
        if (bt_lds) {
            // a use of the last index makes the compiler wait for the index
            // loads, and so for this wave's table loads issued before them,
            // but not for the query loads issued after
#pragma unroll
            for (int k = 0; k < kSteps; ++k) asm volatile("" ::"v"(gv[k]));
            __syncthreads();
        }
        // Branch free: every entry looks up a table entry (a clamped index
        // when it is not owned or past the table), all lookups are issued
        // before any is used, and each error bit is raised once per wave.
        // row: pool row of an owned entry, -1 not owned (or padding, or past
        // the visible prefix: MLA_DEVERR_INDEX), -2 owned with a bad or
        // missing table entry (MLA_DEVERR_BLOCK_TABLE).
        const double inv_n = 1.0 / double(p.n_shards);
        int32_t row[kSteps], jl[kSteps];
        bool bad_index = false, bad_table = false;
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            const int32_t g = gv[k];
            const int32_t gc = g < 0 ? 0 : g;
            const int32_t j = div_by(gc, inv_n);  // local index if owned
            bad_index |= g >= visible;
            const bool owned = g >= 0 && g < visible && gc - j * p.n_shards == s;
            jl[k] = owned ? j : -1;
            const int32_t jb = j / kBlock;
            row[k] = jb < p.max_blocks ? jb : 0;  // table index for now
        }
        if (bt_lds) {
#pragma unroll
            for (int k = 0; k < kSteps; ++k) row[k] = bt_l[row[k]];  // block id for now
        } else {
#pragma unroll
            for (int k = 0; k < kSteps; ++k) row[k] = bt[row[k]];
        }
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            const int32_t j = jl[k], b = row[k];
            const bool ok = j / kBlock < p.max_blocks && b >= 0 && b < p.pool_blocks;
            row[k] = j < 0 ? -1 : ok ? b * kBlock + (j % kBlock) : -2;
            bad_table |= row[k] == -2;
        }
        if (lane == 0 && __ballot(bad_index)) raise_error(p.err, MLA_DEVERR_INDEX);
        if (lane == 0 && __ballot(bad_table)) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            // entries not kept write the spare slot (no branch per entry)
            const uint64_t mask = __ballot(row[k] >= 0);
            sm.rows[row[k] >= 0 ? e_begin + cnt + __popcll(mask & below) : kMaxTopk] = row[k];
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
        // read first, then all write.  Branch free: every read stays inside
        // the list (e_begin + i < kMaxTopk, since slice <= kMaxTopk / NW),
        // and lanes past the count write the spare slot.
        constexpr int kPerLane = kMaxTopk / (NW * 64);
        int32_t mine[kPerLane];
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) mine[k] = sm.rows[e_begin + k * 64 + lane];
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kPerLane; ++k) {
            const int i = k * 64 + lane;
            sm.rows[i < cnt ? base + i : kMaxTopk] = mine[k];
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
    const int rr = lane >> 3;
    const int r_x0 = (((lane & 7) ^ (rr >> 1)) ^ (4 * ((wave * kRopeLoads) & 1))) << 4;
    const int s_row0 = wave * kSclRows + lane;  // scale load (lanes < kSclRows)
    const uint32_t lc0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.codes) + wv * kCodeLoads * 1024);
    const uint32_t lr0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.rope) + wv * kRopeLoads * 1024);
    const uint32_t ls0 = __builtin_amdgcn_readfirstlane(lds_addr(sm.scl) + wv * kSclRows * 16);

    bool bad_slot[kRingF] = {false, false, false};
    // Source of sub-tile j.  Dense: first row in HBM (the zero row for a
    // padding or bad sub-tile); sparse: the list entries from j0.  Rows past
    // `last` re-read row `last`.
    struct SrcF {
        const uint8_t* src;
        int32_t j0;
        int last;
        int v;  // real rows (<= 0: padding)
    };
    // block id of dense sub-tile j.  The main loop reads it one iteration
    // ahead, at a point where no LDS read is in flight, so that waiting for it
    // waits for nothing else.  A padding sub-tile reads the entry of the
    // chunk's last row (in the table; its value is unused).
    const uint32_t last_tok = uint32_t(max(tok1 - 1, 0));
    auto block_of = [&](int j) -> int32_t {
        if constexpr (SPARSE) return -1;
        const uint32_t j0 = uint32_t(tok0 + j * kSub);
        return btc[min(j0, last_tok) / kBlock];
    };
    // Dense: branch free, the source a select between the block's row and the
    // zero row and the validity test one unsigned compare (a negative id wraps
    // past every pool size an int32 id can name).
    const uint32_t pool32 =
        p.pool_blocks > int64_t(0x80000000) ? 0x80000000u : uint32_t(p.pool_blocks);
    auto prep = [&](int j, int32_t blk, auto slot_c) -> SrcF {
        constexpr int slot = decltype(slot_c)::value;
        const int32_t j0 = tok0 + j * kSub;
        const int v = min(kSub, tok1 - j0);  // <= 0: padding
        if constexpr (SPARSE) {
            return SrcF{v > 0 ? p.kv : kZeroRow, j0, (v > 0 ? v : 1) - 1, v};
        } else {
            const bool bad = v > 0 && uint32_t(blk) >= pool32;
            const bool use = v > 0 && !bad;
            const uint64_t mask = 0ull - uint64_t(use);  // all ones when the row is read
            const uint64_t row = reinterpret_cast<uint64_t>(p.kv) +
                                 (uint64_t(uint32_t(blk) & uint32_t(mask)) * kBlock + (uint32_t(j0) % kBlock)) * kRowF;
            const uint64_t src = (row & mask) | (reinterpret_cast<uint64_t>(kZeroRow) & ~mask);
            bad_slot[slot] = bad;
            return SrcF{reinterpret_cast<const uint8_t*>(src), j0, max(v - 1, 0) & int(uint32_t(mask)), v};
        }
    };
    int32_t grow[SPARSE ? kLoads : 1];  // sparse: pool rows of the next sub-tile's loads
    // Load kk of this wave for the sub-tile of r in `slot`: kk < kCodeLoads a
    // code load, then kRopeLoads rope loads, then the scale load.
    auto load_one = [&](const SrcF& r, auto slot_c, auto kk_c) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int kk = decltype(kk_c)::value;
        // an opaque copy of the one base this load uses: its offset is then
        // computed here, not hoisted out of the loop into a dozen live
        // registers.  Row offsets are 24-bit products (t < 32, 656-byte rows).
        auto opaque = [](int x) {
            asm volatile("" : "+v"(x));
            return x;
        };
        if constexpr (!SPARSE) {
            // branch free: rows past r.last re-read row r.last (one v_min per
            // load; a whole sub-tile has r.last = 31 and clamps nothing)
            if constexpr (kk < kCodeLoads) {
                constexpr int k = kk;
                const int t = 2 * (wv * kCodeLoads + k) + h;
                dma16_at<slot * kCodesB + k * 1024>(
                    r.src, (opaque(c_x0) ^ (u_bits(k) << 4)) + int(__umul24(min(t, r.last), kRowF)), lc0);
            } else if constexpr (kk < kCodeLoads + kRopeLoads) {
                constexpr int k = kk - kCodeLoads;
                const int t = 8 * (wv * kRopeLoads + k) + rr;
                dma16_at<slot * kRopeSB + k * 1024>(
                    r.src, (opaque(r_x0) ^ ((4 * (k & 1)) << 4)) + kRopeOff + int(__umul24(min(t, r.last), kRowF)),
                    lr0);
            } else {
                if (lane < kSclRows)
                    dma16_at<slot * kSclB>(r.src, int(__umul24(min(opaque(s_row0), r.last), kRowF)) + kScaleOff,
                                           ls0);
            }
        } else {
            // gathered rows: each lane addresses its own row of the list,
            // whose pool row was read from LDS ahead of time (grow[kk], 0
            // when the sub-tile is padding, with r.src the zero row)
            const uint8_t* rowp = r.src + int64_t(grow[kk]) * kRowF;
            if constexpr (kk < kCodeLoads) {
                constexpr int k = kk;
                dma16_v_at<slot * kCodesB + k * 1024>(rowp + (opaque(c_x0) ^ (u_bits(k) << 4)), lc0);
            } else if constexpr (kk < kCodeLoads + kRopeLoads) {
                constexpr int k = kk - kCodeLoads;
                dma16_v_at<slot * kRopeSB + k * 1024>(rowp + (opaque(r_x0) ^ ((4 * (k & 1)) << 4)) + kRopeOff, lr0);
            } else {
                if (lane < kSclRows) dma16_v_at<slot * kSclB>(rowp + kScaleOff, ls0);
            }
        }
    };
    // Sparse: the pool row behind each of this lane's loads of sub-tile r
    // (the list entry of its token, rows past r.last re-reading r.last), read
    // from LDS in one batch well before the loads are issued, so that no load
    // waits for an LDS read (a wait that would also drain the operand reads
    // in flight).  Padding sub-tiles read entry 0 and use the zero row.
    auto gather_rows = [&](const SrcF& r) {
        if constexpr (SPARSE) {
            const int vmask = r.v > 0 ? -1 : 0;
            static_for<0, kLoads>([&](auto kc) {
                constexpr int kk = decltype(kc)::value;
                int t;
                if constexpr (kk < kCodeLoads) t = 2 * (wv * kCodeLoads + kk) + h;
                else if constexpr (kk < kCodeLoads + kRopeLoads) t = 8 * (wv * kRopeLoads + kk - kCodeLoads) + rr;
                else t = min(s_row0, kSub - 1);
                const int e = (r.j0 + min(t, r.last)) & vmask;
                grow[kk] = sm.rows[e] & vmask;
            });
        }
    };
    // all loads of sub-tile j at once (the two sub-tiles before the loop)
    auto issue = [&](int j, auto slot_c) {
        const SrcF r = prep(j, block_of(j), slot_c);
        gather_rows(r);
        static_for<0, kLoads>([&](auto kc) { load_one(r, slot_c, kc); });
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
    int32_t blk_ahead = block_of(2);  // block id of the next dense sub-tile to load

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
    // Per-lane LDS byte offsets of the operand reads.  The swizzled chunk
    // index sits in bits 4-7 (bits 4-6 for rope) above a row base whose low
    // bits are zero, so every read of a lane is its first read's offset
    // XORed with a constant: code pair s at kb0 ^ 32 (s & 7), plus 256 (s >> 3);
    // rope chunk 2 u + half at kr0 ^ 32 u; V^T tile 4 g + q at
    // vb0 ^ (128 (g & 1) + 32 q), plus 256 (g >> 1) and 8 KB per token half.
    // One base register each instead of a table of 20.
    int kb0 = col * kLatent + ((half ^ f8swz(col)) << 4);
    int kr0 = col * kRope * 2 + ((half ^ rope_swz(col)) << 4);
    int vb0;
    {
        const int g16 = lane >> 4, s16 = lane & 15;
        const int r = s16 >> 1, b = s16 & 1;
        const int t = 8 * (r >> 2) + 4 * (g16 >> 1) + (r & 3);
        vb0 = t * kLatent + (((g16 & 1) ^ f8swz(t)) << 4) + 8 * b;
    }
    auto iteration = [&](int j, auto slot_c) {
        constexpr int sc = decltype(slot_c)::value;  // slot of sub-tile j
        // opaque per iteration: the XORed offsets are formed next to their
        // reads instead of being hoisted into live registers
        asm volatile("" : "+v"(kb0), "+v"(kr0), "+v"(vb0));
        // own loads of sub-tile j are complete once at most one later
        // sub-tile (j+1) remains in flight; the barrier makes all waves'
        // loads visible and frees the slot of sub-tile j-1 for j+2
        if (j + 1 < n_pad) wait_vm<kLoads>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        // Sub-tile j+2 goes to the slot sub-tile j-1 used.  Its loads are dealt
        // over the output product below: issued together, the workgroup's
        // wave-wide loads queue behind each other at the address unit and
        // stall in-order issue.
        // A dense step issues them past the last sub-tile too, reading the
        // zero row into that free slot (no sub-tile reads it again), so the
        // issue path has no branch.
        using SL = std::integral_constant<int, (sc + 2) % kRingF>;
        // (sparse: past the last sub-tile the loads read the zero row into
        // the free slot, as dense ones do)
        const SrcF ld = (!SPARSE || j + 2 < n_pad) ? prep(j + 2, blk_ahead, SL{}) : SrcF{kZeroRow, 0, 0, 0};
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
        // A flat schedule of 36 MFMAs: 4 rope steps into st, then 32 latent
        // steps L (group g = L / 8, code pair L / 2) into the group
        // accumulator ag[g & 1].  Around each MFMA go, after it in program
        // order so that they execute under it: the widening of the next
        // step's codes (4 converts), the code read of the pair two ahead,
        // and, during group g, the 16 scale FMAs of group g - 1 (the two
        // accumulators alternate, so the matrix core never waits for them).
        // A group's scales are read from LDS seven steps before their FMAs:
        // a read consumed one step after issue stalls in-order issue for
        // the LDS latency.
        const MLA_LDS uint8_t* lc = lds_codes + sc * kCodesB;
        const MLA_LDS uint8_t* lr = lds_rope + sc * kRopeSB;
        auto cread = [&](int p2) -> i32x4 {
            return *(const MLA_LDS i32x4*)(lc + (kb0 ^ ((p2 & 7) << 5)) + 256 * (p2 >> 3));
        };
        auto sread = [&](int g, int c) -> f32x4 {  // scales of group g, tokens of st[4c .. 4c + 3]
            return *(const MLA_LDS f32x4*)((const MLA_LDS uint8_t*)&sm.sct[sc][g][0] + 16 * half + 32 * c);
        };
        bf16x8 kro[4], qro[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            kro[u] = *(const MLA_LDS bf16x8*)(lr + (kr0 ^ (u << 5)));
            qro[u] = qread(u);
        }
        i32x4 cw[3];
        cw[0] = cread(0);
        cw[1] = cread(1);
        bf16x8 ka[2];   // widened operand of latent step L in ka[L & 1]
        f32x16 st, ag[2];
        f32x4 scr[4];   // scales of one group, chunk c for st[4c .. 4c + 3]
        auto widen = [&](int L) -> bf16x8 {
            const i32x4& w = cw[(L >> 1) % 3];
            return (L & 1) ? fp8x8_to_bf16(w[2], w[3]) : fp8x8_to_bf16(w[0], w[1]);
        };
        static_for<0, 4 + 32>([&](auto sc_) {
            constexpr int s = decltype(sc_)::value;
            if constexpr (s < 4) {
                if (s == 0) mfma32_v_first(st, kro[0], qro[0]);
                else mfma32_v(st, kro[s], qro[s]);
                if constexpr (s == 3) ka[0] = widen(0);
            } else {
                constexpr int L = s - 4, g = L >> 3, e = L & 7;
                // ka was just written by VALU converts: FRESH leads with the
                // two wait states an MFMA operand read needs after them
                if (e == 0) mfma32_v_first<true>(ag[g & 1], ka[L & 1], qf[L]);
                else mfma32_v<true>(ag[g & 1], ka[L & 1], qf[L]);
                // code pair L / 2 + 2, read two pairs ahead of its first use
                if constexpr ((L & 1) == 0 && (L >> 1) + 2 < 16) cw[((L >> 1) + 2) % 3] = cread((L >> 1) + 2);
                if constexpr (L + 1 < 32) ka[(L + 1) & 1] = widen(L + 1);
                // scale FMAs of the previous group, chunk c at e = c + 3; then
                // chunk c of this group's scales replaces the consumed one
                if constexpr (g >= 1 && e >= 3 && e < 7) {
                    constexpr int c = e - 3;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        st[4 * c + k] = fmaf(scr[c][k], ag[(g - 1) & 1][4 * c + k], st[4 * c + k]);
                }
                if constexpr (e >= 4) scr[e - 4] = sread(g, e - 4);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        {
            // the last group's scale FMAs, after its product has landed;
            // then the first output group's scales, read under the softmax
            mfma_result_wait(ag[1]);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int k = 0; k < 4; ++k) st[4 * c + k] = fmaf(scr[c][k], ag[1][4 * c + k], st[4 * c + k]);
#pragma unroll
            for (int c = 0; c < 4; ++c) scr[c] = sread(0, c);
        }
        // sparse: pool rows of sub-tile j+2's loads, read under the softmax
        gather_rows(ld);
        __builtin_amdgcn_sched_barrier(0);

        // ---- online softmax (log2 domain, lagging reference max) ----------
        if (__builtin_expect(cnt < kSub, 0)) {
            // st[i] holds token (i >> 2) * 8 + 4 half + (i & 3): compared as
            // a constant against cnt - 4 half, formed here (hoisted per-lane
            // token numbers would be spilled out of the full register file)
            int lim = cnt - 4 * half;
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((i >> 2) * 8 + (i & 3) >= lim) st[i] = -INFINITY;
        }
        float mt3[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) mt3[k] = fmaxf(fmaxf(st[3 * k], st[3 * k + 1]), st[3 * k + 2]);
        float mx = fmaxf(fmaxf(fmaxf(mt3[0], mt3[1]), mt3[2]), fmaxf(fmaxf(mt3[3], mt3[4]), st[15]));
        mx = xhalf_max(mx) * sl2;
        // a head whose max grew by more than kLag moves its reference;
        // accumulators of heads that had one rescale
        const bool grow = mx > m + kLag;
        if (__builtin_expect(__any(grow && m != -INFINITY), 0)) {
            const float alpha = grow ? exp2f(m - mx) : 1.f;
#pragma unroll
            for (int i = 0; i < kDvTiles; ++i) scale_acc(acc[i], alpha);
            l *= alpha;
        }
        if (grow) m = mx;
        const float nm = (m == -INFINITY) ? 0.f : -m;
        float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            st[i] = __builtin_amdgcn_exp2f(fmaf(st[i], sl2, nm));
            st[i + 1] = __builtin_amdgcn_exp2f(fmaf(st[i + 1], sl2, nm));
            ps0 += st[i];
            ps1 += st[i + 1];
        }
        l += xhalf_sum(ps0 + ps1);

        // ---- O^T += sum_g C_g^T . (P (.) scale_g)^T ----------------------------
        // A flat schedule of 32 MFMAs u (group g = u / 8, tile 4 g + q with
        // q = u / 2 % 4, token half u % 2).  Around each MFMA: the widening
        // of the next one's V^T codes, the transposing read three ahead, the
        // scaled probabilities of the next group, and (one in three) a load of
        // sub-tile j+2.
        auto vread8 = [&](int u) -> i32x2 {
            const int g = u >> 3, q = (u >> 1) & 3, jj = u & 1;
            return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (MLA_LDS i32x2*)(lc + (vb0 ^ ((8 * (g & 1) + 2 * q) << 4)) + 256 * (g >> 1) + 8192 * jj));
        };
        i32x2 vr[4];
        bf16x8 va[2];     // widened V^T operand of MFMA u in va[u & 1]
        bf16x8 pf[2][2];  // P (.) scale_g of group g in pf[g & 1][token half]
        auto pscale = [&](int g, int c, const f32x4& sv) {
#pragma unroll
            for (int k = 0; k < 4; ++k) pf[g & 1][c >> 1][4 * (c & 1) + k] = (__bf16)(st[4 * c + k] * sv[k]);
        };
#pragma unroll
        for (int u = 0; u < 3; ++u) vr[u] = vread8(u);
#pragma unroll
        for (int c = 0; c < 4; ++c) pscale(0, c, scr[c]);
        va[0] = fp8x8_to_bf16(vr[0][0], vr[0][1]);
        static_for<0, 32>([&](auto uc) {
            constexpr int u = decltype(uc)::value, g = u >> 3, e = u & 7;
            // va (and, for u = 0, pf) were written by VALU converts just before
            mfma32_acc<true>(acc[4 * g + ((u >> 1) & 3)], va[u & 1], pf[g & 1][u & 1]);
            if constexpr (u + 3 < 32) vr[(u + 3) & 3] = vread8(u + 3);
            if constexpr (u + 1 < 32) va[(u + 1) & 1] = fp8x8_to_bf16(vr[(u + 1) & 3][0], vr[(u + 1) & 3][1]);
            // the next group's scaled probabilities: chunk c at e = c + 4,
            // its scales read at e = c
            if constexpr (g < 3 && e < 4) scr[e] = sread(g + 1, e);
            if constexpr (g < 3 && e >= 4) pscale(g + 1, e - 4, scr[e - 4]);
            if constexpr (u % 3 == 1 && u / 3 < kLoads) {
                load_one(ld, SL{}, std::integral_constant<int, u / 3>{});
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        // every LDS read of this iteration has been consumed: the block id of
        // the sub-tile the next iteration loads is requested now
        blk_ahead = block_of(j + 3);
        __builtin_amdgcn_sched_barrier(0);
    };
    for (int j = 0; j < n_pad; j += kRingF) {
        iteration(j, S0{});
        iteration(j + 1, S1{});
        iteration(j + 2, S2{});
    }
    mfma_drain();
    wait_vm<0>();  // the zero-row loads of the last iterations land before the staging below
    if (bad_block && threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);

    // ---- finalise: O = acc / l, LSE = ln 2 * (m + log2 l) --------------------
    const bool empty = l == 0.f;  // NaN stays visible
    const float inv = empty ? 0.f : 1.f / l;
    const float lse = empty ? -INFINITY : (m + log2f(l)) * 0.6931471805599453f;
    // whole row: the shard's output; a chunk of a split row: its partial slot
    const bool direct = id.slot < 0;
    const size_t orow = direct ? size_t(id.row) * p.H + head : size_t(id.slot) * p.H + head;
    // chunk partials stay float32 whatever the output dtype
    if (direct && p.out_dtype == MLA_BF16) {
        // staged through the ring's LDS once every wave is past its last read
        constexpr int kPasses = NW == 2 ? 1 : 2;
        constexpr int kWaveB = 32 * 1024 / kPasses;
        static_assert(sizeof(sm) >= NW * kWaveB, "staging fits the LDS of the ring");
        __syncthreads();
        store_rows_bf16<kPasses>(acc, inv, (MLA_LDS uint8_t*)&sm + wave * kWaveB,
                                    static_cast<uint16_t*>(p.o_out) +
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
