// Matrix-core partial decode for a bf16 latent cache (gfx950).
//
// One workgroup of four waves handles one (shard, request, query token,
// chunk) row and all its query heads.  The shard's local tokens stream
// through a ring of four 32-token sub-tiles in LDS, filled by direct
// global->LDS loads (global_load_lds_dwordx4) three sub-tiles ahead.  The
// four waves split the heads into groups of 32 and, when there are fewer
// than four groups, the 512 output dimensions into DS = 128 / H' parts
// (H' = H padded to a multiple of 32): wave w owns head group w % (4 / DS)
// and output tiles [16 d / DS, 16 (d + 1) / DS) with d = w / (4 / DS).  The
// waves of one head group all form its scores (the work the split repeats);
// the loads, the ring and its layout are the same for every head count.
// Per sub-tile and wave:
//
//   S^T[32 tok x 32 heads] = K[32 x 576] . Q^T[576 x 32]        36 MFMA 32x32x16
//   online softmax per head: the scores of one head sit in one lane (and its
//   partner lane l^32), so the running max / sum need one cross-lane step
//   O^T[512/DS x 32 heads] += V^T[512/DS x 32 tok] . P^T[32 tok x 32 heads]
//                                                         32/DS MFMA 32x32x16
//
// The loop is software pipelined: iteration j issues the score product of
// sub-tile j+1 together with the softmax of sub-tile j, then the output
// product of sub-tile j interleaved with the rest of the score product, so
// the matrix cores keep running while the VALU works and the LDS reads are
// spread over the iteration.
//
// Q^T stays in registers for the whole row (the rope part in LDS).  K rows
// are read from LDS as the A operand (16 B per lane); V^T is read with
// ds_read_b64_tr_b16, which transposes 4 x 4 16-bit blocks across a 16-lane
// group, so each lane gets four consecutive tokens of one latent dimension.
//
// Scores use exact bf16 products with float32 accumulation; probabilities
// are rounded to bf16 for the PV product; the normaliser and LSE are float32.
#pragma once

#include "common.hpp"
#include "mfma_common.hpp"
#include "params.hpp"
#include "sparse_list.hpp"

namespace mla {
namespace mfma {

constexpr int kRing = 4;                 // sub-tiles resident in LDS
constexpr int kAhead = kRing - 1;        // sub-tiles in flight ahead of compute
constexpr int kRowB = kDk * 2;           // 1152 B per bf16 row in the cache
constexpr int kLatB = kLatent * 2;       // 1024 B latent part of a row
constexpr int kRopeB = kRope * 2;        // 128 B rope part of a row
constexpr int kQSteps = kDk / 16;        // 36 K-steps of the score product
constexpr int kLoadsPerWave = kSub / 4 + 1;  // 8 latent rows + 1 rope load per wave

// LDS layout of the ring.  Latent parts of rows, 1 KB each, sit at
//   lat_row(s, t) = (((t % 16) * 4 + s) * 2 + t / 16) * 1024
// for slot s and token t of the sub-tile, so the slot, the token half
// (t / 16) and the 256-byte dimension group of any read differ by a
// compile-time offset that fits the LDS instruction's immediate; rope parts
// (128 B) sit after them at rope_row(s, t).  The 16-byte chunks of a latent
// row are XOR-swizzled within their 256-byte group by
// f(t) = ((t & 3) << 2) | ((t >> 2) & 3), rope chunks by (t >> 1) & 7.  With
// 64 four-byte banks, the 16-lane passes of the K reads (16 rows, one chunk
// each) and the 32-lane passes of the V^T transposing reads (4 rows x 4
// chunks x 2 halves) then hit every bank once.
constexpr int kLatRegion = 16 * kRing * 2 * kLatB;  // 128 KB
constexpr int kRopeRegion = kRing * kSub * kRopeB;  // 16 KB
constexpr int kQRopeB = 128 * kRopeB;               // rope part of Q for 128 heads
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int rswz(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ constexpr int lat_row(int s, int t) {
    return (((t & 15) * kRing + s) * 2 + (t >> 4)) * kLatB;
}
__device__ __forceinline__ constexpr int rope_row(int s, int t) {
    return kLatRegion + (s * kSub + t) * kRopeB;
}

struct alignas(16) SmemBf16 {
    uint8_t ring[kLatRegion + kRopeRegion];
    uint8_t qrope[kQRopeB];  // [head][8 chunks of 16 B], chunk c at c ^ ((head >> 1) & 7)
};

// SPARSE: a top-K step.  The row's tokens are the pool rows a list pass
// (sparse_list.hpp) wrote for it, in entry order, and each wave gathers rows
// 8w .. 8w + 7 of a sub-tile: one direct load per row for the latent parts
// (its row address read from the list through the scalar cache), and one
// load for their rope parts with a per-lane address.  Everything after the
// loads is the dense path's.
template <int DS, bool SPARSE = false>
__global__ void __launch_bounds__(256, 1) decode_mfma_bf16_kernel(DecodeParams p) {
    static_assert(DS == 1 || DS == 2 || DS == 4, "output dimension splits");
    constexpr int kHG = 4 / DS;             // head groups of 32
    constexpr int kDvT = kDvTiles / DS;     // 32-dim output tiles per wave
    __shared__ SmemBf16 sm;
    RowId id;
    if (!work_item(p, blockIdx.x, id)) return;  // past the last planned item
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;  // head within the group (S^T, O^T columns)
    const int dsp = DS == 1 ? 0 : wave / kHG;  // output dimension part of this wave
    const int head = DS == 1 ? wave * 32 + col : (wave % kHG) * 32 + col;
    const bool head_ok = DS < 4 || head < p.H;  // 16 heads: the group's upper half is padding
    const int s = p.shard_begin + id.s_rel;
    const int32_t* bt = p.block_tables + (size_t(id.s_rel) * p.B + id.b) * p.max_blocks;

    // ---- token range of this chunk (sparse: of the row's list) ------------
    int32_t tok0 = 0, tok1 = 0;
    if constexpr (!SPARSE) {
        const int32_t L = p.context_lens[id.b];
        int32_t visible = L - id.qlen + id.t + 1;
        if (visible < 0) visible = 0;
        int32_t local = dev_local_len(visible, s, p.n_shards);
        if ((local + kBlock - 1) / kBlock > p.max_blocks) {
            if (threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
            local = p.max_blocks * kBlock;
        }
        tok0 = id.chunk * id.chunk_tok;
        tok1 = id.chunk_tok ? tok0 + id.chunk_tok : local;
        if (tok1 > local) tok1 = local;
    } else {
        tok1 = ((const __attribute__((address_space(4))) int32_t*)p.sp_count)[id.row];
    }
    const int n_sub = tok1 > tok0 ? (tok1 - tok0 + kSub - 1) / kSub : 0;
    // the pipelined loop below is unrolled by the ring size and always runs
    // whole rounds: padding sub-tiles are zero rows with every score masked
    const int n_pad = (n_sub + kRing - 1) / kRing * kRing;

    // ---- Q^T fragments: head `head`, dims 16 ks + 8 half .. + 8 ------------
    // latent part in registers, rope part in LDS, written by the group's
    // first wave (the barrier before the first score product orders it
    // before the other waves' reads); padding heads are zero
    bf16x8 qf[kQLatSteps];
    const int qr_off = head * kRopeB;
    const int qr_sw = (head >> 1) & 7;
    {
        const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
            static_cast<const uint16_t*>(p.q) + (size_t(id.qi) * p.H + (head_ok ? head : 0)) * kDk);
#pragma unroll
        for (int ks = 0; ks < kQLatSteps; ++ks) qf[ks] = head_ok ? qrow[2 * ks + half] : bf16x8{};
        if (DS == 1 || dsp == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = 2 * u + half;
                *(MLA_LDS bf16x8*)((MLA_LDS uint8_t*)sm.qrope + qr_off + ((c ^ qr_sw) << 4)) =
                    head_ok ? qrow[2 * (kQLatSteps + u) + half] : bf16x8{};
            }
        }
    }

    // ---- sub-tile loads ----------------------------------------------------
    // Wave w loads the latent parts of rows 4k + w (k = 0..7), one row per
    // wave-wide load (lane i fetches the chunk stored at position i), and the
    // rope parts of rows 8w .. 8w + 7 in one load.  Per-lane offsets are
    // computed once; rows at or past a partial sub-tile's valid count re-read
    // its last valid row, and a bad or padding sub-tile reads the zero row.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int dv[kSub / 4];  // latent loads of a full sub-tile
#pragma unroll
    for (int k = 0; k < kSub / 4; ++k) {
        if constexpr (!SPARSE) {
            const int t = 4 * k + wave;
            dv[k] = t * kRowB + ((((lane & 48) | ((lane & 15) ^ swz(t)))) << 4);
        } else {
            // sparse: load k of wave w is row 8w + k, from its own row address
            const int t = 8 * wave + k;
            dv[k] = (((lane & 48) | ((lane & 15) ^ swz(t)))) << 4;
        }
    }
    const int r_row = 8 * wave + (lane >> 3);  // rope load: row and chunk of this lane
    const int r_off = (kLatent / 8 + ((lane & 7) ^ rswz(r_row))) << 4;
    // LDS destinations: lat_row(slot, 4k + w) = w * 8 KB + (k & 3) * 32 KB +
    // (k >> 2) * 1 KB + slot * 2 KB; rope_row(slot, 8w) = rope base + slot * 4 KB + w * 1 KB
    const uint32_t lds0 = lds_addr(sm.ring);
    // sparse: lat_row(slot, 8w + k) = (w & 1) * 64 KB + k * 8 KB + slot * 2 KB + (w >> 1) * 1 KB
    const uint32_t m_lat = __builtin_amdgcn_readfirstlane(
        SPARSE ? lds0 + (wv & 1) * (16 * 4 * kLatB) + (wv >> 1) * kLatB : lds0 + wv * (4 * 2 * kLatB));
    const uint32_t m_rope = __builtin_amdgcn_readfirstlane(lds0 + kLatRegion + wv * 8 * kRopeB);

    // Block ids are read through the scalar cache (the table is read-only
    // here): a vector load would need a vmcnt wait that drains the ring.
    const __attribute__((address_space(4))) int32_t* btc =
        (const __attribute__((address_space(4))) int32_t*)bt;
    bool bad_slot[kRing] = {false, false, false, false};  // sub-tile in the slot had a bad block id
    // Source of sub-tile j: first row in HBM, and the last row to read (rows
    // past it re-read it).
    struct Src {
        const uint8_t* src;
        int last;
    };
    // block id of sub-tile j.  The main loop reads it one iteration before its
    // loads are issued: waiting for a scalar load right before them would
    // stall every wave at the top of each iteration.  A padding sub-tile reads
    // the entry of the chunk's last row (in the table; its value is unused).
    const uint32_t last_tok = uint32_t(max(tok1 - 1, 0));
    auto block_of = [&](int j) -> int32_t {
        const uint32_t j0 = uint32_t(tok0) + uint32_t(j) * kSub;
        return btc[min(j0, last_tok) / kBlock];
    };
    // Branch free: the source is a select between the block's row and the
    // zero row, and the validity test one unsigned compare (a negative id
    // wraps past every pool size an int32 id can name).  On the top-of-
    // iteration path, a chain of branches and a 64-bit vector compare here
    // held back the first K reads.
    const uint32_t pool32 =
        p.pool_blocks > int64_t(0x80000000) ? 0x80000000u : uint32_t(p.pool_blocks);
    // In three stages (validity, row address, select) so that the main loop
    // can deal the scalar chain out over several MFMA slots.
    struct SrcA {
        uint32_t j0;
        int v;
        uint64_t mask;  // all ones when the row is read
    };
    auto source_a = [&](int j, int32_t blk, auto slot_c) -> SrcA {
        constexpr int slot = decltype(slot_c)::value;
        const uint32_t j0 = uint32_t(tok0) + uint32_t(j) * kSub;
        const int v = tok1 - int(j0);  // rows left in the chunk (<= 0: padding)
        const bool bad = v > 0 && uint32_t(blk) >= pool32;
        bad_slot[slot] = bad;
        return SrcA{j0, v, 0ull - uint64_t(v > 0 && !bad)};
    };
    auto source_b = [&](const SrcA& a, int32_t blk) -> uint64_t {
        return reinterpret_cast<uint64_t>(p.kv) +
               (uint64_t(uint32_t(blk) & uint32_t(a.mask)) * kBlock + (a.j0 % kBlock)) * kRowB;
    };
    auto source_c = [&](const SrcA& a, uint64_t row) -> Src {
        const uint64_t src = (row & a.mask) | (reinterpret_cast<uint64_t>(kZeroRow) & ~a.mask);
        return Src{reinterpret_cast<const uint8_t*>(src), max(min(a.v, kSub) - 1, 0) & int(uint32_t(a.mask))};
    };
    auto source = [&](int j, int32_t blk, auto slot_c) -> Src {
        const SrcA a = source_a(j, blk, slot_c);
        return source_c(a, source_b(a, blk));
    };
    // Sparse: the list entries of sub-tile j this wave gathers (rows 8w ..
    // 8w + 7 of the sub-tile), eight 32-bit pool rows read through the scalar
    // cache in one load; a sub-tile past the last reads the list's first
    // (inside the row; its values are unused).
    const int64_t sp_stride = sparse_list_stride(p.topk);
    auto list_of = [&](int j) -> i32x8 {
        if constexpr (!SPARSE) {
            return i32x8{};
        } else {
            const int jj = j < n_sub ? j : 0;
            return *(const __attribute__((address_space(4))) i32x8*)(p.sp_list + size_t(id.row) * sp_stride +
                                                                      jj * kSub + 8 * wv);
        }
    };
    // Source of a sparse sub-tile: the row address of each of the wave's eight
    // latent loads (the zero row for an entry past the list or a sub-tile past
    // the last), and each lane's address for the rope load (row 8w + lane / 8,
    // its chunk).  Formed in two stages (scalar bases, then the per-lane rope
    // address) so that the main loop can deal them out over MFMA slots.
    struct SrcSp {
        uint64_t base[8];
        uint64_t rope;
    };
    auto sp_bases = [&](int j, const i32x8& r, SrcSp& d) {
        const bool in = j < n_sub;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            d.base[k] = in && r[k] >= 0 ? reinterpret_cast<uint64_t>(p.kv) + uint64_t(uint32_t(r[k])) * kRowB
                                        : reinterpret_cast<uint64_t>(kZeroRow);
    };
    auto sp_rope = [&](int j, const i32x8& r, SrcSp& d) {
        int32_t rl = r[0];
#pragma unroll
        for (int k = 1; k < 8; ++k) rl = (lane >> 3) == k ? r[k] : rl;
        const bool ok = j < n_sub && rl >= 0;
        d.rope = (ok ? reinterpret_cast<uint64_t>(p.kv) + uint64_t(uint32_t(rl)) * kRowB
                     : reinterpret_cast<uint64_t>(kZeroRow)) + uint32_t(r_off);
    };
    auto source_sp = [&](int j, const i32x8& r) -> SrcSp {
        SrcSp d;
        sp_bases(j, r, d);
        sp_rope(j, r, d);
        return d;
    };
    // sparse load k: k < 8 the latent part of row 8w + k, k = 8 the rope parts
    // of rows 8w .. 8w + 7
    auto load_sp = [&](const SrcSp& r, auto slot_c, auto k_c) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int k = decltype(k_c)::value;
        if constexpr (k < kSub / 4) {
            constexpr int imm = k * 8 * kLatB + slot * 2 * kLatB;
            dma16_at<imm>(reinterpret_cast<const void*>(r.base[k]), dv[k], m_lat);
        } else {
            constexpr int imm = slot * kSub * kRopeB;
            dma16_v_at<imm>(reinterpret_cast<const void*>(r.rope), m_rope);
        }
    };
    // load k of this wave for a sub-tile in `slot`: k < 8 the latent part of
    // row 4k + w, k = 8 the rope parts of rows 8w .. 8w + 7.  Branch free:
    // rows past r.last re-read row r.last through a row shift that is uniform
    // over the wave for the latent loads (a scalar max) and one v_min for the
    // rope load; a whole sub-tile shifts by 0.  (A wave issues in order, and
    // branches and 64-bit address arithmetic around each of these loads cost
    // more than the loads themselves.)
    auto load = [&](const Src& r, auto slot_c, auto k_c) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int k = decltype(k_c)::value;
        if constexpr (k < kSub / 4) {
            constexpr int imm = (k & 3) * 8 * 4 * kLatB + (k >> 2) * kLatB + slot * 2 * kLatB;
            const int dt = max(4 * k + wv - r.last, 0);
            dma16_at<imm>(r.src, dv[k] - dt * kRowB, m_lat);
        } else {
            constexpr int imm = slot * kSub * kRopeB;
            dma16_at<imm>(r.src, min(r_row, r.last) * kRowB + r_off, m_rope);
        }
    };
    // all loads of sub-tile j, issued together (one branch for the common
    // case of a whole valid sub-tile)
    auto issue = [&](int j, auto slot_c) {
        if constexpr (SPARSE) {
            const SrcSp r = source_sp(j, list_of(j));
            static_for<0, kLoadsPerWave>([&](auto kc) { load_sp(r, slot_c, kc); });
        } else {
            const Src r = source(j, block_of(j), slot_c);
            static_for<0, kLoadsPerWave>([&](auto kc) { load(r, slot_c, kc); });
        }
    };
    // real rows of sub-tile j (0 for padding); its scores past that are masked
    auto sub_count = [&](int j) { return max(0, min(kSub, tok1 - tok0 - j * kSub)); };

    // query fragments in registers before the ring starts (a wait the compiler
    // sees, so it inserts none of its own for them inside the loop)
    __builtin_amdgcn_s_waitcnt(0);
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    if (n_pad > 0) {
        issue(0, S0{});
        issue(1, S1{});
        issue(2, S2{});
    }
    // load source of the next iteration's sub-tile (j + kAhead + 1), formed one
    // iteration ahead, and the block id of the one after it
    using LSrc = std::conditional_t<SPARSE, SrcSp, Src>;
    using LAhead = std::conditional_t<SPARSE, i32x8, int32_t>;  // block id, or the list entries
    LSrc ld_next;
    LAhead blk_ahead;
    if constexpr (SPARSE) {
        ld_next = source_sp(kAhead, list_of(kAhead));
        blk_ahead = list_of(kAhead + 1);
    } else {
        ld_next = source(kAhead, block_of(kAhead), std::integral_constant<int, kAhead % kRing>{});
        blk_ahead = block_of(kAhead + 1);
    }

    f32x16 acc[kDvT];
#pragma unroll
    for (int i = 0; i < kDvT; ++i) acc[i] = f32x16{};
    float m = -INFINITY;  // reference max of this head, log2 domain
    float l = 0.f;        // sum of 2^(s - m)
    const float sl2 = p.scale * 1.4426950408889634f;
    bool bad_block = false;

    // per-lane operand addresses inside slot 0: every read is one of these
    // bases plus a compile-time offset (slot, token half, dimension group)
    int kb[8];  // K latent chunks c = 2 u + half of group g: kb[u] + 256 g
#pragma unroll
    for (int u = 0; u < 8; ++u) kb[u] = lat_row(0, col) + (((2 * u + half) ^ swz(col)) << 4);
    int kr[4];  // K rope chunks 2 u + half
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = rope_row(0, col) + (((2 * u + half) ^ rswz(col)) << 4);
    int vb[2][4];  // V^T reads: [row t / t + 8][mt & 3]; token half jj adds 1 KB
    {
        const int g16 = lane >> 4, s16 = lane & 15;
        const int c0 = 2 * (g16 & 1) + ((s16 & 3) >> 1);  // chunk within a 32-dim tile
        const int bsub = (s16 & 1) * 8;                  // byte within the chunk
        // this wave's first output tile: whole 256-byte dimension groups
        // (kDvT is a multiple of 4), a plain offset outside the swizzle
        const int dgrp = 256 * dsp * (kDvT / 4);
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const int t = 4 * (g16 >> 1) + (s16 >> 2) + 8 * w;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                vb[w][q] = lat_row(0, t) + dgrp + bsub + (((4 * q + c0) ^ swz(t)) << 4);
        }
    }
    const MLA_LDS uint8_t* lds = (const MLA_LDS uint8_t*)sm.ring;
    auto kread = [&](int slot, int ks) -> bf16x8 {
        const int a = ks < kQLatSteps ? kb[ks & 7] + 256 * (ks >> 3) + 2 * kLatB * slot
                                      : kr[ks - kQLatSteps] + kSub * kRopeB * slot;
        return *(const MLA_LDS bf16x8*)(lds + a);
    };
    auto qread = [&](int u) -> bf16x8 {
        return *(const MLA_LDS bf16x8*)((const MLA_LDS uint8_t*)sm.qrope + qr_off +
                                        (((2 * u + half) ^ qr_sw) << 4));
    };
    // V^T fragment of 32-dim tile mt and 16-token half jj: two transposing
    // reads of 4 tokens x 4 dims per 16-lane group
    auto vread = [&](int slot, int jj, int mt) -> bf16x8 {
        const int go = 256 * (mt >> 2) + kLatB * jj + 2 * kLatB * slot;
        const s16x4 r1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(lds + vb[0][mt & 3] + go));
        const s16x4 r2 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)(lds + vb[1][mt & 3] + go));
        i32x4 raw;
        raw[0] = (int)(uint16_t)r1[0] | ((int)(uint16_t)r1[1] << 16);
        raw[1] = (int)(uint16_t)r1[2] | ((int)(uint16_t)r1[3] << 16);
        raw[2] = (int)(uint16_t)r2[0] | ((int)(uint16_t)r2[1] << 16);
        raw[3] = (int)(uint16_t)r2[2] | ((int)(uint16_t)r2[3] << 16);
        return __builtin_bit_cast(bf16x8, raw);
    };
    // QK step order: the four rope steps first (their Q fragments come from
    // LDS and are dead early), then the 32 latent steps
    auto step_ks = [](int r) { return r < 4 ? kQLatSteps + r : r - 4; };

    // ---- main loop: one flat schedule of 36 + 32/DS MFMA slots per sub-tile --
    // Iteration j issues the score product of sub-tile j+1 (36 MFMAs) and the
    // output product of sub-tile j (32/DS MFMAs: the wave's output tiles x 2
    // token halves), with the softmax of sub-tile j spread over the slots.
    // The layout below is the one for all 16 tiles (68 slots); with fewer
    // tiles the token-half-1 phase is shorter and the second half's
    // probabilities are formed two slots apart.  A wave issues in order,
    // and about four independent VALU instructions (or two exponentials)
    // execute under one 32-cycle MFMA; beyond that each costs the matrix core
    // idle cycles, so the VALU work is dealt out at that rate:
    //   slots  0..13  score steps 0..13, with the max tree, the reference
    //                 update and the first eight probabilities (token half 0);
    //                 the max tree comes before the first MFMA, which waits
    //                 for the sub-tile's first K fragments from LDS
    //   slots 14..45  output tiles of token half 0 alternating with score
    //                 steps 14..29, with the other eight probabilities, the
    //                 normaliser, and the nine loads of sub-tile j+3
    //   slots 46..67  output tiles of token half 1, with score steps 30..35
    // The loop is unrolled by the ring size, so every slot offset is a
    // compile-time immediate, and scores alternate between two register sets,
    // so a just-written MFMA result is never copied.  In the last iteration
    // the score slot runs on whatever the next slot holds and its result is
    // dropped.
    constexpr int kAK = 2;  // K fragments read this many score steps ahead
    constexpr int kAV = 2;  // V^T fragments read this many output MFMAs ahead
    constexpr int kSlots = kQSteps + 2 * kDvT;  // 68, 52 or 44
    constexpr int kC0 = 14 + 2 * kDvT;          // first slot of the token-half-1 phase
    // slot of score step r, and of output MFMA u = kDvT jj + mt.  Slots
    // 0..13 hold score steps 0..13; then token half 0's output MFMAs
    // alternate with score steps 14 ..; then token half 1's output MFMAs
    // are spread among the remaining score steps.
    constexpr auto qk_slot = [](int r) {
        if (r < 14) return r;
        if (r < 14 + kDvT) return 15 + 2 * (r - 14);
        const int k = r - 14 - kDvT;  // score steps left for the last phase
        if constexpr (DS == 1) return kC0 + 2 + 3 * k;                 // S after each PV pair
        else if constexpr (DS == 2) return kC0 + 3 * (k >> 1) + 2 * (k & 1);  // S P S
        else return k < 16 ? kC0 + 5 * (k >> 2) + ((k & 3) < 2 ? (k & 3) : (k & 3) + 1)  // S S P S S
                           : kC0 + 20 + (k - 16);
    };
    constexpr auto pv_slot = [](int u) {
        const int mt = u % kDvT;
        if (u < kDvT) return 14 + 2 * mt;
        if constexpr (DS == 1) return mt < 12 ? kC0 + 3 * (mt >> 1) + (mt & 1) : kC0 + 6 + mt;
        else if constexpr (DS == 2) return mt < 7 ? kC0 + 3 * mt + 1 : kC0 + 21;
        else return kC0 + 5 * mt + 2;
    };
    // the probability pair p (elements 2p, 2p + 1): fma, exp2, sum + pack slots
    constexpr auto fma_slot = [](int p) { return p < 4 ? 4 + 2 * p : DS == 1 ? 16 + 4 * (p - 4) : 12 + 2 * (p - 4); };
    constexpr auto exp_slot = [](int p) { return p < 4 ? 5 + 2 * p : DS == 1 ? 18 + 4 * (p - 4) : 13 + 2 * (p - 4); };
    constexpr auto sum_slot = [](int p) { return p < 4 ? 6 + 2 * p : DS == 1 ? 20 + 4 * (p - 4) : 14 + 2 * (p - 4); };
    constexpr int kSumSlot = DS == 1 ? 34 : 21;         // normaliser
    static_assert(sum_slot(7) < pv_slot(kDvT), "token half 1 probabilities before their first MFMA");
    constexpr auto load_slot = [](int k) { return 15 + 3 * k; };  // the nine loads of sub-tile j+3

    f32x16 sA, sB;
    if (n_pad > 0) {
        wait_vm<2 * kLoadsPerWave>();  // sub-tile 0 (n_pad >= 4, so 1 and 2 were issued)
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int r = 0; r < kQSteps; ++r) {
            const int ks = step_ks(r);
            const bf16x8 a = kread(0, ks);
            const bf16x8 b = ks < kQLatSteps ? qf[ks] : qread(ks - kQLatSteps);
            if (r == 0) mfma32_v_first(sA, a, b);
            else if (r == kQSteps - 1) mfma32_v_last(sA, a, b);
            else mfma32_v(sA, a, b);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    auto iteration = [&](int j, auto slot_c, f32x16& cur, f32x16& nxt) {
        constexpr int sc = decltype(slot_c)::value;       // slot of sub-tile j
        constexpr int sn = (sc + 1) % kRing;              // slot of sub-tile j+1
        // own loads of sub-tile j+1 are complete once at most one later
        // sub-tile (j+2) remains in flight; the barrier makes every wave's
        // loads visible and frees the slot of sub-tile j-1 for sub-tile j+3
        if (j + 2 < n_pad) wait_vm<kLoadsPerWave>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        // sub-tile j+3 goes to the slot sub-tile j-1 used.  Its source comes
        // from the block id read at the end of the last iteration (no LDS
        // read is in flight here, so waiting for it waits for nothing else).
        // Past the last sub-tile the loads still go out, reading the zero
        // row into that free slot (no sub-tile uses it again), so the issue
        // path has no branch.
        using SL = std::integral_constant<int, (sc + kAhead) % kRing>;
        // ld was formed in the last iteration.  The source of the next
        // iteration's sub-tile (j + kAhead + 1, into this iteration's slot sc)
        // is formed here in three stages at light score-step slots of the last
        // phase; the block id's scalar load (issued at the end of the last
        // iteration) is waited for at slot 0, together with the first K reads,
        // so that no later wait drains the LDS reads in flight.
        const LSrc ld = ld_next;
        const LAhead blk = blk_ahead;
        SrcA ld_a;
        uint64_t ld_row = 0;
        // a bad block id's sub-tile holds zero rows: all its scores are
        // masked below; no early exit
        const int cnt = bad_slot[sc] ? 0 : sub_count(j);
        bad_block |= bad_slot[sc];

        // K (and rope Q) fragments of sub-tile j+1, kAK score steps ahead
        bf16x8 kf[kAK + 1];
        bf16x8 qrf[kAK + 1];
#pragma unroll
        for (int r = 0; r < kAK; ++r) {
            kf[r] = kread(sn, step_ks(r));
            if (r < 4) qrf[r] = qread(r);
        }
        auto qk_step = [&](int r) {
            if (r + kAK < kQSteps) {
                kf[(r + kAK) % (kAK + 1)] = kread(sn, step_ks(r + kAK));
                if (r + kAK < 4) qrf[(r + kAK) % (kAK + 1)] = qread(r + kAK);
            }
            const bf16x8& a = kf[r % (kAK + 1)];
            const bf16x8& b = r < 4 ? qrf[r % (kAK + 1)] : qf[r - 4];
            if (r == 0) mfma32_v_first(nxt, a, b);
            else mfma32_v(nxt, a, b);
        };
        // V^T fragments of sub-tile j, kAV output MFMAs ahead; probabilities
        // of token half jj in pf[jj]
        bf16x8 vf[kAV + 1];
        bf16x8 pf[2];
        auto pv_step = [&](int u, bool fresh) {
            if (u + kAV < 2 * kDvT) vf[(u + kAV) % (kAV + 1)] = vread(sc, (u + kAV) / kDvT, (u + kAV) % kDvT);
            const int mt = u % kDvT;
            if (fresh) mfma32_acc<true>(acc[mt], vf[u % (kAV + 1)], pf[u / kDvT]);
            else mfma32_acc(acc[mt], vf[u % (kAV + 1)], pf[u / kDvT]);
        };

        // softmax of sub-tile j (log2 domain; the reference max m may lag the
        // running max by kLag): the max is a depth-3 tree of max3, and each
        // probability pair goes through fma, exp2 and sum + pack in three
        // different slots, so no VALU instruction waits on the one before it
        float mt3[5], mu[2];
        float mx = 0.f, nm = 0.f, ps0 = 0.f, ps1 = 0.f;
        static_for<0, kSlots>([&](auto sc_) {
            constexpr int s = decltype(sc_)::value;
            if constexpr (s == 0) {
                // only a partial or masked sub-tile needs masking
                if (__builtin_expect(cnt < kSub, 0)) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int tok = (i >> 2) * 8 + half * 4 + (i & 3);
                        if (tok >= cnt) cur[i] = -INFINITY;
                    }
                }
#pragma unroll
                for (int k = 0; k < 5; ++k) mt3[k] = fmaxf(fmaxf(cur[3 * k], cur[3 * k + 1]), cur[3 * k + 2]);
            } else if constexpr (s == 1) {
                mu[0] = fmaxf(fmaxf(mt3[0], mt3[1]), mt3[2]);
                mu[1] = fmaxf(fmaxf(mt3[3], mt3[4]), cur[15]);
                mx = fmaxf(mu[0], mu[1]);
            } else if constexpr (s == 2) {
                mx = xhalf_max(mx) * sl2;
            } else if constexpr (s == 3) {
                // raw scores are scaled inside the exponent (scale > 0 keeps
                // the order).  A head whose max grew by more than kLag moves
                // its reference; accumulators of heads that had one rescale.
                const bool grow = mx > m + kLag;
                if (__builtin_expect(__any(grow && m != -INFINITY), 0)) {
                    const float alpha = grow ? exp2f(m - mx) : 1.f;
#pragma unroll
                    for (int i = 0; i < kDvT; ++i) scale_acc(acc[i], alpha);
                    l *= alpha;
                }
                if (grow) m = mx;
                // with no valid score yet (m = -inf) every term is 0
                nm = (m == -INFINITY) ? 0.f : -m;
            }
            static_for<0, 8>([&](auto pc) {
                constexpr int pp = decltype(pc)::value;
                constexpr int i = 2 * pp;
                if constexpr (s == fma_slot(pp)) {
                    cur[i] = fmaf(cur[i], sl2, nm);
                    cur[i + 1] = fmaf(cur[i + 1], sl2, nm);
                } else if constexpr (s == exp_slot(pp)) {
                    cur[i] = __builtin_amdgcn_exp2f(cur[i]);
                    cur[i + 1] = __builtin_amdgcn_exp2f(cur[i + 1]);
                } else if constexpr (s == sum_slot(pp)) {
                    ps0 += cur[i];
                    ps1 += cur[i + 1];
                    pf[i >> 3][i & 7] = (__bf16)cur[i];
                    pf[i >> 3][(i & 7) + 1] = (__bf16)cur[i + 1];
                }
            });
            if constexpr (s == kSumSlot) l += xhalf_sum(ps0 + ps1);
            // (each stage's results are pinned to its slot by an empty asm use:
            // the compiler would otherwise sink the chain next to the loads)
            if constexpr (!SPARSE) {
                if constexpr (s == 0) asm volatile("" ::"s"(blk));
                if constexpr (s == kC0 + 2) {
                    ld_a = source_a(j + kAhead + 1, blk, slot_c);
                    asm volatile("" ::"s"(ld_a.j0), "s"(ld_a.v), "s"(ld_a.mask));
                }
                if constexpr (s == kC0 + 5) {
                    ld_row = source_b(ld_a, blk);
                    asm volatile("" ::"s"(ld_row));
                }
                if constexpr (s == kC0 + 8) {
                    ld_next = source_c(ld_a, ld_row);
                    asm volatile("" ::"s"(ld_next.src), "s"(ld_next.last));
                }
            } else {
                if constexpr (s == 0)
                    asm volatile("" ::"s"(blk[0]), "s"(blk[1]), "s"(blk[2]), "s"(blk[3]), "s"(blk[4]),
                                 "s"(blk[5]), "s"(blk[6]), "s"(blk[7]));
                if constexpr (s == kC0 + 2) {
                    sp_bases(j + kAhead + 1, blk, ld_next);
                    asm volatile("" ::"s"(ld_next.base[0]), "s"(ld_next.base[1]), "s"(ld_next.base[2]),
                                 "s"(ld_next.base[3]));
                    asm volatile("" ::"s"(ld_next.base[4]), "s"(ld_next.base[5]), "s"(ld_next.base[6]),
                                 "s"(ld_next.base[7]));
                }
                if constexpr (s == kC0 + 8) {
                    sp_rope(j + kAhead + 1, blk, ld_next);
                    asm volatile("" ::"v"(ld_next.rope));
                }
            }
            // the first two V^T fragments, two slots before the first output MFMA
            if constexpr (s == pv_slot(0) - 2) vf[0] = vread(sc, 0, 0);
            if constexpr (s == pv_slot(0) - 1) vf[1] = vread(sc, 0, 1);
            static_for<0, kLoadsPerWave>([&](auto kc) {
                if constexpr (s == load_slot(decltype(kc)::value)) {
                    if constexpr (SPARSE) load_sp(ld, SL{}, kc);
                    else load(ld, SL{}, kc);
                }
            });
            // the slot's MFMA
            static_for<0, kQSteps>([&](auto rc) {
                if constexpr (qk_slot(decltype(rc)::value) == s) qk_step(decltype(rc)::value);
            });
            static_for<0, 2 * kDvT>([&](auto uc) {
                constexpr int u = decltype(uc)::value;
                // the first output MFMA reads probabilities packed by VALU
                // converts just before: it leads with the two wait states
                if constexpr (pv_slot(u) == s) pv_step(u, u == 0 || u == kDvT);
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        // Every LDS read of this iteration has been consumed: a scalar load
        // issued now is waited for only by the next iteration's source, after
        // its barrier.
        if constexpr (SPARSE) blk_ahead = list_of(j + kAhead + 2);
        else blk_ahead = block_of(j + kAhead + 2);
        __builtin_amdgcn_sched_barrier(0);
        // wait states before the next iteration's VALU reads the scores just
        // accumulated (the compiler does not see the asm as an MFMA)
        asm volatile("s_nop 7\n\ts_nop 3");
    };
    for (int j = 0; j < n_pad; j += kRing) {
        iteration(j, S0{}, sA, sB);
        iteration(j + 1, S1{}, sB, sA);
        iteration(j + 2, S2{}, sA, sB);
        iteration(j + 3, S3{}, sB, sA);
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
    const size_t orow0 = (direct ? size_t(id.row) : size_t(id.slot)) * p.H + (head - col);  // group's head 0
    const int dim0 = dsp * (kLatent / DS);  // this wave's first output dimension
    // chunk partials stay float32 whatever the output dtype
    if (direct && p.out_dtype == MLA_BF16) {
        // staged through the ring's LDS once every wave is past its last read
        static_assert(sizeof(sm) >= 4 * 32 * 1024, "staging fits the LDS of the ring");
        __syncthreads();
        store_tiles_bf16<kDvT>(acc, inv, (MLA_LDS uint8_t*)&sm + wave * 32 * 1024,
                               static_cast<uint16_t*>(p.o_out) + orow0 * kLatent + dim0,
                               min(32, p.H - (head - col)), lane);
    } else if (head_ok) {
        float* o = static_cast<float*>(direct ? p.o_out : p.ws_o) + (orow0 + col) * kLatent + dim0;
#pragma unroll
        for (int mt = 0; mt < kDvT; ++mt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * mt + 8 * q4 + 4 * half;
                *reinterpret_cast<float4*>(o + d) =
                    make_float4(acc[mt][4 * q4] * inv, acc[mt][4 * q4 + 1] * inv,
                                acc[mt][4 * q4 + 2] * inv, acc[mt][4 * q4 + 3] * inv);
            }
    }
    if (half == 0 && dsp == 0 && head_ok) (direct ? p.lse_out : p.ws_lse)[orow0 + col] = lse;
}

}  // namespace mfma
}  // namespace mla
