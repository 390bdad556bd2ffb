// Matrix-core partial decode for a bf16 latent cache (gfx950).
//
// One workgroup of four waves handles one (shard, request, query token,
// chunk) row and all 128 query heads; wave w owns heads [32w, 32w + 32).  The
// shard's local tokens stream through a ring of four 32-token sub-tiles in
// LDS, filled by direct global->LDS loads (global_load_lds_dwordx4) three
// sub-tiles ahead.  Per sub-tile and wave:
//
//   S^T[32 tok x 32 heads] = K[32 x 576] . Q^T[576 x 32]        36 MFMA 32x32x16
//   online softmax per head: the scores of one head sit in one lane (and its
//   partner lane l^32), so the running max / sum need one cross-lane step
//   O^T[512 x 32 heads]  += V^T[512 x 32 tok] . P^T[32 tok x 32 heads]
//                                                               32 MFMA 32x32x16
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

__global__ void __launch_bounds__(256, 1) decode_mfma_bf16_kernel(DecodeParams p) {
    __shared__ SmemBf16 sm;
    RowId id;
    if (!work_item(p, blockIdx.x, id)) return;  // past the last planned item
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;  // head within the wave (S^T, O^T columns)
    const int head = wave * 32 + col;
    const int s = p.shard_begin + id.s_rel;
    const int32_t* bt = p.block_tables + (size_t(id.s_rel) * p.B + id.b) * p.max_blocks;

    // ---- token range of this chunk ---------------------------------------
    const int32_t L = p.context_lens[id.b];
    int32_t visible = L - id.qlen + id.t + 1;
    if (visible < 0) visible = 0;
    int32_t local = dev_local_len(visible, s, p.n_shards);
    if ((local + kBlock - 1) / kBlock > p.max_blocks) {
        if (threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
        local = p.max_blocks * kBlock;
    }
    const int32_t tok0 = id.chunk * id.chunk_tok;
    int32_t tok1 = id.chunk_tok ? tok0 + id.chunk_tok : local;
    if (tok1 > local) tok1 = local;
    const int n_sub = tok1 > tok0 ? (tok1 - tok0 + kSub - 1) / kSub : 0;
    // the pipelined loop below is unrolled by the ring size and always runs
    // whole rounds: padding sub-tiles are zero rows with every score masked
    const int n_pad = (n_sub + kRing - 1) / kRing * kRing;

    // ---- Q^T fragments: head `head`, dims 16 ks + 8 half .. + 8 ------------
    // latent part in registers, rope part in LDS (each wave writes and later
    // reads only its own heads, so program order within the wave suffices)
    bf16x8 qf[kQLatSteps];
    const int qr_off = head * kRopeB;
    const int qr_sw = (head >> 1) & 7;
    {
        const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
            static_cast<const uint16_t*>(p.q) + (size_t(id.qi) * p.H + head) * kDk);
#pragma unroll
        for (int ks = 0; ks < kQLatSteps; ++ks) qf[ks] = qrow[2 * ks + half];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = 2 * u + half;
            *(MLA_LDS bf16x8*)((MLA_LDS uint8_t*)sm.qrope + qr_off + ((c ^ qr_sw) << 4)) =
                qrow[2 * (kQLatSteps + u) + half];
        }
    }

    // ---- sub-tile loads ----------------------------------------------------
    // Wave w loads the latent parts of rows 4k + w (k = 0..7), one row per
    // wave-wide load (lane i fetches the chunk stored at position i), and the
    // rope parts of rows 8w .. 8w + 7 in one load.  A full sub-tile uses
    // per-lane offsets computed once; a partial one (rows at or past its
    // valid count re-read its last valid row) and the zero row of a bad or
    // padding sub-tile take a clamped path.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int dv[kSub / 4];  // latent loads of a full sub-tile
#pragma unroll
    for (int k = 0; k < kSub / 4; ++k) {
        const int t = 4 * k + wave;
        dv[k] = t * kRowB + ((((lane & 48) | ((lane & 15) ^ swz(t)))) << 4);
    }
    const int r_row = 8 * wave + (lane >> 3);  // rope load: row and chunk of this lane
    const int r_off = (kLatent / 8 + ((lane & 7) ^ rswz(r_row))) << 4;
    const int ro_full = r_row * kRowB + r_off;
    // LDS destinations: lat_row(slot, 4k + w) = w * 8 KB + (k & 3) * 32 KB +
    // (k >> 2) * 1 KB + slot * 2 KB; rope_row(slot, 8w) = rope base + slot * 4 KB + w * 1 KB
    const uint32_t lds0 = lds_addr(sm.ring);
    const uint32_t m_lat = __builtin_amdgcn_readfirstlane(lds0 + wv * (4 * 2 * kLatB));
    const uint32_t m_rope = __builtin_amdgcn_readfirstlane(lds0 + kLatRegion + wv * 8 * kRopeB);

    // Block ids are read through the scalar cache (the table is read-only
    // here): a vector load would need a vmcnt wait that drains the ring.
    const __attribute__((address_space(4))) int32_t* btc =
        (const __attribute__((address_space(4))) int32_t*)bt;
    bool bad_slot[kRing] = {false, false, false, false};  // sub-tile in the slot had a bad block id
    // Source of sub-tile j: first row in HBM, and the last row to read (rows
    // past it re-read it); full = a whole sub-tile of one valid block.
    struct Src {
        const uint8_t* src;
        int last;
        bool full;
    };
    auto source = [&](int j, auto slot_c) -> Src {
        constexpr int slot = decltype(slot_c)::value;
        const uint32_t j0 = uint32_t(tok0) + uint32_t(j) * kSub;
        const int v = min(kSub, tok1 - int(j0));  // <= 0: padding
        Src r{kZeroRow, 0, false};
        bool bad = false;
        if (v > 0) {
            const int32_t blk = btc[j0 / kBlock];
            if (blk >= 0 && blk < p.pool_blocks) {
                r.src = p.kv + (int64_t(blk) * kBlock + (j0 % kBlock)) * kRowB;
                r.last = v - 1;
                r.full = v == kSub;
            } else {
                bad = true;
            }
        }
        bad_slot[slot] = bad;
        return r;
    };
    // load k of this wave for a sub-tile in `slot`: k < 8 the latent part of
    // row 4k + w, k = 8 the rope parts of rows 8w .. 8w + 7
    auto load = [&](const Src& r, auto slot_c, auto k_c) {
        constexpr int slot = decltype(slot_c)::value;
        constexpr int k = decltype(k_c)::value;
        if constexpr (k < kSub / 4) {
            constexpr int imm = (k & 3) * 8 * 4 * kLatB + (k >> 2) * kLatB + slot * 2 * kLatB;
            if (r.full) {
                dma16_at<imm>(r.src, dv[k], m_lat);
            } else {
                const int t = 4 * k + wv;
                const int dt = t > r.last ? t - r.last : 0;
                dma16_at<imm>(r.src, dv[k] - dt * kRowB, m_lat);
            }
        } else {
            constexpr int imm = slot * kSub * kRopeB;
            const int ro = r.full ? ro_full : (r_row < r.last ? r_row : r.last) * kRowB + r_off;
            dma16_at<imm>(r.src, ro, m_rope);
        }
    };
    // all loads of sub-tile j, issued together (one branch for the common
    // case of a whole valid sub-tile)
    auto issue = [&](int j, auto slot_c) {
        const Src r = source(j, slot_c);
        if (r.full) {
            const Src f{r.src, kSub - 1, true};
            static_for<0, kLoadsPerWave>([&](auto kc) { load(f, slot_c, kc); });
        } else {
            const Src c{r.src, r.last, false};
            static_for<0, kLoadsPerWave>([&](auto kc) { load(c, slot_c, kc); });
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

    f32x16 acc[kDvTiles];
#pragma unroll
    for (int i = 0; i < kDvTiles; ++i) acc[i] = f32x16{};
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
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const int t = 4 * (g16 >> 1) + (s16 >> 2) + 8 * w;
#pragma unroll
            for (int q = 0; q < 4; ++q) vb[w][q] = lat_row(0, t) + bsub + (((4 * q + c0) ^ swz(t)) << 4);
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

    // ---- main loop, software pipelined ---------------------------------------
    // Iteration j issues the score product of sub-tile j+1 (36 MFMAs) and the
    // output product of sub-tile j (32 MFMAs).  The first kLead score steps
    // carry the softmax of sub-tile j (VALU work that overlaps the matrix
    // cores); the rest alternate with the output tiles, spreading the K and
    // V^T reads from LDS over the iteration.  The loop is unrolled by the ring
    // size, so every slot offset is a compile-time immediate, and scores
    // alternate between two register sets, so a just-written MFMA result is
    // never copied.  In the last iteration the score slot runs on whatever
    // the next slot holds and its result is dropped.
    constexpr int kLead = kQSteps - kDvTiles;  // 20 score steps before the first output tile
    constexpr int kAK = 2;                     // K fragments read this many steps ahead
    constexpr int kAV = 2;                     // V^T tiles read this many tiles ahead

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
        // sub-tile j+3 goes to the slot sub-tile j-1 used
        if (j + kAhead < n_pad) issue(j + kAhead, std::integral_constant<int, (sc + kAhead) % kRing>{});
        // a bad block id's sub-tile holds zero rows: all its scores are
        // masked below; no early exit
        const int cnt = bad_slot[sc] ? 0 : sub_count(j);
        bad_block |= bad_slot[sc];

        // K (and rope Q) fragments are read kAK steps ahead of their MFMA
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

        // ---- phase 1: score steps 0 .. kLead-1 with the softmax of sub-tile j
        // (log2 domain; the reference max m may lag the running max by kLag)
        float mx = 0.f, nm = 0.f, ps = 0.f;
        bf16x8 pf[2];
        bf16x8 vf[kAV + 1][2];
        static_for<0, kLead>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            qk_step(r);
            if (r == 0) {
                // only a partial or masked sub-tile needs masking
                if (cnt < kSub) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int tok = (i >> 2) * 8 + half * 4 + (i & 3);
                        if (tok >= cnt) cur[i] = -INFINITY;
                    }
                }
                mx = fmaxf(fmaxf(cur[0], cur[1]), cur[2]);
#pragma unroll
                for (int i = 3; i < 15; i += 2) mx = fmaxf(fmaxf(mx, cur[i]), cur[i + 1]);
                mx = fmaxf(mx, cur[15]);
            } else if (r == 1) {
                mx = xhalf_max(mx) * sl2;
            } else if (r == 2) {
                // raw scores are scaled inside the exponent (scale > 0 keeps
                // the order).  A head whose max grew by more than kLag moves
                // its reference; accumulators of heads that had one rescale.
                const bool grow = mx > m + kLag;
                if (__any(grow && m != -INFINITY)) {
                    const float alpha = grow ? exp2f(m - mx) : 1.f;
#pragma unroll
                    for (int i = 0; i < kDvTiles; ++i) scale_acc(acc[i], alpha);
                    l *= alpha;
                }
                if (grow) m = mx;
                // with no valid score yet (m = -inf) every term is 0
                nm = (m == -INFINITY) ? 0.f : -m;
            } else if (r >= 3 && r < 19) {
                const int i = r - 3;
                const float e = __builtin_amdgcn_exp2f(fmaf(cur[i], sl2, nm));
                cur[i] = e;
                ps += e;
            } else if (r == 19) {
                ps = xhalf_sum(ps);
                l += ps;
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int e = 0; e < 8; ++e) pf[jj][e] = (__bf16)cur[8 * jj + e];
            }
            if (r == kLead - 2) {
                vf[0][0] = vread(sc, 0, 0);
                vf[0][1] = vread(sc, 1, 0);
            } else if (r == kLead - 1) {
                vf[1][0] = vread(sc, 0, 1);
                vf[1][1] = vread(sc, 1, 1);
            }
            __builtin_amdgcn_sched_barrier(0);
        });

        // ---- phase 2: O^T += V^T . P^T, one output tile per remaining score step
#pragma unroll
        for (int mt = 0; mt < kDvTiles; ++mt) {
            if (mt + kAV < kDvTiles) {
                vf[(mt + kAV) % (kAV + 1)][0] = vread(sc, 0, mt + kAV);
                vf[(mt + kAV) % (kAV + 1)][1] = vread(sc, 1, mt + kAV);
            }
            const int v = mt % (kAV + 1);
            if (mt == 0) mfma32_acc<true>(acc[mt], vf[v][0], pf[0]);
            else mfma32_acc(acc[mt], vf[v][0], pf[0]);
            mfma32_acc(acc[mt], vf[v][1], pf[1]);
            qk_step(kLead + mt);
            __builtin_amdgcn_sched_barrier(0);
        }
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
        static_assert(sizeof(sm) >= 4 * 32 * 1024, "staging fits the LDS of the ring");
        __syncthreads();
        store_rows_bf16<1>(acc, inv, (MLA_LDS uint8_t*)&sm + wave * 32 * 1024,
                            static_cast<uint16_t*>(direct ? p.o_out : p.ws_o) + (orow - col) * kLatent,
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
