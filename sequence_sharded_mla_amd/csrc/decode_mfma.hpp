// Matrix-core partial decode for a bf16 latent cache (gfx950).
//
// One workgroup handles one (shard, request, query token, chunk) row and all
// H query heads; wave w owns heads [32w, 32w + 32).  The shard's local tokens
// stream through a ring of four 32-token sub-tiles in LDS, filled by
// direct global->LDS loads (global_load_lds_dwordx4) three sub-tiles ahead of
// the one being computed.  Per sub-tile and wave:
//
//   S^T[32 tok x 32 heads] = K[32 x 576] . Q^T[576 x 32]        36 MFMA 32x32x16
//   online softmax per head: the scores of one head sit in one lane (and its
//   partner lane l^32), so the running max / sum need one cross-lane step
//   O^T[512 x 32 heads]  += V^T[512 x 32 tok] . P^T[32 tok x 32 heads]
//                                                               32 MFMA 32x32x16
//
// Q^T stays in registers for the whole row.  K rows are read from LDS as the
// A operand (16 B per lane); V^T is read with ds_read_b64_tr_b16, which
// transposes 4 x 4 16-bit blocks across a 16-lane group, so each lane gets
// four consecutive tokens of one latent dimension.  Rows are stored with
// their 16-byte chunks XOR-swizzled by a 4-bit function of the row so that
// both read patterns hit every LDS bank once per pass.
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
constexpr int kRowB = kDk * 2;           // 1152 B per bf16 row
constexpr int kChunks = kRowB / 16;      // 72 16-byte chunks per row
constexpr int kSubB = kSub * kRowB;      // 36864 B per sub-tile
constexpr int kInstPerSub = kSubB / 1024;  // 36 wave-wide 16 B loads
constexpr int kQSteps = kDk / 16;        // 36 K-steps of the score product

// Row swizzle of the 16-byte chunks in LDS.  Chunk c of row t is stored at
// position c ^ f(t) with f(t) = ((t & 3) << 2) | ((t >> 2) & 3): the XOR only
// flips the low 4 bits, so chunks stay inside their aligned 256-byte group.
// The last 8 chunks of a row (the rope part) use f(t) & 7 to stay inside
// the row.  With 64 four-byte banks this makes the 16-lane passes of the
// K-row reads (16 rows, one chunk each) and the 32-lane passes of the V^T
// transposing reads (8 rows x 4 chunk halves) hit every bank once.
__device__ __forceinline__ int swz(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }
__device__ __forceinline__ int swz_pos(int t, int c) {
    const int f = swz(t);
    return c < 64 ? (c ^ f) : (c ^ (f & 7));
}

template <int LPW>
__device__ __forceinline__ void wait_outstanding(int subs) {
    // subs sub-tiles may stay in flight; each is LPW loads of this wave, and
    // loads retire in issue order
    static_assert(2 * LPW < 64, "vmcnt range");
    if (subs >= 2) wait_vm<2 * LPW>();
    else if (subs == 1) wait_vm<LPW>();
    else wait_vm<0>();
}

constexpr int kQRopeB = 128 * kRope * 2;    // rope part of Q for 128 heads

struct alignas(16) SmemBf16 {
    uint8_t ring[kRing][kSubB];
    uint8_t qrope[kQRopeB];  // [head][8 chunks of 16 B], chunk c at c ^ ((head >> 1) & 7)
};

// Per-lane byte offsets (inside a sub-tile) of this wave's LPW direct-to-LDS
// loads: load k of wave w fills LDS bytes [(k*NW + w) * 1024, +1024), 16 bytes
// per lane, i.e. LDS chunk u = (k*NW + w) * 64 + lane = row t, position pos,
// which holds global chunk c = pos ^ swz(t) of row min(t, valid - 1).
template <int NW>
__device__ __forceinline__ int dma_offset(int k, int wave, int lane, int valid) {
    const int ins = k * NW + wave;
    const int u = ins * 64 + lane;
    const int t = u / kChunks;
    const int pos = u - t * kChunks;
    const int c = swz_pos(t, pos);  // the swizzle is its own inverse
    const int tr = t < valid ? t : valid - 1;
    return tr * kRowB + c * 16;
}

template <int NW>
__device__ __forceinline__ void issue_sub(uint8_t* dst, const uint8_t* src, const int* offs,
                                          int wave) {
    constexpr int LPW = kInstPerSub / NW;
    const uint32_t base = lds_addr(dst);
#pragma unroll
    for (int k = 0; k < LPW; ++k)
        dma16(src, offs[k], __builtin_amdgcn_readfirstlane(base + (k * NW + wave) * 1024));
}

template <int NW>
__device__ __forceinline__ void issue_sub_tail(uint8_t* dst, const uint8_t* src, int valid,
                                               int wave, int lane) {
    constexpr int LPW = kInstPerSub / NW;
    const uint32_t base = lds_addr(dst);
#pragma unroll
    for (int k = 0; k < LPW; ++k)
        dma16(src, dma_offset<NW>(k, wave, lane, valid),
              __builtin_amdgcn_readfirstlane(base + (k * NW + wave) * 1024));
}

template <int NW>
__global__ void __launch_bounds__(NW * 64, 1) decode_mfma_bf16_kernel(DecodeParams p) {
    __shared__ SmemBf16 sm;
    constexpr int LPW = kInstPerSub / NW;
    const RowId id = decode_row(p, blockIdx.x);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;  // head within the wave (S^T, O^T columns)
    const int head = wave * 32 + col;
    const int s = p.shard_begin + id.s_rel;
    const int32_t* bt = p.block_tables + (size_t(id.s_rel) * p.B + id.b) * p.max_blocks;

    // ---- token range of this chunk ---------------------------------------
    const int32_t L = p.context_lens[id.b];
    int32_t visible = L - p.Tq + id.t + 1;
    if (visible < 0) visible = 0;
    int32_t local = dev_local_len(visible, s, p.n_shards);
    if ((local + kBlock - 1) / kBlock > p.max_blocks) {
        if (threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
        local = p.max_blocks * kBlock;
    }
    const int32_t tok0 = id.chunk * p.tiles_per_chunk * kBlock;
    int32_t tok1 = tok0 + p.tiles_per_chunk * kBlock;
    if (tok1 > local) tok1 = local;
    const int n_sub = tok1 > tok0 ? (tok1 - tok0 + kSub - 1) / kSub : 0;

    // ---- Q^T fragments: head `head`, dims 16 ks + 8 half .. + 8 ------------
    // latent part in registers, rope part in LDS (each wave writes and later
    // reads only its own heads, so program order within the wave suffices)
    bf16x8 qf[kQLatSteps];
    const int qr_off = head * (kRope * 2);
    const int qr_sw = (head >> 1) & 7;
    {
        const bf16x8* qrow = reinterpret_cast<const bf16x8*>(
            static_cast<const uint16_t*>(p.q) + ((size_t(id.b) * p.Tq + id.t) * p.H + head) * kDk);
#pragma unroll
        for (int ks = 0; ks < kQLatSteps; ++ks) qf[ks] = qrow[2 * ks + half];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = 2 * u + half;
            *(MLA_LDS bf16x8*)((MLA_LDS uint8_t*)sm.qrope + qr_off + ((c ^ qr_sw) << 4)) =
                qrow[2 * (kQLatSteps + u) + half];
        }
    }

    int offs[LPW];
#pragma unroll
    for (int k = 0; k < LPW; ++k) offs[k] = dma_offset<NW>(k, wave, lane, kSub);

    // first row of sub-tile j and its real row count.  A bad block id gives
    // valid = 0: the loads then re-read the zero row and every score of the
    // sub-tile is masked.
    // block ids are read through the scalar cache (the table is read-only
    // here): a vector load would need a vmcnt wait that drains the ring
    const __attribute__((address_space(4))) int32_t* btc =
        (const __attribute__((address_space(4))) int32_t*)bt;
    auto sub_source = [&](int j, int& valid) -> const uint8_t* {
        const int32_t j0 = __builtin_amdgcn_readfirstlane(tok0 + j * kSub);
        valid = min(kSub, tok1 - j0);
        const int32_t blk = btc[j0 / kBlock];
        if (blk < 0 || blk >= p.pool_blocks) {
            valid = 0;
            return kZeroRow;
        }
        return p.kv + (int64_t(blk) * kBlock + (j0 % kBlock)) * kRowB;
    };
    auto issue = [&](int j) {
        int v;
        const uint8_t* src = sub_source(j, v);
        uint8_t* dst = sm.ring[j % kRing];
        if (v == kSub) issue_sub<NW>(dst, src, offs, wave);
        else issue_sub_tail<NW>(dst, src, v > 0 ? v : 1, wave, lane);
    };

    // query fragments in registers before the ring starts (a wait the compiler
    // sees, so it inserts none of its own for them inside the loop)
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
        if (j < n_sub) issue(j);

    f32x16 acc[kDvTiles];
#pragma unroll
    for (int i = 0; i < kDvTiles; ++i) acc[i] = f32x16{};
    float m = -INFINITY;  // reference max of this head, log2 domain
    float l = 0.f;        // sum of 2^(s - m)
    const float sl2 = p.scale * 1.4426950408889634f;
    bool bad_block = false;

    // per-lane operand addresses inside a sub-tile: every read is one of a
    // few per-lane bases plus a compile-time offset
    int kb[8];  // K rows, latent chunks c = 2 ks + half = 16 g + c', ks = 8 g + u
#pragma unroll
    for (int u = 0; u < 8; ++u) kb[u] = col * kRowB + (((2 * u + half) ^ swz(col)) << 4);
    int kr[4];  // K rows, rope chunks 64 .. 71
#pragma unroll
    for (int u = 0; u < 4; ++u) kr[u] = col * kRowB + (swz_pos(col, 64 + 2 * u + half) << 4);
    int vb[2][4];  // V^T reads: [row t / t + 8][mt & 3]; token half jj adds 16 rows
    {
        const int g16 = lane >> 4, s16 = lane & 15;
        const int c0 = 2 * (g16 & 1) + ((s16 & 3) >> 1);  // chunk within a 32-dim tile
        const int bsub = (s16 & 1) * 8;                  // byte within the chunk
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const int t = 4 * (g16 >> 1) + (s16 >> 2) + 8 * w;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                vb[w][q] = t * kRowB + bsub + (((4 * q + c0) ^ swz(t)) << 4);
        }
    }

    for (int j = 0; j < n_sub; ++j) {
        // own loads of sub-tile j are complete once at most
        // min(n_sub - 1 - j, kAhead - 1) later sub-tiles remain in flight
        wait_outstanding<LPW>(min(n_sub - 1 - j, kAhead - 1));
        __builtin_amdgcn_s_barrier();
        if (j + kAhead < n_sub) issue(j + kAhead);
        int cnt;
        (void)sub_source(j, cnt);
        bad_block |= cnt == 0;  // scores all masked below; no early exit (see above)
        uint8_t* tile = sm.ring[j % kRing];

        // ---- scores: S^T = K . Q^T ----------------------------------------
        f32x16 st;
        const MLA_LDS uint8_t* lt = (const MLA_LDS uint8_t*)tile;
        auto kread = [&](int ks) -> bf16x8 {
            const int a = ks < 32 ? kb[ks & 7] + 256 * (ks >> 3) : kr[ks - 32];
            return *(const MLA_LDS bf16x8*)(lt + a);
        };
        auto qread = [&](int u) -> bf16x8 {
            return *(const MLA_LDS bf16x8*)((const MLA_LDS uint8_t*)sm.qrope + qr_off +
                                            (((2 * u + half) ^ qr_sw) << 4));
        };
        // K fragments are read four steps ahead of the MFMA that uses them
        constexpr int kAheadK = 4;
        bf16x8 kf[kAheadK + 1];
        bf16x8 qrf[4];
#pragma unroll
        for (int i = 0; i < kAheadK; ++i) kf[i] = kread(i);
#pragma unroll
        for (int ks = 0; ks < kQSteps; ++ks) {
            if (ks + kAheadK < kQSteps) kf[(ks + kAheadK) % (kAheadK + 1)] = kread(ks + kAheadK);
            if (ks == kQLatSteps - 8) {
#pragma unroll
                for (int u = 0; u < 4; ++u) qrf[u] = qread(u);
            }
            const bf16x8& a = kf[ks % (kAheadK + 1)];
            const bf16x8& b = ks < kQLatSteps ? qf[ks] : qrf[ks - kQLatSteps];
            if (ks == 0) mfma32_v_first(st, a, b);
            else if (ks == kQSteps - 1) mfma32_v_last(st, a, b);
            else mfma32_v(st, a, b);
        }

        // ---- online softmax (log2 domain, lagging reference max) ----------
        // raw scores are scaled inside the exponent (scale > 0 keeps the
        // order, so the max is taken on raw scores); only a partial last
        // sub-tile needs masking
        if (cnt < kSub) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int tok = (i >> 2) * 8 + half * 4 + (i & 3);
                if (tok >= cnt) st[i] = -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(st[0], st[1]), st[2]);
#pragma unroll
        for (int i = 3; i < 16; i += 2) mx = fmaxf(fmaxf(mx, st[i]), st[i + 1]);
        mx = fmaxf(mx, st[15]);
        mx = xhalf_max(mx) * sl2;
        if (m == -INFINITY) {
            m = mx;  // first scores of this head: nothing accumulated yet
        } else if (__any(mx > m + kLag)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = exp2f(m - m_new);
#pragma unroll
            for (int i = 0; i < kDvTiles; ++i) scale_acc(acc[i], alpha);
            l *= alpha;
            m = m_new;
        }
        // with no valid score yet (m = -inf) every term is 0
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
        bf16x8 pf[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[jj][e] = (__bf16)st[8 * jj + e];

        // ---- O^T += V^T . P^T ----------------------------------------------
        // V^T fragment of 32-dim tile mt and 16-token half jj: two transposing
        // reads of 4 tokens x 4 dims per 16-lane group
        auto vread = [&](int jj, int mt) -> bf16x8 {
            const int go = 256 * (mt >> 2) + jj * 16 * kRowB;
            const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (MLA_LDS s16x4*)(lt + vb[0][mt & 3] + go));
            const s16x4 r2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (MLA_LDS s16x4*)(lt + vb[1][mt & 3] + go));
            i32x4 raw;
            raw[0] = (int)(uint16_t)r1[0] | ((int)(uint16_t)r1[1] << 16);
            raw[1] = (int)(uint16_t)r1[2] | ((int)(uint16_t)r1[3] << 16);
            raw[2] = (int)(uint16_t)r2[0] | ((int)(uint16_t)r2[1] << 16);
            raw[3] = (int)(uint16_t)r2[2] | ((int)(uint16_t)r2[3] << 16);
            return __builtin_bit_cast(bf16x8, raw);
        };
        // V^T fragments are read two output tiles ahead of their MFMAs
        constexpr int kAheadV = 2;
        bf16x8 vf[kAheadV + 1][2];
#pragma unroll
        for (int i = 0; i < kAheadV; ++i) {
            vf[i][0] = vread(0, i);
            vf[i][1] = vread(1, i);
        }
#pragma unroll
        for (int mt = 0; mt < kDvTiles; ++mt) {
            if (mt + kAheadV < kDvTiles) {
                vf[(mt + kAheadV) % (kAheadV + 1)][0] = vread(0, mt + kAheadV);
                vf[(mt + kAheadV) % (kAheadV + 1)][1] = vread(1, mt + kAheadV);
            }
            const int r = mt % (kAheadV + 1);
            if (mt == 0) mfma32_acc<true>(acc[mt], vf[r][0], pf[0]);
            else mfma32_acc(acc[mt], vf[r][0], pf[0]);
            mfma32_acc(acc[mt], vf[r][1], pf[1]);
        }
    }
    mfma_drain();
    if (bad_block && threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);

    // ---- finalise: O = acc / l, LSE = ln 2 * (m + log2 l) --------------------
    const bool empty = l == 0.f;  // NaN stays visible
    const float inv = empty ? 0.f : 1.f / l;
    const float lse = empty ? -INFINITY : (m + log2f(l)) * 0.6931471805599453f;
    const size_t hrow = size_t(id.row) * p.H + head;
    const bool direct = p.n_chunks == 1;
    const size_t slot = (size_t(id.row) * p.n_chunks + id.chunk) * p.H + head;
    if (direct && p.out_dtype == MLA_BF16) {
        uint16_t* o = static_cast<uint16_t*>(p.o_out) + hrow * kLatent;
#pragma unroll
        for (int mt = 0; mt < kDvTiles; ++mt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int d = 32 * mt + 8 * q4 + 4 * half;
                uint2 w;
                w.x = uint32_t(f32_to_bf16(acc[mt][4 * q4 + 0] * inv)) |
                      (uint32_t(f32_to_bf16(acc[mt][4 * q4 + 1] * inv)) << 16);
                w.y = uint32_t(f32_to_bf16(acc[mt][4 * q4 + 2] * inv)) |
                      (uint32_t(f32_to_bf16(acc[mt][4 * q4 + 3] * inv)) << 16);
                *reinterpret_cast<uint2*>(o + d) = w;
            }
    } else {
        float* o = direct ? static_cast<float*>(p.o_out) + hrow * kLatent : p.ws_o + slot * kLatent;
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
    if (half == 0) {
        if (direct) p.lse_out[hrow] = lse;
        else p.ws_lse[slot] = lse;
    }
}

}  // namespace mfma
}  // namespace mla
