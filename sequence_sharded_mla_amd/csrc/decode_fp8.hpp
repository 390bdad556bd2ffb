// Matrix-core partial decode for the packed fp8 latent cache (gfx950), dense
// and sparse.
//
// Row format (656 B): 512 E4M3FN codes, 4 float32 scales (one per 128-dim
// group), 64 bf16 rope values.  Latent value d of token t is
// code[t][d] * scale[t][d / 128].
//
// One workgroup of NW waves handles one (shard, request, query token, chunk)
// row; wave w owns query heads [32w, 32w + 32).  Rows stream through a ring
// of three 32-token sub-tiles in LDS (direct global->LDS loads two sub-tiles
// ahead).  Codes are widened to bf16 exactly in registers
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1) right before each MFMA, and the
// group scales are applied in float32 after the products, so the scores are
// exact bf16 x fp8 products accumulated in float32:
//
//   S^T  = K_rope . Q_rope^T + sum_g scale_g (.) (C_g . Q_g^T)      MFMA 32x32x16
//   O^T += sum_g C_g^T . (P (.) scale_g)^T                          MFMA 32x32x16
//
// C_g are the codes of group g, (.) scales token rows.  V^T fragments come
// from ds_read_b64_tr_b8: in each 16-lane group, output lane i receives byte
// i % 8 of source lanes 2r + i / 8 (r = 0..7), so source lane 2r + b loads 8
// codes of token r, which gives each lane 8 tokens of one latent dimension.
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

constexpr int kRowF = 656;                    // bytes per fp8 row
constexpr int kUnitsF = kRowF / 16;           // 41 16-byte units per row
constexpr int kSubF = kSub * kRowF;           // 20992 B per 32-token sub-tile
constexpr int kUnitsSubF = kSub * kUnitsF;    // 1312 units per sub-tile
constexpr int kRingF = 3;                     // sub-tiles resident in LDS
constexpr int kAheadF = kRingF - 1;           // sub-tiles in flight ahead of compute
constexpr int kScaleOff = kLatent;            // byte offset of the scales in a row
constexpr int kRopeOff = kLatent + 16;        // byte offset of the rope part
constexpr int kMaxTopk = 2048;                // longest top-K list kept in LDS

template <int NW, bool SPARSE>
struct alignas(16) SmemFp8 {
    uint8_t ring[kRingF][kSubF];
    uint8_t qrope[NW * 32 * kRope * 2];  // [head][8 chunks], chunk c at c ^ ((head >> 1) & 7)
    float scales[NW][4][kSub];           // per wave: group scales of the current sub-tile
    int32_t rows[SPARSE ? kMaxTopk : 1]; // sparse: pool rows this shard owns, entry order
    int32_t wave_cnt[NW];
};

// 8 E4M3FN codes (two dwords, byte e = token/dim e) -> 8 bf16, exactly.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 c) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false);
    const bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true);
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = d[0]; r[5] = d[1]; r[6] = e[0]; r[7] = e[1];
    return r;
}

template <int LPW>
__device__ __forceinline__ void wait_outstanding_f(int subs) {
    static_assert(LPW < 64, "vmcnt range");
    if (subs >= 1) wait_vm<LPW>();
    else wait_vm<0>();
}

// LDS is filled in 16-byte units with rows kept whole and in order (row t
// at byte 656 t).  Wave w loads units [w * U, (w + 1) * U), U = 1312 / NW, as
// ceil(U / 64) wave-wide loads; lanes past U stay idle.
template <int NW>
struct DmaPlan {
    static constexpr int kU = kUnitsSubF / NW;
    static constexpr int kLoads = (kU + 63) / 64;
};

template <int NW, bool SPARSE>
__global__ void __launch_bounds__(NW * 64, 1) decode_mfma_fp8_kernel(DecodeParams p) {
    __shared__ SmemFp8<NW, SPARSE> sm;
    constexpr int LPW = DmaPlan<NW>::kLoads;
    constexpr int U = DmaPlan<NW>::kU;
    const RowId id = decode_row(p, blockIdx.x);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int half = lane >> 5;
    const int col = lane & 31;
    const int head = wave * 32 + col;
    const int s = p.shard_begin + id.s_rel;
    const int32_t* bt = p.block_tables + (size_t(id.s_rel) * p.B + id.b) * p.max_blocks;
    const __attribute__((address_space(4))) int32_t* btc =
        (const __attribute__((address_space(4))) int32_t*)bt;

    const int32_t L = p.context_lens[id.b];
    int32_t visible = L - p.Tq + id.t + 1;
    if (visible < 0) visible = 0;

    // ---- the tokens this workgroup attends ---------------------------------
    int32_t tok0 = 0, tok1 = 0;  // dense: local token range; sparse: list range
    if (!SPARSE) {
        int32_t local = dev_local_len(visible, s, p.n_shards);
        if ((local + kBlock - 1) / kBlock > p.max_blocks) {
            if (threadIdx.x == 0) raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
            local = p.max_blocks * kBlock;
        }
        tok0 = id.chunk * p.tiles_per_chunk * kBlock;
        tok1 = min(tok0 + p.tiles_per_chunk * kBlock, local);
        if (tok1 < tok0) tok1 = tok0;
    } else {
        // compact the entries this shard owns, in entry order
        const int32_t* idx = p.topk_idx + (size_t(id.b) * p.Tq + id.t) * p.topk;
        int total = 0;
        for (int32_t e0 = 0; e0 < p.topk; e0 += NW * 64) {
            const int32_t e = e0 + threadIdx.x;
            int32_t row = -1;
            if (e < p.topk) {
                const int32_t g = idx[e];
                if (g >= 0) {
                    if (g >= visible) {
                        raise_error(p.err, MLA_DEVERR_INDEX);
                    } else if (g % p.n_shards == s) {
                        const int32_t j = g / p.n_shards;
                        const int32_t blk = j / kBlock < p.max_blocks ? bt[j / kBlock] : -1;
                        if (blk >= 0 && blk < p.pool_blocks) row = blk * kBlock + (j % kBlock);
                        else raise_error(p.err, MLA_DEVERR_BLOCK_TABLE);
                    }
                }
            }
            const uint64_t mask = __ballot(row >= 0);
            const int before = __popcll(mask & ((uint64_t(1) << lane) - 1));
            if (lane == 0) sm.wave_cnt[wave] = __popcll(mask);
            __syncthreads();
            int base = total;
            for (int w = 0; w < NW; ++w) {
                if (w < wave) base += sm.wave_cnt[w];
                total += sm.wave_cnt[w];
            }
            if (row >= 0) sm.rows[base + before] = row;
            __syncthreads();
        }
        tok1 = total;
    }
    const int n_sub = (tok1 - tok0 + kSub - 1) / kSub;

    // ---- query: latent part in registers, rope part in LDS -------------------
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
    __builtin_amdgcn_s_waitcnt(0);

    // ---- sub-tile loads ------------------------------------------------------
    // dense: rows of sub-tile j are contiguous in one pool block; sparse: rows
    // come from the list.  valid = real rows; later rows repeat the last one.
    auto dense_src = [&](int j, int& valid) -> const uint8_t* {
        const int32_t j0 = __builtin_amdgcn_readfirstlane(tok0 + j * kSub);
        valid = min(kSub, tok1 - j0);
        const int32_t blk = btc[j0 / kBlock];
        if (blk < 0 || blk >= p.pool_blocks) {
            valid = 0;
            return kZeroRow;
        }
        return p.kv + (int64_t(blk) * kBlock + (j0 % kBlock)) * kRowF;
    };
    auto issue = [&](int j) {
        uint8_t* dst = sm.ring[j % kRingF];
        const uint32_t lbase = lds_addr(dst) + wave * U * 16;
        if (!SPARSE) {
            int v;
            const uint8_t* src = dense_src(j, v);
#pragma unroll
            for (int k = 0; k < LPW; ++k) {
                const int u = wave * U + k * 64 + lane;  // unit of the sub-tile
                const int t = u / kUnitsF;
                const int voff = t < v ? u * 16 : (v > 0 ? (v - 1) * kRowF + (u - t * kUnitsF) * 16
                                                         : (u - t * kUnitsF) * 16);
                if (k * 64 + lane < U) dma16(src, voff, __builtin_amdgcn_readfirstlane(lbase + k * 1024));
            }
        } else {
            const int j0 = j * kSub;
            const int v = min(kSub, tok1 - j0);
#pragma unroll
            for (int k = 0; k < LPW; ++k) {
                const int u = wave * U + k * 64 + lane;
                const int t = u / kUnitsF;
                const int row = sm.rows[j0 + (t < v ? t : v - 1)];
                const uint8_t* g = p.kv + int64_t(row) * kRowF + (u - t * kUnitsF) * 16;
                if (k * 64 + lane < U) dma16_v(g, __builtin_amdgcn_readfirstlane(lbase + k * 1024));
            }
        }
    };
#pragma unroll
    for (int j = 0; j < kAheadF; ++j)
        if (j < n_sub) issue(j);

    f32x16 acc[kDvTiles];
#pragma unroll
    for (int i = 0; i < kDvTiles; ++i) acc[i] = f32x16{};
    float m = -INFINITY;
    float l = 0.f;
    const float sl2 = p.scale * 1.4426950408889634f;
    bool bad_block = false;

    // per-lane operand addresses inside a sub-tile (plus compile-time offsets)
    const int k_lat = col * kRowF + 8 * half;              // codes of row `col`
    const int k_rope = col * kRowF + kRopeOff + 16 * half;  // rope of row `col`
    // V^T transposing reads: in 16-lane group g16, source lane s16 = 2r + b
    // loads codes of the r-th token of this lane half's k-slice
    int vt_base;
    {
        const int g16 = lane >> 4, s16 = lane & 15;
        const int r = s16 >> 1, b = s16 & 1;
        const int tok = 8 * (r >> 2) + 4 * (g16 >> 1) + (r & 3);
        vt_base = tok * kRowF + 16 * (g16 & 1) + 8 * b;
    }
    // scale transpose: lane handles token lane/2, groups 2(lane&1) .. +1
    const int sc_tok = lane >> 1, sc_g = 2 * (lane & 1);

    for (int j = 0; j < n_sub; ++j) {
        wait_outstanding_f<LPW>(min(n_sub - 1 - j, kAheadF - 1));
        __builtin_amdgcn_s_barrier();
        if (j + kAheadF < n_sub) issue(j + kAheadF);
        int cnt;
        if (!SPARSE) (void)dense_src(j, cnt);
        else cnt = min(kSub, tok1 - j * kSub);
        bad_block |= cnt == 0;
        const MLA_LDS uint8_t* lt = (const MLA_LDS uint8_t*)sm.ring[j % kRingF];

        // group scales of this sub-tile, transposed to [group][token] per wave
        {
            const f32x2 sv = *(const MLA_LDS f32x2*)(lt + sc_tok * kRowF + kScaleOff + 4 * sc_g);
            float* scw = &sm.scales[wave][0][0];
            *(MLA_LDS float*)((MLA_LDS uint8_t*)scw + (sc_g * kSub + sc_tok) * 4) = sv[0];
            *(MLA_LDS float*)((MLA_LDS uint8_t*)scw + ((sc_g + 1) * kSub + sc_tok) * 4) = sv[1];
        }
        // scales of the 16 tokens this lane holds, for group g:
        // tokens (i >> 2) * 8 + 4 half + (i & 3)
        auto load_scales = [&](int g, float (&sc)[16]) {
            const MLA_LDS float* row =
                (const MLA_LDS float*)((const MLA_LDS uint8_t*)&sm.scales[wave][0][0] +
                                       (g * kSub + 4 * half) * 4);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = *(const MLA_LDS f32x4*)(row + 8 * q);
                sc[4 * q] = v[0]; sc[4 * q + 1] = v[1]; sc[4 * q + 2] = v[2]; sc[4 * q + 3] = v[3];
            }
        };

        // ---- scores ------------------------------------------------------------
        f32x16 st;
        {
            // rope part (bf16 values, scale 1)
            bf16x8 kr[4], qr[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                kr[u] = *(const MLA_LDS bf16x8*)(lt + k_rope + 32 * u);
                qr[u] = *(const MLA_LDS bf16x8*)((const MLA_LDS uint8_t*)sm.qrope + qr_off +
                                                 (((2 * u + half) ^ qr_sw) << 4));
            }
            mfma32_v_first(st, kr[0], qr[0]);
            mfma32_v(st, kr[1], qr[1]);
            mfma32_v(st, kr[2], qr[2]);
            mfma32_v_last(st, kr[3], qr[3]);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // codes of group g: 8 K-steps of 16 dims
            i32x2 raw[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                raw[u] = *(const MLA_LDS i32x2*)(lt + k_lat + 128 * g + 16 * u);
            f32x16 ag;
            mfma32_v_first<true>(ag, fp8x8_to_bf16(raw[0]), qf[8 * g]);
#pragma unroll
            for (int u = 1; u < 7; ++u) mfma32_v<true>(ag, fp8x8_to_bf16(raw[u]), qf[8 * g + u]);
            mfma32_v_last<true>(ag, fp8x8_to_bf16(raw[7]), qf[8 * g + 7]);
            float sc[16];
            load_scales(g, sc);
#pragma unroll
            for (int i = 0; i < 16; ++i) st[i] = fmaf(sc[i], ag[i], st[i]);
        }

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
        for (int i = 3; i < 16; i += 2) mx = fmaxf(fmaxf(mx, st[i]), st[i + 1]);
        mx = fmaxf(mx, st[15]);
        mx = xhalf_max(mx) * sl2;
        if (m == -INFINITY) {
            m = mx;
        } else if (__any(mx > m + kLag)) {
            const float m_new = fmaxf(m, mx);
            const float alpha = exp2f(m - m_new);
#pragma unroll
            for (int i = 0; i < kDvTiles; ++i) scale_acc(acc[i], alpha);
            l *= alpha;
            m = m_new;
        }
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
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float sc[16];
            load_scales(g, sc);
            bf16x8 pf[2];
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[jj][e] = (__bf16)(st[8 * jj + e] * sc[8 * jj + e]);
            i32x2 vr[4][2];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
                    vr[q][jj] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (MLA_LDS i32x2*)(lt + vt_base + jj * 16 * kRowF + 32 * (4 * g + q)));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int mt = 4 * g + q;
                mfma32_acc<true>(acc[mt], fp8x8_to_bf16(vr[q][0]), pf[0]);
                mfma32_acc<true>(acc[mt], fp8x8_to_bf16(vr[q][1]), pf[1]);
            }
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
