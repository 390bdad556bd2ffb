// Helpers shared by the matrix-core decode kernels (gfx950): operand types,
// inline-asm MFMA forms with explicit accumulator placement, direct
// global->LDS loads, explicit vmcnt waits, cross-half reductions.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mla {
namespace mfma {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;

#define MLA_LDS __attribute__((address_space(3)))

constexpr int kSub = 32;                   // tokens per sub-tile
constexpr int kDvTiles = kLatent / 32;     // 16 32-dim tiles of the output
constexpr int kQLatSteps = kLatent / 16;   // 32 K-steps over the latent dims

// vmcnt-only wait (expcnt / lgkmcnt left at their maxima), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Score-product MFMAs with the accumulator in VGPRs.  The output
// accumulators fill the AGPR file, and the compiler would otherwise place
// this accumulator there too and shuttle output tiles through VGPRs.
// Back-to-back accumulation into the same registers needs no wait states;
// the last MFMA of a chain is followed by enough NOPs for a VALU read of the
// result (an 8-pass XDL write needs 11).
//
// FRESH = an A or B operand may have been written by a VALU instruction
// right before (e.g. fp8 codes widened in registers).  The hardware does not
// interlock a VALU write against a following MFMA read of the same VGPR (two
// wait states are required); the compiler pads its own MFMAs but cannot see
// into asm, so these forms lead with two NOP cycles.
template <bool FRESH = false>
__device__ __forceinline__ void mfma32_v_first(f32x16& c, const bf16x8& a, const bf16x8& b) {
    if constexpr (FRESH)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
template <bool FRESH = false>
__device__ __forceinline__ void mfma32_v(f32x16& c, const bf16x8& a, const bf16x8& b) {
    if constexpr (FRESH)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
template <bool FRESH = false>
__device__ __forceinline__ void mfma32_v_last(f32x16& c, const bf16x8& a, const bf16x8& b) {
    if constexpr (FRESH)
        asm volatile(
            "s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
            "s_nop 7\n\ts_nop 7\n\ts_nop 7"
            : "+v"(c)
            : "v"(a), "v"(b));
    else
        asm volatile(
            "v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\t"
            "s_nop 7\n\ts_nop 7\n\ts_nop 7"
            : "+v"(c)
            : "v"(a), "v"(b));
}

// Output-product MFMA with the accumulator pinned to AGPRs.  Issued as
// inline asm so the whole 256-register output accumulator stays in the AGPR
// file.  FRESH as above (operands converted in registers just before).
template <bool FRESH = false>
__device__ __forceinline__ void mfma32_acc(f32x16& c, const bf16x8& a, const bf16x8& b) {
    if constexpr (FRESH)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// Wait states between an asm MFMA chain into c and the first VALU read of
// c.  c is a tied operand, so the compiler cannot move a reader above it.
__device__ __forceinline__ void mfma_result_wait(f32x16& c) {
    asm volatile("s_nop 7\n\ts_nop 3" : "+v"(c));
}

// Wait states after the last asm MFMA writes before ordinary code reads the
// accumulators (the compiler does not see the asm as an MFMA).
__device__ __forceinline__ void mfma_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// max / sum of x over lanes i and i ^ 32 (one cross-half VALU swap)
__device__ __forceinline__ float xhalf_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One wave-wide direct-to-LDS load: lane i copies 16 bytes from
// gbase + voff(i) (gbase uniform, in SGPRs) to LDS byte lds_base + 16 i.  Issued as inline asm so the
// compiler does not see an LDS write in flight: it would otherwise wait for
// every outstanding load (vmcnt 0) before each LDS transpose read.  The
// waits that order these loads before their LDS readers are explicit
// (wait_vm + barrier).  M0 holds the LDS base; writing M0 needs one wait
// state before the load.
__device__ __forceinline__ void dma16(const void* gbase, int voff, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(gbase), "s"(lds_base)
        : "memory", "m0");
}

// f(integral_constant<int, K>) for K = K0 .. K1 - 1, unrolled at compile time
template <int K0, int K1, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (K0 < K1) {
        f(std::integral_constant<int, K0>{});
        static_for<K0 + 1, K1>(f);
    }
}

// The same load with the LDS base given as a uniform register plus a
// compile-time byte offset, summed straight into M0.
template <int IMM>
__device__ __forceinline__ void dma16_at(const void* gbase, int voff, uint32_t lds_base) {
    asm volatile(
        "s_add_u32 m0, %2, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voff), "s"(gbase), "s"(lds_base), "n"(IMM)
        : "memory", "m0", "scc");
}

// Per-lane 64-bit global address, LDS base in a register plus a
// compile-time offset.
template <int IMM>
__device__ __forceinline__ void dma16_v_at(const void* gptr, uint32_t lds_base) {
    asm volatile(
        "s_add_u32 m0, %1, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gptr), "s"(lds_base), "n"(IMM)
        : "memory", "m0", "scc");
}

// One wave-wide 4-byte direct-to-LDS load: lane i copies 4 bytes from
// gbase + voff(i) to LDS byte lds_base + IMM + 4 i.
template <int IMM>
__device__ __forceinline__ void dma4_at(const void* gbase, int voff, uint32_t lds_base) {
    asm volatile(
        "s_add_u32 m0, %2, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %0, %1"
        :
        : "v"(voff), "s"(gbase), "s"(lds_base), "n"(IMM)
        : "memory", "m0", "scc");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((const MLA_LDS void*)p));
}

// Same load with a 64-bit per-lane global address (gathered rows).
__device__ __forceinline__ void dma16_v(const void* gptr, uint32_t lds_base) {
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gptr), "s"(lds_base)
        : "memory", "m0");
}

// A finite, all-zero row: the load source for sub-tiles whose block id is
// invalid (their scores are masked; zeros keep 0 * value finite).
__device__ const __attribute__((aligned(16))) uint8_t kZeroRow[1152] = {};

// acc *= a for one 16-register accumulator tile held in AGPRs.  Written as
// register moves + a multiply so the accumulators never leave the AGPR file.
__device__ __forceinline__ void scale_acc(f32x16& acc, float a) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        float x = acc[e];
        float tmp;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(x), "=&v"(tmp)
            : "v"(a));
        acc[e] = x;
    }
}

// The bf16 output rows of one wave (32 heads x 512 values, O = acc * inv)
// leave through LDS so that global stores write whole 512-byte or 1 KB runs
// of head rows: acc[mt][4 q4 + e] holds dimension 32 mt + 8 q4 + 4 half + e
// of head `col`.  PASSES splits the dimensions (1: all 512 at once, 32 KB of
// LDS per wave; 2: 256 at a time, 16 KB).  `stage` is this wave's region;
// 16-byte chunk c of staged row r sits at chunk c ^ r, so the 8-byte writes
// of one instruction spread over the banks and a read returns contiguous
// row bytes.  Every lane takes part in every step (no lane-dependent
// branch), and LDS accesses of one wave complete in order, so the passes
// need no barrier; the caller makes sure no other wave still reads the
// region.  `out` points at the wave's first head row.
template <int PASSES>
__device__ __forceinline__ void store_rows_bf16(const f32x16 (&acc)[kDvTiles], float inv,
                                                MLA_LDS uint8_t* stage, uint16_t* out, int lane) {
    static_assert(PASSES == 1 || PASSES == 2, "dimension passes");
    constexpr int kRB = 1024 / PASSES;        // bytes of a staged row
    constexpr int kCh = kRB / 16;             // 16-byte chunks per staged row
    constexpr int kMt = kDvTiles / PASSES;    // output tiles per pass
    constexpr int kRowsPerOp = 64 / kCh;      // staged rows per 64-lane read
    const int col = lane & 31, half = lane >> 5;
    MLA_LDS uint8_t* wrow = stage + col * kRB + 8 * half;
    const int rsub = lane / kCh, j = lane % kCh;
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
#pragma unroll
        for (int mt = 0; mt < kMt; ++mt)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x16& a = acc[pass * kMt + mt];
                i32x2 w;
                w[0] = int(bf16x2_rne(a[4 * q4 + 0] * inv, a[4 * q4 + 1] * inv));
                w[1] = int(bf16x2_rne(a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv));
                *(MLA_LDS i32x2*)(wrow + (((4 * mt + q4) ^ col) << 4)) = w;
            }
#pragma unroll
        for (int k = 0; k < 32 / kRowsPerOp; ++k) {
            const int r = k * kRowsPerOp + rsub;
            const i32x4 v = *(const MLA_LDS i32x4*)(stage + r * kRB + ((j ^ r) << 4));
            *reinterpret_cast<i32x4*>(out + size_t(r) * kLatent + pass * (kLatent / PASSES) + 8 * j) = v;
        }
    }
}

// O^T tiles of one wave (32 heads x NT 32-dim tiles, scaled by inv) to bf16
// rows out + r * kLatent for heads r < rows: each lane packs its values
// into a per-head row of the staging area (16-byte chunks XOR-swizzled by
// the head), then every lane stores 16 contiguous bytes of a row.
template <int NT>
__device__ __forceinline__ void store_tiles_bf16(const f32x16 (&acc)[NT], float inv,
                                                 MLA_LDS uint8_t* stage, uint16_t* out, int rows,
                                                 int lane) {
    static_assert(NT == 4 || NT == 8 || NT == 16, "output tiles per wave");
    constexpr int kRB = NT * 64;            // bytes of a staged row
    constexpr int kCh = kRB / 16;           // 16-byte chunks per staged row
    constexpr int kRowsPerOp = 64 / kCh;    // staged rows per 64-lane read
    const int col = lane & 31, half = lane >> 5;
    MLA_LDS uint8_t* wrow = stage + col * kRB + 8 * half;
    const int rsub = lane / kCh, j = lane % kCh;
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x16& a = acc[mt];
            i32x2 w;
            w[0] = int(bf16x2_rne(a[4 * q4 + 0] * inv, a[4 * q4 + 1] * inv));
            w[1] = int(bf16x2_rne(a[4 * q4 + 2] * inv, a[4 * q4 + 3] * inv));
            *(MLA_LDS i32x2*)(wrow + (((4 * mt + q4) ^ (col & (kCh - 1))) << 4)) = w;
        }
#pragma unroll
    for (int k = 0; k < 32 / kRowsPerOp; ++k) {
        const int r = k * kRowsPerOp + rsub;
        const i32x4 v = *(const MLA_LDS i32x4*)(stage + r * kRB + ((j ^ (r & (kCh - 1))) << 4));
        if (r < rows) *reinterpret_cast<i32x4*>(out + size_t(r) * kLatent + 8 * j) = v;
    }
}

// Growth of a head's running max (log2 units) tolerated before the
// accumulators are rescaled: probabilities are formed against a reference
// max that may lag the true running max by at most this much, so they stay
// below 2^kLag; O and the normaliser share the reference, so the result is
// unchanged.
constexpr float kLag = 8.f;

}  // namespace mfma
}  // namespace mla
