// Device-side building blocks shared by the forward and backward kernels:
// vector types, the 32x32 MFMA wrappers, buffer and LDS-direct copies, the
// LDS tile layouts and their operand reads, and the workgroup maps.
//
// MFMA register layouts used throughout (CDNA3/CDNA4 32x32 shapes, wave64):
//   A operand (M x K):  lane l holds row m = l % 32, k-group l / 32.
//   B operand (K x N):  lane l holds col n = l % 32, k-group l / 32.
//   C/D (M x N, 16 f32 per lane): item t of lane l is
//       row m = (t / 4) * 8 + (l / 32) * 4 + (t % 4),  col n = l % 32.
// Only the A/B agreement on which (lane-group, slot) meets which k matters
// for a product, so every operand pair below is loaded with one mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_launch.h"

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// 2^x on the hardware transcendental unit (v_exp_f32): -inf -> 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^x on the FMA pipe instead of the transcendental unit ("FlashAttention
// 1～4 全解汇总", FlashAttention-4, software-emulated exponential): x = n + f
// with n = floor(x) and f in [0, 1); 2^f by a degree-3 polynomial in Horner
// form whose coefficients minimise the maximum relative error on [0, 1] (a
// Remez exchange fit, exp2_poly.py beside this package: |p(f) / 2^f - 1| <=
// 7.5e-5, far below bf16's 2^-9 rounding of P); 2^n goes into the exponent
// with ldexp.  x is first raised to -200 (NaN kept), so -inf -- a masked
// score -- and anything below -150 give exactly 0.
__device__ __forceinline__ float exp2_poly(float x) {
    x = x < -200.f ? -200.f : x;
    const float n = floorf(x);
    const float f = x - n;
    float p = fmaf(0x1.3f96a4p-4f, f, 0x1.cefc4cp-3f);
    p = fmaf(p, f, 0x1.64444cp-1f);
    p = fmaf(p, f, 0x1.fff632p-1f);
    return ldexpf(p, (int)n);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ u32x4 ldg128(const void* p) { return *(const u32x4*)p; }

// Raw buffer resource over `bytes` bytes at `base`.  Loads through it return
// zero for any 16-byte chunk at or past `bytes`, which is how ragged tails are
// read without branches.  (Word 3 = 0x00020000: 32-bit raw data format.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16-byte buffer load at byte offset voff (per lane) + soff (uniform).
__device__ __forceinline__ u32x4 buf_load128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// A 16-byte-per-lane HBM -> LDS copy (buffer_load_dwordx4 ... lds: lane l's
// data lands at the LDS address in M0 + 16*l, no VGPRs) issued through
// inline asm, so the compiler's memory-wait analysis does not see it: with
// the builtin form it would wait for the copy before every LDS read and
// every barrier, since it cannot tell which LDS buffer the copy fills.
// Completion MUST be awaited explicitly with vmem_wait_all() before any
// wave reads the destination.
//   rsrc: raw buffer descriptor words (wave-uniform);
//   lds_addr: LDS byte address of lane 0's 16 bytes (wave-uniform).
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(p);
}

__device__ __forceinline__ void async_load_lds16(i32x4 rsrc, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
    // M0 holds the LDS destination; it is bound as an input operand, so the
    // compiler writes it and knows the statement reads it.  The compiler's
    // hazard checks do not look inside the statement, so it starts with the
    // wait states the load needs itself: 1 after an SALU write of M0 and 5
    // after a VALU write (v_readfirstlane / v_readlane) of an SGPR it reads.
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory");
}

// Eight such copies in one statement: 1 KiB each to LDS addresses
// lds_addr, lds_addr + STEP, ... (STEP >= 1024: consecutive pieces, or
// pieces with padding between them) from per-lane offsets off[i] + soff.
// M0 is a tied input/output operand: the compiler writes lds_addr into it
// before the statement, the statement steps it by STEP per copy, and the
// compiler regards it as changed afterwards.  The compiler's hazard checks
// do not look inside the statement, so it pays the wait states itself:
// 5 up front (a VALU write of an SGPR operand -- v_readfirstlane -- before
// a buffer load that reads it) and 1 after each M0 step (an SALU write of M0
// before an LDS-direct load), as gfx950 requires.
template <uint32_t STEP = 1024>
__device__ __forceinline__ void async_load_lds16_x8(i32x4 rsrc, uint32_t lds_addr, const uint32_t (&off)[8],
                                                    uint32_t soff) {
    uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %[o0], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o1], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o2], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o3], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o4], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o5], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o6], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o7], %[rs], %[so] offen lds"
        : [m0] "+{m0}"(m0)
        : [o0] "v"(off[0]), [o1] "v"(off[1]), [o2] "v"(off[2]), [o3] "v"(off[3]), [o4] "v"(off[4]),
          [o5] "v"(off[5]), [o6] "v"(off[6]), [o7] "v"(off[7]), [rs] "s"(rsrc), [so] "s"(soff), [st] "i"(STEP)
        : "memory", "scc");
}

// The same for four copies.
template <uint32_t STEP = 1024>
__device__ __forceinline__ void async_load_lds16_x4(i32x4 rsrc, uint32_t lds_addr, const uint32_t (&off)[4],
                                                    uint32_t soff) {
    uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %[o0], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o1], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o2], %[rs], %[so] offen lds\n\t"
        "s_add_u32 m0, m0, %[st]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[o3], %[rs], %[so] offen lds"
        : [m0] "+{m0}"(m0)
        : [o0] "v"(off[0]), [o1] "v"(off[1]), [o2] "v"(off[2]), [o3] "v"(off[3]), [rs] "s"(rsrc), [so] "s"(soff),
          [st] "i"(STEP)
        : "memory", "scc");
}

__device__ __forceinline__ void vmem_wait_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cache warm-up: one 4-byte load per lane from rsrc at voff + soff, written
// to the 256-byte LDS area at sink_lds (lane l's bytes at sink_lds + 4*l;
// nothing reads it), so that the 128-byte line holding it is in the L2 when
// a copy asks for it later.  An LDS-destination load needs no VGPR to hold
// its result while in flight.  It is counted by vmcnt like the copies, and
// vector memory operations complete in issue order, so a wait for a copy
// issued after it waits for it too: issue it where that wait comes late
// anyway, and await it before the workgroup can end.  Out-of-range offsets
// read nothing (the buffer range check).  Wait states as in async_load_lds16.
__device__ __forceinline__ void l2_touch(i32x4 rsrc, uint32_t sink_lds, uint32_t voff, uint32_t soff) {
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dword %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(__builtin_amdgcn_readfirstlane(sink_lds))
        : "memory");
}

// An empty statement that reads `x`.  The compiler's wait analysis does not
// treat an explicit s_waitcnt as completing the loads it tracks, but it does
// place its own wait before an instruction that reads their results and then
// regards them as complete.  Reading every register loaded before a tile
// loop, at a point where the hardware has already waited for them (after the
// prologue's vmcnt(0)), keeps it from putting waits inside the loop, where
// the hardware counter also counts the asynchronous copies of the next tile.
template <typename T>
__device__ __forceinline__ void mark_loaded(const T& x) {
    asm volatile("" ::"v"(x));
}

// Workgroup barrier between LDS phases of the tile loops.  The scheduling
// barriers keep every instruction on its side of it, whatever the machine
// scheduler's alias reasoning about the asynchronous copies (which it cannot
// see) would allow.
__device__ __forceinline__ void tile_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
}

// ds_read_b64_tr_b16 (gfx950): inside each 16-lane group, lane i receives
// element i%4 of the 8 bytes read by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const void* p) {
    typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 v4bf;
    typedef __attribute__((address_space(3))) v4bf lds_v4bf;
    const v4bf r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_v4bf*)(p));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 concat8(bf16x4 lo, bf16x4 hi) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r[i] = lo[i];
        r[i + 4] = hi[i];
    }
    return r;
}

// v_permlane32_swap exchanges the two 32-lane halves; the pair it returns
// holds {x[l], x[l ^ 32]} in every lane, so max / sum over the pair combine a
// lane with its partner in the other half without touching LDS.
__device__ __forceinline__ float xhalf_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ u32x4 zero_u32x4() {
    u32x4 z;
    z[0] = z[1] = z[2] = z[3] = 0u;
    return z;
}

// ---------------------------------------------------------------------------
// LDS tiles of D-wide bf16 rows ([rows][D], row-major, 16-byte chunks
// permuted per row).  The permutation is chosen so that (a) 16 consecutive
// rows read at one logical chunk (ds_read_b128 of an MFMA A operand: lane =
// row, 8 consecutive columns) and (b) 4 consecutive rows x 4 consecutive
// chunks (one 32-lane half of a ds_read_b64_tr_b16 transposed read) each land
// on distinct bank groups, so both access patterns are conflict-free.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ uint32_t tile_swizzle(uint32_t row) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 128) {
        return ((row & 3u) << 2) | ((row >> 2) & 3u);
    } else {
        const uint32_t j = row >> 1;
        return ((j & 1u) << 2) | ((j >> 1) & 3u);
    }
}

// Byte offset of logical 16-byte chunk `chunk` of row `row` in such a tile.
template <int D>
__device__ __forceinline__ uint32_t tile_offset(uint32_t row, uint32_t chunk) {
    return row * (D * 2) + ((chunk ^ tile_swizzle<D>(row)) << 4);
}

// Transposed operand read from a swizzled tile: for the 16-row k-step
// starting at row r0 and the 32 columns starting at c0, returns the MFMA
// A operand whose lane l holds column c0 + l%32 at the 8 rows the 32x32
// accumulator layout hands out for k-group l/32:
//   rows r0 + 4g + {0..3} and r0 + 8 + 4g + {0..3},  g = l / 32.
// (Two ds_read_b64_tr_b16: inside each 16-lane group, lane i receives
// element i%4 of the 8 bytes read by lanes 4e + i/4, e = 0..3.)
template <int D>
__device__ __forceinline__ bf16x8 tile_read_tr(const char* tile, uint32_t r0, uint32_t c0, int lane) {
    const uint32_t gi = lane & 15, hg = (lane >> 5) & 1;
    const uint32_t row = r0 + 4 * hg + (gi >> 2);
    const uint32_t col = c0 + (lane & 16) + 4 * (gi & 3);
    const bf16x4 lo = lds_read_tr16(tile + tile_offset<D>(row, col >> 3) + (col & 4) * 2);
    const bf16x4 hi = lds_read_tr16(tile + tile_offset<D>(row + 8, col >> 3) + (col & 4) * 2);
    return concat8(lo, hi);
}

// Row read: lane l gets the 8 columns 8*(2*kk + l/32) .. +7 of row r0 + l%32
// (the MFMA A operand of a product over the tile's columns).
template <int D>
__device__ __forceinline__ bf16x8 tile_read_row(const char* tile, uint32_t r0, int kk, int lane) {
    return *(const bf16x8*)(tile + tile_offset<D>(r0 + (lane & 31), 2 * kk + ((lane >> 5) & 1)));
}

// Asynchronous copy of ROWS x D bf16 rows of a contiguous [N][D] array into
// a swizzled LDS tile by WAVES waves (`wave` must be wave-uniform, e.g. from
// readfirstlane, so the LDS addresses stay scalar): each wave moves LOADS 1 KiB pieces
// (64 lanes x 16 bytes), lane by lane in LDS order, fetching the logical
// chunk the swizzle puts there.  Rows past the buffer resource's end read
// as zero.  Completion must be awaited with vmem_wait_all() and a barrier.
template <int D, int ROWS, int WAVES>
struct TileCopy {
    static constexpr int BYTES = ROWS * D * 2;
    static constexpr int LOADS = BYTES / 1024 / WAVES;
    static_assert(BYTES % (1024 * WAVES) == 0, "tile splits into whole 1 KiB pieces per wave");
    uint32_t goff[LOADS];
    uint32_t lds_off;
    __device__ __forceinline__ TileCopy(int wave, int lane) {
        lds_off = (uint32_t)(wave * LOADS) * 1024u;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const uint32_t lin = (uint32_t)((wave * LOADS + i) * 1024 + lane * 16);
            const uint32_t row = lin / (D * 2), pch = (lin % (D * 2)) / 16;
            goff[i] = row * (D * 2) + ((pch ^ tile_swizzle<D>(row)) << 4);
        }
    }
    // Copy rows [row0, row0 + ROWS) of the array behind `rsrc` into the tile
    // at LDS byte address `dst` (wave-uniform, like `wave`).  The row offset
    // goes into the scalar offset: on gfx950 the raw-buffer range check
    // covers per-lane offset + scalar offset, dword by dword (checked on the
    // device), so rows past the end still read as zero.
    __device__ __forceinline__ void issue(const i32x4& rsrc, int row0, uint32_t dst) const {
        const uint32_t soff = (uint32_t)row0 * D * 2;
        if constexpr (LOADS == 8) {
            async_load_lds16_x8(rsrc, dst + lds_off, goff, soff);
        } else if constexpr (LOADS == 4) {
            async_load_lds16_x4(rsrc, dst + lds_off, goff, soff);
        } else {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) async_load_lds16(rsrc, dst + lds_off + i * 1024, goff[i], soff);
        }
    }
};

// ---------------------------------------------------------------------------
// LDS tiles of 128-wide bf16 rows with immediate operand offsets (the d = 128
// forward kernel).  A tile of R rows is R/4 pieces of 1 KiB; piece p holds
// rows p, p + R/4, p + 2R/4, p + 3R/4, each as 256 contiguous bytes, and the
// pieces lie PS bytes apart:
//   offset(row, chunk) = (row % (R/4)) * PS + 256 * (row / (R/4)) + 16 * chunk.
// Then
//   * one asynchronous copy (64 lanes x 16 bytes to consecutive LDS
//     addresses) fills one piece, and each 16-lane group of it reads one
//     whole 256-byte row from HBM;
//   * the MFMA A-operand row read (lane = row r0 + l%32, chunk 2kk + l/32)
//     and the transposed read (tile_read_tr's lanes) are a per-lane base
//     plus an offset that depends only on the k-step and column block, so
//     every operand address in a loop is base register + immediate;
//   * with PS = kLinPieceK = 1040 the row reads of 16 consecutive rows hit
//     16 distinct 16-byte bank groups (consecutive rows are consecutive
//     pieces, 1040 = 65 * 16), and with PS = kLinPieceV = 1088 each 32-lane
//     half of a transposed read covers the 64 banks once (1088 = 136 * 8).
// K and the query tile use the first stride, V the second.
// ---------------------------------------------------------------------------
constexpr uint32_t kLinPieceK = 1040, kLinPieceV = 1088;

template <int ROWS, uint32_t PS>
constexpr int lin_tile_bytes() {
    static_assert(ROWS % 4 == 0, "whole pieces");
    return ROWS / 4 * (int)PS;
}

// Byte offset of logical chunk `chunk` (16 bytes) of row `row`.
template <int ROWS, uint32_t PS>
__device__ __forceinline__ uint32_t lin_offset(uint32_t row, uint32_t chunk) {
    constexpr uint32_t NP = ROWS / 4;
    return (row % NP) * PS + 256 * (row / NP) + 16 * chunk;
}

// Per-lane base of the row read: lin_offset(l%32, l/32).
template <int ROWS, uint32_t PS>
__device__ __forceinline__ uint32_t lin_row_base(int lane) {
    return lin_offset<ROWS, PS>(lane & 31, (lane >> 5) & 1);
}

// Row read (as tile_read_row): lane l gets the 8 columns 8*(2*kk + l/32) ..
// +7 of row r0 + l%32; `p` = tile + lin_row_base(lane), r0 a multiple of 32.
template <int ROWS>
__device__ __forceinline__ bf16x8 lin_read_row(const char* p, uint32_t r0, int kk) {
    return *(const bf16x8*)(p + 256 * (r0 / (ROWS / 4)) + 32 * kk);
}

// Per-lane base of the transposed read on a 64-row tile: the address
// tile_read_tr's lane reads for r0 = c0 = 0 (row 4*(l/32) + (l%16)/4,
// column 16*((l/16)%2) + 4*(l%4), 8 bytes).
template <uint32_t PS>
__device__ __forceinline__ uint32_t lin_tr_base(int lane) {
    const uint32_t gi = lane & 15, hg = (lane >> 5) & 1, g16 = (lane >> 4) & 1;
    const uint32_t col = 16 * g16 + 4 * (gi & 3);
    return lin_offset<64, PS>(4 * hg + (gi >> 2), col >> 3) + (col & 4) * 2;
}

// Transposed read (as tile_read_tr) on a 64-row tile: the A operand whose
// lane l holds column c0 + l%32 at rows r0 + 4g + {0..3} and r0 + 8 + 4g +
// {0..3}, g = l/32; `p` = tile + lin_tr_base(lane), r0 a multiple of 16, c0
// of 32.
template <uint32_t PS>
__device__ __forceinline__ bf16x8 lin_read_tr(const char* p, uint32_t r0, uint32_t c0) {
    const char* q = p + 256 * (r0 / 16) + 2 * c0;
    return concat8(lds_read_tr16(q), lds_read_tr16(q + 8 * PS));
}

// Asynchronous copy of ROWS x 128 bf16 rows into such a tile by WAVES waves
// (the TileCopy interface): wave w fills pieces w*LOADS .. +LOADS-1.
template <int ROWS, int WAVES, uint32_t PS>
struct LinTileCopy {
    static constexpr int NP = ROWS / 4;
    static constexpr int LOADS = NP / WAVES;
    static_assert(NP % WAVES == 0 && (LOADS == 4 || LOADS == 8), "whole pieces, 4 or 8 per wave");
    uint32_t goff[LOADS];
    uint32_t lds_off;
    __device__ __forceinline__ LinTileCopy(int wave, int lane) {
        lds_off = (uint32_t)(wave * LOADS) * PS;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const uint32_t row = (uint32_t)(wave * LOADS + i) + NP * (uint32_t)(lane >> 4);
            goff[i] = row * 256 + 16 * (uint32_t)(lane & 15);
        }
    }
    __device__ __forceinline__ void issue(const i32x4& rsrc, int row0, uint32_t dst) const {
        const uint32_t soff = (uint32_t)row0 * 256;
        if constexpr (LOADS == 8) async_load_lds16_x8<PS>(rsrc, dst + lds_off, goff, soff);
        else async_load_lds16_x4<PS>(rsrc, dst + lds_off, goff, soff);
    }
};

// Workgroup id -> (batch*head, tile index), for total = (batch*head count) x
// n_tiles workgroups.  Consecutive workgroup ids go to the 8 XCDs round
// robin, so ids are regrouped to give each XCD a contiguous run of heads
// (their K/V, or Q/dO, then share that XCD's L2).  Within the run, the tiles
// of two consecutive heads alternate: 0 of head 2g, 0 of head 2g+1, 1 of 2g,
// ...  Callers issue the heaviest causal tile first, so the heavy tiles of
// both heads start before the light ones of either; the light tiles then
// fill the slots that free up at the end instead of one head's last heavy
// tiles running alone (a greedy-dispatch model of one XCD gives a tail of
// 10% of the run with one head at a time, none with two).  An odd last head
// keeps its own order.
//
// unequal: the tiles' work falls from index 0 (causal tiles, heaviest first,
// not paired).  Unless every XCD's run is whole two-head groups (batch*head
// count a multiple of 16), runs cut into such groups would give one XCD the
// heavy tiles of a group and the next its light ones; then the XCDs take
// equal runs of mirrored pairs instead (tiles j and n-1-j of a head: equal
// causal work), head-major: an XCD's workgroups first take the heavy tile of
// each pair of its run in order, then the light tiles in reverse order, so
// the lightest tiles fill the end.  Needs an even tile count and a multiple
// of 16 workgroups (whole pairs per XCD); otherwise the map above is kept.
__device__ __forceinline__ void map_head_tile(int w, int total, int n_tiles, int& bh, int& tile,
                                              bool unequal = false) {
    if (unequal && (total & 15) == 0 && (n_tiles & 1) == 0 && (total >> 3) % (2 * n_tiles) != 0) {
        const int per = total >> 3, half = per >> 1, l = w >> 3, np = n_tiles >> 1;
        const bool heavy = l < half;
        const int u = (w & 7) * half + (heavy ? l : per - 1 - l);   // pair, head-major
        bh = u / np;
        const int j = u - bh * np;
        tile = heavy ? j : n_tiles - 1 - j;
        return;
    }
    int L = w;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        L = (w & 7) * per + (w >> 3);
    }
    const int n_heads = total / n_tiles;
    const int g = L / (2 * n_tiles), r = L - g * 2 * n_tiles;
    if (2 * g + 1 < n_heads) {
        bh = 2 * g + (r & 1);
        tile = r >> 1;
    } else {
        bh = 2 * g;
        tile = r;
    }
}

// Lengths of one (batch, head)'s sequence and its first rows in the
// [rows, d] views of the tensors.
struct SeqGeometry {
    int Nq, Nk;
    size_t q_row0, k_row0;
};

// Workgroup w of a variable-length launch with n_slots tiles per (batch,
// head) pair.  The pairs (batch-major, b*H + h) are taken in chunks of
// kVarlenChunk; within a chunk the ids run slot-major: slot 0 of every pair
// of the chunk, then slot 1, ...  So each pair's tiles are spread
// kVarlenChunk ids apart -- close enough that several of them run at once
// and share the pair's K/V in L2 -- and, kVarlenChunk being a multiple of 8,
// a pair stays on one XCD while the pairs of a chunk (the heads of one or
// two sequences) spread over all eight.  Within a chunk each pair's heavy
// causal tiles come first.  (Slot-major over all pairs measured 1.39x
// slower on a 32-sequence batch: a pair's tiles were B*H ids apart, never
// resident together, so each re-read its K/V from HBM.)
// (32, 64 and 128 measured within 2% of each other on batches of 32
// sequences of 67..8078 tokens and of 128 sequences of 64..995.)
constexpr int kVarlenChunk = 64;

__device__ __forceinline__ void varlen_slot(const VarlenParams& v, int n_slots, int w, int& bh,
                                            int& slot) {
    const int pairs = v.B * v.H;
    const int c = w / (kVarlenChunk * n_slots);             // chunk
    const int r = w - c * kVarlenChunk * n_slots;
    const int in_chunk = min(kVarlenChunk, pairs - c * kVarlenChunk);
    slot = r / in_chunk;
    bh = c * kVarlenChunk + (r - slot * in_chunk);
}

// The geometry of (batch, head) bh of a variable-length batch.  Offsets are
// clamped into [0, total] and lengths to the stated maxima, so that
// inconsistent offsets cannot move any access outside the tensors (the
// results for such a sequence are then unspecified).
__device__ __forceinline__ SeqGeometry seq_geometry(const VarlenParams& v, int bh) {
    const int b = bh / v.H, h = bh - b * v.H;
    const int qs = min(max(v.cu_q[b], 0), v.total_q), qe = min(max(v.cu_q[b + 1], qs), v.total_q);
    const int ks = min(max(v.cu_k[b], 0), v.total_k), ke = min(max(v.cu_k[b + 1], ks), v.total_k);
    SeqGeometry g;
    g.Nq = min(qe - qs, v.max_q);
    g.Nk = min(ke - ks, v.max_k);
    g.q_row0 = (size_t)h * v.total_q + qs;
    g.k_row0 = (size_t)h * v.total_k + ks;
    return g;
}

}  // namespace fa
