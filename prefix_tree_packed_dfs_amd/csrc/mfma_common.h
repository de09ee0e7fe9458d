// Device helpers shared by the matrix-core kernels.
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (checked on gfx950 with an
// in-bounds probe): for C = A B with A 32x16 and B 16x32,
//   A: lane l, slot i holds A[l % 32][(l / 32) * 8 + i]
//   B: lane l, slot i holds B[(l / 32) * 8 + i][l % 32]
//   C: lane l, reg r  holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// so a lane of the accumulator owns one column and 16 rows: rows
// {8j + 4h + (0..3)} for j = 0..3, h = l / 32.  Registers 8c..8c+7 of an
// accumulator are therefore a valid B (or A-transposed) operand for the
// 16-row chunk c of the next product, provided the other operand lists those
// 16 rows in the same order: row m of the chunk is stored at position
// phys16(m), which puts lane half h's eight rows next to each other.
#pragma once

#include "device.h"

namespace treeattn {

// Wave issue priority (s_setprio 0 or 1), fenced so that the compiler keeps
// the instructions of a phase on their side of the change.
__device__ __forceinline__ void prio(int level) {
    __builtin_amdgcn_sched_barrier(0);
    if (level) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Position of row m (0..15) of a 16-row chunk in the permuted layout, and back.
__device__ __forceinline__ int phys16(int m) { return ((m >> 2) & 1) * 8 + (m >> 3) * 4 + (m & 3); }
__device__ __forceinline__ int inv_phys16(int w) { return ((w & 7) >> 2) * 8 + (w >> 3) * 4 + (w & 3); }

// Row of accumulator register r for lane half h.
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r] = 0.f;
}

// Position of 16-byte chunk c of a row of D bf16 values in LDS: c ^ row_swizzle<D>(row).
// Two read patterns touch these rows.  Operand loads (ds_read_b128) take one
// chunk of 16 consecutive rows per 16 lanes; transposed loads
// (ds_read_b64_tr_b16) take 4 consecutive rows x 4 consecutive chunks per
// half wave.  With 64 four-byte banks both hit 16 distinct 16-byte bank
// groups: the swizzle is a bijection on row % 16, and the four rows of an
// aligned quad land in four different chunk quads (D = 128: rows of 256
// bytes) or in two chunk quads of the two row parities (D = 64: rows of 128
// bytes, two rows per 256-byte bank window).
template <int D>
__device__ __forceinline__ int row_swizzle(int r) {
    static_assert(D == 64 || D == 128, "head dim");
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Transposed LDS load (checked on gfx950 with an in-bounds probe): in each
// group of 16 lanes, lane i receives element i % 4 of the 8 bytes addressed
// by lanes 4k + i / 4 of the group, k = 0..3, in that order.  Two such loads
// give the 8 values of one MFMA operand: lo fills slots 0-3, hi slots 4-7.
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
__device__ __forceinline__ bf16x8 ld_tr(const void* lo, const void* hi) {
    typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4;
    const bf16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lo));
    const bf16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(hi));
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// LDS loads at 32-bit LDS offsets.  With rows of a multiple of 128 bytes at
// 256-byte aligned bases and chunks swizzled only in bits 4-7, the address of
// chunk c of a row is (base + this lane's chunk-0 offset) XOR 32 c, and row
// blocks, halves and arrays are immediate offsets: one register per array
// instead of one per chunk.
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
__device__ __forceinline__ uint32_t lds_off(const void* p) { return (uint32_t)(uintptr_t)(const lds_char_t*)p; }
__device__ __forceinline__ bf16x8 lds_ld16(uint32_t a) { return *(lds_bf16x8_t*)a; }
__device__ __forceinline__ bf16x8 lds_ld_tr(uint32_t lo, uint32_t hi) {
    const bf16x4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)lo);
    const bf16x4_t y = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)hi);
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Transposed-load offset of this lane for head-dim block 0, first half: the
// lane supplies row 4 (lane / 32) + (lane / 4) % 4 (+ 8 for slots 4-7) and
// column 16 ((lane / 16) % 2) + 4 (lane % 4) (+ 32 per head-dim block).  Block
// db, half h is (offset XOR (64 db + 32 h)) + 8 h rows.
template <int D>
__device__ __forceinline__ uint32_t tr_offset0(int lane) {
    constexpr int ROWB = D * 2;
    const int row = 4 * (lane >> 5) + ((lane >> 2) & 3);
    const int chunk = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return (uint32_t)(row * ROWB + ((chunk ^ row_swizzle<D>(row)) * 16) + 8 * (lane & 1));
}
// The transposed operand of 16 rows starting `rows16` rows into the array at
// LDS offset `base` (= array start + tr_offset0), head-dim block db.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_block(uint32_t base, int db, int rows16) {
    constexpr int ROWB = D * 2;
    return lds_ld_tr((base ^ (64u * db)) + rows16 * ROWB, (base ^ (64u * db + 32u)) + rows16 * ROWB + 8 * ROWB);
}

// First tile index >= from (and <= t_last) whose largest subtree_end reaches
// i0; -1 if none.  Wave-uniform: 64 tiles are tested per step with one ballot.
__device__ __forceinline__ int next_visible(const int32_t* __restrict__ tmaxb, int from, int t_last, int i0) {
    const int lane = threadIdx.x & 63;
    for (int base = from; base <= t_last; base += 64) {
        const int t = base + lane;
        const bool vis = t <= t_last && tmaxb[t] >= i0;
        const unsigned long long m = __ballot(vis);
        if (m) return base + __ffsll((long long)m) - 1;
    }
    return -1;
}

// ---------------------------------------------------------------------------
// Direct global -> LDS loads and explicit synchronisation.
//
// global_load_lds_dwordx4 writes lane i's 16 bytes to LDS at base + 16 * i
// (base is wave-uniform), so one instruction fills 1 KB of LDS and needs no
// registers.  The loads are tracked by vmcnt, which counts in issue order:
// wait_vmcnt<n>() returns once at most n of this wave's vector memory
// operations are still in flight.  __syncthreads() would wait for all of
// them (vmcnt(0)); barrier() does not, so prefetches of later tiles stay in
// flight across it.  Every wave must wait for its own loads before the
// barrier that publishes them.
// ---------------------------------------------------------------------------
// The loads are written as inline assembly: through the compiler builtin,
// the wait-count pass cannot tell the DMA's LDS destination from the stage
// being read and drains every in-flight prefetch (vmcnt(0)) before each LDS
// read.  As assembly they are invisible to that pass; the explicit waits
// below carry the dependency.  Vector memory operations complete in issue
// order, so the compiler's own waits for older loads stay correct.
// LDS byte address of a pointer into shared memory, as a wave-uniform scalar
// (callers pass per-wave bases; readfirstlane puts them in an SGPR for M0).
// The low 32 bits of a generic address inside the LDS aperture are the LDS
// offset, so no address-space cast (and the null test it implies) is needed.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds_addr(lds_base))
                 : "memory");
}
__device__ __forceinline__ void dma4(const void* gsrc, void* lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "s"(lds_addr(lds_base))
                 : "memory");
}

// Same loads from a wave-uniform base (an SGPR pair) plus a 32-bit per-lane
// byte offset: the per-lane part of the address stays in one register.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, void* lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(lds_addr(lds_base))
                 : "memory");
}
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, void* lds_base) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr(lds_base))
                 : "memory");
}

// Lane index recomputed where it is used (volatile: never hoisted or kept in
// a register across a loop, where register pressure would spill it).
__device__ __forceinline__ int lane_id_here() {
    int r;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(r));
    return r;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt low bits [3:0], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// max / sum of a value with the lane 32 positions away (v_permlane32_swap
// exchanges the two halves of a wave without going through LDS).
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace treeattn
