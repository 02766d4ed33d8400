// kda_lds.hpp -- LDS tile helpers for the producer/consumer state passes on
// gfx950: direct global->LDS copies, XOR-swizzled bf16 tiles, and MFMA
// operand fragments read from them.
//
// A swizzled tile [R][C] (bf16, C in {32, 64, 128}) stores row r contiguously
// (2C bytes) with its 16-byte chunks permuted: logical chunk c sits at chunk
// c ^ swz(r).  The permutations are chosen so that the two read patterns used
// on a tile are free of bank conflicts:
//   - row-fragment reads: 16 consecutive rows, 8 bytes each, same column;
//   - transposed reads (ds_read_b64_tr_b16): 4 consecutive rows starting at a
//     multiple of 4, 32 consecutive bytes each.
// A direct copy writes 1 KB of LDS per wavefront instruction (lane L's 16
// bytes at +16 L), so a tile is filled in 1 KB pieces whose lanes fetch the
// global chunk that belongs at their LDS position.
#pragma once

#include "kda_device.hpp"

namespace kda {

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

template <int C>
__device__ __forceinline__ int swz(int r) {
    if constexpr (C == 128) return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8);  // 16 chunks per row
    else if constexpr (C == 64) return (r >> 1) & 7;                           // 8 chunks per row
    else return 0;                                                             // 4 chunks: 4 rows fill the banks
}

// Byte offset of element (r, c) in a swizzled [R][C] bf16 tile.
template <int C>
__device__ __forceinline__ int swz_off(int r, int c) {
    return r * (2 * C) + ((((2 * c) >> 4) ^ swz<C>(r)) << 4) + ((2 * c) & 15);
}

// 16-byte direct copy global -> LDS for this lane; `lds` is the (wavefront
// uniform) LDS base of the instruction's 1 KB piece.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_t*)lds, 16, 0, 0);
}

// Piece q (1 KB) of a [64][C] bf16 tile whose global rows are `pitch`
// elements apart: lane L fills LDS chunk L of the piece.
// Global rows at or past rmax are read from row rmax - 1 instead (the caller
// masks them), so that no access leaves the source rows.
template <int C>
__device__ __forceinline__ void dma_tile_piece(const uint16_t* g, int64_t pitch, uint8_t* lds, int q, int lane,
                                               int rmax = 1 << 30) {
    constexpr int CPR = C / 8;           // 16-byte chunks per row
    constexpr int RPP = 1024 / (2 * C);  // rows per piece
    const int r = q * RPP + lane / CPR;
    const int c = (lane % CPR) ^ swz<C>(r);
    const int rg = r < rmax ? r : rmax - 1;
    dma16(g + rg * pitch + c * 8, lds + q * 1024);
}

// MFMA A fragment (16x16x32, bf16) from a swizzled [R][C] tile, rows m0..m0+15,
// in the permuted contraction order of a register-resident B operand: lane
// group lg = lane / 16 supplies k0 + 4 lg + (0..3) and k0 + 16 + 4 lg + (0..3).
template <int C>
__device__ __forceinline__ bf16x8 frag_rows(const uint8_t* tile, int m0, int k0, int lane) {
    const int r = m0 + (lane & 15), lg = lane >> 4;
    const bf16x4_t lo = *reinterpret_cast<const bf16x4_t*>(tile + swz_off<C>(r, k0 + 4 * lg));
    const bf16x4_t hi = *reinterpret_cast<const bf16x4_t*>(tile + swz_off<C>(r, k0 + 16 + 4 * lg));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Transposed read: in each 16-lane group, lane i receives rows r0 .. r0+3 of
// column c0 + i (r0 a multiple of 4, the group's choice).
template <int C>
__device__ __forceinline__ bf16x4_t tr4(const uint8_t* tile, int r0, int c0, int lane) {
    const int i = lane & 15;
    const uint8_t* a = tile + swz_off<C>(r0 + (i >> 2), c0 + 4 * (i & 3));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)a);
}

// MFMA A fragment of the transpose of a swizzled [R][C] tile: A[m][k] =
// tile[k][m] for m = m0 .. m0+15, permuted contraction order as frag_rows.
template <int C>
__device__ __forceinline__ bf16x8 frag_cols(const uint8_t* tile, int m0, int k0, int lane) {
    const int lg = lane >> 4;
    const bf16x4_t lo = tr4<C>(tile, k0 + 4 * lg, m0, lane);
    const bf16x4_t hi = tr4<C>(tile, k0 + 16 + 4 * lg, m0, lane);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// B fragment from two register-resident accumulator tiles (rows 16 a .. and
// 16 (a+1) .. of the contraction), rounded to bf16: matches frag_rows /
// frag_cols with k0 = 16 a.
__device__ __forceinline__ bf16x8 frag_acc(f32x4 lo, f32x4 hi) {
    return bf16x8{(__bf16)lo[0], (__bf16)lo[1], (__bf16)lo[2], (__bf16)lo[3],
                  (__bf16)hi[0], (__bf16)hi[1], (__bf16)hi[2], (__bf16)hi[3]};
}

// B fragment in the natural MFMA contraction order (lane group g holds k = 8 g
// .. 8 g + 7 of a 32-row k-step) from two accumulator tiles: lo holds rows
// 0..15 of the k-step, hi rows 16..31, each lane rows 4 g .. 4 g + 3 of its
// tile.  Rounded to bf16, then regrouped by a 32-lane and a 16-lane swap.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, bf16x2_t{static_cast<__bf16>(a), static_cast<__bf16>(b)});
}
__device__ __forceinline__ bf16x8 frag_acc_nat(f32x4 lo, f32x4 hi) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(pack_bf16(lo[0], lo[1]), pack_bf16(hi[0], hi[1]), false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(pack_bf16(lo[2], lo[3]), pack_bf16(hi[2], hi[3]), false, false);
    const auto u0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
    const auto u1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
    return __builtin_bit_cast(bf16x8, u32x4_t{u0[0], u1[0], u0[1], u1[1]});
}

// s_waitcnt vmcnt(n) (n < 64), other counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmem() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
__device__ __forceinline__ void wait_vmem_all() { wait_vmem<0>(); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// operations, not for its outstanding global memory operations (direct copies
// into LDS included, which the caller waits for itself as far as needed).
__device__ __forceinline__ void barrier_lds() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace kda
