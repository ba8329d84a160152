// Pieces shared by the Q-stationary kernels (forward and the backward's dQ
// pass): a workgroup of 8 waves owns a tile of 256 query rows, 32 per wave,
// and streams 64-key K/V blocks of its sequence through LDS with
// direct-to-LDS copies. Each tile's rows meet the keys in the order the host
// plan gives ("Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell With
// 3x Less Code" (ainewsbites.com), sections "What TLX changes" and
// "Optimizations layered on top": persistent programs, multi-buffered K/V).
#pragma once

#include "device.h"
#include "internal.h"

namespace jfa {
namespace qtile {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
static_assert(kFwdBlockM == 32 * kWaves && kFwdBlockN == 64, "Q-tile geometry");

// 16-byte chunk swizzles of LDS tiles (stored chunk = chunk XOR f(row)),
// chosen for LDS reads (64 banks x 4 bytes, 16 lanes per cycle for 16-byte
// reads, 32 for 8-byte ones):
//  - swz_k: rows read as 32x32x16 MFMA A operands (16 lanes = 16 rows, one
//    16-byte chunk each);
//  - swz_rt: rows read that way and also by the transposed reads of
//    tr_operand_offsets (a half wave reads 4 consecutive rows x 64 bytes):
//    a bijection on every 16 rows, with rows 4q .. 4q+3 in different
//    64-byte quarters of the bank space (D = 128: row mod 4 in bits 2-3; D =
//    64, two rows per 256 bytes: rows 4q and 4q + 2 differ in bit 2).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
    return D == 128 ? (r & 15) : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz_rt(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Offsets (within a tile of natural [rows][D] bf16 rows swizzled by swz_rt)
// of the transposed reads (ds_read_b64_tr_b16) that give the 32x32x16 A
// operand X^T[32md + lr][16 rows of chunk c] of a product whose B operand is
// an accumulator fed back: register r of lane half h holds row 8(r/4) + 4h +
// r%4 of its 32, so B's 8 values of chunk c in half h are rows 16c + 4h +
// {0-3, 8-11}, and A must hold the same rows in the same order. Read t (t =
// 0, 1) of this lane's 16-lane group (d span 32md + 16g .. +15) addresses
// rows 16c + 8t + 4h + e, e = 0..3 (lanes 4e .. 4e+3 point at row e, 8
// bytes each); the lane receives its own d at those 4 rows. The swizzle
// depends on the row modulo 16 only, so chunk c adds an immediate 16c rows.
template <int D>
__device__ __forceinline__ void tr_operand_offsets(int lane, int (&off)[2][D / 32]) {
    const int n16 = lane & 15, e = n16 >> 2, cq = n16 & 3, g = (lane >> 4) & 1, h = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int r = 8 * t + 4 * h + e;
#pragma unroll
        for (int md = 0; md < D / 32; ++md)
            off[t][md] = r * D * 2 + (((4 * md + 2 * g + (cq >> 1)) ^ swz_rt<D>(r)) << 4) + 8 * (cq & 1);
    }
}

// Direct-to-LDS copy of 16 bytes per lane: lane l's bytes at g land at
// lds_wave_base + 16 l (lds_wave_base wave-uniform). Issued as inline
// assembly so that the compiler does not treat every later LDS read as
// possibly overlapping the copy (it would wait for all copies in flight
// before each of them); completion is awaited explicitly with wait_vmem()
// or wait_vmem_keep() followed by a workgroup barrier.
__device__ __forceinline__ void load_lds16(const uint16_t* g, char* lds_wave_base) {
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(lds)
        : "memory");
}

// The same copy from sbase + voff bytes: sbase wave-uniform (an SGPR pair,
// the scalar-base form of the instruction), voff this lane's 32-bit byte
// offset, so the lane's address costs no 64-bit vector arithmetic.
__device__ __forceinline__ void load_lds16_s(const void* sbase, uint32_t voff, char* lds_wave_base) {
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
}

// Direct-to-LDS copy of 4 bytes per lane: lane l's dword at g lands at
// lds_wave_base + 4 l (same conventions as load_lds16).
__device__ __forceinline__ void load_lds4(const void* g, char* lds_wave_base) {
    const uint32_t lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)lds_wave_base;
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dword %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(g), "s"(lds)
        : "memory");
}

// One tile of a Q-tile plan (wave-uniform): Q tile t of sequence b, head h,
// visiting positions k0 .. k0+work-1 of the tile's block list (k0 > 0 only
// for a chunk of a split broadcast-Q dQ tile). Banded mode: the list is the
// KV blocks c0, c0+1, ... and wl, wr are the window bounds (-1: none).
struct TileInfo {
    int b, h, t, k0, work, kv0, L, c0, wl, wr;
    const int* sp;   // block-sparse list of the tile (4c + keep bits), else null
};

// chunk_div: 0, or for a chunked plan the number of Q tiles per sequence,
// the record's third field being t + chunk_div * k0
template <int MODE>
__device__ __forceinline__ TileInfo tile_info(const int32_t* tiles, const int32_t* kv_off,
                                              const int32_t* sp_ptr, const int32_t* sp_idx,
                                              int32_t mask_q_blocks, int chunk_div, int win_left,
                                              int win_right, int ti) {
    TileInfo T;
    T.b = ld_uniform(tiles + 4 * ti + 0);
    T.h = ld_uniform(tiles + 4 * ti + 1);
    const int f2 = ld_uniform(tiles + 4 * ti + 2);
    T.t = chunk_div > 0 ? f2 % chunk_div : f2;
    T.k0 = chunk_div > 0 ? f2 / chunk_div : 0;
    T.work = ld_uniform(tiles + 4 * ti + 3);
    T.kv0 = ld_uniform(kv_off + T.b);
    T.L = ld_uniform(kv_off + T.b + 1) - T.kv0;
    T.sp = nullptr;
    if (MODE == kSparse) T.sp = sp_idx + ld_uniform(sp_ptr + T.b * ((mask_q_blocks + 1) >> 1) + T.t);
    T.wl = win_left;
    T.wr = win_right;
    T.c0 = 0;   // the first key the tile's rows see, in blocks
    if (MODE == kCausal && win_left >= 0) T.c0 = max(0, T.t * kFwdBlockM - win_left) / kFwdBlockN;
    return T;
}

// 64-key block of the sequence visited at position i of a tile
template <int MODE>
__device__ __forceinline__ int seq_block(const TileInfo& T, int i) {
    if (MODE == kSparse) return 2 * (ld_uniform(T.sp + (i >> 1)) >> 2) + (i & 1);
    if (MODE == kCausal) return T.c0 + i;
    return i;
}

// Which blocks a wave takes and which need the tail masks: rows row0 ..
// row0+31 of the wave, block n of the sequence (position i of the tile).
template <int MODE>
__device__ __forceinline__ void block_flags(const TileInfo& T, int i, int n, int row0, bool wave_rows,
                                            int wave, bool& skip, bool& masked) {
    skip = !wave_rows;
    if (MODE == kCausal) {
        // rows R0..R1 see keys [R0 - wl, R1 + wr]; every row sees the whole
        // block [K0, K1] iff K0 >= R1 - wl and K1 <= R0 + wr
        const int64_t R0 = row0, R1 = row0 + 31, K0 = (int64_t)kFwdBlockN * n, K1 = K0 + kFwdBlockN - 1;
        skip = skip || (T.wr >= 0 && K0 > R1 + T.wr) || (T.wl >= 0 && K1 < R0 - T.wl);
        masked = (T.wr >= 0 && K1 > R0 + T.wr) || (T.wl >= 0 && K0 < R1 - T.wl) ||
                 kFwdBlockN * (n + 1) > T.L;
    } else {
        masked = kFwdBlockN * (n + 1) > T.L;
        if (MODE == kSparse) skip = skip || !((ld_uniform(T.sp + (i >> 1)) >> (wave >> 2)) & 1);
    }
}

}  // namespace qtile
}  // namespace jfa
