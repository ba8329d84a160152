// MXFP8 operand helpers shared by the MXFP8 forward and the MXFP8 dQ pass
// (gfx950 scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with OCP E4M3 data and
// E8M0 block scales; D = 128).
#pragma once

#include "device.h"

namespace jfa {
namespace mxops {

// ---- MXFP8 operands (D = 128, two 64-wide steps j along d). A 16-byte chunk
// c of key r of a K block sits at chunk c ^ ((r >> 1) & 7) (the 16 lanes of a
// read pass, 16 keys, cover all banks); chunk c of row d of a V^T block at
// c ^ ((d >> 2) & 3).
__device__ __forceinline__ int swz_k8(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_vt8(int d) { return (d >> 2) & 3; }
// A natural [64 keys][128 d] block read by mx_pv_tr: chunk c of key r at
// c ^ swz_v8(r). A half wave's transposed reads take 8 keys x 32 bytes
// (keys 16h + 0-3 and 8-11, or 4-7 and 12-15); the even (odd) keys among them
// then sit in 4 different 32-byte spans of a 256-byte bank period.
__device__ __forceinline__ int swz_v8(int r) { return 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1); }
constexpr int kP8Scale = 127 - 8;   // E8M0 code of P's block scale 2^-8

// S^T = K Q^T of a block's two 32-key tiles. Lane (key 32mb + lr, half hf),
// step j: bytes 0-15 hold d 64j + 16hf .. +15 (scale block 2j), bytes 16-31
// d 64j + 32 + 16hf .. +15 (block 2j + 1); the Q fragment uses the same
// slots, and the lane gives the scale of d block 2j + hf.
__device__ __forceinline__ void mx_scores(f32x16 (&acc)[2], const char* kb, const char* ksb,
                                          const i32x8 (&qf)[2], const int (&qsc)[2], int lr, int hf) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int r = 32 * mb + lr;
        const char* row = kb + r * 128;
        const uint32_t ks = *(const uint32_t*)(ksb + 4 * r);
        acc[mb] = f32x16{};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32x4 lo = *(const u32x4*)(row + 16 * ((4 * j + hf) ^ swz_k8(r)));
            const u32x4 hi = *(const u32x4*)(row + 16 * ((4 * j + 2 + hf) ^ swz_k8(r)));
            const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            acc[mb] = mfma_mx(av, qf[j], (ks >> (8 * (2 * j + hf))) & 255, qsc[j], acc[mb]);
        }
    }
}

// P^T (probabilities already exponentiated, at most 1) as the B operand of
// O^T += V^T P^T over a 64-key block (scale block kb = key tile kb), each
// value divided by P's fixed scale 2^-8 and rounded to E4M3. Accumulator
// register r of lane half h holds key 8(r/4) + 4h + r%4: packed four at a
// time (dword g: keys 8g + 4h .. +3) and regrouped across the halves with two
// lane-half swaps, so that half h holds keys 16h .. 16h+15 of each tile, as
// dwords of keys 0-3, 8-11, 4-7, 12-15 (relative to 16h).
__device__ __forceinline__ i32x8 mx_pack_p(const f32x16 (&p)[2]) {
    i32x8 out;
    const float sc = 1.0f / 256.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        uint32_t d[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            d[g] = pack4_fp8(p[mb][4 * g], p[mb][4 * g + 1], p[mb][4 * g + 2], p[mb][4 * g + 3], sc);
        const auto r02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
        const auto r13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
        out[4 * mb + 0] = (int)r02[0];
        out[4 * mb + 1] = (int)r13[0];
        out[4 * mb + 2] = (int)r02[1];
        out[4 * mb + 3] = (int)r13[1];
    }
    return out;
}

// The same packing for values with one scale per 32-key tile (scale[mb] for
// tile mb; callers keep |value / scale| <= 448): the dS^T operand of the
// MXFP8 dQ pass.
__device__ __forceinline__ i32x8 mx_pack_scaled(const f32x16 (&x)[2], const float (&scale)[2]) {
    i32x8 out;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        uint32_t d[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
            d[g] = pack4_fp8(x[mb][4 * g], x[mb][4 * g + 1], x[mb][4 * g + 2], x[mb][4 * g + 3], scale[mb]);
        const auto r02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
        const auto r13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
        out[4 * mb + 0] = (int)r02[0];
        out[4 * mb + 1] = (int)r13[0];
        out[4 * mb + 2] = (int)r02[1];
        out[4 * mb + 3] = (int)r13[1];
    }
    return out;
}

// O^T[d, qrow] += V^T[d, key] P^T[key, qrow]: lane (d = 32md + lr, half hf)
// takes keys 16hf .. +15 (tile 0) and 32 + 16hf .. +15 (tile 1) of row d in
// the dword order of mx_pack_p, and the scale of V block (d, 2n + hf); bsc
// is the E8M0 scale of this lane's P^T block (block hf of its row).
__device__ __forceinline__ void mx_pv(f32x16 (&oacc)[4], const i32x8& pb, const char* vtb,
                                      const char* vsb, int bsc, int lr, int hf) {
#pragma unroll
    for (int md = 0; md < 4; ++md) {
        const int d = 32 * md + lr;
        const char* row = vtb + d * 64;
        const u32x4 lo = *(const u32x4*)(row + 16 * (hf ^ swz_vt8(d)));
        const u32x4 hi = *(const u32x4*)(row + 16 * ((2 + hf) ^ swz_vt8(d)));
        const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                          (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const int vs = *(const uint8_t*)(vsb + hf * 128 + d);
        oacc[md] = mfma_mx(av, pb, vs, bsc, oacc[md]);
    }
}

// mx_pv with the V^T operands read straight from the natural V block (keys
// swizzled by swz_v8) by byte-transposed reads (ds_read_b64_tr_b8: lanes 2e,
// 2e+1 of a 16-lane group address row e, 8 bytes each, and lane i receives
// byte i of the 8 rows). Lane (d = 32md + lr, half hf) needs keys 16hf +
// (0-3, 8-11, 4-7, 12-15) and the same + 32: four reads of 8 keys, at rows
// 16hf + (0-3, 8-11) + {0, 4, 32, 36}. vo[md] is this lane's offset of the
// first read (mx_tr_offsets); the others add 4, 32 and 36 rows.
__device__ __forceinline__ void mx_tr_offsets(int lane, int (&vo)[4]) {
    const int n16 = lane & 15, e = n16 >> 1, g = (lane >> 4) & 1, hf = lane >> 5;
    const int r = 16 * hf + (e < 4 ? e : e + 4);
#pragma unroll
    for (int md = 0; md < 4; ++md) vo[md] = r * 128 + (((2 * md + g) ^ swz_v8(r)) << 4) + 8 * (n16 & 1);
}
__device__ __forceinline__ void mx_pv_tr(f32x16 (&oacc)[4], const i32x8& pb, const char* vb,
                                         const int (&vo)[4], const char* vsb, int bsc, int lr, int hf) {
    typedef int v2i32 __attribute__((vector_size(8)));
    typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
    typedef __attribute__((address_space(3))) const char lds_char;
    const uint32_t base = (uint32_t)(uintptr_t)(lds_char*)vb;
#pragma unroll
    for (int md = 0; md < 4; ++md) {
        const int d = 32 * md + lr;
        v2i32 x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            constexpr int rows[4] = {0, 4, 32, 36};
            x[t] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_v2i32*)((lds_char*)(uintptr_t)(base + vo[md]) + 128 * rows[t]));
        }
        const i32x8 av = {x[0][0], x[0][1], x[1][0], x[1][1], x[2][0], x[2][1], x[3][0], x[3][1]};
        const int vs = *(const uint8_t*)(vsb + hf * 128 + d);
        oacc[md] = mfma_mx(av, pb, vs, bsc, oacc[md]);
    }
}

// V [64 keys][128 d] (E4M3) -> V^T [128 d][64 keys]: thread t transposes the
// 4 x 4 byte tile of keys 4(t/32) .. +3 and d 4(t%32) .. +3 in registers.
// Within each 16-key chunk of a V^T row the four 4-key dwords are stored in
// the order keys 0-3, 8-11, 4-7, 12-15 (relative to the chunk): the dword
// order of the packed P^T operand, so a chunk read is an A operand as is.
__device__ __forceinline__ void mx_transpose_v(const char* v, char* vt, int tid) {
    const int b = tid & 31, aq = tid >> 5;
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = *(const uint32_t*)(v + (4 * aq + i) * 128 + 4 * b);
    // byte i of column j = byte j of row i
    const uint32_t lo01 = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);
    const uint32_t hi01 = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);
    const uint32_t lo23 = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
    const uint32_t hi23 = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
    uint32_t c[4];
    c[0] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
    c[1] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
    c[2] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
    c[3] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int d = 4 * b + j;
        const int g = aq & 3, pos = g == 1 ? 2 : g == 2 ? 1 : g;   // dword order 0, 2, 1, 3
        *(uint32_t*)(vt + d * 64 + 16 * ((aq >> 2) ^ swz_vt8(d)) + 4 * pos) = c[j];
    }
}

}  // namespace mxops
}  // namespace jfa
