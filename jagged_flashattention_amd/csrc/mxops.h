// MXFP8 operand helpers shared by the MXFP8 forward, dQ and dK/dV passes
// (gfx950 scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4 with OCP E4M3 data and
// E8M0 block scales; D = 128).
#pragma once

#include "device.h"

namespace jfa {
namespace mxops {

// ---- MXFP8 operands (D = 128, two 64-wide steps j along d). A 16-byte chunk
// c of key r of a K block sits at chunk c ^ ((r >> 1) & 7) (the 16 lanes of a
// read pass, 16 keys, cover all banks).
__device__ __forceinline__ int swz_k8(int r) { return (r >> 1) & 7; }
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

// O^T[d, qrow] += V^T[d, key] P^T[key, qrow] over a 64-key block, P^T packed
// by mx_pack_p (lane half hf: keys 16hf .. +15 of each 32-key tile, dwords
// of keys 0-3, 8-11, 4-7, 12-15), V's scale that of block (d, 2n + hf); bsc
// is the E8M0 scale of this lane's P^T block. The V^T operands are read
// straight from the natural V block (keys swizzled by swz_v8) by
// byte-transposed reads (ds_read_b64_tr_b8: lanes 2e,
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
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
__device__ __forceinline__ void mx_pv_tr(f32x16 (&oacc)[4], const i32x8& pb, const char* vb,
                                         const int (&vo)[4], const char* vsb, int bsc, int lr, int hf) {
    const uint32_t base = lds_addr(vb);
#pragma unroll
    for (int md = 0; md < 4; ++md) {
        const int d = 32 * md + lr;
        const uint32_t a = base + vo[md];
        const i32x2 x0 = lds_read_tr8_at(a, 0), x1 = lds_read_tr8_at(a, 4 * 128);
        const i32x2 x2 = lds_read_tr8_at(a, 32 * 128), x3 = lds_read_tr8_at(a, 36 * 128);
        const i32x8 av = {x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
        const int vs = *(const uint8_t*)(vsb + hf * 128 + d);
        oacc[md] = mfma_mx(av, pb, vs, bsc, oacc[md]);
    }
}

}  // namespace mxops
}  // namespace jfa
