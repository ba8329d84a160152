// MXFP8 encoding of Q, K and V for the MXFP8 forward.
//
// The pages describe an MXFP8 version of the kernel whose products run in
// microscaling precision ("TLX porta l'attenzione jagged su Blackwell"
// (ai-radar.it), section "The turning point") without fixing the format; this
// is OCP MXFP8: E4M3 elements sharing one E8M0 scale per 32 elements along
// the contraction dimension of each product. A block x_1..x_32 gets the
// exponent e = floor(log2 max|x_i|) - 8 (clamped to [-127, 127]; an all-zero
// block takes -127) and elements E4M3(x_i / 2^e), rounded to nearest even,
// magnitudes above 448 clamped. Blocks run along d for Q and K, and along 32
// consecutive keys of one sequence for V.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"

namespace jfa {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// exponent e of a block with largest magnitude amax (finite, >= 0)
__device__ __forceinline__ int block_exp(float amax) {
    const int E = (__float_as_uint(amax) >> 23) & 255;   // 0: zero or below 2^-126
    return E == 0 ? -127 : max(E - 127 - 8, -127);
}

// E4M3 code of x / 2^e (exact scaling; clamped to +-448, then rounded to
// nearest even by the hardware conversion), two values per call
template <bool HI>
__device__ __forceinline__ int pack2(float x0, float x1, int e, int old) {
    const float y0 = fminf(fmaxf(__builtin_ldexpf(x0, -e), -448.0f), 448.0f);
    const float y1 = fminf(fmaxf(__builtin_ldexpf(x1, -e), -448.0f), 448.0f);
    return __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, old, HI);
}

// the same with its own exponent per value
template <bool HI>
__device__ __forceinline__ int pack2_e(float x0, float x1, int e0, int e1, int old) {
    const float y0 = fminf(fmaxf(__builtin_ldexpf(x0, -e0), -448.0f), 448.0f);
    const float y1 = fminf(fmaxf(__builtin_ldexpf(x1, -e1), -448.0f), 448.0f);
    return __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, old, HI);
}

// One thread per 32-element block of a [rows, H, D] tensor (blocks along d):
// codes [rows, H, D], scales [H, rows, D/32].
__global__ void __launch_bounds__(256) quant_rows_kernel(const uint16_t* __restrict__ src, int64_t rows,
                                                         int32_t H, int32_t D, uint8_t* __restrict__ codes,
                                                         uint8_t* __restrict__ scales) {
    const int nb = D / 32;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= rows * H * nb) return;
    const int blk = (int)(idx % nb);
    const int64_t rh = idx / nb;
    const int h = (int)(rh % H);
    const int64_t row = rh / H;
    // [row][h][32 blk .. 32 blk + 31] is element 32 idx onwards
    float x[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const u32x4 v = *(const u32x4*)(src + 32 * idx + 8 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[8 * c + 2 * j] = bf16_to_f32((uint16_t)(v[j] & 0xFFFF));
            x[8 * c + 2 * j + 1] = bf16_to_f32((uint16_t)(v[j] >> 16));
        }
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const int e = block_exp(amax);
    u32x4 out[2];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        int d = pack2<false>(x[4 * w], x[4 * w + 1], e, 0);
        d = pack2<true>(x[4 * w + 2], x[4 * w + 3], e, d);
        out[w >> 2][w & 3] = (uint32_t)d;
    }
    *(u32x4*)(codes + 32 * idx) = out[0];
    *(u32x4*)(codes + 32 * idx + 16) = out[1];
    scales[((int64_t)h * rows + row) * nb + blk] = (uint8_t)(e + 127);
}

// One thread per (32-key block j of the batch, head h, 8 columns g): it finds
// its sequence by binary search over the block offsets, holds the block's
// 32 rows of its 8 columns in registers, takes the column maxima, and writes
// 8 bytes of codes per row and the 8 scale codes. Consecutive threads take
// consecutive columns, then heads, so a wave reads whole key rows. Codes
// [T_k, H, D], scales [H, NB, D].
__global__ void __launch_bounds__(256) quant_v_kernel(const uint16_t* __restrict__ v,
                                                      const int32_t* __restrict__ kv_off,
                                                      const int32_t* __restrict__ boff, int32_t B, int32_t H,
                                                      int32_t D, int32_t nbt, uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
    const int groups = D / 8;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)nbt * H * groups) return;
    const int g = (int)(idx % groups);
    const int h = (int)((idx / groups) % H);
    const int j = (int)(idx / ((int64_t)groups * H));
    // the last sequence b with boff[b] <= j (its blocks [boff[b], boff[b+1]) hold j)
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (boff[mid] <= j) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo, blk = j - boff[b];
    const int k0 = kv_off[b], L = kv_off[b + 1] - k0;
    const int n = min(32, L - 32 * blk);
    const int64_t rs = (int64_t)H * D;
    const int64_t base = (int64_t)(k0 + 32 * blk) * rs + (int64_t)h * D + 8 * g;
    u32x4 x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = i < n ? *(const u32x4*)(v + base + i * rs) : u32x4{0, 0, 0, 0};
    // column maxima of |x| on the bf16 bits (sign cleared; bf16 magnitudes
    // order like their bit patterns)
    uint32_t m[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 32; ++i)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t a = x[i][c] & 0x7FFF7FFFu;
            m[c] = max(m[c] & 0xFFFFu, a & 0xFFFFu) | (max(m[c] >> 16, a >> 16) << 16);
        }
    int e[8];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        e[2 * c] = block_exp(bf16_to_f32((uint16_t)(m[c] & 0xFFFF)));
        e[2 * c + 1] = block_exp(bf16_to_f32((uint16_t)(m[c] >> 16)));
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        if (i < n) {
            uint32_t w[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint32_t lo_ = x[i][2 * q], hi_ = x[i][2 * q + 1];
                int p = pack2_e<false>(bf16_to_f32((uint16_t)(lo_ & 0xFFFF)), bf16_to_f32((uint16_t)(lo_ >> 16)),
                                       e[4 * q], e[4 * q + 1], 0);
                p = pack2_e<true>(bf16_to_f32((uint16_t)(hi_ & 0xFFFF)), bf16_to_f32((uint16_t)(hi_ >> 16)),
                                  e[4 * q + 2], e[4 * q + 3], p);
                w[q] = (uint32_t)p;
            }
            *(uint2*)(codes + base + i * rs) = make_uint2(w[0], w[1]);
        }
    }
    uint32_t sc[2] = {0, 0};
#pragma unroll
    for (int c = 0; c < 8; ++c) sc[c >> 2] |= (uint32_t)(e[c] + 127) << (8 * (c & 3));
    *(uint2*)(scales + ((int64_t)h * nbt + j) * D + 8 * g) = make_uint2(sc[0], sc[1]);
}

}  // namespace

int32_t launch_mx_quant_rows(const uint16_t* src, int64_t rows, int32_t H, int32_t D, uint8_t* codes,
                             uint8_t* scales, void* stream) {
    const int64_t n = rows * H * (D / 32);
    if (n == 0) return 0;
    hipLaunchKernelGGL(quant_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, src, rows, H, D, codes, scales);
    return (int32_t)hipGetLastError();
}

int32_t launch_mx_quant_v(const uint16_t* v, const int32_t* kv_off, const int32_t* boff, int32_t B,
                          int32_t H, int32_t D, int32_t nbt, uint8_t* codes, uint8_t* scales,
                          void* stream) {
    const int64_t n = (int64_t)nbt * H * (D / 8);
    if (B == 0 || n == 0) return 0;
    hipLaunchKernelGGL(quant_v_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, (hipStream_t)stream, v,
                       kv_off, boff, B, H, D, nbt, codes, scales);
    return (int32_t)hipGetLastError();
}

}  // namespace jfa
