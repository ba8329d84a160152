// Jagged FlashAttention backward for gfx950: preprocess and the KV-stationary
// dK/dV pass (the dQ pass is Q-stationary, in its own kernel).
//
//   1. preprocess: delta = rowsum(dO * O) in fp32 (the standard FlashAttention
//      backward step; the pages only name the backward's persistent, tiled
//      structure: "Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell"
//      (ainewsbites.com), section "Optimizations layered on top");
//   2. dK/dV: one persistent workgroup per worker walking a KV-tile plan. A
//      workgroup owns a 128-key KV tile (32 keys per wave) and streams the
//      64-row Q/dO blocks that see it; dK and dV are accumulated per KV tile
//      in registers and written once, as whole rows through LDS.
//
// Per Q block and wave (keys on lanes, query rows in registers):
//   S   = Q K^T          A = Q rows from LDS,    B = K (registers)
//   P   = exp2(S*scale*log2e - LSE*log2e)
//   dP  = dO V^T         A = dO rows from LDS,   B = V rows from LDS
//   dS  = P * (dP - delta)
//   dV^T += dO^T P       A = dO^T from LDS (rows in sigma order), B = P
//   dK^T += Q^T dS       A = Q^T from LDS (rows in sigma order),  B = dS
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace jfa {
namespace {

constexpr int kThreads = 256;
constexpr int kPad = 8;

// LDS layout. Tiles whose rows are read as MFMA operands by 16 lanes at a
// time are laid out so that those 16 rows hit distinct banks:
//  - natural [row][D] tiles (Q, dO, and at tile start K, V; at tile end the
//    dK/dV staging): 16-byte chunk c of row r is stored at chunk c ^ swz(r),
//    swz(r) = (r + r/CH) mod CH, CH = D/8 chunks per row;
//  - Q^T, dO^T: [d][64 rows] padded by 16 bytes per row;
//  - rows of Q^T/dO^T are stored in the "sigma" order of each 16-group (0-3,
//    8-11, 4-7, 12-15), so that the 8 values one lane feeds to a 32x32x16
//    MFMA (rows 16c + sigma(8h..8h+7)) are one 16-byte read and match the
//    accumulator registers they are multiplied with.
// Region R holds the Q-block tiles during the loop, the natural K tile during
// the tile prologue, and the dK/dV staging in the tile epilogue. The natural
// V tile stays in its own region for the whole tile (its rows are the B
// operand of dP = dO V^T).
template <int D>
struct BwdLds {
    static constexpr int R = 0;
    static constexpr int QN = R;                                    // [64][D]
    static constexpr int DN = QN + kBwdBlockM * D * 2;              // [64][D]
    static constexpr int QT = DN + kBwdBlockM * D * 2;              // [D][72]
    static constexpr int DT = QT + D * (kBwdBlockM + 8) * 2;        // [D][72]
    static constexpr int KN = R;                                    // [128][D]
    static constexpr int DKS = R;                                   // [128][D] (epilogue)
    static constexpr int DVS = R + kBwdBlockN * D * 2;              // [128][D] (epilogue)
    static constexpr int R_BYTES = (DT + D * (kBwdBlockM + 8) * 2 - R) > 2 * kBwdBlockN * D * 2
                                       ? (DT + D * (kBwdBlockM + 8) * 2 - R)
                                       : 2 * kBwdBlockN * D * 2;
    static constexpr int VN = R + R_BYTES;                          // [128][D]
    static constexpr int LSE = VN + kBwdBlockN * D * 2;
    static constexpr int DELTA = LSE + kBwdBlockM * 4;
    static constexpr int BYTES = DELTA + kBwdBlockM * 4;
};

// position of row q (within its group of 16) in sigma order
__device__ __forceinline__ int sigma_pos(int q) {
    const int g = (q >> 2) & 3;
    return (q & ~15) | (((g >> 1) | ((g & 1) << 1)) << 2) | (q & 3);
}

template <int D>
__device__ __forceinline__ int swz(int r) {
    constexpr int CH = D / 8;
    constexpr int SH = (D == 128) ? 4 : 3;
    return (r + (r >> SH)) & (CH - 1);
}

// byte offset of element (row r, element c8*8 + e) of a natural [row][D] tile
template <int D>
__device__ __forceinline__ int nat_off(int r, int chunk) {
    return r * D * 2 + ((chunk ^ swz<D>(r)) << 4);
}

// 4 rows x 8 bf16 (one 16-byte chunk per row) -> 8 columns x 4 rows
__device__ __forceinline__ void transpose4x8(const u32x4 (&x)[4], u32x2 (&y)[8]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        y[2 * k][0] = (x[0][k] & 0xffffu) | (x[1][k] << 16);
        y[2 * k][1] = (x[2][k] & 0xffffu) | (x[3][k] << 16);
        y[2 * k + 1][0] = (x[0][k] >> 16) | (x[1][k] & 0xffff0000u);
        y[2 * k + 1][1] = (x[2][k] >> 16) | (x[3][k] & 0xffff0000u);
    }
}

template <int D, int MODE, bool BCAST>
__global__ void __launch_bounds__(kThreads) dkdv_kernel(BwdArgs a) {
    using LY = BwdLds<D>;
    __shared__ __attribute__((aligned(16))) char smem[LY::BYTES];
    constexpr int KC = D / 16;
    constexpr int MD = D / 32;
    constexpr int CH = D / 8;
    constexpr int KPP = 4 * (kThreads / CH);       // keys per pass of the tile loader
    constexpr int KPASS = kBwdBlockN / KPP;        // 2 (D=128) or 1 (D=64)
    auto lds = [&](int byte_off) -> char* { return smem + byte_off; };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;
    // Q/dO block loader: 4 rows (4qg..4qg+3) x one 16-byte chunk dc per thread
    const int ld_qg = tid & 15, ld_dc = tid >> 4;
    const bool ld_on = ld_dc < CH;
    // K/V tile loader: chunk tdc of keys 4tkg..4tkg+3 (+KPP per pass); a load
    // instruction covers whole 16*CH-byte rows
    const int tdc = tid % CH, tkg = tid / CH;

    // per-lane pieces of the swizzled addresses of natural rows 32mb + lr
    int nat_base[2], nat_x[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * mb + lr;
        const int sw = swz<D>(row);
        nat_base[mb] = row * D * 2 + 16 * (hf ^ (sw & 1));
        nat_x[mb] = sw >> 1;
    }
    // natural K/V tile rows of this lane's key (row 32*wave + lr)
    int kv_base, kv_x;
    {
        const int row = 32 * wave + lr;
        const int sw = swz<D>(row);
        kv_base = row * D * 2 + 16 * (hf ^ (sw & 1));
        kv_x = sw >> 1;
    }

    const int w = worker_id(a.num_workers);
    const int t_begin = ld_uniform(a.worker_ptr + w), t_end = ld_uniform(a.worker_ptr + w + 1);

    for (int ti = t_begin; ti < t_end; ++ti) {
        const int b = ld_uniform(a.tiles + 4 * ti + 0);
        const int hd = ld_uniform(a.tiles + 4 * ti + 1);
        const int n = ld_uniform(a.tiles + 4 * ti + 2);
        const int work = ld_uniform(a.tiles + 4 * ti + 3);
        const int kv0 = ld_uniform(a.kv_off + b);
        const int L = ld_uniform(a.kv_off + b + 1) - kv0;
        int q0, Lq, orow0;
        if (BCAST) {
            q0 = 0;
            Lq = a.lq;
            orow0 = b * a.lq;
        } else {
            q0 = ld_uniform(a.q_off + b);
            Lq = ld_uniform(a.q_off + b + 1) - q0;
            orow0 = q0;
        }
        const int* sp = nullptr;
        if (MODE == kSparse) sp = a.sp_idx + ld_uniform(a.sp_ptr + b * a.mask_kv_blocks + n);
        const int r0 = (MODE == kCausal) ? (n * kBwdBlockN) / kBwdBlockM : 0;
        auto qblk = [&](int i) -> int {
            if (MODE == kSparse) return 2 * ld_uniform(sp + (i >> 1)) + (i & 1);
            return r0 + i;
        };
        const int nmasked = (MODE == kCausal) ? min(2, work) : 0;
        const int key = n * kBwdBlockN + wave * 32 + lr;   // local key of this lane
        const int64_t kvrow0 = (int64_t)kv0 * rs + (int64_t)hd * D;

        // Q / dO / LSE / delta of a block: global -> registers (raw values only:
        // any arithmetic on a loaded value here would make the wave wait for
        // the whole prefetch right away) -> LDS at the end of the iteration
        u32x4 qv[4], dv[4];
        float rowv = 0.f;
        int ld_r = 0;   // Q block of the registers, for the zero fill at store time
        auto gload = [&](int r) {
            // unconditional loads from a row clamped into the sequence (Lq >= 1
            // whenever a block exists); rows past the end are zeroed in sstore
            ld_r = r;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int qi = min(r * kBwdBlockM + 4 * ld_qg + p, Lq - 1);
                qv[p] = *(const u32x4*)(a.q + (int64_t)(q0 + qi) * rs + (int64_t)hd * D + 8 * (ld_dc & (CH - 1)));
                dv[p] = *(const u32x4*)(a.d_o + (int64_t)(orow0 + qi) * rs + (int64_t)hd * D + 8 * (ld_dc & (CH - 1)));
            }
            {
                // wave 0 loads LSE, wave 1 delta (a wave-uniform choice keeps the
                // base pointers scalar)
                const int qi = min(r * kBwdBlockM + lane, Lq - 1);
                const int64_t idx = (int64_t)hd * a.total_q + orow0 + qi;
                if (wave == 0) rowv = a.lse[idx];
                else if (wave == 1) rowv = a.delta[idx];
            }
        };
        auto sstore = [&]() {
            if (ld_on) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    if (ld_r * kBwdBlockM + 4 * ld_qg + p >= Lq) {
                        qv[p] = u32x4{};
                        dv[p] = u32x4{};
                    }
                }
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int o = nat_off<D>(4 * ld_qg + p, ld_dc);
                    *(u32x4*)lds(LY::QN + o) = qv[p];
                    *(u32x4*)lds(LY::DN + o) = dv[p];
                }
                u32x2 y[8];
                const int pos2 = 2 * sigma_pos(4 * ld_qg);
                transpose4x8(qv, y);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(u32x2*)lds(LY::QT + (8 * ld_dc + e) * (kBwdBlockM + 8) * 2 + pos2) = y[e];
                transpose4x8(dv, y);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    *(u32x2*)lds(LY::DT + (8 * ld_dc + e) * (kBwdBlockM + 8) * 2 + pos2) = y[e];
            }
            // LSE in the exp2 domain; a row without keys (LSE = -inf) or outside
            // the sequence gets +inf so that its P is 0
            const bool in_seq = ld_r * kBwdBlockM + lane < Lq;
            if (wave == 0)
                ((float*)lds(LY::LSE))[lane] = (!in_seq || rowv == -INFINITY) ? INFINITY : rowv * kLog2e;
            else if (wave == 1)
                ((float*)lds(LY::DELTA))[lane] = in_seq ? rowv : 0.f;
        };

        // ---- tile prologue: the K and V tiles are loaded as whole rows, stored
        // to LDS, then each wave reads its K fragments; block 0 is loaded
        // meanwhile
        {
            u32x4 kx[KPASS][4], vx[KPASS][4];
#pragma unroll
            for (int pass = 0; pass < KPASS; ++pass)
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int kk = min(n * kBwdBlockN + KPP * pass + 4 * tkg + p, L - 1);
                    kx[pass][p] = *(const u32x4*)(a.k + kvrow0 + (int64_t)kk * rs + 8 * tdc);
                    vx[pass][p] = *(const u32x4*)(a.v + kvrow0 + (int64_t)kk * rs + 8 * tdc);
                }
#pragma unroll
            for (int pass = 0; pass < KPASS; ++pass) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int kl = KPP * pass + 4 * tkg + p;   // key within the tile
                    if (n * kBwdBlockN + kl >= L) {
                        kx[pass][p] = u32x4{};
                        vx[pass][p] = u32x4{};
                    }
                    const int o = nat_off<D>(kl, tdc);
                    *(u32x4*)lds(LY::KN + o) = kx[pass][p];
                    *(u32x4*)lds(LY::VN + o) = vx[pass][p];
                }
            }
        }
        __syncthreads();
        if (work > 0) gload(qblk(0));
        // this wave's K rows as MFMA B operands (keys on lanes); its V rows are
        // read from LDS where they are used
        bf16x8 kf[KC];
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
            kf[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)lds(LY::KN + kv_base + 32 * (kc ^ kv_x)));
        f32x16 dk_acc[MD], dv_acc[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) {
            dk_acc[md] = f32x16{};
            dv_acc[md] = f32x16{};
        }
        __syncthreads();   // region R changes from K/V to the Q-block tiles
        if (work > 0) sstore();
        // block 0 landed; nothing left in flight (see wait_vmem)
        wait_vmem();
        __syncthreads();

        auto body = [&](int i, auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int r = qblk(i);
            if (i + 1 < work) gload(qblk(i + 1));

            // the block in two halves of 32 query rows (mb), to keep the live
            // register set small
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const int off = nat_base[mb] + 32 * (kc ^ nat_x[mb]);
                    const bf16x8 qa = __builtin_bit_cast(bf16x8, *(const u32x4*)lds(LY::QN + off));
                    s = mfma32(qa, kf[kc], s);
                    const bf16x8 da = __builtin_bit_cast(bf16x8, *(const u32x4*)lds(LY::DN + off));
                    const bf16x8 vb =
                        __builtin_bit_cast(bf16x8, *(const u32x4*)lds(LY::VN + kv_base + 32 * (kc ^ kv_x)));
                    dp = mfma32(da, vb, dp);
                }
                // P and dS; register r is query row 32mb + 8(r/4) + 4hf + r%4
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = 32 * mb + 8 * g + 4 * hf;
                    const f32x4 l4 = *(const f32x4*)lds(LY::LSE + 4 * row);
                    const f32x4 d4 = *(const f32x4*)lds(LY::DELTA + 4 * row);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float p = __builtin_amdgcn_exp2f(s[4 * g + j] * a.scale_log2 - l4[j]);
                        if (MASKED) {
                            if (key > r * kBwdBlockM + row + j) p = 0.f;
                        }
                        s[4 * g + j] = p;
                        dp[4 * g + j] = p * (dp[4 * g + j] - d4[j]);
                    }
                }
                // dV^T += dO^T P ; dK^T += Q^T dS over this half's 32 query rows
                // (16-row chunks c = 2mb, 2mb + 1)
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int c = 2 * mb + cc;
                    f32x8 x, y;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        x[j] = s[8 * cc + j];
                        y[j] = dp[8 * cc + j];
                    }
                    const bf16x8 pb = to_bf16x8(x), sb = to_bf16x8(y);
#pragma unroll
                    for (int md = 0; md < MD; ++md) {
                        const int o = (32 * md + lr) * (kBwdBlockM + 8) * 2 + (16 * c + 8 * hf) * 2;
                        const bf16x8 da = __builtin_bit_cast(bf16x8, *(const u32x4*)lds(LY::DT + o));
                        dv_acc[md] = mfma32(da, pb, dv_acc[md]);
                        const bf16x8 qa = __builtin_bit_cast(bf16x8, *(const u32x4*)lds(LY::QT + o));
                        dk_acc[md] = mfma32(qa, sb, dk_acc[md]);
                    }
                }
            }
            // every wave is done with this block's tiles before they are replaced
            __syncthreads();
            if (i + 1 < work) sstore();
            __syncthreads();
        };

        int i = 0;
        for (; i < nmasked; ++i) body(i, std::true_type{});
        for (; i < work; ++i) body(i, std::false_type{});

        // ---- tile epilogue: stage dK = scale * (dK^T)^T and dV (bf16) in region
        // R as natural rows, then write whole rows to global memory
        {
            const int row = wave * 32 + lr;
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 x, y;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        x[j] = dk_acc[md][4 * g + j] * a.scale;
                        y[j] = dv_acc[md][4 * g + j];
                    }
                    const int o = nat_off<D>(row, 4 * md + g) + 8 * hf;
                    *(u32x2*)lds(LY::DKS + o) = __builtin_bit_cast(u32x2, to_bf16x4(x));
                    *(u32x2*)lds(LY::DVS + o) = __builtin_bit_cast(u32x2, to_bf16x4(y));
                }
        }
        __syncthreads();
#pragma unroll
        for (int pass = 0; pass < KPASS; ++pass)
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int kl = KPP * pass + 4 * tkg + p;
                const int o = nat_off<D>(kl, tdc);
                const u32x4 xk = *(const u32x4*)lds(LY::DKS + o);
                const u32x4 xv = *(const u32x4*)lds(LY::DVS + o);
                if (n * kBwdBlockN + kl < L) {
                    const int64_t g = kvrow0 + (int64_t)(n * kBwdBlockN + kl) * rs + 8 * tdc;
                    *(u32x4*)(a.dk + g) = xk;
                    *(u32x4*)(a.dv + g) = xv;
                }
            }
        // LDS is rewritten by the next tile
        __syncthreads();
    }
}

// delta[h, row] = sum_d dO[row,h,d] * O[row,h,d] in fp32.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ d_o,
                                                      float* __restrict__ delta, int64_t rows_h,
                                                      int32_t H, int32_t total_q) {
    constexpr int LPR = D / 8;  // lanes per (row, head)
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    const int64_t groups = nthreads / LPR;
    const int sub = threadIdx.x % LPR;
    // every lane runs the same trip count so the shuffles see a full wave
    for (int64_t base = 0; base < rows_h; base += groups) {
        const int64_t rh = base + gtid / LPR;
        float acc = 0.f;
        if (rh < rows_h) {
            const u32x4 x = *(const u32x4*)(o + rh * D + sub * 8);
            const u32x4 y = *(const u32x4*)(d_o + rh * D + sub * 8);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                acc += __uint_as_float(x[j] << 16) * __uint_as_float(y[j] << 16);
                acc += __uint_as_float(x[j] & 0xffff0000u) * __uint_as_float(y[j] & 0xffff0000u);
            }
        }
#pragma unroll
        for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
        if (rh < rows_h && sub == 0) {
            const int64_t row = rh / H;
            const int h = (int)(rh % H);
            delta[(int64_t)h * total_q + row] = acc;
        }
    }
}

template <int D, int MODE, bool BCAST>
int32_t launch_main(const BwdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((dkdv_kernel<D, MODE, BCAST>), dim3(a.num_workers), dim3(kThreads), 0, s, a);
    return (int32_t)hipGetLastError();
}

template <int D>
int32_t launch_d(const BwdArgs& a, Mode mode, bool bcast, int32_t stages, hipStream_t s) {
    const int64_t rows_h = (int64_t)a.total_q * a.num_heads;
    if ((stages & JFA_BWD_PREPROCESS) && rows_h > 0) {
        const int64_t want = (rows_h * (D / 8) + 255) / 256;
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, 4096));
        hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(grid), dim3(256), 0, s, a.o, a.d_o, a.delta,
                           rows_h, a.num_heads, a.total_q);
        const int32_t e = (int32_t)hipGetLastError();
        if (e) return e;
    }
    if ((stages & JFA_BWD_DKDV) && a.num_workers > 0) {
        int32_t e;
        if (mode == kCausal) e = launch_main<D, kCausal, false>(a, s);
        else if (mode == kSparse)
            e = bcast ? launch_main<D, kSparse, true>(a, s) : launch_main<D, kSparse, false>(a, s);
        else
            e = bcast ? launch_main<D, kDense, true>(a, s) : launch_main<D, kDense, false>(a, s);
        if (e) return e;
    }
    return 0;
}

}  // namespace

int32_t launch_bwd(const BwdArgs& a, int32_t head_dim, Mode mode, bool broadcast, int32_t stages,
                   void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (head_dim == 64) return launch_d<64>(a, mode, broadcast, stages, s);
    return launch_d<128>(a, mode, broadcast, stages, s);
}

}  // namespace jfa
