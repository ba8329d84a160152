// Jagged FlashAttention backward for gfx950.
//
// Three launches in stream order:
//   1. preprocess: delta = rowsum(dO * O) in fp32, dq_accum cleared;
//   2. main: one persistent workgroup per worker walking a KV-tile plan.
//      A workgroup owns a 128-key KV tile (32 keys per wave) and streams the
//      64-row Q/dO blocks that see it. dK and dV are accumulated per KV tile
//      in registers. dS of the whole tile is staged through LDS and the
//      workgroup's dQ partial for the Q block (all 128 keys reduced inside
//      the MFMA) is added into the fp32 dq_accum;
//   3. convert: dq = bf16(dq_accum).
// In broadcast-Q mode every KV tile of every sequence adds into the same
// [lq, H, D] dQ: the contended cross-program reduction the pages single out
// as the main backward bottleneck ("Meta's 3.2K-line Triton kernel outruns
// FlashAttention-4 on jagged Blackwell attention" (theclarity.today), second
// paragraph; "Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell"
// (ainewsbites.com), section "Optimizations layered on top", multi-stage dQ
// staging).
//
// Per Q block and wave (keys on lanes, query rows in registers):
//   S   = Q K^T          A = Q rows from LDS,    B = K (registers)
//   P   = exp2(S*scale*log2e - LSE*log2e)
//   dP  = dO V^T         A = dO rows from LDS,   B = V (registers)
//   dS  = P * (dP - delta)
//   dV^T += dO^T P       A = dO^T via transposed LDS reads, B = P
//   dK^T += Q^T dS       A = Q^T via transposed LDS reads,  B = dS
//   dQ   = dS K          A = dS via transposed reads of the staged dS^T,
//                        B = K via transposed reads of the K tile
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace jfa {
namespace {

constexpr int kThreads = 256;
constexpr int kPad = 8;

template <int D>
struct BwdSmem {
    uint16_t k[kBwdBlockN][D + kPad];            // K tile, row-major
    uint16_t q[2][kBwdBlockM][D + kPad];         // Q block, double-buffered
    uint16_t dout[2][kBwdBlockM][D + kPad];      // dO block, double-buffered
    uint16_t dst[kBwdBlockN][kBwdBlockM + kPad]; // dS^T of the tile (bf16)
    float lse[2][kBwdBlockM];                    // LSE*log2(e); +inf = no row
    float delta[2][kBwdBlockM];
};

template <int D, int MODE, bool BCAST>
__global__ void __launch_bounds__(kThreads) bwd_kernel(BwdArgs a) {
    __shared__ BwdSmem<D> sm;
    constexpr int KC = D / 16;
    constexpr int MD = D / 32;
    constexpr int CPR = D / 8;
    constexpr int RPP = kThreads / CPR;       // rows per load pass
    constexpr int NPQ = kBwdBlockM / RPP;     // passes for a 64-row block
    constexpr int NPK = kBwdBlockN / RPP;     // passes for the 128-key tile
    constexpr int QS = D + kPad;              // LDS row strides (elements)
    constexpr int SS = kBwdBlockM + kPad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;
    const int g16 = lane >> 4, n16 = lane & 15;
    const int tr_row = 4 * (g16 >> 1) + (n16 >> 2);
    const int tr_col = (g16 & 1) * 16 + 4 * (n16 & 3);
    const int ld_row = tid / CPR, ld_col = (tid % CPR) * 8;

    const int w = worker_id(a.num_workers);
    const int t_begin = a.worker_ptr[w], t_end = a.worker_ptr[w + 1];

    for (int ti = t_begin; ti < t_end; ++ti) {
        const int b = a.tiles[4 * ti + 0];
        const int hd = a.tiles[4 * ti + 1];
        const int n = a.tiles[4 * ti + 2];
        const int work = a.tiles[4 * ti + 3];
        const int kv0 = a.kv_off[b];
        const int L = a.kv_off[b + 1] - kv0;
        int q0, Lq, orow0;
        if (BCAST) {
            q0 = 0;
            Lq = a.lq;
            orow0 = b * a.lq;
        } else {
            q0 = a.q_off[b];
            Lq = a.q_off[b + 1] - q0;
            orow0 = q0;
        }
        const int* sp = nullptr;
        if (MODE == kSparse) sp = a.sp_idx + a.sp_ptr[b * a.mask_kv_blocks + n];
        const int r0 = (MODE == kCausal) ? (n * kBwdBlockN) / kBwdBlockM : 0;
        auto qblk = [&](int i) -> int {
            if (MODE == kSparse) return 2 * sp[i >> 1] + (i & 1);
            return r0 + i;
        };
        const int nmasked = (MODE == kCausal) ? min(2, work) : 0;

        // K tile into LDS; this wave's K and V rows into registers
        const int key = n * kBwdBlockN + wave * 32 + lr;   // local key of this lane
#pragma unroll
        for (int p = 0; p < NPK; ++p) {
            const int kk = n * kBwdBlockN + ld_row + p * RPP;
            u32x4 x = u32x4{};
            if (kk < L) x = *(const u32x4*)(a.k + (int64_t)(kv0 + kk) * rs + (int64_t)hd * D + ld_col);
            *(u32x4*)&sm.k[ld_row + p * RPP][ld_col] = x;
        }
        bf16x8 kf[KC], vf[KC];
        if (key < L) {
            const int64_t off = (int64_t)(kv0 + key) * rs + (int64_t)hd * D + 8 * hf;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                kf[kc] = load_bf16x8(a.k + off + 16 * kc);
                vf[kc] = load_bf16x8(a.v + off + 16 * kc);
            }
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                kf[kc] = bf16x8{};
                vf[kc] = bf16x8{};
            }
        }
        f32x16 dk_acc[MD], dv_acc[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) {
            dk_acc[md] = f32x16{};
            dv_acc[md] = f32x16{};
        }

        // Q / dO / LSE / delta block loader (registers, then LDS)
        u32x4 qr[NPQ], dr[NPQ];
        float rowv = 0.f;
        auto gload = [&](int r) {
#pragma unroll
            for (int p = 0; p < NPQ; ++p) {
                const int qi = r * kBwdBlockM + ld_row + p * RPP;
                if (qi < Lq) {
                    qr[p] = *(const u32x4*)(a.q + (int64_t)(q0 + qi) * rs + (int64_t)hd * D + ld_col);
                    dr[p] = *(const u32x4*)(a.d_o + (int64_t)(orow0 + qi) * rs + (int64_t)hd * D + ld_col);
                } else {
                    qr[p] = u32x4{};
                    dr[p] = u32x4{};
                }
            }
            if (tid < 2 * kBwdBlockM) {
                const int qi = r * kBwdBlockM + (tid & (kBwdBlockM - 1));
                const bool is_lse = tid < kBwdBlockM;
                if (qi < Lq) {
                    const int64_t idx = (int64_t)hd * a.total_q + orow0 + qi;
                    if (is_lse) {
                        const float l = a.lse[idx];
                        rowv = (l == -INFINITY) ? INFINITY : l * kLog2e;
                    } else {
                        rowv = a.delta[idx];
                    }
                } else {
                    rowv = is_lse ? INFINITY : 0.f;
                }
            }
        };
        auto sstore = [&](int buf) {
#pragma unroll
            for (int p = 0; p < NPQ; ++p) {
                *(u32x4*)&sm.q[buf][ld_row + p * RPP][ld_col] = qr[p];
                *(u32x4*)&sm.dout[buf][ld_row + p * RPP][ld_col] = dr[p];
            }
            if (tid < kBwdBlockM) sm.lse[buf][tid] = rowv;
            else if (tid < 2 * kBwdBlockM) sm.delta[buf][tid - kBwdBlockM] = rowv;
        };

        if (work > 0) {
            gload(qblk(0));
            sstore(0);
        }
        __syncthreads();

        auto body = [&](int i, auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int buf = i & 1;
            const int r = qblk(i);
            if (i + 1 < work) gload(qblk(i + 1));

            f32x16 s[2], dp[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                s[mb] = f32x16{};
                dp[mb] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const bf16x8 qa = load_bf16x8(&sm.q[buf][32 * mb + lr][16 * kc + 8 * hf]);
                    s[mb] = mfma32(qa, kf[kc], s[mb]);
                }
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const bf16x8 da = load_bf16x8(&sm.dout[buf][32 * mb + lr][16 * kc + 8 * hf]);
                    dp[mb] = mfma32(da, vf[kc], dp[mb]);
                }
            }
            // P and dS; register r of block mb is query row 32mb + 8(r/4) + 4hf + r%4
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int row = 32 * mb + 8 * g + 4 * hf;
                    const f32x4 l4 = *(const f32x4*)&sm.lse[buf][row];
                    const f32x4 d4 = *(const f32x4*)&sm.delta[buf][row];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float p = __builtin_amdgcn_exp2f(s[mb][4 * g + j] * a.scale_log2 - l4[j]);
                        if (MASKED) {
                            if (key > r * kBwdBlockM + row + j) p = 0.f;
                        }
                        s[mb][4 * g + j] = p;
                        dp[mb][4 * g + j] = p * (dp[mb][4 * g + j] - d4[j]);
                    }
                }
            bf16x8 pb[4], sb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                f32x8 x, y;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    x[j] = s[c >> 1][8 * (c & 1) + j];
                    y[j] = dp[c >> 1][8 * (c & 1) + j];
                }
                pb[c] = to_bf16x8(x);
                sb[c] = to_bf16x8(y);
            }
            // dV^T += dO^T P ; dK^T += Q^T dS   (reduction over the 64 query rows)
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint16_t* dp_ = &sm.dout[buf][16 * c + tr_row][32 * md + tr_col];
                    const bf16x8 da = concat(lds_read_tr(dp_), lds_read_tr(dp_ + 8 * QS));
                    dv_acc[md] = mfma32(da, pb[c], dv_acc[md]);
                    const uint16_t* qp_ = &sm.q[buf][16 * c + tr_row][32 * md + tr_col];
                    const bf16x8 qa = concat(lds_read_tr(qp_), lds_read_tr(qp_ + 8 * QS));
                    dk_acc[md] = mfma32(qa, sb[c], dk_acc[md]);
                }
            // stage dS^T[key][row] of the whole tile
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 x;
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = dp[mb][4 * g + j];
                    *(u32x2*)&sm.dst[wave * 32 + lr][32 * mb + 8 * g + 4 * hf] =
                        __builtin_bit_cast(u32x2, to_bf16x4(x));
                }
            __syncthreads();
            // dQ[row, d] = sum over the tile's 128 keys of dS[row, key] K[key, d]:
            // this wave computes rows 32*(wave/2).. and d blocks 2*(wave%2), +1
            {
                const int mq = wave >> 1;
                f32x16 dq[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int c = 0; c < kBwdBlockN / 16; ++c) {
                    const uint16_t* sp_ = &sm.dst[16 * c + tr_row][32 * mq + tr_col];
                    const bf16x8 sa = concat(lds_read_tr(sp_), lds_read_tr(sp_ + 8 * SS));
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int nd = 2 * (wave & 1) + j;
                        if (nd < MD) {
                            const uint16_t* kp_ = &sm.k[16 * c + tr_row][32 * nd + tr_col];
                            const bf16x8 kb = concat(lds_read_tr(kp_), lds_read_tr(kp_ + 8 * QS));
                            dq[j] = mfma32(sa, kb, dq[j]);
                        }
                    }
                }
                // register rr is query row 32mq + 8(rr/4) + 4hf + rr%4, column d = 32nd + lr
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int nd = 2 * (wave & 1) + j;
                    if (nd < MD) {
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            const int qi = r * kBwdBlockM + 32 * mq + 8 * (rr >> 2) + 4 * hf + (rr & 3);
                            if (qi < Lq)
                                unsafeAtomicAdd(a.dq_accum + (int64_t)(q0 + qi) * rs + (int64_t)hd * D +
                                                    32 * nd + lr,
                                                dq[j][rr] * a.scale);
                        }
                    }
                }
            }
            if (i + 1 < work) sstore(buf ^ 1);
            __syncthreads();
        };

        int i = 0;
        for (; i < nmasked; ++i) body(i, std::true_type{});
        for (; i < work; ++i) body(i, std::false_type{});

        // dK = scale * (dK^T)^T, dV: lane = key, register = d
        if (key < L) {
            const int64_t base = (int64_t)(kv0 + key) * rs + (int64_t)hd * D + 4 * hf;
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
                    *(u32x2*)(a.dk + base + 32 * md + 8 * g) = __builtin_bit_cast(u32x2, to_bf16x4(x));
                    *(u32x2*)(a.dv + base + 32 * md + 8 * g) = __builtin_bit_cast(u32x2, to_bf16x4(y));
                }
        }
        // the K tile in LDS is rewritten by the next tile
        __syncthreads();
    }
}

// delta[h, row] = sum_d dO[row,h,d] * O[row,h,d]; also clears dq_accum.
template <int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ d_o,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_accum,
                                                      int64_t rows_h, int32_t H, int32_t total_q,
                                                      int64_t accum_n4) {
    constexpr int LPR = D / 8;  // lanes per (row, head)
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = gtid; i < accum_n4; i += nthreads) ((f32x4*)dq_accum)[i] = f32x4{};
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

__global__ void __launch_bounds__(256) dq_convert_kernel(const float* __restrict__ src,
                                                         uint16_t* __restrict__ dst, int64_t n8) {
    const int64_t gtid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = gtid; i < n8; i += nthreads) {
        const f32x4 a = ((const f32x4*)src)[2 * i];
        const f32x4 b = ((const f32x4*)src)[2 * i + 1];
        f32x8 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[j] = a[j];
            x[4 + j] = b[j];
        }
        ((u32x4*)dst)[i] = __builtin_bit_cast(u32x4, to_bf16x8(x));
    }
}

template <int D, int MODE, bool BCAST>
int32_t launch_main(const BwdArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((bwd_kernel<D, MODE, BCAST>), dim3(a.num_workers), dim3(kThreads), 0, s, a);
    return (int32_t)hipGetLastError();
}

template <int D>
int32_t launch_d(const BwdArgs& a, Mode mode, bool bcast, int32_t stages, hipStream_t s) {
    const int64_t rows_h = (int64_t)a.total_q * a.num_heads;
    const int64_t accum_n = (int64_t)a.q_rows * a.num_heads * D;
    if (stages & JFA_BWD_PREPROCESS) {
        const int64_t want = (rows_h * (D / 8) + 255) / 256;
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>(want, 4096));
        hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3(grid), dim3(256), 0, s, a.o, a.d_o, a.delta,
                           a.dq_accum, rows_h, a.num_heads, a.total_q, accum_n / 4);
        const int32_t e = (int32_t)hipGetLastError();
        if (e) return e;
    }
    if ((stages & JFA_BWD_MAIN) && a.num_workers > 0) {
        int32_t e;
        if (mode == kCausal) e = launch_main<D, kCausal, false>(a, s);
        else if (mode == kSparse)
            e = bcast ? launch_main<D, kSparse, true>(a, s) : launch_main<D, kSparse, false>(a, s);
        else
            e = bcast ? launch_main<D, kDense, true>(a, s) : launch_main<D, kDense, false>(a, s);
        if (e) return e;
    }
    if (stages & JFA_BWD_FINISH) {
        const int64_t n8 = accum_n / 8;
        const int grid = (int)std::max<int64_t>(1, std::min<int64_t>((n8 + 255) / 256, 4096));
        hipLaunchKernelGGL(dq_convert_kernel, dim3(grid), dim3(256), 0, s, a.dq_accum, a.dq, n8);
        return (int32_t)hipGetLastError();
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
