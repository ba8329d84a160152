// Jagged FlashAttention forward for gfx950.
//
// The pages describe a persistent forward kernel (one program per processor
// looping over tiles), K/V staged through multi-buffered on-chip memory, an
// online softmax with a correction step, and a KV loop peeled into a
// branch-free bulk pass plus a small masked tail ("Meta's TLX Jagged Flash
// Attention Beats FA4 on Blackwell With 3x Less Code" (ainewsbites.com),
// sections "What TLX changes" and "Optimizations layered on top"). The
// warp-specialised Blackwell machinery is not reproduced; on CDNA4 the same
// goals map to:
//   - a persistent grid that walks a host-built tile list (sorted by KV work,
//     dealt in zigzag order), with an XCD-aware workgroup -> worker map;
//   - 4 waves per workgroup, each owning 32 query rows of a 128-row tile, Q
//     held in VGPRs as the B operand of S^T = K Q^T (32x32x16 bf16 MFMA) so a
//     lane owns one query row: row max / row sum stay in-lane and need one
//     cross-half exchange;
//   - K and V of a 64-key block double-buffered in LDS from 16-byte global
//     loads issued one block ahead; K rows are stored with a chunk swizzle and
//     V is transposed on its way into LDS (keys in the order the P^T
//     accumulator registers hold them), so every MFMA operand is one
//     conflict-free 16-byte LDS read;
//   - fp32 running max and sum in the exp2 domain, rescaling of the O
//     accumulator skipped when no row max moved;
//   - a bulk loop without any mask arithmetic and a tail loop (last partial
//     block, causal diagonal) with it.
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace jfa {
namespace {

constexpr int kThreads = 256;

template <int D>
struct FwdSmem {
    uint16_t k[2][kFwdBlockN][D];            // K rows, 16-byte chunks swizzled
    uint16_t vt[2][D][kFwdBlockN + 8];       // V^T, keys in sigma order
};

// position of key q (within its group of 16) in sigma order 0-3, 8-11, 4-7, 12-15
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
__global__ void __launch_bounds__(kThreads, 2) fwd_kernel(FwdArgs a) {
    __shared__ FwdSmem<D> sm;
    constexpr int KC = D / 16;              // 16-wide d chunks of S^T = K Q^T
    constexpr int MD = D / 32;              // 32-row d blocks of O^T
    constexpr int CH = D / 8;               // 16-byte chunks per K/V row

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;
    // loader: keys 4kg..4kg+3 x one 16-byte chunk dc per thread
    const int ld_kg = tid & 15, ld_dc = tid >> 4;
    const bool ld_on = ld_dc < CH;
    const int ld_pos = sigma_pos(4 * ld_kg);
    // swizzled K-row addresses of this lane (rows 32mb + lr)
    int nat_base[2], nat_x[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int row = 32 * mb + lr;
        const int s = swz<D>(row);
        nat_base[mb] = row * D + 8 * (hf ^ (s & 1));
        nat_x[mb] = s >> 1;
    }

    const int w = worker_id(a.num_workers);
    const int t_begin = a.worker_ptr[w], t_end = a.worker_ptr[w + 1];

    for (int ti = t_begin; ti < t_end; ++ti) {
        const int b = a.tiles[4 * ti + 0];
        const int hd = a.tiles[4 * ti + 1];
        const int t = a.tiles[4 * ti + 2];
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
        const int qrow = t * kFwdBlockM + wave * 32 + lr;
        const int* sp = nullptr;
        if (MODE == kSparse) sp = a.sp_idx + a.sp_ptr[b * a.mask_q_blocks + t];
        auto blk = [&](int i) -> int {
            if (MODE == kSparse) return 2 * sp[i >> 1] + (i & 1);
            return i;
        };
        int nbulk;
        if (MODE == kDense) {
            nbulk = L / kFwdBlockN;
        } else if (MODE == kCausal) {
            nbulk = min(2 * t, L / kFwdBlockN);
        } else {
            nbulk = work;
            if (work > 0 && kFwdBlockN * (blk(work - 1) + 1) > L) nbulk = work - 1;
        }
        nbulk = min(nbulk, work);

        bf16x8 qf[KC];
        if (qrow < Lq) {
            const uint16_t* qp = a.q + (int64_t)(q0 + qrow) * rs + (int64_t)hd * D + 8 * hf;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) qf[kc] = load_bf16x8(qp + 16 * kc);
        } else {
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) qf[kc] = bf16x8{};
        }

        f32x16 oacc[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};
        float m_run = -1e30f, l_run = 0.f;

        // (threads past the row width load a valid chunk and never store it)
        const uint16_t* kbase = a.k + (int64_t)kv0 * rs + (int64_t)hd * D + 8 * (ld_dc & (CH - 1));
        const uint16_t* vbase = a.v + (int64_t)kv0 * rs + (int64_t)hd * D + 8 * (ld_dc & (CH - 1));
        u32x4 kr[4], vr[4];
        int ld_n = 0;   // KV block held in the registers, for the zero fill at store time
        auto gload = [&](int n) {
            // unconditional loads from a key clamped into the sequence (L >= 1
            // whenever a block exists); keys past the end are zeroed in sstore
            ld_n = n;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int key = min(kFwdBlockN * n + 4 * ld_kg + p, L - 1);
                kr[p] = *(const u32x4*)(kbase + (int64_t)key * rs);
                vr[p] = *(const u32x4*)(vbase + (int64_t)key * rs);
            }
        };
        auto sstore = [&](int buf) {
            if (ld_on) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    if (kFwdBlockN * ld_n + 4 * ld_kg + p >= L) {
                        kr[p] = u32x4{};
                        vr[p] = u32x4{};
                    }
                }
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int row = 4 * ld_kg + p;
                    *(u32x4*)&sm.k[buf][row][8 * (ld_dc ^ swz<D>(row))] = kr[p];
                }
                u32x2 y[8];
                transpose4x8(vr, y);
#pragma unroll
                for (int e = 0; e < 8; ++e) *(u32x2*)&sm.vt[buf][8 * ld_dc + e][ld_pos] = y[e];
            }
        };

        if (work > 0) {
            gload(blk(0));
            sstore(0);
        }
        // Nothing may be left in flight here: otherwise the compiler's wait
        // counters, merged over the loop back edge, make the first MFMAs of
        // every iteration wait for that iteration's prefetch loads.
        wait_vmem();
        __syncthreads();

        auto body = [&](int i, auto masked_tag) {
            constexpr bool MASKED = decltype(masked_tag)::value;
            const int buf = i & 1;
            const int n = blk(i);
            if (i + 1 < work) gload(blk(i + 1));

            // S^T[key, qrow] for the 64 keys of the block: two 32-key halves
            f32x16 s[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                s[mb] = f32x16{};
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const bf16x8 kf =
                        load_bf16x8(&sm.k[buf][0][0] + nat_base[mb] + 16 * (kc ^ nat_x[mb]));
                    s[mb] = mfma32(kf, qf[kc], s[mb]);
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[mb][r];
                    if (MASKED) {
                        const int kk = kFwdBlockN * n + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3);
                        bool ok = kk < L;
                        if (MODE == kCausal) ok = ok && kk <= qrow;
                        x = ok ? x : -INFINITY;
                    }
                    s[mb][r] = x;
                    mx = fmaxf(mx, x);
                }
            // running max in the exp2 domain of the scaled scores
            mx = pair_max(mx) * a.scale_log2;
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float ls = 0.f;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][r], a.scale_log2, -m_new));
                    s[mb][r] = p;
                    ls += p;
                }
            l_run = l_run * alpha + ls;
            m_run = m_new;
            if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
            }
            // P^T as the B operand: chunk c holds keys 16c..16c+15 of the block
            bf16x8 pb[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                f32x8 x;
#pragma unroll
                for (int j = 0; j < 8; ++j) x[j] = s[c >> 1][8 * (c & 1) + j];
                pb[c] = to_bf16x8(x);
            }
            // O^T[d, qrow] += V^T[d, key] P^T[key, qrow]
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bf16x8 vf = load_bf16x8(&sm.vt[buf][32 * md + lr][16 * c + 8 * hf]);
                    oacc[md] = mfma32(vf, pb[c], oacc[md]);
                }
            if (i + 1 < work) sstore(buf ^ 1);
            __syncthreads();
        };

        int i = 0;
        for (; i < nbulk; ++i) body(i, std::false_type{});
        for (; i < work; ++i) body(i, std::true_type{});

        const float l_tot = pair_sum(l_run);
        if (qrow < Lq) {
            const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
            const int orow = orow0 + qrow;
            uint16_t* op = a.o + (int64_t)orow * rs + (int64_t)hd * D + 4 * hf;
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 x;
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = oacc[md][4 * g + j] * inv;
                    *(u32x2*)(op + 32 * md + 8 * g) = __builtin_bit_cast(u32x2, to_bf16x4(x));
                }
            if (hf == 0)
                a.lse[(int64_t)hd * a.total_q + orow] =
                    l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <int D, int MODE, bool BCAST>
int32_t launch(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_kernel<D, MODE, BCAST>), dim3(a.num_workers), dim3(kThreads), 0,
                       stream, a);
    return (int32_t)hipGetLastError();
}

template <int D>
int32_t launch_d(const FwdArgs& a, Mode mode, bool bcast, hipStream_t s) {
    if (mode == kCausal) return launch<D, kCausal, false>(a, s);
    if (mode == kSparse)
        return bcast ? launch<D, kSparse, true>(a, s) : launch<D, kSparse, false>(a, s);
    return bcast ? launch<D, kDense, true>(a, s) : launch<D, kDense, false>(a, s);
}

}  // namespace

int32_t launch_fwd(const FwdArgs& a, int32_t head_dim, Mode mode, bool broadcast, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (head_dim == 64) return launch_d<64>(a, mode, broadcast, s);
    return launch_d<128>(a, mode, broadcast, s);
}

}  // namespace jfa
