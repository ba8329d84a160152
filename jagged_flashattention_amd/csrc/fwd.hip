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
//   - K and V of a 64-key block double-buffered in LDS from coalesced 16-byte
//     global loads issued one block ahead; V stays row-major and is fed to
//     O^T += V^T P^T through ds_read_tr16_b64 transposed reads;
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
constexpr int kPad = 8;  // bf16 elements of padding per LDS row

template <int D>
struct FwdSmem {
    uint16_t k[2][kFwdBlockN][D + kPad];
    uint16_t v[2][kFwdBlockN][D + kPad];
};

template <int D, int MODE, bool BCAST>
__global__ void __launch_bounds__(kThreads, 2) fwd_kernel(FwdArgs a) {
    __shared__ FwdSmem<D> sm;
    constexpr int KC = D / 16;              // 16-wide d chunks of S^T = K Q^T
    constexpr int MD = D / 32;              // 32-row d blocks of O^T
    constexpr int CPR = D / 8;              // 16-byte chunks per K/V row
    constexpr int RPP = kThreads / CPR;     // rows per load pass
    constexpr int NP = kFwdBlockN / RPP;    // load passes per block
    constexpr int VSTRIDE = D + kPad;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;

    // lane constants of the transposed V read (see lds_read_tr)
    const int g16 = lane >> 4, n16 = lane & 15;
    const int tr_row = 4 * (g16 >> 1) + (n16 >> 2);
    const int tr_col = (g16 & 1) * 16 + 4 * (n16 & 3);
    const int ld_row = tid / CPR, ld_col = (tid % CPR) * 8;

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

        u32x4 kr[NP], vr[NP];
        auto gload = [&](int n) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                const int key = kFwdBlockN * n + ld_row + p * RPP;
                if (key < L) {
                    const int64_t off = (int64_t)(kv0 + key) * rs + (int64_t)hd * D + ld_col;
                    kr[p] = *(const u32x4*)(a.k + off);
                    vr[p] = *(const u32x4*)(a.v + off);
                } else {
                    kr[p] = u32x4{};
                    vr[p] = u32x4{};
                }
            }
        };
        auto sstore = [&](int buf) {
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                *(u32x4*)&sm.k[buf][ld_row + p * RPP][ld_col] = kr[p];
                *(u32x4*)&sm.v[buf][ld_row + p * RPP][ld_col] = vr[p];
            }
        };

        if (work > 0) {
            gload(blk(0));
            sstore(0);
        }
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
                    const bf16x8 kf = load_bf16x8(&sm.k[buf][32 * mb + lr][16 * kc + 8 * hf]);
                    s[mb] = mfma32(kf, qf[kc], s[mb]);
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float x = s[mb][r] * a.scale_log2;
                    if (MASKED) {
                        const int kk = kFwdBlockN * n + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3);
                        bool ok = kk < L;
                        if (MODE == kCausal) ok = ok && kk <= qrow;
                        x = ok ? x : -INFINITY;
                    }
                    s[mb][r] = x;
                    mx = fmaxf(mx, x);
                }
            mx = pair_max(mx);
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            float ls = 0.f;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(s[mb][r] - m_new);
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
                    const uint16_t* vp = &sm.v[buf][16 * c + tr_row][32 * md + tr_col];
                    const bf16x8 vf = concat(lds_read_tr(vp), lds_read_tr(vp + 8 * VSTRIDE));
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
