// MXFP8 dQ pass of the jagged FlashAttention backward for gfx950 (head_dim
// 128).
//
// The pages describe an MXFP8 version of the kernel whose matrix products run
// in microscaling precision with probabilities quantised to FP8 on the fly
// ("TLX porta l'attenzione jagged su Blackwell" (ai-radar.it), section "The
// turning point"). This is the dQ pass of that backward, built like the bf16
// Q-stationary dQ pass (a 256-row tile keeps dQ^T in registers while 64-key
// blocks stream past; broadcast Q: per-worker partials summed in worker order
// by the bf16 pass's reduce), with its three products as OCP MXFP8 scaled
// MFMAs (E4M3 data, one E8M0 scale per 32 elements along the contraction):
//   S^T  = K Q^T     K and Q encoded along d
//   dP^T = V dO^T    V and dO encoded along d
//   dQ^T += K^T dS^T K encoded along the keys of its sequence (32-key blocks,
//                    as V is for the MXFP8 forward), its K^T operands
//                    byte-transposed LDS reads of the natural rows; dS^T
//                    quantised on the fly with one scale per (row, 32-key
//                    tile): the smallest power of two 2^e with max|dS| / 2^e
//                    <= 448, so that no value is clamped (the encoders' rule
//                    2^(floor(log2 max) - 8) can put the largest values of a
//                    block above 448, which E4M3 clamps: up to 12.5% off)
// P^T = exp2(S^T c - LSE c) and dS^T = P^T (dP^T - delta) stay fp32; delta =
// rowsum(dO * O) is formed from the bf16 dO and O rows in the tile prologue
// and written out for the dK/dV pass (which stays bf16).
#include "mxops.h"
#include "qtile.h"

namespace jfa {
namespace {

using namespace qtile;
using namespace mxops;

constexpr int kMxAhead = 2;                 // block j+2 is copied while block j is computed
constexpr int kMxSlots = kMxAhead + 1;      // rings: blocks j .. j+kMxAhead
constexpr int kMxStageRows = 8;             // fp32 dQ rows per wave per epilogue round

struct DqMxLds {
    static constexpr int D = 128;
    static constexpr int BLK = kFwdBlockN * D;         // one E4M3 block [64][128]
    static constexpr int SC = 256;                      // its scales
    static constexpr int K = 0;                         // K along d (rows swizzled by swz_k8)
    static constexpr int KS = K + kMxSlots * BLK;       // K scales: a dword per key
    static constexpr int V = KS + kMxSlots * SC;        // V along d (as K)
    static constexpr int VS = V + kMxSlots * BLK;       // V scales: a dword per key
    static constexpr int KK = VS + kMxSlots * SC;       // K along keys (rows swizzled by swz_v8)
    static constexpr int KKS = KK + kMxSlots * BLK;     // its scales [2 blocks][128 d]
    static constexpr int RW = 32 * D * 2;               // one wave's 32 bf16 rows
    static constexpr int STG = KKS + kMxSlots * SC;     // per-wave stage areas
    static constexpr int BYTES = STG + kWaves * RW;
    static_assert(BLK == 16 * kThreads, "one 16-byte copy per thread per block and tensor");
    static_assert(kMxStageRows * D * 4 <= RW, "epilogue staging fits a wave's area");
};

template <int MODE, bool BCAST>
__global__ void __launch_bounds__(kThreads, 1) dq_mx_kernel(DqArgs a) {
    using LY = DqMxLds;
    constexpr int D = LY::D;
    constexpr int MD = D / 32;              // 32-row d blocks of dQ^T
    constexpr int CH = D / 8;               // 16-byte chunks per bf16 row
    constexpr int CH4 = D / 4;              // 16-byte chunks per fp32 dQ row
    __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;      // row stride: elements (bf16), bytes (E4M3)

    const int w = worker_id(a.num_workers);
    const int t_begin = ld_uniform(a.worker_ptr + w), t_end = ld_uniform(a.worker_ptr + w + 1);
    auto tile_info = [&](int ti) {
        return qtile::tile_info<MODE>(a.tiles, a.kv_off, a.sp_ptr, a.sp_idx, a.mask_q_blocks,
                                      a.chunk_div, a.win_left, a.win_right, ti);
    };

    // ---- loader: the worker's blocks in plan order, kMxAhead blocks ahead.
    // Per block one 16-byte chunk of each E4M3 tensor per thread (key q/8,
    // chunk q%8 of its 128-byte row, q = 64 wave + lane) and the scales:
    // wave 0 K's, wave 1 V's (a dword per key), wave 2 those of K's two
    // 32-key blocks (lanes 0-31 block 2n, 32-63 block 2n+1, clamped to the
    // sequence's last block). Keys past the sequence read its last row.
    int l_ti = t_begin, l_i = 0, l_slot = 0;
    TileInfo LT;
    LT.work = 0;
    auto l_settle = [&]() {
        while (l_i >= LT.work) {
            ++l_ti;
            l_i = 0;
            if (l_ti >= t_end) return;
            LT = tile_info(l_ti);
        }
    };
    auto l_issue = [&]() {
        if (l_ti >= t_end) return;
        const int n = seq_block<MODE>(LT, LT.k0 + l_i);
        const int sl = l_slot % kMxSlots;
        // (from the block's first key row, a wave-uniform base; E4M3 rows are
        // rs bytes, below 2^24)
        const int64_t blk0 = (int64_t)(LT.kv0 + kFwdBlockN * n) * rs + (int64_t)LT.h * D;
        const int q = 64 * wave + lane, r = q >> 3, cs = q & 7;
        const uint32_t ro = __umul24((uint32_t)min(r, LT.L - 1 - kFwdBlockN * n), (uint32_t)rs);
        load_lds16_s(a.k8 + blk0, ro + 16 * (cs ^ swz_k8(r)), smem + LY::K + sl * LY::BLK + 1024 * wave);
        load_lds16_s(a.v8 + blk0, ro + 16 * (cs ^ swz_k8(r)), smem + LY::V + sl * LY::BLK + 1024 * wave);
        load_lds16_s(a.kk8 + blk0, ro + 16 * (cs ^ swz_v8(r)), smem + LY::KK + sl * LY::BLK + 1024 * wave);
        if (wave < 2) {
            const int kk = min(kFwdBlockN * n + lane, LT.L - 1);
            const uint8_t* src = wave == 0 ? a.k_sc : a.v_sc;
            load_lds4(src + ((int64_t)LT.h * a.total_kv + LT.kv0 + kk) * 4,
                      smem + (wave == 0 ? LY::KS : LY::VS) + sl * LY::SC);
        } else if (wave == 2) {
            const int b0 = ld_uniform(a.kk_boff + LT.b), nbk = ld_uniform(a.kk_boff + LT.b + 1) - b0;
            const int blk = min(2 * n + (lane >> 5), nbk - 1);
            load_lds4(a.kk_sc + ((int64_t)LT.h * a.kk_nb + b0 + blk) * D + 4 * (lane & 31),
                      smem + LY::KKS + sl * LY::SC);
        }
        ++l_slot;
        ++l_i;
        l_settle();
    };
    int kt_vo[4];   // this lane's offsets of the byte-transposed K^T reads
    mx_tr_offsets(lane, kt_vo);

    if (t_begin < t_end) {
        LT = tile_info(t_begin);
        l_settle();
    }
    int total = 0;   // stream length
    for (int ti = t_begin; ti < t_end; ++ti) total += ld_uniform(a.tiles + 4 * ti + 3);
    if (total > 0) {   // block 0 landed, block 1 in flight
        l_issue();
        wait_vmem();
        __syncthreads();
        l_issue();
    }

    // dQ^T accumulator: register r of acc[md] is d = 32md + 8(r/4) + 4hf + r%4
    // of this lane's query row
    f32x16 acc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = f32x16{};

    char* const stg = smem + LY::STG + wave * LY::RW;   // this wave's stage area
    // fp32 rows of scale * dQ through the wave's stage area, handed to
    // store(row, chunk, value) as 16-byte chunks
    auto stage_out = [&](auto store) {
#pragma unroll
        for (int rd = 0; rd < 32 / kMxStageRows; ++rd) {
            if ((lr >> 3) == rd) {
                const int r = lr & 7;
#pragma unroll
                for (int md = 0; md < MD; ++md)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        f32x4 x;
#pragma unroll
                        for (int j = 0; j < 4; ++j) x[j] = acc[md][4 * g + j] * a.scale;
                        const int chunk = 8 * md + 2 * g + hf;
                        *(f32x4*)(stg + r * D * 4 + ((chunk ^ r) << 4)) = x;
                    }
            }
            wave_sync_lds();
#pragma unroll
            for (int v = 0; v < kMxStageRows * CH4 / 64; ++v) {
                const int k = lane + 64 * v;
                const int r = k / CH4, chunk = k % CH4;
                const f32x4 x = *(const f32x4*)(stg + r * D * 4 + ((chunk ^ r) << 4));
                store(32 * wave + kMxStageRows * rd + r, chunk, x);
            }
            wave_sync_lds();
        }
    };

    // Q^T fragments of this lane's row (E4M3 along d, the slots of
    // mx_scores); with a broadcast Q every tile of the worker shares them
    i32x8 qf8[2];
    int qsc[2];
    int qf_h = -1, qf_t = -1;
    int s = 0;   // stream position of the consumer
    for (int ti = t_begin; ti < t_end; ++ti) {
        const TileInfo T = tile_info(ti);
        int q0, Lq, orow0;
        if (BCAST) {
            q0 = 0;
            Lq = a.lq;
            orow0 = T.b * a.lq;
        } else {
            q0 = ld_uniform(a.q_off + T.b);
            Lq = ld_uniform(a.q_off + T.b + 1) - q0;
            orow0 = q0;
        }
        const int row0 = T.t * kFwdBlockM + 32 * wave;   // first row of this wave
        const int qrow = row0 + lr;
        const bool wave_rows = row0 < Lq;                // wave-uniform
        const int qr = min(qrow, Lq - 1);                // rows past the sequence read its last row
        const float lse = a.lse[(int64_t)T.h * a.total_q + orow0 + qr];

        // delta = rowsum(dO * O) from the bf16 rows: dO through the wave's
        // stage area with row-contiguous copies, O into registers in the same
        // layout, summed over the lanes of a row and handed to the row's
        // lanes through LDS; the tile's first chunk writes it out
        float dlt;
        {
            constexpr int NI = 32 * CH / 64;   // 16-byte copies per lane
            bf16x8 ov[NI];
#pragma unroll
            for (int u = 0; u < NI; ++u) {
                const int p = 64 * u + lane, r = p / CH, cs = p % CH;
                const int row = min(row0 + r, Lq - 1);
                const int64_t g = (int64_t)(orow0 + row) * rs + (int64_t)T.h * D + 8 * cs;
                load_lds16(a.d_o + g, stg + 1024 * u);
                ov[u] = load_bf16x8(a.o + g);
            }
            wait_vmem();
            wave_sync_lds();
            float dsum[NI];
#pragma unroll
            for (int u = 0; u < NI; ++u) {
                const bf16x8 dd = *(const bf16x8*)(stg + 1024 * u + 16 * lane);
                float part = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) part = fmaf((float)dd[j], (float)ov[u][j], part);
#pragma unroll
                for (int m = CH / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m);
                dsum[u] = part;
            }
            wave_sync_lds();
            float* dl = (float*)stg;
            if (lane % CH == 0) {
#pragma unroll
                for (int u = 0; u < NI; ++u) dl[(64 * u + lane) / CH] = dsum[u];
            }
            wave_sync_lds();
            dlt = dl[lr];
            wave_sync_lds();   // read before the stage area is next written
        }
        if (hf == 0 && T.k0 == 0 && qrow < Lq) a.delta[(int64_t)T.h * a.total_q + orow0 + qrow] = dlt;

        // dO^T fragments of this lane's row (E4M3 along d, as Q's)
        i32x8 df8[2];
        int dsc[2];
        {
            const int64_t dr = orow0 + qr;
            const uint8_t* dp = a.do8 + dr * rs + (int64_t)T.h * D;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4 lo = *(const u32x4*)(dp + 64 * j + 16 * hf);
                const u32x4 hi = *(const u32x4*)(dp + 64 * j + 32 + 16 * hf);
                df8[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
            const uint32_t ds = *(const uint32_t*)(a.do_sc + ((int64_t)T.h * a.total_q + dr) * 4);
#pragma unroll
            for (int j = 0; j < 2; ++j) dsc[j] = (ds >> (8 * (2 * j + hf))) & 255;
        }
        if (!BCAST || T.h != qf_h || T.t != qf_t) {
            const int64_t qq = q0 + qr;
            const uint8_t* qp = a.q8 + qq * rs + (int64_t)T.h * D;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4 lo = *(const u32x4*)(qp + 64 * j + 16 * hf);
                const u32x4 hi = *(const u32x4*)(qp + 64 * j + 32 + 16 * hf);
                qf8[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
            const uint32_t qs = *(const uint32_t*)(a.q_sc + ((int64_t)T.h * a.q_rows + qq) * 4);
#pragma unroll
            for (int j = 0; j < 2; ++j) qsc[j] = (qs >> (8 * (2 * j + hf))) & 255;
            qf_h = T.h;
            qf_t = T.t;
        }
        // a row without visible keys (LSE = -inf) gets P = 0
        const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
        if (!BCAST) {
#pragma unroll
            for (int md = 0; md < MD; ++md) acc[md] = f32x16{};
        }
        wait_vmem();

        for (int i = 0; i < T.work; ++i, ++s) {
            if (i > 0) wait_vmem();   // block s+1 landed (the only copies in flight)
            // every wave is past block s-1: its slots are free
            __syncthreads();
            l_issue();                              // block s+kMxAhead

            const int n = seq_block<MODE>(T, T.k0 + i);
            bool skip, masked;
            block_flags<MODE>(T, T.k0 + i, n, row0, wave_rows, wave, skip, masked);
            if (skip) continue;
            const int sl = s % kMxSlots;
            f32x16 sc[2], dp[2];
            mx_scores(sc, smem + LY::K + sl * LY::BLK, smem + LY::KS + sl * LY::SC, qf8, qsc, lr, hf);
            mx_scores(dp, smem + LY::V + sl * LY::BLK, smem + LY::VS + sl * LY::SC, df8, dsc, lr, hf);
            // register r of tile mb is key 64n + 32mb + 8(r/4) + 4hf + r%4
            if (masked) {   // keys past the sequence or (banded) outside [lo, lim]
                int lim = T.L - 1, lo = 0;
                if (MODE == kCausal) {
                    if (T.wr >= 0 && qrow <= T.L - 1 - T.wr) lim = qrow + T.wr;
                    if (T.wl >= 0) lo = qrow - T.wl;
                }
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = kFwdBlockN * n + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3);
                        sc[mb][r] = (kk <= lim && kk >= lo) ? sc[mb][r] : -INFINITY;
                    }
            }
            // dS^T = P^T (dP^T - delta), then E4M3 with one scale per
            // (row, 32-key tile) from the tile's largest |dS| (both halves of
            // the row see it): 2^e with e = floor(log2 max) - 8, one more if
            // max / 2^e > 448; a tile whose values are all below 2^-100 is
            // sent as zeros (their products are far below fp32's resolution
            // of the sum)
            float scl[2];
            int sce[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                float amax = 0.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[mb][r], a.scale_log2, -lse2));
                    const float ds = p * (dp[mb][r] - dlt);
                    sc[mb][r] = ds;
                    amax = fmaxf(amax, fabsf(ds));
                }
                amax = pair_max(amax);
                if (amax < 0x1p-100f) {
                    scl[mb] = 1.0f;
                    sce[mb] = -127;
#pragma unroll
                    for (int r = 0; r < 16; ++r) sc[mb][r] = 0.f;
                } else {
                    // (|dS| <= max <= 448 * 2^e: nothing to clamp)
                    int e = (int)((__float_as_uint(amax) >> 23) & 255) - 127 - 8;
                    if (amax > 448.0f * __uint_as_float((uint32_t)(e + 127) << 23)) ++e;
                    sce[mb] = e;
                    scl[mb] = __uint_as_float((uint32_t)(e + 127) << 23);
                }
            }
            const i32x8 ds8 = mx_pack_scaled(sc, scl);
            // dQ^T[d, row] += K^T[d, key] dS^T[key, row]; this lane gives the
            // scale of tile hf of its row
            mx_pv_tr(acc, ds8, smem + LY::KK + sl * LY::BLK, kt_vo, smem + LY::KKS + sl * LY::SC,
                  (hf ? sce[1] : sce[0]) + 127, lr, hf);
        }

        if (!BCAST) {
            // dQ rows of this tile: dq_accum (fp32) and dq (bf16)
            if (wave_rows) {
                const int64_t base = (int64_t)T.h * D;
                stage_out([&](int r, int chunk, const f32x4& x) {
                    const int row = T.t * kFwdBlockM + r;
                    if (row < Lq) {
                        const int64_t g = (int64_t)(q0 + row) * rs + base + 4 * chunk;
                        *(f32x4*)(a.dq_accum + g) = x;
                        *(bf16x4*)(a.dq + g) = to_bf16x4(x);
                    }
                });
            }
        }
    }
    if (BCAST) {
        // this worker's partial sum over its tiles (all of one (head, Q tile)
        // group): rows 0..255 of the tile, fp32 (zeros for a worker without
        // tiles, so that the reduce reads every partial unconditionally)
        float* part = a.partial + (int64_t)w * kFwdBlockM * D;
        stage_out([&](int r, int chunk, const f32x4& x) {
            *(f32x4*)(part + (int64_t)r * D + 4 * chunk) = x;
        });
    }
}

template <int MODE, bool BCAST>
int32_t launch(const DqArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((dq_mx_kernel<MODE, BCAST>), dim3(a.num_workers), dim3(kThreads), 0, stream, a);
    return (int32_t)hipGetLastError();
}

}  // namespace

int32_t launch_dq_mx(const DqArgs& a, Mode mode, bool broadcast, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (a.num_workers == 0) return 0;
    if (mode == kCausal) return launch<kCausal, false>(a, s);
    if (mode == kSparse) return broadcast ? launch<kSparse, true>(a, s) : launch<kSparse, false>(a, s);
    return broadcast ? launch<kDense, true>(a, s) : launch<kDense, false>(a, s);
}

}  // namespace jfa
