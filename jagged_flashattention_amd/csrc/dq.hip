// Q-stationary dQ pass of the jagged FlashAttention backward for gfx950, and
// the deterministic reduction of its broadcast-Q partials.
//
// With a broadcast Q, dQ of a query row sums the contributions of every
// sequence; the pages single this cross-program reduction out as the main
// backward bottleneck and describe staging it through on-chip memory in two
// stages ("Meta's 3.2K-line Triton kernel outruns FlashAttention-4 on jagged
// Blackwell attention" (theclarity.today), second paragraph; "Meta's TLX
// Jagged Flash Attention Beats FA4 on Blackwell" (ainewsbites.com), section
// "Optimizations layered on top", dQ staging). Here the reduction is split
// the other way round: dQ is computed Q-stationary, like the forward (a tile
// of 256 rows keeps its dQ^T accumulator in registers while K/V blocks
// stream past), so no fp32 atomics are needed at all:
//   - per-sequence Q: a tile owns its rows and writes dq / dq_accum directly;
//   - broadcast Q: the plan deals the tiles of each (head, Q tile) group to
//     a worker range of its own; each worker sums its tiles in registers
//     (stage 1) and writes one fp32 partial; a reduce kernel adds the partials
//     of each group in worker order (stage 2), so the result does not depend
//     on timing. The alternative second stage (ATOMIC): each worker adds its
//     sum into the zeroed dq_accum with fp32 atomic adds, and a last kernel
//     rounds dq_accum to bf16.
// Per 64-key block and wave (32 query rows, one per lane column):
//   S^T  = K Q^T        A = K rows from LDS,   B = Q^T (VGPRs)
//   dP^T = V dO^T       A = V rows from LDS,   B = dO^T (VGPRs)
//   P^T  = exp2(S^T * scale*log2e - LSE*log2e), dS^T = P^T (dP^T - delta)
//   dQ^T += K^T dS^T    A = K^T: transposed reads of the K rows, B = dS^T
// (a transposed read of a 16-lane group takes the 4 keys that the lane's dS^T
// registers hold, in their order, so no transposed copy of K is made).
#include <algorithm>

#include "qtile.h"

namespace jfa {
namespace {

using namespace qtile;

constexpr int kAhead = 2;               // block j+2 is copied while block j is computed
constexpr int kSlots = kAhead + 1;      // K and V rings: blocks j .. j+kAhead
constexpr int kReadAhead = 4;           // LDS operand reads kept in flight ahead of the MFMAs
constexpr int kStageRows = 8;           // fp32 dQ rows per wave per epilogue round

template <int D>
struct DqLds {
    static constexpr int BLK = kFwdBlockN * D * 2;     // one K or V block (bf16)
    static constexpr int K = 0;                         // kSlots natural K blocks
    static constexpr int V = K + kSlots * BLK;          // kSlots natural V blocks
    static constexpr int RW = 32 * D * 2;               // one wave's 32 dO rows (tile prologue)
    static constexpr int STG = V + kSlots * BLK;        // a stage area per wave
    static constexpr int BYTES = STG + kWaves * RW;
    static constexpr int ST_WAVE = kStageRows * D * 4;  // fp32 staging of one wave
    static_assert(ST_WAVE <= RW, "dQ staging fits the wave's stage area");
};

template <int D, int MODE, bool BCAST, bool ATOMIC>
__global__ void __launch_bounds__(kThreads, 1) dq_kernel(DqArgs a) {
    using LY = DqLds<D>;
    __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];
    constexpr int KC = D / 16;              // 16-wide d chunks of S^T and dP^T
    constexpr int MD = D / 32;              // 32-row d blocks of dQ^T
    constexpr int CH = D / 8;               // 16-byte chunks per K/V row
    constexpr int CH4 = D / 4;              // 16-byte chunks per fp32 dQ row
    constexpr int LPW = (kFwdBlockN * CH) / (64 * kWaves);   // K (and V) copies per wave per block

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;

    // direct-to-LDS copy: copy u of this wave fills chunk positions
    // 64 (LPW wave + u) + lane of a block: key r, stored chunk cp. K and V
    // share the swizzle that serves both the operand reads and (K) the
    // transposed reads.
    // The lane's byte offset from the block's first key row (32 bits: at
    // most 64 rows of H*D*2 bytes, H bounded by the planner).
    const uint32_t rs_b = (uint32_t)rs * 2;
    int ld_row[LPW];
    uint32_t ld_o[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int p = 64 * (LPW * wave + u) + lane;
        const int r = p / CH, cp = p % CH;
        ld_row[u] = r;
        ld_o[u] = r * rs_b + 16 * (cp ^ swz_rt<D>(r));
    }
    // A operands: K / V row 32mb + lr, chunk 2kc + hf (swz_rt depends on the
    // row's low 4 bits only)
    int kv_off[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) kv_off[kc] = lr * D * 2 + (((2 * kc + hf) ^ swz_rt<D>(lr)) << 4);
    // K^T[32md + lr][keys of 16-key chunk c, in dS^T's order]: two transposed
    // reads of the natural K rows
    int kt_off[2][MD];
    tr_operand_offsets<D>(lane, kt_off);

    const int w = worker_id(a.num_workers);
    const int t_begin = ld_uniform(a.worker_ptr + w), t_end = ld_uniform(a.worker_ptr + w + 1);
    auto tile_info = [&](int ti) {
        return qtile::tile_info<MODE>(a.tiles, a.kv_off, a.sp_ptr, a.sp_idx, a.mask_q_blocks,
                                      a.chunk_div, a.win_left, a.win_right, ti);
    };

    // ---- loader: the worker's blocks in plan order, kAhead blocks ahead
    int l_ti = t_begin, l_i = 0, l_slot = 0;
    TileInfo LT;
    LT.work = 0;
    auto l_settle = [&]() {   // skip to the next tile with blocks (LT is l_ti's)
        while (l_i >= LT.work) {
            ++l_ti;
            l_i = 0;
            if (l_ti >= t_end) return;
            LT = tile_info(l_ti);
        }
    };
    // keys past the sequence are clamped to its last row (finite data whose
    // probabilities the tail path zeroes)
    auto l_issue = [&]() {
        if (l_ti >= t_end) return;
        const int n = seq_block<MODE>(LT, LT.k0 + l_i);
        char* kdst = smem + LY::K + (l_slot % kSlots) * LY::BLK;
        char* vdst = smem + LY::V + (l_slot % kSlots) * LY::BLK;
        // the block's first key row (wave-uniform); a partial last block
        // moves its rows past the sequence back onto the last row
        const int64_t blk0 = (int64_t)(LT.kv0 + kFwdBlockN * n) * rs + (int64_t)LT.h * D;
        const uint16_t* kb = a.k + blk0;
        const uint16_t* vb = a.v + blk0;
        const int last = LT.L - 1 - kFwdBlockN * n;
#pragma unroll
        for (int u = 0; u < LPW; ++u) {
            uint32_t back = 0;
            if (last < kFwdBlockN - 1) back = (uint32_t)max(ld_row[u] - last, 0) * rs_b;
            load_lds16_s(kb, ld_o[u] - back, kdst + 1024 * (LPW * wave + u));
            load_lds16_s(vb, ld_o[u] - back, vdst + 1024 * (LPW * wave + u));
        }
        ++l_slot;
        ++l_i;
        l_settle();
    };
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

    // fp32 rows of scale * dQ through this wave's own stage area (no
    // workgroup barrier needed), handed to store(row, chunk, value) as
    // 16-byte chunks: 4 rows x 256 bytes per instruction
    auto stage_out = [&](auto store) {
        char* st = smem + LY::STG + wave * LY::RW;
#pragma unroll
        for (int rd = 0; rd < 32 / kStageRows; ++rd) {
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
                        *(f32x4*)(st + r * D * 4 + ((chunk ^ r) << 4)) = x;
                    }
            }
            wave_sync_lds();
#pragma unroll
            for (int v = 0; v < kStageRows * CH4 / 64; ++v) {
                const int k = lane + 64 * v;
                const int r = k / CH4, chunk = k % CH4;
                const f32x4 x = *(const f32x4*)(st + r * D * 4 + ((chunk ^ r) << 4));
                store(32 * wave + kStageRows * rd + r, chunk, x);
            }
            wave_sync_lds();
        }
    };

    // Q^T fragments of this lane's row; with a broadcast Q every tile of the
    // worker has the same (head, Q tile), so they are loaded once
    bf16x8 qf[KC];
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
        // Q^T and dO^T fragments, LSE (exp2 domain) and delta of this lane's
        // row (rows past the sequence read its last row; their dQ is dropped)
        const int qr = min(qrow, Lq - 1);
        const float lse = a.lse[(int64_t)T.h * a.total_q + orow0 + qr];
        // delta = rowsum(dO * O) of each row (the standard FlashAttention
        // backward quantity); the tile's first chunk writes it out for the
        // dK/dV pass
        bf16x8 df[KC];
        float dlt;
        if constexpr (BCAST) {
            // dO and O of the wave's 32 rows, fetched with row-contiguous
            // copies (row-strided dO^T fragment loads cost the vector memory
            // unit one cache line per row and instruction): dO into the
            // wave's own stage area, O into registers in the same layout.
            // The dO^T fragments are then read from LDS, and delta is formed
            // in the copy layout, summed over the lanes of a row and handed
            // to the fragment lanes through LDS. (Per-sequence Q keeps the
            // direct loads below: its extra live Q rows would spill.)
            char* rg = smem + LY::STG + wave * LY::RW;
            constexpr int NI = 32 * CH / 64;   // 16-byte copies per lane
            bf16x8 ov[NI];
#pragma unroll
            for (int u = 0; u < NI; ++u) {
                const int p = 64 * u + lane, r = p / CH, cs = p % CH;
                const int row = min(row0 + r, Lq - 1);
                const int64_t g = (int64_t)(orow0 + row) * rs + (int64_t)T.h * D + 8 * (cs ^ swz_rt<D>(r));
                load_lds16(a.d_o + g, rg + 1024 * u);
                ov[u] = load_bf16x8(a.o + g);
            }
            wait_vmem();
            wave_sync_lds();
#pragma unroll
            for (int kc = 0; kc < KC; ++kc)
                df[kc] = *(const bf16x8*)(rg + lr * D * 2 + (((2 * kc + hf) ^ swz_rt<D>(lr)) << 4));
            float dsum[NI];
#pragma unroll
            for (int u = 0; u < NI; ++u) {
                const bf16x8 dd = *(const bf16x8*)(rg + 1024 * u + 16 * lane);
                float part = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) part = fmaf((float)dd[j], (float)ov[u][j], part);
#pragma unroll
                for (int m = CH / 2; m >= 1; m >>= 1) part += __shfl_xor(part, m);
                dsum[u] = part;
            }
            wave_sync_lds();
            float* dl = (float*)rg;   // delta of the wave's 32 rows
            if (lane % CH == 0) {
#pragma unroll
                for (int u = 0; u < NI; ++u) dl[(64 * u + lane) / CH] = dsum[u];
            }
            wave_sync_lds();
            dlt = dl[lr];
        } else {
            // this lane's half of d of its row, then the other half's lane
            const uint16_t* dp = a.d_o + (int64_t)(orow0 + qr) * rs + (int64_t)T.h * D + 8 * hf;
            const uint16_t* op = a.o + (int64_t)(orow0 + qr) * rs + (int64_t)T.h * D + 8 * hf;
            float part = 0.f;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                df[kc] = load_bf16x8(dp + 16 * kc);
                const bf16x8 of = load_bf16x8(op + 16 * kc);
#pragma unroll
                for (int j = 0; j < 8; ++j) part = fmaf((float)df[kc][j], (float)of[j], part);
            }
            dlt = pair_sum(part);
        }
        if (hf == 0 && T.k0 == 0 && qrow < Lq) a.delta[(int64_t)T.h * a.total_q + orow0 + qrow] = dlt;
        // Q^T fragments (with a broadcast Q: once per worker)
        if (!BCAST || T.h != qf_h || T.t != qf_t) {
            const uint16_t* qp = a.q + (int64_t)(q0 + qr) * rs + (int64_t)T.h * D + 8 * hf;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) qf[kc] = load_bf16x8(qp + 16 * kc);
            qf_h = T.h;
            qf_t = T.t;
        }
        // a row without visible keys (LSE = -inf) gets P = 0
        const float lse2 = lse == -INFINITY ? INFINITY : lse * kLog2e;
        if (!BCAST) {
#pragma unroll
            for (int md = 0; md < MD; ++md) acc[md] = f32x16{};
        }
        // the rows above and the previous tile's stores: nothing the compiler
        // tracks stays pending inside the block loop
        wait_vmem();

        for (int i = 0; i < T.work; ++i, ++s) {
            if (i > 0) wait_vmem();   // block s+1 landed (the only copies in flight)
            // every wave is past block s-1: its slots are free
            __syncthreads();
            l_issue();                              // block s+kAhead

            const int n = seq_block<MODE>(T, T.k0 + i);
            bool skip, masked;
            block_flags<MODE>(T, T.k0 + i, n, row0, wave_rows, wave, skip, masked);
            if (skip) continue;
            const char* kb = smem + LY::K + (s % kSlots) * LY::BLK;
            const char* vb = smem + LY::V + (s % kSlots) * LY::BLK;
            // the block in two halves of 32 keys (hb)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                f32x16 sc = f32x16{}, dp = f32x16{};
                {
                    bf16x8 kf[KC], vf[KC];
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        kf[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + 32 * D * 2 * hb + kv_off[kc]));
                        vf[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(vb + 32 * D * 2 * hb + kv_off[kc]));
                    }
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc) {
                        sc = mfma32(kf[kc], qf[kc], sc);
                        dp = mfma32(vf[kc], df[kc], dp);
                    }
                    pipeline_reads_mfma<2 * KC, kReadAhead>();
                }
                // register r is key 64n + 32hb + 8(r/4) + 4hf + r%4
                if (masked) {   // keys past the sequence or (banded) outside [lo, lim]
                    int lim = T.L - 1, lo = 0;
                    if (MODE == kCausal) {
                        if (T.wr >= 0 && qrow <= T.L - 1 - T.wr) lim = qrow + T.wr;
                        if (T.wl >= 0) lo = qrow - T.wl;
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kk = kFwdBlockN * n + 32 * hb + 8 * (r >> 2) + 4 * hf + (r & 3);
                        sc[r] = (kk <= lim && kk >= lo) ? sc[r] : -INFINITY;
                    }
                }
                bf16x8 db[2];
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    f32x8 x;
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int r = 8 * c2 + j;
                        const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], a.scale_log2, -lse2));
                        x[j] = p * (dp[r] - dlt);
                    }
                    db[c2] = to_bf16x8(x);
                }
                // dQ^T[d, row] += K^T[d, key] dS^T[key, row] over 16-key chunks 2hb, 2hb+1
                {
                    bf16x8 kt[2 * MD];
#pragma unroll
                    for (int j = 0; j < 2 * MD; ++j) {
                        const char* rows = kb + 16 * D * 2 * (2 * hb + (j & 1));
                        kt[j] = concat(lds_read_tr((const uint16_t*)(rows + kt_off[0][j >> 1])),
                                       lds_read_tr((const uint16_t*)(rows + kt_off[1][j >> 1])));
                    }
#pragma unroll
                    for (int j = 0; j < 2 * MD; ++j) acc[j >> 1] = mfma32(kt[j], db[j & 1], acc[j >> 1]);
                    pipeline_reads_mfma<2 * MD, kReadAhead, 2>();
                }
            }
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
        if (kTileLog && a.tile_log != nullptr) {
            const int fl = (T.b < 0 || T.b >= a.batch ? kLogBadBatch : 0) |
                           (T.h < 0 || T.h >= H ? kLogBadHead : 0) |
                           (T.t < 0 || T.k0 < 0 || T.t * kFwdBlockM >= Lq ? kLogBadTile : 0);
            tile_log(a.tile_log, a.tile_log_cap, ti - t_begin,
                     {2, w, T.b, T.h, T.t + a.chunk_div * T.k0, T.work, s, fl});
        }
    }
    if (BCAST && ATOMIC) {
        // this worker's sum over its tiles (all of one (head, Q tile) group)
        // added into dq_accum, element by element, with fp32 atomic adds (a
        // worker without tiles adds nothing)
        if (t_begin < t_end) {
            const TileInfo T0 = tile_info(t_begin);
            float* acc0 = a.dq_accum + (int64_t)T0.h * D;
            stage_out([&](int r, int chunk, const f32x4& x) {
                const int row = T0.t * kFwdBlockM + r;
                if (row < a.lq) {
                    float* p = acc0 + (int64_t)row * H * D + 4 * chunk;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        __hip_atomic_fetch_add(p + j, x[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            });
        }
    } else if (BCAST) {
        // this worker's partial sum over its tiles (all of one (head, Q tile)
        // group): rows 0..255 of the tile, fp32 (zeros for a worker without
        // tiles, so that the reduce reads every partial unconditionally)
        float* part = a.partial + (int64_t)w * kFwdBlockM * D;
        stage_out([&](int r, int chunk, const f32x4& x) {
            *(f32x4*)(part + (int64_t)r * D + 4 * chunk) = x;
        });
    }
}

// dq_accum[row, h, :] = sum over the group's workers w (in order) of
// partial[w][row % 256][:], dq = bf16 of it. A workgroup covers 64 items
// (16 bytes of a (row, head)); its 4 waves sum quarters of the worker range
// and the quarters are added in wave order.
template <int D>
__global__ void __launch_bounds__(256) dq_reduce_kernel(DqReduceArgs a) {
    constexpr int C4 = D / 4;
    __shared__ f32x4 part[4][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t items = (int64_t)a.lq * a.num_heads * C4;
    const int64_t item = (int64_t)blockIdx.x * 64 + lane;
    const int nqt = (a.lq + kFwdBlockM - 1) / kFwdBlockM;
    const int64_t G = (int64_t)a.num_heads * nqt;
    f32x4 sum = f32x4{};
    int64_t out = 0;
    int row = 0;
    if (item < items) {
        const int c4 = (int)(item % C4);
        const int64_t rh = item / C4;
        const int h = (int)(rh % a.num_heads);
        row = (int)(rh / a.num_heads);
        out = rh * D + 4 * c4;
        const int64_t g = (int64_t)h * nqt + row / kFwdBlockM;
        const int w0 = (int)(g * a.num_workers / G), w1 = (int)((g + 1) * a.num_workers / G);
        const int nw = w1 - w0;
        const int q0 = w0 + (nw * wave) / 4, q1 = w0 + (nw * (wave + 1)) / 4;
        const float* src = a.partial + (int64_t)(row % kFwdBlockM) * D + 4 * c4;
        // null worker_ptr: the plan has no tiles, dQ = 0. The loads of 8
        // partials are issued before their adds (same order of addition)
        if (a.worker_ptr != nullptr) {
#pragma unroll 8
            for (int wk = q0; wk < q1; ++wk) sum += *(const f32x4*)(src + (int64_t)wk * kFwdBlockM * D);
        }
    }
    part[wave][lane] = sum;
    __syncthreads();
    if (wave == 0 && item < items) {
        const f32x4 x = ((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane];
        *(f32x4*)(a.dq_accum + out) = x;
        *(bf16x4*)(a.dq + out) = to_bf16x4(x);
    }
}

// dq_accum = 0 (the atomic reduction adds into it)
__global__ void __launch_bounds__(256) dq_zero_kernel(float* __restrict__ acc, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        ((f32x4*)acc)[i] = f32x4{};
}

// dq = bf16(dq_accum), 4 elements per thread
__global__ void __launch_bounds__(256) dq_convert_kernel(const float* __restrict__ acc,
                                                          uint16_t* __restrict__ dq, int64_t n4) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        ((bf16x4*)dq)[i] = to_bf16x4(((const f32x4*)acc)[i]);
}

template <int D, int MODE, bool BCAST, bool ATOMIC = false>
int32_t launch(const DqArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((dq_kernel<D, MODE, BCAST, ATOMIC>), dim3(a.num_workers), dim3(kThreads), 0,
                       stream, a);
    return (int32_t)hipGetLastError();
}

template <int D>
int32_t launch_d(const DqArgs& a, Mode mode, bool bcast, bool atomic, hipStream_t s) {
    if (mode == kCausal) return launch<D, kCausal, false>(a, s);
    if (mode == kSparse) {
        if (!bcast) return launch<D, kSparse, false>(a, s);
        return atomic ? launch<D, kSparse, true, true>(a, s) : launch<D, kSparse, true>(a, s);
    }
    if (!bcast) return launch<D, kDense, false>(a, s);
    return atomic ? launch<D, kDense, true, true>(a, s) : launch<D, kDense, true>(a, s);
}

int grid_for(int64_t n4) { return (int)std::max<int64_t>(1, std::min<int64_t>((n4 + 255) / 256, 2048)); }

}  // namespace

int32_t launch_dq(const DqArgs& a, int32_t head_dim, Mode mode, bool broadcast, bool atomic,
                  void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (head_dim == 64) return launch_d<64>(a, mode, broadcast, atomic, s);
    return launch_d<128>(a, mode, broadcast, atomic, s);
}

int32_t launch_dq_zero(float* dq_accum, int64_t n, void* stream) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(dq_zero_kernel, dim3(grid_for(n / 4)), dim3(256), 0, (hipStream_t)stream,
                       dq_accum, n / 4);
    return (int32_t)hipGetLastError();
}

int32_t launch_dq_convert(const float* dq_accum, uint16_t* dq, int64_t n, void* stream) {
    if (n == 0) return 0;
    hipLaunchKernelGGL(dq_convert_kernel, dim3(grid_for(n / 4)), dim3(256), 0, (hipStream_t)stream,
                       dq_accum, dq, n / 4);
    return (int32_t)hipGetLastError();
}

int32_t launch_dq_reduce(const DqReduceArgs& a, int32_t head_dim, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const int64_t items = (int64_t)a.lq * a.num_heads * (head_dim / 4);
    if (items == 0) return 0;
    const dim3 grid((unsigned)((items + 63) / 64));
    if (head_dim == 64) hipLaunchKernelGGL(dq_reduce_kernel<64>, grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL(dq_reduce_kernel<128>, grid, dim3(256), 0, s, a);
    return (int32_t)hipGetLastError();
}

}  // namespace jfa
