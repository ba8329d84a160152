// Jagged FlashAttention backward for gfx950: preprocess and the KV-stationary
// dK/dV pass (the dQ pass is Q-stationary, in its own kernel).
//
//   1. preprocess: delta = rowsum(dO * O) in fp32 (the standard FlashAttention
//      backward step; the pages only name the backward's persistent, tiled
//      structure: "Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell"
//      (ainewsbites.com), section "Optimizations layered on top"). A stage of
//      its own for callers that want delta alone: the full backward forms it
//      inside the dQ pass, which runs first;
//   2. dK/dV: one persistent workgroup of 8 waves per CU walking a KV-tile
//      plan. A workgroup owns a 256-key KV tile (32 keys per wave, K in VGPRs
//      as a B operand, V in LDS) and streams the 32-row Q/dO blocks that see
//      it. The worker's blocks form one stream across its tiles: Q and dO of
//      block j+2 are copied global -> LDS with direct-to-LDS loads while block
//      j is computed. dK and dV stay in registers for the whole tile and
//      leave as whole rows through LDS.
//
// Per Q block and wave (keys on lanes, query rows in registers):
//   S   = Q K^T          A = Q rows from LDS,    B = K (VGPRs)
//   P   = exp2(S*scale*log2e - LSE*log2e)
//   dP  = dO V^T         A = dO rows from LDS,   B = V rows from LDS
//   dS  = P * (dP - delta)
//   dV^T += dO^T P       A = dO^T: transposed reads of the dO rows, B = P
//   dK^T += Q^T dS       A = Q^T: transposed reads of the Q rows,  B = dS
// (a transposed read of a 16-lane group takes the 4 rows that the lane's P or
// dS registers hold, in their order, so no transposed copy is made)
#include <climits>

#include "qtile.h"

namespace jfa {
namespace {

using namespace qtile;

constexpr int kAhead = 2;            // block j+2 is copied while block j is computed
constexpr int kSlots = kAhead + 1;   // Q/dO ring: blocks j .. j+kAhead
constexpr int kReadAhead = 4;        // LDS operand reads kept in flight ahead of the MFMAs
static_assert(kBwdBlockN == 32 * kWaves && kBwdBlockM == 32, "dK/dV tile geometry");

template <int D>
struct DkdvLds {
    static constexpr int QB = kBwdBlockM * D * 2;            // a Q or dO block [32][D] bf16
    static constexpr int ROWV = 2 * QB;                       // LSE*log2e [32], delta [32] fp32
    static constexpr int SLOT = 2 * QB + 512;                 // Q, dO, row values
    static constexpr int RING = 0;                            // kSlots slots
    static constexpr int ST = RING + kSlots * SLOT;           // epilogue staging, one area per wave
    static constexpr int ST_WAVE = 16 * D * 2;                // 16 rows of one wave
    static constexpr int V = ST + kWaves * ST_WAVE;           // V tile [256][D]
    static constexpr int BYTES = V + kBwdBlockN * D * 2;
};

template <int D, int MODE, bool BCAST>
__global__ void __launch_bounds__(kThreads, 1) dkdv_kernel(BwdArgs a) {
    using LY = DkdvLds<D>;
    __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];
    constexpr int KC = D / 16;              // 16-wide d chunks of S and dP
    constexpr int MD = D / 32;              // 32-row d blocks of dK^T, dV^T
    constexpr int CH = D / 8;               // 16-byte chunks per row
    constexpr int QPW = (2 * kBwdBlockM * CH) / (64 * kWaves);   // Q + dO copies per wave per block
    constexpr int VPW = (kBwdBlockN * CH) / (64 * kWaves);       // V copies per wave per tile
    static_assert(QPW >= 1, "copy split");

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;
    // row stride in bytes, below 2^24 (H bounded by the planner): a block's
    // rows are 24-bit multiples of it from its first row
    const uint32_t rs_b = (uint32_t)rs * 2;

    constexpr int QH = (kBwdBlockM * CH) / 64;   // copies per tensor (Q or dO) per block
    // A operands: Q / dO row lr, chunk 2kc + hf; the V rows (B operand) of
    // this wave's keys use the same pattern 32 rows further per wave
    // (2kc + hf) ^ x = 2 (kc ^ x/2) + ((hf ^ x) & 1): one base and one XOR mask
    const int ro_x = swz_rt<D>(lr);
    const int ro_base = lr * D * 2 + (((hf ^ ro_x) & 1) << 4), ro_xh = ro_x >> 1;
    auto row_off = [&](int kc) { return ro_base + ((kc ^ ro_xh) << 5); };
    // Q^T / dO^T [32md + lr][rows of chunk c, in P's and dS's order]: two
    // transposed reads of the natural rows (chunk c and dO's place after Q in
    // the slot are immediate offsets)
    int to_off[2][MD];
    tr_operand_offsets<D>(lane, to_off);

    const int w = worker_id(a.num_workers);
    const int t_begin = ld_uniform(a.worker_ptr + w), t_end = ld_uniform(a.worker_ptr + w + 1);
    const int kv_tiles_per_row = (a.mask_kv_blocks + 1) >> 1;

    struct KvTile {
        int b, h, n, work, kv0, L, q0, Lq, orow0, r0;
        const int* sp;
    };
    auto tile_info = [&](int ti) {
        KvTile T;
        T.b = ld_uniform(a.tiles + 4 * ti + 0);
        T.h = ld_uniform(a.tiles + 4 * ti + 1);
        T.n = ld_uniform(a.tiles + 4 * ti + 2);
        T.work = ld_uniform(a.tiles + 4 * ti + 3);
        T.kv0 = ld_uniform(a.kv_off + T.b);
        T.L = ld_uniform(a.kv_off + T.b + 1) - T.kv0;
        if (BCAST) {
            T.q0 = 0;
            T.Lq = a.lq;
            T.orow0 = T.b * a.lq;
        } else {
            T.q0 = ld_uniform(a.q_off + T.b);
            T.Lq = ld_uniform(a.q_off + T.b + 1) - T.q0;
            T.orow0 = T.q0;
        }
        // banded: the first Q block whose rows see the tile's keys (rows
        // i >= j - right for key j)
        T.r0 = MODE == kCausal && a.win_right >= 0 ? max(0, T.n * kBwdBlockN - a.win_right) / kBwdBlockM : 0;
        T.sp = nullptr;
        if (MODE == kSparse) T.sp = a.sp_idx + ld_uniform(a.sp_ptr + T.b * kv_tiles_per_row + T.n);
        return T;
    };
    // Q block (32-row block index in the sequence) at position i of a tile
    auto q_block = [&](const KvTile& T, int i) -> int {
        if (MODE == kSparse) return 4 * (ld_uniform(T.sp + (i >> 2)) >> 2) + (i & 3);
        return T.r0 + i;
    };

    // ---- loader: the worker's Q/dO blocks in plan order, kAhead blocks ahead
    int l_ti = t_begin, l_i = 0, l_slot = 0;
    KvTile LT;
    LT.work = 0;
    auto l_settle = [&]() {
        while (l_i >= LT.work) {
            ++l_ti;
            l_i = 0;
            if (l_ti >= t_end) return;
            LT = tile_info(l_ti);
        }
    };
    // row values of the loader's latest block: wave 0 lanes 0-31 LSE, 32-63
    // delta of rows 0..31 (raw, with a flag for rows inside the sequence; made
    // into exp2-domain values when written to LDS one iteration later)
    float pend_v = 0.f;
    bool pend_in = false;
    // rows past the sequence are clamped to its last row (finite data; their
    // LSE is set to +inf so that P = 0)
    auto l_issue = [&]() {
        if (l_ti >= t_end) return;
        const int rb = q_block(LT, l_i);
        char* dst = smem + LY::RING + (l_slot % kSlots) * LY::SLOT;
        // the block's first Q and dO rows (wave-uniform); a partial last
        // block moves its rows past the sequence back onto the last row
        const int64_t hq = (int64_t)LT.h * D;
        const uint16_t* qb0 = a.q + (int64_t)(LT.q0 + kBwdBlockM * rb) * rs + hq;
        const uint16_t* db0 = a.d_o + (int64_t)(LT.orow0 + kBwdBlockM * rb) * rs + hq;
        const int last = LT.Lq - 1 - kBwdBlockM * rb;
        // copy u of this wave is copy g = QPW*wave + u of the block (first
        // half Q, second half dO) and fills chunk positions 64 (g mod QH) +
        // lane: row r, stored chunk cp (g and the tensor are wave-uniform)
#pragma unroll
        for (int u = 0; u < QPW; ++u) {
            const int g = QPW * wave + u;
            const bool is_do = g >= QH;
            const int p = 64 * (g % QH) + lane;
            const int r = p / CH, cp = p % CH;
            const uint32_t off = __umul24((uint32_t)min(r, last), rs_b) + 16 * (cp ^ swz_rt<D>(r));
            load_lds16_s(is_do ? db0 : qb0, off, dst + (is_do ? LY::QB : 0) + 1024 * (g % QH));
        }
        if (wave == 0) {
            const int row = kBwdBlockM * rb + lr;
            const int qi = min(row, LT.Lq - 1);
            const int64_t idx = (int64_t)LT.h * a.total_q + LT.orow0 + qi;
            pend_v = hf ? a.delta[idx] : a.lse[idx];
            pend_in = row < LT.Lq;
        }
        ++l_slot;
        ++l_i;
        l_settle();
    };
    auto put_rowvals = [&](int s) {   // row values of block s (loaded one step earlier)
        if (wave == 0) {
            float* rv = (float*)(smem + LY::RING + (s % kSlots) * LY::SLOT + LY::ROWV);
            float x;
            if (hf == 0) x = (!pend_in || pend_v == -INFINITY) ? INFINITY : pend_v * kLog2e;
            else x = pend_in ? -pend_v : 0.f;   // -delta: the dP accumulators start there
            rv[lane] = x;
        }
    };
    if (t_begin < t_end) {
        LT = tile_info(t_begin);
        l_settle();
    }
    int total = 0;   // stream length
    for (int ti = t_begin; ti < t_end; ++ti) total += ld_uniform(a.tiles + 4 * ti + 3);
    if (total > 0) {   // block 0 landed and prepared, block 1 in flight
        l_issue();
        wait_vmem();
        __syncthreads();
        put_rowvals(0);
        l_issue();
    }

    // V tile of T to LDS and this wave's K rows of T to VGPRs (keys past the
    // sequence are clamped to its last row; their dK/dV are not stored). The
    // addresses are recomputed per tile rather than kept live across it.
    bf16x8 kf[KC];
    auto load_kv = [&](const KvTile& T) {
        const int64_t kvrow0 = (int64_t)T.kv0 * rs + (int64_t)T.h * D;
        const int lane_t = opaque(lane);
#pragma unroll
        for (int u = 0; u < VPW; ++u) {   // copy u fills chunk positions 64 (VPW wave + u) + lane
            const int p = 64 * (VPW * wave + u) + lane_t;
            const int r = p / CH, cp = p % CH;
            const int key = min(T.n * kBwdBlockN + r, T.L - 1);
            load_lds16(a.v + kvrow0 + (int64_t)key * rs + 8 * (cp ^ swz_rt<D>(r)),
                       smem + LY::V + 1024 * (VPW * wave + u));
        }
        const int key = min(T.n * kBwdBlockN + 32 * wave + (lane_t & 31), T.L - 1);
        const uint16_t* kp = a.k + kvrow0 + (int64_t)key * rs + 8 * (lane_t >> 5);
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) kf[kc] = load_bf16x8(kp + 16 * kc);
    };
    if (t_begin < t_end) load_kv(tile_info(t_begin));
    wait_vmem();
    __syncthreads();
    // This wave's 32 rows of a tile's K or V (row-contiguous direct-to-LDS
    // copies) into its own V rows, the layout load_kv gives V
    auto copy_rows = [&](const uint16_t* src, const KvTile& T) {
        const int64_t kvrow0 = (int64_t)T.kv0 * rs + (int64_t)T.h * D;
        const int lane_t = opaque(lane);
#pragma unroll
        for (int u = 0; u < VPW; ++u) {
            const int p = 64 * (VPW * wave + u) + lane_t;
            const int r = p / CH, cp = p % CH;
            const int key = min(T.n * kBwdBlockN + r, T.L - 1);
            load_lds16(src + kvrow0 + (int64_t)key * rs + 8 * (cp ^ swz_rt<D>(r)),
                       smem + LY::V + 1024 * (VPW * wave + u));
        }
    };

    int s = 0;   // stream position of the consumer
    for (int ti = t_begin; ti < t_end; ++ti) {
        const KvTile T = tile_info(ti);
        const int key0 = T.n * kBwdBlockN + 32 * wave;   // first key of this wave (tile-local)
        const bool wave_keys = key0 < T.L;               // wave-uniform
        f32x16 dk_acc[MD], dv_acc[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) {
            dk_acc[md] = f32x16{};
            dv_acc[md] = f32x16{};
        }
        const char* vb = smem + LY::V + 32 * wave * D * 2;   // this wave's V rows

        for (int i = 0; i < T.work; ++i, ++s) {
            if (i > 0) wait_vmem();   // block s+1 landed (the only copies in flight)
            // every wave is past block s-1: its slot is free
            __syncthreads();
            // (past the end of the stream this works on stale, unread data)
            put_rowvals(s + 1);
            l_issue();                               // block s+kAhead

            const int rb = q_block(T, i);
            bool skip = !wave_keys, masked = false;
            if (MODE == kCausal) {
                // row i sees key j iff j - wr <= i <= j + wl: rows R0..R1 and
                // this wave's keys K0..K1 meet iff R1 >= K0 - wr and R0 <=
                // K1 + wl; every pair is visible iff R0 >= K1 - wr and R1 <= K0 + wl
                const int64_t R0 = kBwdBlockM * rb, R1 = R0 + kBwdBlockM - 1, K0 = key0, K1 = key0 + 31;
                skip = skip || (a.win_right >= 0 && R1 < K0 - a.win_right) ||
                       (a.win_left >= 0 && R0 > K1 + a.win_left);
                masked = (a.win_right >= 0 && R0 < K1 - a.win_right) ||
                         (a.win_left >= 0 && R1 > K0 + a.win_left);
            } else if (MODE == kSparse) {
                skip = skip || !((ld_uniform(T.sp + (i >> 2)) >> (wave >> 2)) & 1);
            }
            if (skip) continue;
            const char* qb = smem + LY::RING + (s % kSlots) * LY::SLOT;
            const char* db = qb + LY::QB;
            const float* rv = (const float*)(qb + LY::ROWV);

            // dP accumulates onto -delta (row values), so it ends as dP - delta
            f32x16 sc = f32x16{}, dp;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 d4 = *(const f32x4*)(rv + 32 + 8 * g + 4 * hf);
#pragma unroll
                for (int j = 0; j < 4; ++j) dp[4 * g + j] = d4[j];
            }
            {
                bf16x8 qa[KC], da[KC], vf[KC];
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    qa[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qb + row_off(kc)));
                    da[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(db + row_off(kc)));
                    vf[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(vb + row_off(kc)));
                }
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    sc = mfma32(qa[kc], kf[kc], sc);
                    dp = mfma32(da[kc], vf[kc], dp);
                }
                // two d chunks of reads ahead, then 2 MFMAs per 3 reads
                __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
                for (int kc = 2; kc < KC; ++kc) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            // P and dS; register r is query row 32rb + 8(r/4) + 4hf + r%4, the
            // column this lane's key 32wave + lr (tile-local). Banded: with
            // c = 8(r/4) + r%4, key - row = base - c, visible iff
            // c_lo <= c <= c_hi
            int c_lo = INT_MIN, c_hi = INT_MAX;
            if (MODE == kCausal && masked) {
                const int base = key0 + lr - kBwdBlockM * rb - 4 * hf;
                if (a.win_right >= 0) c_lo = base - a.win_right;
                if (a.win_left >= 0) c_hi = base + a.win_left;
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int row = 8 * g + 4 * hf;
                const f32x4 l4 = *(const f32x4*)(rv + row);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float p = __builtin_amdgcn_exp2f(fmaf(sc[4 * g + j], a.scale_log2, -l4[j]));
                    if (MODE == kCausal && masked) {
                        const int c = 8 * g + j;
                        if (c < c_lo || c > c_hi) p = 0.f;
                    }
                    sc[4 * g + j] = p;
                    dp[4 * g + j] = p * dp[4 * g + j];
                }
            }
            bf16x8 pb[2], sb[2];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                f32x8 x, y;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    x[j] = sc[8 * c + j];
                    y[j] = dp[8 * c + j];
                }
                pb[c] = to_bf16x8(x);
                sb[c] = to_bf16x8(y);
            }
            // dV^T += dO^T P ; dK^T += Q^T dS over the block's 32 rows
            {
                // (one address per (t, md), shared by Q and dO)
                const uint32_t lq = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)qb;
                uint32_t ta[2][MD];
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int md = 0; md < MD; ++md) ta[t][md] = lq + to_off[t][md];
                bf16x8 dta[2 * MD], qta[2 * MD];
#pragma unroll
                for (int j = 0; j < 2 * MD; ++j) {
                    const int o = 16 * D * 2 * (j & 1);
                    dta[j] = concat(lds_read_tr_at(ta[0][j >> 1], LY::QB + o),
                                    lds_read_tr_at(ta[1][j >> 1], LY::QB + o));
                    qta[j] = concat(lds_read_tr_at(ta[0][j >> 1], o), lds_read_tr_at(ta[1][j >> 1], o));
                }
#pragma unroll
                for (int j = 0; j < 2 * MD; ++j) {
                    dv_acc[j >> 1] = mfma32(dta[j], pb[j & 1], dv_acc[j >> 1]);
                    dk_acc[j >> 1] = mfma32(qta[j], sb[j & 1], dk_acc[j >> 1]);
                }
                pipeline_reads_mfma<4 * MD, kReadAhead, 2>();
            }
        }

        // ---- tile end, wave by wave: a wave's V rows, K rows and staging area
        // are its own, so no workgroup barrier is needed here (the next
        // block's barrier orders the ring). dK = scale * (dK^T)^T and dV leave
        // as bf16 rows through the wave's staging area, 16 keys at a time.
        // Meanwhile the wave fetches the next tile's K rows into its own V
        // rows with row-contiguous copies (row-strided fragment loads cost the
        // vector memory unit one cache line per key and instruction; the V
        // reads of its last block were consumed by its dP products), reads
        // its K fragments from there once dK is out, and then fetches the
        // next V rows in their place while dV leaves.
        // (The banded mode keeps the direct K loads: the staged form spills
        // there.)
        if (kTileLog && a.tile_log != nullptr) {
            const int fl = (T.b < 0 || T.b >= a.batch ? kLogBadBatch : 0) |
                           (T.h < 0 || T.h >= H ? kLogBadHead : 0) |
                           (T.n < 0 || T.n * kBwdBlockN >= T.L ? kLogBadTile : 0);
            tile_log(a.tile_log, a.tile_log_cap, ti - t_begin, {1, w, T.b, T.h, T.n, T.work, s, fl});
        }
        constexpr bool kStageK = MODE != kCausal;
        const bool has_next = ti + 1 < t_end;
        const KvTile NT = has_next ? tile_info(ti + 1) : T;
        if (has_next) {
            if (kStageK) copy_rows(a.k, NT);
            else load_kv(NT);
        }
        {
            const int64_t kvrow0 = (int64_t)T.kv0 * rs + (int64_t)T.h * D;
            char* st = smem + LY::ST + wave * LY::ST_WAVE;
            const int lane_e = opaque(lane), lr_e = lane_e & 31, hf_e = lane_e >> 5;
#pragma unroll
            for (int pass = 0; pass < 4; ++pass) {   // dK keys 0-15, 16-31, then dV
                if (kStageK && pass == 2 && has_next) {
                    wait_vmem();   // the K rows landed (and the dK stores are done)
                    wave_sync_lds();
#pragma unroll
                    for (int kc = 0; kc < KC; ++kc)
                        kf[kc] = __builtin_bit_cast(bf16x8, *(const u32x4*)(vb + row_off(kc)));
                    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): read before overwritten
                    wave_sync_lds();
                    copy_rows(a.v, NT);
                }
                const int rd = pass & 1;
                if ((lr_e >> 4) == rd) {
                    const int r = lr_e & 15;
#pragma unroll
                    for (int md = 0; md < MD; ++md)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            f32x4 x;
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                x[j] = pass < 2 ? dk_acc[md][4 * g + j] * a.scale : dv_acc[md][4 * g + j];
                            const int chunk = 4 * md + g;
                            *(bf16x4*)(st + r * D * 2 + ((chunk ^ (r & (CH - 1))) << 4) + 8 * hf_e) =
                                to_bf16x4(x);
                        }
                }
                wave_sync_lds();
                uint16_t* out = pass < 2 ? a.dk : a.dv;
#pragma unroll
                for (int v = 0; v < 16 * CH / 64; ++v) {
                    const int k = lane_e + 64 * v;
                    const int r = k / CH, chunk = k % CH;
                    const u32x4 x = *(const u32x4*)(st + r * D * 2 + ((chunk ^ (r & (CH - 1))) << 4));
                    const int key = key0 + 16 * rd + r;
                    if (key < T.L) *(u32x4*)(out + kvrow0 + (int64_t)key * rs + 8 * chunk) = x;
                }
                wave_sync_lds();
            }
        }
        // this wave's next V and K rows landed (and its stores are done)
        wait_vmem();
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
