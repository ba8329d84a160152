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
//   - one persistent workgroup of 8 waves per CU walking a host-built tile
//     list (sorted by KV work, dealt in zigzag order). A tile is 256 query
//     rows, 32 per wave, so a 64-key K/V block brought into LDS serves 256
//     rows (for a broadcast Q of 256 rows: every K/V row is read once);
//   - the worker's blocks form one stream across its tiles: K and V of block
//     j+3 are copied global -> LDS with direct-to-LDS loads while block j is
//     computed (4-slot K and V rings; a block's copies get two iterations to
//     land), so the copy costs no VGPRs and no LDS store instructions, and
//     tile boundaries do not drain the pipe;
//   - the V^T operands of O^T += V^T P^T come straight from the natural V
//     block through transposed LDS reads (ds_read_b64_tr_b16): each 16-lane
//     group reads the 4 key rows that the lane's P^T registers hold, in
//     their order, so no transposed copy of V is made (MXFP8 reads its E4M3
//     V^T operands the same way with byte-transposed reads);
//   - per wave: S^T = K Q^T (32x32x16 bf16 MFMA, Q in VGPRs as the B operand,
//     so a lane owns one query row and row max / row sum stay in-lane), fp32
//     online softmax in the exp2 domain (bf16: the running max moves, and
//     O^T is rescaled, only when a row's max rises by more than 2^8; MXFP8:
//     whenever it rises), O^T += V^T P^T with P^T straight from the
//     accumulators;
//   - the peel is per block, not per loop: scalar flags computed for each
//     block send it down the bulk path (no mask arithmetic) or the masked
//     tail path (partial last block, causal diagonal) with a wave-uniform
//     branch, and blocks a wave's rows cannot see (causal, or dropped by its
//     block-sparse mask row) are skipped by that wave. The block body is
//     compiled once: two copies of it (a bulk loop and a tail loop) would
//     double the kernel's largest code region for the few scalar
//     instructions the flags cost;
//   - O leaves through a per-wave LDS staging area (in the K and V slots the
//     tile's last block has released) as whole 16-byte-per-lane rows, so
//     each store instruction writes 4 full rows.
// Every LDS tile is XOR-swizzled at 16-byte granularity so that the MFMA
// operand reads and the transposed reads are free of bank conflicts (reads
// see 64 banks x 4 bytes; a half wave's transposed reads cover 4 rows x 64
// bytes).
#include "mxops.h"
#include "qtile.h"

namespace jfa {
namespace {

// bf16 forward: the online softmax's running max is moved only when a block
// raises some row's max by more than this (exp2 domain), so P <= 2^8: exact
// after the final O / l, safe in bf16 and fp32, and the O^T rescale runs
// about once per tile instead of on most blocks.
constexpr float kMaxSlack = 8.0f;

using namespace qtile;
using namespace mxops;
constexpr int kAhead = 3;        // block j+kAhead is copied while block j is computed
constexpr int kKSlots = kAhead + 1;   // K ring: blocks j .. j+kAhead
constexpr int kReadAhead = 4;    // LDS operand reads kept in flight ahead of the MFMAs
constexpr int kStageRows = 16;   // O rows per wave per epilogue round


template <int D, bool MX>
struct FwdLds {
    static constexpr int VSLOTS = kAhead + 1;                  // V ring: blocks j .. j+kAhead
    static constexpr int BLK = kFwdBlockN * D * 2;            // one K or V block
    static constexpr int K = 0;                                // kKSlots K blocks
    static constexpr int V = K + kKSlots * BLK;                // VSLOTS V blocks
    static constexpr int CLAIM = V + VSLOTS * BLK;             // int [2][64]: claimed tiles
    static constexpr int QUEUE = CLAIM + 2 * 64 * 4;           // int [kWaves][8]: tile queues
    static constexpr int BYTES = QUEUE + kWaves * 8 * 4;
    static constexpr int OST_WAVE = kStageRows * D * 2;        // O staging of one wave
    static_assert(4 * OST_WAVE == BLK, "staging: 4 waves per released block");
};

// MXFP8 (D = 128): E4M3 K/V blocks are half the size; their scales ride
// along (K: 4 bytes per key, V: 2 x 128 bytes per 64-key block); the V^T
// operands are byte-transposed reads of the natural V block; O has a staging
// area of its own.
template <int D>
struct FwdLds<D, true> {
    static constexpr int VSLOTS = kAhead + 1;
    static constexpr int BLK = kFwdBlockN * D;                 // one E4M3 K or V block
    static constexpr int SC = 256;                              // its scales
    static constexpr int K = 0;                                 // kKSlots K blocks [64][128]
    static constexpr int KS = K + kKSlots * BLK;                // kKSlots K scales [64][4]
    static constexpr int V = KS + kKSlots * SC;                 // VSLOTS V blocks [64][128]
    static constexpr int VS = V + VSLOTS * BLK;                 // kKSlots V scales [2][128]
    static constexpr int OST_WAVE = kStageRows * D * 2;
    static constexpr int OST = VS + kKSlots * SC;               // O staging, kWaves areas
    static constexpr int CLAIM = OST + kWaves * OST_WAVE;
    static constexpr int QUEUE = CLAIM + 2 * 64 * 4;
    static constexpr int BYTES = QUEUE + kWaves * 8 * 4;
    static_assert(D == 128 && BLK == 64 * kThreads / 4, "one 16-byte copy per thread per block");
};

template <int D, int MODE, bool BCAST, bool MX>
__global__ void __launch_bounds__(kThreads, 1) fwd_kernel(FwdArgs a) {
    using LY = FwdLds<D, MX>;
    constexpr int kVSlots = LY::VSLOTS;
    __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];
    constexpr int KC = D / 16;              // 16-wide d chunks of S^T = K Q^T
    constexpr int MD = D / 32;              // 32-row d blocks of O^T
    constexpr int CH = D / 8;               // 16-byte chunks per K/V row
    constexpr int LPW = (kFwdBlockN * CH) / (64 * kWaves);   // K (and V) loads per wave per block

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;

    // direct-to-LDS copy: load u of this wave fills chunk positions 64u'+lane
    // (u' = LPW*wave + u) of a block, i.e. key r, stored chunk cp; the lane's
    // byte offsets from the block's first key row (K and V swizzles; rows
    // fit 32 bits: at most 64 rows of H*D*2 bytes, H bounded by the planner)
    const uint32_t rs_b = (uint32_t)rs * 2;
    int ld_row[LPW];
    uint32_t ld_ok[LPW], ld_ov[LPW];
#pragma unroll
    for (int u = 0; u < LPW; ++u) {
        const int p = 64 * (LPW * wave + u) + lane;
        const int r = p / CH, cp = p % CH;
        ld_row[u] = r;
        ld_ok[u] = r * rs_b + 16 * (cp ^ swz_k<D>(r));
        ld_ov[u] = r * rs_b + 16 * (cp ^ swz_rt<D>(r));
    }
    // S^T operand: K row 32mb + lr, chunk 2kc + hf (swz_k(32mb + lr) == swz_k(lr))
    int k_off[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) k_off[kc] = lr * D * 2 + (((2 * kc + hf) ^ swz_k<D>(lr)) << 4);
    // O^T operand V^T[32md + lr][keys of chunk c, in P^T's order]: two
    // transposed reads of the natural V block
    int vo_off[2][MD];
    tr_operand_offsets<D>(lane, vo_off);

    const int w = worker_id(a.num_workers);
    const int t_begin = ld_uniform(a.worker_ptr + w), t_end = ld_uniform(a.worker_ptr + w + 1);
    const bool dynamic = a.counter != nullptr;

    auto tile_info = [&](int ti) {
        return qtile::tile_info<MODE>(a.tiles, a.kv_off, a.sp_ptr, a.sp_idx, a.mask_q_blocks, 0,
                                      a.win_left, a.win_right, ti);
    };
    auto seq_block = [&](const TileInfo& T, int i) { return qtile::seq_block<MODE>(T, i); };
    // Q / O rows of a tile's sequence: first Q row, row count, first O row
    auto rows_of = [&](const TileInfo& T, int& q0, int& Lq, int& orow0) {
        if (BCAST) {
            q0 = 0;
            Lq = a.lq;
            orow0 = T.b * a.lq;
        } else {
            q0 = ld_uniform(a.q_off + T.b);
            Lq = ld_uniform(a.q_off + T.b + 1) - q0;
            orow0 = q0;
        }
    };

    // ---- the worker's tiles. Static plan: t_begin .. t_end-1. Dynamic plan:
    // tile t_begin (= w), then tiles claimed one at a time from the counter
    // (num_workers + its old value) until a claim falls past the list. A claim
    // is made (lane 0 of wave 0) when the loader starts on the last block of
    // its tile, a few blocks before this workgroup needs the next tile, so the
    // next tile goes to a workgroup that is about to be free; its value
    // reaches the other waves through LDS after the next barrier, when the
    // loader needs it. The loader hands each tile with blocks to the consumer
    // through a per-wave queue in LDS (it is at most kAhead blocks ahead, so
    // at most kAhead + 1 tiles are queued); a tile without blocks (an empty
    // sequence, or no kept block) gets O = 0, LSE = -inf from the loader.
    int* const claim_lds = (int*)(smem + LY::CLAIM);
    int* const queue_lds = (int*)(smem + LY::QUEUE) + 8 * wave;
    int q_head = 0, q_tail = 0;          // consumer queue cursors (wave-uniform)
    int l_next = dynamic && t_begin < t_end ? t_begin : -1;   // tile after the loader's
    bool l_have = dynamic;               // l_next is known
    bool l_claiming = false;             // a claim is made and not yet received
    int n_claims = 0;                    // claims received (parity picks the LDS slot)
    int claim_ret = 0;                   // wave 0, lane 0: the counter's old value
    auto claim = [&]() {
        // One atomic, by lane 0 of wave 0, waited for at once (see
        // atomic_inc_lane0): the other waves go on meanwhile.
        if (wave == 0) claim_ret = atomic_inc_lane0(a.counter);
        l_claiming = true;
    };
    // wave 0 puts a claimed value in LDS before a barrier; every wave reads it
    // (lane 0's) after that barrier. Two slots: a slot is rewritten only after
    // the barrier that follows its read.
    auto publish = [&]() {
        if (l_claiming && wave == 0) claim_lds[64 * (n_claims & 1) + lane] = claim_ret;
    };
    auto receive = [&]() {
        if (l_claiming) {
            const int v = __builtin_amdgcn_readfirstlane(claim_lds[64 * (n_claims & 1)]) + a.num_workers;
            ++n_claims;
            l_claiming = false;
            l_next = (unsigned)v < (unsigned)a.num_tiles ? v : -1;   // past the list: done
            l_have = true;
        }
    };
    auto claim_now = [&]() {   // the next tile is needed before the next barrier
        if (!l_claiming) claim();
        publish();
        __syncthreads();
        receive();
    };
    auto zero_rows = [&](const TileInfo& Z) {   // O = 0, LSE = -inf for the tile's rows
        int q0, Lq, orow0;
        rows_of(Z, q0, Lq, orow0);
        const int r0 = Z.t * kFwdBlockM, r1 = min(Lq, r0 + kFwdBlockM);
        for (int k = tid; k < (r1 - r0) * CH; k += kThreads) {
            const int r = r0 + k / CH, c = k % CH;
            *(u32x4*)(a.o + (int64_t)(orow0 + r) * rs + (int64_t)Z.h * D + 8 * c) = u32x4{0, 0, 0, 0};
        }
        for (int r = r0 + tid; r < r1; r += kThreads) a.lse[(int64_t)Z.h * a.total_q + orow0 + r] = -INFINITY;
    };

    // loader cursor: tile l_ti (info LT), next block l_i, blocks issued l_slot
    int l_ti = t_begin - 1, l_i = 0, l_slot = 0;
    bool l_end = false;
    TileInfo LT;
    LT.work = 0;
    int log_n = 0;   // tiles taken (executed-tile log)
    auto advance = [&]() {   // to the next tile with blocks, or the end
        while (!l_end && l_i >= LT.work) {
            int nt;
            if (dynamic) {
                if (!l_have) claim_now();
                nt = l_next;
                l_have = false;
            } else {
                nt = l_ti + 1 < t_end ? l_ti + 1 : -1;
            }
            if (nt < 0) {
                l_end = true;
                break;
            }
            l_ti = nt;
            l_i = 0;
            LT = tile_info(nt);
            if (kTileLog && a.tile_log != nullptr) {
                int lq0, lLq, lrow0;
                rows_of(LT, lq0, lLq, lrow0);
                const int fl = (LT.b < 0 || LT.b >= a.batch ? kLogBadBatch : 0) |
                               (LT.h < 0 || LT.h >= a.num_heads ? kLogBadHead : 0) |
                               (LT.t < 0 || LT.t * kFwdBlockM >= lLq ? kLogBadTile : 0);
                tile_log(a.tile_log, a.tile_log_cap, log_n++, {0, w, LT.b, LT.h, LT.t, LT.work, -1, fl});
            }
            if (LT.work == 0) {
                zero_rows(LT);
            } else {
                queue_lds[q_tail & 7] = nt;
                ++q_tail;
            }
        }
    };
    // issue the copies of the loader's next block into ring slots (K: slot
    // l_slot % kKSlots, V: l_slot % kVSlots); keys past the sequence are
    // clamped to its last row (always finite data, masked out of the softmax
    // by the tail path)
    auto l_issue = [&]() {
        if (l_i >= LT.work) advance();
        if (l_end) return;
        // the last block of the loader's tile: claim the tile after it now,
        // ahead of the copies
        if (dynamic && l_i == LT.work - 1 && !l_have && !l_claiming) claim();
        const int n = seq_block(LT, l_i);
        const int64_t base = (int64_t)LT.kv0 * rs + (int64_t)LT.h * D;
        char* kdst = smem + LY::K + (l_slot % kKSlots) * LY::BLK;
        char* vdst = smem + LY::V + (l_slot % kVSlots) * LY::BLK;
        if constexpr (MX) {
            // one 16-byte chunk of the K and of the V block per thread: key
            // q/8, stored chunk q%8 (q = 64 wave + lane); the scales of the
            // block's 64 keys (wave 0, a dword per key) and of V's two 32-key
            // blocks (wave 1: lanes 0-31 block 2n, 32-63 block 2n+1, clamped
            // to the sequence's last block)
            const int q = 64 * wave + lane, r = q >> 3, cs = q & 7;
            const int key = min(kFwdBlockN * n + r, LT.L - 1);
            const int64_t row = base + (int64_t)key * rs;
            load_lds16((const uint16_t*)(a.k8 + row + 16 * (cs ^ swz_k8(r))), kdst + 1024 * wave);
            load_lds16((const uint16_t*)(a.v8 + row + 16 * (cs ^ swz_v8(r))), vdst + 1024 * wave);
            if (wave == 0) {
                const int kk = min(kFwdBlockN * n + lane, LT.L - 1);
                load_lds4(a.k_sc + ((int64_t)LT.h * a.total_kv + LT.kv0 + kk) * 4,
                          smem + LY::KS + (l_slot % kKSlots) * LY::SC);
            } else if (wave == 1) {
                const int b0 = ld_uniform(a.v_boff + LT.b), nbk = ld_uniform(a.v_boff + LT.b + 1) - b0;
                const int blk = min(2 * n + (lane >> 5), nbk - 1);
                // (kKSlots deep like K: block s's scales are read at iteration s,
                // after the V slot itself was recycled)
                load_lds4(a.v_sc + ((int64_t)LT.h * a.v_nb + b0 + blk) * D + 4 * (lane & 31),
                          smem + LY::VS + (l_slot % kKSlots) * LY::SC);
            }
        } else {
            // the block's first key row (wave-uniform); a partial last block
            // moves its rows past the sequence back onto the last row
            const int64_t blk0 = base + (int64_t)(kFwdBlockN * n) * rs;
            const uint16_t* kb = a.k + blk0;
            const uint16_t* vb = a.v + blk0;
            const int last = LT.L - 1 - kFwdBlockN * n;
#pragma unroll
            for (int u = 0; u < LPW; ++u) {
                uint32_t back = 0;
                if (last < kFwdBlockN - 1) back = (uint32_t)max(ld_row[u] - last, 0) * rs_b;
                load_lds16_s(kb, ld_ok[u] - back, kdst + 1024 * (LPW * wave + u));
                load_lds16_s(vb, ld_ov[u] - back, vdst + 1024 * (LPW * wave + u));
            }
        }
        ++l_slot;
        ++l_i;
    };
    // MXFP8: this lane's offsets of the byte-transposed V^T reads
    int mx_vo[4];
    if constexpr (MX) mx_tr_offsets(lane, mx_vo);

    // prologue: block 0 landed, blocks 1 .. kAhead-1 in flight
    l_issue();
    if (l_slot > 0) {
        wait_vmem();
        __syncthreads();
#pragma unroll
        for (int k = 1; k < kAhead; ++k) l_issue();
    }

    int s = 0;   // stream position of the consumer
    // the loader queues a tile no later than the iteration that consumes the
    // previous tile's last block, so an empty queue means the end
    while (q_head != q_tail) {
        const int ti = __builtin_amdgcn_readfirstlane(queue_lds[q_head & 7]);
        ++q_head;
        const TileInfo T = tile_info(ti);
        int q0, Lq, orow0;
        rows_of(T, q0, Lq, orow0);
        const int row0 = T.t * kFwdBlockM + 32 * wave;   // first row of this wave
        const int qrow = row0 + lr;
        const bool wave_rows = row0 < Lq;                // wave-uniform
        // Q^T fragments of this lane's row (rows past the sequence read its last
        // row; a tile exists only when Lq >= 1, and a wave without rows skips
        // every block)
        bf16x8 qf[KC];
        i32x8 qf8[2];   // MXFP8: the two 64-d steps (slots as in mx_scores)
        int qsc[2];
        if constexpr (MX) {
            const int qr = q0 + min(qrow, Lq - 1);
            const uint8_t* qp = a.q8 + (int64_t)qr * rs + (int64_t)T.h * D;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const u32x4 lo = *(const u32x4*)(qp + 64 * j + 16 * hf);
                const u32x4 hi = *(const u32x4*)(qp + 64 * j + 32 + 16 * hf);
                qf8[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            }
            const uint32_t qs = *(const uint32_t*)(a.q_sc + ((int64_t)T.h * a.q_rows + qr) * 4);
#pragma unroll
            for (int j = 0; j < 2; ++j) qsc[j] = (qs >> (8 * (2 * j + hf))) & 255;
        } else {
            const int qr = min(qrow, Lq - 1);
            const uint16_t* qp = a.q + (int64_t)(q0 + qr) * rs + (int64_t)T.h * D + 8 * hf;
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) qf[kc] = load_bf16x8(qp + 16 * kc);
        }
        f32x16 oacc[MD];
#pragma unroll
        for (int md = 0; md < MD; ++md) oacc[md] = f32x16{};
        float m_run = -1e30f, l_run = 0.f;

        // The tile's Q rows and the previous tile's stores are younger than
        // the copies in flight: wait for everything once here, so that no
        // load the compiler tracks is pending inside the block loop.
        wait_vmem();
        // S^T of a landed block (K slot of stream position p) into acc
        auto compute_s = [&](f32x16 (&acc)[2], int p) {
            const char* kb = smem + LY::K + (p % kKSlots) * LY::BLK;
            acc[0] = f32x16{};
            acc[1] = f32x16{};
            bf16x8 kf[2 * KC];
#pragma unroll
            for (int j = 0; j < 2 * KC; ++j)
                kf[j] = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + 32 * D * 2 * (j & 1) + k_off[j >> 1]));
#pragma unroll
            for (int j = 0; j < 2 * KC; ++j) acc[j & 1] = mfma32(kf[j], qf[j >> 1], acc[j & 1]);
        };
        // exp2 of the scaled scores against the new running max, their row
        // sum, and P^T as bf16 B operands (chunk c: keys 16c..16c+15)
        auto exp_pack = [&](f32x16 (&sc)[2], float m_new, float& ls, bf16x8 (&pb)[4]) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                f32x8 x;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sc[c >> 1][8 * (c & 1) + j], a.scale_log2, -m_new));
                    ls += p;
                    x[j] = p;
                }
                pb[c] = to_bf16x8(x);
            }
        };
        // O^T[d, qrow] += V^T[d, key] P^T[key, qrow] (V slot of stream position p)
        auto pv = [&](const bf16x8 (&pb)[4], int p) {
            const char* vb = smem + LY::V + (p % kVSlots) * LY::BLK;
            bf16x8 vf[4 * MD];
#pragma unroll
            for (int j = 0; j < 4 * MD; ++j) {
                const char* rows = vb + 16 * D * 2 * (j & 3);
                vf[j] = concat(lds_read_tr((const uint16_t*)(rows + vo_off[0][j >> 2])),
                               lds_read_tr((const uint16_t*)(rows + vo_off[1][j >> 2])));
            }
#pragma unroll
            for (int j = 0; j < 4 * MD; ++j) oacc[j >> 2] = mfma32(vf[j], pb[j & 3], oacc[j >> 2]);
            pipeline_reads_mfma<4 * MD, kReadAhead, 2>();
        };

        for (int i = 0; i < T.work; ++i, ++s) {
            // Block s+1 landed; in steady state the copies of block s+2 (the
            // wave's 2*LPW most recent vector memory operations) stay in flight.
            if (i > 0) {
                if (l_slot != s + kAhead) wait_vmem();
                else if (!MX) wait_vmem_keep<2 * LPW>();
                else if (wave < 2) wait_vmem_keep<3>();   // MXFP8: K, V chunks (+ scales)
                else wait_vmem_keep<2>();
            }
            publish();
            // every wave is past block s-1: its K and V slots are free
            __syncthreads();
            receive();
            l_issue();                                // block s+kAhead

            const int n = seq_block(T, i);
            bool skip, masked;
            block_flags<MODE>(T, i, n, row0, wave_rows, wave, skip, masked);
            if (!skip) {
                f32x16 sc[2];
                if constexpr (MX) {
                    mx_scores(sc, smem + LY::K + (s % kKSlots) * LY::BLK,
                              smem + LY::KS + (s % kKSlots) * LY::SC, qf8, qsc, lr, hf);
                } else {
                    compute_s(sc, s);
                    pipeline_reads_mfma<2 * KC, kReadAhead>();
                }
                // masked tail: keys past the sequence (and, banded, outside the
                // row's window [lo, lim]) -> -inf
                if (masked) {
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
                float mx = -INFINITY;
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mb][r]);
                // running max in the exp2 domain of the scaled scores
                mx = pair_max(mx) * a.scale_log2;
                float ls = 0.f;
                if constexpr (MX) {
                    // P is encoded with the fixed scale of a value <= 1: the
                    // running max follows every rise
                    const float m_new = fmaxf(m_run, mx);
                    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                    m_run = m_new;
                    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
                        for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
                    }
                    // P (fp32, at most 1; its row sum stays fp32) to E4M3
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float p = __builtin_amdgcn_exp2f(fmaf(sc[mb][r], a.scale_log2, -m_new));
                            ls += p;
                            sc[mb][r] = p;
                        }
                    const i32x8 pb8 = mx_pack_p(sc);
                    l_run = l_run * alpha + ls;
                    mx_pv_tr(oacc, pb8, smem + LY::V + (s % kVSlots) * LY::BLK, mx_vo,
                          smem + LY::VS + (s % kKSlots) * LY::SC, kP8Scale, lr, hf);
                } else {
                    // The running max moves (and O^T and l are rescaled) only
                    // when some row's block max rises more than kMaxSlack above
                    // it; otherwise P = exp2(s - m_run) <= 2^kMaxSlack is kept
                    // against the stale max, which O / l cancels exactly
                    if (__builtin_amdgcn_ballot_w64(mx > m_run + kMaxSlack) != 0) {
                        const float m_new = fmaxf(m_run, mx);
                        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                        m_run = m_new;
#pragma unroll
                        for (int md = 0; md < MD; ++md) oacc[md] *= alpha;
                        l_run *= alpha;
                    }
                    bf16x8 pb[4];
                    exp_pack(sc, m_run, ls, pb);
                    l_run += ls;
                    pv(pb, s);
                }
            }
        }

        // ---- epilogue: O = O^T / l through this wave's staging area, LSE.
        // The staging areas are the K slot of block s-1 (no copy in flight
        // targets it: those are blocks s .. s+kAhead-1) for waves 0-3 and the
        // V slot of block s-1 for waves 4-7, free once every wave is past
        // block s-1; both are next written after the next iteration's barrier.
        // (MXFP8 has staging of its own.)
        const float l_tot = pair_sum(l_run);
        const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
        __syncthreads();
        if (wave_rows) {
            char* st;
            if constexpr (MX) {
                st = smem + LY::OST + wave * LY::OST_WAVE;
            } else {
                st = wave < 4 ? smem + LY::K + ((s + kKSlots - 1) % kKSlots) * LY::BLK + wave * LY::OST_WAVE
                              : smem + LY::V + ((s + kVSlots - 1) % kVSlots) * LY::BLK + (wave - 4) * LY::OST_WAVE;
            }
#pragma unroll
            for (int rd = 0; rd < 32 / kStageRows; ++rd) {
                if ((lr >> 4) == rd) {
                    const int r = lr & 15;
#pragma unroll
                    for (int md = 0; md < MD; ++md)
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            f32x4 x;
#pragma unroll
                            for (int j = 0; j < 4; ++j) x[j] = oacc[md][4 * g + j] * inv;
                            const int chunk = 4 * md + g;
                            *(bf16x4*)(st + r * D * 2 + ((chunk ^ (r & (CH - 1))) << 4) + 8 * hf) =
                                to_bf16x4(x);
                        }
                }
                wave_sync_lds();
#pragma unroll
                for (int v = 0; v < kStageRows * CH / 64; ++v) {
                    const int k = lane + 64 * v;
                    const int r = k / CH, chunk = k % CH;
                    const u32x4 x = *(const u32x4*)(st + r * D * 2 + ((chunk ^ (r & (CH - 1))) << 4));
                    const int orow = row0 + kStageRows * rd + r;
                    if (orow < Lq)
                        *(u32x4*)(a.o + (int64_t)(orow0 + orow) * rs + (int64_t)T.h * D + 8 * chunk) = x;
                }
                wave_sync_lds();
            }
            if (hf == 0 && qrow < Lq)
                a.lse[(int64_t)T.h * a.total_q + orow0 + qrow] =
                    l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
    // Dynamic plan: every claim of this workgroup has returned (the last one
    // ended its stream). The last workgroup to get here sees all the others'
    // claims done and leaves the counters zero for the next launch.
    if (dynamic && tid == 0) {
        __threadfence();
        if (atomicAdd(a.counter + 1, 1) == (int)gridDim.x - 1) {
            atomicExch(a.counter, 0);
            atomicExch(a.counter + 1, 0);
        }
    }
}

template <int D, int MODE, bool BCAST, bool MX = false>
int32_t launch(const FwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_kernel<D, MODE, BCAST, MX>), dim3(a.num_workers), dim3(kThreads), 0,
                       stream, a);
    return (int32_t)hipGetLastError();
}

template <int D, bool MX = false>
int32_t launch_d(const FwdArgs& a, Mode mode, bool bcast, hipStream_t s) {
    if (mode == kCausal) return launch<D, kCausal, false, MX>(a, s);
    if (mode == kSparse)
        return bcast ? launch<D, kSparse, true, MX>(a, s) : launch<D, kSparse, false, MX>(a, s);
    return bcast ? launch<D, kDense, true, MX>(a, s) : launch<D, kDense, false, MX>(a, s);
}

}  // namespace

int32_t launch_fwd(const FwdArgs& a, int32_t head_dim, Mode mode, bool broadcast, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (head_dim == 64) return launch_d<64>(a, mode, broadcast, s);
    return launch_d<128>(a, mode, broadcast, s);
}

int32_t launch_fwd_mx(const FwdArgs& a, Mode mode, bool broadcast, void* stream) {
    return launch_d<128, true>(a, mode, broadcast, (hipStream_t)stream);
}

}  // namespace jfa
