// MXFP8 dK/dV pass of the jagged FlashAttention backward for gfx950 (head_dim
// 128).
//
// The pages describe an MXFP8 version of the kernel whose matrix products run
// in microscaling precision with probabilities quantised to FP8 on the fly,
// and report its backward at parity on dense shapes ("TLX porta l'attenzione
// jagged su Blackwell" (ai-radar.it), section "The turning point"). This is
// the KV-stationary dK/dV pass of that backward, built like the bf16 one (one
// persistent workgroup of 8 waves per CU, 256-key KV tiles with 32 keys per
// wave, 32-row Q/dO blocks streamed through a direct-to-LDS ring), with its
// four products as OCP MXFP8 scaled MFMAs (E4M3 data, one E8M0 scale per 32
// elements along the contraction):
//   S    = Q K^T      Q and K encoded along d
//   dP   = dO V^T     dO and V encoded along d
//   dV^T += dO^T P    dO encoded along its rows (32-row blocks of one
//                     sequence, as V along keys for the forward); P rounded
//                     to E4M3 on the fly with the fixed block scale 2^-8
//                     (P = exp(S - LSE) <= 1)
//   dK^T += Q^T dS    Q encoded along its rows; dS rounded to E4M3 on the fly
//                     with one scale per (key, 32-row block): the smallest
//                     power of two 2^e with max|dS| / 2^e <= 448, so no value
//                     is clamped
// A 32-row block fills one of the two 32-element scale blocks of the 64-long
// contraction of the scaled MFMA; the other is zero. The dO^T and Q^T
// operands are byte-transposed LDS reads (ds_read_b64_tr_b8) of the Q and dO
// blocks encoded along rows, which the slot holds back to back as one 64-row
// block (Q rows, then dO rows), swizzled by swz_v8. P = exp2(S c - LSE c) and dS = P (dP - delta) stay fp32; dK and dV
// accumulate in fp32 and leave as bf16.
#include <climits>

#include "mxops.h"
#include "qtile.h"

namespace jfa {
namespace {

using namespace qtile;
using namespace mxops;

constexpr int kAhead = 2;            // block j+2 is copied while block j is computed
constexpr int kSlots = kAhead + 1;   // Q/dO ring: blocks j .. j+kAhead
static_assert(kBwdBlockN == 32 * kWaves && kBwdBlockM == 32, "dK/dV tile geometry");

struct DkdvMxLds {
    static constexpr int D = 128;
    static constexpr int QB = kBwdBlockM * D;       // one E4M3 block [32][128]
    // ring slot: Q and dO along d (rows swizzled by swz_k8), Q and dO along
    // rows (back to back, one [64][128] block read by byte-transposed reads,
    // rows swizzled by swz_v8), their scales, the block's row values
    static constexpr int QD = 0;
    static constexpr int DD = QD + QB;
    static constexpr int QR = DD + QB;
    static constexpr int DR = QR + QB;
    static constexpr int QDS = DR + QB;              // [32 rows][4] Q along-d scales,
    static constexpr int DDS = QDS + 128;            // then dO's
    static constexpr int QRS = DDS + 128;            // [128 d] Q along-rows scales,
    static constexpr int DRS = QRS + 128;            // then dO's
    static constexpr int ROWV = DRS + 128;           // LSE*log2e [32], delta [32] fp32
    static constexpr int SLOT = ROWV + 256;
    static constexpr int RING = 0;
    static constexpr int V = RING + kSlots * SLOT;   // V tile along d [256][128] (swz_k8);
    static constexpr int VS = V + kBwdBlockN * D;    // it stages dK/dV at a tile end
    static constexpr int K = VS + kBwdBlockN * 4;    // K tile along d [256][128] (swz_k8)
    static constexpr int KS = K + kBwdBlockN * D;
    static constexpr int BYTES = KS + kBwdBlockN * 4;
    static_assert(kWaves * 16 * D * 2 <= kBwdBlockN * D, "epilogue staging fits the V tile");
    static_assert(SLOT % 256 == 0, "slot alignment");
};

// Sixteen values of a 32-row key column (this lane half's rows, register
// order) divided by `scale` as E4M3, regrouped across the lane halves so that
// half h holds rows 16h .. 16h+15 as dwords of rows 0-3, 8-11, 4-7, 12-15
// (relative to 16h): the B-operand bytes 0-15 of one 32-row scale block.
__device__ __forceinline__ u32x4 pack_col(const f32x16& x, float scale) {
    uint32_t d[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) d[g] = pack4_fp8(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3], scale);
    const auto r02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
    const auto r13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
    return u32x4{r02[0], r13[0], r02[1], r13[1]};
}

template <int MODE, bool BCAST>
__global__ void __launch_bounds__(kThreads, 1) dkdv_mx_kernel(BwdArgs a) {
    using LY = DkdvMxLds;
    constexpr int D = LY::D;
    constexpr int MD = D / 32;              // 32-row d blocks of dK^T, dV^T
    constexpr int CH = D / 8;               // 16-byte chunks per bf16 row
    __shared__ __attribute__((aligned(1024))) char smem[LY::BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lr = lane & 31, hf = lane >> 5;
    const int H = a.num_heads;
    const int64_t rs = (int64_t)H * D;      // row stride: elements (bf16), bytes (E4M3)

    const int w = worker_id(a.num_workers);
    const int t_begin = ld_uniform(a.worker_ptr + w), t_end = ld_uniform(a.worker_ptr + w + 1);
    const int kv_tiles_per_row = (a.mask_kv_blocks + 1) >> 1;

    struct KvTile {
        int b, h, n, work, kv0, L, q0, Lq, orow0, r0, qb0, db0;
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
            T.qb0 = 0;   // the one shared Q: its blocks are the sequence's
        } else {
            T.q0 = ld_uniform(a.q_off + T.b);
            T.Lq = ld_uniform(a.q_off + T.b + 1) - T.q0;
            T.orow0 = T.q0;
            T.qb0 = ld_uniform(a.qr_boff + T.b);
        }
        T.db0 = ld_uniform(a.dor_boff + T.b);
        T.r0 = MODE == kCausal && a.win_right >= 0 ? max(0, T.n * kBwdBlockN - a.win_right) / kBwdBlockM : 0;
        T.sp = nullptr;
        if (MODE == kSparse) T.sp = a.sp_idx + ld_uniform(a.sp_ptr + T.b * kv_tiles_per_row + T.n);
        return T;
    };
    auto q_block = [&](const KvTile& T, int i) -> int {
        if (MODE == kSparse) return 4 * (ld_uniform(T.sp + (i >> 2)) >> 2) + (i & 3);
        return T.r0 + i;
    };

    // ---- loader: the worker's Q/dO blocks in plan order, kAhead blocks ahead.
    // Copy u of a thread: chunk p = 512u + tid of the slot's four E4M3 blocks
    // (tensor p / 256: Q along d, dO along d, Q along rows, dO along rows;
    // wave-uniform), row r = (p % 256) / 8; wave 1 copies the along-d scales
    // (a dword per row: lanes 0-31 Q's, 32-63 dO's), wave 2 the along-rows
    // scales (lanes 0-31 Q's, 32-63 dO's, four d per dword). Rows past the
    // sequence read its last row (their P and dS are 0).
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
    float pend_v = 0.f;
    bool pend_in = false;
    auto l_issue = [&]() {
        if (l_ti >= t_end) return;
        const int rb = q_block(LT, l_i);
        char* dst = smem + LY::RING + (l_slot % kSlots) * LY::SLOT;
        const int64_t hq = (int64_t)LT.h * D;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int tensor = 2 * u + (wave >> 2);     // wave-uniform
            const int q = 64 * (wave & 3) + lane, r = q >> 3, pos = q & 7;
            const int qi = min(kBwdBlockM * rb + r, LT.Lq - 1);
            const uint8_t* src;
            if (tensor == 0) src = a.q8 + (int64_t)(LT.q0 + qi) * rs + hq + 16 * (pos ^ swz_k8(r));
            else if (tensor == 1) src = a.do8 + (int64_t)(LT.orow0 + qi) * rs + hq + 16 * (pos ^ swz_k8(r));
            else if (tensor == 2) src = a.qr8 + (int64_t)(LT.q0 + qi) * rs + hq + 16 * (pos ^ swz_v8(r));
            else src = a.dor8 + (int64_t)(LT.orow0 + qi) * rs + hq + 16 * (pos ^ swz_v8(r));
            load_lds16((const uint16_t*)src, dst + LY::QB * tensor + 1024 * (wave & 3));
        }
        if (wave == 0) {
            const int row = kBwdBlockM * rb + lr;
            const int qi = min(row, LT.Lq - 1);
            const int64_t idx = (int64_t)LT.h * a.total_q + LT.orow0 + qi;
            pend_v = hf ? a.delta[idx] : a.lse[idx];
            pend_in = row < LT.Lq;
        } else if (wave == 1) {
            const int qi = min(kBwdBlockM * rb + lr, LT.Lq - 1);
            const uint8_t* src = hf ? a.do_sc + ((int64_t)LT.h * a.total_q + LT.orow0 + qi) * 4
                                    : a.q_sc + ((int64_t)LT.h * a.q_rows + LT.q0 + qi) * 4;
            load_lds4(src, dst + LY::QDS);
        } else if (wave == 2) {
            const uint8_t* src = hf ? a.dor_sc + ((int64_t)LT.h * a.dor_nb + LT.db0 + rb) * D + 4 * lr
                                    : a.qr_sc + ((int64_t)LT.h * a.qr_nb + LT.qb0 + rb) * D + 4 * lr;
            load_lds4(src, dst + LY::QRS);
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
            else x = pend_in ? pend_v : 0.f;
            rv[lane] = x;
        }
    };
    int tr_vo[4];   // this lane's offsets of the byte-transposed Q^T / dO^T reads
    mx_tr_offsets(lane, tr_vo);

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

    // The tile's K and V along d (rows swizzled by swz_k8) and their scale
    // dwords into LDS (keys past the sequence read its last row; their dK/dV
    // are not stored).
    auto load_kv = [&](const KvTile& T) {
        const int64_t kvrow0 = (int64_t)T.kv0 * rs + (int64_t)T.h * D;
        const int lane_t = opaque(lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) {   // chunk p = 512u + tid: key p/8, stored chunk p%8
            const int p = 512 * u + tid;
            const int r = p >> 3, pos = p & 7;
            const int vk = min(T.n * kBwdBlockN + r, T.L - 1);
            const int64_t off = kvrow0 + (int64_t)vk * rs + 16 * (pos ^ swz_k8(r));
            load_lds16((const uint16_t*)(a.k8 + off), smem + LY::K + 1024 * (8 * u + wave));
            load_lds16((const uint16_t*)(a.v8 + off), smem + LY::V + 1024 * (8 * u + wave));
        }
        const int vk = min(T.n * kBwdBlockN + 64 * (wave & 3) + lane_t, T.L - 1);
        const int64_t so = ((int64_t)T.h * a.total_kv + T.kv0 + vk) * 4;
        load_lds4((wave < 4 ? a.k_sc : a.v_sc) + so, smem + (wave < 4 ? LY::KS : LY::VS) + 256 * (wave & 3));
    };
    if (t_begin < t_end) load_kv(tile_info(t_begin));
    wait_vmem();
    __syncthreads();

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
        const int vr = 32 * wave + lr;                    // this lane's K and V row of the tile

        for (int i = 0; i < T.work; ++i, ++s) {
            wait_vmem();   // block s+1 landed (the only copies in flight)
            // every wave is past block s-1: its slot is free
            __syncthreads();
            // (past the end of the stream this works on stale, unread data)
            put_rowvals(s + 1);
            l_issue();                               // block s+kAhead

            const int rb = q_block(T, i);
            bool skip = !wave_keys, masked = false;
            if (MODE == kCausal) {
                const int64_t R0 = kBwdBlockM * rb, R1 = R0 + kBwdBlockM - 1, K0 = key0, K1 = key0 + 31;
                skip = skip || (a.win_right >= 0 && R1 < K0 - a.win_right) ||
                       (a.win_left >= 0 && R0 > K1 + a.win_left);
                masked = (a.win_right >= 0 && R0 < K1 - a.win_right) ||
                         (a.win_left >= 0 && R1 > K0 + a.win_left);
            } else if (MODE == kSparse) {
                skip = skip || !((ld_uniform(T.sp + (i >> 2)) >> (wave >> 2)) & 1);
            }
            if (skip) continue;
            const char* sl = smem + LY::RING + (s % kSlots) * LY::SLOT;

            // S = Q K^T and dP = dO V^T: A = the block's rows along d (lane =
            // row lr), B = this lane's key along d; the lane gives the scale
            // of d block 2j + hf of its row / key
            f32x16 sc = f32x16{}, dp = f32x16{};
            {
                const uint32_t qsd = *(const uint32_t*)(sl + LY::QDS + 4 * lr);
                const uint32_t dsd = *(const uint32_t*)(sl + LY::DDS + 4 * lr);
                const uint32_t ksd = *(const uint32_t*)(smem + LY::KS + 4 * vr);
                const uint32_t vsd = *(const uint32_t*)(smem + LY::VS + 4 * vr);
                const char* krow = smem + LY::K + vr * D;
                const char* vrow = smem + LY::V + vr * D;
                const char* qrow = sl + LY::QD + lr * D;
                const char* drow = sl + LY::DD + lr * D;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int c0 = 16 * ((4 * j + hf) ^ swz_k8(lr)), c1 = 16 * ((4 * j + 2 + hf) ^ swz_k8(lr));
                    const int e0 = 16 * ((4 * j + hf) ^ swz_k8(vr)), e1 = 16 * ((4 * j + 2 + hf) ^ swz_k8(vr));
                    const u32x4 ql = *(const u32x4*)(qrow + c0), qh = *(const u32x4*)(qrow + c1);
                    const u32x4 dl = *(const u32x4*)(drow + c0), dh = *(const u32x4*)(drow + c1);
                    const u32x4 vl = *(const u32x4*)(vrow + e0), vh = *(const u32x4*)(vrow + e1);
                    const u32x4 kl = *(const u32x4*)(krow + e0), kh = *(const u32x4*)(krow + e1);
                    const int sh = 8 * (2 * j + hf);
                    sc = mfma_mx(i32x8{(int)ql[0], (int)ql[1], (int)ql[2], (int)ql[3], (int)qh[0], (int)qh[1], (int)qh[2], (int)qh[3]},
                                 i32x8{(int)kl[0], (int)kl[1], (int)kl[2], (int)kl[3], (int)kh[0], (int)kh[1], (int)kh[2], (int)kh[3]},
                                 (qsd >> sh) & 255, (ksd >> sh) & 255, sc);
                    dp = mfma_mx(i32x8{(int)dl[0], (int)dl[1], (int)dl[2], (int)dl[3], (int)dh[0], (int)dh[1], (int)dh[2], (int)dh[3]},
                                 i32x8{(int)vl[0], (int)vl[1], (int)vl[2], (int)vl[3], (int)vh[0], (int)vh[1], (int)vh[2], (int)vh[3]},
                                 (dsd >> sh) & 255, (vsd >> sh) & 255, dp);
                }
                // the operand reads of one step, then its two products
                __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
            __builtin_amdgcn_sched_barrier(0);   // (keeps later reads out of this phase)
            // P and dS; register r is query row 32rb + 8(r/4) + 4hf + r%4, the
            // column this lane's key. Banded: with c = 8(r/4) + r%4, visible
            // iff c_lo <= c <= c_hi
            int c_lo = INT_MIN, c_hi = INT_MAX;
            if (MODE == kCausal && masked) {
                const int base = key0 + lr - kBwdBlockM * rb - 4 * hf;
                if (a.win_right >= 0) c_lo = base - a.win_right;
                if (a.win_left >= 0) c_hi = base + a.win_left;
            }
            const float* rv = (const float*)(sl + LY::ROWV);
            float amax = 0.f;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int row = 8 * g + 4 * hf;
                const f32x4 l4 = *(const f32x4*)(rv + row);
                const f32x4 d4 = *(const f32x4*)(rv + 32 + row);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float p = __builtin_amdgcn_exp2f(fmaf(sc[4 * g + j], a.scale_log2, -l4[j]));
                    if (MODE == kCausal && masked) {
                        const int c = 8 * g + j;
                        if (c < c_lo || c > c_hi) p = 0.f;
                    }
                    const float ds = p * (dp[4 * g + j] - d4[j]);
                    sc[4 * g + j] = p;
                    dp[4 * g + j] = ds;
                    amax = fmaxf(amax, fabsf(ds));
                }
            }
            // dS's scale per (key, 32-row block): 2^e with e = floor(log2 max)
            // - 8, one more if max / 2^e > 448 (both halves of the key column
            // see the same max); a block below 2^-100 goes as zeros
            amax = pair_max(amax);
            float dscale;
            int dcode;
            if (amax < 0x1p-100f) {
                dscale = 1.0f;
                dcode = 0;
#pragma unroll
                for (int r = 0; r < 16; ++r) dp[r] = 0.f;
            } else {
                int e = (int)((__float_as_uint(amax) >> 23) & 255) - 127 - 8;
                if (amax > 448.0f * __uint_as_float((uint32_t)(e + 127) << 23)) ++e;
                dcode = e + 127;
                dscale = __uint_as_float((uint32_t)dcode << 23);
            }
            const u32x4 pb = pack_col(sc, 1.0f / 256.0f);
            const u32x4 sb = pack_col(dp, dscale);
            const i32x8 pb8 = {(int)pb[0], (int)pb[1], (int)pb[2], (int)pb[3], 0, 0, 0, 0};
            const i32x8 sb8 = {(int)sb[0], (int)sb[1], (int)sb[2], (int)sb[3], 0, 0, 0, 0};
            // the B scales: block 0 (this block's rows) from lane half 0, block
            // 1 (zeros) from half 1
            const int pcode = hf ? 127 : kP8Scale;
            const int scode = hf ? 127 : dcode;
            __builtin_amdgcn_sched_barrier(0);
            // dV^T[d, key] += dO^T[d, rows] P[rows, key]; dK^T += Q^T dS: A
            // = rows 16hf .. 16hf+15 of the Q (dO) block at d, in the dword
            // order of pack_col, by two byte-transposed reads each (rows
            // 16hf + (0-3, 8-11), then + 4; dO 32 rows further)
            const uint32_t qrb = lds_addr(sl + LY::QR);
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                const int d = 32 * md + lr;
                const uint32_t ta = qrb + tr_vo[md];
                const i32x2 q0 = lds_read_tr8_at(ta, 0), q1 = lds_read_tr8_at(ta, 4 * 128);
                const i32x2 d0 = lds_read_tr8_at(ta, 32 * 128), d1 = lds_read_tr8_at(ta, 36 * 128);
                const int qrs = hf ? 127 : *(const uint8_t*)(sl + LY::QRS + d);
                const int drs = hf ? 127 : *(const uint8_t*)(sl + LY::DRS + d);
                dv_acc[md] = mfma_mx(i32x8{d0[0], d0[1], d1[0], d1[1], 0, 0, 0, 0}, pb8, drs, pcode, dv_acc[md]);
                dk_acc[md] = mfma_mx(i32x8{q0[0], q0[1], q1[0], q1[1], 0, 0, 0, 0}, sb8, qrs, scode, dk_acc[md]);
            }
            // reads one d block ahead of the products
            __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
            for (int md = 1; md < MD; ++md) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }

        // ---- tile end: every wave is done with V. dK = scale * (dK^T)^T and
        // dV leave as bf16 rows staged through the V tile (16 keys per wave
        // at a time), then the next tile's K and V come in.
        __syncthreads();
        {
            const int64_t kvrow0 = (int64_t)T.kv0 * rs + (int64_t)T.h * D;
            char* st = smem + LY::V + wave * (16 * D * 2);
            const int lane_e = opaque(lane), lr_e = lane_e & 31, hf_e = lane_e >> 5;
#pragma unroll
            for (int pass = 0; pass < 4; ++pass) {   // dK keys 0-15, 16-31, then dV
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
                            *(bf16x4*)(st + r * D * 2 + ((chunk ^ (r & (CH - 1))) << 4) + 8 * hf_e) = to_bf16x4(x);
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
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): staging read before it is overwritten
                wave_sync_lds();
            }
        }
        __syncthreads();   // every wave's staging is read: the V tile is free
        if (ti + 1 < t_end) load_kv(tile_info(ti + 1));
        // the next tile's K and V landed (and this tile's stores are done)
        wait_vmem();
        __syncthreads();
    }
}

template <int MODE, bool BCAST>
int32_t launch(const BwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((dkdv_mx_kernel<MODE, BCAST>), dim3(a.num_workers), dim3(kThreads), 0, stream, a);
    return (int32_t)hipGetLastError();
}

}  // namespace

int32_t launch_dkdv_mx(const BwdArgs& a, Mode mode, bool broadcast, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (a.num_workers == 0) return 0;
    if (mode == kCausal) return launch<kCausal, false>(a, s);
    if (mode == kSparse) return broadcast ? launch<kSparse, true>(a, s) : launch<kSparse, false>(a, s);
    return broadcast ? launch<kDense, true>(a, s) : launch<kDense, false>(a, s);
}

}  // namespace jfa
