// Host tile planner and problem validation (plain C++17, no HIP calls).
//
// The planner follows the scheduling the pages describe for the forward
// kernel: tiles sorted on the host by KV workload, largest first, and handed
// to the processors in a zigzag pattern, plus software load balancing across
// length skew ("Meta's TLX Jagged Flash Attention Beats FA4 on Blackwell With
// 3x Less Code" (ainewsbites.com), section "Optimizations layered on top").
// The backward pass reuses it with KV tiles. The pages fix no tile size, work
// measure, tie order or meaning of "zigzag"; the readings used here are:
// work = inner-loop trip count of the tile, stable sort (ties keep (b,h,t)
// order) on the work (forward, dQ) or on the tile's estimated time on the
// dK/dV kernel (backward: work * (kBwdBlockFixed + waves holding keys) +
// kBwdTileFixed, so the partial last tile of a sequence does not count as a
// full one), snake deal (round r goes left-to-right when r is even, else
// right-to-left).
// A dynamic forward plan keeps the same sort but deals only the first W
// tiles (one per worker); the rest are claimed at run time, in sorted order,
// through a device counter: the counterpart of the cluster launch control the
// pages pair with the host sort (same page, sections "What TLX changes" and
// "Optimizations layered on top").
// A natural plan (the ablation baseline for the sort and the deal) skips the
// sort and deals the tiles in enumeration order round-robin.
#include "hostlog.h"
#include "internal.h"

#include <algorithm>
#include <cstring>
#include <numeric>
#include <vector>

namespace jfa {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// backward sort key: units of one wave's share of a Q block's products; a
// block also costs kBwdBlockFixed of them in copies and barriers, a tile
// boundary (K/V fetch, dK/dV stores) kBwdTileFixed (measured on the kernel)
constexpr int64_t kBwdWaveKeys = 32;   // keys per wave: kBwdBlockN over the kernel's 8 waves
constexpr int64_t kBwdBlockFixed = 4;
constexpr int64_t kBwdTileFixed = 42;

int32_t check_offsets(const int32_t* off, int32_t batch) {
    if (off == nullptr) return JFA_ERR_INVALID_ARG;
    if (off[0] != 0) return JFA_ERR_BAD_OFFSETS;
    for (int32_t b = 0; b < batch; ++b)
        if (off[b + 1] < off[b]) return JFA_ERR_BAD_OFFSETS;
    return JFA_OK;
}

int32_t check_problem(const jfa_problem* p) {
    if (p == nullptr) return JFA_ERR_INVALID_ARG;
    if (p->batch < 0 || p->num_heads < 1 || p->lq < 0) return JFA_ERR_INVALID_ARG;
    if (p->broadcast_q != 0 && p->broadcast_q != 1) return JFA_ERR_INVALID_ARG;
    if (p->causal != 0 && p->causal != 1) return JFA_ERR_INVALID_ARG;
    if (p->head_dim != 64 && p->head_dim != 128) return JFA_ERR_UNSUPPORTED;
    // a token row (H*D bf16) below 2^24 bytes: the kernels address the rows
    // of a block as 24-bit multiples of it from the block's first row
    if (p->num_heads > 32768) return JFA_ERR_UNSUPPORTED;
    // finite and positive (the kernels take the row max before scaling)
    if (!(p->softmax_scale > 0.0f) || p->softmax_scale > 3.0e38f) return JFA_ERR_INVALID_ARG;
    if (p->window_left < -1 || p->window_right < -1) return JFA_ERR_INVALID_ARG;
    const bool banded = p->causal || p->window_left >= 0 || p->window_right >= 0;
    if (banded && p->broadcast_q) return JFA_ERR_UNSUPPORTED;
    const bool sparse = p->mask_q_blocks != 0 || p->mask_kv_blocks != 0;
    if (sparse && (p->mask_q_blocks < 1 || p->mask_kv_blocks < 1)) return JFA_ERR_BAD_MASK;
    if (sparse && banded) return JFA_ERR_UNSUPPORTED;
    // rows of the packed tensors are addressed as int32 * H * D elements in 64 bits;
    // keep H*D within int32
    if ((int64_t)p->num_heads * p->head_dim > (1 << 24)) return JFA_ERR_INVALID_ARG;
    return JFA_OK;
}

namespace {

struct Tile { int32_t b, h, t, work; };

struct Lens {
    std::vector<int32_t> q, kv;
    int64_t total_q = 0, total_kv = 0;
};

int32_t lengths_of(const jfa_problem* p, const int32_t* qo, const int32_t* ko, Lens& L) {
    int32_t st = check_offsets(ko, p->batch);
    if (st) return st;
    L.kv.resize(p->batch);
    L.q.resize(p->batch);
    for (int32_t b = 0; b < p->batch; ++b) L.kv[b] = ko[b + 1] - ko[b];
    L.total_kv = ko[p->batch];
    if (p->broadcast_q) {
        for (int32_t b = 0; b < p->batch; ++b) L.q[b] = p->lq;
        L.total_q = (int64_t)p->batch * p->lq;
        if (L.total_q > INT32_MAX) return JFA_ERR_INVALID_ARG;
    } else {
        st = check_offsets(qo, p->batch);
        if (st) return st;
        for (int32_t b = 0; b < p->batch; ++b) L.q[b] = qo[b + 1] - qo[b];
        L.total_q = qo[p->batch];
        if (band_of(p).on)
            for (int32_t b = 0; b < p->batch; ++b)
                if (L.q[b] != L.kv[b]) return JFA_ERR_UNSUPPORTED;
    }
    const bool sparse = p->mask_q_blocks != 0;
    if (sparse)
        for (int32_t b = 0; b < p->batch; ++b)
            if (cdiv(L.q[b], kMaskBlock) > p->mask_q_blocks ||
                cdiv(L.kv[b], kMaskBlock) > p->mask_kv_blocks)
                return JFA_ERR_BAD_MASK;
    return JFA_OK;
}

inline bool kept(const jfa_problem* p, const uint8_t* mask, int32_t b, int32_t m, int32_t c) {
    return mask[((int64_t)b * p->mask_q_blocks + m) * p->mask_kv_blocks + c] != 0;
}

// Mask rows per forward tile.
constexpr int32_t kRowsPerTile = kFwdBlockM / kMaskBlock;
static_assert(kRowsPerTile * kMaskBlock == kFwdBlockM && kRowsPerTile <= 2, "tile/mask geometry");

// Bits of the mask rows of forward tile (b, t) that keep 128-key block c (bit
// k: row kRowsPerTile*t + k; rows past the mask or the sequence count as not
// keeping it).
inline int32_t fwd_bits(const jfa_problem* p, const uint8_t* mask, int32_t b, int32_t t, int32_t c,
                        int32_t lq) {
    int32_t bits = 0;
    for (int32_t k = 0; k < kRowsPerTile; ++k) {
        const int32_t m = kRowsPerTile * t + k;
        if (m < p->mask_q_blocks && (int64_t)kMaskBlock * m < lq && kept(p, mask, b, m, c))
            bits |= 1 << k;
    }
    return bits;
}

// Mask columns per backward KV tile.
constexpr int32_t kColsPerTile = kBwdBlockN / kMaskBlock;
static_assert(kColsPerTile * kMaskBlock == kBwdBlockN && kColsPerTile <= 2, "tile/mask geometry");

// Bits of the mask columns of backward KV tile (b, t) that keep 128-row mask
// row m (bit k: column kColsPerTile*t + k; columns past the mask or the
// sequence count as not keeping it).
inline int32_t bwd_bits(const jfa_problem* p, const uint8_t* mask, int32_t b, int32_t t, int32_t m,
                        int32_t lk) {
    int32_t bits = 0;
    for (int32_t k = 0; k < kColsPerTile; ++k) {
        const int32_t c = kColsPerTile * t + k;
        if (c < p->mask_kv_blocks && (int64_t)kMaskBlock * c < lk && kept(p, mask, b, m, c))
            bits |= 1 << k;
    }
    return bits;
}

int32_t tile_work(const jfa_problem* p, const uint8_t* mask, int32_t pass, int32_t b, int32_t t,
                  int32_t lq, int32_t lk) {
    const bool sparse = p->mask_q_blocks != 0;
    if (pass != JFA_PASS_BWD) {
        if (sparse) {
            int64_t w = 0;
            for (int32_t c = 0; c < cdiv(lk, kMaskBlock); ++c)
                if (fwd_bits(p, mask, b, t, c, lq))
                    w += cdiv(std::min<int64_t>((int64_t)kMaskBlock * (c + 1), lk) -
                                  (int64_t)kMaskBlock * c,
                              kFwdBlockN);
            return (int32_t)w;
        }
        const Band bd = band_of(p);
        if (bd.on) {   // the tile's rows see the contiguous key range j0..j1
            const int64_t r0 = (int64_t)t * kFwdBlockM, r1 = std::min<int64_t>(r0 + kFwdBlockM, lq) - 1;
            const int64_t j0 = bd.left < 0 ? 0 : std::max<int64_t>(0, r0 - bd.left);
            const int64_t j1 = bd.right < 0 ? lk - 1 : std::min<int64_t>(lk - 1, r1 + bd.right);
            return j1 < j0 ? 0 : (int32_t)(j1 / kFwdBlockN - j0 / kFwdBlockN + 1);
        }
        return (int32_t)cdiv(lk, kFwdBlockN);
    }
    const int32_t nqb = (int32_t)cdiv(lq, kBwdBlockM);
    if (sparse) {
        int64_t w = 0;
        for (int32_t m = 0; m < cdiv(lq, kMaskBlock); ++m)
            if (bwd_bits(p, mask, b, t, m, lk))
                w += cdiv(std::min<int64_t>((int64_t)kMaskBlock * (m + 1), lq) - (int64_t)kMaskBlock * m,
                          kBwdBlockM);
        return (int32_t)w;
    }
    const Band bd = band_of(p);
    if (bd.on) {   // rows i see key j iff j - right <= i <= j + left
        const int64_t k0 = (int64_t)t * kBwdBlockN, k1 = std::min<int64_t>(k0 + kBwdBlockN, lk) - 1;
        const int64_t i0 = bd.right < 0 ? 0 : std::max<int64_t>(0, k0 - bd.right);
        const int64_t i1 = bd.left < 0 ? lq - 1 : std::min<int64_t>(lq - 1, k1 + bd.left);
        return i1 < i0 ? 0 : (int32_t)(i1 / kBwdBlockM - i0 / kBwdBlockM + 1);
    }
    return nqb;
}

int32_t plan_impl(const jfa_problem* p, const int32_t* qo, const int32_t* ko, const uint8_t* mask,
                  int32_t pass_flags, int32_t W, jfa_plan_info* info, int32_t* worker_ptr,
                  int32_t* tiles_out, int32_t* sp_ptr, int32_t* sp_idx, bool build) {
    if (info == nullptr) return JFA_ERR_INVALID_ARG;
    int32_t st = check_problem(p);
    if (st) return st;
    const bool dynamic = (pass_flags & JFA_PLAN_DYNAMIC) != 0;
    const bool natural = (pass_flags & JFA_PLAN_NATURAL) != 0;
    const int32_t pass = pass_flags & ~(JFA_PLAN_DYNAMIC | JFA_PLAN_NATURAL);
    if (pass != JFA_PASS_FWD && pass != JFA_PASS_BWD && pass != JFA_PASS_DQ)
        return JFA_ERR_INVALID_ARG;
    if (dynamic && (pass != JFA_PASS_FWD || natural)) return JFA_ERR_INVALID_ARG;
    if (W < 1) return JFA_ERR_INVALID_ARG;
    // Q-tile passes (forward, dQ) enumerate Q tiles; the backward KV tiles
    const bool qtiles = pass != JFA_PASS_BWD;
    const bool sparse = p->mask_q_blocks != 0;
    if (sparse && mask == nullptr) return JFA_ERR_BAD_MASK;
    Lens L;
    st = lengths_of(p, qo, ko, L);
    if (st) return st;

    const int32_t bm = qtiles ? kFwdBlockM : kBwdBlockM;
    const int32_t bn = qtiles ? kFwdBlockN : kBwdBlockN;

    // 1-2. enumerate tiles with their work
    std::vector<Tile> tiles;
    int64_t n_total = 0;
    for (int32_t b = 0; b < p->batch; ++b)
        n_total += (int64_t)p->num_heads * (qtiles ? cdiv(L.q[b], bm) : cdiv(L.kv[b], bn));
    if (n_total > INT32_MAX / 4) return JFA_ERR_INVALID_ARG;
    tiles.reserve((size_t)n_total);
    int64_t total_work = 0;
    int32_t max_work = 0;
    for (int32_t b = 0; b < p->batch; ++b) {
        const int32_t nt = (int32_t)(qtiles ? cdiv(L.q[b], bm) : cdiv(L.kv[b], bn));
        for (int32_t h = 0; h < p->num_heads; ++h)
            for (int32_t t = 0; t < nt; ++t) {
                const int32_t w = tile_work(p, mask, pass, b, t, L.q[b], L.kv[b]);
                tiles.push_back({b, h, t, w});
                total_work += w;
                max_work = std::max(max_work, w);
            }
    }

    // block-sparse lists
    int64_t sp_rows = 0, sp_nnz = 0;
    const int32_t fwd_rows = (int32_t)cdiv(p->mask_q_blocks, kRowsPerTile);
    const int32_t bwd_cols = (int32_t)cdiv(p->mask_kv_blocks, kColsPerTile);
    if (sparse) {
        if (qtiles) {
            sp_rows = (int64_t)p->batch * fwd_rows;
            for (int32_t b = 0; b < p->batch; ++b)
                for (int32_t t = 0; t < fwd_rows; ++t)
                    for (int32_t c = 0; c < cdiv(L.kv[b], kMaskBlock); ++c)
                        sp_nnz += fwd_bits(p, mask, b, t, c, L.q[b]) != 0;
        } else {
            sp_rows = (int64_t)p->batch * bwd_cols;
            for (int32_t b = 0; b < p->batch; ++b)
                for (int32_t t = 0; t < bwd_cols; ++t)
                    for (int32_t m = 0; m < cdiv(L.q[b], kMaskBlock); ++m)
                        sp_nnz += bwd_bits(p, mask, b, t, m, L.kv[b]) != 0;
        }
        if (sp_rows > INT32_MAX - 1 || sp_nnz > INT32_MAX) return JFA_ERR_INVALID_ARG;
    }

    // dQ pass with broadcast Q: tiles grouped by (head, Q tile); group g owns
    // the workers [g W' / G, (g+1) W' / G) of W' = max(G, min(W, G n)) workers
    // (n: the largest chunk count of a group, counted below). A tile
    // of w > kDqChunkBlocks blocks is split into n = ceil(w / kDqChunkBlocks)
    // chunks of consecutive list positions, the first (w mod n) one block
    // longer; a chunk starting at position k0 is stored with t + nqt * k0 in
    // place of t (every chunk adds into the same partial sum).
    const bool grouped = pass == JFA_PASS_DQ && p->broadcast_q;
    const int32_t nqt = (int32_t)cdiv(p->lq, bm);
    const int64_t G = grouped ? (int64_t)p->num_heads * nqt : 0;
    if (grouped) {
        if (G > INT32_MAX / 2) return JFA_ERR_INVALID_ARG;
        if ((int64_t)nqt * max_work > INT32_MAX) return JFA_ERR_INVALID_ARG;
        std::vector<Tile> chunks;
        chunks.reserve(tiles.size());
        max_work = 0;
        for (const Tile& t : tiles) {
            const int32_t n = std::max<int32_t>(1, (int32_t)cdiv(t.work, kDqChunkBlocks));
            const int32_t q = t.work / n, r = t.work % n;
            int32_t k0 = 0;
            for (int32_t c = 0; c < n; ++c) {
                const int32_t len = q + (c < r ? 1 : 0);
                chunks.push_back({t.b, t.h, t.t + nqt * k0, len});
                max_work = std::max(max_work, len);
                k0 += len;
            }
        }
        if (chunks.size() > (size_t)(INT32_MAX / 4)) return JFA_ERR_INVALID_ARG;
        tiles.swap(chunks);
        // W' = max(G, min(W, G * n)), n the largest chunk count of a group:
        // no group gets more workers than it has chunks
        if (G > 0) {
            std::vector<int64_t> per_group((size_t)G, 0);
            for (const Tile& t : tiles) ++per_group[(size_t)((int64_t)t.h * nqt + t.t % nqt)];
            const int64_t n = *std::max_element(per_group.begin(), per_group.end());
            W = (int32_t)std::max<int64_t>(G, std::min<int64_t>(W, G * n));
        }
    }
    info->pass = pass_flags & ~JFA_PLAN_NATURAL;   // laid out as the static plan of its pass
    info->num_workers = W;
    info->num_tiles = (int32_t)tiles.size();
    info->block_m = bm;
    info->block_n = bn;
    info->total_q = (int32_t)L.total_q;
    info->total_kv = (int32_t)L.total_kv;
    info->sparse_rows = (int32_t)sp_rows;
    info->sparse_nnz = (int32_t)sp_nnz;
    info->max_work = max_work;
    info->total_work = total_work;
    if (!build) return JFA_OK;
    if (worker_ptr == nullptr || (tiles_out == nullptr && !tiles.empty()))
        return JFA_ERR_INVALID_ARG;
    if (sparse && (sp_ptr == nullptr || (sp_idx == nullptr && sp_nnz > 0)))
        return JFA_ERR_INVALID_ARG;

    // 3. stable sort by the key, descending (within each group when grouped)
    std::vector<int64_t> key(tiles.size());
    for (size_t i = 0; i < tiles.size(); ++i) {
        const Tile& t = tiles[i];
        if (pass == JFA_PASS_BWD) {
            const int64_t keys = std::min<int64_t>(bn, (int64_t)L.kv[t.b] - (int64_t)t.t * bn);
            key[i] = (int64_t)t.work * (kBwdBlockFixed + cdiv(keys, kBwdWaveKeys)) + kBwdTileFixed;
        } else {
            key[i] = t.work;
        }
    }
    std::vector<int32_t> order(tiles.size());
    std::iota(order.begin(), order.end(), 0);
    auto group_of = [&](const Tile& t) -> int64_t {
        return grouped ? (int64_t)t.h * nqt + t.t % nqt : 0;
    };
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t c) {
        const int64_t ga = group_of(tiles[a]), gc = group_of(tiles[c]);
        if (ga != gc) return ga < gc;
        return !natural && key[a] > key[c];   // natural: enumeration order
    });
    if (dynamic) {   // the sorted list itself; worker w starts with tile w
        for (int32_t w = 0; w <= W; ++w) worker_ptr[w] = (int32_t)std::min<size_t>(w, order.size());
        for (size_t i = 0; i < order.size(); ++i) {
            const Tile& t = tiles[order[i]];
            int32_t* dst = tiles_out + 4 * (int64_t)i;
            dst[0] = t.b;
            dst[1] = t.h;
            dst[2] = t.t;
            dst[3] = t.work;
        }
    }
    // 4. snake deal over the group's workers; 5. emit per worker in increasing
    // deal position
    std::vector<int32_t> count(dynamic ? 0 : W, 0), owner(dynamic ? 0 : order.size());
    for (size_t i = 0; i < owner.size();) {
        const int64_t g = group_of(tiles[order[i]]);
        size_t e = i;
        while (e < order.size() && group_of(tiles[order[e]]) == g) ++e;
        const int32_t w0 = grouped ? (int32_t)(g * W / G) : 0;
        const int32_t nw = grouped ? (int32_t)((g + 1) * W / G) - w0 : W;
        for (size_t k = i; k < e; ++k) {
            const size_t j = k - i;
            const int32_t pos = (int32_t)(j % nw);
            const int32_t w = w0 + ((natural || (j / nw) % 2 == 0) ? pos : nw - 1 - pos);
            owner[k] = w;
            ++count[w];
        }
        i = e;
    }
    if (!dynamic) {
        worker_ptr[0] = 0;
        for (int32_t w = 0; w < W; ++w) worker_ptr[w + 1] = worker_ptr[w] + count[w];
    }
    std::vector<int32_t> cursor(worker_ptr, worker_ptr + (dynamic ? 0 : W));
    for (size_t i = 0; i < owner.size(); ++i) {
        const Tile& t = tiles[order[i]];
        int32_t* dst = tiles_out + 4 * (int64_t)cursor[owner[i]]++;
        dst[0] = t.b;
        dst[1] = t.h;
        dst[2] = t.t;
        dst[3] = t.work;
    }

    if (sparse) {
        int32_t n = 0;
        sp_ptr[0] = 0;
        int32_t r = 0;
        if (qtiles) {
            for (int32_t b = 0; b < p->batch; ++b)
                for (int32_t t = 0; t < fwd_rows; ++t) {
                    for (int32_t c = 0; c < cdiv(L.kv[b], kMaskBlock); ++c) {
                        const int32_t bits = fwd_bits(p, mask, b, t, c, L.q[b]);
                        if (bits) sp_idx[n++] = 4 * c + bits;
                    }
                    sp_ptr[++r] = n;
                }
        } else {
            for (int32_t b = 0; b < p->batch; ++b)
                for (int32_t t = 0; t < bwd_cols; ++t) {
                    for (int32_t m = 0; m < cdiv(L.q[b], kMaskBlock); ++m) {
                        const int32_t bits = bwd_bits(p, mask, b, t, m, L.kv[b]);
                        if (bits) sp_idx[n++] = 4 * m + bits;
                    }
                    sp_ptr[++r] = n;
                }
        }
    }
    return JFA_OK;
}

}  // namespace
}  // namespace jfa

extern "C" {

int32_t jfa_offsets_from_lengths(const int32_t* h_lengths, int32_t batch, int32_t* h_offsets) {
    if (batch < 0 || h_offsets == nullptr || (batch > 0 && h_lengths == nullptr))
        return JFA_ERR_INVALID_ARG;
    int64_t acc = 0;
    for (int32_t b = 0; b < batch; ++b) {
        if (h_lengths[b] < 0) return JFA_ERR_BAD_OFFSETS;
        acc += h_lengths[b];
        if (acc > INT32_MAX) return JFA_ERR_BAD_OFFSETS;
    }
    acc = 0;
    h_offsets[0] = 0;
    for (int32_t b = 0; b < batch; ++b) {
        acc += h_lengths[b];
        h_offsets[b + 1] = (int32_t)acc;
    }
    return JFA_OK;
}

int32_t jfa_plan_query(const jfa_problem* prob, const int32_t* h_q_offsets,
                       const int32_t* h_kv_offsets, const uint8_t* h_block_mask, int32_t pass,
                       int32_t num_workers, jfa_plan_info* info) {
    return jfa::logged("jfa_plan_query", prob, info, pass, [&]() -> int32_t {
        return jfa::plan_impl(prob, h_q_offsets, h_kv_offsets, h_block_mask, pass, num_workers, info,
                              nullptr, nullptr, nullptr, nullptr, false);
    });
}

int32_t jfa_plan_build(const jfa_problem* prob, const int32_t* h_q_offsets,
                       const int32_t* h_kv_offsets, const uint8_t* h_block_mask, int32_t pass,
                       int32_t num_workers, jfa_plan_info* info, int32_t* h_worker_ptr,
                       int32_t* h_tiles, int32_t* h_sparse_ptr, int32_t* h_sparse_idx) {
    return jfa::logged("jfa_plan_build", prob, info, pass, [&]() -> int32_t {
        return jfa::plan_impl(prob, h_q_offsets, h_kv_offsets, h_block_mask, pass, num_workers, info,
                              h_worker_ptr, h_tiles, h_sparse_ptr, h_sparse_idx, true);
    });
}

}  // extern "C"
