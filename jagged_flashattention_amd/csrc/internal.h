// Internal declarations shared by the host API, the planner and the kernels.
#pragma once

#include <stdint.h>

#include "jfa.h"

namespace jfa {

// Tile geometry. Forward (and the Q-stationary dQ pass): a workgroup of 8
// waves owns 256 query rows (32 per wave) and streams 64-key K/V blocks.
// dK/dV pass: a workgroup of 8 waves owns a 256-key KV tile (32 keys per
// wave) and streams 32-row Q/dO blocks. The block-sparse mask has 128-row x
// 128-key granularity.
constexpr int32_t kFwdBlockM = 256;
constexpr int32_t kFwdBlockN = 64;
constexpr int32_t kBwdBlockM = 32;
constexpr int32_t kBwdBlockN = 256;
constexpr int32_t kMaskBlock = 128;
// Broadcast-Q dQ plans split a tile of more than this many 64-key blocks into
// chunks of at most this many.
constexpr int32_t kDqChunkBlocks = 16;

int32_t check_problem(const jfa_problem* p);
int32_t check_offsets(const int32_t* off, int32_t batch);

// kCausal is the banded mode: causal and sliding-window attention (a key
// window [i - left, i + right] per query row i, a bound < 0 meaning none).
enum Mode : int32_t { kDense = 0, kCausal = 1, kSparse = 2 };

struct Band {
    bool on;
    int32_t left, right;   // -1: unbounded
};
inline Band band_of(const jfa_problem* p) {
    Band b;
    b.left = p->window_left;
    b.right = p->causal ? 0 : p->window_right;
    b.on = p->causal || p->window_left >= 0 || p->window_right >= 0;
    return b;
}

struct FwdArgs {
    const int32_t* worker_ptr;
    const int32_t* tiles;
    const int32_t* sp_ptr;
    const int32_t* sp_idx;
    const int32_t* q_off;   // null in broadcast mode
    const int32_t* kv_off;
    const uint16_t* q;      // bf16 bit patterns
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int32_t num_heads;
    int32_t lq;
    int32_t total_q;
    int32_t mask_q_blocks;
    int32_t num_workers;
    int32_t num_tiles;
    int32_t win_left, win_right;   // banded mode: window bounds (-1: none)
    int32_t* counter;       // dynamic plan: [0] tiles claimed, [1] workgroups done; else null
    float scale_log2;       // softmax_scale * log2(e)
    // MXFP8 forward only (q, k, v above unused): E4M3 codes and E8M0 scales
    const uint8_t* q8;      // [q rows, H, D]
    const uint8_t* k8;      // [T_k, H, D]
    const uint8_t* v8;      // [T_k, H, D]
    const uint8_t* q_sc;    // [H, q rows, D/32]
    const uint8_t* k_sc;    // [H, T_k, D/32]
    const uint8_t* v_sc;    // [H, NB, D]: 32-key blocks of each sequence
    const int32_t* v_boff;  // [B+1]: first V scale block of each sequence
    int32_t q_rows;         // lq (broadcast) or T_q
    int32_t total_kv;
    int32_t v_nb;           // NB
    // executed-tile log of debug builds (see tile_log in device.h)
    int32_t batch;
    int32_t* tile_log;       // null: off
    int32_t tile_log_cap;    // records per worker
};

// Workspace of a dynamic forward plan (two int32 counters, padded).
constexpr int64_t kFwdCounterBytes = 256;

// KV-stationary dK/dV pass of the backward (JFA_PASS_BWD plan) and the
// delta preprocess.
struct BwdArgs {
    const int32_t* worker_ptr;
    const int32_t* tiles;
    const int32_t* sp_ptr;
    const int32_t* sp_idx;
    const int32_t* q_off;
    const int32_t* kv_off;
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* o;
    const float* lse;
    const uint16_t* d_o;
    uint16_t* dk;
    uint16_t* dv;
    float* delta;
    int32_t num_heads;
    int32_t lq;
    int32_t total_q;
    int32_t mask_kv_blocks;
    int32_t num_workers;
    int32_t win_left, win_right;   // banded mode: window bounds (-1: none)
    float scale;
    float scale_log2;
    // MXFP8 dK/dV pass (head_dim 128): E4M3 codes and E8M0 scale codes
    const uint8_t* q8;       // Q along d: [q_rows, H, D], scales [H, q_rows, D/32]
    const uint8_t* q_sc;
    const uint8_t* k8;       // K along d: [T_k, H, D], scales [H, T_k, D/32]
    const uint8_t* k_sc;
    const uint8_t* v8;       // V along d: [T_k, H, D], scales [H, T_k, D/32]
    const uint8_t* v_sc;
    const uint8_t* do8;      // dO along d: [T_q, H, D], scales [H, T_q, D/32]
    const uint8_t* do_sc;
    const uint8_t* qr8;      // Q along its rows: [q_rows, H, D], scales [H, qr_nb, D]
    const uint8_t* qr_sc;
    const uint8_t* dor8;     // dO along its rows: [T_q, H, D], scales [H, dor_nb, D]
    const uint8_t* dor_sc;
    const int32_t* qr_boff;  // first 32-row Q block of each sequence [B+1] (per-sequence Q)
    const int32_t* dor_boff; // first 32-row dO block of each sequence [B+1]
    int32_t qr_nb, dor_nb;
    int32_t q_rows;
    int32_t total_kv;
    // executed-tile log of debug builds (see tile_log in device.h)
    int32_t batch;
    int32_t* tile_log;       // null: off
    int32_t tile_log_cap;    // records per worker
};

// Q-stationary dQ pass of the backward (JFA_PASS_DQ plan).
struct DqArgs {
    const int32_t* worker_ptr;
    const int32_t* tiles;
    const int32_t* sp_ptr;
    const int32_t* sp_idx;
    const int32_t* q_off;    // null in broadcast mode
    const int32_t* kv_off;
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* d_o;
    const uint16_t* o;       // the forward's output, for delta
    const float* lse;
    float* delta;            // written: rowsum(dO * O) of every row
    uint16_t* dq;            // per-sequence Q: bf16 [T_q, H, D]
    float* dq_accum;         // per-sequence Q: fp32 [T_q, H, D]
    float* partial;          // broadcast Q: fp32 [W][256][D] per-worker partial sums
    int32_t chunk_div;       // broadcast Q: Q tiles per sequence (chunked tile records), else 0
    int32_t win_left, win_right;   // banded mode: window bounds (-1: none)
    int32_t num_heads;
    int32_t lq;
    int32_t total_q;
    int32_t mask_q_blocks;
    int32_t num_workers;
    float scale;
    float scale_log2;
    // MXFP8 dQ pass (head_dim 128): E4M3 codes and E8M0 scale codes
    const uint8_t* q8;       // Q along d: [q_rows, H, D], scales [H, q_rows, D/32]
    const uint8_t* q_sc;
    const uint8_t* k8;       // K along d: [T_k, H, D], scales [H, T_k, D/32]
    const uint8_t* k_sc;
    const uint8_t* v8;       // V along d: [T_k, H, D], scales [H, T_k, D/32]
    const uint8_t* v_sc;
    const uint8_t* do8;      // dO along d: [T_q, H, D], scales [H, T_q, D/32]
    const uint8_t* do_sc;
    const uint8_t* kk8;      // K along keys: [T_k, H, D], scales [H, NB, D]
    const uint8_t* kk_sc;
    const int32_t* kk_boff;  // first 32-key block of each sequence [B+1]
    int32_t kk_nb;           // NB
    int32_t q_rows;
    int32_t total_kv;
    // executed-tile log of debug builds (see tile_log in device.h)
    int32_t batch;
    int32_t* tile_log;       // null: off
    int32_t tile_log_cap;    // records per worker
};

// Deterministic sum of the broadcast-Q dQ partials of each (head, Q tile)
// group in worker order, into dq_accum (fp32) and dq (bf16), both [lq, H, D].
struct DqReduceArgs {
    const int32_t* worker_ptr;   // the DQ plan's (to skip workers without tiles)
    const float* partial;
    float* dq_accum;
    uint16_t* dq;
    int32_t num_heads;
    int32_t lq;
    int32_t num_workers;         // W' of the DQ plan
};

// Launchers (return a hipError_t value as int32).
int32_t launch_fwd(const FwdArgs& a, int32_t head_dim, Mode mode, bool broadcast, void* stream);
int32_t launch_fwd_mx(const FwdArgs& a, Mode mode, bool broadcast, void* stream);
int32_t launch_bwd(const BwdArgs& a, int32_t head_dim, Mode mode, bool broadcast, int32_t stages,
                   void* stream);
int32_t launch_dq(const DqArgs& a, int32_t head_dim, Mode mode, bool broadcast, bool atomic,
                  void* stream);
int32_t launch_dq_reduce(const DqReduceArgs& a, int32_t head_dim, void* stream);
// broadcast Q, atomic reduction: dq_accum = 0 before the dQ pass, then
// dq = bf16(dq_accum) after it (n = lq * H * D elements)
int32_t launch_dq_zero(float* dq_accum, int64_t n, void* stream);
int32_t launch_dq_convert(const float* dq_accum, uint16_t* dq, int64_t n, void* stream);
int32_t launch_dq_mx(const DqArgs& a, Mode mode, bool broadcast, void* stream);
int32_t launch_dkdv_mx(const BwdArgs& a, Mode mode, bool broadcast, void* stream);
int32_t launch_mx_quant_rows(const uint16_t* src, int64_t rows, int32_t H, int32_t D, uint8_t* codes,
                             uint8_t* scales, void* stream);
// Device address, on the current device, of the library's own scratch area
// of JFA_NOALLOC_SCRATCH_BYTES (the workspace of jfa_bwd_noalloc): looked up
// once per device and kept. Returns a hipError_t value as int32.
int32_t noalloc_scratch(void** out);
int32_t launch_mx_quant_v(const uint16_t* v, const int32_t* kv_off, const int32_t* boff, int32_t B,
                          int32_t H, int32_t D, int32_t nbt, uint8_t* codes, uint8_t* scales,
                          void* stream);

}  // namespace jfa
