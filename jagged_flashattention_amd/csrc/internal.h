// Internal declarations shared by the host API, the planner and the kernels.
#pragma once

#include <stdint.h>

#include "jfa.h"

namespace jfa {

// Tile geometry. Forward (and the Q-stationary dQ pass): a workgroup of 8
// waves owns 256 query rows (32 per wave) and streams 64-key K/V blocks.
// Backward: a workgroup owns a 128-key KV tile (32 keys per wave) and streams
// 64-row Q/dO blocks. The block-sparse mask has 128-row x 128-key granularity.
constexpr int32_t kFwdBlockM = 256;
constexpr int32_t kFwdBlockN = 64;
constexpr int32_t kBwdBlockM = 64;
constexpr int32_t kBwdBlockN = 128;
constexpr int32_t kMaskBlock = 128;

int32_t check_problem(const jfa_problem* p);
int32_t check_offsets(const int32_t* off, int32_t batch);

enum Mode : int32_t { kDense = 0, kCausal = 1, kSparse = 2 };

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
    float scale_log2;       // softmax_scale * log2(e)
};

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
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* dq_accum;
    float* delta;
    int32_t num_heads;
    int32_t lq;
    int32_t total_q;
    int32_t q_rows;          // rows of q / dq (lq in broadcast mode, else T_q)
    int32_t mask_kv_blocks;
    int32_t num_workers;
    float scale;
    float scale_log2;
};

// Launchers (return a hipError_t value as int32).
int32_t launch_fwd(const FwdArgs& a, int32_t head_dim, Mode mode, bool broadcast, void* stream);
int32_t launch_bwd(const BwdArgs& a, int32_t head_dim, Mode mode, bool broadcast, int32_t stages,
                   void* stream);

}  // namespace jfa
