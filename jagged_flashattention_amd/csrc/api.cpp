// C ABI entry points: argument validation and kernel launches on the caller's
// stream. Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "hostlog.h"
#include "internal.h"

namespace {

#ifdef JFA_TILE_LOG
constexpr bool kTileLogBuild = true;
#else
constexpr bool kTileLogBuild = false;
#endif

thread_local int32_t g_last_hip_error = 0;

int32_t hip_status(int32_t e) {
    if (e == 0) return JFA_OK;
    g_last_hip_error = e;
    return JFA_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

jfa::Mode mode_of(const jfa_problem* p) {
    if (p->mask_q_blocks != 0) return jfa::kSparse;
    if (jfa::band_of(p).on) return jfa::kCausal;   // banded: causal or sliding window
    return jfa::kDense;
}

// Checks shared by jfa_fwd and jfa_bwd.
int32_t check_common(const jfa_problem* p, const jfa_plan_info* info, int32_t pass,
                     const int32_t* d_worker_ptr, const int32_t* d_tiles,
                     const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                     const int32_t* d_q_offsets, const int32_t* d_kv_offsets) {
    int32_t st = jfa::check_problem(p);
    if (st) return st;
    if (info == nullptr) return JFA_ERR_INVALID_ARG;
    // a dynamic plan is a FWD plan with its own deal
    const int32_t ipass = info->pass == (JFA_PASS_FWD | JFA_PLAN_DYNAMIC) ? JFA_PASS_FWD : info->pass;
    if (ipass != pass) return JFA_ERR_PLAN_MISMATCH;
    const bool qtiles = pass != JFA_PASS_BWD;
    const int32_t bm = qtiles ? jfa::kFwdBlockM : jfa::kBwdBlockM;
    const int32_t bn = qtiles ? jfa::kFwdBlockN : jfa::kBwdBlockN;
    if (info->block_m != bm || info->block_n != bn) return JFA_ERR_PLAN_MISMATCH;
    if (info->num_workers < 1 || info->num_tiles < 0 || info->total_q < 0 || info->total_kv < 0)
        return JFA_ERR_PLAN_MISMATCH;
    if (p->broadcast_q && info->total_q != (int64_t)p->batch * p->lq) return JFA_ERR_PLAN_MISMATCH;
    const bool sparse = p->mask_q_blocks != 0;
    if (sparse) {
        const int64_t rows =
            (int64_t)p->batch * (qtiles ? (p->mask_q_blocks + jfa::kFwdBlockM / jfa::kMaskBlock - 1) /
                                              (jfa::kFwdBlockM / jfa::kMaskBlock)
                                        : (p->mask_kv_blocks + jfa::kBwdBlockN / jfa::kMaskBlock - 1) /
                                              (jfa::kBwdBlockN / jfa::kMaskBlock));
        if (info->sparse_rows != rows) return JFA_ERR_PLAN_MISMATCH;
        if (d_sparse_ptr == nullptr || (info->sparse_nnz > 0 && d_sparse_idx == nullptr))
            return JFA_ERR_INVALID_ARG;
    } else if (info->sparse_rows != 0) {
        return JFA_ERR_PLAN_MISMATCH;
    }
    if (info->num_tiles > 0 && (d_worker_ptr == nullptr || d_tiles == nullptr))
        return JFA_ERR_INVALID_ARG;
    if (info->num_tiles > 0 && d_kv_offsets == nullptr) return JFA_ERR_INVALID_ARG;
    if (info->num_tiles > 0 && !p->broadcast_q && d_q_offsets == nullptr)
        return JFA_ERR_INVALID_ARG;
    return JFA_OK;
}

bool tensor_ok(const void* ptr, int64_t elems) {
    if (elems == 0) return true;
    return ptr != nullptr && aligned16(ptr);
}

// E8M0 scale arrays (read a dword at a time): may be NULL when empty
bool scales_ok(const void* ptr, int64_t bytes) {
    if (bytes == 0) return true;
    return ptr != nullptr && aligned4(ptr);
}

// Executed-tile log of debug builds: where the kernels write it (null: off).
std::atomic<int32_t*> g_tile_log{nullptr};
std::atomic<int32_t> g_tile_log_cap{0};

template <typename Args>
void set_debug_fields(Args& a, int32_t batch) {
    a.batch = batch;
    a.tile_log = kTileLogBuild ? g_tile_log.load() : nullptr;
    a.tile_log_cap = g_tile_log_cap.load();
}

}  // namespace

namespace jfa {

bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("JFA_LOG");
        return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
    }();
    return on;
}

void log_line(const char* what, const jfa_problem* p, const jfa_plan_info* info, int32_t extra,
              int32_t status, double host_us) {
    char buf[512];
    int n = std::snprintf(buf, sizeof buf, "jfa: %s", what);
    if (p != nullptr && n > 0 && n < (int)sizeof buf)
        n += std::snprintf(buf + n, sizeof buf - n, " B=%d H=%d D=%d %s lq=%d causal=%d window=[%d,%d] mask=%dx%d",
                           p->batch, p->num_heads, p->head_dim, p->broadcast_q ? "broadcast-q" : "per-seq-q",
                           p->lq, p->causal, p->window_left, p->window_right, p->mask_q_blocks,
                           p->mask_kv_blocks);
    // a planner call's info is its output: only meaningful when it succeeded
    const bool info_out = std::strncmp(what, "jfa_plan", 8) == 0;
    if (info != nullptr && (status == JFA_OK || !info_out) && n > 0 && n < (int)sizeof buf)
        n += std::snprintf(buf + n, sizeof buf - n, " pass=%d workers=%d tiles=%d work=%lld",
                           info->pass, info->num_workers, info->num_tiles, (long long)info->total_work);
    if (n > 0 && n < (int)sizeof buf)
        std::snprintf(buf + n, sizeof buf - n, " arg=%d -> %s (%d) %.1f us host\n", extra,
                      jfa_status_string(status), status, host_us);
    std::fputs(buf, stderr);
}

}  // namespace jfa

extern "C" {

int32_t jfa_abi_version(void) { return JFA_ABI_VERSION; }

const char* jfa_status_string(int32_t status) {
    switch (status) {
        case JFA_OK: return "ok";
        case JFA_ERR_INVALID_ARG: return "invalid argument";
        case JFA_ERR_BAD_OFFSETS: return "bad offsets (offsets[0] != 0, decreasing, or overflow)";
        case JFA_ERR_UNSUPPORTED: return "unsupported problem (head_dim, causal/window mode or mask)";
        case JFA_ERR_PLAN_MISMATCH: return "plan does not match the problem or pass";
        case JFA_ERR_WORKSPACE: return "workspace too small";
        case JFA_ERR_HIP: return "HIP call failed";
        case JFA_ERR_BAD_MASK: return "block mask missing or too small";
        default: return "unknown status";
    }
}

int32_t jfa_last_hip_error(void) { return g_last_hip_error; }

int32_t jfa_device_workers(int32_t device, int32_t* num_cus) {
    if (num_cus == nullptr) return JFA_ERR_INVALID_ARG;
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess) return hip_status((int32_t)e);
    if (device < 0 || device >= count) return JFA_ERR_INVALID_ARG;
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_status((int32_t)e);
    *num_cus = cus;
    return JFA_OK;
}

int32_t jfa_fwd_workspace_bytes(const jfa_problem* prob, const jfa_plan_info* info,
                                int64_t* bytes) {
    if (bytes == nullptr || info == nullptr) return JFA_ERR_INVALID_ARG;
    int32_t st = jfa::check_problem(prob);
    if (st) return st;
    if (info->pass == JFA_PASS_FWD) *bytes = 0;
    else if (info->pass == (JFA_PASS_FWD | JFA_PLAN_DYNAMIC)) *bytes = jfa::kFwdCounterBytes;
    else return JFA_ERR_PLAN_MISMATCH;
    return JFA_OK;
}

}  // extern "C"

// Validation and argument set-up shared by jfa_fwd and jfa_fwd_mx; returns
// JFA_OK with *launch = false when there is nothing to do.
static int32_t fwd_args(const jfa_problem* prob, const jfa_plan_info* info, const int32_t* d_worker_ptr,
                        const int32_t* d_tiles, const int32_t* d_sparse_ptr,
                        const int32_t* d_sparse_idx, const int32_t* d_q_offsets,
                        const int32_t* d_kv_offsets, void* o, float* lse, void* workspace,
                        int64_t workspace_bytes, jfa::FwdArgs& a, bool* launch) {
    *launch = false;
    int32_t st = check_common(prob, info, JFA_PASS_FWD, d_worker_ptr, d_tiles, d_sparse_ptr,
                              d_sparse_idx, d_q_offsets, d_kv_offsets);
    if (st) return st;
    int64_t need = 0;
    st = jfa_fwd_workspace_bytes(prob, info, &need);
    if (st) return st;
    if (workspace_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace))))
        return JFA_ERR_WORKSPACE;
    if (info->num_tiles == 0) return JFA_OK;  // no output row exists
    const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
    if (!tensor_ok(o, (int64_t)info->total_q * hd)) return JFA_ERR_INVALID_ARG;
    if (lse == nullptr || !aligned4(lse)) return JFA_ERR_INVALID_ARG;
    a = jfa::FwdArgs{};
    a.worker_ptr = d_worker_ptr;
    a.tiles = d_tiles;
    a.sp_ptr = d_sparse_ptr;
    a.sp_idx = d_sparse_idx;
    a.q_off = prob->broadcast_q ? nullptr : d_q_offsets;
    a.kv_off = d_kv_offsets;
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.num_heads = prob->num_heads;
    a.lq = prob->lq;
    a.total_q = info->total_q;
    a.mask_q_blocks = prob->mask_q_blocks;
    a.num_workers = info->num_workers;
    a.num_tiles = info->num_tiles;
    const jfa::Band bd = jfa::band_of(prob);
    a.win_left = bd.left;
    a.win_right = bd.right;
    a.counter = need > 0 ? static_cast<int32_t*>(workspace) : nullptr;
    a.scale_log2 = prob->softmax_scale * 1.4426950408889634f;
    a.q_rows = prob->broadcast_q ? prob->lq : info->total_q;
    a.total_kv = info->total_kv;
    set_debug_fields(a, prob->batch);
    *launch = true;
    return JFA_OK;
}

extern "C" {

int32_t jfa_fwd(const jfa_problem* prob, const jfa_plan_info* info, const int32_t* d_worker_ptr,
                const int32_t* d_tiles, const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                const int32_t* d_q_offsets, const int32_t* d_kv_offsets, const void* q,
                const void* k, const void* v, void* o, float* lse, void* workspace,
                int64_t workspace_bytes, void* stream) {
    return jfa::logged("jfa_fwd", prob, info, 0, [&]() -> int32_t {
        jfa::FwdArgs a;
        bool launch = false;
        int32_t st = fwd_args(prob, info, d_worker_ptr, d_tiles, d_sparse_ptr, d_sparse_idx, d_q_offsets,
                              d_kv_offsets, o, lse, workspace, workspace_bytes, a, &launch);
        if (st || !launch) return st;
        const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
        if (!tensor_ok(q, (int64_t)a.q_rows * hd) || !tensor_ok(k, info->total_kv * hd) ||
            !tensor_ok(v, info->total_kv * hd))
            return JFA_ERR_INVALID_ARG;
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        return hip_status(jfa::launch_fwd(a, prob->head_dim, mode_of(prob), prob->broadcast_q != 0,
                                          stream));
    });
}

int32_t jfa_mx_block_offsets(const int32_t* h_kv_offsets, int32_t batch, int32_t* h_block_offsets) {
    if (batch < 0 || h_kv_offsets == nullptr || h_block_offsets == nullptr) return JFA_ERR_INVALID_ARG;
    int32_t st = jfa::check_offsets(h_kv_offsets, batch);
    if (st) return st;
    int64_t acc = 0;
    h_block_offsets[0] = 0;
    for (int32_t b = 0; b < batch; ++b) {
        acc += ((int64_t)h_kv_offsets[b + 1] - h_kv_offsets[b] + 31) / 32;
        h_block_offsets[b + 1] = (int32_t)acc;
    }
    return JFA_OK;
}

int32_t jfa_mx_quantize_rows(const void* src, int64_t rows, int32_t num_heads, int32_t head_dim,
                             void* codes, void* scales, void* stream) {
    if (rows < 0 || num_heads < 1 || head_dim < 32 || head_dim % 32 != 0) return JFA_ERR_INVALID_ARG;
    const int64_t n = rows * num_heads * head_dim;
    if (n > 0 && (src == nullptr || codes == nullptr || scales == nullptr || !aligned16(src) ||
                  !aligned16(codes)))
        return JFA_ERR_INVALID_ARG;
    return hip_status(jfa::launch_mx_quant_rows(static_cast<const uint16_t*>(src), rows, num_heads,
                                                head_dim, static_cast<uint8_t*>(codes),
                                                static_cast<uint8_t*>(scales), stream));
}

int32_t jfa_mx_quantize_v(const void* v, const int32_t* d_kv_offsets, const int32_t* d_block_offsets,
                          int32_t batch, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                          void* codes, void* scales, void* stream) {
    if (batch < 0 || num_heads < 1 || head_dim < 32 || head_dim > 128 || head_dim % 32 != 0 ||
        num_blocks < 0)
        return JFA_ERR_INVALID_ARG;
    if (batch > 0 && (d_kv_offsets == nullptr || d_block_offsets == nullptr)) return JFA_ERR_INVALID_ARG;
    if (num_blocks > 0 && (v == nullptr || codes == nullptr || scales == nullptr))
        return JFA_ERR_INVALID_ARG;
    return hip_status(jfa::launch_mx_quant_v(static_cast<const uint16_t*>(v), d_kv_offsets,
                                             d_block_offsets, batch, num_heads, head_dim, num_blocks,
                                             static_cast<uint8_t*>(codes),
                                             static_cast<uint8_t*>(scales), stream));
}

int32_t jfa_fwd_mx(const jfa_problem* prob, const jfa_plan_info* info, const int32_t* d_worker_ptr,
                   const int32_t* d_tiles, const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                   const int32_t* d_q_offsets, const int32_t* d_kv_offsets,
                   const int32_t* d_block_offsets, int32_t num_blocks, const void* q_codes,
                   const void* q_scales, const void* k_codes, const void* k_scales,
                   const void* v_codes, const void* v_scales, void* o, float* lse, void* workspace,
                   int64_t workspace_bytes, void* stream) {
    return jfa::logged("jfa_fwd_mx", prob, info, 0, [&]() -> int32_t {
        int32_t st = jfa::check_problem(prob);
        if (st) return st;
        if (prob->head_dim != 128) return JFA_ERR_UNSUPPORTED;
        jfa::FwdArgs a;
        bool launch = false;
        st = fwd_args(prob, info, d_worker_ptr, d_tiles, d_sparse_ptr, d_sparse_idx, d_q_offsets,
                      d_kv_offsets, o, lse, workspace, workspace_bytes, a, &launch);
        if (st || !launch) return st;
        // one 32-key V block per 32 keys of each sequence: at least T_k / 32
        if (num_blocks < (info->total_kv + 31) / 32 || d_block_offsets == nullptr) return JFA_ERR_INVALID_ARG;
        const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
        const int64_t H = prob->num_heads, nbd = prob->head_dim / 32;
        if (!tensor_ok(q_codes, (int64_t)a.q_rows * hd) || !tensor_ok(k_codes, info->total_kv * hd) ||
            !tensor_ok(v_codes, info->total_kv * hd) || !scales_ok(q_scales, H * a.q_rows * nbd) ||
            !scales_ok(k_scales, H * info->total_kv * nbd) ||
            !scales_ok(v_scales, H * (int64_t)num_blocks * prob->head_dim))
            return JFA_ERR_INVALID_ARG;
        a.q8 = static_cast<const uint8_t*>(q_codes);
        a.k8 = static_cast<const uint8_t*>(k_codes);
        a.v8 = static_cast<const uint8_t*>(v_codes);
        a.q_sc = static_cast<const uint8_t*>(q_scales);
        a.k_sc = static_cast<const uint8_t*>(k_scales);
        a.v_sc = static_cast<const uint8_t*>(v_scales);
        a.v_boff = d_block_offsets;
        a.v_nb = num_blocks;
        return hip_status(jfa::launch_fwd_mx(a, mode_of(prob), prob->broadcast_q != 0, stream));
    });
}

int32_t jfa_bwd_workspace_bytes(const jfa_problem* prob, const jfa_plan_info* dq_info,
                                int64_t* bytes) {
    if (bytes == nullptr || dq_info == nullptr) return JFA_ERR_INVALID_ARG;
    int32_t st = jfa::check_problem(prob);
    if (st) return st;
    if (dq_info->pass != JFA_PASS_DQ || dq_info->num_workers < 1) return JFA_ERR_PLAN_MISMATCH;
    // broadcast Q: one fp32 [256][D] partial per dQ worker
    *bytes = prob->broadcast_q
                 ? (int64_t)dq_info->num_workers * jfa::kFwdBlockM * prob->head_dim * 4
                 : 0;
    return JFA_OK;
}

static int32_t check_plan(const jfa_problem* prob, const jfa_device_plan* plan, int32_t pass,
                          const int32_t* d_q_offsets, const int32_t* d_kv_offsets) {
    if (plan == nullptr) return JFA_ERR_INVALID_ARG;
    return check_common(prob, plan->info, pass, plan->worker_ptr, plan->tiles, plan->sparse_ptr,
                        plan->sparse_idx, d_q_offsets, d_kv_offsets);
}

int32_t jfa_bwd_stages(int32_t stages, const jfa_problem* prob, const jfa_device_plan* kv_plan,
                       const jfa_device_plan* dq_plan, const int32_t* d_q_offsets,
                       const int32_t* d_kv_offsets, const void* q, const void* k, const void* v,
                       const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                       void* dv, float* dq_accum, float* delta, void* workspace,
                       int64_t workspace_bytes, void* stream) {
    return jfa::logged("jfa_bwd_stages", prob, kv_plan != nullptr ? kv_plan->info : nullptr, stages, [&]() -> int32_t {
        if (stages < 0 || stages > (JFA_BWD_ALL | JFA_BWD_PREPROCESS | JFA_BWD_DQ_ATOMIC))
            return JFA_ERR_INVALID_ARG;
        int32_t st = check_plan(prob, kv_plan, JFA_PASS_BWD, d_q_offsets, d_kv_offsets);
        if (st) return st;
        st = check_plan(prob, dq_plan, JFA_PASS_DQ, d_q_offsets, d_kv_offsets);
        if (st) return st;
        const jfa_plan_info* ki = kv_plan->info;
        const jfa_plan_info* qi = dq_plan->info;
        if (ki->total_q != qi->total_q || ki->total_kv != qi->total_kv) return JFA_ERR_PLAN_MISMATCH;
        int64_t need = 0;
        st = jfa_bwd_workspace_bytes(prob, qi, &need);
        if (st) return st;
        if (workspace_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace))))
            return JFA_ERR_WORKSPACE;
        const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
        const int64_t q_rows = prob->broadcast_q ? prob->lq : ki->total_q;
        const int64_t tq = ki->total_q, tk = ki->total_kv;
        if (!tensor_ok(q, q_rows * hd) || !tensor_ok(k, tk * hd) || !tensor_ok(v, tk * hd) ||
            !tensor_ok(o, tq * hd) || !tensor_ok(d_o, tq * hd) || !tensor_ok(dq, q_rows * hd) ||
            !tensor_ok(dk, tk * hd) || !tensor_ok(dv, tk * hd) || !tensor_ok(dq_accum, q_rows * hd))
            return JFA_ERR_INVALID_ARG;
        if (tq > 0 && (lse == nullptr || delta == nullptr || !aligned4(lse) || !aligned4(delta)))
            return JFA_ERR_INVALID_ARG;
        if (tq == 0 && q_rows == 0 && tk == 0) return JFA_OK;
        const jfa::Mode mode = mode_of(prob);
        const bool bcast = prob->broadcast_q != 0;
        const bool atomic = bcast && (stages & JFA_BWD_DQ_ATOMIC) != 0;

        jfa::BwdArgs a{};
        set_debug_fields(a, prob->batch);
        a.worker_ptr = kv_plan->worker_ptr;
        a.tiles = kv_plan->tiles;
        a.sp_ptr = kv_plan->sparse_ptr;
        a.sp_idx = kv_plan->sparse_idx;
        a.q_off = bcast ? nullptr : d_q_offsets;
        a.kv_off = d_kv_offsets;
        a.q = static_cast<const uint16_t*>(q);
        a.k = static_cast<const uint16_t*>(k);
        a.v = static_cast<const uint16_t*>(v);
        a.o = static_cast<const uint16_t*>(o);
        a.lse = lse;
        a.d_o = static_cast<const uint16_t*>(d_o);
        a.dk = static_cast<uint16_t*>(dk);
        a.dv = static_cast<uint16_t*>(dv);
        a.delta = delta;
        a.num_heads = prob->num_heads;
        a.lq = prob->lq;
        a.total_q = ki->total_q;
        a.mask_kv_blocks = prob->mask_kv_blocks;
        a.num_workers = ki->num_tiles > 0 ? ki->num_workers : 0;  // 0: no dK/dV launch
        const jfa::Band bd = jfa::band_of(prob);
        a.win_left = bd.left;
        a.win_right = bd.right;
        a.scale = prob->softmax_scale;
        a.scale_log2 = prob->softmax_scale * 1.4426950408889634f;
        if (stages & JFA_BWD_PREPROCESS) {
            st = hip_status(jfa::launch_bwd(a, prob->head_dim, mode, bcast, JFA_BWD_PREPROCESS, stream));
            if (st) return st;
        }

        if ((stages & JFA_BWD_DQ) && atomic) {
            st = hip_status(jfa::launch_dq_zero(dq_accum, q_rows * hd, stream));
            if (st) return st;
        }
        if ((stages & JFA_BWD_DQ) && qi->num_tiles > 0) {
            jfa::DqArgs d{};
            d.worker_ptr = dq_plan->worker_ptr;
            d.tiles = dq_plan->tiles;
            d.sp_ptr = dq_plan->sparse_ptr;
            d.sp_idx = dq_plan->sparse_idx;
            d.q_off = bcast ? nullptr : d_q_offsets;
            d.kv_off = d_kv_offsets;
            d.q = a.q;
            d.k = a.k;
            d.v = a.v;
            d.d_o = a.d_o;
            d.o = a.o;
            d.lse = lse;
            d.delta = delta;
            d.dq = static_cast<uint16_t*>(dq);
            d.dq_accum = dq_accum;
            d.partial = static_cast<float*>(workspace);
            d.chunk_div = bcast ? (prob->lq + jfa::kFwdBlockM - 1) / jfa::kFwdBlockM : 0;
            d.win_left = bd.left;
            d.win_right = bd.right;
            d.num_heads = prob->num_heads;
            d.lq = prob->lq;
            d.total_q = qi->total_q;
            d.mask_q_blocks = prob->mask_q_blocks;
            d.num_workers = qi->num_workers;
            d.scale = prob->softmax_scale;
            d.scale_log2 = a.scale_log2;
            set_debug_fields(d, prob->batch);
            st = hip_status(jfa::launch_dq(d, prob->head_dim, mode, bcast, atomic, stream));
            if (st) return st;
        }
        if (stages & JFA_BWD_DKDV) {
            st = hip_status(jfa::launch_bwd(a, prob->head_dim, mode, bcast, JFA_BWD_DKDV, stream));
            if (st) return st;
        }
        if ((stages & JFA_BWD_DQ_REDUCE) && atomic) {
            st = hip_status(jfa::launch_dq_convert(dq_accum, static_cast<uint16_t*>(dq), q_rows * hd, stream));
            if (st) return st;
        } else if ((stages & JFA_BWD_DQ_REDUCE) && bcast) {
            jfa::DqReduceArgs r;
            r.worker_ptr = dq_plan->worker_ptr;
            r.partial = static_cast<const float*>(workspace);
            r.dq_accum = dq_accum;
            r.dq = static_cast<uint16_t*>(dq);
            r.num_heads = prob->num_heads;
            r.lq = prob->lq;
            r.num_workers = qi->num_workers;
            if (qi->num_tiles > 0 && r.worker_ptr == nullptr) return JFA_ERR_INVALID_ARG;
            if (qi->num_tiles == 0) r.worker_ptr = nullptr;
            st = hip_status(jfa::launch_dq_reduce(r, prob->head_dim, stream));
            if (st) return st;
        }
        return JFA_OK;
    });
}

int32_t jfa_bwd_dq_mx(const jfa_problem* prob, const jfa_device_plan* dq_plan,
                      const int32_t* d_q_offsets, const int32_t* d_kv_offsets,
                      const int32_t* d_key_block_offsets, int32_t num_key_blocks, const void* o,
                      const float* lse, const void* d_o, const jfa_mx_bwd_operands* ops, void* dq,
                      float* dq_accum, float* delta, void* workspace, int64_t workspace_bytes,
                      void* stream) {
    return jfa::logged("jfa_bwd_dq_mx", prob, dq_plan != nullptr ? dq_plan->info : nullptr, 0, [&]() -> int32_t {
        int32_t st = check_plan(prob, dq_plan, JFA_PASS_DQ, d_q_offsets, d_kv_offsets);
        if (st) return st;
        if (prob->head_dim != 128) return JFA_ERR_UNSUPPORTED;
        const jfa_plan_info* qi = dq_plan->info;
        int64_t need = 0;
        st = jfa_bwd_workspace_bytes(prob, qi, &need);
        if (st) return st;
        if (workspace_bytes < need || (need > 0 && (workspace == nullptr || !aligned16(workspace))))
            return JFA_ERR_WORKSPACE;
        const bool bcast = prob->broadcast_q != 0;
        const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
        const int64_t q_rows = bcast ? prob->lq : qi->total_q;
        if (ops == nullptr || d_key_block_offsets == nullptr || num_key_blocks < (qi->total_kv + 31) / 32)
            return JFA_ERR_INVALID_ARG;
        // (no query row at all: O, dO, LSE, delta and dQ may be empty)
        if (qi->total_q > 0 && (lse == nullptr || delta == nullptr || !aligned4(lse) || !aligned4(delta)))
            return JFA_ERR_INVALID_ARG;
        if (!tensor_ok(o, qi->total_q * hd) || !tensor_ok(d_o, qi->total_q * hd) ||
            !tensor_ok(ops->q_codes, q_rows * hd) ||
            !tensor_ok(ops->k_codes, qi->total_kv * hd) || !tensor_ok(ops->v_codes, qi->total_kv * hd) ||
            !tensor_ok(ops->do_codes, qi->total_q * hd) || !tensor_ok(ops->kk_codes, qi->total_kv * hd))
            return JFA_ERR_INVALID_ARG;
        const int64_t H = prob->num_heads, nbd = prob->head_dim / 32;
        if (!scales_ok(ops->q_scales, H * q_rows * nbd) || !scales_ok(ops->k_scales, H * qi->total_kv * nbd) ||
            !scales_ok(ops->v_scales, H * qi->total_kv * nbd) ||
            !scales_ok(ops->do_scales, H * qi->total_q * nbd) ||
            !scales_ok(ops->kk_scales, H * (int64_t)num_key_blocks * prob->head_dim))
            return JFA_ERR_INVALID_ARG;
        if (!bcast && (!tensor_ok(dq, qi->total_q * hd) || (qi->total_q > 0 && dq_accum == nullptr)))
            return JFA_ERR_INVALID_ARG;
        if (qi->num_tiles == 0) return JFA_OK;
        const jfa::Band bd = jfa::band_of(prob);
        jfa::DqArgs d{};
        d.worker_ptr = dq_plan->worker_ptr;
        d.tiles = dq_plan->tiles;
        d.sp_ptr = dq_plan->sparse_ptr;
        d.sp_idx = dq_plan->sparse_idx;
        d.q_off = bcast ? nullptr : d_q_offsets;
        d.kv_off = d_kv_offsets;
        d.d_o = static_cast<const uint16_t*>(d_o);
        d.o = static_cast<const uint16_t*>(o);
        d.lse = lse;
        d.delta = delta;
        d.dq = static_cast<uint16_t*>(dq);
        d.dq_accum = dq_accum;
        d.partial = static_cast<float*>(workspace);
        d.chunk_div = bcast ? (prob->lq + jfa::kFwdBlockM - 1) / jfa::kFwdBlockM : 0;
        d.win_left = bd.left;
        d.win_right = bd.right;
        d.num_heads = prob->num_heads;
        d.lq = prob->lq;
        d.total_q = qi->total_q;
        d.mask_q_blocks = prob->mask_q_blocks;
        d.num_workers = qi->num_workers;
        d.scale = prob->softmax_scale;
        d.scale_log2 = prob->softmax_scale * 1.4426950408889634f;
        d.q8 = static_cast<const uint8_t*>(ops->q_codes);
        d.q_sc = static_cast<const uint8_t*>(ops->q_scales);
        d.k8 = static_cast<const uint8_t*>(ops->k_codes);
        d.k_sc = static_cast<const uint8_t*>(ops->k_scales);
        d.v8 = static_cast<const uint8_t*>(ops->v_codes);
        d.v_sc = static_cast<const uint8_t*>(ops->v_scales);
        d.do8 = static_cast<const uint8_t*>(ops->do_codes);
        d.do_sc = static_cast<const uint8_t*>(ops->do_scales);
        d.kk8 = static_cast<const uint8_t*>(ops->kk_codes);
        d.kk_sc = static_cast<const uint8_t*>(ops->kk_scales);
        d.kk_boff = d_key_block_offsets;
        d.kk_nb = num_key_blocks;
        d.q_rows = (int32_t)q_rows;
        d.total_kv = qi->total_kv;
        set_debug_fields(d, prob->batch);
        return hip_status(jfa::launch_dq_mx(d, mode_of(prob), bcast, stream));
    });
}

int32_t jfa_bwd_dkdv_mx(const jfa_problem* prob, const jfa_device_plan* kv_plan,
                        const int32_t* d_q_offsets, const int32_t* d_kv_offsets,
                        const int32_t* d_q_row_block_offsets, int32_t num_q_row_blocks,
                        const int32_t* d_do_row_block_offsets, int32_t num_do_row_blocks,
                        const float* lse, const float* delta, const jfa_mx_dkdv_operands* ops,
                        void* dk, void* dv, void* stream) {
    return jfa::logged("jfa_bwd_dkdv_mx", prob, kv_plan != nullptr ? kv_plan->info : nullptr, 0, [&]() -> int32_t {
        int32_t st = check_plan(prob, kv_plan, JFA_PASS_BWD, d_q_offsets, d_kv_offsets);
        if (st) return st;
        if (prob->head_dim != 128) return JFA_ERR_UNSUPPORTED;
        const jfa_plan_info* ki = kv_plan->info;
        const bool bcast = prob->broadcast_q != 0;
        const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
        const int64_t q_rows = bcast ? prob->lq : ki->total_q;
        const int64_t tq = ki->total_q, tk = ki->total_kv;
        if (ops == nullptr || num_q_row_blocks < 0 || num_do_row_blocks < 0) return JFA_ERR_INVALID_ARG;
        // one 32-row block per 32 rows of each sequence: at least rows / 32
        if (num_q_row_blocks < (q_rows + 31) / 32 || num_do_row_blocks < (tq + 31) / 32)
            return JFA_ERR_INVALID_ARG;
        if (ki->num_tiles > 0 && (d_do_row_block_offsets == nullptr ||
                                  (!bcast && d_q_row_block_offsets == nullptr)))
            return JFA_ERR_INVALID_ARG;
        if (!tensor_ok(dk, tk * hd) || !tensor_ok(dv, tk * hd) || !tensor_ok(ops->q_codes, q_rows * hd) ||
            !tensor_ok(ops->k_codes, tk * hd) || !tensor_ok(ops->v_codes, tk * hd) ||
            !tensor_ok(ops->do_codes, tq * hd) || !tensor_ok(ops->qr_codes, q_rows * hd) ||
            !tensor_ok(ops->dor_codes, tq * hd))
            return JFA_ERR_INVALID_ARG;
        const int64_t H = prob->num_heads, nbd = prob->head_dim / 32;
        if (!scales_ok(ops->q_scales, H * q_rows * nbd) || !scales_ok(ops->k_scales, H * tk * nbd) ||
            !scales_ok(ops->v_scales, H * tk * nbd) || !scales_ok(ops->do_scales, H * tq * nbd) ||
            !scales_ok(ops->qr_scales, H * (int64_t)num_q_row_blocks * prob->head_dim) ||
            !scales_ok(ops->dor_scales, H * (int64_t)num_do_row_blocks * prob->head_dim))
            return JFA_ERR_INVALID_ARG;
        if (tq > 0 && (lse == nullptr || delta == nullptr || !aligned4(lse) || !aligned4(delta)))
            return JFA_ERR_INVALID_ARG;
        if (ki->num_tiles == 0) return JFA_OK;
        const jfa::Band bd = jfa::band_of(prob);
        jfa::BwdArgs a{};
        set_debug_fields(a, prob->batch);
        a.worker_ptr = kv_plan->worker_ptr;
        a.tiles = kv_plan->tiles;
        a.sp_ptr = kv_plan->sparse_ptr;
        a.sp_idx = kv_plan->sparse_idx;
        a.q_off = bcast ? nullptr : d_q_offsets;
        a.kv_off = d_kv_offsets;
        a.lse = lse;
        a.delta = const_cast<float*>(delta);
        a.dk = static_cast<uint16_t*>(dk);
        a.dv = static_cast<uint16_t*>(dv);
        a.num_heads = prob->num_heads;
        a.lq = prob->lq;
        a.total_q = ki->total_q;
        a.mask_kv_blocks = prob->mask_kv_blocks;
        a.num_workers = ki->num_workers;
        a.win_left = bd.left;
        a.win_right = bd.right;
        a.scale = prob->softmax_scale;
        a.scale_log2 = prob->softmax_scale * 1.4426950408889634f;
        a.q8 = static_cast<const uint8_t*>(ops->q_codes);
        a.q_sc = static_cast<const uint8_t*>(ops->q_scales);
        a.k8 = static_cast<const uint8_t*>(ops->k_codes);
        a.k_sc = static_cast<const uint8_t*>(ops->k_scales);
        a.v8 = static_cast<const uint8_t*>(ops->v_codes);
        a.v_sc = static_cast<const uint8_t*>(ops->v_scales);
        a.do8 = static_cast<const uint8_t*>(ops->do_codes);
        a.do_sc = static_cast<const uint8_t*>(ops->do_scales);
        a.qr8 = static_cast<const uint8_t*>(ops->qr_codes);
        a.qr_sc = static_cast<const uint8_t*>(ops->qr_scales);
        a.dor8 = static_cast<const uint8_t*>(ops->dor_codes);
        a.dor_sc = static_cast<const uint8_t*>(ops->dor_scales);
        a.qr_boff = d_q_row_block_offsets;
        a.dor_boff = d_do_row_block_offsets;
        a.qr_nb = num_q_row_blocks;
        a.dor_nb = num_do_row_blocks;
        a.q_rows = (int32_t)q_rows;
        a.total_kv = ki->total_kv;
        return hip_status(jfa::launch_dkdv_mx(a, mode_of(prob), bcast, stream));
    });
}

int32_t jfa_bwd_noalloc(const jfa_problem* prob, const jfa_device_plan* kv_plan,
                        const jfa_device_plan* dq_plan, const int32_t* d_q_offsets,
                        const int32_t* d_kv_offsets, const void* q, const void* k, const void* v,
                        const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                        void* dv, float* dq_accum, float* delta, void* stream) {
    if (dq_plan == nullptr) return JFA_ERR_INVALID_ARG;
    int64_t need = 0;
    int32_t st = jfa_bwd_workspace_bytes(prob, dq_plan->info, &need);
    if (st) return st;
    if (need > (int64_t)JFA_NOALLOC_SCRATCH_BYTES) return JFA_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        st = hip_status(jfa::noalloc_scratch(&ws));
        if (st) return st;
        if (ws == nullptr || !aligned16(ws)) return JFA_ERR_HIP;
    }
    return jfa_bwd_stages(JFA_BWD_ALL, prob, kv_plan, dq_plan, d_q_offsets, d_kv_offsets, q, k, v,
                          o, lse, d_o, dq, dk, dv, dq_accum, delta, ws, need, stream);
}

int32_t jfa_bwd(const jfa_problem* prob, const jfa_device_plan* kv_plan,
                const jfa_device_plan* dq_plan, const int32_t* d_q_offsets,
                const int32_t* d_kv_offsets, const void* q, const void* k, const void* v,
                const void* o, const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                float* dq_accum, float* delta, void* workspace, int64_t workspace_bytes,
                void* stream) {
    return jfa_bwd_stages(JFA_BWD_ALL, prob, kv_plan, dq_plan, d_q_offsets, d_kv_offsets, q, k, v,
                          o, lse, d_o, dq, dk, dv, dq_accum, delta, workspace, workspace_bytes,
                          stream);
}

int32_t jfa_debug_tile_log(int32_t* d_log, int32_t records_per_worker) {
    if (!kTileLogBuild) return JFA_ERR_UNSUPPORTED;
    if (d_log != nullptr && (records_per_worker < 0 || !aligned16(d_log))) return JFA_ERR_INVALID_ARG;
    g_tile_log_cap.store(d_log != nullptr ? records_per_worker : 0);
    g_tile_log.store(d_log);
    return JFA_OK;
}

}  // extern "C"
