// C ABI entry points: argument validation and kernel launches on the caller's
// stream. Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>

#include "internal.h"

namespace {

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
    if (p->causal) return jfa::kCausal;
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
    if (info->pass != pass) return JFA_ERR_PLAN_MISMATCH;
    const int32_t bm = pass == JFA_PASS_FWD ? jfa::kFwdBlockM : jfa::kBwdBlockM;
    const int32_t bn = pass == JFA_PASS_FWD ? jfa::kFwdBlockN : jfa::kBwdBlockN;
    if (info->block_m != bm || info->block_n != bn) return JFA_ERR_PLAN_MISMATCH;
    if (info->num_workers < 1 || info->num_tiles < 0 || info->total_q < 0 || info->total_kv < 0)
        return JFA_ERR_PLAN_MISMATCH;
    if (p->broadcast_q && info->total_q != (int64_t)p->batch * p->lq) return JFA_ERR_PLAN_MISMATCH;
    const bool sparse = p->mask_q_blocks != 0;
    if (sparse) {
        const int64_t rows =
            (int64_t)p->batch * (pass == JFA_PASS_FWD
                                     ? (p->mask_q_blocks + jfa::kFwdBlockM / jfa::kMaskBlock - 1) /
                                           (jfa::kFwdBlockM / jfa::kMaskBlock)
                                     : p->mask_kv_blocks);
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

}  // namespace

extern "C" {

int32_t jfa_abi_version(void) { return JFA_ABI_VERSION; }

const char* jfa_status_string(int32_t status) {
    switch (status) {
        case JFA_OK: return "ok";
        case JFA_ERR_INVALID_ARG: return "invalid argument";
        case JFA_ERR_BAD_OFFSETS: return "bad offsets (offsets[0] != 0, decreasing, or overflow)";
        case JFA_ERR_UNSUPPORTED: return "unsupported problem (head_dim, causal mode or mask)";
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

int32_t jfa_fwd(const jfa_problem* prob, const jfa_plan_info* info, const int32_t* d_worker_ptr,
                const int32_t* d_tiles, const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                const int32_t* d_q_offsets, const int32_t* d_kv_offsets, const void* q,
                const void* k, const void* v, void* o, float* lse, void* stream) {
    int32_t st = check_common(prob, info, JFA_PASS_FWD, d_worker_ptr, d_tiles, d_sparse_ptr,
                              d_sparse_idx, d_q_offsets, d_kv_offsets);
    if (st) return st;
    if (info->num_tiles == 0) return JFA_OK;  // no output row exists
    const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
    const int64_t q_rows = prob->broadcast_q ? prob->lq : info->total_q;
    if (!tensor_ok(q, q_rows * hd) || !tensor_ok(k, info->total_kv * hd) ||
        !tensor_ok(v, info->total_kv * hd) || !tensor_ok(o, (int64_t)info->total_q * hd))
        return JFA_ERR_INVALID_ARG;
    if (lse == nullptr || !aligned4(lse)) return JFA_ERR_INVALID_ARG;

    jfa::FwdArgs a;
    a.worker_ptr = d_worker_ptr;
    a.tiles = d_tiles;
    a.sp_ptr = d_sparse_ptr;
    a.sp_idx = d_sparse_idx;
    a.q_off = prob->broadcast_q ? nullptr : d_q_offsets;
    a.kv_off = d_kv_offsets;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<uint16_t*>(o);
    a.lse = lse;
    a.num_heads = prob->num_heads;
    a.lq = prob->lq;
    a.total_q = info->total_q;
    a.mask_q_blocks = prob->mask_q_blocks;
    a.num_workers = info->num_workers;
    a.scale_log2 = prob->softmax_scale * 1.4426950408889634f;
    return hip_status(jfa::launch_fwd(a, prob->head_dim, mode_of(prob), prob->broadcast_q != 0,
                                      stream));
}

int32_t jfa_bwd_workspace_bytes(const jfa_problem* prob, const jfa_plan_info* info,
                                int64_t* bytes) {
    if (bytes == nullptr || info == nullptr) return JFA_ERR_INVALID_ARG;
    int32_t st = jfa::check_problem(prob);
    if (st) return st;
    if (info->pass != JFA_PASS_BWD) return JFA_ERR_PLAN_MISMATCH;
    *bytes = 0;
    return JFA_OK;
}

int32_t jfa_bwd_stages(int32_t stages, const jfa_problem* prob, const jfa_plan_info* info,
                       const int32_t* d_worker_ptr, const int32_t* d_tiles,
                       const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                       const int32_t* d_q_offsets, const int32_t* d_kv_offsets, const void* q,
                       const void* k, const void* v, const void* o, const float* lse,
                       const void* d_o, void* dq, void* dk, void* dv, float* dq_accum,
                       float* delta, void* workspace, int64_t workspace_bytes, void* stream) {
    if (stages < 0 || stages > JFA_BWD_ALL) return JFA_ERR_INVALID_ARG;
    int32_t st = check_common(prob, info, JFA_PASS_BWD, d_worker_ptr, d_tiles, d_sparse_ptr,
                              d_sparse_idx, d_q_offsets, d_kv_offsets);
    if (st) return st;
    int64_t need = 0;
    st = jfa_bwd_workspace_bytes(prob, info, &need);
    if (st) return st;
    if (workspace_bytes < need || (need > 0 && workspace == nullptr)) return JFA_ERR_WORKSPACE;
    const int64_t hd = (int64_t)prob->num_heads * prob->head_dim;
    const int64_t q_rows = prob->broadcast_q ? prob->lq : info->total_q;
    const int64_t tq = info->total_q, tk = info->total_kv;
    if (!tensor_ok(q, q_rows * hd) || !tensor_ok(k, tk * hd) || !tensor_ok(v, tk * hd) ||
        !tensor_ok(o, tq * hd) || !tensor_ok(d_o, tq * hd) || !tensor_ok(dq, q_rows * hd) ||
        !tensor_ok(dk, tk * hd) || !tensor_ok(dv, tk * hd) || !tensor_ok(dq_accum, q_rows * hd))
        return JFA_ERR_INVALID_ARG;
    if (tq > 0 && (lse == nullptr || delta == nullptr || !aligned4(lse) || !aligned4(delta)))
        return JFA_ERR_INVALID_ARG;
    if (tq == 0 && q_rows == 0 && tk == 0) return JFA_OK;

    jfa::BwdArgs a;
    a.worker_ptr = d_worker_ptr;
    a.tiles = d_tiles;
    a.sp_ptr = d_sparse_ptr;
    a.sp_idx = d_sparse_idx;
    a.q_off = prob->broadcast_q ? nullptr : d_q_offsets;
    a.kv_off = d_kv_offsets;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.o = static_cast<const uint16_t*>(o);
    a.lse = lse;
    a.d_o = static_cast<const uint16_t*>(d_o);
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.dq_accum = dq_accum;
    a.delta = delta;
    a.num_heads = prob->num_heads;
    a.lq = prob->lq;
    a.total_q = info->total_q;
    a.q_rows = (int32_t)q_rows;
    a.mask_kv_blocks = prob->mask_kv_blocks;
    a.num_workers = info->num_tiles > 0 ? info->num_workers : 0;  // 0: no main launch
    a.scale = prob->softmax_scale;
    a.scale_log2 = prob->softmax_scale * 1.4426950408889634f;
    return hip_status(jfa::launch_bwd(a, prob->head_dim, mode_of(prob), prob->broadcast_q != 0,
                                      stages, stream));
}

int32_t jfa_bwd(const jfa_problem* prob, const jfa_plan_info* info, const int32_t* d_worker_ptr,
                const int32_t* d_tiles, const int32_t* d_sparse_ptr, const int32_t* d_sparse_idx,
                const int32_t* d_q_offsets, const int32_t* d_kv_offsets, const void* q,
                const void* k, const void* v, const void* o, const float* lse, const void* d_o,
                void* dq, void* dk, void* dv, float* dq_accum, float* delta, void* workspace,
                int64_t workspace_bytes, void* stream) {
    return jfa_bwd_stages(JFA_BWD_ALL, prob, info, d_worker_ptr, d_tiles, d_sparse_ptr,
                          d_sparse_idx, d_q_offsets, d_kv_offsets, q, k, v, o, lse, d_o, dq, dk,
                          dv, dq_accum, delta, workspace, workspace_bytes, stream);
}

}  // extern "C"
