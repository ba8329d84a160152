"""Python binding of libjfa.so, the jagged FlashAttention library for MI355X.

Argument marshalling only: every step of forward and backward runs in the HIP
kernels behind the C ABI (include/jfa.h). The functions keep the C names;
torch is used for device memory and the current HIP stream. If the library is
not built, every call raises -- there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import dataclasses
import os
import time
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# JFA_LIBRARY names another build of the same library to load instead (the
# host-check build that the CPU tests run under the sanitizers).
LIB_PATH = os.environ.get("JFA_LIBRARY") or os.path.join(_HERE, "libjfa.so")
# the same library with the executed-tile log compiled in (jfa_debug_tile_log)
DEBUG_LIB_PATH = os.path.join(_HERE, "libjfa_debug.so")

JFA_OK = 0
JFA_ERR_INVALID_ARG = -1
JFA_ERR_BAD_OFFSETS = -2
JFA_ERR_UNSUPPORTED = -3
JFA_ERR_PLAN_MISMATCH = -4
JFA_ERR_WORKSPACE = -5
JFA_ERR_HIP = -6
JFA_ERR_BAD_MASK = -7
JFA_PASS_FWD = 0
JFA_PASS_BWD = 1
JFA_PASS_DQ = 2
JFA_PLAN_DYNAMIC = 16
JFA_PLAN_NATURAL = 32

EXPORTS = (
    "jfa_abi_version", "jfa_status_string", "jfa_last_hip_error", "jfa_device_workers",
    "jfa_offsets_from_lengths", "jfa_plan_query", "jfa_plan_build", "jfa_fwd_workspace_bytes",
    "jfa_fwd", "jfa_bwd_workspace_bytes", "jfa_bwd", "jfa_bwd_stages", "jfa_mx_block_offsets",
    "jfa_mx_quantize_rows", "jfa_mx_quantize_v", "jfa_fwd_mx", "jfa_bwd_dq_mx",
    "jfa_bwd_noalloc", "jfa_bwd_dkdv_mx", "jfa_debug_tile_log",
)
JFA_BWD_PREPROCESS = 1
JFA_BWD_DQ = 2
JFA_BWD_DKDV = 4
JFA_BWD_DQ_REDUCE = 8
JFA_BWD_ALL = 14
JFA_BWD_DQ_ATOMIC = 16


class JfaProblem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("broadcast_q", ctypes.c_int32),
                ("lq", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("mask_q_blocks", ctypes.c_int32), ("mask_kv_blocks", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32)]


class JfaPlanInfo(ctypes.Structure):
    _fields_ = [("pass_", ctypes.c_int32), ("num_workers", ctypes.c_int32),
                ("num_tiles", ctypes.c_int32), ("block_m", ctypes.c_int32),
                ("block_n", ctypes.c_int32), ("total_q", ctypes.c_int32),
                ("total_kv", ctypes.c_int32), ("sparse_rows", ctypes.c_int32),
                ("sparse_nnz", ctypes.c_int32), ("max_work", ctypes.c_int32),
                ("total_work", ctypes.c_int64)]


class JfaDevicePlan(ctypes.Structure):
    _fields_ = [("info", ctypes.POINTER(JfaPlanInfo)), ("worker_ptr", ctypes.c_void_p),
                ("tiles", ctypes.c_void_p), ("sparse_ptr", ctypes.c_void_p),
                ("sparse_idx", ctypes.c_void_p)]


class JfaMxBwdOperands(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales", "do_codes",
        "do_scales", "kk_codes", "kk_scales")]


class JfaMxDkdvOperands(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "q_codes", "q_scales", "k_codes", "k_scales", "v_codes", "v_scales", "do_codes",
        "do_scales", "qr_codes", "qr_scales", "dor_codes", "dor_scales")]


class JfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = "%s failed: %s (%d)" % (where, jfa_status_string(status), status)
        if status == JFA_ERR_HIP:
            msg += ", hipError %d" % _lib().jfa_last_hip_error()
        super().__init__(msg)
        self.status = status


_LIB = None

_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)


def _lib():
    global _LIB
    if _LIB is None:
        _LIB = load_library(LIB_PATH)
    return _LIB


def load_library(path):
    """A ctypes handle of a build of the library at ``path`` with every
    entry point's signature set."""
    if not os.path.exists(path):
        raise RuntimeError("%s is not built (run jagged_flashattention_amd/build.py); "
                           "there is no fallback implementation" % os.path.basename(path))
    lib = ctypes.CDLL(path)
    i32, i64 = ctypes.c_int32, ctypes.c_int64
    prob, info = ctypes.POINTER(JfaProblem), ctypes.POINTER(JfaPlanInfo)
    dplan = ctypes.POINTER(JfaDevicePlan)
    sig = {
        "jfa_abi_version": (i32, []),
        "jfa_status_string": (ctypes.c_char_p, [i32]),
        "jfa_last_hip_error": (i32, []),
        "jfa_device_workers": (i32, [i32, _I32P]),
        "jfa_offsets_from_lengths": (i32, [_P, i32, _P]),
        "jfa_plan_query": (i32, [prob, _P, _P, _P, i32, i32, info]),
        "jfa_plan_build": (i32, [prob, _P, _P, _P, i32, i32, info, _P, _P, _P, _P]),
        "jfa_fwd_workspace_bytes": (i32, [prob, info, ctypes.POINTER(i64)]),
        "jfa_fwd": (i32, [prob, info] + [_P] * 12 + [i64, _P]),
        "jfa_bwd_workspace_bytes": (i32, [prob, info, ctypes.POINTER(i64)]),
        "jfa_bwd": (i32, [prob, dplan, dplan] + [_P] * 14 + [i64, _P]),
        "jfa_bwd_stages": (i32, [i32, prob, dplan, dplan] + [_P] * 14 + [i64, _P]),
        "jfa_bwd_noalloc": (i32, [prob, dplan, dplan] + [_P] * 14),
        "jfa_bwd_dkdv_mx": (i32, [prob, dplan, _P, _P, _P, i32, _P, i32, _P, _P,
                                  ctypes.POINTER(JfaMxDkdvOperands), _P, _P, _P]),
        "jfa_mx_block_offsets": (i32, [_P, i32, _P]),
        "jfa_mx_quantize_rows": (i32, [_P, i64, i32, i32, _P, _P, _P]),
        "jfa_mx_quantize_v": (i32, [_P, _P, _P, i32, i32, i32, i32, _P, _P, _P]),
        "jfa_fwd_mx": (i32, [prob, info] + [_P] * 7 + [i32] + [_P] * 9 + [i64, _P]),
        "jfa_bwd_dq_mx": (i32, [prob, dplan, _P, _P, _P, i32, _P, _P, _P,
                                ctypes.POINTER(JfaMxBwdOperands), _P, _P, _P, _P, i64, _P]),
        "jfa_debug_tile_log": (i32, [_P, i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


@contextlib.contextmanager
def using_library(lib):
    """Route every call of this module to ``lib`` (a load_library handle,
    e.g. of the debug build) inside the block."""
    global _LIB
    old = _LIB
    _LIB = lib
    try:
        yield lib
    finally:
        _LIB = old


def _check(status: int, where: str):
    if status != JFA_OK:
        raise JfaError(status, where)


def _np_ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(_P)


def _dev_ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------- C functions

def jfa_abi_version() -> int:
    return _lib().jfa_abi_version()


def jfa_status_string(status: int) -> str:
    return _lib().jfa_status_string(status).decode()


def jfa_device_workers(device: int = 0) -> int:
    n = ctypes.c_int32(0)
    _check(_lib().jfa_device_workers(device, ctypes.byref(n)), "jfa_device_workers")
    return n.value


def jfa_offsets_from_lengths(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, dtype=np.int32)
    out = np.zeros(len(ln) + 1, dtype=np.int32)
    _check(_lib().jfa_offsets_from_lengths(_np_ptr(ln), len(ln), _np_ptr(out)),
           "jfa_offsets_from_lengths")
    return out


@dataclasses.dataclass
class Problem:
    batch: int
    num_heads: int
    head_dim: int
    broadcast_q: bool
    lq: int = 0
    causal: bool = False
    mask_q_blocks: int = 0
    mask_kv_blocks: int = 0
    softmax_scale: float = 0.0
    window_left: int = -1     # sliding window bounds (-1: none)
    window_right: int = -1

    def c(self) -> JfaProblem:
        return JfaProblem(self.batch, self.num_heads, self.head_dim, int(self.broadcast_q),
                          self.lq, int(self.causal), self.mask_q_blocks, self.mask_kv_blocks,
                          self.softmax_scale, self.window_left, self.window_right)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def jfa_plan_query(prob: Problem, q_offsets, kv_offsets, block_mask, pass_: int,
                   num_workers: int) -> JfaPlanInfo:
    info = JfaPlanInfo()
    qo, ko = _i32(q_offsets), _i32(kv_offsets)
    m = None if block_mask is None else np.ascontiguousarray(block_mask, dtype=np.uint8)
    cp = prob.c()
    _check(_lib().jfa_plan_query(ctypes.byref(cp), _np_ptr(qo), _np_ptr(ko), _np_ptr(m), pass_,
                                 num_workers, ctypes.byref(info)), "jfa_plan_query")
    return info


@dataclasses.dataclass
class HostPlan:
    info: JfaPlanInfo
    worker_ptr: np.ndarray
    tiles: np.ndarray          # [N, 4] int32 (b, h, t, work)
    sparse_ptr: Optional[np.ndarray]
    sparse_idx: Optional[np.ndarray]


def jfa_plan_build(prob: Problem, q_offsets, kv_offsets, block_mask, pass_: int,
                   num_workers: int) -> HostPlan:
    info = jfa_plan_query(prob, q_offsets, kv_offsets, block_mask, pass_, num_workers)
    qo, ko = _i32(q_offsets), _i32(kv_offsets)
    m = None if block_mask is None else np.ascontiguousarray(block_mask, dtype=np.uint8)
    wp = np.zeros(info.num_workers + 1, dtype=np.int32)
    tiles = np.zeros((info.num_tiles, 4), dtype=np.int32)
    sparse = prob.mask_q_blocks != 0
    sp = np.zeros(info.sparse_rows + 1, dtype=np.int32) if sparse else None
    si = np.zeros(max(info.sparse_nnz, 1), dtype=np.int32) if sparse else None
    info2 = JfaPlanInfo()
    cp = prob.c()
    _check(_lib().jfa_plan_build(ctypes.byref(cp), _np_ptr(qo), _np_ptr(ko), _np_ptr(m), pass_,
                                 num_workers, ctypes.byref(info2), _np_ptr(wp), _np_ptr(tiles),
                                 _np_ptr(sp), _np_ptr(si)), "jfa_plan_build")
    if sparse:
        si = si[:info2.sparse_nnz]
    return HostPlan(info2, wp, tiles, sp, si)


@dataclasses.dataclass
class DevicePlan:
    """A host plan copied to the device (torch int32 tensors)."""
    info: JfaPlanInfo
    worker_ptr: object
    tiles: object
    sparse_ptr: object
    sparse_idx: object


def to_device(plan: HostPlan, device="cuda") -> DevicePlan:
    import torch
    f = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return DevicePlan(plan.info, f(plan.worker_ptr), f(plan.tiles.reshape(-1)),
                      f(plan.sparse_ptr), f(plan.sparse_idx))


def upload_int32(arrays, device="cuda"):
    """Device copies of several host int32 arrays (None stays None) made by
    one host-to-device copy of their concatenation: views into one device
    buffer, each starting on a 16-byte boundary."""
    import torch
    parts, starts, n = [], [], 0
    for a in arrays:
        if a is None:
            starts.append(None)
            continue
        a = np.ascontiguousarray(a, dtype=np.int32).reshape(-1)
        starts.append((n, a.size))
        parts.append((n, a))
        n += -(-max(a.size, 1) // 4) * 4
    host = np.zeros(max(n, 4), dtype=np.int32)
    for off, a in parts:
        host[off:off + a.size] = a
    dev = torch.from_numpy(host).to(device)
    return [None if st is None else dev[st[0]:st[0] + st[1]] for st in starts]


def plans_to_device(plans, extra=(), device="cuda"):
    """DevicePlans of several host plans plus device copies of the ``extra``
    int32 arrays, all from one host-to-device copy."""
    arrays = []
    for p in plans:
        arrays += [p.worker_ptr, p.tiles.reshape(-1), p.sparse_ptr, p.sparse_idx]
    arrays += list(extra)
    dev = upload_int32(arrays, device)
    out = [DevicePlan(p.info, *dev[4 * i:4 * i + 4]) for i, p in enumerate(plans)]
    return out, dev[4 * len(plans):]


def jfa_fwd_workspace_bytes(prob: Problem, info: JfaPlanInfo) -> int:
    """Device scratch bytes jfa_fwd needs for a FWD plan (the counter of a
    dynamic plan)."""
    n = ctypes.c_int64(0)
    cp = prob.c()
    _check(_lib().jfa_fwd_workspace_bytes(ctypes.byref(cp), ctypes.byref(info), ctypes.byref(n)),
           "jfa_fwd_workspace_bytes")
    return n.value


def jfa_fwd(prob: Problem, plan: DevicePlan, q_offsets, kv_offsets, q, k, v, o, lse,
            workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    """Enqueue the forward on ``stream`` (default: torch's current stream).
    q_offsets / kv_offsets are device int32 tensors (q_offsets None when
    broadcast); q, k, v, o bf16 and lse fp32 device tensors (see jfa.h). A
    dynamic plan needs a zero-initialised workspace (each launch leaves it
    zero again)."""
    cp = prob.c()
    _check(_lib().jfa_fwd(ctypes.byref(cp), ctypes.byref(plan.info), _dev_ptr(plan.worker_ptr),
                          _dev_ptr(plan.tiles), _dev_ptr(plan.sparse_ptr),
                          _dev_ptr(plan.sparse_idx), _dev_ptr(q_offsets), _dev_ptr(kv_offsets),
                          _dev_ptr(q), _dev_ptr(k), _dev_ptr(v), _dev_ptr(o), _dev_ptr(lse),
                          _dev_ptr(workspace), int(workspace_bytes), _stream(stream)), "jfa_fwd")


def jfa_bwd_workspace_bytes(prob: Problem, dq_info: JfaPlanInfo) -> int:
    """Device scratch bytes jfa_bwd needs for a DQ plan."""
    n = ctypes.c_int64(0)
    cp = prob.c()
    _check(_lib().jfa_bwd_workspace_bytes(ctypes.byref(cp), ctypes.byref(dq_info),
                                          ctypes.byref(n)), "jfa_bwd_workspace_bytes")
    return n.value


def _c_plan(plan: DevicePlan) -> JfaDevicePlan:
    return JfaDevicePlan(ctypes.pointer(plan.info), _dev_ptr(plan.worker_ptr), _dev_ptr(plan.tiles),
                         _dev_ptr(plan.sparse_ptr), _dev_ptr(plan.sparse_idx))


def jfa_bwd(prob: Problem, kv_plan: DevicePlan, dq_plan: DevicePlan, q_offsets, kv_offsets, q, k,
            v, o, lse, d_o, dq, dk, dv, dq_accum, delta, workspace=None,
            workspace_bytes: int = 0, stream=None) -> None:
    """Enqueue the whole backward on ``stream``: the dQ pass (which also forms
    delta = rowsum(dO * O)), dK/dV, and with a broadcast Q the dQ reduce."""
    jfa_bwd_stages(JFA_BWD_ALL, prob, kv_plan, dq_plan, q_offsets, kv_offsets, q, k, v, o, lse,
                   d_o, dq, dk, dv, dq_accum, delta, workspace, workspace_bytes, stream)


def jfa_bwd_stages(stages: int, prob: Problem, kv_plan: DevicePlan, dq_plan: DevicePlan,
                   q_offsets, kv_offsets, q, k, v, o, lse, d_o, dq, dk, dv, dq_accum, delta,
                   workspace=None, workspace_bytes: int = 0, stream=None) -> None:
    """Enqueue the selected backward stages (JFA_BWD_* flags) on ``stream``."""
    cp = prob.c()
    kp, qp = _c_plan(kv_plan), _c_plan(dq_plan)
    _check(_lib().jfa_bwd_stages(stages, ctypes.byref(cp), ctypes.byref(kp), ctypes.byref(qp),
                                 _dev_ptr(q_offsets), _dev_ptr(kv_offsets), _dev_ptr(q),
                                 _dev_ptr(k), _dev_ptr(v), _dev_ptr(o), _dev_ptr(lse),
                                 _dev_ptr(d_o), _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dv),
                                 _dev_ptr(dq_accum), _dev_ptr(delta), _dev_ptr(workspace),
                                 int(workspace_bytes), _stream(stream)), "jfa_bwd_stages")


JFA_NOALLOC_SCRATCH_BYTES = 32 << 20


def jfa_bwd_noalloc(prob: Problem, kv_plan: DevicePlan, dq_plan: DevicePlan, q_offsets,
                    kv_offsets, q, k, v, o, lse, d_o, dq, dk, dv, dq_accum, delta,
                    stream=None) -> None:
    """The whole backward like jfa_bwd, with the library's own scratch area
    in place of a workspace (nothing is allocated by the call)."""
    cp = prob.c()
    kp, qp = _c_plan(kv_plan), _c_plan(dq_plan)
    _check(_lib().jfa_bwd_noalloc(ctypes.byref(cp), ctypes.byref(kp), ctypes.byref(qp),
                                  _dev_ptr(q_offsets), _dev_ptr(kv_offsets), _dev_ptr(q),
                                  _dev_ptr(k), _dev_ptr(v), _dev_ptr(o), _dev_ptr(lse),
                                  _dev_ptr(d_o), _dev_ptr(dq), _dev_ptr(dk), _dev_ptr(dv),
                                  _dev_ptr(dq_accum), _dev_ptr(delta), _stream(stream)),
           "jfa_bwd_noalloc")


# ------------------------------------------------------------------ MXFP8

def jfa_bwd_dq_mx(prob: Problem, dq_plan: DevicePlan, q_offsets, kv_offsets, key_block_offsets,
                  num_key_blocks, o, lse, d_o, ops: dict, dq, dq_accum, delta, workspace=None,
                  workspace_bytes: int = 0, stream=None) -> None:
    """Enqueue the MXFP8 dQ pass (operands: qc/qs, kc/ks, vdc/vds, doc/dos,
    kkc/kks device tensors as produced by JaggedAttention.quantize_mx_bwd)."""
    cp = prob.c()
    qp = _c_plan(dq_plan)
    mo = JfaMxBwdOperands(*[_dev_ptr(ops[n]) for n in (
        "qc", "qs", "kc", "ks", "vdc", "vds", "doc", "dos", "kkc", "kks")])
    _check(_lib().jfa_bwd_dq_mx(ctypes.byref(cp), ctypes.byref(qp), _dev_ptr(q_offsets),
                                _dev_ptr(kv_offsets), _dev_ptr(key_block_offsets),
                                int(num_key_blocks), _dev_ptr(o), _dev_ptr(lse), _dev_ptr(d_o),
                                ctypes.byref(mo), _dev_ptr(dq), _dev_ptr(dq_accum), _dev_ptr(delta),
                                _dev_ptr(workspace), int(workspace_bytes), _stream(stream)),
           "jfa_bwd_dq_mx")


def jfa_bwd_dkdv_mx(prob: Problem, kv_plan: DevicePlan, q_offsets, kv_offsets, q_row_block_offsets,
                    num_q_row_blocks, do_row_block_offsets, num_do_row_blocks, lse, delta,
                    ops: dict, dk, dv, stream=None) -> None:
    """Enqueue the MXFP8 dK/dV pass (operands: qc/qs, kc/ks, vdc/vds, doc/dos
    along d, qrc/qrs, dorc/dors along rows, as produced by
    JaggedAttention.quantize_mx_dkdv)."""
    cp = prob.c()
    kp = _c_plan(kv_plan)
    mo = JfaMxDkdvOperands(*[_dev_ptr(ops[n]) for n in (
        "qc", "qs", "kc", "ks", "vdc", "vds", "doc", "dos", "qrc", "qrs", "dorc", "dors")])
    _check(_lib().jfa_bwd_dkdv_mx(ctypes.byref(cp), ctypes.byref(kp), _dev_ptr(q_offsets),
                                  _dev_ptr(kv_offsets), _dev_ptr(q_row_block_offsets),
                                  int(num_q_row_blocks), _dev_ptr(do_row_block_offsets),
                                  int(num_do_row_blocks), _dev_ptr(lse), _dev_ptr(delta),
                                  ctypes.byref(mo), _dev_ptr(dk), _dev_ptr(dv), _stream(stream)),
           "jfa_bwd_dkdv_mx")


def jfa_debug_tile_log(log, records_per_worker: int) -> None:
    """Set (a device int32 tensor) or clear (None) the executed-tile log of
    the debug build; the product library raises JfaError (unsupported)."""
    _check(_lib().jfa_debug_tile_log(_dev_ptr(log), int(records_per_worker)), "jfa_debug_tile_log")


def read_tile_log(log, num_workers: int, records_per_worker: int):
    """The records of an executed-tile log as a list per worker of int32
    [n, 8] arrays (pass, worker, b, h, t, work, blocks, flags), plus the
    number of tiles each worker took."""
    a = log.cpu().numpy().reshape(-1)[:num_workers * (8 + 8 * records_per_worker)]
    a = a.reshape(num_workers, 8 + 8 * records_per_worker)
    counts = a[:, 0].copy()
    recs = [a[w, 8:].reshape(records_per_worker, 8)[:min(int(counts[w]), records_per_worker)]
            for w in range(num_workers)]
    return recs, counts


def jfa_mx_block_offsets(kv_offsets) -> np.ndarray:
    """First V scale block of each sequence (prefix sums of ceil(L_b / 32))."""
    ko = _i32(kv_offsets)
    out = np.zeros(len(ko), dtype=np.int32)
    _check(_lib().jfa_mx_block_offsets(_np_ptr(ko), len(ko) - 1, _np_ptr(out)),
           "jfa_mx_block_offsets")
    return out


def jfa_mx_quantize_rows(src, codes, scales, stream=None) -> None:
    """bf16 [rows, H, D] -> E4M3 codes [rows, H, D] (uint8) and scales [H, rows, D/32]."""
    rows, H, D = src.shape
    _check(_lib().jfa_mx_quantize_rows(_dev_ptr(src), rows, H, D, _dev_ptr(codes), _dev_ptr(scales),
                                       _stream(stream)), "jfa_mx_quantize_rows")


def jfa_mx_quantize_v(v, kv_offsets, block_offsets, num_blocks, codes, scales, stream=None) -> None:
    """bf16 V [T_k, H, D] -> codes [T_k, H, D] and scales [H, NB, D] (device offsets)."""
    _, H, D = v.shape
    _check(_lib().jfa_mx_quantize_v(_dev_ptr(v), _dev_ptr(kv_offsets), _dev_ptr(block_offsets),
                                    kv_offsets.numel() - 1, H, D, int(num_blocks), _dev_ptr(codes),
                                    _dev_ptr(scales), _stream(stream)), "jfa_mx_quantize_v")


def jfa_fwd_mx(prob: Problem, plan: DevicePlan, q_offsets, kv_offsets, block_offsets, num_blocks,
               qc, qs, kc, ks, vc, vs, o, lse, workspace=None, workspace_bytes: int = 0,
               stream=None) -> None:
    """Enqueue the MXFP8 forward (codes / scales as produced by the quantizers)."""
    cp = prob.c()
    _check(_lib().jfa_fwd_mx(ctypes.byref(cp), ctypes.byref(plan.info), _dev_ptr(plan.worker_ptr),
                             _dev_ptr(plan.tiles), _dev_ptr(plan.sparse_ptr),
                             _dev_ptr(plan.sparse_idx), _dev_ptr(q_offsets), _dev_ptr(kv_offsets),
                             _dev_ptr(block_offsets), int(num_blocks), _dev_ptr(qc), _dev_ptr(qs),
                             _dev_ptr(kc), _dev_ptr(ks), _dev_ptr(vc), _dev_ptr(vs), _dev_ptr(o),
                             _dev_ptr(lse), _dev_ptr(workspace), int(workspace_bytes),
                             _stream(stream)), "jfa_fwd_mx")


# ------------------------------------------------------- convenience wrappers

def default_workers(device: int = 0, per_cu: int = 1) -> int:
    return jfa_device_workers(device) * per_cu


class JaggedAttention:
    """Plans once for fixed offsets and runs forward/backward on torch tensors.

    q: [lq,H,D] (broadcast) or [T_q,H,D]; k, v: [T_k,H,D]; bf16 on the GPU.
    Host copies of the offsets are needed for planning (the planner runs on
    the CPU); device copies are made here.
    """

    def __init__(self, prob: Problem, kv_offsets, q_offsets=None, block_mask=None,
                 fwd_workers: Optional[int] = None, bwd_workers: Optional[int] = None,
                 dq_workers: Optional[int] = None, fwd_dynamic: Optional[bool] = None,
                 natural_plans: bool = False, device="cuda"):
        """fwd_dynamic: True claims forward tiles at run time, False deals
        them statically, None (default) claims them only when there are more
        tiles than workers (with no more, each worker has at most one tile
        and the claims would only cost their atomics). natural_plans: the
        unsorted round-robin plans (the ablation baseline) for all three
        passes; the forward is then static."""
        import torch
        self.prob = prob
        self.device = device
        cus = jfa_device_workers(torch.device(device).index or 0)
        nat = JFA_PLAN_NATURAL if natural_plans else 0
        if fwd_dynamic is None and not natural_plans:
            qi = jfa_plan_query(prob, q_offsets, kv_offsets, block_mask, JFA_PASS_FWD,
                                fwd_workers or cus)
            fwd_dynamic = qi.num_tiles > qi.num_workers
        fwd_pass = JFA_PASS_FWD | (JFA_PLAN_DYNAMIC if fwd_dynamic and not natural_plans else nat)
        t0 = time.perf_counter()
        self.fwd_plan_host = jfa_plan_build(prob, q_offsets, kv_offsets, block_mask,
                                            fwd_pass, fwd_workers or cus)
        self.bwd_plan_host = jfa_plan_build(prob, q_offsets, kv_offsets, block_mask,
                                            JFA_PASS_BWD | nat, bwd_workers or cus)
        self.dq_plan_host = jfa_plan_build(prob, q_offsets, kv_offsets, block_mask,
                                           JFA_PASS_DQ | nat, dq_workers or cus)
        t1 = time.perf_counter()
        # the three plans and the offsets reach the device in one copy
        (self.fwd_plan, self.bwd_plan, self.dq_plan), (self.kv_offsets, self.q_offsets) = \
            plans_to_device([self.fwd_plan_host, self.bwd_plan_host, self.dq_plan_host],
                            [kv_offsets, q_offsets], device)
        if torch.device(device).type == "cuda":
            torch.cuda.synchronize(device)
        t2 = time.perf_counter()
        self.planner_ms = (t1 - t0) * 1e3     # the host planner, three passes
        self.upload_ms = (t2 - t1) * 1e3      # packing and the host-to-device copy
        self.total_q = self.fwd_plan.info.total_q
        self.total_kv = self.fwd_plan.info.total_kv
        self.ws_bytes = jfa_bwd_workspace_bytes(prob, self.dq_plan.info)
        self.workspace = (torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
                          if self.ws_bytes else None)
        # the dynamic forward's tile counter starts at zero and every launch
        # leaves it zero
        self.fwd_ws_bytes = jfa_fwd_workspace_bytes(prob, self.fwd_plan.info)
        self.fwd_workspace = (torch.zeros(self.fwd_ws_bytes, dtype=torch.uint8, device=device)
                              if self.fwd_ws_bytes else None)

    def _expect(self, **named):
        """Raise ValueError unless every given tensor is a contiguous CUDA
        tensor of its expected shape and dtype (the kernels take raw pointers:
        a mismatch would read or write out of bounds)."""
        import torch
        H, D = self.prob.num_heads, self.prob.head_dim
        q_rows = self.prob.lq if self.prob.broadcast_q else self.total_q
        bf, f32 = torch.bfloat16, torch.float32
        want = {"q": ((q_rows, H, D), bf), "k": ((self.total_kv, H, D), bf),
                "v": ((self.total_kv, H, D), bf), "o": ((self.total_q, H, D), bf),
                "d_o": ((self.total_q, H, D), bf), "lse": ((H, self.total_q), f32),
                "dq": ((q_rows, H, D), bf), "dk": ((self.total_kv, H, D), bf),
                "dv": ((self.total_kv, H, D), bf), "dq_accum": ((q_rows, H, D), f32),
                "delta": ((H, self.total_q), f32)}
        for name, t in named.items():
            shape, dtype = want[name]
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise ValueError("%s: a CUDA tensor is needed" % name)
            if t.dtype != dtype or tuple(t.shape) != shape or not t.is_contiguous():
                raise ValueError("%s: expected a contiguous %s tensor of shape %s, got %s %s%s"
                                 % (name, dtype, shape, t.dtype, tuple(t.shape),
                                    "" if t.is_contiguous() else " (not contiguous)"))

    def forward(self, q, k, v, o=None, lse=None):
        import torch
        H, D = self.prob.num_heads, self.prob.head_dim
        if o is None:
            o = torch.empty((self.total_q, H, D), dtype=torch.bfloat16, device=self.device)
        if lse is None:
            lse = torch.empty((H, self.total_q), dtype=torch.float32, device=self.device)
        self._expect(q=q, k=k, v=v, o=o, lse=lse)
        jfa_fwd(self.prob, self.fwd_plan, self.q_offsets, self.kv_offsets, q, k, v, o, lse,
                self.fwd_workspace, self.fwd_ws_bytes)
        return o, lse

    def quantize_mx(self, q, k, v):
        """MXFP8 encodings of bf16 q, k, v (device tensors) for forward_mx."""
        import torch
        if not hasattr(self, "v_block_offsets"):
            boff = jfa_mx_block_offsets(self.kv_offsets.cpu().numpy())
            self.v_num_blocks = int(boff[-1])
            self.v_block_offsets = torch.from_numpy(boff).to(self.device)
        self._expect(q=q, k=k, v=v)
        H, D = self.prob.num_heads, self.prob.head_dim
        u8 = dict(dtype=torch.uint8, device=self.device)
        mxq = dict(qc=torch.empty(q.shape, **u8), qs=torch.empty((H, q.shape[0], D // 32), **u8),
                   kc=torch.empty(k.shape, **u8), ks=torch.empty((H, k.shape[0], D // 32), **u8),
                   vc=torch.empty(v.shape, **u8),
                   vs=torch.empty((H, max(self.v_num_blocks, 1), D), **u8))
        jfa_mx_quantize_rows(q, mxq["qc"], mxq["qs"])
        jfa_mx_quantize_rows(k, mxq["kc"], mxq["ks"])
        jfa_mx_quantize_v(v, self.kv_offsets, self.v_block_offsets, self.v_num_blocks, mxq["vc"],
                          mxq["vs"])
        return mxq

    def forward_mx(self, mxq, o=None, lse=None):
        """The MXFP8 forward on encodings from quantize_mx."""
        import torch
        H, D = self.prob.num_heads, self.prob.head_dim
        if o is None:
            o = torch.empty((self.total_q, H, D), dtype=torch.bfloat16, device=self.device)
        if lse is None:
            lse = torch.empty((H, self.total_q), dtype=torch.float32, device=self.device)
        self._expect(o=o, lse=lse)
        jfa_fwd_mx(self.prob, self.fwd_plan, self.q_offsets, self.kv_offsets, self.v_block_offsets,
                   self.v_num_blocks, mxq["qc"], mxq["qs"], mxq["kc"], mxq["ks"], mxq["vc"],
                   mxq["vs"], o, lse, self.fwd_workspace, self.fwd_ws_bytes)
        return o, lse

    def quantize_mx_bwd(self, mxq, k, v, d_o):
        """The further MXFP8 encodings of the MXFP8 dQ pass: V and dO along d,
        K along the keys of its sequence (added to quantize_mx's dict)."""
        import torch
        self._expect(k=k, v=v, d_o=d_o)
        H, D = self.prob.num_heads, self.prob.head_dim
        u8 = dict(dtype=torch.uint8, device=self.device)
        ops = dict(mxq)
        ops.update(vdc=torch.empty(v.shape, **u8), vds=torch.empty((H, v.shape[0], D // 32), **u8),
                   doc=torch.empty(d_o.shape, **u8),
                   dos=torch.empty((H, d_o.shape[0], D // 32), **u8),
                   kkc=torch.empty(k.shape, **u8),
                   kks=torch.empty((H, max(self.v_num_blocks, 1), D), **u8))
        jfa_mx_quantize_rows(v, ops["vdc"], ops["vds"])
        jfa_mx_quantize_rows(d_o, ops["doc"], ops["dos"])
        jfa_mx_quantize_v(k, self.kv_offsets, self.v_block_offsets, self.v_num_blocks, ops["kkc"],
                          ops["kks"])
        return ops

    def quantize_mx_dkdv(self, ops, q, d_o):
        """The further MXFP8 encodings of the MXFP8 dK/dV pass: Q and dO along
        their rows, in 32-row blocks of one sequence (added to
        quantize_mx_bwd's dict)."""
        import torch
        self._expect(q=q, d_o=d_o)
        H, D = self.prob.num_heads, self.prob.head_dim
        if not hasattr(self, "q_row_boff"):
            B = self.kv_offsets.numel() - 1
            if self.prob.broadcast_q:
                q_rows_off = np.array([0, self.prob.lq], dtype=np.int32)
                do_rows_off = (np.arange(B + 1) * self.prob.lq).astype(np.int32)
            else:
                q_rows_off = do_rows_off = self.q_offsets.cpu().numpy()
            qb, db = jfa_mx_block_offsets(q_rows_off), jfa_mx_block_offsets(do_rows_off)
            self.q_row_nb, self.do_row_nb = int(qb[-1]), int(db[-1])
            (self.q_rows_off, self.do_rows_off, self.q_row_boff, self.do_row_boff) = upload_int32(
                [q_rows_off, do_rows_off, qb, db], self.device)
        u8 = dict(dtype=torch.uint8, device=self.device)
        out = dict(ops)
        out.update(qrc=torch.empty(q.shape, **u8), qrs=torch.empty((H, max(self.q_row_nb, 1), D), **u8),
                   dorc=torch.empty(d_o.shape, **u8),
                   dors=torch.empty((H, max(self.do_row_nb, 1), D), **u8))
        jfa_mx_quantize_v(q, self.q_rows_off, self.q_row_boff, self.q_row_nb, out["qrc"], out["qrs"])
        jfa_mx_quantize_v(d_o, self.do_rows_off, self.do_row_boff, self.do_row_nb, out["dorc"],
                          out["dors"])
        return out

    def backward_mx(self, q, k, v, o, lse, d_o, ops, out=None, stages=JFA_BWD_ALL):
        """Backward with the MXFP8 dQ pass (in place of JFA_BWD_DQ) and, when
        ops holds the along-rows encodings of quantize_mx_dkdv, the MXFP8
        dK/dV pass (in place of JFA_BWD_DKDV); the other selected stages are
        the bf16 ones."""
        import torch
        if out is None:
            out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                       dq_accum=torch.empty(q.shape, dtype=torch.float32, device=self.device),
                       delta=torch.empty((self.prob.num_heads, self.total_q), dtype=torch.float32,
                                         device=self.device))
        # in the order of jfa_bwd_stages: delta alone, dQ, dK/dV, dQ reduce
        if stages & JFA_BWD_PREPROCESS:
            self.backward(q, k, v, o, lse, d_o, out, stages=JFA_BWD_PREPROCESS)
        if stages & JFA_BWD_DQ:
            self._expect(o=o, lse=lse, d_o=d_o, dq=out["dq"], dq_accum=out["dq_accum"],
                         delta=out["delta"])
            jfa_bwd_dq_mx(self.prob, self.dq_plan, self.q_offsets, self.kv_offsets,
                          self.v_block_offsets, self.v_num_blocks, o, lse, d_o, ops, out["dq"],
                          out["dq_accum"], out["delta"], self.workspace, self.ws_bytes)
        if stages & JFA_BWD_DKDV:
            if "qrc" in ops:
                self._expect(lse=lse, delta=out["delta"], dk=out["dk"], dv=out["dv"])
                jfa_bwd_dkdv_mx(self.prob, self.bwd_plan, self.q_offsets, self.kv_offsets,
                                self.q_row_boff, self.q_row_nb, self.do_row_boff, self.do_row_nb,
                                lse, out["delta"], ops, out["dk"], out["dv"])
            else:
                self.backward(q, k, v, o, lse, d_o, out, stages=JFA_BWD_DKDV)
        # (the MXFP8 dQ pass writes per-worker partials: the fixed-order reduce)
        if stages & JFA_BWD_DQ_REDUCE:
            self.backward(q, k, v, o, lse, d_o, out, stages=JFA_BWD_DQ_REDUCE)
        return out

    def backward(self, q, k, v, o, lse, d_o, out=None, stages=JFA_BWD_ALL):
        import torch
        if out is None:
            out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                       dq_accum=torch.empty(q.shape, dtype=torch.float32, device=self.device),
                       delta=torch.empty((self.prob.num_heads, self.total_q), dtype=torch.float32,
                                         device=self.device))
        self._expect(q=q, k=k, v=v, o=o, lse=lse, d_o=d_o,
                     **{n: out[n] for n in ("dq", "dk", "dv", "dq_accum", "delta")})
        jfa_bwd_stages(stages, self.prob, self.bwd_plan, self.dq_plan, self.q_offsets,
                       self.kv_offsets, q, k, v, o, lse, d_o, out["dq"], out["dk"], out["dv"],
                       out["dq_accum"], out["delta"], self.workspace, self.ws_bytes)
        return out
