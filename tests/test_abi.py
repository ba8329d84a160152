"""The C ABI library on the CPU: it loads, exports every symbol the header
declares, and its host-side logic (offsets, planner, argument validation)
behaves as documented. No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

import jagged_flashattention_amd as J
import workloads as W
from oracle import planner as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "jfa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(jfa_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(J.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(J.EXPORTS)


def test_version_and_status_strings():
    assert J.jfa_abi_version() == 10
    for st in range(-7, 1):
        assert J.jfa_status_string(st) not in ("", "unknown status")
    assert J.jfa_status_string(-99) == "unknown status"


def test_offsets_from_lengths_matches_oracle():
    x = W.make_inputs(2)
    assert np.array_equal(J.jfa_offsets_from_lengths(x.lengths),
                          OP.offsets_from_lengths(x.lengths))
    assert list(J.jfa_offsets_from_lengths([])) == [0]
    with pytest.raises(J.JfaError) as e:
        J.jfa_offsets_from_lengths([3, -1])
    assert e.value.status == J.JFA_ERR_BAD_OFFSETS
    with pytest.raises(J.JfaError):
        J.jfa_offsets_from_lengths([2**30, 2**30, 2**30])


def _prob(**kw):
    base = dict(batch=2, num_heads=1, head_dim=64, broadcast_q=True, lq=8, softmax_scale=0.125)
    base.update(kw)
    return J.Problem(**base)


@pytest.mark.parametrize("kw,qoff,kvoff,mask,status", [
    (dict(head_dim=96), None, [0, 3, 5], None, J.JFA_ERR_UNSUPPORTED),
    (dict(num_heads=32769), None, [0, 3, 5], None, J.JFA_ERR_UNSUPPORTED),
    (dict(causal=True), None, [0, 3, 5], None, J.JFA_ERR_UNSUPPORTED),
    (dict(), None, [1, 3, 5], None, J.JFA_ERR_BAD_OFFSETS),
    (dict(), None, [0, 3, 2], None, J.JFA_ERR_BAD_OFFSETS),
    (dict(broadcast_q=False, causal=True), [0, 3, 6], [0, 3, 5], None, J.JFA_ERR_UNSUPPORTED),
    (dict(broadcast_q=False), None, [0, 3, 5], None, J.JFA_ERR_INVALID_ARG),
    (dict(num_heads=0), None, [0, 3, 5], None, J.JFA_ERR_INVALID_ARG),
    (dict(batch=-1), None, [0], None, J.JFA_ERR_INVALID_ARG),
    (dict(mask_q_blocks=1, mask_kv_blocks=1), None, [0, 3, 5], None, J.JFA_ERR_BAD_MASK),
    (dict(mask_q_blocks=1, mask_kv_blocks=1), None, [0, 300, 305],
     np.ones((2, 1, 1), np.uint8), J.JFA_ERR_BAD_MASK),
    (dict(mask_q_blocks=1, mask_kv_blocks=0), None, [0, 3, 5], None, J.JFA_ERR_BAD_MASK),
    (dict(broadcast_q=False, causal=True, mask_q_blocks=1, mask_kv_blocks=1), [0, 3, 5],
     [0, 3, 5], np.ones((2, 1, 1), np.uint8), J.JFA_ERR_UNSUPPORTED),
    (dict(softmax_scale=float("nan")), None, [0, 3, 5], None, J.JFA_ERR_INVALID_ARG),
    (dict(softmax_scale=-0.5), None, [0, 3, 5], None, J.JFA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), None, [0, 3, 5], None, J.JFA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("inf")), None, [0, 3, 5], None, J.JFA_ERR_INVALID_ARG),
    (dict(window_left=4), None, [0, 3, 5], None, J.JFA_ERR_UNSUPPORTED),       # window, broadcast
    (dict(broadcast_q=False, window_right=-2), [0, 3, 5], [0, 3, 5], None, J.JFA_ERR_INVALID_ARG),
    (dict(broadcast_q=False, window_left=3), [0, 3, 6], [0, 3, 5], None, J.JFA_ERR_UNSUPPORTED),
    (dict(broadcast_q=False, window_left=3, mask_q_blocks=1, mask_kv_blocks=1), [0, 3, 5],
     [0, 3, 5], np.ones((2, 1, 1), np.uint8), J.JFA_ERR_UNSUPPORTED),
])
def test_planner_rejects_bad_problems(kw, qoff, kvoff, mask, status):
    with pytest.raises(J.JfaError) as e:
        J.jfa_plan_build(_prob(**kw), qoff, kvoff, mask, J.JFA_PASS_FWD, 4)
    assert e.value.status == status


def test_planner_rejects_zero_workers_and_bad_pass():
    with pytest.raises(J.JfaError) as e:
        J.jfa_plan_query(_prob(), None, [0, 3, 5], None, J.JFA_PASS_FWD, 0)
    assert e.value.status == J.JFA_ERR_INVALID_ARG
    with pytest.raises(J.JfaError) as e:
        J.jfa_plan_query(_prob(), None, [0, 3, 5], None, 7, 4)
    assert e.value.status == J.JFA_ERR_INVALID_ARG


def test_empty_batch_plan():
    p = J.jfa_plan_build(_prob(batch=0), None, [0], None, J.JFA_PASS_FWD, 8)
    assert p.info.num_tiles == 0 and list(p.worker_ptr) == [0] * 9


class _FakeTensor:
    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _call_fwd(prob, info, ws_bytes=0, **over):
    t = _FakeTensor(0x1000)
    args = dict(worker_ptr=t, tiles=t, sparse_ptr=None, sparse_idx=None, q_off=None, kv_off=t,
                q=t, k=t, v=t, o=t, lse=t, ws=None)
    args.update(over)
    cp = prob.c()
    f = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    return J._lib().jfa_fwd(ctypes.byref(cp), ctypes.byref(info), f(args["worker_ptr"]),
                            f(args["tiles"]), f(args["sparse_ptr"]), f(args["sparse_idx"]),
                            f(args["q_off"]), f(args["kv_off"]), f(args["q"]), f(args["k"]),
                            f(args["v"]), f(args["o"]), f(args["lse"]), f(args["ws"]), ws_bytes,
                            None)


def test_fwd_validation_returns_before_launch():
    prob = _prob()
    fwd = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_FWD, 4)
    bwd = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_BWD, 4)
    assert _call_fwd(prob, bwd.info) == J.JFA_ERR_PLAN_MISMATCH          # wrong pass
    assert _call_fwd(prob, fwd.info, q=_FakeTensor(0x1008)) == J.JFA_ERR_INVALID_ARG  # misaligned
    assert _call_fwd(prob, fwd.info, o=None) == J.JFA_ERR_INVALID_ARG
    assert _call_fwd(prob, fwd.info, tiles=None) == J.JFA_ERR_INVALID_ARG
    assert _call_fwd(_prob(lq=9), fwd.info) == J.JFA_ERR_PLAN_MISMATCH   # T_q != B*lq
    assert _call_fwd(_prob(head_dim=32), fwd.info) == J.JFA_ERR_UNSUPPORTED
    sp = _prob(mask_q_blocks=1, mask_kv_blocks=1)
    assert _call_fwd(sp, fwd.info) == J.JFA_ERR_PLAN_MISMATCH            # dense plan, sparse prob
    # an empty problem is a no-op that launches nothing
    e = J.jfa_plan_build(_prob(batch=0), None, [0], None, J.JFA_PASS_FWD, 4)
    assert _call_fwd(_prob(batch=0), e.info, worker_ptr=None, tiles=None, q=None, k=None, v=None,
                     o=None, lse=None, kv_off=None) == J.JFA_OK


def test_fwd_workspace_query_and_validation():
    prob = _prob()
    static = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_FWD, 4)
    dyn = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_FWD | J.JFA_PLAN_DYNAMIC, 4)
    assert J.jfa_fwd_workspace_bytes(prob, static.info) == 0
    need = J.jfa_fwd_workspace_bytes(prob, dyn.info)
    assert need == 256
    assert _call_fwd(prob, dyn.info) == J.JFA_ERR_WORKSPACE                    # no counter
    assert _call_fwd(prob, dyn.info, need - 4, ws=_FakeTensor(0x2000)) == J.JFA_ERR_WORKSPACE
    assert _call_fwd(prob, dyn.info, need, ws=_FakeTensor(0x2008)) == J.JFA_ERR_WORKSPACE
    bwd = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_BWD, 4)
    with pytest.raises(J.JfaError) as e:
        J.jfa_fwd_workspace_bytes(prob, bwd.info)
    assert e.value.status == J.JFA_ERR_PLAN_MISMATCH


def test_bwd_workspace_query():
    prob = _prob()
    dq = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_DQ, 4)
    # broadcast Q: one fp32 [256][D] partial per dQ worker
    assert J.jfa_bwd_workspace_bytes(prob, dq.info) == dq.info.num_workers * 256 * prob.head_dim * 4
    per_seq = _prob(broadcast_q=False, lq=0)
    dq2 = J.jfa_plan_build(per_seq, [0, 2, 4], [0, 3, 5], None, J.JFA_PASS_DQ, 4)
    assert J.jfa_bwd_workspace_bytes(per_seq, dq2.info) == 0
    for p in (J.JFA_PASS_FWD, J.JFA_PASS_BWD):
        other = J.jfa_plan_build(prob, None, [0, 3, 5], None, p, 4)
        with pytest.raises(J.JfaError) as e:
            J.jfa_bwd_workspace_bytes(prob, other.info)
        assert e.value.status == J.JFA_ERR_PLAN_MISMATCH


def _call_bwd(prob, kv, dq, ws_bytes, **over):
    t = _FakeTensor(0x1000)
    f = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    args = dict(q=t, k=t, v=t, o=t, lse=t, d_o=t, dq=t, dk=t, dv=t, dq_accum=t, delta=t, ws=t)
    args.update(over)
    plans = [J.JfaDevicePlan(ctypes.pointer(p.info), 0x1000, 0x1000, None, None) for p in (kv, dq)]
    cp = prob.c()
    return J._lib().jfa_bwd(ctypes.byref(cp), ctypes.byref(plans[0]), ctypes.byref(plans[1]),
                            None, ctypes.c_void_p(0x1000), *[f(args[k]) for k in
                            ("q", "k", "v", "o", "lse", "d_o", "dq", "dk", "dv", "dq_accum",
                             "delta", "ws")], ws_bytes, None)


def test_bwd_validation_returns_before_launch():
    prob = _prob()
    kv = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_BWD, 4)
    dq = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_DQ, 4)
    fwd = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_FWD, 4)
    need = J.jfa_bwd_workspace_bytes(prob, dq.info)
    assert _call_bwd(prob, dq, dq, need) == J.JFA_ERR_PLAN_MISMATCH      # KV plan of the wrong pass
    assert _call_bwd(prob, kv, fwd, need) == J.JFA_ERR_PLAN_MISMATCH     # dQ plan of the wrong pass
    assert _call_bwd(prob, kv, dq, need - 1) == J.JFA_ERR_WORKSPACE
    assert _call_bwd(prob, kv, dq, need, ws=None) == J.JFA_ERR_WORKSPACE
    assert _call_bwd(prob, kv, dq, need, dk=_FakeTensor(0x1004)) == J.JFA_ERR_INVALID_ARG
    assert _call_bwd(_prob(lq=9), kv, dq, need) == J.JFA_ERR_PLAN_MISMATCH


def _call_dq_mx(prob, dq_plan, ws_bytes, nkb=1, ops=True, **over):
    t = _FakeTensor(0x1000)
    f = lambda x: None if x is None else ctypes.c_void_p(x.data_ptr())
    args = dict(o=t, lse=t, d_o=t, dq=t, dq_accum=t, delta=t, ws=t, kbo=t)
    args.update(over)
    sc = dict(q_scales=0x1000, k_scales=0x1000, v_scales=0x1000, do_scales=0x1000, kk_scales=0x1000)
    sc.update({k: v for k, v in over.items() if k.endswith("_scales")})
    mx = J.JfaMxBwdOperands(q_codes=0x1000, k_codes=0x1000, v_codes=0x1000, do_codes=0x1000,
                            kk_codes=0x1000, **sc)
    plan = J.JfaDevicePlan(ctypes.pointer(dq_plan.info), 0x1000, 0x1000, None, None)
    cp = prob.c()
    return J._lib().jfa_bwd_dq_mx(ctypes.byref(cp), ctypes.byref(plan), None,
                                  ctypes.c_void_p(0x1000), f(args["kbo"]), nkb, f(args["o"]),
                                  f(args["lse"]), f(args["d_o"]),
                                  ctypes.byref(mx) if ops else None, f(args["dq"]),
                                  f(args["dq_accum"]), f(args["delta"]), f(args["ws"]), ws_bytes,
                                  None)


def test_bwd_dq_mx_validation_returns_before_launch():
    prob = _prob(head_dim=128)
    dq = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_DQ, 4)
    kv = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_BWD, 4)
    need = J.jfa_bwd_workspace_bytes(prob, dq.info)
    # two sequences of 3 and 2 keys: one 32-key block each
    assert _call_dq_mx(prob, kv, need, nkb=2) == J.JFA_ERR_PLAN_MISMATCH      # not a DQ plan
    assert _call_dq_mx(prob, dq, need - 1, nkb=2) == J.JFA_ERR_WORKSPACE
    assert _call_dq_mx(prob, dq, need, nkb=2, ws=None) == J.JFA_ERR_WORKSPACE
    assert _call_dq_mx(prob, dq, need, nkb=2, ops=False) == J.JFA_ERR_INVALID_ARG
    assert _call_dq_mx(prob, dq, need, nkb=0) == J.JFA_ERR_INVALID_ARG      # too few key blocks
    assert _call_dq_mx(prob, dq, need, nkb=2, kbo=None) == J.JFA_ERR_INVALID_ARG
    assert _call_dq_mx(prob, dq, need, nkb=2, kk_scales=0x1002) == J.JFA_ERR_INVALID_ARG  # unaligned
    assert _call_dq_mx(prob, dq, need, nkb=2, d_o=_FakeTensor(0x1004)) == J.JFA_ERR_INVALID_ARG
    assert _call_dq_mx(prob, dq, need, nkb=2, delta=None) == J.JFA_ERR_INVALID_ARG
    p64 = _prob(head_dim=64)
    dq64 = J.jfa_plan_build(p64, None, [0, 3, 5], None, J.JFA_PASS_DQ, 4)
    assert _call_dq_mx(p64, dq64, J.jfa_bwd_workspace_bytes(p64, dq64.info), nkb=2) == J.JFA_ERR_UNSUPPORTED


def test_bwd_dq_mx_accepts_a_problem_without_query_rows():
    """Per-sequence Q whose sequences all have 0 rows: O, dO, LSE, delta and
    dQ are empty (null pointers, as empty tensors give) and the call does
    nothing (it used to refuse the null LSE)."""
    prob = _prob(head_dim=128, broadcast_q=False, lq=0)
    dq = J.jfa_plan_build(prob, [0, 0, 0], [0, 3, 5], None, J.JFA_PASS_DQ, 4)
    assert dq.info.total_q == 0 and dq.info.num_tiles == 0
    need = J.jfa_bwd_workspace_bytes(prob, dq.info)
    assert _call_dq_mx(prob, dq, need, nkb=2, o=None, lse=None, d_o=None, dq=None, dq_accum=None,
                       delta=None) == J.JFA_OK


def test_jagged_attention_rejects_mismatched_tensors(monkeypatch):
    """The high-level wrapper checks every tensor before anything reaches the
    kernels (raw pointers: a wrong shape, dtype or layout would be read out of
    bounds). Runs without a GPU: the checks come first, so CPU tensors are
    refused as well."""
    torch = pytest.importorskip("torch")
    prob = _prob(head_dim=64, lq=8)
    att = J.JaggedAttention.__new__(J.JaggedAttention)
    att.prob, att.total_q, att.total_kv = prob, 16, 5
    good = dict(q=(8, 1, 64), k=(5, 1, 64), v=(5, 1, 64), o=(16, 1, 64), d_o=(16, 1, 64))

    class T:   # stands in for a CUDA tensor (shape, dtype, layout only)
        def __init__(self, shape, dtype=torch.bfloat16, contiguous=True):
            self.shape, self.dtype, self._c = shape, dtype, contiguous
            self.is_cuda = True

        def is_contiguous(self):
            return self._c
    monkeypatch.setattr(torch, "Tensor", T)
    att._expect(**{n: T(s) for n, s in good.items()}, lse=T((1, 16), torch.float32))
    for bad in (dict(q=T((16, 1, 64))),                       # per-sequence shape, broadcast problem
                dict(k=T((5, 1, 64), torch.float16)),          # wrong dtype
                dict(v=T((5, 1, 64), contiguous=False)),       # a view
                dict(lse=T((1, 16))),                          # bf16 LSE
                dict(delta=T((16, 1), torch.float32))):        # transposed
        with pytest.raises(ValueError):
            att._expect(**bad)
    class Host(T):
        def __init__(self, shape):
            super().__init__(shape)
            self.is_cuda = False
    with pytest.raises(ValueError):
        att._expect(o=Host((16, 1, 64)))


def test_bench_refuses_more_than_one_gpu():
    """The benchmark runs on one GPU: asked for more it says so and exits
    with status 2 before touching a device."""
    import subprocess
    import sys
    root = __import__("os").path.dirname(__import__("os").path.dirname(__file__))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_bwd_noalloc_rejects_plans_beyond_its_scratch():
    """jfa_bwd_noalloc returns JFA_ERR_WORKSPACE, before touching the GPU,
    for a DQ plan whose partials exceed the library's scratch area: a
    broadcast Q of 16 heads x 8,192 rows has 512 (head, Q tile) groups, so
    512 dQ workers x 256 x 128 x 4 bytes = 64 MiB > 32 MiB."""
    prob = J.Problem(batch=2, num_heads=16, head_dim=128, broadcast_q=True, lq=8192,
                     softmax_scale=0.088)
    kv = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_BWD, 256)
    dq = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_DQ, 256)
    assert J.jfa_bwd_workspace_bytes(prob, dq.info) == 64 << 20 > J.JFA_NOALLOC_SCRATCH_BYTES
    plans = [J.JfaDevicePlan(ctypes.pointer(p.info), 0x1000, 0x1000, None, None) for p in (kv, dq)]
    cp = prob.c()
    t = ctypes.c_void_p(0x1000)
    st = J._lib().jfa_bwd_noalloc(ctypes.byref(cp), ctypes.byref(plans[0]), ctypes.byref(plans[1]),
                                  None, t, *([t] * 11), None)
    assert st == J.JFA_ERR_WORKSPACE
    # a DQ plan of the wrong pass is refused the same way as by jfa_bwd
    st = J._lib().jfa_bwd_noalloc(ctypes.byref(cp), ctypes.byref(plans[0]), ctypes.byref(plans[0]),
                                  None, t, *([t] * 11), None)
    assert st == J.JFA_ERR_PLAN_MISMATCH


def test_bwd_stage_flags_validated_before_launch():
    """The stage mask accepts the JFA_BWD_* flags and the atomic dQ modifier,
    and refuses any other bit before launching anything."""
    prob = _prob()
    kv = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_BWD, 4)
    dq = J.jfa_plan_build(prob, None, [0, 3, 5], None, J.JFA_PASS_DQ, 4)
    need = J.jfa_bwd_workspace_bytes(prob, dq.info)
    t = _FakeTensor(0x1000)
    f = lambda x: ctypes.c_void_p(x.data_ptr())
    plans = [J.JfaDevicePlan(ctypes.pointer(p.info), 0x1000, 0x1000, None, None) for p in (kv, dq)]
    cp = prob.c()

    def call(stages, **over):
        args = [t] * 11
        return J._lib().jfa_bwd_stages(stages, ctypes.byref(cp), ctypes.byref(plans[0]),
                                       ctypes.byref(plans[1]), None, ctypes.c_void_p(0x1000),
                                       *[f(x) for x in args], f(t), need, None)
    for bad in (-1, 32, 64, J.JFA_BWD_ALL | 32):
        assert call(bad) == J.JFA_ERR_INVALID_ARG, bad
    # a valid mask gets past the flag check to the next validation step (a
    # misaligned dq_accum here), so nothing is launched in this test
    args = [t] * 11
    args[9] = _FakeTensor(0x1004)
    st = J._lib().jfa_bwd_stages(J.JFA_BWD_ALL | J.JFA_BWD_DQ_ATOMIC, ctypes.byref(cp),
                                 ctypes.byref(plans[0]), ctypes.byref(plans[1]), None,
                                 ctypes.c_void_p(0x1000), *[f(x) for x in args], f(t), need, None)
    assert st == J.JFA_ERR_INVALID_ARG


def test_tile_log_is_debug_only():
    """The product library has no executed-tile log; the debug build takes a
    16-byte-aligned log or NULL (argument checks only: nothing launches)."""
    with pytest.raises(J.JfaError) as e:
        J.jfa_debug_tile_log(None, 0)
    assert e.value.status == J.JFA_ERR_UNSUPPORTED
    dbg = J.load_library(J.DEBUG_LIB_PATH)
    assert dbg.jfa_abi_version() == J.jfa_abi_version()
    assert dbg.jfa_debug_tile_log(ctypes.c_void_p(0x1008), 4) == J.JFA_ERR_INVALID_ARG
    assert dbg.jfa_debug_tile_log(ctypes.c_void_p(0x1000), -1) == J.JFA_ERR_INVALID_ARG
    assert dbg.jfa_debug_tile_log(None, 0) == J.JFA_OK


def test_jfa_log_writes_one_line_per_call():
    """JFA_LOG=1: each planner / entry point call writes one line to stderr
    with its name, the problem and its status; unset: nothing."""
    import subprocess
    import sys
    code = ("import jagged_flashattention_amd as J\n"
            "p = J.Problem(batch=2, num_heads=1, head_dim=64, broadcast_q=True, lq=8, softmax_scale=0.125)\n"
            "J.jfa_plan_build(p, None, [0, 3, 5], None, J.JFA_PASS_BWD, 4)\n"
            "try:\n"
            "    J.jfa_plan_build(p, None, [0, 3, 2], None, J.JFA_PASS_FWD, 4)\n"
            "except J.JfaError:\n"
            "    pass\n")
    env = dict(os.environ, JFA_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    lines = [l for l in r.stderr.splitlines() if l.startswith("jfa: ")]
    assert len(lines) == 3, r.stderr                       # query + build, then the failing query
    assert "jfa_plan_query" in lines[0] and "jfa_plan_build" in lines[1]
    assert "B=2 H=1 D=64" in lines[1] and "pass=1" in lines[1] and "-> ok (0)" in lines[1]
    assert "-> bad offsets" in lines[2] and "(-2)" in lines[2] and "workers=" not in lines[2]
    env["JFA_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode == 0 and "jfa: " not in r.stderr
