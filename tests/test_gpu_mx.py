"""MXFP8 variant on the GPU (through the C ABI) against the oracle.

The encoders must equal the oracle's encoder bit for bit (integer codes and
scales). The MXFP8 forward computes attention on the decoded Q, K, V; the
only other rounding besides fp32 accumulation is P's own E4M3 rounding inside
the kernel, so against the oracle's exact attention on the decoded inputs:

  |O_gpu - O| <= sum_j max(2^-4 P_ij, 2^-18) |v_jd|  +  2^-8 |O|  +  1e-3

per element (E4M3 rounds P, scaled by 2^8 and at most 256, to nearest even:
relative error <= 2^-4 in its normal range, absolute <= 2^-10 * 2^-8 below
it; the second term is O's bf16 rounding, the third fp32 accumulation), and
LSE (fp32 softmax on exactly computed scores) within 1e-2.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle import attention as A
from oracle import mx as OMX

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import jagged_flashattention_amd as J  # noqa: E402
from test_gpu_parity import SMALL_CASES, _custom, dev, host_f64, problem_of  # noqa: E402


def _u8(t):
    return t.cpu().numpy().astype(np.uint8)


def test_quantize_rows_bit_exact():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((300, 3, 128)).astype(np.float32)
    x *= np.exp(rng.standard_normal((300, 3, 1)) * 4).astype(np.float32)
    x[5, 1, :32] = 0.0
    x[6, 2, 40] = -0.0
    x[7, 0, :] = 1e-30                                  # below the normal range
    bits = W.f32_to_bf16_bits(x)
    src = dev(bits)
    codes = torch.empty(src.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((3, 300, 4), dtype=torch.uint8, device="cuda")
    J.jfa_mx_quantize_rows(src, codes, scales)
    torch.cuda.synchronize()
    oc, os_ = OMX.quantize_rows(W.bf16_bits_to_f32(bits).astype(np.float64))
    assert np.array_equal(_u8(codes), oc)
    assert np.array_equal(_u8(scales), os_)


@pytest.mark.parametrize("D", [32, 64, 96, 128])
def test_quantize_v_bit_exact(D):
    rng = np.random.default_rng(4)
    lens = np.array([0, 1, 31, 32, 33, 100, 257, 0, 64, 1000])
    off = W.offsets_of(lens)
    v = rng.standard_normal((int(off[-1]), 2, D)).astype(np.float32) * 3
    v *= np.exp(rng.standard_normal((1, 2, D)) * 2).astype(np.float32)   # column scales apart
    v[40] *= 500.0
    v[518:550, 1, :5] = 0.0              # all-zero columns of the last sequence's first block
    bits = W.f32_to_bf16_bits(v)
    boff = J.jfa_mx_block_offsets(off)
    assert np.array_equal(boff, OMX.mx_block_offsets(off))
    nb = int(boff[-1])
    src = dev(bits)
    codes = torch.empty(src.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty((2, nb, D), dtype=torch.uint8, device="cuda")
    J.jfa_mx_quantize_v(src, torch.from_numpy(off).cuda(), torch.from_numpy(boff).cuda(), nb,
                        codes, scales)
    torch.cuda.synchronize()
    oc, os_ = OMX.quantize_v(W.bf16_bits_to_f32(bits).astype(np.float64), off)
    assert np.array_equal(_u8(codes), oc)
    assert np.array_equal(_u8(scales), os_)


def _decoded(x):
    """The oracle's decoding of the oracle's encoding of the bf16 inputs."""
    q = W.bf16_bits_to_f32(x.q).astype(np.float64)
    k = W.bf16_bits_to_f32(x.k).astype(np.float64)
    v = W.bf16_bits_to_f32(x.v).astype(np.float64)
    q = OMX.dequantize_rows(*OMX.quantize_rows(q))
    k = OMX.dequantize_rows(*OMX.quantize_rows(k))
    v = OMX.dequantize_v(*OMX.quantize_v(v, x.kv_offsets), x.kv_offsets)
    return q, k, v


def _check_mx(x, o_gpu, lse_gpu, seqs=None, heads=None):
    w = x.workload
    q, k, v = _decoded(x)
    kw = dict(scale=w.scale, broadcast_q=w.broadcast_q, q_offsets=x.q_offsets, causal=w.causal,
              block_mask=x.block_mask, window=w.window)
    o, lse = A.forward(q, k, v, x.kv_offsets, seqs=seqs, heads=heads, **kw)
    B = x.batch
    total_err, n_el = 0.0, 0
    for b in (range(B) if seqs is None else seqs):
        k0, k1 = int(x.kv_offsets[b]), int(x.kv_offsets[b + 1])
        if w.broadcast_q:
            qs, os_ = slice(0, w.lq), slice(b * w.lq, (b + 1) * w.lq)
        else:
            qs = os_ = slice(int(x.q_offsets[b]), int(x.q_offsets[b + 1]))
        n_rows = os_.stop - os_.start
        if n_rows == 0:
            continue
        vis = A.visibility(n_rows, k1 - k0, causal=w.causal, window=w.window,
                           mask_b=None if x.block_mask is None else x.block_mask[b])
        for h in (range(w.heads) if heads is None else heads):
            lse_ref = lse[h, os_]
            fin = np.isfinite(lse_ref)
            s = w.scale * (q[qs, h] @ k[k0:k1, h].T)
            p = np.where(vis, np.exp(s - np.where(fin, lse_ref, 0.0)[:, None]), 0.0)
            av = np.abs(v[k0:k1, h])
            bound = (2.0 ** -4 * p @ av + 2.0 ** -18 * (vis.astype(float) @ av)
                     + 2.0 ** -8 * np.abs(o[os_, h]) + 1e-3)
            err = np.abs(o_gpu[os_, h] - o[os_, h])
            assert np.all(err <= bound), (b, h, float((err - bound).max()))
            total_err += err.sum()
            n_el += err.size
            assert np.array_equal(fin, np.isfinite(lse_gpu[h, os_]))
            if fin.any():
                assert np.abs(lse_gpu[h, os_][fin] - lse_ref[fin]).max() <= 1e-2, (b, h)
    # and on average far inside that bound (a systematic error would not be)
    assert total_err / max(n_el, 1) <= 1e-2


def _run_mx(x, dynamic=True):
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask, fwd_dynamic=dynamic)
    mxq = att.quantize_mx(dev(x.q), dev(x.k), dev(x.v))
    H, D = prob.num_heads, prob.head_dim
    o = torch.full((att.total_q, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda")
    att.forward_mx(mxq, o, lse)
    torch.cuda.synchronize()
    return (W.bf16_bits_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64),
            lse.cpu().numpy().astype(np.float64))


MX_CASES = ["bcast_ragged_d128", "perseq_d128", "causal_d128", "sparse_d128", "window_band_d128",
            "window_causal_d128", "cfg2_small", "cfg3_small", "cfg5_small"]


@pytest.mark.parametrize("case", MX_CASES)
def test_mx_forward_small(case):
    print("case", case, flush=True)
    x = SMALL_CASES[case]()
    o, lse = _run_mx(x)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _check_mx(x, o, lse)


def test_mx_forward_static_plan_and_bitwise_repeat():
    x = SMALL_CASES["cfg2_small"]()
    o1, l1 = _run_mx(x, dynamic=False)
    o2, l2 = _run_mx(x, dynamic=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_mx_forward_full_size_sampled():
    print("full-size GEM broadcast-Q, MXFP8", flush=True)
    x = W.make_inputs(2)
    o, lse = _run_mx(x)
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    lens = x.lengths
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 7})
    _check_mx(x, o, lse, seqs=seqs, heads=[1])


def test_mx_rejects_unsupported_head_dim():
    x = SMALL_CASES["bcast_ragged_d64"]()
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask)
    with pytest.raises(J.JfaError) as e:
        mxq = att.quantize_mx(dev(x.q), dev(x.k), dev(x.v))
        att.forward_mx(mxq)
    assert e.value.status == J.JFA_ERR_UNSUPPORTED


MXB_CASES = ["bcast_ragged_d128", "perseq_d128", "causal_d128", "sparse_d128", "window_band_d128",
             "cfg2_small", "cfg3_small", "cfg5_small"]


def _f64(bits):
    return W.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("case", MXB_CASES)
def test_mx_dq_pass(case):
    """The MXFP8 dQ pass against the oracle's definition of it (exact dS) on
    the oracle's own O and LSE: the GPU rounds dS to E4M3 with one scale per
    (row, 32-key tile) 2^e, the smallest power of two with max|dS| / 2^e <=
    448 (so 2^e <= max|dS| 2^-7 and nothing is clamped); per element

      |dQ_gpu - dQ| <= scale sum_j (2^-4 |dS_ij| + 2^-17 max_j' |dS_ij'|) |k_jd|
                       + 1e-4 scale sum_j |dS_ij| |k_jd|
                       + 2^-17 scale sum_j P_ij (sum_d |do_id v_jd| + sum_d |do_id o_id|) |k_jd|
                       + 1e-6

    (half an E4M3 step: relative 2^-4 in the normal range, at most 2^-10 2^e
    below it; fp32 sums; and the fp32 sums of D = 128 terms that form dP and
    delta, within D 2^-24 = 2^-17 of the magnitudes summed, which is not
    relative to dS = P (dP - delta): where dP and delta nearly cancel it is
    the largest term), and delta within fp32 summation error."""
    print("case", case, flush=True)
    _check_mx_dq(SMALL_CASES[case]())


def _check_mx_dq(x, mean_frac=0.25):
    """The check of test_mx_dq_pass on the instance x (mean_frac: see
    _check_mx_dkdv)."""
    w = x.workload
    off = x.kv_offsets
    qf, kf, vf, dof = _f64(x.q), _f64(x.k), _f64(x.v), _f64(x.do)
    q_d = OMX.dequantize_rows(*OMX.quantize_rows(qf))
    k_d = OMX.dequantize_rows(*OMX.quantize_rows(kf))
    v_d = OMX.dequantize_rows(*OMX.quantize_rows(vf))
    do_d = OMX.dequantize_rows(*OMX.quantize_rows(dof))
    k_keys = OMX.dequantize_v(*OMX.quantize_v(kf, off), off)
    v_keys = OMX.dequantize_v(*OMX.quantize_v(vf, off), off)
    kw = dict(scale=w.scale, broadcast_q=w.broadcast_q, q_offsets=x.q_offsets, causal=w.causal,
              block_mask=x.block_mask, window=w.window)
    # the forward's O (bf16) and LSE: the oracle's attention on the MXFP8
    # forward's operands
    o, lse = A.forward(q_d, k_d, v_keys, off, **kw)
    o_bits = W.f32_to_bf16_bits(o.astype(np.float32))
    o_bf = _f64(o_bits)
    dq, delta, abs_sum, floor_sum, acc_sum = OMX.dq_mx(q_d, k_d, v_d, do_d, k_keys, dof, o_bf, lse, off, **kw)

    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask)
    qg, kg, vg, dog = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    mxq = att.quantize_mx(qg, kg, vg)
    ops = att.quantize_mx_bwd(mxq, kg, vg, dog)
    H, D = prob.num_heads, prob.head_dim
    out = dict(dq=torch.full(qg.shape, float("nan"), dtype=torch.bfloat16, device="cuda"),
               dk=torch.empty_like(kg), dv=torch.empty_like(vg),
               dq_accum=torch.full(qg.shape, float("nan"), dtype=torch.float32, device="cuda"),
               delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda"))
    att.backward_mx(qg, kg, vg, dev(o_bits), torch.from_numpy(lse.astype(np.float32)).cuda(), dog, ops,
                    out, stages=J.JFA_BWD_DQ | J.JFA_BWD_DQ_REDUCE)
    torch.cuda.synchronize()
    gdq = out["dq_accum"].cpu().numpy().astype(np.float64)
    gdelta = out["delta"].cpu().numpy().astype(np.float64)
    assert not np.isnan(gdq).any() and not np.isnan(gdelta).any()
    bound = 2.0 ** -4 * abs_sum + 2.0 ** -17 * floor_sum + 1e-4 * abs_sum + 2.0 ** -17 * acc_sum + 1e-6
    err = np.abs(gdq - dq)
    assert np.all(err <= bound), float((err - bound).max())
    # and on average far inside it
    if mean_frac is not None and err.size:
        assert err.mean() <= mean_frac * bound.mean(), ("mean", float(err.mean() / bound.mean()))
    dbound = 2 * D * 2.0 ** -24 * np.einsum("rhd,rhd->hr", np.abs(dof), np.abs(o_bf)) + 1e-30
    assert np.all(np.abs(gdelta - delta) <= dbound), ("delta", float(np.max(np.abs(gdelta - delta) - dbound, initial=0)))
    # the bf16 dq is the rounding of the fp32 sum
    e16 = float(np.max(np.abs(host_f64(out["dq"]) - gdq), initial=0.0))
    assert e16 <= 2 ** -8 * float(np.max(np.abs(gdq), initial=0.0)) + 1e-30, ("bf16 dq", e16)


def test_mx_dq_pass_full_size_one_head():
    """The MXFP8 dQ pass on the full GEM-shaped broadcast-Q workload, in the
    launch configuration the benchmark times, checked on head 1 (every row:
    the broadcast dQ sums over all sequences) against the oracle with the
    bound of test_mx_dq_pass. The other heads get O = 0 and LSE = 30 (their
    P is negligible); they are computed but not checked."""
    print("full-size GEM broadcast-Q, MXFP8 dQ pass, head 1", flush=True)
    x = W.make_inputs(2)
    w = x.workload
    off = x.kv_offsets
    h = 1
    one = lambda a: _f64(a)[:, h:h + 1]
    qf, kf, vf, dof = one(x.q), one(x.k), one(x.v), one(x.do)
    q_d = OMX.dequantize_rows(*OMX.quantize_rows(qf))
    k_d = OMX.dequantize_rows(*OMX.quantize_rows(kf))
    v_d = OMX.dequantize_rows(*OMX.quantize_rows(vf))
    do_d = OMX.dequantize_rows(*OMX.quantize_rows(dof))
    k_keys = OMX.dequantize_v(*OMX.quantize_v(kf, off), off)
    v_keys = OMX.dequantize_v(*OMX.quantize_v(vf, off), off)
    kw = dict(scale=w.scale, broadcast_q=True, q_offsets=None, causal=False)
    o, lse = A.forward(q_d, k_d, v_keys, off, **kw)
    o_bits = W.f32_to_bf16_bits(o.astype(np.float32))
    o_bf = _f64(o_bits)
    dq, delta, abs_sum, floor_sum, acc_sum = OMX.dq_mx(q_d, k_d, v_d, do_d, k_keys, dof, o_bf, lse, off, **kw)

    prob = problem_of(x)
    cus = J.jfa_device_workers(0)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask, fwd_workers=cus,
                            bwd_workers=cus)
    qg, kg, vg, dog = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    H, D = prob.num_heads, prob.head_dim
    o_all = np.zeros((att.total_q, H, D), dtype=np.uint16)
    o_all[:, h] = o_bits[:, 0]
    lse_all = np.full((H, att.total_q), 30.0, dtype=np.float32)
    lse_all[h] = lse[0]
    mxq = att.quantize_mx(qg, kg, vg)
    ops = att.quantize_mx_bwd(mxq, kg, vg, dog)
    out = dict(dq=torch.empty_like(qg), dk=torch.empty_like(kg), dv=torch.empty_like(vg),
               dq_accum=torch.full(qg.shape, float("nan"), dtype=torch.float32, device="cuda"),
               delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda"))
    att.backward_mx(qg, kg, vg, dev(o_all), torch.from_numpy(lse_all).cuda(), dog, ops, out,
                    stages=J.JFA_BWD_DQ | J.JFA_BWD_DQ_REDUCE)
    torch.cuda.synchronize()
    gdq = out["dq_accum"].cpu().numpy().astype(np.float64)
    assert not np.isnan(gdq).any()
    gdq = gdq[:, h:h + 1]
    gdelta = out["delta"].cpu().numpy().astype(np.float64)[h:h + 1]
    bound = 2.0 ** -4 * abs_sum + 2.0 ** -17 * floor_sum + 1e-4 * abs_sum + 2.0 ** -17 * acc_sum + 1e-6
    err = np.abs(gdq - dq)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.mean() <= 0.25 * bound.mean()
    dbound = 2 * D * 2.0 ** -24 * np.einsum("rhd,rhd->hr", np.abs(dof), np.abs(o_bf)) + 1e-30
    assert np.all(np.abs(gdelta - delta) <= dbound)


def test_mx_element_offsets_beyond_int32():
    """The MXFP8 encoders, forward and dQ pass on a batch whose K and V hold
    more than 2^31 elements (a first sequence of 4,198,400 keys with zero dO
    rows, then three random sequences that start past element 2^31). The
    later sequences' O, LSE and the batch-summed dQ (to which the first
    sequence adds exactly nothing) against the oracle on the later
    sequences' own encodings (an MX block never spans two rows or two
    sequences), with the bounds of test_mx_forward_small and
    test_mx_dq_pass."""
    from test_gpu_parity import beyond_int32_inputs
    print("MXFP8, element offsets beyond 2^31", flush=True)
    x, big, later = beyond_int32_inputs()
    w = x.workload
    H, D, lq = w.heads, w.head_dim, w.lq
    sub = dataclasses.replace(x, lengths=np.array(later, dtype=np.int32),
                              kv_offsets=W.offsets_of(np.array(later)), k=x.k[big:], v=x.v[big:],
                              do=x.do[lq:])
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask)
    qg, kg, vg, dog = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    mxq = att.quantize_mx(qg, kg, vg)
    o = torch.full((att.total_q, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda")
    att.forward_mx(mxq, o, lse)
    torch.cuda.synchronize()
    o_h = W.bf16_bits_to_f32(o[lq:].view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    _check_mx(sub, o_h, lse[:, lq:].cpu().numpy().astype(np.float64))

    # the dQ pass on the oracle's O and LSE of the later sequences (the first
    # sequence's rows get O = 0, LSE = 0: with dO = 0 its dS is zero anyway)
    off = sub.kv_offsets
    qf, kf, vf, dof = _f64(sub.q), _f64(sub.k), _f64(sub.v), _f64(sub.do)
    q_d = OMX.dequantize_rows(*OMX.quantize_rows(qf))
    k_d = OMX.dequantize_rows(*OMX.quantize_rows(kf))
    v_d = OMX.dequantize_rows(*OMX.quantize_rows(vf))
    do_d = OMX.dequantize_rows(*OMX.quantize_rows(dof))
    k_keys = OMX.dequantize_v(*OMX.quantize_v(kf, off), off)
    v_keys = OMX.dequantize_v(*OMX.quantize_v(vf, off), off)
    kw = dict(scale=w.scale, broadcast_q=True)
    o_r, lse_r = A.forward(q_d, k_d, v_keys, off, **kw)
    o_bits = W.f32_to_bf16_bits(o_r.astype(np.float32))
    dq, _, abs_sum, floor_sum, acc_sum = OMX.dq_mx(q_d, k_d, v_d, do_d, k_keys, dof, _f64(o_bits), lse_r, off,
                                          **kw)
    o_all = np.zeros((att.total_q, H, D), dtype=np.uint16)
    o_all[lq:] = o_bits
    lse_all = np.zeros((H, att.total_q), dtype=np.float32)
    lse_all[:, lq:] = lse_r
    ops = att.quantize_mx_bwd(mxq, kg, vg, dog)
    out = dict(dq=torch.empty_like(qg), dk=torch.empty_like(kg), dv=torch.empty_like(vg),
               dq_accum=torch.full(qg.shape, float("nan"), dtype=torch.float32, device="cuda"),
               delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda"))
    att.backward_mx(qg, kg, vg, dev(o_all), torch.from_numpy(lse_all).cuda(), dog, ops, out,
                    stages=J.JFA_BWD_DQ | J.JFA_BWD_DQ_REDUCE)
    torch.cuda.synchronize()
    gdq = out["dq_accum"].cpu().numpy().astype(np.float64)
    assert not np.isnan(gdq).any()
    bound = 2.0 ** -4 * abs_sum + 2.0 ** -17 * floor_sum + 1e-4 * abs_sum + 2.0 ** -17 * acc_sum + 1e-6
    err = np.abs(gdq - dq)
    assert np.all(err <= bound), float((err - bound).max())
    assert err.mean() <= 0.25 * bound.mean()


def test_mx_only_empty_sequences():
    """Three empty sequences under a broadcast Q of 5 rows through the MXFP8
    encoders, forward and dQ pass: O = 0, LSE = -inf, delta = 0, dQ = 0 (rows
    without a visible key), no canary left."""
    x = _custom("me", broadcast=True, H=2, D=128, lengths=[0, 0, 0], lq=5)
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask)
    qg, kg, vg, dog = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    H, D = prob.num_heads, prob.head_dim
    mxq = att.quantize_mx(qg, kg, vg)
    o = torch.full((att.total_q, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda")
    att.forward_mx(mxq, o, lse)
    ops = att.quantize_mx_bwd(mxq, kg, vg, dog)
    out = dict(dq=torch.full(qg.shape, float("nan"), dtype=torch.bfloat16, device="cuda"),
               dk=torch.empty_like(kg), dv=torch.empty_like(vg),
               dq_accum=torch.full(qg.shape, float("nan"), dtype=torch.float32, device="cuda"),
               delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda"))
    att.backward_mx(qg, kg, vg, o, lse, dog, ops, out, stages=J.JFA_BWD_DQ | J.JFA_BWD_DQ_REDUCE)
    torch.cuda.synchronize()
    assert float(o.float().abs().max()) == 0.0
    assert bool(torch.all(lse == float("-inf")))
    assert float(out["dq_accum"].abs().max()) == 0.0 and float(out["dq"].float().abs().max()) == 0.0
    assert float(out["delta"].abs().max()) == 0.0


MXKV_CASES = ["bcast_ragged_d128", "perseq_d128", "causal_d128", "sparse_d128", "window_band_d128",
              "window_causal_d128", "cfg2_small", "cfg3_small", "cfg5_small"]


def _row_offsets(x):
    """Offsets of the Q rows and of the dO rows of each sequence (the
    along-rows encodings' block boundaries)."""
    w = x.workload
    if w.broadcast_q:
        return np.array([0, w.lq], dtype=np.int32), (np.arange(x.batch + 1) * w.lq).astype(np.int32)
    return x.q_offsets, x.q_offsets


def _mx_dkdv_case(x, heads=None):
    """The oracle's MXFP8 dK/dV (and its bound terms) and the GPU's, on the
    oracle's own O and LSE of the MXFP8 forward operands; delta from the
    standalone preprocess of the same bf16 O and dO. With ``heads`` only those
    heads carry the case (the others get O = 0, LSE = 30: P negligible)."""
    w = x.workload
    off = x.kv_offsets
    hs = list(range(w.heads)) if heads is None else heads
    sel = lambda a: _f64(a)[:, hs]
    qf, kf, vf, dof = sel(x.q), sel(x.k), sel(x.v), sel(x.do)
    q_d = OMX.dequantize_rows(*OMX.quantize_rows(qf))
    k_d = OMX.dequantize_rows(*OMX.quantize_rows(kf))
    v_d = OMX.dequantize_rows(*OMX.quantize_rows(vf))
    do_d = OMX.dequantize_rows(*OMX.quantize_rows(dof))
    v_keys = OMX.dequantize_v(*OMX.quantize_v(vf, off), off)
    q_off_rows, do_off_rows = _row_offsets(x)
    q_r = OMX.dequantize_v(*OMX.quantize_v(qf, q_off_rows), q_off_rows)
    do_r = OMX.dequantize_v(*OMX.quantize_v(dof, do_off_rows), do_off_rows)
    kw = dict(scale=w.scale, broadcast_q=w.broadcast_q, q_offsets=x.q_offsets, causal=w.causal,
              block_mask=x.block_mask, window=w.window)
    o, lse = A.forward(q_d, k_d, v_keys, off, **kw)
    o_bits = W.f32_to_bf16_bits(o.astype(np.float32))
    ref = OMX.dkdv_mx(q_d, k_d, v_d, do_d, q_r, do_r, dof, _f64(o_bits), lse, off, **kw)

    prob = problem_of(x)
    cus = J.jfa_device_workers(0)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask, fwd_workers=cus,
                            bwd_workers=cus)
    qg, kg, vg, dog = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    H, D = prob.num_heads, prob.head_dim
    o_all = np.zeros((att.total_q, H, D), dtype=np.uint16)
    o_all[:, hs] = o_bits
    lse_all = np.full((H, att.total_q), 30.0, dtype=np.float32)
    lse_all[hs] = lse
    mxq = att.quantize_mx(qg, kg, vg)
    ops = att.quantize_mx_dkdv(att.quantize_mx_bwd(mxq, kg, vg, dog), qg, dog)
    out = dict(dq=torch.empty_like(qg), dk=torch.full_like(kg, float("nan")),
               dv=torch.full_like(vg, float("nan")),
               dq_accum=torch.empty(qg.shape, dtype=torch.float32, device="cuda"),
               delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda"))
    att.backward_mx(qg, kg, vg, dev(o_all), torch.from_numpy(lse_all).cuda(), dog, ops, out,
                    stages=J.JFA_BWD_PREPROCESS | J.JFA_BWD_DKDV)
    torch.cuda.synchronize()
    return ref, host_f64(out["dk"])[:, hs], host_f64(out["dv"])[:, hs]


def _check_mx_dkdv(ref, gdk, gdv, mean_frac=0.25):
    """Against the oracle's exact-P, exact-dS values, per element:
      |dV_gpu - dV| <= 2^-4 P^T|dO_r| + 2^-18 vis^T|dO_r| + 2^-8 |dV| + 1e-4 P^T|dO_r| + 1e-6
      |dK_gpu - dK| <= 2^-4 scale|dS|^T|Q_r| + 2^-17 scale max|dS| sum|Q_r| + 2^-8 |dK|
                        + 1e-4 scale|dS|^T|Q_r|
                        + 2^-17 scale (P (|dO||V|^T + sum_d |dO O|))^T |Q_r| + 1e-6
    (P, at most 1, scaled by 2^8 and rounded to E4M3: relative 2^-4 in its
    normal range, 2^-10 2^-8 below it; dS with its (key, 32-row block) scale
    2^e <= max|dS| 2^-7: relative 2^-4, at most 2^-10 2^e below; the bf16
    rounding of dK, dV; fp32 sums; the fp32 sums of D = 128 terms that form
    dP and delta, as for the dQ pass), and on average inside mean_frac of it.
    A systematic error would not be: unbiased round-to-nearest leaves a mean
    error of at most half its worst case (error uniform within half a step),
    and sums over many terms partly cancel, hence 0.25 on these cases; where
    an element is a single rounded term (a broadcast Q of one row: dV_j =
    P_1j dO_1) the mean reaches about 0.35, so random problems use 0.5; and
    where only a few rounded terms make up every element (a handful of rows
    or keys) the mean says nothing: mean_frac None skips it."""
    dk, dv, pa, pf, ka, kf, kacc = ref
    assert not np.isnan(gdk).any() and not np.isnan(gdv).any()
    bv = 2.0 ** -4 * pa + 2.0 ** -18 * pf + 2.0 ** -8 * np.abs(dv) + 1e-4 * pa + 1e-6
    bk = (2.0 ** -4 * ka + 2.0 ** -17 * kf + 2.0 ** -8 * np.abs(dk) + 1e-4 * ka
          + 2.0 ** -17 * kacc + 1e-6)
    ev, ek = np.abs(gdv - dv), np.abs(gdk - dk)
    if not ev.size:   # no key at all
        return
    assert np.all(ev <= bv), ("dV", float((ev - bv).max()))
    assert np.all(ek <= bk), ("dK", float((ek - bk).max()))
    if mean_frac is not None:
        assert ev.mean() <= mean_frac * bv.mean() and ek.mean() <= mean_frac * bk.mean(), (
            "mean", float(ev.mean() / bv.mean()), float(ek.mean() / bk.mean()))


@pytest.mark.parametrize("case", MXKV_CASES)
def test_mx_dkdv_pass(case):
    """The MXFP8 dK/dV pass against the oracle's definition of it."""
    print("case", case, flush=True)
    x = SMALL_CASES[case]()
    _check_mx_dkdv(*_mx_dkdv_case(x))


def test_mx_dkdv_pass_full_size_one_head():
    """The MXFP8 dK/dV pass on the full GEM-shaped broadcast-Q workload, in
    the launch configuration the benchmark times, checked on every key of
    head 1 against the oracle with the bounds of test_mx_dkdv_pass."""
    print("full-size GEM broadcast-Q, MXFP8 dK/dV pass, head 1", flush=True)
    x = W.make_inputs(2)
    _check_mx_dkdv(*_mx_dkdv_case(x, heads=[1]))


def test_mx_dkdv_rejects_unsupported_head_dim_and_missing_encodings():
    x = SMALL_CASES["bcast_ragged_d64"]()
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask)
    t = torch.zeros(16, dtype=torch.uint8, device="cuda")
    ops = {n: t for n in ("qc", "qs", "kc", "ks", "vdc", "vds", "doc", "dos", "qrc", "qrs", "dorc", "dors")}
    lse = torch.zeros((prob.num_heads, att.total_q), dtype=torch.float32, device="cuda")
    with pytest.raises(J.JfaError) as e:
        J.jfa_bwd_dkdv_mx(prob, att.bwd_plan, None, att.kv_offsets, att.kv_offsets, 64,
                          att.kv_offsets, 64, lse, lse, ops, t, t)
    assert e.value.status == J.JFA_ERR_UNSUPPORTED
