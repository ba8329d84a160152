"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small cases: the oracle evaluates every output; they span several tiles and
ragged tails of every mode (broadcast Q, per-sequence Q, causal, sliding window, block-sparse,
D = 64 and 128, empty and one-key sequences, Lq not a multiple of the tile).
Full sizes: the five workloads run in the launch configuration the benchmark
times, and sampled outputs are compared with the oracle row by row.

Tolerances (stated for this path): O and LSE max |gpu - oracle| <= 1e-2;
dQ, dK, dV max |gpu - oracle| / max |oracle| <= 2e-2.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle import attention as A

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import jagged_flashattention_amd as J  # noqa: E402

TOL_O = 1e-2
TOL_GRAD = 2e-2


def o_err_ok(got, ref):
    """|O_gpu - O| <= TOL_O + 2^-8 |O| element-wise. O is bf16 by contract: a
    correctly rounded bf16 value lies within half a unit in its last place,
    at most 2^-8 |O|, of the exact one, which alone exceeds 1e-2 once |O| >
    2.56 (rows that see one or a few keys, O close to one N(0,1) V row). The
    1e-2 applies on top of that output rounding."""
    return bool(np.all(np.abs(got - ref) <= TOL_O + 2.0 ** -8 * np.abs(ref)))


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_f64(t):
    u = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return W.bf16_bits_to_f32(u).astype(np.float64)


def problem_of(x):
    w = x.workload
    mq, mk = (x.block_mask.shape[1], x.block_mask.shape[2]) if x.block_mask is not None else (0, 0)
    return J.Problem(batch=x.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0,
                     causal=w.causal, mask_q_blocks=mq, mask_kv_blocks=mk,
                     softmax_scale=w.scale, window_left=_bound(w.window, 0),
                     window_right=_bound(w.window, 1))


def _bound(window, k):
    """ABI encoding of one side of a sliding window (-1: none)."""
    return -1 if window is None or window[k] is None else int(window[k])


@dataclasses.dataclass
class GpuRun:
    o: object
    lse: object
    dq: object
    dk: object
    dv: object
    dq_accum: object
    delta: object


def run_gpu(x, fwd_workers=None, bwd_workers=None, dq_workers=None, canary=True,
            fwd_dynamic=True, natural_plans=False):
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask,
                            fwd_workers=fwd_workers, bwd_workers=bwd_workers,
                            dq_workers=dq_workers, fwd_dynamic=fwd_dynamic,
                            natural_plans=natural_plans)
    q, k, v, do = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    H, D = prob.num_heads, prob.head_dim
    o = torch.empty((att.total_q, H, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((H, att.total_q), dtype=torch.float32, device="cuda")
    if canary:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    att.forward(q, k, v, o, lse)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dq_accum=torch.empty(q.shape, dtype=torch.float32, device="cuda"),
               delta=torch.empty((H, att.total_q), dtype=torch.float32, device="cuda"))
    if canary:
        for t in out.values():
            t.fill_(float("nan"))
    att.backward(q, k, v, o, lse, do, out)
    torch.cuda.synchronize()
    return GpuRun(o, lse, **out)


def oracle_full(x):
    q, k, v, do = (x.as_f64(n) for n in ("q", "k", "v", "do"))
    w = x.workload
    kw = dict(scale=w.scale, broadcast_q=w.broadcast_q, q_offsets=x.q_offsets, causal=w.causal,
              block_mask=x.block_mask, window=w.window)
    o, lse = A.forward(q, k, v, x.kv_offsets, **kw)
    dq, dk, dv, delta = A.backward(q, k, v, do, x.kv_offsets, **kw)
    return o, lse, dq, dk, dv, delta


def rel_err(got, ref):
    if ref.size == 0:   # e.g. no query rows at all
        return 0.0
    scale = np.abs(ref).max()
    return np.abs(got - ref).max() / (scale if scale > 0 else 1.0)


def _max_abs(a):
    return float(np.abs(a).max()) if a.size else 0.0


def oracle_kw(x):
    w = x.workload
    return dict(scale=w.scale, broadcast_q=w.broadcast_q, q_offsets=x.q_offsets, causal=w.causal,
                block_mask=x.block_mask, window=w.window)


def check_all(x, g):
    """The whole path (the GPU backward fed the GPU forward's O and LSE)
    against the exact oracle. dQ and dK may also move by what forming delta
    from the stored bf16 O costs (oracle.attention.delta_slack), on top of the
    gradient tolerance; check_bwd_given_o holds the backward alone to the
    gradient tolerance with that effect taken out."""
    o, lse, dq, dk, dv, delta = oracle_full(x)
    q64, k64, v64, do64 = (x.as_f64(n) for n in ("q", "k", "v", "do"))
    sq, sk = A.delta_slack(q64, k64, v64, do64, x.kv_offsets, **oracle_kw(x))
    go, glse = host_f64(g.o), g.lse.cpu().numpy().astype(np.float64)
    assert not np.isnan(go).any() and not np.isnan(glse).any()
    fin = np.isfinite(lse)
    assert np.array_equal(fin, np.isfinite(glse)), "rows without keys must give LSE=-inf"
    assert o_err_ok(go, o), ("o", _max_abs(go - o))
    if fin.any():
        assert _max_abs(glse[fin] - lse[fin]) <= TOL_O, ("lse", _max_abs(glse[fin] - lse[fin]))
    gdq, gdk, gdv = host_f64(g.dq), host_f64(g.dk), host_f64(g.dv)
    gacc = g.dq_accum.cpu().numpy().astype(np.float64)
    for name, got, ref, slack in (("dq", gdq, dq, sq), ("dk", gdk, dk, sk), ("dv", gdv, dv, 0.0),
                                  ("dq_accum", gacc, dq, sq)):
        assert not np.isnan(got).any(), name
        allowed = TOL_GRAD * _max_abs(ref) + slack
        assert np.all(np.abs(got - ref) <= allowed), (name, rel_err(got, ref))
    gdelta = g.delta.cpu().numpy()
    assert _max_abs(gdelta - delta) <= 2e-2 * max(1.0, _max_abs(delta)), ("delta", _max_abs(gdelta - delta))


def run_gpu_bwd_given(x, o_bits, lse32, bwd_workers=None, dq_workers=None, canary=True, **_):
    """The GPU backward alone, fed O (bf16 bits) and LSE (float32) from the
    caller."""
    att = J.JaggedAttention(problem_of(x), x.kv_offsets, x.q_offsets, x.block_mask,
                            bwd_workers=bwd_workers, dq_workers=dq_workers)
    q, k, v, do, o = dev(x.q), dev(x.k), dev(x.v), dev(x.do), dev(o_bits)
    lse = torch.from_numpy(np.ascontiguousarray(lse32, dtype=np.float32)).cuda()
    H = x.workload.heads
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dq_accum=torch.empty(q.shape, dtype=torch.float32, device="cuda"),
               delta=torch.empty((H, att.total_q), dtype=torch.float32, device="cuda"))
    if canary:
        for t in out.values():
            t.fill_(float("nan"))
    att.backward(q, k, v, o, lse, do, out)
    torch.cuda.synchronize()
    return out


def check_bwd_given_o(x, **plan):
    """The GPU backward fed the oracle's O rounded to bf16 (as the forward
    stores it) and its LSE in float32, against the oracle's backward that
    forms delta from that same O: dQ, dK, dV, dq_accum and delta to the
    gradient tolerance, with nothing added for the stored O."""
    q64, k64, v64, do64 = (x.as_f64(n) for n in ("q", "k", "v", "do"))
    kw = oracle_kw(x)
    o, lse = A.forward(q64, k64, v64, x.kv_offsets, **kw)
    o_bits = W.f32_to_bf16_bits(o.astype(np.float32))
    o_st = W.bf16_bits_to_f32(o_bits).astype(np.float64)
    dq, dk, dv, delta = A.backward(q64, k64, v64, do64, x.kv_offsets, o=o_st, **kw)
    out = run_gpu_bwd_given(x, o_bits, lse.astype(np.float32), **plan)
    for name, ref in (("dq", dq), ("dk", dk), ("dv", dv)):
        got = host_f64(out[name])
        assert not np.isnan(got).any(), name
        assert rel_err(got, ref) <= TOL_GRAD, (name, rel_err(got, ref))
    e = rel_err(out["dq_accum"].cpu().numpy().astype(np.float64), dq)
    assert e <= TOL_GRAD, ("dq_accum", e)
    gdelta = out["delta"].cpu().numpy()
    assert _max_abs(gdelta - delta) <= 2e-2 * max(1.0, _max_abs(delta)), ("delta", _max_abs(gdelta - delta))


def _custom(name, *, broadcast, H, D, lengths, lq=0, causal=False, mask_seed=None, seed=11,
            q_lengths=None, window=None):
    w = W.Workload(name, len(lengths), H, D, broadcast, lq, causal, "const:1", seed=seed,
                   mask_seed=mask_seed, window=window)
    x = W.make_inputs(w, lengths=np.array(lengths))
    if q_lengths is not None:
        # per-sequence Q with its own lengths: redraw Q / dO rows for them
        rng = np.random.default_rng(seed + 1000)
        q_off = W.offsets_of(np.array(q_lengths))
        tq = int(q_off[-1])
        x = dataclasses.replace(
            x, q_offsets=q_off,
            q=W.f32_to_bf16_bits(rng.standard_normal((tq, H, D), dtype=np.float32)),
            do=W.f32_to_bf16_bits(rng.standard_normal((tq, H, D), dtype=np.float32)))
    return x


RAGGED = [0, 1, 15, 16, 63, 64, 65, 127, 128, 129, 200, 300]
CAUSAL = [1, 63, 64, 65, 128, 129, 257, 400]
WINDOWED = [1, 5, 64, 129, 300, 600, 0]

SMALL_CASES = {
    "cfg1": lambda: W.make_inputs(1),
    "bcast_ragged_d128": lambda: _custom("b128", broadcast=True, H=2, D=128, lengths=RAGGED, lq=100),
    "bcast_ragged_d64": lambda: _custom("b64", broadcast=True, H=3, D=64, lengths=RAGGED, lq=200),
    "perseq_d128": lambda: _custom("p128", broadcast=False, H=2, D=128,
                                   lengths=[70, 3, 200, 129, 0], q_lengths=[5, 130, 64, 1, 7]),
    "causal_d128": lambda: _custom("c128", broadcast=False, H=2, D=128, lengths=CAUSAL, causal=True),
    "causal_d64": lambda: _custom("c64", broadcast=False, H=2, D=64, lengths=CAUSAL, causal=True),
    # sliding windows: causal with a left bound, two-sided, one-sided, zero width
    "window_causal_d128": lambda: _custom("w1", broadcast=False, H=2, D=128, lengths=WINDOWED,
                                          causal=True, window=(100, None)),
    "window_band_d128": lambda: _custom("w2", broadcast=False, H=2, D=128, lengths=WINDOWED,
                                        window=(300, 40)),
    "window_right_d64": lambda: _custom("w3", broadcast=False, H=2, D=64, lengths=WINDOWED,
                                        window=(None, 70)),
    "window_zero_d64": lambda: _custom("w4", broadcast=False, H=2, D=64, lengths=WINDOWED,
                                       window=(0, 0)),
    "window_wide_d128": lambda: _custom("w5", broadcast=False, H=1, D=128, lengths=[1200, 700, 1],
                                        causal=True, window=(513, None)),
    "sparse_d128": lambda: _custom("s128", broadcast=True, H=2, D=128, lq=256, mask_seed=5,
                                   lengths=[1, 64, 65, 127, 128, 129, 300, 513, 640]),
    "sparse_d64": lambda: _custom("s64", broadcast=True, H=2, D=64, lq=200, mask_seed=7,
                                  lengths=[1, 64, 65, 127, 128, 129, 300, 513]),
    # long sequences: broadcast dQ tiles split into chunks (odd chunk starts
    # inside the block-sparse lists too)
    "bcast_long_d64": lambda: _custom("bl64", broadcast=True, H=2, D=64, lq=300,
                                      lengths=[1500, 33, 2100, 1025]),
    "sparse_long_d128": lambda: _custom("sl128", broadcast=True, H=2, D=128, lq=256, mask_seed=9,
                                        lengths=[2500, 1100, 64, 3000]),
    "cfg2_small": lambda: W.make_inputs(2, batch=16, heads=2),
    "cfg3_small": lambda: W.make_inputs(3, batch=3, heads=2),
    "cfg4_small": lambda: W.make_inputs(4, batch=2, heads=2),
    "cfg5_small": lambda: W.make_inputs(5, batch=12, heads=2),
}


@pytest.mark.parametrize("case", list(SMALL_CASES))
def test_small_parity(case):
    print("case", case, flush=True)
    x = SMALL_CASES[case]()
    check_all(x, run_gpu(x))
    check_bwd_given_o(x)


def test_one_key_sequence_is_bitwise_v_row():
    x = _custom("onekey", broadcast=True, H=2, D=128, lengths=[1, 5, 1], lq=70)
    g = run_gpu(x)
    o = g.o.view(torch.int16).cpu().numpy().view(np.uint16)
    for b, row in ((0, 0), (2, 6)):
        for h in range(2):
            assert np.array_equal(o[b * 70:(b + 1) * 70, h], np.broadcast_to(x.v[row, h], (70, 128)))


def test_zero_width_window_is_bitwise_v():
    """Window (0, 0): each row sees its own key alone, so P = 1 exactly: O is
    bitwise the bf16 V row and dV bitwise dO. dK = scale (dP - delta) q is
    zero up to the rounding of dP - delta (two fp32 sums of the same
    products in different orders)."""
    x = SMALL_CASES["window_zero_d64"]()
    g = run_gpu(x)
    o = g.o.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(o, x.v)
    assert np.array_equal(g.dv.view(torch.int16).cpu().numpy().view(np.uint16), x.do)
    assert g.dk.float().abs().max().item() <= 1e-5


@pytest.mark.parametrize("case", ["bcast_ragged_d128", "perseq_d128", "causal_d64", "sparse_d128",
                                  "cfg2_small"])
def test_delta_of_dq_pass_and_standalone_stage(case):
    """delta = rowsum(dO * O) of the GPU's own bf16 O and dO, formed by the dQ
    pass (full backward) and by the standalone preprocess stage: both within
    fp32 summation error (D terms, each rounded at most twice: 2 D 2^-24 of
    the sum of |dO * O|) of the fp64 sum, for every row, empty sequences
    included."""
    print("case", case, flush=True)
    x = SMALL_CASES[case]()
    g = run_gpu(x)
    H, D = x.workload.heads, x.workload.head_dim
    o, do = host_f64(g.o), x.as_f64("do")
    ref = np.einsum("rhd,rhd->hr", do, o)
    bound = 2 * D * 2.0 ** -24 * np.einsum("rhd,rhd->hr", np.abs(do), np.abs(o)) + 1e-30
    d_dq = g.delta.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(d_dq - ref) <= bound)
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask)
    out = dict(dq=g.dq, dk=g.dk, dv=g.dv, dq_accum=g.dq_accum,
               delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda"))
    att.backward(dev(x.q), dev(x.k), dev(x.v), g.o, g.lse, dev(x.do), out,
                 stages=J.JFA_BWD_PREPROCESS)
    torch.cuda.synchronize()
    d_pre = out["delta"].cpu().numpy().astype(np.float64)
    assert np.all(np.abs(d_pre - ref) <= bound)


def test_zero_q_gives_mean_of_v():
    x = _custom("zeroq", broadcast=True, H=1, D=64, lengths=[7, 300], lq=40)
    x = dataclasses.replace(x, q=np.zeros_like(x.q))
    g = run_gpu(x)
    o = host_f64(g.o)
    v = W.bf16_bits_to_f32(x.v).astype(np.float64)
    assert o_err_ok(o[:40], np.broadcast_to(v[0:7].mean(axis=0), o[:40].shape))
    assert o_err_ok(o[40:], np.broadcast_to(v[7:307].mean(axis=0), o[40:].shape))
    lse = g.lse.cpu().numpy()
    np.testing.assert_allclose(lse[0, :40], np.log(7), atol=1e-5)
    np.testing.assert_allclose(lse[0, 40:], np.log(300), atol=1e-5)


@pytest.mark.parametrize("case", ["bcast_ragged_d128", "causal_d128", "sparse_d128"])
def test_deterministic_across_plans_and_runs(case):
    """O, LSE, dK, dV are bitwise identical for any worker count (each tile is
    computed by one workgroup in a fixed order). dQ is bitwise identical from
    run to run of the same plans (no atomics; broadcast partials are summed in
    worker order); across dQ plans with other worker counts only the grouping
    of the fp32 sum changes."""
    x = SMALL_CASES[case]()
    runs = [run_gpu(x, fwd_workers=fw, bwd_workers=bw, dq_workers=qw)
            for fw, bw, qw in ((None, None, None), (1, 1, 1), (7, 13, 5), (None, None, None))]
    ref = runs[0]
    for name in ("dq_accum", "dq"):
        a, b = getattr(ref, name), getattr(runs[3], name)
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), name
    for r in runs[1:]:
        for name in ("o", "lse", "dk", "dv", "delta"):
            a, b = getattr(ref, name), getattr(r, name)
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)), name
        d = (ref.dq_accum - r.dq_accum).abs().max().item()
        assert d <= 1e-4 * max(1.0, ref.dq_accum.abs().max().item())


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("case", ["bcast_ragged_d128", "perseq_d128", "causal_d64", "sparse_d128",
                                  "window_band_d128",
                                  "cfg2_small"])
def test_dynamic_forward_equals_static(case):
    """The dynamic plan (tiles claimed at run time) gives O and LSE bitwise
    equal to the static plan's, for any worker count (more workers than
    tiles, one worker), and back-to-back launches on one workspace (the
    counter resets itself) agree."""
    print("case", case, flush=True)
    x = SMALL_CASES[case]()
    ref = run_gpu(x, fwd_dynamic=False)
    prob = problem_of(x)
    q, k, v = dev(x.q), dev(x.k), dev(x.v)
    H, D = prob.num_heads, prob.head_dim
    for fw in (None, 1, 3, 4096):
        att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask, fwd_workers=fw,
                                fwd_dynamic=True)
        assert att.fwd_ws_bytes > 0
        for rep_ in range(3):
            o = torch.full((att.total_q, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
            lse = torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda")
            att.forward(q, k, v, o, lse)
            torch.cuda.synchronize()
            assert torch.equal(_bits(o), _bits(ref.o)), (fw, rep_)
            assert torch.equal(_bits(lse), _bits(ref.lse)), (fw, rep_)
        assert int(att.fwd_workspace.view(torch.int32)[:2].abs().sum().item()) == 0


# ----------------------------------------------------------------- full sizes

def _head_f64(bits, h, rows=None):
    sl = bits[:, h, :] if rows is None else bits[rows, h, :]
    return W.bf16_bits_to_f32(sl).astype(np.float64)[:, None, :]


# One workload's full-size run at a time, shared by its tests below (the run
# takes a second; the oracle's comparisons are split so that no test nears
# the per-test time limit).
_FULL = {}


def full_run(cfg):
    if cfg not in _FULL:
        _FULL.clear()
        x = W.make_inputs(cfg)
        _FULL[cfg] = (x, run_gpu(x, canary=True))
    return _FULL[cfg]


def sampled_sequences(x, cfg):
    """The longest, the shortest and one random sequence of the workload."""
    rng = np.random.default_rng(100 + cfg)
    lens = x.lengths
    return {"longest": int(np.argmax(lens)), "shortest": int(np.argmin(lens)),
            "random": int(rng.integers(0, x.batch))}


FULL_CASES = [(cfg, part) for cfg in (2, 3, 4, 5, 6)
              for part in ("invariants", "longest", "shortest", "random")
              + (("dq_rows",) if W.WORKLOADS[cfg].broadcast_q else ())]


@pytest.mark.parametrize("cfg,part", FULL_CASES)
def test_full_size(cfg, part):
    """The workloads at full size, in the launch configuration the benchmark
    times (dynamic forward plan, one workgroup per CU), outputs NaN-filled
    before the run.
      invariants: every output free of NaN, and for every sequence and head
        the identities sum dK = 0, sum dV = sum dO, sum dV v^T = sum dO O^T,
        sum dK k^T = sum q dq^T (per head over the batch with a broadcast Q)
        and O inside the range of the visible V (tests/parity_checks.py);
      longest / shortest / random: that sequence's O, LSE, dK, dV (and dQ
        rows with per-sequence Q) of every head against the oracle;
      dq_rows: rows of the batch-summed dQ of every head against the oracle
        (each needs one row of every sequence's scores)."""
    print("full-size workload", cfg, part, flush=True)
    x, g = full_run(cfg)
    w = x.workload
    if part == "invariants":
        import parity_checks as PC
        ratios, viol = PC.check_invariants(x, g.o, g.lse, g.dk, g.dv, g.dq, g.dq_accum, g.delta,
                                           dev(x.q), dev(x.k), dev(x.v), dev(x.do))
        print("identity ratios / tolerance:",
              {n: round(r / PC.TOL, 3) for n, (r, _) in ratios.items()}, "O range:", viol, flush=True)
        # the bf16 dq is the rounding of the fp32 sum
        gdq, gdq16 = g.dq_accum.double(), g.dq.double()
        assert float((gdq16 - gdq).abs().max()) <= 2 ** -8 * float(gdq.abs().max())
        return
    heads = list(range(w.heads))
    if part == "dq_rows":
        rng = np.random.default_rng(200 + cfg)
        rows = np.array(sorted(set([0, w.lq - 1] + list(rng.integers(0, w.lq, size=4)))))
        gdq = g.dq_accum.cpu().numpy()
        for h in heads:
            ref = A.broadcast_dq_rows(_head_f64(x.q, h), _head_f64(x.k, h), _head_f64(x.v, h),
                                      _head_f64(x.do, h), x.kv_offsets, 0, rows, scale=w.scale,
                                      block_mask=x.block_mask)
            assert rel_err(gdq[rows, h], ref) <= TOL_GRAD, h
        return
    b = sampled_sequences(x, cfg)[part]
    k0, k1 = int(x.kv_offsets[b]), int(x.kv_offsets[b + 1])
    if w.broadcast_q:
        qs, os_ = slice(0, w.lq), slice(b * w.lq, (b + 1) * w.lq)
    else:
        qs = os_ = slice(int(x.q_offsets[b]), int(x.q_offsets[b + 1]))
    off = np.array([0, k1 - k0], dtype=np.int32)
    qoff = None if w.broadcast_q else np.array([0, qs.stop - qs.start], dtype=np.int32)
    mask = None if x.block_mask is None else x.block_mask[b:b + 1]
    kw = dict(scale=w.scale, broadcast_q=w.broadcast_q, q_offsets=qoff, causal=w.causal,
              block_mask=mask, window=w.window)
    cols = lambda t, sl: t[sl].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    go, gdk, gdv = cols(g.o, os_), cols(g.dk, slice(k0, k1)), cols(g.dv, slice(k0, k1))
    glse = g.lse[:, os_].cpu().numpy()
    gdq = g.dq_accum[qs].cpu().numpy()
    for h in heads:
        q1, k1_, v1 = _head_f64(x.q, h, qs), _head_f64(x.k, h, slice(k0, k1)), _head_f64(x.v, h, slice(k0, k1))
        do1 = _head_f64(x.do, h, os_)
        o, lse = A.forward(q1, k1_, v1, off, **kw)
        dq, dk, dv, _ = A.backward(q1, k1_, v1, do1, off, **kw)
        assert o_err_ok(W.bf16_bits_to_f32(go[:, h]), o[:, 0]), (b, h)
        assert np.abs(glse[h] - lse[0]).max() <= TOL_O, (b, h)
        assert rel_err(W.bf16_bits_to_f32(gdk[:, h]), dk[:, 0]) <= TOL_GRAD, (b, h)
        assert rel_err(W.bf16_bits_to_f32(gdv[:, h]), dv[:, 0]) <= TOL_GRAD, (b, h)
        if not w.broadcast_q:
            assert rel_err(gdq[:, h], dq[:, 0]) <= TOL_GRAD, (b, h)


@pytest.mark.parametrize("case", ["bcast_ragged_d128", "bcast_ragged_d64", "sparse_d128",
                                  "bcast_long_d64", "cfg2_small", "perseq_d128"])
def test_atomic_dq_reduction(case):
    """The atomic second stage of the broadcast-Q dQ reduction
    (JFA_BWD_DQ_ATOMIC): dq_accum against the oracle and within fp32 summation
    error of the fixed-order reduce (only the order of the fp32 adds differs),
    dq the bf16 rounding of it; dK, dV and delta do not depend on the dQ
    scheme (bit for bit). With per-sequence Q the flag changes nothing."""
    print("case", case, flush=True)
    x = SMALL_CASES[case]()
    ref = run_gpu(x)
    prob = problem_of(x)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask)
    q, k, v, do = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    H = prob.num_heads
    out = dict(dq=torch.full_like(q, float("nan")), dk=torch.full_like(k, float("nan")),
               dv=torch.full_like(v, float("nan")),
               dq_accum=torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda"),
               delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32, device="cuda"))
    for _ in range(2):   # the stage zeroes dq_accum itself: a second run adds nothing twice
        att.backward(q, k, v, ref.o, ref.lse, do, out, stages=J.JFA_BWD_ALL | J.JFA_BWD_DQ_ATOMIC)
    torch.cuda.synchronize()
    for name in ("dk", "dv", "delta"):
        assert torch.equal(_bits(out[name]), _bits(getattr(ref, name))), name
    if not prob.broadcast_q:
        for name in ("dq", "dq_accum"):
            assert torch.equal(_bits(out[name]), _bits(getattr(ref, name))), name
        return
    got, base = out["dq_accum"].double(), ref.dq_accum.double()
    assert not torch.isnan(got).any()
    assert float((got - base).abs().max()) <= 1e-5 * max(1.0, float(base.abs().max()))
    assert torch.equal(_bits(out["dq"]), _bits(out["dq_accum"].to(torch.bfloat16)))
    _, _, dq, _, _, _ = oracle_full(x)
    assert rel_err(got.cpu().numpy(), dq) <= TOL_GRAD


def beyond_int32_inputs():
    """Broadcast Q (H=4, D=128, 256 rows) over a first sequence of 4,198,400
    keys (1,025 copies of one random 4,096-key block; its dO rows zero) and
    three random ones that start past element 2^31 of K and V. Returns
    (inputs, length of the first sequence, lengths of the others)."""
    H, D, lq, blk, reps = 4, 128, 256, 4096, 1025
    later = [1000, 37, 300]
    base = _custom("i32", broadcast=True, H=H, D=D, lengths=[blk] + later, lq=lq, seed=9)
    big = blk * reps
    assert big * H * D > 2 ** 31
    lens = np.array([big] + later, dtype=np.int32)
    tile_rows = lambda a: np.concatenate([np.tile(a[:blk], (reps, 1, 1)), a[blk:]])
    do = base.do.copy()
    do[:lq] = 0
    x = dataclasses.replace(base, lengths=lens, kv_offsets=W.offsets_of(lens), k=tile_rows(base.k),
                            v=tile_rows(base.v), do=do)
    return x, big, later


def test_element_offsets_beyond_int32():
    """A first sequence of 4,198,400 keys (H=4, D=128: K and V hold more than
    2^31 elements, 4.3 GB each) puts every later sequence past element 2^31,
    so any 32-bit element index would wrap. Its keys are 1,025 copies of one
    random 4,096-key block and its dO rows are zero (so its dK, dV and its
    share of the batch-summed dQ are exactly zero); the three later sequences
    are random. Checked against the oracle: O and LSE of two rows of the long
    sequence, O, LSE, dK, dV of the later sequences, every row of dQ."""
    print("element offsets beyond 2^31", flush=True)
    x, big, later = beyond_int32_inputs()
    H, D, lq = x.workload.heads, x.workload.head_dim, x.workload.lq
    g = run_gpu(x, canary=True)
    w = x.workload
    off = x.kv_offsets
    # the long sequence: no gradient
    for t in (g.dk, g.dv):
        assert float(t[:big].abs().amax()) == 0.0
    go = g.o.view(torch.int16).cpu().numpy().view(np.uint16)
    glse = g.lse.cpu().numpy()
    gdk = g.dk[big:].view(torch.int16).cpu().numpy().view(np.uint16)
    gdv = g.dv[big:].view(torch.int16).cpu().numpy().view(np.uint16)
    gdq = g.dq_accum.cpu().numpy()
    kw = dict(scale=w.scale, broadcast_q=True)
    h = 1
    rows = [0, lq - 1]
    q_rows = _head_f64(x.q, h)[rows]
    o0, lse0 = A.forward(q_rows, _head_f64(x.k, h, slice(0, big)), _head_f64(x.v, h, slice(0, big)),
                         np.array([0, big], dtype=np.int32), **kw)
    assert o_err_ok(W.bf16_bits_to_f32(go[rows, h]), o0[:, 0])
    assert np.abs(glse[h, rows] - lse0[0]).max() <= TOL_O
    # the later sequences, as a batch of their own (broadcast dQ sums them)
    sub = W.offsets_of(np.array(later))
    q_all = x.as_f64("q")
    k_s = W.bf16_bits_to_f32(x.k[big:]).astype(np.float64)
    v_s = W.bf16_bits_to_f32(x.v[big:]).astype(np.float64)
    do_s = W.bf16_bits_to_f32(x.do[lq:]).astype(np.float64)
    o, lse = A.forward(q_all, k_s, v_s, sub, **kw)
    dq, dk, dv, _ = A.backward(q_all, k_s, v_s, do_s, sub, **kw)
    assert o_err_ok(W.bf16_bits_to_f32(go[lq:]), o)
    assert np.abs(glse[:, lq:] - lse).max() <= TOL_O
    assert rel_err(W.bf16_bits_to_f32(gdk), dk) <= TOL_GRAD
    assert rel_err(W.bf16_bits_to_f32(gdv), dv) <= TOL_GRAD
    assert rel_err(gdq, dq) <= TOL_GRAD


def test_long_sequence_sampled():
    """One sequence of 262,181 keys (1,025 KV tiles, a dQ tile cut into 257
    chunks per (head, Q tile)) beside an empty, a one-key and a 4,999-key
    sequence, with a ragged broadcast Q of 300 rows (two Q tiles): O, LSE,
    dK, dV of the long sequence and the other sequences against the oracle,
    rows of the batch-summed dQ too."""
    print("long sequence", flush=True)
    x = _custom("long", broadcast=True, H=2, D=128, lengths=[262181, 0, 1, 4999], lq=300, seed=5)
    g = run_gpu(x, canary=True)
    w = x.workload
    go = g.o.view(torch.int16).cpu().numpy().view(np.uint16)
    glse = g.lse.cpu().numpy()
    gdk = g.dk.view(torch.int16).cpu().numpy().view(np.uint16)
    gdv = g.dv.view(torch.int16).cpu().numpy().view(np.uint16)
    gdq = g.dq_accum.cpu().numpy()
    h = 1
    for b in (0, 2, 3):
        k0, k1 = int(x.kv_offsets[b]), int(x.kv_offsets[b + 1])
        os_ = slice(b * w.lq, (b + 1) * w.lq)
        q1, k1_, v1 = _head_f64(x.q, h), _head_f64(x.k, h, slice(k0, k1)), _head_f64(x.v, h, slice(k0, k1))
        do1 = _head_f64(x.do, h, os_)
        off = np.array([0, k1 - k0], dtype=np.int32)
        kw = dict(scale=w.scale, broadcast_q=True)
        o, lse = A.forward(q1, k1_, v1, off, **kw)
        _, dk, dv, _ = A.backward(q1, k1_, v1, do1, off, **kw)
        assert o_err_ok(W.bf16_bits_to_f32(go[os_, h]), o[:, 0]), b
        assert np.abs(glse[h, os_] - lse[0]).max() <= TOL_O, b
        assert rel_err(W.bf16_bits_to_f32(gdk[k0:k1, h]), dk[:, 0]) <= TOL_GRAD, b
        assert rel_err(W.bf16_bits_to_f32(gdv[k0:k1, h]), dv[:, 0]) <= TOL_GRAD, b
    # the empty sequence: O = 0, LSE = -inf
    os1 = slice(w.lq, 2 * w.lq)
    assert not W.bf16_bits_to_f32(go[os1]).any() and np.all(glse[:, os1] == -np.inf)
    rows = np.array([0, 1, 255, 256, 299])
    ref = A.broadcast_dq_rows(_head_f64(x.q, h), _head_f64(x.k, h), _head_f64(x.v, h),
                              _head_f64(x.do, h), x.kv_offsets, 0, rows, scale=w.scale)
    assert rel_err(gdq[rows, h], ref) <= TOL_GRAD


@pytest.mark.parametrize("kind", ["empty_batch", "all_empty_sequences", "perseq_all_empty"])
def test_degenerate_batches(kind):
    """No sequence at all (B = 0, a broadcast Q of 7 rows), three empty
    sequences under a broadcast Q of 5 rows, and per-sequence Q with empty Q
    and KV everywhere: every kernel either launches nothing or writes the
    defined values (O = 0, LSE = -inf, delta = 0, dQ = 0; the oracle's
    reading of rows without a visible key), and no canary survives."""
    print("degenerate batch", kind, flush=True)
    if kind == "empty_batch":
        x = _custom("e0", broadcast=True, H=2, D=64, lengths=[], lq=7)
    elif kind == "all_empty_sequences":
        x = _custom("e1", broadcast=True, H=2, D=128, lengths=[0, 0, 0], lq=5)
    else:
        x = _custom("e2", broadcast=False, H=2, D=64, lengths=[0, 0], q_lengths=[0, 0])
    g = run_gpu(x, canary=True)
    o, lse, dq, dk, dv, delta = oracle_full(x)
    go = host_f64(g.o)
    assert go.shape == o.shape and np.array_equal(go, np.zeros_like(go))
    glse = g.lse.cpu().numpy()
    assert glse.shape == lse.shape and np.all(glse == -np.inf) and np.all(lse == -np.inf)
    for got, ref in ((g.dq_accum.cpu().numpy(), dq), (host_f64(g.dq), dq)):
        assert got.shape == ref.shape and np.array_equal(got, np.zeros_like(got))
        assert np.array_equal(ref, np.zeros_like(ref))
    assert g.dk.numel() == 0 and g.dv.numel() == 0
    if x.t_q > 0:
        assert np.array_equal(g.delta.cpu().numpy(), np.zeros((x.workload.heads, x.t_q)))


@pytest.mark.parametrize("case", ["bcast_ragged_d128", "causal_d64", "sparse_d128", "cfg2_small"])
def test_natural_plans(case):
    """The unsorted round-robin plans (the benchmark's ablation) through every
    kernel: each tile's O, LSE, dK and dV are computed by one workgroup
    whatever the order, so they equal the sorted plans' bit for bit; dQ
    (per-worker partial sums with a broadcast Q) against the oracle."""
    print("case", case, flush=True)
    x = SMALL_CASES[case]()
    ref = run_gpu(x)
    g = run_gpu(x, natural_plans=True)
    for name in ("o", "lse", "dk", "dv"):
        assert torch.equal(_bits(getattr(g, name)), _bits(getattr(ref, name))), name
    _, _, dq, _, _, _ = oracle_full(x)
    assert rel_err(g.dq_accum.cpu().numpy().astype(np.float64), dq) <= TOL_GRAD
