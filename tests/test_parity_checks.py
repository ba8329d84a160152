"""The whole-tensor checks of the full-size GPU tests, run on the oracle's own
outputs (rounded to bf16 like the GPU's): they pass on the correct result and
fail on each planted mistake a lost or misplaced tile would make (the
mistakes are planted in the oracle's outputs, on the CPU)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention as A

import parity_checks as PC

torch = pytest.importorskip("torch")


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def oracle_outputs(x):
    w = x.workload
    q, k, v, do = (x.as_f64(n) for n in ("q", "k", "v", "do"))
    kw = dict(scale=w.scale, broadcast_q=w.broadcast_q, q_offsets=x.q_offsets, causal=w.causal,
              block_mask=x.block_mask, window=w.window)
    o, lse = A.forward(q, k, v, x.kv_offsets, **kw)
    dq, dk, dv, delta = A.backward(q, k, v, do, x.kv_offsets, **kw)
    return dict(o=bf16(o), lse=torch.from_numpy(lse.astype(np.float32)), dk=bf16(dk), dv=bf16(dv),
                dq=bf16(dq), dq_accum=torch.from_numpy(dq.astype(np.float32)),
                delta=torch.from_numpy(delta.astype(np.float32)),
                q=PC.to_torch_bf16(x.q, "cpu"), k=PC.to_torch_bf16(x.k, "cpu"),
                v=PC.to_torch_bf16(x.v, "cpu"), do=PC.to_torch_bf16(x.do, "cpu"))


CASES = {
    "broadcast": lambda: W.make_inputs(2, lengths=np.array([700, 16, 300, 1100, 40]), heads=2),
    "causal": lambda: W.make_inputs(3, lengths=np.array([600, 129, 300]), heads=2),
    "window": lambda: W.make_inputs(6, lengths=np.array([1500, 200]), heads=2),
    "sparse": lambda: W.make_inputs(5, lengths=np.array([700, 16, 300, 900]), heads=2),
}


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    x = CASES[request.param]()
    return x, oracle_outputs(x)


def run(x, r):
    return PC.check_invariants(x, *(r[n] for n in ("o", "lse", "dk", "dv", "dq", "dq_accum",
                                                    "delta", "q", "k", "v", "do")))


def test_correct_result_passes(case):
    x, r = case
    ratios, viol = run(x, r)
    # the bf16 rounding of the outputs alone stays far inside the tolerance
    assert max(r_ for r_, _ in ratios.values()) < PC.TOL / 4 and viol < 0


def _fails(x, r):
    with pytest.raises(AssertionError):
        run(x, r)


def test_dropped_kv_tile_is_caught(case):
    """One 256-key tile of one head never written (zeros instead of NaN)."""
    x, r = case
    b = int(np.argmax(x.lengths))
    k0 = int(x.kv_offsets[b])
    for name in ("dk", "dv"):
        bad = dict(r)
        bad[name] = r[name].clone()
        bad[name][k0:k0 + 256, 1] = 0
        _fails(x, bad)


def test_misscaled_kv_tile_is_caught(case):
    """One tile's dK and dV written with a wrong factor (e.g. a lost scale)."""
    x, r = case
    b = int(np.argmax(x.lengths))
    k0 = int(x.kv_offsets[b])
    bad = dict(r)
    bad["dv"] = r["dv"].clone()
    bad["dv"][k0 + 64:k0 + 128, 0] *= 1.5
    _fails(x, bad)
    bad = dict(r)
    bad["dk"] = r["dk"].clone()
    bad["dk"][k0 + 64:k0 + 128, 0] *= 2.0
    _fails(x, bad)


def test_misplaced_key_rows_are_caught(case):
    """A tile's dK rows written one key off (rows shifted inside the tile)."""
    x, r = case
    b = int(np.argmax(x.lengths))
    k0 = int(x.kv_offsets[b])
    bad = dict(r)
    bad["dk"] = r["dk"].clone()
    bad["dk"][k0 + 1:k0 + 257, 1] = r["dk"][k0:k0 + 256, 1]
    _fails(x, bad)


def test_misscaled_dq_rows_are_caught(case):
    """Part of dQ lost (a 64-row block of one head scaled by 1/2)."""
    x, r = case
    bad = dict(r)
    bad["dq_accum"] = r["dq_accum"].clone()
    bad["dq_accum"][64:128, 1] *= 0.5
    _fails(x, bad)


def test_o_row_of_another_sequence_is_caught(case):
    """The O rows of one sequence taken from the wrong V (its rows shifted
    onto another sequence's values)."""
    x, r = case
    roff = PC.q_row_offsets(x)
    b = int(np.argmin(x.lengths))
    bad = dict(r)
    bad["o"] = r["o"].clone()
    n = int(roff[b + 1] - roff[b])
    # O of a short sequence replaced by 3x another sequence's V rows (far
    # outside its own V's range)
    k0 = int(x.kv_offsets[int(np.argmax(x.lengths))])
    bad["o"][roff[b]:roff[b] + n] = 3 * torch.from_numpy(W.bf16_bits_to_f32(x.v[k0:k0 + n])).to(torch.bfloat16)
    _fails(x, bad)


def test_nan_left_anywhere_is_caught(case):
    x, r = case
    for name in ("o", "lse", "dk", "dv", "dq", "dq_accum", "delta"):
        bad = dict(r)
        bad[name] = r[name].clone()
        bad[name].view(-1)[bad[name].numel() // 2] = float("nan")
        _fails(x, bad)
