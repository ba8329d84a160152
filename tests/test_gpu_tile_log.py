"""The executed-tile log of the debug build (jfa_debug_tile_log) against the
plans: every worker of the forward, dK/dV and dQ kernels takes exactly its
plan's tiles in plan order (the dynamic forward: its first tile, then claims
in increasing order, every tile taken once over all workers), the stream
bookkeeping of the backward passes matches the plan's block counts, no
record carries an index outside the problem, and the debug build's outputs
equal the product library's bit for bit."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import jagged_flashattention_amd as J  # noqa: E402
from test_gpu_parity import dev, problem_of  # noqa: E402

CASES = {
    "gem_full_dynamic": (lambda: W.make_inputs(2), True),
    "gem_full_static": (lambda: W.make_inputs(2), False),
    "causal": (lambda: W.make_inputs(3, lengths=np.array([600, 129, 300, 1000, 0, 2100]), heads=2),
               True),
    "window": (lambda: W.make_inputs(6, lengths=np.array([1500, 200, 3000]), heads=2), True),
    "sparse": (lambda: W.make_inputs(5, lengths=np.array([700, 16, 300, 900, 0]), heads=2), True),
}


def _run(x, dynamic, lib, cap):
    """Forward, dQ pass, dK/dV pass and dQ reduce with lib; the tile log of
    each kernel when cap > 0."""
    torch.manual_seed(0)
    with J.using_library(lib):
        prob = problem_of(x)
        att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask, fwd_dynamic=dynamic)
        q, k, v, do = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
        W_max = max(att.fwd_plan.info.num_workers, att.bwd_plan.info.num_workers,
                    att.dq_plan.info.num_workers)
        log = torch.zeros(W_max * (8 + 8 * cap), dtype=torch.int32, device="cuda")
        logs = {}

        def take(name, plan):
            torch.cuda.synchronize()
            logs[name] = J.read_tile_log(log, plan.info.num_workers, cap)
            log.zero_()
            torch.cuda.synchronize()

        if cap:
            J.jfa_debug_tile_log(log, cap)
        try:
            o, lse = att.forward(q, k, v)
            take("fwd", att.fwd_plan)
            out = att.backward(q, k, v, o, lse, do, stages=J.JFA_BWD_DQ)
            take("dq", att.dq_plan)
            att.backward(q, k, v, o, lse, do, out=out, stages=J.JFA_BWD_DKDV)
            take("dkdv", att.bwd_plan)
            att.backward(q, k, v, o, lse, do, out=out, stages=J.JFA_BWD_DQ_REDUCE)
            torch.cuda.synchronize()
        finally:
            if cap:
                J.jfa_debug_tile_log(None, 0)
    out.update(o=o, lse=lse)
    return att, out, logs


def _check_static(recs, counts, host_plan, pass_id, streamed):
    wp, tiles = host_plan.worker_ptr, host_plan.tiles
    for w in range(len(wp) - 1):
        mine = tiles[wp[w]:wp[w + 1]]
        assert counts[w] == len(mine), (pass_id, w, counts[w], len(mine))
        r = recs[w]
        assert len(r) == len(mine)
        if not len(mine):
            continue
        assert (r[:, 0] == pass_id).all() and (r[:, 1] == w).all()
        assert np.array_equal(r[:, 2:6], mine), (pass_id, w)
        assert (r[:, 7] == 0).all(), ("index flags", pass_id, w, r[:, 7])
        if streamed:
            # the stream position at each tile's end = blocks of the tiles so far
            assert np.array_equal(r[:, 6], np.cumsum(mine[:, 3])), (pass_id, w)


def _check_dynamic(recs, counts, host_plan):
    tiles = host_plan.tiles
    N = len(tiles)
    index = {tuple(t[:3]): i for i, t in enumerate(tiles)}
    assert len(index) == N
    seen = np.zeros(N, dtype=np.int64)
    for w, r in enumerate(recs):
        assert counts[w] == len(r)
        if not len(r):
            assert w >= N, ("worker without tiles", w)
            continue
        assert (r[:, 0] == 0).all() and (r[:, 1] == w).all() and (r[:, 7] == 0).all()
        idx = np.array([index[tuple(t)] for t in r[:, 2:5]])
        assert np.array_equal(r[:, 5], tiles[idx, 3])
        assert idx[0] == w, ("first tile of a worker is its own", w, idx[0])
        assert (np.diff(idx) > 0).all(), ("claims in increasing order", w)
        seen[idx] += 1
    assert (seen == 1).all(), ("every tile taken once", np.flatnonzero(seen != 1)[:10])


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


@pytest.fixture(scope="module")
def debug_lib():
    return J.load_library(J.DEBUG_LIB_PATH)


@pytest.mark.parametrize("case", list(CASES))
def test_executed_tiles_follow_the_plan(case, debug_lib):
    make, dynamic = CASES[case]
    x = make()
    cap = 0
    att0 = J.JaggedAttention(problem_of(x), x.kv_offsets, x.q_offsets, x.block_mask,
                             fwd_dynamic=dynamic)
    for p in (att0.fwd_plan_host, att0.bwd_plan_host, att0.dq_plan_host):
        cap = max(cap, int(np.diff(p.worker_ptr).max(initial=0)), 1)
    # the dynamic forward: a worker may claim any number of tiles
    cap = max(cap, len(att0.fwd_plan_host.tiles))
    print("tile log", case, "cap", cap, flush=True)
    att, got, logs = _run(x, dynamic, debug_lib, cap)
    if att.fwd_plan.info.pass_ & J.JFA_PLAN_DYNAMIC:
        _check_dynamic(*logs["fwd"], att.fwd_plan_host)
    else:
        _check_static(*logs["fwd"], att.fwd_plan_host, 0, streamed=False)
    _check_static(*logs["dq"], att.dq_plan_host, 2, streamed=True)
    _check_static(*logs["dkdv"], att.bwd_plan_host, 1, streamed=True)
    # the product library computes the same bits
    _, ref, _ = _run(x, dynamic, J._lib(), 0)
    for name in ("o", "lse", "dq", "dk", "dv", "dq_accum", "delta"):
        assert torch.equal(_bits(got[name]), _bits(ref[name])), name


def test_product_library_has_no_tile_log():
    log = torch.zeros(64, dtype=torch.int32, device="cuda")
    with pytest.raises(J.JfaError) as e:
        J.jfa_debug_tile_log(log, 1)
    assert e.value.status == J.JFA_ERR_UNSUPPORTED
