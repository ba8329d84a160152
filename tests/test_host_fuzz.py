"""Seeded random problems through the C++ host planner (CPU only): valid ones
must give the oracle planner's plan bit for bit, malformed ones (bad
offsets, masks, windows, worker counts) a status code. Run on the library as
built and, by tests/test_host_sanitized.py, on the host-check build under
AddressSanitizer and UndefinedBehaviorSanitizer."""
import numpy as np
import pytest

import jagged_flashattention_amd as J
from oracle import planner as OP

FWD_BM, FWD_BN, BWD_BM, BWD_BN = 256, 64, 32, 256
MASK = 128
N_CASES = 120


def _random_problem(rng):
    """A valid problem of a random kind with small, ragged sizes (lengths
    include 0 and values just past tile multiples)."""
    kind = rng.choice(["bcast", "causal", "window", "sparse", "sparse_self"])
    B = int(rng.integers(0, 7))
    H = int(rng.integers(1, 4))
    choices = np.array([0, 1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 700])
    lens = rng.choice(choices, size=B) if rng.random() < 0.5 else rng.integers(0, 800, size=B)
    lens = lens.astype(np.int64)
    kw = dict(batch=B, num_heads=H, head_dim=int(rng.choice([64, 128])), softmax_scale=0.125)
    q_lens, qoff, mask, window = None, None, None, None
    if kind in ("bcast", "sparse"):
        lq = int(rng.choice([1, 31, 32, 200, 256, 257, 600]))
        kw.update(broadcast_q=True, lq=lq)
        q_lens = [lq] * B
    else:
        kw.update(broadcast_q=False, lq=0)
        q_lens = lens
        qoff = OP.offsets_from_lengths(lens)
    if kind == "causal":
        kw.update(causal=True)
    if kind == "window":
        left, right = int(rng.integers(0, 300)), int(rng.integers(-1, 200))
        if right < 0:
            kw.update(causal=True)
            right = 0
        kw.update(window_left=left, window_right=right)
        window = (left, right)
    if kind in ("sparse", "sparse_self"):
        mq = max(1, -(-max([int(x) for x in q_lens] + [1]) // MASK)) + int(rng.integers(0, 2))
        mk = max(1, -(-max([int(x) for x in lens] + [1]) // MASK)) + int(rng.integers(0, 2))
        mask = (rng.random((B, mq, mk)) < rng.uniform(0.1, 0.9)).astype(np.uint8)
        kw.update(mask_q_blocks=mq, mask_kv_blocks=mk)
    return J.Problem(**kw), lens, q_lens, qoff, mask, window


def _oracle_plan(prob, lens, q_lens, mask, window, pass_, workers):
    causal = prob.causal
    if pass_ == J.JFA_PASS_DQ:
        return OP.plan_dq(q_lens, lens, prob.num_heads, workers, broadcast_q=prob.broadcast_q,
                          lq=prob.lq, block_m=FWD_BM, block_n=FWD_BN, causal=causal,
                          block_mask=mask, window=window)
    base = pass_ & ~J.JFA_PLAN_DYNAMIC
    bm, bn = (FWD_BM, FWD_BN) if base == J.JFA_PASS_FWD else (BWD_BM, BWD_BN)
    return OP.plan(q_lens, lens, prob.num_heads, workers, base, block_m=bm, block_n=bn,
                   causal=causal, block_mask=mask, window=window,
                   dynamic=bool(pass_ & J.JFA_PLAN_DYNAMIC))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_valid_problem_plans_equal_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    prob, lens, q_lens, qoff, mask, window = _random_problem(rng)
    kvoff = OP.offsets_from_lengths(lens)
    workers = int(rng.choice([1, 2, 3, 17, 256, 600]))
    for pass_ in (J.JFA_PASS_FWD, J.JFA_PASS_FWD | J.JFA_PLAN_DYNAMIC, J.JFA_PASS_BWD,
                  J.JFA_PASS_DQ):
        hp = J.jfa_plan_build(prob, qoff, kvoff, mask, pass_, workers)
        wp, tiles = _oracle_plan(prob, lens, q_lens, mask, window, pass_, workers)
        assert np.array_equal(hp.worker_ptr, wp), (seed, pass_)
        assert np.array_equal(hp.tiles, tiles), (seed, pass_)
        if mask is not None and pass_ != J.JFA_PASS_DQ:
            base = pass_ & ~J.JFA_PLAN_DYNAMIC
            bm, bn = (FWD_BM, FWD_BN) if base == J.JFA_PASS_FWD else (BWD_BM, BWD_BN)
            sp, si = OP.sparse_lists(mask, q_lens, lens, base, block_m=bm, block_n=bn)
            assert np.array_equal(hp.sparse_ptr, sp) and np.array_equal(hp.sparse_idx, si)


def _corrupt(rng, prob, lens, qoff, mask):
    """One malformed variant of a valid problem and the statuses it may get."""
    kvoff = OP.offsets_from_lengths(lens).astype(np.int64)
    what = rng.choice(["kv_first", "kv_decreasing", "kv_overflow", "q_decreasing", "heads",
                       "batch", "mask_missing", "mask_blocks", "window", "lq", "scale"])
    qo = None if qoff is None else np.array(qoff, dtype=np.int64)
    m = mask
    bad = {J.JFA_ERR_BAD_OFFSETS}
    p = J.Problem(**prob.__dict__)
    if what == "kv_first":
        kvoff = kvoff + int(rng.integers(1, 5))
    elif what == "kv_decreasing":
        if len(kvoff) < 2:
            kvoff = np.array([0, 5, 2])
            p.batch = 2
            if not p.broadcast_q:
                qo = np.array([0, 1, 2])
            if m is not None:
                m = np.ones((2, p.mask_q_blocks, p.mask_kv_blocks), np.uint8)
        else:
            i = int(rng.integers(1, len(kvoff)))
            kvoff[i] = kvoff[i - 1] - int(rng.integers(1, 4))
    elif what == "kv_overflow":
        # a running sum that wrapped around int32
        kvoff = np.array([0, 2**31 - 1, -2**31 + 10], dtype=np.int64)
        p.batch = 2
        qo = None if qo is None else np.array([0, 3, 6])
        m = None if m is None else np.ones((2, p.mask_q_blocks, p.mask_kv_blocks), np.uint8)
    elif what == "q_decreasing" and qo is not None and len(qo) >= 2:
        qo[-1] = qo[0] - 1
    elif what == "heads":
        p.num_heads = int(rng.choice([0, -3]))
        bad = {J.JFA_ERR_INVALID_ARG}
    elif what == "batch":
        p.batch = -1
        bad = {J.JFA_ERR_INVALID_ARG}
    elif what == "mask_missing" and p.mask_q_blocks:
        m = None
        bad = {J.JFA_ERR_BAD_MASK, J.JFA_ERR_INVALID_ARG}
    elif what == "mask_blocks" and p.mask_q_blocks and p.batch > 0:
        # too few mask columns for the longest sequence
        p.mask_kv_blocks = max(0, -(-int(max(lens)) // MASK) - 1)
        if p.mask_kv_blocks == 0 and p.mask_q_blocks:
            bad = {J.JFA_ERR_BAD_MASK, J.JFA_ERR_INVALID_ARG}
        elif int(max(lens)) == 0:
            return None
        else:
            bad = {J.JFA_ERR_BAD_MASK}
        m = np.ones((p.batch, p.mask_q_blocks, max(p.mask_kv_blocks, 1)), np.uint8)
    elif what == "window" and not p.broadcast_q:
        p.window_right = -int(rng.integers(2, 9))
        p.window_left = max(p.window_left, 0)
        bad = {J.JFA_ERR_INVALID_ARG, J.JFA_ERR_UNSUPPORTED}
    elif what == "lq" and p.broadcast_q:
        p.lq = -int(rng.integers(1, 100))
        bad = {J.JFA_ERR_INVALID_ARG}
    elif what == "scale":
        p.softmax_scale = float(rng.choice([0.0, -1.0, np.nan, np.inf]))
        bad = {J.JFA_ERR_INVALID_ARG}
    else:
        return None
    return p, qo, kvoff, m, bad


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_malformed_problem_gets_a_status(seed):
    rng = np.random.default_rng(5000 + seed)
    prob, lens, _, qoff, mask, _ = _random_problem(rng)
    got = None
    for _ in range(8):
        got = _corrupt(rng, prob, lens, qoff, mask)
        if got is not None:
            break
    if got is None:
        pytest.skip("no applicable corruption for this draw")
    p, qo, kvoff, m, bad = got
    kv32 = np.asarray(kvoff).astype(np.int64)
    if kv32.max(initial=0) >= 2**31 or kv32.min(initial=0) < -2**31:
        pytest.skip("offsets outside int32")
    for pass_ in (J.JFA_PASS_FWD, J.JFA_PASS_BWD, J.JFA_PASS_DQ):
        with pytest.raises(J.JfaError) as e:
            J.jfa_plan_build(p, qo, kv32, m, pass_, 8)
        assert e.value.status in bad, (seed, pass_, e.value.status, bad)
