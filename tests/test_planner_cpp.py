"""The C++ host planner equals the oracle planner bit for bit (CPU only)."""
import numpy as np
import pytest

import jagged_flashattention_amd as J
import workloads as W
from oracle import planner as OP

FWD_BM, FWD_BN, BWD_BM, BWD_BN = 256, 64, 32, 256


def _problem_of(x):
    w = x.workload
    mq, mk = (x.block_mask.shape[1], x.block_mask.shape[2]) if x.block_mask is not None else (0, 0)
    return J.Problem(batch=x.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0, causal=w.causal,
                     mask_q_blocks=mq, mask_kv_blocks=mk, softmax_scale=w.scale)


def _lengths_only(cfg):
    """Workload lengths (and mask) without drawing the big tensors."""
    w = W.WORKLOADS[cfg]
    rng = np.random.default_rng(w.seed)
    lens = W.draw_lengths(w.lengths, w.batch, rng)
    mask = None
    if w.mask_seed is not None:
        mask = W.draw_block_mask(lens, w.lq, w.mask_seed)
    return w, lens, mask


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("workers", [1, 7, 255, 256, 512])
@pytest.mark.parametrize("pass_", [J.JFA_PASS_FWD, J.JFA_PASS_BWD])
def test_cpp_plan_equals_oracle_plan(cfg, workers, pass_):
    w, lens, mask = _lengths_only(cfg)
    kv_off = W.offsets_of(lens)
    q_off = None if w.broadcast_q else kv_off
    mq, mk = (mask.shape[1], mask.shape[2]) if mask is not None else (0, 0)
    prob = J.Problem(batch=w.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0, causal=w.causal,
                     mask_q_blocks=mq, mask_kv_blocks=mk, softmax_scale=w.scale)
    hp = J.jfa_plan_build(prob, q_off, kv_off, mask, pass_, workers)
    q_lens = [w.lq] * w.batch if w.broadcast_q else lens
    bm, bn = (FWD_BM, FWD_BN) if pass_ == J.JFA_PASS_FWD else (BWD_BM, BWD_BN)
    wp, tiles = OP.plan(q_lens, lens, w.heads, workers, pass_, block_m=bm, block_n=bn,
                        causal=w.causal, block_mask=mask)
    assert np.array_equal(hp.worker_ptr, wp)
    assert np.array_equal(hp.tiles, tiles)
    assert hp.info.num_tiles == len(tiles)
    assert hp.info.total_work == int(tiles[:, 3].sum())
    assert hp.info.max_work == int(tiles[:, 3].max())
    assert hp.info.block_m == bm and hp.info.block_n == bn
    assert hp.info.total_kv == int(kv_off[-1])
    if mask is not None:
        sp, si = OP.sparse_lists(mask, q_lens, lens, pass_, block_m=bm, block_n=bn)
        assert np.array_equal(hp.sparse_ptr, sp)
        assert np.array_equal(hp.sparse_idx, si)
    else:
        assert hp.sparse_ptr is None and hp.info.sparse_rows == 0


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
@pytest.mark.parametrize("workers", [1, 3, 7, 255, 256, 512])
def test_cpp_dq_plan_equals_oracle(cfg, workers):
    w, lens, mask = _lengths_only(cfg)
    kv_off = W.offsets_of(lens)
    q_off = None if w.broadcast_q else kv_off
    mq, mk = (mask.shape[1], mask.shape[2]) if mask is not None else (0, 0)
    prob = J.Problem(batch=w.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0, causal=w.causal,
                     mask_q_blocks=mq, mask_kv_blocks=mk, softmax_scale=w.scale)
    hp = J.jfa_plan_build(prob, q_off, kv_off, mask, J.JFA_PASS_DQ, workers)
    q_lens = [w.lq] * w.batch if w.broadcast_q else lens
    wp, tiles = OP.plan_dq(q_lens, lens, w.heads, workers, broadcast_q=w.broadcast_q,
                           lq=w.lq if w.broadcast_q else 0, block_m=FWD_BM, block_n=FWD_BN,
                           causal=w.causal, block_mask=mask)
    assert hp.info.block_m == FWD_BM and hp.info.block_n == FWD_BN
    assert hp.info.num_workers == len(wp) - 1
    assert np.array_equal(hp.worker_ptr, wp)
    assert np.array_equal(hp.tiles, tiles)
    if mask is not None:
        sp, si = OP.sparse_lists(mask, q_lens, lens, OP.FWD, block_m=FWD_BM)
        assert np.array_equal(hp.sparse_ptr, sp) and np.array_equal(hp.sparse_idx, si)


def test_cpp_plan_random_small_problems():
    rng = np.random.default_rng(42)
    for trial in range(40):
        B = int(rng.integers(0, 6))
        lens = rng.integers(0, 600, size=B).astype(np.int32)
        kv_off = W.offsets_of(lens)
        mode = trial % 4
        H = int(rng.integers(1, 4))
        W_ = int(rng.integers(1, 20))
        lq = int(rng.integers(0, 400))
        mask = None
        if mode == 0:
            prob = J.Problem(B, H, 64, True, lq=lq, softmax_scale=0.1)
            q_off, q_lens, causal = None, [lq] * B, False
        elif mode == 1:
            prob = J.Problem(B, H, 128, False, softmax_scale=0.1)
            q_lens = rng.integers(0, 500, size=B).astype(np.int32)
            q_off, causal = W.offsets_of(q_lens), False
        elif mode == 2:
            prob = J.Problem(B, H, 128, False, causal=True, softmax_scale=0.1)
            q_off, q_lens, causal = kv_off, lens, True
        else:
            nq = max(1, -(-lq // 128))
            nk = max(1, -(-int(lens.max(initial=1)) // 128))
            mask = (rng.random((B, nq, nk)) < 0.5).astype(np.uint8)
            prob = J.Problem(B, H, 64, True, lq=lq, mask_q_blocks=nq, mask_kv_blocks=nk,
                             softmax_scale=0.1)
            q_off, q_lens, causal = None, [lq] * B, False
        for pass_, bm, bn in ((0, FWD_BM, FWD_BN), (1, BWD_BM, BWD_BN)):
            hp = J.jfa_plan_build(prob, q_off, kv_off, mask, pass_, W_)
            wp, tiles = OP.plan(q_lens, lens, H, W_, pass_, block_m=bm, block_n=bn,
                                causal=causal, block_mask=mask)
            assert np.array_equal(hp.worker_ptr, wp), (trial, pass_)
            assert np.array_equal(hp.tiles, tiles), (trial, pass_)
            if mask is not None:
                sp, si = OP.sparse_lists(mask, q_lens, lens, pass_, block_m=bm, block_n=bn)
                assert np.array_equal(hp.sparse_ptr, sp) and np.array_equal(hp.sparse_idx, si)
        hp = J.jfa_plan_build(prob, q_off, kv_off, mask, J.JFA_PASS_DQ, W_)
        wp, tiles = OP.plan_dq(q_lens, lens, H, W_, broadcast_q=bool(prob.broadcast_q),
                               lq=prob.lq, block_m=FWD_BM, block_n=FWD_BN, causal=causal,
                               block_mask=mask)
        assert np.array_equal(hp.worker_ptr, wp), (trial, "dq")
        assert np.array_equal(hp.tiles, tiles), (trial, "dq")


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("workers", [1, 7, 256, 5000])
def test_cpp_dynamic_plan_equals_oracle(cfg, workers):
    w, lens, mask = _lengths_only(cfg)
    kv_off = W.offsets_of(lens)
    q_off = None if w.broadcast_q else kv_off
    mq, mk = (mask.shape[1], mask.shape[2]) if mask is not None else (0, 0)
    prob = J.Problem(batch=w.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0, causal=w.causal,
                     mask_q_blocks=mq, mask_kv_blocks=mk, softmax_scale=w.scale)
    hp = J.jfa_plan_build(prob, q_off, kv_off, mask, J.JFA_PASS_FWD | J.JFA_PLAN_DYNAMIC, workers)
    q_lens = [w.lq] * w.batch if w.broadcast_q else lens
    wp, tiles = OP.plan(q_lens, lens, w.heads, workers, OP.FWD, block_m=FWD_BM, block_n=FWD_BN,
                        causal=w.causal, block_mask=mask, dynamic=True)
    assert hp.info.pass_ == J.JFA_PASS_FWD | J.JFA_PLAN_DYNAMIC
    assert hp.info.num_workers == workers
    assert np.array_equal(hp.worker_ptr, wp)
    assert np.array_equal(hp.tiles, tiles)


def test_cpp_dynamic_plan_only_for_forward():
    prob = J.Problem(2, 1, 64, True, lq=8, softmax_scale=0.1)
    for p in (J.JFA_PASS_BWD, J.JFA_PASS_DQ):
        with pytest.raises(J.JfaError) as e:
            J.jfa_plan_build(prob, None, [0, 3, 5], None, p | J.JFA_PLAN_DYNAMIC, 4)
        assert e.value.status == J.JFA_ERR_INVALID_ARG


def test_cpp_band_plans_equal_oracle():
    """Sliding-window problems: C++ FWD, BWD and DQ plans equal the oracle's."""
    rng = np.random.default_rng(7)
    for trial in range(30):
        B = int(rng.integers(1, 6))
        lens = rng.integers(0, 1500, size=B).astype(np.int32)
        off = W.offsets_of(lens)
        causal = bool(trial % 3 == 0)
        wl = int(rng.integers(-1, 700))
        wr = -1 if causal else int(rng.integers(-1, 400))
        if wl < 0 and wr < 0 and not causal:
            wl = 5
        prob = J.Problem(B, 2, 128, False, causal=causal, softmax_scale=0.1,
                         window_left=wl, window_right=wr)
        window = (None if wl < 0 else wl, None if wr < 0 else wr)
        W_ = int(rng.integers(1, 40))
        for pass_, bm, bn in ((0, FWD_BM, FWD_BN), (1, BWD_BM, BWD_BN)):
            hp = J.jfa_plan_build(prob, off, off, None, pass_, W_)
            wp, tiles = OP.plan(lens, lens, 2, W_, pass_, block_m=bm, block_n=bn, causal=causal,
                                window=window)
            assert np.array_equal(hp.worker_ptr, wp), (trial, pass_)
            assert np.array_equal(hp.tiles, tiles), (trial, pass_)
        hp = J.jfa_plan_build(prob, off, off, None, J.JFA_PASS_DQ, W_)
        wp, tiles = OP.plan_dq(lens, lens, 2, W_, broadcast_q=False, block_m=FWD_BM,
                               block_n=FWD_BN, causal=causal, window=window)
        assert np.array_equal(hp.tiles, tiles), (trial, "dq")


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
@pytest.mark.parametrize("workers", [1, 7, 256])
def test_cpp_natural_plan_equals_oracle(cfg, workers):
    """The unsorted round-robin ablation plans, bit for bit, every pass."""
    w, lens, mask = _lengths_only(cfg)
    kv_off = W.offsets_of(lens)
    q_off = None if w.broadcast_q else kv_off
    mq, mk = (mask.shape[1], mask.shape[2]) if mask is not None else (0, 0)
    prob = J.Problem(batch=w.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0, causal=w.causal,
                     mask_q_blocks=mq, mask_kv_blocks=mk, softmax_scale=w.scale)
    q_lens = [w.lq] * w.batch if w.broadcast_q else lens
    for pass_, bm, bn in ((OP.FWD, FWD_BM, FWD_BN), (OP.BWD, BWD_BM, BWD_BN)):
        hp = J.jfa_plan_build(prob, q_off, kv_off, mask, pass_ | J.JFA_PLAN_NATURAL, workers)
        wp, tiles = OP.plan(q_lens, lens, w.heads, workers, pass_, block_m=bm, block_n=bn,
                            causal=w.causal, block_mask=mask, natural=True)
        assert hp.info.pass_ == pass_
        assert np.array_equal(hp.worker_ptr, wp) and np.array_equal(hp.tiles, tiles), pass_
    hp = J.jfa_plan_build(prob, q_off, kv_off, mask, J.JFA_PASS_DQ | J.JFA_PLAN_NATURAL, workers)
    wp, tiles = OP.plan_dq(q_lens, lens, w.heads, workers, broadcast_q=w.broadcast_q, lq=w.lq,
                           block_m=FWD_BM, block_n=FWD_BN, causal=w.causal, block_mask=mask,
                           natural=True)
    assert hp.info.pass_ == J.JFA_PASS_DQ
    assert np.array_equal(hp.worker_ptr, wp) and np.array_equal(hp.tiles, tiles)


def test_cpp_natural_plan_is_static():
    prob = J.Problem(2, 1, 64, True, lq=8, softmax_scale=0.1)
    with pytest.raises(J.JfaError) as e:
        J.jfa_plan_build(prob, None, [0, 3, 5], None,
                         J.JFA_PASS_FWD | J.JFA_PLAN_DYNAMIC | J.JFA_PLAN_NATURAL, 4)
    assert e.value.status == J.JFA_ERR_INVALID_ARG
