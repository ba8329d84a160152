"""Pins of the oracle's MXFP8 encoder (CPU only).

E4M3 decoding and round-to-nearest-even encoding are checked against
PyTorch's float8_e4m3fn conversions (a library implementation of the same OCP
format) over every code and over random and tie values; the block exponent
rule and the block layout (32 along d for Q/K, 32 keys of one sequence for V)
against values built by hand.
"""
import numpy as np
import pytest
import torch

from oracle import mx


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.nanmax(got) == 448.0 and np.nanmin(got) == -448.0
    assert got[1] == 2.0 ** -9 and got[8] == 2.0 ** -6 and got[0x38] == 1.0


def test_encode_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.standard_normal(5000).astype(np.float32) * 1e-3,       # subnormal range
        np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10,
                    1.0625, 1.1875, 272.0, 1.03125, 1.09375, 15.5, 7.5]),  # ties and edges
    ])
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_encode_clamps_and_round_trips():
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = mx.e4m3_decode(finite)
    assert np.array_equal(mx.e4m3_decode(mx.e4m3_encode(vals)), vals)
    assert list(mx.e4m3_encode([449.0, 479.0, 1e9, -600.0])) == [0x7E, 0x7E, 0x7E, 0xFE]


@pytest.mark.parametrize("k", [-20, -3, 0, 1, 7, 12])
def test_block_exponent_rule(k):
    # amax in [2^k, 2^(k+1)) gives e = k - 8, so amax / 2^e lies in [256, 512)
    for amax in (2.0 ** k, 2.0 ** k * 1.5, 2.0 ** (k + 1) * (1 - 2 ** -12)):
        assert mx.block_exponent(amax) == k - 8
    assert mx.block_exponent(0.0) == -127
    assert mx.block_exponent(2.0 ** -140) == -127
    assert mx.block_exponent(2.0 ** 130) == 122


def test_quantize_rows_blocks_and_error_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((5, 3, 128)) * np.exp(rng.standard_normal((5, 3, 1)) * 3)).astype(np.float32)
    x = x.astype(np.float64)
    x[2, 1, 32:64] = 0.0                                   # an all-zero block
    codes, scales = mx.quantize_rows(x)
    assert codes.shape == (5, 3, 128) and scales.shape == (3, 5, 4)
    assert scales[1, 2, 1] == 0
    y = mx.dequantize_rows(codes, scales)
    for r in range(5):
        for h in range(3):
            for blk in range(4):
                xb = x[r, h, 32 * blk:32 * blk + 32]
                yb = y[r, h, 32 * blk:32 * blk + 32]
                e = int(scales[h, r, blk]) - 127
                assert e == mx.block_exponent(np.abs(xb).max())
                # each element: E4M3 rounding of x / 2^e (clamped at 448)
                t = np.minimum(np.abs(xb) / 2.0 ** e, 448.0)
                err = np.abs(np.abs(yb) / 2.0 ** e - t)
                assert np.all(err <= np.maximum(t * 2.0 ** -4, 2.0 ** -10) + 1e-12)


def test_mx_block_offsets():
    off = np.cumsum([0, 0, 1, 32, 33, 64])
    assert list(mx.mx_block_offsets(off)) == [0, 0, 1, 2, 4, 6]


def test_quantize_v_blocks_stay_inside_sequences():
    rng = np.random.default_rng(2)
    lens = [33, 5, 64, 0, 40]
    off = np.concatenate([[0], np.cumsum(lens)])
    v = rng.standard_normal((off[-1], 2, 64))
    v[32] *= 1000.0                           # last key of sequence 0: its own one-key block
    codes, scales = mx.quantize_v(v, off)
    boff = mx.mx_block_offsets(off)
    assert scales.shape == (2, int(boff[-1]), 64)
    y = mx.dequantize_v(codes, scales, off)
    for b in range(len(lens)):
        for j, s0 in enumerate(range(off[b], off[b + 1], 32)):
            s1 = min(s0 + 32, off[b + 1])
            e = scales[:, boff[b] + j, :].astype(int) - 127
            assert np.array_equal(e, mx.block_exponent(np.abs(v[s0:s1]).max(axis=0)))
    # the scaled-up key did not coarsen sequence 1's first block
    assert np.abs(y[33:38] - v[33:38]).max() <= 2.0 ** -4 * np.abs(v[33:38]).max() * 2
    assert np.abs(y[32] - v[32]).max() <= 2.0 ** -4 * np.abs(v[32]).max() * 2


def _small(broadcast):
    import workloads as W
    rng = np.random.default_rng(7)
    lens = np.array([5, 0, 70, 33])
    off = W.offsets_of(lens)
    H, D = 2, 64
    k = rng.standard_normal((off[-1], H, D))
    v = rng.standard_normal((off[-1], H, D))
    if broadcast:
        q = rng.standard_normal((9, H, D))
        do = rng.standard_normal((9 * len(lens), H, D))
        return q, k, v, do, off, None
    q = rng.standard_normal((off[-1], H, D))
    do = rng.standard_normal((off[-1], H, D))
    return q, k, v, do, off, off


@pytest.mark.parametrize("broadcast", [True, False])
def test_dq_mx_without_quantisation_is_the_attention_gradient(broadcast):
    """With every encoding the identity (the operands undecoded) and the
    forward's own O and LSE, the MXFP8 dQ definition is the attention dQ and
    delta of oracle.attention.backward; dQ is linear in the K used for its
    last product and blind to it in S."""
    from oracle import attention as A
    q, k, v, do, off, qoff = _small(broadcast)
    kw = dict(scale=0.125, broadcast_q=broadcast, q_offsets=qoff, causal=not broadcast)
    o, lse = A.forward(q, k, v, off, **kw)
    dq_ref, _, _, delta_ref = A.backward(q, k, v, do, off, **kw)
    dq, delta, abs_sum, floor_sum, acc_sum = mx.dq_mx(q, k, v, do, k, do, o, lse, off, **kw)
    assert np.allclose(dq, dq_ref, rtol=0, atol=1e-12) and np.allclose(delta, delta_ref, atol=1e-12)
    assert np.all(abs_sum >= np.abs(dq) - 1e-12) and np.all(floor_sum >= 0)
    # |dP - delta| <= sum_d |do v| + sum_d |do o|, so the accumulation term
    # dominates the one of dS itself
    assert np.all(acc_sum >= abs_sum - 1e-12)
    dq2, *_ = mx.dq_mx(q, k, v, do, 2 * k, do, o, lse, off, **kw)
    assert np.allclose(dq2, 2 * dq, rtol=0, atol=1e-12)


@pytest.mark.parametrize("broadcast", [True, False])
def test_dkdv_mx_without_quantisation_is_the_attention_gradient(broadcast):
    """With every encoding the identity and the forward's own O and LSE, the
    MXFP8 dK/dV definition is the attention dK and dV of
    oracle.attention.backward; dV is linear in the dO of its product and
    blind to the Q of dK's, and dK the other way round (which pins which
    encoding each product takes); the rounding-bound terms dominate |dK|,
    |dV|."""
    from oracle import attention as A
    q, k, v, do, off, qoff = _small(broadcast)
    kw = dict(scale=0.125, broadcast_q=broadcast, q_offsets=qoff, causal=not broadcast)
    o, lse = A.forward(q, k, v, off, **kw)
    _, dk_ref, dv_ref, _ = A.backward(q, k, v, do, off, **kw)
    dk, dv, pa, pf, ka, kf, kacc = mx.dkdv_mx(q, k, v, do, q, do, do, o, lse, off, **kw)
    assert np.allclose(dk, dk_ref, rtol=0, atol=1e-12) and np.allclose(dv, dv_ref, rtol=0, atol=1e-12)
    assert np.all(pa >= np.abs(dv) - 1e-12) and np.all(pf >= pa - 1e-12)
    assert np.all(ka >= np.abs(dk) - 1e-12) and np.all(kf >= 0) and np.all(kacc >= ka - 1e-12)
    dk2, dv2, *_ = mx.dkdv_mx(q, k, v, do, 3 * q, 2 * do, do, o, lse, off, **kw)
    assert np.allclose(dv2, 2 * dv, rtol=0, atol=1e-12) and np.allclose(dk2, 3 * dk, rtol=0, atol=1e-12)
