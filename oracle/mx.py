"""MXFP8 (microscaling FP8) encoding -- oracle (test infrastructure only).

The pages describe an MXFP8 version of the kernel: its matrix products run in
microscaling precision, with P quantised to FP8 on the fly ([radar] section
"The turning point"). They give no block size, element or scale format. The
plainest reading is the OCP Microscaling (MX) format MXFP8: FP8 E4M3 elements
(OCP encoding: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, 0x7F / 0xFF are NaN, largest finite 448) sharing one E8M0 scale
(a power of two 2^(c-127), code c in 0..254) per block of 32 consecutive
elements along the contraction dimension of each product. A block x_1..x_32
is encoded as

  e     = floor(log2(max_i |x_i|)) - 8      (8: exponent of E4M3's largest
                                             power of two; clamped to
                                             [-127, 127]; an all-zero block
                                             takes -127)
  q_i   = E4M3(x_i / 2^e)                    (round to nearest, ties to even,
                                             magnitudes above 448 clamped)

and decodes to q_i * 2^e. The blocks run along d for Q and K (the d of
S = Q K^T), and along the keys of each sequence for V (the keys of O = P V):
32 consecutive keys of one sequence, the last block of a sequence possibly
shorter, never spanning two sequences.

Layouts (uint8): Q codes [rows, H, D], Q scales [H, rows, D/32]; K likewise;
V codes [T_k, H, D], V scales [H, NB, D] with NB = sum_b ceil(L_b / 32), the
blocks of sequence b starting at mx_block_offsets(kv_offsets)[b].

The attention the MXFP8 variant computes is then softmax attention on the
decoded Q, K, V (``oracle.attention`` on the decoded tensors). P's own FP8
quantisation happens inside the kernel, in whichever order its online softmax
visits the keys; the oracle keeps P exact and the tests bound the difference
(every P element is rounded to E4M3 with a relative error of at most 2^-4,
or, below E4M3's normal range, an absolute error of at most 2^-18).

The same page reports the MXFP8 version's backward at parity on dense shapes
without describing it. ``dq_mx`` and ``dkdv_mx`` are the plainest reading
for its two passes. ``dq_mx``, the dQ pass:
every product of the FlashAttention dQ computation on MXFP8 operands, each
encoded along that product's contraction dimension (Q, K, dO, V along d for
S and dP; K along the keys of its sequence for dQ = dS K), with delta from
the bf16 dO and O. The kernel rounds dS to E4M3 on the fly; the oracle keeps
it exact and the tests bound the rounding. ``dkdv_mx``, the dK/dV pass: the
same S and dP, then dV = P^T dO and dK = dS^T Q with Q and dO encoded along
their rows (32-row blocks of one sequence, never spanning two, as V along
keys: ``quantize_v`` with row offsets); the kernel rounds P and dS to E4M3.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8        # exponent of the largest power of two E4M3 holds
E8M0_BIAS = 127


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3 codes (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    out = sign * mag
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(y) -> np.ndarray:
    """E4M3 codes of float64 values: magnitudes above 448 are clamped to 448,
    the rest rounded to the nearest E4M3 value, ties to the even mantissa."""
    y = np.asarray(y, dtype=np.float64)
    neg = np.signbit(y)
    a = np.minimum(np.abs(y), E4M3_MAX)
    # spacing of E4M3 values around a: 2^(e-3) for a in [2^e, 2^(e+1)), e >= -6;
    # 2^-9 in the subnormal range below 2^-6
    _, ex = np.frexp(np.where(a > 0, a, 1.0))          # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    step = np.ldexp(1.0, e - 3)
    q = np.rint(a / step) * step                        # exact: a is a short binary fraction
    q = np.where(a > 0, q, 0.0)
    # back to fields: q is on the E4M3 grid (rounding up may reach 2^(e+1))
    _, qx = np.frexp(np.where(q > 0, q, 1.0))
    qe = qx - 1
    normal = (q >= 2.0 ** -6)
    exp_field = np.where(normal, qe + 7, 0)
    man = np.where(normal, q / np.ldexp(1.0, qe) - 1.0, q / 2.0 ** -6) * 8.0
    man = np.rint(man).astype(np.int64)
    code = (exp_field.astype(np.int64) << 3) | man
    code = np.where(q > 0, code, 0)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def block_exponent(amax) -> np.ndarray:
    """Shared exponent e of a block with largest magnitude amax (see above)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))   # floor(log2(amax)) = ex - 1
    e = np.where(amax > 0, ex - 1 - E4M3_EMAX, -E8M0_BIAS)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def _encode_blocks(x):
    """x [..., 32] -> (codes [..., 32], scale codes [...])."""
    e = block_exponent(np.abs(x).max(axis=-1))
    codes = e4m3_encode(np.ldexp(x, -e[..., None]))
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def quantize_rows(x):
    """Q or K [rows, H, D] (D a multiple of 32) -> codes [rows, H, D], scales
    [H, rows, D/32]: one block per 32 consecutive d of a (row, head)."""
    x = np.asarray(x, dtype=np.float64)
    rows, H, D = x.shape
    codes, sc = _encode_blocks(x.reshape(rows, H, D // BLOCK, BLOCK))
    return codes.reshape(rows, H, D), np.ascontiguousarray(sc.transpose(1, 0, 2))


def dequantize_rows(codes, scales):
    rows, H, D = codes.shape
    s = np.ldexp(1.0, scales.astype(np.int64) - E8M0_BIAS)             # [H, rows, D/32]
    s = np.repeat(s.transpose(1, 0, 2), BLOCK, axis=2)                  # [rows, H, D]
    return e4m3_decode(codes) * s


def mx_block_offsets(kv_offsets) -> np.ndarray:
    """First V scale block of each sequence: prefix sums of ceil(L_b / 32)."""
    lens = np.diff(np.asarray(kv_offsets, dtype=np.int64))
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(-(-lens // BLOCK))
    return out.astype(np.int32)


def quantize_v(v, kv_offsets):
    """V [T_k, H, D] -> codes [T_k, H, D], scales [H, NB, D]: one block per 32
    consecutive keys of a sequence (the last one possibly shorter) per (head, d)."""
    v = np.asarray(v, dtype=np.float64)
    T, H, D = v.shape
    boff = mx_block_offsets(kv_offsets)
    codes = np.zeros((T, H, D), dtype=np.uint8)
    scales = np.zeros((H, int(boff[-1]), D), dtype=np.uint8)
    for b in range(len(kv_offsets) - 1):
        k0, k1 = int(kv_offsets[b]), int(kv_offsets[b + 1])
        for j, s0 in enumerate(range(k0, k1, BLOCK)):
            s1 = min(s0 + BLOCK, k1)
            blk = v[s0:s1]                                   # [n, H, D]
            e = block_exponent(np.abs(blk).max(axis=0))      # [H, D]
            codes[s0:s1] = e4m3_encode(np.ldexp(blk, -e[None]))
            scales[:, boff[b] + j, :] = (e + E8M0_BIAS).astype(np.uint8)
    return codes, scales


def dequantize_v(codes, scales, kv_offsets):
    T, H, D = codes.shape
    boff = mx_block_offsets(kv_offsets)
    out = e4m3_decode(codes)
    for b in range(len(kv_offsets) - 1):
        k0, k1 = int(kv_offsets[b]), int(kv_offsets[b + 1])
        for j, s0 in enumerate(range(k0, k1, BLOCK)):
            s1 = min(s0 + BLOCK, k1)
            s = np.ldexp(1.0, scales[:, boff[b] + j, :].astype(np.int64) - E8M0_BIAS)   # [H, D]
            out[s0:s1] *= s[None]
    return out


def dq_mx(q_d, k_d, v_d, do_d, k_keys, do, o, lse, kv_offsets, *, scale, broadcast_q,
          q_offsets=None, causal=False, block_mask=None, window=None):
    """What the MXFP8 dQ pass computes ([radar] section "The turning point":
    the MXFP8 version's backward; the reading is in the module header), with
    dS kept exact (the kernel rounds it to E4M3 per (row, 32-key tile);
    tests bound that rounding).

    Per sequence and head, with every operand float64 and already decoded:
      S     = scale * q_d k_d^T          (Q and K encoded along d)
      P     = exp(S - lse) on visible keys, 0 elsewhere (lse given: the
              forward's)
      delta = rowsum(do * o)             (the bf16 dO and O)
      dP    = do_d v_d^T                 (dO and V encoded along d)
      dS    = P (dP - delta)
      dQ   += scale * dS k_keys          (K encoded along keys)
    the broadcast dQ summing over sequences. Returns (dq, delta, abs_sum,
    floor_sum, acc_sum): abs_sum = scale * |dS| |k_keys| and floor_sum =
    scale * max_j |dS_ij| * sum_j |k_keys_j| (per sequence), the two terms a
    bound on dS's rounding needs, and acc_sum = scale * (P (|do_d| |v_d|^T +
    sum_d |do o|)) |k_keys|, the magnitudes that dP and delta sum over d: a
    kernel forms both as fp32 sums of D terms, whose error (up to D 2^-24
    times these magnitudes) is not relative to dS = P (dP - delta) itself
    and dominates it where dP and delta nearly cancel."""
    import oracle.attention as A
    B = len(kv_offsets) - 1
    H = k_d.shape[1]
    if broadcast_q:
        lq = q_d.shape[0]
        t_q = B * lq
    else:
        t_q = int(q_offsets[-1])
    dq = np.zeros(q_d.shape)
    abs_sum = np.zeros(q_d.shape)
    floor_sum = np.zeros(q_d.shape)
    acc_sum = np.zeros(q_d.shape)
    delta = np.zeros((H, t_q))
    for b in range(B):
        k0, k1 = int(kv_offsets[b]), int(kv_offsets[b + 1])
        if broadcast_q:
            qs, os_ = slice(0, lq), slice(b * lq, (b + 1) * lq)
        else:
            qs = os_ = slice(int(q_offsets[b]), int(q_offsets[b + 1]))
        n_rows = qs.stop - qs.start
        vis = A.visibility(n_rows, k1 - k0, causal=causal, window=window,
                           mask_b=None if block_mask is None else block_mask[b])
        for h in range(H):
            lse_b = lse[h, os_]
            fin = np.isfinite(lse_b)
            s = scale * (q_d[qs, h] @ k_d[k0:k1, h].T)
            p = np.where(vis & fin[:, None], np.exp(s - np.where(fin, lse_b, 0.0)[:, None]), 0.0)
            dl = np.sum(do[os_, h] * o[os_, h], axis=1)
            ds = p * (do_d[os_, h] @ v_d[k0:k1, h].T - dl[:, None])
            kk = k_keys[k0:k1, h]
            dq[qs, h] += scale * (ds @ kk)
            abs_sum[qs, h] += scale * (np.abs(ds) @ np.abs(kk))
            amax = np.abs(ds).max(axis=1, initial=0.0)
            floor_sum[qs, h] += scale * amax[:, None] * np.abs(kk).sum(axis=0)[None, :]
            mag = np.abs(do_d[os_, h]) @ np.abs(v_d[k0:k1, h]).T + np.sum(np.abs(do[os_, h] * o[os_, h]), axis=1)[:, None]
            acc_sum[qs, h] += scale * ((p * mag) @ np.abs(kk))
            delta[h, os_] = dl
    return dq, delta, abs_sum, floor_sum, acc_sum


def dkdv_mx(q_d, k_d, v_d, do_d, q_r, do_r, do, o, lse, kv_offsets, *, scale, broadcast_q,
            q_offsets=None, causal=False, block_mask=None, window=None):
    """What the MXFP8 dK/dV pass computes ([radar] section "The turning point":
    the MXFP8 version's backward; the reading is in the module header and
    below), with P and dS kept exact (the kernel rounds P to E4M3 with the
    fixed block scale 2^-8 and dS with one scale per (key, 32-row block);
    tests bound that rounding).

    Every product of the FlashAttention dK/dV computation on MXFP8 operands,
    each encoded along that product's contraction dimension: Q, K, dO, V
    along d for S and dP; Q and dO along their rows (32-row blocks of one
    sequence, as V is encoded along keys for the forward) for dK = dS^T Q and
    dV = P^T dO. Per sequence and head, every operand float64 and decoded:
      S     = scale * q_d k_d^T
      P     = exp(S - lse) on visible keys, 0 elsewhere (lse given: the forward's)
      delta = rowsum(do * o)             (the bf16 dO and O)
      dP    = do_d v_d^T
      dS    = P (dP - delta)
      dV    = P^T do_r
      dK    = scale * dS^T q_r
    Returns (dk, dv, dv_p_abs, dv_p_floor, dk_abs, dk_floor, dk_acc): dv_p_abs
    = P^T |do_r| and dv_p_floor = vis^T |do_r| (the terms of P's rounding
    bound), dk_abs = scale |dS|^T |q_r| and dk_floor = scale * (max_i |dS_ij|)
    * sum_i |q_r_i| per key (those of dS's), and dk_acc = scale * (P (|do_d|
    |v_d|^T + sum_d |do o|))^T |q_r|, the magnitudes behind the fp32 sums
    that form dP and delta (as for dq_mx's acc_sum)."""
    import oracle.attention as A
    B = len(kv_offsets) - 1
    T_k, H, D = k_d.shape
    dk = np.zeros((T_k, H, D))
    dv = np.zeros((T_k, H, D))
    dv_p_abs = np.zeros((T_k, H, D))
    dv_p_floor = np.zeros((T_k, H, D))
    dk_abs = np.zeros((T_k, H, D))
    dk_floor = np.zeros((T_k, H, D))
    dk_acc = np.zeros((T_k, H, D))
    lq = q_d.shape[0] if broadcast_q else None
    for b in range(B):
        k0, k1 = int(kv_offsets[b]), int(kv_offsets[b + 1])
        if broadcast_q:
            qs, os_ = slice(0, lq), slice(b * lq, (b + 1) * lq)
        else:
            qs = os_ = slice(int(q_offsets[b]), int(q_offsets[b + 1]))
        n_rows = qs.stop - qs.start
        if n_rows == 0 or k1 == k0:
            continue
        vis = A.visibility(n_rows, k1 - k0, causal=causal, window=window,
                           mask_b=None if block_mask is None else block_mask[b])
        for h in range(H):
            lse_b = lse[h, os_]
            fin = np.isfinite(lse_b)
            visf = vis & fin[:, None]
            s = scale * (q_d[qs, h] @ k_d[k0:k1, h].T)
            p = np.where(visf, np.exp(s - np.where(fin, lse_b, 0.0)[:, None]), 0.0)
            dl = np.sum(do[os_, h] * o[os_, h], axis=1)
            ds = p * (do_d[os_, h] @ v_d[k0:k1, h].T - dl[:, None])
            dv[k0:k1, h] = p.T @ do_r[os_, h]
            dk[k0:k1, h] = scale * (ds.T @ q_r[qs, h])
            dv_p_abs[k0:k1, h] = p.T @ np.abs(do_r[os_, h])
            dv_p_floor[k0:k1, h] = visf.astype(np.float64).T @ np.abs(do_r[os_, h])
            dk_abs[k0:k1, h] = scale * (np.abs(ds).T @ np.abs(q_r[qs, h]))
            amax = np.abs(ds).max(axis=0, initial=0.0)
            dk_floor[k0:k1, h] = scale * amax[:, None] * np.abs(q_r[qs, h]).sum(axis=0)[None, :]
            mag = np.abs(do_d[os_, h]) @ np.abs(v_d[k0:k1, h]).T + np.sum(np.abs(do[os_, h] * o[os_, h]), axis=1)[:, None]
            dk_acc[k0:k1, h] = scale * ((p * mag).T @ np.abs(q_r[qs, h]))
    return dk, dv, dv_p_abs, dv_p_floor, dk_abs, dk_floor, dk_acc
