"""Exact jagged softmax attention in float64 -- oracle (test infrastructure only).

What is computed. The pages say the kernel applies the FlashAttention algorithm
directly to packed Q/K/V tensors whose sequence boundaries sit in an offsets
array, never materialising a padded token ([bites] section "Why attention in
GEM needed a rewrite"; [clarity] third paragraph). FlashAttention is an exact
reformulation of softmax attention, so the oracle is softmax attention itself,
written per sequence and head with dense fp64 matrix products:

  s_ij  = scale * <q_i, k_j>                  for the keys j visible to row i
  LSE_i = ln sum_{j visible} exp(s_ij)         (natural log of scaled scores)
  P_ij  = exp(s_ij - LSE_i)
  o_i   = sum_j P_ij v_j

Backward, for the loss L = sum(dO * O):
  delta_i = <dO_i, o_i>
  dV_j    = sum_i P_ij dO_i
  dP_ij   = <dO_i, v_j>
  dS_ij   = P_ij (dP_ij - delta_i)
  dq_i    = scale * sum_j dS_ij k_j
  dk_j    = scale * sum_i dS_ij q_i

Broadcast-Q: one dense Q is shared by every sequence and its gradient is the
sum over the whole batch ([clarity] second paragraph; [bites] section
"Optimizations layered on top"). Output rows of sequence b are b*Lq + i.

Visibility. All keys of the row's own sequence; with ``causal`` only keys
j <= i (local indices, Q and KV share offsets); with a block mask only keys
whose 128-key block is kept for the row's 128-row Q tile ([radar] section "The
turning point": the block-sparse variant iterates only over selected blocks);
with a sliding window (left, right) only keys i - left <= j <= i + right, a
bound being None when absent (the pages name sliding-window attention as one
of the variants the kernel serves -- [clarity] fourth paragraph, [bites] "Why
attention in GEM needed a rewrite", [radar] introduction -- without defining it; this band of local
indices is the usual meaning, and causal is the band (None, 0)).
A row with no visible key has O = 0, LSE = -inf and contributes no gradient.

Inputs are float64 arrays holding bf16-representable values:
q [Lq|T_q, H, D], k/v [T_k, H, D], dO [T_q, H, D]; offsets int [B+1].
LSE and delta are returned as [H, T_q].
"""
from __future__ import annotations

import numpy as np

MASK_BLOCK = 128


def _q_rows(b, kv_offsets, q_offsets, lq, broadcast_q):
    """(slice into q, slice into the output rows) of sequence b."""
    if broadcast_q:
        return slice(0, lq), slice(b * lq, (b + 1) * lq)
    lo, hi = int(q_offsets[b]), int(q_offsets[b + 1])
    return slice(lo, hi), slice(lo, hi)


def visibility(n_rows, n_keys, *, causal=False, window=None, mask_b=None, rows=None):
    """bool [len(rows), n_keys]: key j visible to local query row i."""
    i = np.arange(n_rows) if rows is None else np.asarray(rows)
    j = np.arange(n_keys)
    vis = np.ones((len(i), n_keys), dtype=bool)
    if causal:
        vis &= j[None, :] <= i[:, None]
    if window is not None:
        left, right = window
        if left is not None:
            vis &= j[None, :] >= i[:, None] - left
        if right is not None:
            vis &= j[None, :] <= i[:, None] + right
    if mask_b is not None:
        vis &= mask_b[(i // MASK_BLOCK)[:, None], (j // MASK_BLOCK)[None, :]].astype(bool)
    return vis


def _softmax_stats(s, vis):
    """LSE per row and P, for scores s with invisible entries excluded."""
    s = np.where(vis, s, -np.inf)
    row_max = s.max(axis=1, initial=-np.inf)
    finite = np.isfinite(row_max)
    shift = np.where(finite, row_max, 0.0)
    e = np.exp(s - shift[:, None])          # exp(-inf) = 0 for invisible keys
    tot = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, shift + np.log(tot), -np.inf)
    p = np.where(finite[:, None], e / np.where(finite, tot, 1.0)[:, None], 0.0)
    return lse, p


def _problem(q, kv_offsets, q_offsets, broadcast_q):
    B = len(kv_offsets) - 1
    if broadcast_q:
        lq = q.shape[0]
        t_q = B * lq
    else:
        lq = 0
        t_q = int(q_offsets[-1])
    return B, lq, t_q


def forward(q, k, v, kv_offsets, *, scale, broadcast_q, q_offsets=None, causal=False,
            block_mask=None, seqs=None, heads=None, window=None):
    """O [T_q,H,D] and LSE [H,T_q] (float64). Rows of sequences not in ``seqs``
    (default: all) stay 0 / -inf."""
    B, lq, t_q = _problem(q, kv_offsets, q_offsets, broadcast_q)
    H, D = k.shape[1], k.shape[2]
    o = np.zeros((t_q, H, D))
    lse = np.full((H, t_q), -np.inf)
    for b in (range(B) if seqs is None else seqs):
        qs, os_ = _q_rows(b, kv_offsets, q_offsets, lq, broadcast_q)
        ks = slice(int(kv_offsets[b]), int(kv_offsets[b + 1]))
        n_rows, n_keys = qs.stop - qs.start, ks.stop - ks.start
        vis = visibility(n_rows, n_keys, causal=causal, window=window,
                         mask_b=None if block_mask is None else block_mask[b])
        for h in (range(H) if heads is None else heads):
            s = scale * (q[qs, h, :] @ k[ks, h, :].T)
            l, p = _softmax_stats(s, vis)
            o[os_, h, :] = p @ v[ks, h, :]
            lse[h, os_] = l
    return o, lse


def forward_rows(q, k, v, kv_offsets, b, h, rows, *, scale, broadcast_q, q_offsets=None,
                 causal=False, block_mask=None, window=None):
    """O [len(rows), D] and LSE [len(rows)] for local query rows of (b, h) only."""
    B, lq, _ = _problem(q, kv_offsets, q_offsets, broadcast_q)
    qs, _ = _q_rows(b, kv_offsets, q_offsets, lq, broadcast_q)
    ks = slice(int(kv_offsets[b]), int(kv_offsets[b + 1]))
    rows = np.asarray(rows)
    vis = visibility(qs.stop - qs.start, ks.stop - ks.start, causal=causal, window=window,
                     mask_b=None if block_mask is None else block_mask[b], rows=rows)
    s = scale * (q[qs.start + rows, h, :] @ k[ks, h, :].T)
    l, p = _softmax_stats(s, vis)
    return p @ v[ks, h, :], l


def backward(q, k, v, do, kv_offsets, *, scale, broadcast_q, q_offsets=None, causal=False,
             block_mask=None, seqs=None, heads=None, window=None, o=None):
    """dQ (shape of q), dK, dV [T_k,H,D] and delta [H,T_q], all float64.

    With ``seqs`` given, only those sequences contribute (their dK/dV rows are
    exact; a broadcast dQ is then the partial sum over ``seqs``). ``o`` is the
    forward output as a backward receives it ([T_q,H,D], e.g. as stored in
    bf16): delta_i = <dO_i, o_i> is formed from it, everything else from the
    exact softmax; by default it is the exact O, and the result the exact
    gradients."""
    B, lq, t_q = _problem(q, kv_offsets, q_offsets, broadcast_q)
    H, D = k.shape[1], k.shape[2]
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    delta = np.zeros((H, t_q))
    for b in (range(B) if seqs is None else seqs):
        qs, os_ = _q_rows(b, kv_offsets, q_offsets, lq, broadcast_q)
        ks = slice(int(kv_offsets[b]), int(kv_offsets[b + 1]))
        n_rows, n_keys = qs.stop - qs.start, ks.stop - ks.start
        vis = visibility(n_rows, n_keys, causal=causal, window=window,
                         mask_b=None if block_mask is None else block_mask[b])
        for h in (range(H) if heads is None else heads):
            qb, kb, vb, dob = q[qs, h, :], k[ks, h, :], v[ks, h, :], do[os_, h, :]
            _, p = _softmax_stats(scale * (qb @ kb.T), vis)
            ob = p @ vb if o is None else o[os_, h, :]
            dl = np.sum(dob * ob, axis=1)
            dp = dob @ vb.T
            ds = p * (dp - dl[:, None])
            dq[qs, h, :] += scale * (ds @ kb)
            dk[ks, h, :] = scale * (ds.T @ qb)
            dv[ks, h, :] = p.T @ dob
            delta[h, os_] = dl
    return dq, dk, dv, delta


def delta_slack(q, k, v, do, kv_offsets, *, scale, broadcast_q, q_offsets=None, causal=False,
                block_mask=None, window=None):
    """Element-wise bounds (dQ, dK; float64, shapes of q and k) on how far
    the gradients move when delta_i = <dO_i, o_i> is formed from O as the
    forward stores it rather than from the exact O.

    O is stored in bf16 (the layout the pages fix for the kernel's tensors)
    and a kernel forms it from probabilities rounded to bf16 for its matrix
    products, so an element of the stored O may be off by up to 2^-9 sum_j
    p_ij |v_jd| (the rounded probabilities) plus 2^-9 |o_id| (the rounding of
    O itself); both are taken at 2^-8 here. Then |d delta_i| <= eps_i =
    sum_d |dO_id| * 2^-8 (sum_j p_ij |v_jd| + |o_id|), dS_ij moves by
    p_ij d delta_i, and so dq_i by at most scale * eps_i * sum_j p_ij |k_j|
    and dk_j by at most scale * sum_i p_ij eps_i |q_i| (summed over the batch
    for a broadcast Q, as dQ is). Where dP_ij - delta_i nearly cancels this
    is the larger part of the gradients' error. Test infrastructure only."""
    B, lq, t_q = _problem(q, kv_offsets, q_offsets, broadcast_q)
    H = k.shape[1]
    sq = np.zeros(q.shape)
    sk = np.zeros(k.shape)
    for b in range(B):
        qs, os_ = _q_rows(b, kv_offsets, q_offsets, lq, broadcast_q)
        ks = slice(int(kv_offsets[b]), int(kv_offsets[b + 1]))
        vis = visibility(qs.stop - qs.start, ks.stop - ks.start, causal=causal, window=window,
                         mask_b=None if block_mask is None else block_mask[b])
        for h in range(H):
            qb, kb, vb, dob = q[qs, h, :], k[ks, h, :], v[ks, h, :], do[os_, h, :]
            _, p = _softmax_stats(scale * (qb @ kb.T), vis)
            ob = p @ vb
            eps = 2.0 ** -8 * np.sum(np.abs(dob) * (p @ np.abs(vb) + np.abs(ob)), axis=1)
            sq[qs, h, :] += scale * eps[:, None] * (p @ np.abs(kb))
            sk[ks, h, :] = scale * ((p * eps[:, None]).T @ np.abs(qb))
    return sq, sk


def broadcast_dq_rows(q, k, v, do, kv_offsets, h, rows, *, scale, block_mask=None):
    """Rows of the batch-summed broadcast dQ for head h: sum over every sequence
    b of scale * sum_j dS_b[i, j] k_j. Each row needs only its own row of the
    scores of every sequence, so this stays cheap at full size."""
    B = len(kv_offsets) - 1
    lq = q.shape[0]
    rows = np.asarray(rows)
    out = np.zeros((len(rows), q.shape[2]))
    for b in range(B):
        ks = slice(int(kv_offsets[b]), int(kv_offsets[b + 1]))
        vis = visibility(lq, ks.stop - ks.start,
                         mask_b=None if block_mask is None else block_mask[b], rows=rows)
        kb, vb = k[ks, h, :], v[ks, h, :]
        _, p = _softmax_stats(scale * (q[rows, h, :] @ kb.T), vis)
        dob = do[b * lq + rows, h, :]
        dl = np.sum(dob * (p @ vb), axis=1)
        ds = p * (dob @ vb.T - dl[:, None])
        out += scale * (ds @ kb)
    return out
