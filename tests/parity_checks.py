"""Whole-tensor checks of a forward/backward result that hold at any size.

Used by the full-size GPU parity tests, which compare only sampled sequences
with the oracle element by element, so that every sequence and head is still
checked by identities the mathematics fixes. With P_ij = exp(s_ij - LSE_i)
over the keys j that row i sees, O_i = sum_j P_ij v_j, dV_j = sum_i P_ij dO_i,
dS_ij = P_ij (dP_ij - delta_i), dK_j = scale sum_i dS_ij q_i and
dq_i = scale sum_j dS_ij k_j (per sequence; a broadcast Q's dQ sums them):

  I0  no NaN survives in any output (the outputs are NaN-filled before the
      run, so a tile that was never computed leaves NaN behind);
  I1  sum_j dK_j = 0, since sum_j dS_ij = delta_i - delta_i sum_j P_ij = 0;
  I2  sum_j dV_j = sum_i dO_i over the rows that see a key (sum_j P_ij = 1);
  I3  sum_j dV_j v_j^T = sum_i dO_i O_i^T  (both are sum_ij P_ij dO_i v_j^T);
  I4  sum_j dK_j k_j^T = sum_i q_i dq_i^T  (both are scale sum_ij dS_ij q_i
      k_j^T): ties each sequence's dK, from the dK/dV kernel, to dQ, from the
      dQ pass; with a broadcast Q, per head over the whole batch;
  I5  every O element lies inside the [min, max] of the V rows its row sees
      (O_i is a convex combination of them).
I1-I3 hold per (sequence, head), I4 per (sequence, head) or per head.

Tolerances. The GPU rounds P, dS, O, dK, dV to bf16 (unit roundoff
u = 2^-8) and accumulates in fp32, so each term t of a sum above carries an
error of about u |t| (half of it on average) in a random direction, and the
error of the sum is about u times the root-sum-square (RSS) of its terms.
Each identity is therefore checked as |lhs - rhs| <= TOL * RSS, with the RSS
taken over the terms of both sides and TOL = 2^-4: 16 u, i.e. ~30 standard
deviations of the rounding noise. (The worst-case bound, u times the sum of
|terms|, is far looser: by sqrt(#terms).) A lost, misplaced or mis-scaled
block of keys moves a sum by the RSS of its own terms, sqrt(64 / L) of the
RSS for a 64-key block of a sequence of L keys, which is above TOL for every
workload's sequences up to thousands of keys. I5 allows 2^-7 max_j |v_jd|:
the P V product uses bf16 P normalised by their fp32 row sum (weights summing
to 1 within 2^-8) and O is rounded to bf16 once more.

The functions take torch tensors on any device: the GPU tests pass the GPU's
outputs, a CPU test passes the oracle's outputs, with and without a planted
mistake, to show that the checks pass on a correct result and catch one.
"""
from __future__ import annotations

import numpy as np

TOL = 2.0 ** -4
O_RANGE_SLACK = 2.0 ** -7


def _torch():
    import torch
    return torch


def nan_in(**tensors):
    """Names of the tensors that hold a NaN (empty list: none)."""
    torch = _torch()
    return [n for n, t in tensors.items()
            if t is not None and t.numel() > 0 and bool(torch.isnan(t).any())]


def q_row_offsets(x):
    """Offsets of each sequence's output rows ([B+1]): b*lq for a broadcast Q."""
    w = x.workload
    if w.broadcast_q:
        return np.arange(x.batch + 1, dtype=np.int64) * w.lq
    return np.asarray(x.q_offsets, dtype=np.int64)


def rows_with_keys(x):
    """bool [T_q]: output rows that see at least one key (band: the row's
    window inside the sequence is not empty; block mask: a kept block inside
    the sequence; else a non-empty sequence)."""
    w = x.workload
    roff = q_row_offsets(x)
    out = np.zeros(int(roff[-1]), dtype=bool)
    left = None if w.window is None else w.window[0]
    right = 0 if w.causal else (None if w.window is None else w.window[1])
    for b in range(x.batch):
        L = int(x.kv_offsets[b + 1] - x.kv_offsets[b])
        n = int(roff[b + 1] - roff[b])
        if L == 0 or n == 0:
            continue
        i = np.arange(n)
        if x.block_mask is not None:
            nk = -(-L // 128)
            out[roff[b]:roff[b + 1]] = x.block_mask[b, i // 128, :nk].any(axis=1)
        elif left is not None or right is not None:
            lo = np.zeros(n, dtype=np.int64) if left is None else np.maximum(0, i - left)
            hi = np.full(n, L - 1, dtype=np.int64) if right is None else np.minimum(L - 1, i + right)
            out[roff[b]:roff[b + 1]] = lo <= hi
        else:
            out[roff[b]:roff[b + 1]] = True
    return out


def _ratio(diff, rss):
    """max |diff| / rss over the entries (rss = 0 needs diff = 0)."""
    torch = _torch()
    bad = (rss <= 0) & (diff != 0)
    if bool(bad.any()):
        return float("inf")
    r = diff.abs() / torch.where(rss > 0, rss, torch.ones_like(rss))
    return float(r.max()) if r.numel() else 0.0


def _outer_sum(a, b):
    """sum_r a_r b_r^T per head: a, b [n, H, D] fp64 -> [H, D, D]."""
    torch = _torch()
    at = a.permute(1, 2, 0).contiguous()    # [H, D, n]
    bt = b.permute(1, 0, 2).contiguous()    # [H, n, D]
    return torch.bmm(at, bt)


def identity_ratios(x, o, dk, dv, do, dq, q, k, v):
    """The worst |lhs - rhs| / RSS of I1-I4 over all sequences and heads, as a
    dict {name: (ratio, sequence)} (sequence -1: a pooled broadcast check)."""
    torch = _torch()
    f64 = lambda t: t.double()
    koff = np.asarray(x.kv_offsets, dtype=np.int64)
    roff = q_row_offsets(x)
    vis = torch.as_tensor(rows_with_keys(x), device=do.device)
    bcast = x.workload.broadcast_q
    worst = {n: (0.0, -1) for n in ("I1 sum dK", "I2 sum dV", "I3 dV v^T", "I4 dK k^T")}

    def upd(name, r, b):
        if r > worst[name][0]:
            worst[name] = (r, b)

    if bcast:
        qf = f64(q)
        H, D = qf.shape[1], qf.shape[2]
        lhs4 = torch.zeros((H, D, D), dtype=torch.float64, device=q.device)
        ss4 = torch.zeros_like(lhs4)
    for b in range(x.batch):
        k0, k1 = int(koff[b]), int(koff[b + 1])
        r0, r1 = int(roff[b]), int(roff[b + 1])
        dkb, dvb = f64(dk[k0:k1]), f64(dv[k0:k1])
        kb, vb = f64(k[k0:k1]), f64(v[k0:k1])
        dob = f64(do[r0:r1]) * vis[r0:r1, None, None]
        ob = f64(o[r0:r1])
        # I1, I2: per (head, d)
        upd("I1 sum dK", _ratio(dkb.sum(0), dkb.square().sum(0).sqrt()), b)
        upd("I2 sum dV", _ratio(dvb.sum(0) - dob.sum(0),
                                (dvb.square().sum(0) + dob.square().sum(0)).sqrt()), b)
        # I3: per (head, d, e)
        lhs = _outer_sum(dvb, vb) - _outer_sum(dob, ob)
        rss = (_outer_sum(dvb.square(), vb.square()) + _outer_sum(dob.square(), ob.square())).sqrt()
        upd("I3 dV v^T", _ratio(lhs, rss), b)
        # I4
        if bcast:
            lhs4 += _outer_sum(dkb, kb)
            ss4 += _outer_sum(dkb.square(), kb.square())
        else:
            qb, dqb = f64(q[r0:r1]), f64(dq[r0:r1])
            lhs = _outer_sum(dkb, kb) - _outer_sum(qb, dqb)
            rss = (_outer_sum(dkb.square(), kb.square()) + _outer_sum(qb.square(), dqb.square())).sqrt()
            upd("I4 dK k^T", _ratio(lhs, rss), b)
    if bcast:
        dqf = f64(dq)
        lhs4 -= _outer_sum(qf, dqf)
        ss4 += _outer_sum(qf.square(), dqf.square())
        upd("I4 dK k^T", _ratio(lhs4, ss4.sqrt()), -1)
    return worst


def o_range_violation(x, o, v):
    """Largest amount (over every output element) by which O leaves the
    [min, max] of the V rows its row sees, widened by the slack, as a
    fraction of max |v| of that sequence and head (<= 0: inside)."""
    torch = _torch()
    w = x.workload
    roff = q_row_offsets(x)
    right = 0 if w.causal else (None if w.window is None else w.window[1])
    banded = w.causal or w.window is not None
    worst = -float("inf")
    for b in range(x.batch):
        k0, k1 = int(x.kv_offsets[b]), int(x.kv_offsets[b + 1])
        r0, r1 = int(roff[b]), int(roff[b + 1])
        L, n = k1 - k0, r1 - r0
        if L == 0 or n == 0:
            continue
        vs = v[k0:k1].float()                        # [L, H, D]
        ob = o[r0:r1].float()                        # [n, H, D]
        amax = vs.abs().amax(dim=0)                  # [H, D]
        slack = O_RANGE_SLACK * amax + 1e-6
        if x.block_mask is not None:
            nk = -(-L // 128)
            pad = nk * 128 - L
            vp = torch.cat([vs, vs[-1:].expand(pad, -1, -1)]) if pad else vs
            bmin = vp.reshape(nk, 128, *vs.shape[1:]).amin(dim=1)   # [nk, H, D]
            bmax = vp.reshape(nk, 128, *vs.shape[1:]).amax(dim=1)
            m = torch.as_tensor(x.block_mask[b, :, :nk].astype(bool), device=vs.device)   # [nq, nk]
            inf = torch.tensor(float("inf"), device=vs.device)
            tmin = torch.where(m[:, :, None, None], bmin[None], inf).amin(dim=1)    # [nq, H, D]
            tmax = torch.where(m[:, :, None, None], bmax[None], -inf).amax(dim=1)
            tile = torch.arange(n, device=vs.device) // 128
            lo, hi = tmin[tile], tmax[tile]
            seen = m.any(dim=1)[tile]
            lo = torch.where(seen[:, None, None], lo, ob)   # rows without keys: O = 0 is checked elsewhere
            hi = torch.where(seen[:, None, None], hi, ob)
        elif banded and right is not None:
            # rows see keys j <= min(L-1, i + right): the prefix range is a
            # superset of the row's window, so the bound is valid (looser
            # where the window also has a left bound)
            pmin = torch.cummin(vs, dim=0).values
            pmax = torch.cummax(vs, dim=0).values
            last = torch.clamp(torch.arange(n, device=vs.device) + right, max=L - 1)
            lo, hi = pmin[last], pmax[last]
        else:
            lo, hi = vs.amin(dim=0)[None], vs.amax(dim=0)[None]
        over = torch.maximum(ob - (hi + slack), (lo - slack) - ob) / torch.clamp(amax, min=1e-30)
        worst = max(worst, float(over.max()))
    return worst


def check_invariants(x, o, lse, dk, dv, dq, dq_accum, delta, q, k, v, do):
    """Assert I0-I5 (tensors on any device; dq_accum is the fp32 dQ)."""
    bad = nan_in(o=o, lse=lse, dk=dk, dv=dv, dq=dq, dq_accum=dq_accum, delta=delta)
    assert not bad, "NaN left in %s" % bad
    ratios = identity_ratios(x, o, dk, dv, do, dq_accum, q, k, v)
    for name, (r, b) in ratios.items():
        assert r <= TOL, (name, "sequence", b, r)
    viol = o_range_violation(x, o, v)
    assert viol <= 0.0, ("I5 O outside the range of the visible V", viol)
    return ratios, viol


def to_torch_bf16(bits, device):
    """bf16 bit patterns (uint16 numpy) as a bf16 torch tensor on ``device``."""
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
