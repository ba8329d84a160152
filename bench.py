"""Benchmark: jagged FlashAttention forward + backward on one MI355X.

One step = the whole hot path over one batch of synthetic input: jfa_fwd
(O, LSE) then the backward stages (dQ kernel, which also forms delta =
rowsum(dO*O); dK/dV kernel; dQ reduce). Inputs are resident in HBM before timing starts. The default
workload is the GEM-shaped broadcast-Q one (B=256 sequences with lognormal
lengths, H=4, D=128, one shared Q of 256 rows).

Prints ONE JSON line with the throughput (algorithmic fwd+bwd TFLOP/s), the
roofline of the dominant kernel (timed with HIP events on the launch stream)
and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
METRIC = "JFA fwd+bwd TFLOP/s (bf16) and % of MFMA peak, jagged broadcast-Q"


def work_model(x, dq_workers: int = 256):
    """Algorithmic FLOPs and bytes of one step (see the design notes).
    ``dq_workers``: workers of the dQ plan (broadcast Q: each writes one fp32
    partial of a 256-row Q tile, which the reduce reads back)."""
    import numpy as np
    w = x.workload
    H, D = w.heads, w.head_dim
    lens = x.lengths.astype(np.int64)
    B = len(lens)
    t_k = int(lens.sum())
    if w.broadcast_q:
        q_rows, t_q = w.lq, B * w.lq
        q_lens = np.full(B, w.lq, dtype=np.int64)
    else:
        q_lens = np.diff(x.q_offsets.astype(np.int64))
        q_rows = t_q = int(q_lens.sum())
    kv_read_rows = t_k
    if x.block_mask is not None:
        pairs = 0
        kv_read_rows = 0
        mask = x.block_mask
        for b in range(B):
            nk = -(-int(lens[b]) // 128)
            nq = -(-int(q_lens[b]) // 128)
            rows = np.minimum(128, q_lens[b] - 128 * np.arange(nq))
            keys = np.minimum(128, lens[b] - 128 * np.arange(nk))
            m = mask[b, :nq, :nk].astype(np.int64)
            pairs += int(rows @ m @ keys)
            kv_read_rows += int(keys[m.any(axis=0)].sum())
    elif w.causal or w.window is not None:
        # visible pairs of the band j in [i - left, i + right] (causal: right = 0)
        left = None if w.window is None else w.window[0]
        right = 0 if w.causal else (None if w.window is None else w.window[1])
        pairs = 0
        for L in lens:
            i = np.arange(int(L), dtype=np.int64)
            lo = np.zeros_like(i) if left is None else np.maximum(0, i - left)
            hi = np.full_like(i, L - 1) if right is None else np.minimum(L - 1, i + right)
            pairs += int(np.maximum(0, hi - lo + 1).sum())
    else:
        pairs = int((q_lens * lens).sum())
    e = H * D * 2   # bytes of one bf16 row of all heads
    # each kernel: its inputs read once, its outputs written once
    fwd_bytes = q_rows * e + 2 * kv_read_rows * e + t_q * e + t_q * H * 4
    pre_bytes = 2 * t_q * e + t_q * H * 4
    dkdv_bytes = q_rows * e + 2 * kv_read_rows * e + t_q * e + 2 * t_q * H * 4 + 2 * t_k * e
    # the dQ pass also forms delta: it reads O and writes delta. Broadcast Q:
    # it writes the workers' fp32 partials, which the reduce reads back
    # before writing dq_accum (fp32) and dq; per-sequence Q: it writes those
    # two itself
    dq_out = q_rows * H * D * 4 + q_rows * e
    partials = dq_workers * 256 * D * 4 if w.broadcast_q else 0
    dq_bytes = (q_rows * e + 2 * kv_read_rows * e + 2 * t_q * e + 2 * t_q * H * 4
                + (partials if w.broadcast_q else dq_out))
    reduce_bytes = partials + dq_out if w.broadcast_q else 0
    # FLOPs: the forward's two GEMMs; the backward's five (S, dP, dV, dK in the
    # dK/dV kernel, dQ in the dQ kernel; the dQ kernel's recomputation of S
    # and dP is not counted)
    return dict(pairs=pairs, fwd_flop=4 * H * D * pairs, bwd_flop=10 * H * D * pairs,
                dkdv_flop=8 * H * D * pairs, dq_flop=2 * H * D * pairs,
                fwd_bytes=fwd_bytes, pre_bytes=pre_bytes, dkdv_bytes=dkdv_bytes,
                dq_bytes=dq_bytes, reduce_bytes=reduce_bytes, t_q=t_q, t_k=t_k, q_rows=q_rows)


def cpu_baseline(x, budget_s: float):
    """The fp64 oracle (as it stands) on the first sequences of the same
    workload until ``budget_s`` seconds of CPU work are spent, its BLAS
    threads pinned to the host cores this process may use (the CPU set of
    the process, capped by OMP_NUM_THREADS where that is set)."""
    from threadpoolctl import threadpool_info, threadpool_limits
    import numpy as np
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    with threadpool_limits(limits=threads, user_api="blas"):
        used = max([p.get("num_threads", 1) for p in threadpool_info()
                    if p.get("user_api") == "blas"] or [1])
        res = _oracle_sample(x, budget_s)
    res["cores"] = used
    return res


def _oracle_sample(x, budget_s: float):
    import numpy as np
    from oracle import attention as A
    import workloads as W
    w = x.workload
    q = x.as_f64("q") if w.broadcast_q else None
    done, flop, t_used = 0, 0.0, 0.0
    kw = dict(scale=w.scale, broadcast_q=w.broadcast_q, causal=w.causal, window=w.window)
    for b in range(x.batch):
        k0, k1 = int(x.kv_offsets[b]), int(x.kv_offsets[b + 1])
        k = W.bf16_bits_to_f32(x.k[k0:k1]).astype(np.float64)
        v = W.bf16_bits_to_f32(x.v[k0:k1]).astype(np.float64)
        off = np.array([0, k1 - k0], dtype=np.int32)
        if w.broadcast_q:
            qb, os_ = q, slice(b * w.lq, (b + 1) * w.lq)
            qoff = None
            n_rows = w.lq
        else:
            q0, q1 = int(x.q_offsets[b]), int(x.q_offsets[b + 1])
            qb = W.bf16_bits_to_f32(x.q[q0:q1]).astype(np.float64)
            os_ = slice(q0, q1)
            qoff = np.array([0, q1 - q0], dtype=np.int32)
            n_rows = q1 - q0
        do = W.bf16_bits_to_f32(x.do[os_]).astype(np.float64)
        mask = None if x.block_mask is None else x.block_mask[b:b + 1]
        t0 = time.perf_counter()
        A.forward(qb, k, v, off, q_offsets=qoff, block_mask=mask, **kw)
        A.backward(qb, k, v, do, off, q_offsets=qoff, block_mask=mask, **kw)
        t_used += time.perf_counter() - t0
        L = k1 - k0
        if mask is not None:
            vis = A.visibility(n_rows, L, mask_b=mask[0])
            pairs = int(vis.sum())
        elif w.window is not None:
            pairs = int(A.visibility(n_rows, L, causal=w.causal, window=w.window).sum())
        elif w.causal:
            pairs = L * (L + 1) // 2
        else:
            pairs = n_rows * L
        flop += 14.0 * w.heads * w.head_dim * pairs
        done += 1
        if t_used >= budget_s:
            break
    return {"value": flop / t_used / 1e12, "unit": "TFLOP/s", "cores": None, "kind": "oracle",
            "sample": "fp64 oracle fwd+bwd of the first %d of %d sequences (all %d heads) of the "
                      "same workload, %.1f s" % (done, x.batch, w.heads, t_used)}


def counters_for(kernel: str, workload: str):
    """The committed rocprofv3 counter summary of one kernel (HBM bytes and
    MFMA busy cycles per launch), if it was taken on the current kernel
    source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "%s.%s.traffic.txt" % (kernel, workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    digest = source_digest(kv.get("source", ""))
    if digest is None or digest != kv.get("source_sha256_16"):
        return None
    return kv


def code_only(text: bytes) -> bytes:
    """C/C++ source without its comments, every run of white space (line
    breaks included) outside string and character literals made one blank:
    what stays is the code's token stream."""
    def scan(t, on_comment, on_space):
        out, i, n = bytearray(), 0, len(t)
        while i < n:
            c = t[i:i + 1]
            if c in (b'"', b"'"):
                j = i + 1
                while j < n and t[j:j + 1] != c:
                    j += 2 if t[j:j + 1] == b"\\" else 1
                out += t[i:j + 1]
                i = j + 1
            elif on_comment and t.startswith(b"//", i):
                while i < n and t[i:i + 1] != b"\n":
                    i += 1
                out += b" "
            elif on_comment and t.startswith(b"/*", i):
                j = t.find(b"*/", i + 2)
                i = n if j < 0 else j + 2
                out += b" "
            elif on_space and c.isspace():
                while i < n and t[i:i + 1].isspace():
                    i += 1
                out += b" "
            else:
                out += c
                i += 1
        return bytes(out)
    return scan(scan(text, True, False), False, True).strip()


def source_digest(name: str, root: str = ROOT):
    """sha256 (first 16 hex digits) of a kernel source together with every
    header it includes from the library's own directories (transitively),
    comments left out, so that a change to the code, shared inner-loop code
    included, marks a counter summary stale and a change to a comment or to
    the layout of the text does not; None if the source does not exist."""
    import hashlib
    import re
    dirs = [os.path.join(root, "jagged_flashattention_amd", "csrc"), os.path.join(root, "include")]
    first = os.path.join(dirs[0], name)
    if not name or not os.path.exists(first):
        return None
    seen, todo, h = [], [first], hashlib.sha256()
    while todo:
        path = todo.pop(0)
        if path in seen:
            continue
        seen.append(path)
        text = open(path, "rb").read()
        h.update(os.path.basename(path).encode() + b"\0" + code_only(text))
        for inc in re.findall(rb'^\s*#\s*include\s+"([^"]+)"', text, re.M):
            for d in dirs:
                cand = os.path.join(d, inc.decode())
                if os.path.exists(cand):
                    todo.append(cand)
                    break
    return h.hexdigest()[:16]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=2, help="1..6 (2: GEM-shaped broadcast-Q; 6: sliding window)")
    ap.add_argument("--fwd-workers-per-cu", type=int, default=1)
    ap.add_argument("--bwd-workers-per-cu", type=int, default=1)
    ap.add_argument("--mx", type=int, default=1,
                    help="also time the MXFP8 forward and dQ pass on the same inputs (head_dim 128; 0: skip)")
    ap.add_argument("--fwd-plan", choices=("dynamic", "static"), default="dynamic",
                    help="forward tiles claimed at run time from the sorted list (when there "
                         "are more tiles than workers), or the static snake deal")
    ap.add_argument("--ablation", type=int, default=1,
                    help="also time the kernels with the natural (unsorted, round-robin) plans "
                         "and with the other forward plan (0: skip)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle CPU work for the baseline (0: skip)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one device copy of this many MiB (a known-size kernel "
                         "that scales the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only; --gpus %d is not supported "
              "(the multi-GPU sharding is described in the design notes, not built)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import jagged_flashattention_amd as J
    import workloads as W

    x = W.make_inputs(args.workload)
    w = x.workload
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    # two resident copies of the inputs (and outputs), used by alternate
    # steps, so that no step finds the previous step's tensors in L2 or the
    # MALL (the GEM workload's K and V alone exceed the 256 MiB MALL, the
    # others fit in it)
    sets = [tuple(dev(a) for a in (x.q, x.k, x.v, x.do)) for _ in range(2)]
    q, k, v, do = sets[0]
    mq, mk = (x.block_mask.shape[1], x.block_mask.shape[2]) if x.block_mask is not None else (0, 0)
    prob = J.Problem(batch=x.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0, causal=w.causal,
                     mask_q_blocks=mq, mask_kv_blocks=mk, softmax_scale=w.scale,
                     window_left=-1 if w.window is None or w.window[0] is None else w.window[0],
                     window_right=-1 if w.window is None or w.window[1] is None else w.window[1])
    cus = J.jfa_device_workers(0)
    mk_att = lambda: J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask,
                                       fwd_workers=cus * args.fwd_workers_per_cu,
                                       bwd_workers=cus * args.bwd_workers_per_cu,
                                       fwd_dynamic=None if args.fwd_plan == "dynamic" else False)
    att = mk_att()
    # host planning: the three plans on the CPU, then their one copy to the
    # device (median of a few re-plans; the first also pays for warm-up)
    replans = [mk_att() for _ in range(5)]
    plan_ms = {"planner_ms": float(np.median([a.planner_ms for a in replans])),
               "upload_ms": float(np.median([a.upload_ms for a in replans]))}
    del replans
    model = work_model(x, att.dq_plan.info.num_workers)
    H, D = w.heads, w.head_dim
    def outputs():
        return (torch.empty((att.total_q, H, D), dtype=torch.bfloat16, device="cuda"),
                torch.empty((H, att.total_q), dtype=torch.float32, device="cuda"),
                dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                     dq_accum=torch.empty(q.shape, dtype=torch.float32, device="cuda"),
                     delta=torch.empty((H, att.total_q), dtype=torch.float32, device="cuda")))
    outs = [outputs() for _ in range(2)]
    o, lse, out = outs[0]
    stages = (J.JFA_BWD_DQ, J.JFA_BWD_DKDV, J.JFA_BWD_DQ_REDUCE)
    nev = len(stages) + 2

    def step(ev=None, i=0, a=att):
        qi, ki, vi, doi = sets[i % 2]
        oi, lsei, outi = outs[i % 2]
        if ev is not None:
            ev[0].record()
        a.forward(qi, ki, vi, oi, lsei)
        for j, st in enumerate(stages):
            if ev is not None:
                ev[1 + j].record()
            a.backward(qi, ki, vi, oi, lsei, doi, outi, stages=st)
        if ev is not None:
            ev[-1].record()

    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    names = ("fwd", "bwd_dq", "bwd_dkdv", "bwd_dq_reduce")
    # The side measurements (plan ablation, MXFP8 passes, standalone delta)
    # run first, the headline steps last: a GPU that has just come out of idle
    # runs below its sustained clock for tens of milliseconds.

    # plan ablation (the sort and zigzag deal against the unsorted
    # round-robin plan, and the static zigzag forward against the dynamic
    # one): the same steps with other plans. The plans take turns, round by
    # round (the order reversed every other round), so that a clock that
    # drifts while the GPU warms up or heats up weighs on each plan alike;
    # per-kernel medians over every round's steps.
    def timed_rounds(atts, rounds=4):
        for a in atts:
            for i in range(args.warmup):
                step(i=i, a=a)
        samples = [{n: [] for n in names} for _ in atts]
        for r in range(rounds):
            order = list(range(len(atts)))
            if r % 2:
                order.reverse()
            for k in order:
                ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
                      for _ in range(args.steps)]
                for i in range(args.steps):
                    step(ev[i], i, atts[k])
                torch.cuda.synchronize()
                for j, n in enumerate(names):
                    samples[k][n] += [e[j].elapsed_time(e[j + 1]) for e in ev]
        return [{n: float(np.median(v)) for n, v in smp.items()} for smp in samples]
    ablation = None
    if args.ablation:
        kw = dict(fwd_workers=cus * args.fwd_workers_per_cu, bwd_workers=cus * args.bwd_workers_per_cu)
        srt, nat, stat = timed_rounds([
            att,
            J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask,
                              natural_plans=True, **kw),
            J.JaggedAttention(prob, x.kv_offsets, x.q_offsets, x.block_mask,
                              fwd_dynamic=args.fwd_plan != "dynamic", **kw)])
        ablation = {"kernel_ms_sorted_plans": srt, "kernel_ms_natural_plans": nat,
                    ("fwd_ms_static_zigzag" if args.fwd_plan == "dynamic" else "fwd_ms_dynamic"):
                    stat["fwd"],
                    "fwd_speedup_sorted_vs_natural": nat["fwd"] / srt["fwd"],
                    "bwd_speedup_sorted_vs_natural": (sum(nat[n] for n in names[1:])
                                                      / sum(srt[n] for n in names[1:])),
                    "dkdv_speedup_sorted_vs_natural": nat["bwd_dkdv"] / srt["bwd_dkdv"]}

    def time_alone(fn):
        """Median over the timed steps of fn(i) (i alternates the two input
        sets), recorded with HIP events around each call, after the warm-up."""
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for i, (e0, e1) in enumerate(ev):
            e0.record()
            fn(i)
            e1.record()
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))

    # the MXFP8 forward of the same problem (inputs encoded once per input
    # set, outside the timed loop; same plan), timed alone
    mx = None
    if args.mx and D == 128:
        mxqs = [att.quantize_mx(*sets[i][:3]) for i in range(2)]
        mx_ms = time_alone(lambda i: att.forward_mx(mxqs[i % 2], outs[i % 2][0], outs[i % 2][1]))
        # the encoding of bf16 Q, K, V into MXFP8, timed on its own
        qz_ms = time_alone(lambda i: att.quantize_mx(*sets[i % 2][:3]))
        mx = {"fwd_ms": mx_ms, "fwd_tflops": model["fwd_flop"] / (mx_ms * 1e-3) / 1e12,
              "pct_fp8_peak": 100.0 * model["fwd_flop"] / (mx_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS,
              "encode_ms": qz_ms,
              "fwd_with_encode_tflops": model["fwd_flop"] / ((mx_ms + qz_ms) * 1e-3) / 1e12}
        # the MXFP8 dQ pass (the backward's other encodings made once, outside
        # the timed loop), timed alone; then the step with both MXFP8 passes in
        # place of their bf16 ones
        opss = [att.quantize_mx_bwd(mxqs[i], sets[i][1], sets[i][2], sets[i][3]) for i in range(2)]

        def mx_dq(i):
            qi, ki, vi, doi = sets[i % 2]
            oi, lsei, outi = outs[i % 2]
            att.backward_mx(qi, ki, vi, oi, lsei, doi, opss[i % 2], outi, stages=J.JFA_BWD_DQ)
        mdq_ms = time_alone(mx_dq)
        qzb_ms = time_alone(lambda i: att.quantize_mx_bwd(mxqs[i % 2], *sets[i % 2][1:]))
        # the MXFP8 dK/dV pass (Q and dO also encoded along their rows, once,
        # outside the timed loop), timed alone
        opsk = [att.quantize_mx_dkdv(opss[i], sets[i][0], sets[i][3]) for i in range(2)]

        def mx_dkdv(i):
            qi, ki, vi, doi = sets[i % 2]
            oi, lsei, outi = outs[i % 2]
            att.backward_mx(qi, ki, vi, oi, lsei, doi, opsk[i % 2], outi, stages=J.JFA_BWD_DKDV)
        mdkdv_ms = time_alone(mx_dkdv)
        qzk_ms = time_alone(lambda i: att.quantize_mx_dkdv(opss[i % 2], sets[i % 2][0], sets[i % 2][3]))
        mx.update({"dq_ms": mdq_ms,
                   "dq_issued_tflops": 3 * model["dq_flop"] / (mdq_ms * 1e-3) / 1e12,
                   "encode_bwd_ms": qzb_ms,
                   "dkdv_ms": mdkdv_ms,
                   "dkdv_tflops": model["dkdv_flop"] / (mdkdv_ms * 1e-3) / 1e12,
                   "encode_dkdv_rows_ms": qzk_ms})

    # the two second stages of the broadcast-Q dQ reduction, each timed alone
    # on the same inputs: the per-worker partials plus the fixed-order reduce
    # (the step's scheme), and fp32 atomic adds into the zeroed dq_accum plus
    # the bf16 conversion
    def stage(st):
        def f(i):
            qi, ki, vi, doi = sets[i % 2]
            oi, lsei, outi = outs[i % 2]
            att.backward(qi, ki, vi, oi, lsei, doi, outi, stages=st)
        return f
    dq_scheme = None
    if w.broadcast_q:
        at = J.JFA_BWD_DQ_ATOMIC
        red = (time_alone(stage(J.JFA_BWD_DQ)), time_alone(stage(J.JFA_BWD_DQ_REDUCE)))
        ato = (time_alone(stage(J.JFA_BWD_DQ | at)), time_alone(stage(J.JFA_BWD_DQ_REDUCE | at)))
        dq_scheme = {"partials_reduce": {"dq_ms": red[0], "reduce_ms": red[1], "total_ms": sum(red)},
                     "atomic": {"dq_ms": ato[0], "convert_ms": ato[1], "total_ms": sum(ato)}}
        # leave the step's outputs as the step's scheme makes them
        for i in range(2):
            stage(J.JFA_BWD_DQ | J.JFA_BWD_DQ_REDUCE)(i)

    # the standalone delta preprocess (not part of the step: the dQ kernel
    # forms delta itself), timed alone for its HBM rate
    def pre(i):
        qi, ki, vi, doi = sets[i % 2]
        oi, lsei, outi = outs[i % 2]
        att.backward(qi, ki, vi, oi, lsei, doi, outi, stages=J.JFA_BWD_PREPROCESS)
    pre_ms = time_alone(pre)

    for i in range(args.warmup):
        step(i=i)
    torch.cuda.synchronize()
    # the timed steps: the step's launches only (the per-kernel event records,
    # a few microseconds each, are taken in a second pass of the same steps)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(None, i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    t1 = time.perf_counter()
    for i in range(args.steps):
        step(events[i], i)
    torch.cuda.synchronize()
    ms_step_with_events = (time.perf_counter() - t1) * 1e3 / args.steps
    names = ("fwd", "bwd_dq", "bwd_dkdv", "bwd_dq_reduce")
    # per-kernel: the median over the timed steps
    per = {n: float(np.median([e[j].elapsed_time(e[j + 1]) for e in events]))
           for j, n in enumerate(names)}
    per_mean = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in events]))
                for j, n in enumerate(names)}

    if mx is not None:
        mixed_ms = mx["fwd_ms"] + mx["dq_ms"] + per["bwd_dkdv"] + per["bwd_dq_reduce"]
        all_ms = mx["fwd_ms"] + mx["dq_ms"] + mx["dkdv_ms"] + per["bwd_dq_reduce"]
        mx.update({"dq_vs_bf16_dq": per["bwd_dq"] / mx["dq_ms"],
                   "dkdv_vs_bf16_dkdv": per["bwd_dkdv"] / mx["dkdv_ms"],
                   "step_mx_fwd_mx_dq_ms": mixed_ms,
                   "step_mx_fwd_mx_dq_tflops": (model["fwd_flop"] + model["bwd_flop"])
                   / (mixed_ms * 1e-3) / 1e12,
                   "step_all_mx_ms": all_ms,
                   "step_all_mx_tflops": (model["fwd_flop"] + model["bwd_flop"]) / (all_ms * 1e-3) / 1e12})

    flop = model["fwd_flop"] + model["bwd_flop"]
    value = flop / (ms_step * 1e-3) / 1e12
    wl_name = w.name
    fwd_tf = model["fwd_flop"] / (per["fwd"] * 1e-3) / 1e12
    bwd_ms = per["bwd_dq"] + per["bwd_dkdv"] + per["bwd_dq_reduce"]
    bwd_tf = model["bwd_flop"] / (bwd_ms * 1e-3) / 1e12

    kernels = {
        "fwd": ("fwd.hip", model["fwd_flop"], model["fwd_bytes"]),
        "bwd_dkdv": ("bwd.hip", model["dkdv_flop"], model["dkdv_bytes"]),
        "bwd_dq": ("dq.hip", model["dq_flop"], model["dq_bytes"]),
    }
    dom = max(kernels, key=lambda n: per[n])
    _, kflop, kbytes = kernels[dom]
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    t_s = per_mean[dom] * 1e-3   # the average launch, as rocprofv3's statistics give it
    if kflop / kbytes >= ridge:
        roof = {"bound": "mfma", "achieved": kflop / t_s / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": kbytes / t_s / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    cnt = {n: counters_for(n, wl_name) for n in kernels}
    roof["traffic"] = float(cnt[dom]["hbm_bytes_per_launch"]) if cnt[dom] else None
    roof["kernel"] = dom
    roof["avg_ms"] = per_mean[dom]
    roof["algorithmic_flop"] = kflop
    roof["algorithmic_bytes"] = kbytes

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl_name, "batch": x.batch, "heads": H, "head_dim": D,
                   "broadcast_q": w.broadcast_q, "lq": w.lq if w.broadcast_q else None,
                   "causal": w.causal, "block_sparse": x.block_mask is not None,
                   "window": w.window,
                   "lengths": w.lengths, "seed": w.seed, "total_kv": model["t_k"],
                   "total_q": model["t_q"],
                   "fwd_workers": att.fwd_plan.info.num_workers,
                   "fwd_plan": ("dynamic" if att.fwd_plan.info.pass_ & J.JFA_PLAN_DYNAMIC
                                else "static"),
                   "bwd_workers": att.bwd_plan.info.num_workers,
                   "dq_workers": att.dq_plan.info.num_workers},
        "pct_mfma_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "fwd_tflops": fwd_tf,
        "bwd_tflops": bwd_tf,
        "kernel_ms": per,
        "kernel_ms_mean": per_mean,
        "ms_per_step_with_kernel_events": ms_step_with_events,
        "hbm_gbps": {"bwd_dq_reduce": (model["reduce_bytes"] / (per["bwd_dq_reduce"] * 1e-3) / 1e9
                                       if model["reduce_bytes"] else None),
                     "bwd_preprocess_standalone": model["pre_bytes"] / (pre_ms * 1e-3) / 1e9},
        "bwd_preprocess_standalone_ms": pre_ms,
        "mfma_busy_pct_counters": {n: float(c["mfma_busy_pct"]) for n, c in cnt.items()
                                   if c and "mfma_busy_pct" in c},
        # achieved shader clock: GRBM_GUI_ACTIVE per launch (summed over the
        # 8 XCDs, from the committed counter run) over this run's mean launch
        "clock_ghz_counters": {n: float(c["grbm_gui_active"]) / 8 / (per_mean[n] * 1e-3) / 1e9
                               for n, c in cnt.items() if c and "grbm_gui_active" in c},
        "plan_host_ms": plan_ms,
        "roofline": roof,
    }
    if mx is not None:
        res["mxfp8"] = mx
    if ablation is not None:
        res["plan_ablation"] = ablation
    if dq_scheme is not None:
        res["dq_reduction_schemes"] = dq_scheme
    if args.cpu_budget > 0:
        res["cpu_baseline"] = cpu_baseline(x, args.cpu_budget)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
