"""jfa_bwd_noalloc (the backward with the library's own scratch area instead
of a caller workspace) through the C ABI against jfa_bwd on the same inputs
and plans: the kernels are the same, so every output must agree bit for bit.
Two calls in a row, the second on a smaller batch (the area keeps the first
call's partials, which the second must not see), then a per-sequence-Q
problem (no scratch needed)."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import jagged_flashattention_amd as J  # noqa: E402


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run_both(x):
    w = x.workload
    prob = J.Problem(batch=x.batch, num_heads=w.heads, head_dim=w.head_dim,
                     broadcast_q=w.broadcast_q, lq=w.lq if w.broadcast_q else 0, causal=w.causal,
                     softmax_scale=w.scale)
    att = J.JaggedAttention(prob, x.kv_offsets, x.q_offsets)
    q, k, v, do = dev(x.q), dev(x.k), dev(x.v), dev(x.do)
    o, lse = att.forward(q, k, v)
    H, D = w.heads, w.head_dim

    def outputs():
        return dict(dq=torch.full_like(q, float("nan")), dk=torch.full_like(k, float("nan")),
                    dv=torch.full_like(v, float("nan")),
                    dq_accum=torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda"),
                    delta=torch.full((H, att.total_q), float("nan"), dtype=torch.float32,
                                     device="cuda"))
    ref, got = outputs(), outputs()
    J.jfa_bwd(prob, att.bwd_plan, att.dq_plan, att.q_offsets, att.kv_offsets, q, k, v, o, lse, do,
              ref["dq"], ref["dk"], ref["dv"], ref["dq_accum"], ref["delta"], att.workspace,
              att.ws_bytes)
    J.jfa_bwd_noalloc(prob, att.bwd_plan, att.dq_plan, att.q_offsets, att.kv_offsets, q, k, v, o,
                      lse, do, got["dq"], got["dk"], got["dv"], got["dq_accum"], got["delta"])
    torch.cuda.synchronize()
    for name in ref:
        assert not torch.isnan(got[name]).any(), name
        assert torch.equal(_bits(got[name]), _bits(ref[name])), name
    return att


@pytest.mark.parametrize("step", ["first", "second"])
def test_noalloc_backward_equals_backward(step):
    """Broadcast Q (GEM-shaped recipe): 48 sequences, then 9 shorter ones."""
    print("no-alloc backward", step, flush=True)
    if step == "first":
        x = W.make_inputs(2, batch=48, heads=4)
    else:
        x = W.make_inputs(2, batch=9, heads=2, lq=100, seed=7)
    att = _run_both(x)
    assert 0 < att.ws_bytes <= J.JFA_NOALLOC_SCRATCH_BYTES


def test_noalloc_backward_per_sequence_causal():
    print("no-alloc backward, per-sequence causal", flush=True)
    x = W.make_inputs(3, lengths=np.array([300, 129, 1, 700]), heads=2)
    att = _run_both(x)
    assert att.ws_bytes == 0
