"""Seeded random problems (the GPU fuzz's generator, head_dim 128) through
the MXFP8 path against the oracle run on the decoded operands: the forward
(every output row within the E4M3 bound of P), the dQ pass and the dK/dV
pass (within the bounds derived for dS and P rounded to E4M3 with their
block scales), each as in tests/test_gpu_mx.py, with the mean error held to
half the mean bound (problems include single-term elements; see
_check_mx_dkdv) where at least 64 query rows and 64 keys make it a mean of
many independent roundings."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import numpy as np  # noqa: E402

from test_gpu_fuzz import _problem  # noqa: E402
from test_gpu_mx import _check_mx, _check_mx_dkdv, _check_mx_dq, _mx_dkdv_case, _run_mx  # noqa: E402

N_CASES = 120


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_problem_mx_matches_oracle(seed):
    kind, x, plan = _problem(seed, head_dims=(128,))
    print("mx fuzz seed", seed, kind, "lengths", list(x.lengths), "H", x.workload.heads, flush=True)
    o, lse = _run_mx(x, dynamic=plan["fwd_dynamic"])
    assert not np.isnan(o).any() and not np.isnan(lse).any()
    _check_mx(x, o, lse)
    mean_frac = 0.5 if x.t_q >= 64 and int(x.kv_offsets[-1]) >= 64 else None
    _check_mx_dq(x, mean_frac=mean_frac)
    _check_mx_dkdv(*_mx_dkdv_case(x), mean_frac=mean_frac)
