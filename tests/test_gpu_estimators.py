"""GPU parity of the residual estimator variants ([paper] §5 Table 4, App.
D.4): mean-only, scalar affine and diagonal affine corrections, next to the
default full ridge with output-subspace projection.  Everything before the
fit (layout, routing, probes, probe rows) is the same call and is checked
bit-exact / to the usual bar; the folded gain g and offset c and the final
output are compared with the oracle."""
import pytest

import synthgen as sg
from harness import compare_head, oracle_head, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("estimator", ["mean", "scalar", "diagonal"])
@pytest.mark.parametrize("head_dim,dtype", [(128, "bf16"), (64, "f32")])
def test_estimator_variants(estimator, head_dim, dtype):
    w = sg.small_workload(name=f"est_{estimator}_{head_dim}", heads=2, n=2100, head_dim=head_dim,
                          dtype=dtype, components=12, kv_split=2, rho="0.3", seed=51)
    heads = sg.make_call(w)
    g = run_gpu(w, heads, estimator=estimator)
    for h in range(w.heads):
        r = oracle_head(w, heads[h], estimator=estimator)
        errs = compare_head(w, g, h, r, hd=heads[h])
        say(f"[{estimator} {dtype} d={head_dim}] head {h}: {errs}")
