"""Property-based parity on tiny shapes: hypothesis draws the shape (heads,
tokens, head size, dtype, group counts, K/V split, density target, probe
count, rank, layout, estimator, call order) and the seed of the synthetic
inputs; every drawn call runs through the C ABI on the GPU and is compared
with the oracle exactly like the fixed parity cases (integers bit-exact,
floating outputs within the path's tolerance, per-row bounds).  The examples
are derandomized, so every run tests the same cases."""
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import synthgen as sg
from harness import compare_head, oracle_head, run_gpu, say

pytestmark = pytest.mark.gpu


@st.composite
def calls(draw):
    dtype = draw(st.sampled_from(["bf16", "bf16", "f32"]))
    n = draw(st.integers(1, 700))
    comps = draw(st.integers(1, 40))
    w = sg.small_workload(
        name="fuzz", heads=draw(st.integers(1, 3)), n=n,
        head_dim=draw(st.sampled_from([64, 128])), dtype=dtype, components=comps,
        kv_split=draw(st.integers(1, 3)),
        rho=draw(st.sampled_from(["0.05", "0.2", "0.26", "0.5", "1"])),
        m=draw(st.integers(1, 64)), r=draw(st.integers(0, 16)),
        seed=draw(st.integers(0, 10 ** 6)))
    opts = {
        "layout": draw(st.sampled_from(["hnd", "nhd"])),
        "estimator": draw(st.sampled_from(["full", "full", "mean", "scalar", "diagonal"])),
        "fused": draw(st.booleans()),
    }
    return w, opts


@settings(max_examples=30, deadline=None, derandomize=True, database=None,
          suppress_health_check=list(HealthCheck))
@given(calls())
def test_tiny_calls_match_oracle(case):
    w, opts = case
    say(f"[fuzz] {w} {opts}")
    data = sg.make_call(w)
    g = run_gpu(w, data, **opts)
    for h, hd in enumerate(data):
        r = oracle_head(w, hd, estimator=opts["estimator"])
        compare_head(w, g, h, r, hd=hd, fused=opts["fused"])
