"""Exact probe rows when scores rise along the key order.

The probe-row kernel forms each tile's exponentials against running class
references and takes the class maxima only where a class first appears in a
key chunk or a score passes its reference by more than the slack (8 in log2
units).  Here every key row is scaled by a factor growing along the token
order (1 to 4), so inside each chunk later keys pass the references by far
more than the slack and that branch runs again and again; the dense and
sparse probe rows, the fit and the output are checked against the oracle."""
import numpy as np
import pytest

import synthgen as sg
from harness import compare_head, oracle_head, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("head_dim", [128, 64])
def test_probe_rows_with_rising_scores(head_dim):
    w = sg.small_workload(name=f"rise{head_dim}", heads=2, n=3000, head_dim=head_dim,
                          components=12, kv_split=2, rho="0.3", seed=131)
    data = sg.make_call(w)
    n = w.n
    ramp = (1.0 + 3.0 * np.arange(n, dtype=np.float32) / n)[:, None]
    for hd in data:
        k = hd["k"] * ramp
        hd["k_bits"] = sg.f32_to_bf16_bits(k.astype(np.float32))
        hd["k"] = sg.bf16_bits_to_f32(hd["k_bits"])
    # the scores of a probe-like row really pass a reference by more than
    # the slack inside a chunk (64 chunks of the group-major keys)
    c2 = np.log2(np.e) / np.sqrt(head_dim)
    hd = data[0]
    order = np.argsort(hd["labels_kv"], kind="stable")
    per = -(-n // 64)
    s = (hd["k"][order] @ hd["q"][0]) * c2
    rise = max(float(np.max(s[c:c + per]) - s[c]) for c in range(0, n, per))
    say(f"[rising {head_dim}] largest rise inside a chunk {rise:.1f} (log2 units)")
    assert rise > 16.0
    g = run_gpu(w, data)
    for h, hd in enumerate(data):
        r = oracle_head(w, hd)
        errs = compare_head(w, g, h, r, hd=hd)
        say(f"[rising {head_dim}] head {h}: {errs}")
