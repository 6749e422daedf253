"""A whole call (usual or probe-first order, whole or over head ranges on
several streams) captured in a HIP graph (SparsePRCall.capture) and replayed:
every replay, with eager calls and synchronisations between the replays,
gives the eager call's output bit for bit.  The library allocates nothing
and issues no memset inside a call, so the capture holds only its kernels."""
import numpy as np
import pytest

import synthgen as sg
from harness import say, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("head_dim,kv_split,fused,chunks", [(64, 2, False, 1), (128, 4, False, 1),
                                                        (128, 4, True, 1), (64, 2, True, [1, 2])])
def test_graph_replays_match_eager_calls(head_dim, kv_split, fused, chunks):
    import torch
    import free_block_sparse_major_amd as fb
    w = sg.small_workload(name=f"graph_{head_dim}_{fused}", heads=3, n=3000, head_dim=head_dim,
                          components=16, kv_split=kv_split, rho="0.26", seed=91)
    say(f"[graph] {w}")
    data = sg.make_call(w)
    q, k, v, lq, lk = upload(w, data)
    call = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, fb.BF16, w.c_q, w.c_k, m=w.m,
                           rank=w.r, rho=w.rho, out_dtype=fb.BF16, fused=fused,
                           head_chunks=chunks)
    eager = call(lq, lk, q, k, v).clone()
    torch.cuda.synchronize()
    call.capture(lq, lk, q, k, v)
    for i in range(3):
        out = call.replay().clone()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        again = call(lq, lk, q, k, v).clone()
        torch.cuda.synchronize()
        assert torch.equal(again, eager), f"eager call after replay {i}"
