"""Benchmark of one SparsePR attention call on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan]

A step is one whole attention call (layout, routing, sparse attention,
probes + fit on a side stream, correction) over all heads of the workload,
inputs resident in HBM.  For the workload `wan_rcp` the step also builds the
partition itself (response-coupled partitioning) before the call, and the
probe distances use the query-response coordinates.  Prints one JSON line:
the mean time of the timed steps (`value`), the per-call median and minimum
from events between the steps, the attention kernel against the bf16 MFMA
peak (`roofline`), the CPU oracle on a bounded sample (`cpu_baseline`) and,
for inputs that fit the Infinity Cache, calls timed after a 512 MB cache-
evicting write.  Only one GPU is used; the path shards by head, and --gpus
above 1 is refused.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3        # MI355X fp32 matrix (v_mfma_f32_*_f32)
HBM_PEAK_GBS = 8000.0
METRIC = "ms per sparse-attention call (all heads) + executed-pair TFLOPS, % bf16 peak"
PROFILE_PMC = os.path.join(ROOT, "profiles", "attn_bf16_kernel_wan_pmc.txt")
KERNEL_SRC = os.path.join(ROOT, "free_block_sparse_major_amd", "csrc", "attn.hip")



def _item_waves(heads, n_q, c_q):
    """Waves per work item the attention launch picks for bf16 inputs (the
    library's rule: the best busy-wave share for the mean group size in
    {4, 8, 12}, largest on ties; 4 when that gives fewer items than CUs)."""
    q = -(-n_q // (32 * c_q))
    best, best_eff = 4, 0.0
    for w in (4, 8, 12):
        eff = q / (w * -(-q // w))
        if eff >= best_eff - 1e-12:
            best, best_eff = w, eff
    if heads * c_q * -(-q // best) < 256:
        return 4
    return best

def _src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic_from_profile(workload_name):
    """HBM bytes per attention launch from the committed PMC summary, or None
    if there is none or the kernel source changed since it was taken."""
    if not os.path.exists(PROFILE_PMC):
        return None
    txt = open(PROFILE_PMC).read()
    m_hash = re.search(r"attn_src_sha256_16\s*=\s*([0-9a-f]+)", txt)
    m_wl = re.search(r"workload\s*=\s*(\S+)", txt)
    m_b = re.search(r"hbm_bytes_per_launch\s*=\s*([0-9.eE+]+)", txt)
    if not (m_hash and m_b and m_wl) or m_hash.group(1) != _src_hash(KERNEL_SRC):
        return None
    if m_wl.group(1) != workload_name:
        return None
    return float(m_b.group(1))


def host_info():
    """The host the oracle is timed on: CPU model, logical CPUs usable by this
    process, physical cores (from lscpu, if present) and numpy's BLAS."""
    import subprocess
    import numpy as np
    info = {"logical_cpus": os.cpu_count()}
    try:
        info["usable_cpus"] = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        out = subprocess.run(["lscpu", "-p=core,socket"], capture_output=True, text=True,
                             timeout=20).stdout
        cores = {l for l in out.splitlines() if l and not l.startswith("#")}
        if cores:
            info["physical_cores"] = len(cores)
    except Exception:  # pragma: no cover
        pass
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        info["blas"] = f"{blas.get('name')} {blas.get('version')}"
    except Exception:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if pools:
            info["blas_threads"] = max(p.get("num_threads", 1) for p in pools)
            info["blas_internal"] = pools[0].get("internal_api")
    except Exception:  # pragma: no cover
        pass
    return info


def _head0_inputs(w, arrays, rcp_params):
    """Head 0 of the workload as the oracle takes it (fp32 values of the bf16
    inputs), with its partition: the given labels, or the oracle's own
    response-coupled partition."""
    import numpy as np
    import oracle
    h = 0
    if w.dtype == "bf16":
        f32 = lambda a: (a.astype(np.uint32) << 16).view(np.float32)
    else:
        f32 = lambda a: a
    q, k, v = f32(arrays["q"][h]), f32(arrays["k"][h]), f32(arrays["v"][h])
    lq, lk = arrays["labels_q"][h], arrays["labels_kv"][h]
    feats = None
    if rcp_params is not None:
        import synthgen as sg
        ik, iq = sg.rcp_init(w, h)
        part = oracle.rcp.rcp_partition(q, k, rcp_params["m_s"], rcp_params["r_k"], w.c_k,
                                        rcp_params["r_q"], w.c_q, ik, iq, rcp_params["iters"])
        lq, lk, feats = part["labels_q"], part["labels_kv"], part["phi_q"]
    return q, k, v, lq, lk, feats


def cpu_baseline(w, arrays, budget_seconds=10.0, rcp_params=None, estimator="full",
                 route_rule="global"):
    """The oracle, as it is, on the host cores, extrapolated from head 0:
    routing, probes and fit of head 0 in full (fp64), then the sparse
    attention + correction on whole query groups (largest first) until
    ~budget_seconds, once in the oracle's fp32 arithmetic mode (`value`) and
    once in fp64 (`value_fp64`, half the budget); each scaled to all rows and
    all heads of the call (ms per call)."""
    import numpy as np
    import oracle
    info = host_info()
    t0 = time.time()
    q, k, v, lq, lk, feats = _head0_inputs(w, arrays, rcp_params)
    r = oracle.run_head(q, k, v, lq, lk, w.c_q, w.c_k, w.rho, m=w.m, rank=w.r, lam=w.lam,
                        features=feats, query_rows=np.zeros(0, np.int64), estimator=estimator,
                        route_rule=route_rule)
    t_fixed = time.time() - t0
    sizes = np.diff(r["offsets_q"])

    def rows_timed(dtype, budget):
        rows_done, t_rows = 0, 0.0
        for a in np.argsort(-sizes, kind="stable"):
            if t_rows > budget or sizes[a] == 0:
                break
            rows = r["perm_q"][r["offsets_q"][a]:r["offsets_q"][a + 1]]
            t1 = time.time()
            o, _ = oracle.sparse_attention_rows(q[rows], lq[rows], k, v, lk, r["z"], r["scale"],
                                                dtype=dtype)
            if estimator == "full":
                oracle.apply_correction(o, r["fit"])
            else:
                oracle.apply_estimator(o, r["fit"])
            t_rows += time.time() - t1
            rows_done += rows.size
        return rows_done, t_rows

    n32, t32 = rows_timed(np.float32, budget_seconds)
    n64, t64 = rows_timed(np.float64, budget_seconds / 2)
    ms = lambda n_rows, t: (t_fixed + t * (w.n / max(n_rows, 1))) * w.heads * 1e3
    cores = info.get("blas_threads") or info.get("usable_cpus") or os.cpu_count() or 1
    return {"value": ms(n32, t32), "unit": "ms/call", "cores": int(cores), "kind": "oracle",
            "value_fp64": ms(n64, t64),
            "sample": (f"extrapolated from head 0 of {w.heads}: "
                       f"{'partition/' if rcp_params else ''}routing/probes/fit in full (fp64, "
                       f"{t_fixed:.1f} s); sparse attention + correction on whole query groups, "
                       f"largest first: {n32} of {w.n} rows in {t32:.1f} s in the fp32 mode "
                       f"(value), {n64} rows in {t64:.1f} s in fp64 (value_fp64); each scaled "
                       f"to {w.heads} heads x {w.n} rows"),
            "host": info}


def correction_quality(w, arrays, call, rcp_params=None, count=2048):
    """Per-row relative error against dense attention on `count` evenly spaced
    unprobed rows of head 0, before and after the correction (mean, p99): the
    oracle's own hard-drop and corrected rows, and the GPU call's.  Information
    only (the synthetic inputs are not the pages' activations)."""
    import numpy as np
    import oracle
    q, k, v, lq, lk, feats = _head0_inputs(w, arrays, rcp_params)
    rep = oracle.correction_report(q, k, v, lq, lk, w.c_q, w.c_k, w.rho, m=w.m, rank=w.r,
                                   lam=w.lam, count=count, features=feats)
    rows = rep["rows"]
    out = {"head": 0, "rows": int(rows.size), "rho_exec": round(rep["rho_exec"], 6),
           "oracle": {"before": rep["before"], "after": rep["after"]}}
    if rcp_params is None:
        if call.fused:
            # the probe-first order stores no O_sp: the uncorrected rows come
            # from the plain attention call on the same layout and cells
            call.attend()
        perm = call.perm_q[0].cpu().numpy()
        inv = np.empty_like(perm)
        inv[perm] = np.arange(perm.size)
        o_sp = call.o_sp[0].cpu().numpy()[inv[rows]]
        o_out = call.out[0].float().cpu().numpy()[rows]
        out["gpu"] = {"before": oracle.row_error_stats(o_sp, rep["dense"]),
                      "after": oracle.row_error_stats(o_out, rep["dense"]),
                      "output_dtype": str(call.out.dtype).replace("torch.", "")}
    for side in ("oracle", "gpu"):
        for when in out.get(side, {}):
            if isinstance(out[side][when], dict):
                out[side][when] = {k2: (round(v2, 5) if isinstance(v2, float) else v2)
                                   for k2, v2 in out[side][when].items()}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--rho", default=None, help="override the executed-density target")
    ap.add_argument("--estimator", default="full", choices=("full", "mean", "scalar", "diagonal"),
                    help="residual estimator (the full ridge with projection is the default)")
    ap.add_argument("--route-rule", default="global", choices=("global", "per_group"),
                    help="cell selection: one executed-pair budget per head (default) or a "
                         "key-token budget per query group")
    ap.add_argument("--head-chunks", type=lambda x: [int(v) for v in x.split(",")] if "," in x
                    else int(x), default=1,
                    help="split each call into this many head ranges on alternating streams "
                         "(layout and routing of one range overlap the attention of the last)")
    ap.add_argument("--lead", default="auto", choices=("auto", "fused", "unfused"),
                    help="fused order over head ranges: unfused lets the first range attend as "
                         "soon as it is routed and take the correction kernel after its fit; "
                         "auto: unfused where --order auto picks the fused order")
    ap.add_argument("--order", default="auto", choices=("auto", "usual", "fused"),
                    help="usual: attention, probe fit on a side stream, then the correction "
                         "kernel; fused: probe fit first, correction in the attention epilogue; "
                         "auto: fused over two head ranges (a quarter of the heads, then the "
                         "rest, the first range unfused) for bf16 calls of 16 heads or more "
                         "(measured faster there), "
                         "usual otherwise")
    ap.add_argument("--rcp-warm", action="store_true",
                    help="with a response-coupled workload: after a first call in the warm-up, "
                         "every step runs a later call from the previous call's state")
    ap.add_argument("--warm-iters", type=int, default=None,
                    help="Lloyd iterations of later calls (default: those of the first call)")
    ap.add_argument("--serial", action="store_true",
                    help="run the probe fit on the main stream after the attention (no side "
                         "stream): per-kernel durations without sharing the GPU")
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto",
                    help="also time calls each preceded by a 512 MB scratch write that evicts "
                         "the inputs from the caches (auto: when Q, K and V fit in the 256 MB "
                         "Infinity Cache)")
    ap.add_argument("--flush-calls", type=int, default=10)
    ap.add_argument("--dense-own", action="store_true",
                    help="also time this library in dense mode (one group, every cell)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SparsePR call shards by head with no "
              "communication; its multi-GPU throughput is N times the single-GPU figure "
              "and is not measured here.",
              file=sys.stderr)
        sys.exit(2)

    import dataclasses

    import numpy as np
    import torch

    import free_block_sparse_major_amd as fb
    import synthgen as sg

    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "copies": 5}))
        return

    w = sg.workload(args.workload)
    if args.rho:
        w = dataclasses.replace(w, rho=args.rho)
    if args.order == "auto":
        big = w.dtype == "bf16" and w.heads >= 16 and w.r <= 16
        args.order = "fused" if big else "usual"
        if big and args.head_chunks == 1:
            # a quarter of the heads first: its probe fit is short and its
            # attention starts early; the rest are fitted meanwhile
            args.head_chunks = [w.heads // 4, w.heads - w.heads // 4]
        if big and args.lead == "auto":
            # the first range's fit then runs beside its attention instead of
            # in front of it
            args.lead = "unfused"
    t0 = time.time()
    arr = sg.make_call_arrays(w)
    gen_s = time.time() - t0
    dev = torch.device("cuda")
    if w.dtype == "bf16":
        up = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        up = lambda a: torch.from_numpy(a).to(dev)
    q, k, v = up(arr["q"]), up(arr["k"]), up(arr["v"])
    lq = torch.from_numpy(arr["labels_q"]).to(dev)
    lk = torch.from_numpy(arr["labels_kv"]).to(dev)
    dtype = fb.BF16 if w.dtype == "bf16" else fb.F32
    rcp = w.name.endswith("_rcp")
    rp = sg.RCP_PARAMS if rcp else None
    call = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, dtype, w.c_q, w.c_k, m=w.m, rank=w.r,
                           lam=w.lam, rho=w.rho, out_dtype=fb.BF16 if w.dtype == "bf16" else fb.F32,
                           feat_dim=rp["r_q"] if rcp else 0, estimator=args.estimator,
                           route_rule=args.route_rule, head_chunks=args.head_chunks,
                           overlap=not args.serial, fused=args.order == "fused",
                           lead_unfused=args.lead == "unfused")
    part = None
    if rcp:
        part = fb.RcpPartition(w.heads, w.n, w.n, w.head_dim, dtype, w.c_q, w.c_k, **rp,
                               keep_state=args.rcp_warm)
        ik, iq = sg.rcp_init_arrays(w)
        init_k, init_q = torch.from_numpy(ik).to(dev), torch.from_numpy(iq).to(dev)
        call.probe_feat = part.phi_q
    rcp_events = []
    warm_iters = args.warm_iters or (rp["iters"] if rcp else None)

    def step(c):
        """One whole call; with response-coupled partitioning the partition
        is built first (timed with events on the current stream): a first
        call, or with --rcp-warm a later call once a first one has run."""
        if part is None:
            return c(lq, lk, q, k, v)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if args.rcp_warm and part.has_state:
            part(q, k, warm=True, iters=warm_iters)
        else:
            part(q, k, init_q, init_k)
        e1.record()
        rcp_events.append((e0, e1))
        return c(part.labels_q, part.labels_kv, q, k, v)

    # attention launches are bracketed with events on the stream they run on
    attn_events = []
    attn_name = "attend_correct" if call.fused else "attend"
    orig_attend = getattr(call, attn_name)

    def timed_attend(stream=None, part=None):
        s = torch.cuda.current_stream() if stream is None else stream
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        orig_attend(stream, part)
        e1.record(s)
        attn_events.append((e0, e1))

    for _ in range(args.warmup):
        step(call)
    torch.cuda.synchronize()
    setattr(call, attn_name, timed_attend)
    attn_events.clear()
    rcp_events.clear()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # events between the steps give per-call times (median, minimum) within
    # the same timed region
    step_marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps - 1)]
    e_start.record()
    for i in range(args.steps):
        step(call)
        if i + 1 < args.steps:
            step_marks[i].record()
    e_end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    ms_call = e_start.elapsed_time(e_end) / args.steps
    rcp_ms = (sum(a.elapsed_time(b) for a, b in rcp_events) / len(rcp_events)
              if rcp_events else None)
    if call.chunks is not None:
        # launches of a split call overlap other work on the other streams: the
        # kernel is timed on launches over all heads, back to back
        attn_events.clear()
        for _ in range(3):
            getattr(call, attn_name)()
    torch.cuda.synchronize()
    attn_ms = sum(a.elapsed_time(b) for a, b in attn_events) / len(attn_events)
    setattr(call, attn_name, orig_attend)
    marks = [e_start] + step_marks + [e_end]
    per_call = sorted(a.elapsed_time(b) for a, b in zip(marks[:-1], marks[1:]))
    call_ms_median = per_call[len(per_call) // 2]
    call_ms_min = per_call[0]

    # cache-flushed calls: a 512 MB write (a fill kernel) before each call,
    # outside the events that time the call
    input_bytes = sum(t.numel() * t.element_size() for t in (q, k, v))
    flushed_ms = None
    if args.flush == "on" or (args.flush == "auto" and input_bytes < (256 << 20)):
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        times = []
        for _ in range(args.flush_calls):
            scratch.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(call)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        del scratch
        flushed_ms = sorted(times)[len(times) // 2]

    routed = int(call.routed_pairs.sum().item())
    H, n, d, m_eff = w.heads, w.n, w.head_dim, min(w.m, w.n)
    attn_flop = 4.0 * d * routed
    exec_flop = 4.0 * d * (routed + H * m_eff * n)
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    attn_tflops = attn_flop / (attn_ms * 1e-3) / 1e12
    call_tflops = exec_flop / (ms_call * 1e-3) / 1e12
    rho_route = routed / (H * n * n)
    rho_exec = rho_route + m_eff / n

    out = {
        "metric": METRIC,
        "value": round(ms_call, 4),
        "unit": "ms/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_call, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": (f"{w.name}: {H} heads x {n} tokens, d={d}, {w.dtype}, "
                         f"C_q={w.c_q}, C_k={w.c_k}, rho*={w.rho}, M={w.m}, r={w.r}, "
                         f"lambda={w.lam}, seed={w.seed}"),
            "heads": H, "tokens": n, "head_dim": d, "c_q": w.c_q, "c_k": w.c_k,
            "rho_target": w.rho, "m": w.m, "r": w.r, "lambda": w.lam,
            "estimator": args.estimator,
            "route_rule": args.route_rule,
            "head_chunks": args.head_chunks,
            "order": args.order + (" (first range unfused)"
                                   if args.order == "fused" and args.lead == "unfused" else ""),
            "probe_fit": ("first range: beside its attention, then the correction kernel; "
                          "later ranges: before the attention, correction in its epilogue"
                          if args.order == "fused" and args.lead == "unfused" else
                          "before the attention, correction in its epilogue"
                          if args.order == "fused" else
                          "main stream after the attention" if args.serial else "side stream"),
            "parallelism": "single GPU",
        },
        "executed_pair_tflops": round(call_tflops, 2),
        "pct_bf16_peak": round(100 * call_tflops / BF16_PEAK_TFLOPS, 2),
        "attn_ms": round(attn_ms, 4),
        "attn_tflops": round(attn_tflops, 2),
        "attn_pct_peak": round(100 * attn_tflops / peak, 2),
        "routed_pairs": routed,
        "rho_route": round(rho_route, 6),
        "rho_exec": round(rho_exec, 6),
        "wall_ms_per_call": round(wall_ms, 4),
        "call_ms_median": round(call_ms_median, 4),
        "call_ms_min": round(call_ms_min, 4),
        "input_generation_s": round(gen_s, 1),
    }
    if flushed_ms is not None:
        out["call_ms_flushed_median"] = round(flushed_ms, 4)
    if rcp:
        out["config"]["partition"] = ("response-coupled on the GPU: M_s=%d, r_K=%d, r_Q=%d, "
                                      "%d Lloyd iterations" % (rp["m_s"], rp["r_k"], rp["r_q"],
                                                               rp["iters"]))
        if args.rcp_warm:
            # a first call on the same inputs, for comparison (resets the state)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            part(q, k, init_q, init_k)
            e1.record()
            torch.cuda.synchronize()
            rcp_first_ms = e0.elapsed_time(e1)
            out["config"]["partition"] += (
                "; timed steps are later calls: two subspace iterations from the previous bases, "
                "k-means from the previous centroids, %d Lloyd iterations" % warm_iters)
            out["rcp_partition_first_call_ms"] = round(rcp_first_ms, 4)
        out["rcp_partition_ms"] = round(rcp_ms, 4)
        lab = part.labels_q.cpu().numpy()
        out["nonempty_query_groups_mean"] = round(float(np.mean(
            [(np.bincount(l, minlength=w.c_q) > 0).sum() for l in lab])), 1)
        # the step (partition + call) across executed-density targets
        sweep = {}
        for rho in ("0.12", "0.22", "0.26", "0.35"):
            cs = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, dtype, w.c_q, w.c_k, m=w.m,
                                 rank=w.r, lam=w.lam, rho=rho,
                                 out_dtype=fb.BF16 if w.dtype == "bf16" else fb.F32,
                                 feat_dim=rp["r_q"], route_rule=args.route_rule,
                                 head_chunks=args.head_chunks, fused=args.order == "fused")
            cs.probe_feat = part.phi_q
            for _ in range(2):
                step(cs)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                step(cs)
            e1.record()
            torch.cuda.synchronize()
            sweep[rho] = {"step_ms": round(e0.elapsed_time(e1) / 3, 3),
                          "rho_exec": round(int(cs.routed_pairs.sum().item()) / (H * n * n)
                                            + m_eff / n, 6)}
            del cs
        out["density_sweep"] = sweep
    traffic = _traffic_from_profile(w.name)
    out["roofline"] = {
        "bound": "mfma",
        "kernel": ("attn_bf16_kernel<%d, %d%s>" % (d, _item_waves(w.heads, w.n, w.c_q),
                                                    ", fused correction" if call.fused else "")
                   if w.dtype == "bf16" else "attn_f32_kernel<%d>" % d),
        "achieved": round(attn_tflops, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(attn_tflops / peak, 4),
        "traffic": traffic,
        "launch": ("all heads, inside the timed calls" if call.chunks is None else
                   "all heads, back to back after the timed calls (the calls run it in %d head "
                   "ranges)" % len(call.chunks)),
    }
    def own_dense_ms():
        # this library with one query group, one K/V group and every cell kept
        zq = torch.zeros_like(lq)
        dcall = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, dtype, 1, 1, m=w.m, rank=w.r,
                                lam=w.lam, budget=w.n * w.n,
                                out_dtype=fb.BF16 if w.dtype == "bf16" else fb.F32)
        dcall.layout(zq, zq, q, k, v)
        dcall.route()
        dcall.attend()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            dcall.attend()
        e1.record()
        torch.cuda.synchronize()
        del dcall
        return e0.elapsed_time(e1) / 3

    if not args.no_dense:
        qq, kk, vv = q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0)
        for _ in range(2):
            torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)
        e1.record()
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / 3
        out["dense_sdpa_ms"] = round(dense_ms, 3)
        out["speedup_vs_dense_sdpa"] = round(dense_ms / ms_call, 3)
        del qq, kk, vv
        own_ms = own_dense_ms()
        out["dense_own_attn_ms"] = round(own_ms, 3)
        out["dense_own_tflops"] = round(4.0 * d * H * n * n / (own_ms * 1e-3) / 1e12, 1)
        # the whole call at 26% executed density against the faster dense attention
        c26 = fb.SparsePRCall(w.heads, w.n, w.n, w.head_dim, dtype, w.c_q, w.c_k, m=w.m,
                              rank=w.r, lam=w.lam, rho="0.26",
                              out_dtype=fb.BF16 if w.dtype == "bf16" else fb.F32,
                              feat_dim=rp["r_q"] if rcp else 0, route_rule=args.route_rule,
                              head_chunks=args.head_chunks, fused=args.order == "fused")
        c26.probe_feat = part.phi_q if rcp else None
        for _ in range(2):
            step(c26)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            step(c26)
        e1.record()
        torch.cuda.synchronize()
        ms26 = e0.elapsed_time(e1) / 5
        best_dense = min(dense_ms, own_ms)
        out["density_0.26"] = {
            "call_ms": round(ms26, 3),
            "rho_exec": round(int(c26.routed_pairs.sum().item()) / (H * n * n) + m_eff / n, 6),
            "faster_dense_ms": round(best_dense, 3),
            "speedup_vs_faster_dense": round(best_dense / ms26, 3),
        }
        del c26
    elif args.dense_own:
        own_ms = own_dense_ms()
        out["dense_own_attn_ms"] = round(own_ms, 3)
        out["dense_own_tflops"] = round(4.0 * d * H * n * n / (own_ms * 1e-3) / 1e12, 1)
    if not args.no_cpu_baseline:
        if args.estimator == "full" and args.route_rule == "global":
            # the same call once more, so its outputs are this workload's
            step(call)
            torch.cuda.synchronize()
            out["correction_error"] = correction_quality(w, arr, call, rcp_params=rp)
        out["cpu_baseline"] = cpu_baseline(w, arr, rcp_params=rp, estimator=args.estimator,
                                           route_rule=args.route_rule)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 1)
        out["cpu_baseline"]["value_fp64"] = round(out["cpu_baseline"]["value_fp64"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
