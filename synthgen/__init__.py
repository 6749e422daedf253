"""Seeded synthetic inputs for one SparsePR attention call.

This module only draws random numbers and lays them out; it holds none of
the method's arithmetic (no grouping, routing, attention or fitting).  It is
the single source of inputs shared by the CPU oracle and the GPU path.

Workloads.  The pages evaluate video diffusion transformers whose attention
calls see 720p latents (45 x 80 spatial tokens) over 21 or 33 latent frames,
and a 480p CogVideoX-like latent (30 x 45 over 13 frames).  Real activations
and model weights are not available, so each call is replaced by a Gaussian
mixture with the same token counts, head counts and head dimensions:

* every token n carries one mixture label c_n, drawn uniformly;
* q_n = mu^Q[c_n] + 0.5 * eps_q + 0.3 * pos(n),
  k_n = mu^K[c_n] + 0.5 * eps_k + 0.3 * pos(n),  v_n ~ N(0, I);
* component means mu^Q, mu^K ~ N(0, 1.5^2 I), drawn independently for Q and
  K (variant ``near_exact`` uses mu^K = mu^Q, which makes the routed cells
  hold nearly all attention mass);
* pos(n) is a 3-D sinusoidal position code of the token's (t, y, x) cell.

The query partition is the mixture label.  The key/value partition is the
label too, or, with ``kv_split = s``, label c is cut into s consecutive runs
of its tokens (in ascending token order), giving group s*c + j.

Per head h the draws come from numpy ``PCG64(SeedSequence([seed, h]))`` in
the order: labels, mu^Q, mu^K, Q noise, K noise, V.  bf16 workloads are
rounded from float32 to bfloat16 with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
from fractions import Fraction
from typing import Optional

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "small_workload",
    "make_head",
    "make_call",
    "make_call_arrays",
    "position_code",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "RCP_PARAMS",
    "rcp_init",
    "rcp_init_arrays",
    "drift_head",
    "drift_arrays",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    n: int                 # N_q = N_k tokens (self-attention)
    head_dim: int
    dtype: str             # "bf16" or "f32"
    components: int        # mixture components = query groups C_q
    kv_split: int          # K/V groups per component (C_k = components * kv_split)
    grid: Optional[tuple]  # (T, Y, X) latent grid, or None for no position code
    rho: str               # executed-pair density target, decimal string
    m: int = 64            # probe rows per head
    r: int = 16            # output-subspace rank
    lam: float = 0.1       # ridge strength
    seed: int = 0
    mean_std: float = 1.5
    spread: float = 0.5
    pos_scale: float = 0.3

    @property
    def c_q(self) -> int:
        return self.components

    @property
    def c_k(self) -> int:
        return self.components * self.kv_split

    @property
    def rho_fraction(self) -> Fraction:
        return Fraction(self.rho)


WORKLOADS = {
    # single fp32 head, 32 x 32 cells, no position code
    "tiny_fp32": Workload("tiny_fp32", heads=1, n=4096, head_dim=64, dtype="f32",
                          components=32, kv_split=1, grid=None, rho="0.26", seed=0),
    # CogVideoX-like 480p latent, 13 x 30 x 45 tokens
    "cogvideox": Workload("cogvideox", heads=8, n=17550, head_dim=64, dtype="bf16",
                          components=64, kv_split=1, grid=(13, 30, 45), rho="0.26", seed=1),
    # Wan2.2-like 720p, 81 frames -> 21 x 45 x 80 tokens
    "wan": Workload("wan", heads=40, n=75600, head_dim=128, dtype="bf16",
                    components=256, kv_split=4, grid=(21, 45, 80), rho="0.22", seed=2),
    # HunyuanVideo-like 720p, 129 frames -> 33 x 45 x 80 tokens
    "hunyuan": Workload("hunyuan", heads=24, n=118800, head_dim=128, dtype="bf16",
                        components=256, kv_split=4, grid=(33, 45, 80), rho="0.26", seed=3),
    # the Wan-like call with the partition built from the activations
    # (response-coupled partitioning); the mixture labels are not used
    "wan_rcp": Workload("wan_rcp", heads=40, n=75600, head_dim=128, dtype="bf16",
                        components=256, kv_split=4, grid=(21, 45, 80), rho="0.22", seed=4),
}

# Response-coupled partitioning settings of the pages' full pipeline: M_s
# sampled query rows, coordinate ranks r_K / r_Q, Lloyd iterations; the
# requested group counts are the workload's C_k and C_q.
RCP_PARAMS = {"m_s": 256, "r_k": 48, "r_q": 64, "iters": 10}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def small_workload(name="small", heads=2, n=700, head_dim=64, dtype="bf16", components=8,
                   kv_split=1, grid=None, rho="0.3", m=64, r=16, lam=0.1, seed=11,
                   **kw) -> Workload:
    """A reduced workload with the same generator (test sizes)."""
    return Workload(name, heads=heads, n=n, head_dim=head_dim, dtype=dtype,
                    components=components, kv_split=kv_split, grid=grid, rho=rho,
                    m=m, r=r, lam=lam, seed=seed, **kw)


# ----------------------------------------------------------------------------
# bfloat16 bit helpers (input encoding only)
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# position code
# ----------------------------------------------------------------------------

def position_code(grid, d: int) -> np.ndarray:
    """3-D sinusoidal code, float32 [T*Y*X, d].

    Token n = (t*Y + y)*X + x.  Channels split as [t | y | x] with
    d_y = d_x = 2*floor(d/6) and d_t = d - d_y - d_x.  An axis chunk of 2m
    channels holds sin(p*w_j) for j < m followed by cos(p*w_j), with
    w_j = 10000^(-j/m).
    """
    T, Y, X = grid
    dy = dx = 2 * (d // 6)
    dt = d - dy - dx
    t = np.repeat(np.arange(T), Y * X)
    y = np.tile(np.repeat(np.arange(Y), X), T)
    x = np.tile(np.arange(X), T * Y)

    def axis(p, width):
        m = width // 2
        w = 10000.0 ** (-np.arange(m) / m)
        ang = p[:, None].astype(np.float64) * w[None, :]
        return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)

    return np.concatenate([axis(t, dt), axis(y, dy), axis(x, dx)], axis=1).astype(np.float32)


# ----------------------------------------------------------------------------
# per-head draw
# ----------------------------------------------------------------------------

def _kv_labels(labels: np.ndarray, components: int, split: int) -> np.ndarray:
    if split == 1:
        return labels.copy()
    out = np.empty_like(labels)
    for c in range(components):
        idx = np.nonzero(labels == c)[0]          # ascending token order
        n = idx.size
        bounds = [(j * n) // split for j in range(split + 1)]
        for j in range(split):
            out[idx[bounds[j]:bounds[j + 1]]] = split * c + j
    return out


class _Scratch:
    """Per-shape scratch buffers reused across heads (fresh allocations are
    avoided: first-touch page faults dominate generation time otherwise)."""

    def __init__(self, n, d):
        self.f = np.empty((n, d), np.float32)
        self.g = np.empty((n, d), np.float32)
        self.u = np.empty((n, d), np.uint32)


def _encode_into(src: np.ndarray, dst: np.ndarray, scratch: _Scratch, bf16: bool):
    """src float32 [n, d] -> dst (uint16 bf16 bits, nearest-even, or float32)."""
    if not bf16:
        np.copyto(dst, src)
        return
    u = src.view(np.uint32)
    t = scratch.u
    np.right_shift(u, np.uint32(16), out=t)
    np.bitwise_and(t, np.uint32(1), out=t)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(u, t, out=t)
    np.right_shift(t, np.uint32(16), out=t)
    np.copyto(dst, t, casting="unsafe")
    nan = np.isnan(src)
    if nan.any():
        dst[nan] = np.uint16(0x7FC0)


def _draw_head_into(w: Workload, h: int, variant: str, pos_scaled, qo, ko, vo, scratch):
    """Draws head h and writes the encoded q, k, v into qo, ko, vo ([n, d]
    uint16 bf16 bits or float32).  Returns (labels_q, labels_kv)."""
    if variant not in ("default", "near_exact"):
        raise ValueError(variant)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, h])))
    n, d, C = w.n, w.head_dim, w.components
    bf16 = w.dtype == "bf16"
    if w.dtype not in ("bf16", "f32"):
        raise ValueError(w.dtype)
    labels = rng.integers(0, C, size=n).astype(np.int32)
    mu_q = (rng.standard_normal((C, d), dtype=np.float32) * np.float32(w.mean_std))
    mu_k = (rng.standard_normal((C, d), dtype=np.float32) * np.float32(w.mean_std))
    if variant == "near_exact":
        mu_k = mu_q
    f, g = scratch.f, scratch.g
    for mu, out in ((mu_q, qo), (mu_k, ko)):
        rng.standard_normal(dtype=np.float32, out=f)
        f *= np.float32(w.spread)
        np.take(mu, labels, axis=0, out=g, mode="clip")  # unbuffered gather
        f += g
        if pos_scaled is not None:
            f += pos_scaled
        _encode_into(f, out, scratch, bf16)
    rng.standard_normal(dtype=np.float32, out=f)
    _encode_into(f, vo, scratch, bf16)
    return labels, _kv_labels(labels, C, w.kv_split).astype(np.int32)


def _pos_scaled(w: Workload, pos=None):
    if w.grid is None:
        return None
    if pos is None:
        pos = position_code(w.grid, w.head_dim)
    return pos * np.float32(w.pos_scale)


def make_head(w: Workload, h: int, variant: str = "default", pos: Optional[np.ndarray] = None):
    """Draw head h.  Returns dict with float32 q, k, v [N, d] (bf16-exact for
    bf16 workloads), uint16 bits (bf16 only) and int32 labels_q, labels_kv."""
    n, d = w.n, w.head_dim
    bf16 = w.dtype == "bf16"
    et = np.uint16 if bf16 else np.float32
    qo, ko, vo = (np.empty((n, d), et) for _ in range(3))
    lq, lk = _draw_head_into(w, h, variant, _pos_scaled(w, pos), qo, ko, vo, _Scratch(n, d))
    out = {"labels_q": lq, "labels_kv": lk}
    if bf16:
        for name, arr in (("q", qo), ("k", ko), ("v", vo)):
            out[name + "_bits"] = arr
            out[name] = bf16_bits_to_f32(arr)
    else:
        out["q"], out["k"], out["v"] = qo, ko, vo
    return out


def make_call(w: Workload, variant: str = "default", heads=None):
    """Draw every head (or the listed ones).  Returns a list of per-head dicts."""
    pos = position_code(w.grid, w.head_dim) if w.grid is not None else None
    hs = range(w.heads) if heads is None else heads
    return [make_head(w, h, variant, pos) for h in hs]


def make_call_arrays(w: Workload, variant: str = "default", threads: Optional[int] = None):
    """All heads packed for upload: q, k, v [H, N, d] (uint16 bf16 bits or
    float32) and labels_q, labels_kv int32 [H, N].  Same values as make_head.
    Heads are drawn in parallel threads (independent generators per head)."""
    import concurrent.futures as cf
    import os

    n, d, H = w.n, w.head_dim, w.heads
    et = np.uint16 if w.dtype == "bf16" else np.float32
    q, k, v = (np.empty((H, n, d), et) for _ in range(3))
    lq = np.empty((H, n), np.int32)
    lk = np.empty((H, n), np.int32)
    ps = _pos_scaled(w)
    nt = threads or max(1, min(8, os.cpu_count() or 1, H))

    def work(tid):
        scratch = _Scratch(n, d)
        for h in range(tid, H, nt):
            lq[h], lk[h] = _draw_head_into(w, h, variant, ps, q[h], k[h], v[h], scratch)

    with cf.ThreadPoolExecutor(nt) as ex:
        list(ex.map(work, range(nt)))
    return {"q": q, "k": k, "v": v, "labels_q": lq, "labels_kv": lk}


def rcp_init(w: Workload, h: int):
    """Initial k-means centre indices of head h for response-coupled
    partitioning: C_k then C_q token indices drawn uniformly with replacement
    from numpy PCG64(SeedSequence([seed, h, 1])) (a stream of its own, so the
    activation draws are unchanged)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, h, 1])))
    init_k = g.integers(0, w.n, size=w.c_k, dtype=np.int64).astype(np.int32)
    init_q = g.integers(0, w.n, size=w.c_q, dtype=np.int64).astype(np.int32)
    return init_k, init_q


def rcp_init_arrays(w: Workload):
    """rcp_init for every head: int32 [H, C_k] and [H, C_q]."""
    ik = np.empty((w.heads, w.c_k), np.int32)
    iq = np.empty((w.heads, w.c_q), np.int32)
    for h in range(w.heads):
        ik[h], iq[h] = rcp_init(w, h)
    return ik, iq


def _drift_gen(w: Workload, h: int, step: int):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, h, 2, step])))


def drift_head(w: Workload, hd: dict, h: int, step: int, eps: float, names=("q", "k", "v")):
    """The activations of a later call of the same layer (the next denoising
    step): x + eps * N(0, 1) for each tensor in `names`, drawn in that order
    from PCG64(SeedSequence([seed, h, 2, step])), nearest-even bf16 for bf16
    workloads.  Labels are copied unchanged."""
    g = _drift_gen(w, h, step)
    out = dict(hd)
    for name in names:
        x = hd[name].astype(np.float32) + np.float32(eps) * g.standard_normal(
            hd[name].shape, dtype=np.float32)
        if w.dtype == "bf16":
            out[name + "_bits"] = f32_to_bf16_bits(x)
            out[name] = bf16_bits_to_f32(out[name + "_bits"])
        else:
            out[name] = x
    return out


def drift_arrays(w: Workload, arr: dict, step: int, eps: float, names=("q", "k"),
                 threads: Optional[int] = None):
    """drift_head for packed [H, N, d] arrays (make_call_arrays), in place of
    a copy; same values head by head.  Heads run in parallel threads."""
    import concurrent.futures as cf
    import os

    out = dict(arr)
    for name in names:
        out[name] = np.empty_like(arr[name])
    bf16 = w.dtype == "bf16"
    nt = threads or max(1, min(8, os.cpu_count() or 1, w.heads))

    def work(tid):
        for h in range(tid, w.heads, nt):
            g = _drift_gen(w, h, step)
            for name in names:
                src = bf16_bits_to_f32(arr[name][h]) if bf16 else arr[name][h]
                x = src + np.float32(eps) * g.standard_normal(src.shape, dtype=np.float32)
                out[name][h] = f32_to_bf16_bits(x) if bf16 else x

    with cf.ThreadPoolExecutor(nt) as ex:
        list(ex.map(work, range(nt)))
    return out
