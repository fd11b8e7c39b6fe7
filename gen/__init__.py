"""Seeded synthetic inputs for one GPU's share of the expert-parallel MoE FFN.

This module only draws inputs. It holds none of the arithmetic of the path
(no routing scan, no expert MLP, no reduction): both the CPU oracle and the
HIP library receive exactly the arrays made here.

What a rank receives after dispatch (DeepEP issue #48, "How to apply MoE MLP
to recv_x ..."): each token arrives once as a row of ``recv_x`` together with
its top-k expert ids and gate weights; an id of -1 marks a route that is not
local to this rank or a padding row (DeepEP issue #760, repro script, where
padding TP ranks carry all -1 routes and zero weights).

Five workloads, all synthetic (the pages use model weights and traces that are
not available; only their shapes are kept):

* ``c1`` tiny fp32 check case.
* ``c2`` an EP16 share of a 256-expert, hidden-7168 model with uniform routing
  (the shapes of the DeepEP PR #1 measurement: hidden 7168, top-8 of 256).
* ``c3`` low-batch decode in the vLLM TP8/SP one-token layout of DeepEP issue
  #760: hidden 3584, 896 experts over 32 ranks (28 local), top-16 with weight
  1/16, one real row in every 8 (the rest all -1 and zero).
* ``c4`` a DP-padded global batch as in SGLang PR #6092: 8 workers of 120 rows,
  batch sizes [120,1,1,1,1,1,1,1], so 127 real rows in a 960-row buffer; Zipf
  (s=1.2) expert popularity so several local experts receive nothing.
* ``c5`` prefill: 16384 tokens, Zipf (s=1.0) popularity, top-8 of 256 with 32
  local.

Randomness: ``numpy.random.SeedSequence(seed).spawn(3 + 2E)`` gives one
independent PCG64 stream each for routing, gate logits, x, and then W1[e] and
W2[e] per local expert, so experts can be drawn in parallel and any subset can
be regenerated alone. Every float is drawn in fp32; bf16 tensors are the fp32
draw rounded once to nearest-even and are stored as raw ``uint16`` bits.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

__all__ = [
    "CONFIGS",
    "custom_spec",
    "Workload",
    "make_workload",
    "make_weights",
    "make_expert_outputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class ConfigSpec:
    name: str
    T: int               # received rows (buffer rows, pads included)
    K: int               # top-k slots per row
    E: int               # local experts
    G: int               # global experts
    H: int               # hidden
    I: int               # SwiGLU intermediate
    dtype: str           # "bf16" or "f32"
    routing: str         # "uniform" | "stride" | "zipf"
    zipf_s: float = 0.0
    need_local: bool = False   # resample a real row until >=1 route is local
    seed: int = 0


CONFIGS = {
    "c1": ConfigSpec("c1", T=64, K=2, E=8, G=8, H=256, I=128, dtype="f32",
                     routing="uniform", seed=101),
    "c2": ConfigSpec("c2", T=4096, K=8, E=16, G=256, H=7168, I=2048, dtype="bf16",
                     routing="uniform", need_local=True, seed=102),
    "c3": ConfigSpec("c3", T=8, K=16, E=28, G=896, H=3584, I=2048, dtype="bf16",
                     routing="stride", seed=103),
    "c4": ConfigSpec("c4", T=960, K=8, E=32, G=256, H=7168, I=2048, dtype="bf16",
                     routing="zipf", zipf_s=1.2, seed=104),
    "c5": ConfigSpec("c5", T=16384, K=8, E=32, G=256, H=7168, I=2048, dtype="bf16",
                     routing="zipf", zipf_s=1.0, need_local=True, seed=105),
}

# SGLang PR #6092: eight DP workers with batch sizes [120, 1, ..., 1] share one
# FFN buffer of 8 x 120 rows.
C4_WORKER_ROWS = 120
C4_WORKER_COUNTS = (120, 1, 1, 1, 1, 1, 1, 1)


def custom_spec(name: str, T: int, K: int, E: int, G: int, H: int, I: int, dtype: str = "bf16",
                routing: str = "zipf", zipf_s: float = 1.0, need_local: bool = True,
                seed: int = 1) -> ConfigSpec:
    """A workload spec outside the five named ones (reduced sizes for checks
    that the CPU oracle must finish in seconds). Registered under `name`."""
    spec = ConfigSpec(name, T=T, K=K, E=E, G=G, H=H, I=I, dtype=dtype, routing=routing,
                      zipf_s=zipf_s, need_local=need_local, seed=seed)
    CONFIGS[name] = spec
    return spec


@dataclasses.dataclass
class Workload:
    name: str
    T: int
    K: int
    E: int
    G: int
    H: int
    I: int
    dtype: str                 # "bf16" (arrays hold uint16 bits) or "f32"
    seed: int
    idx: np.ndarray            # int64 [T, K]: local id in [0, E) or -1
    global_idx: np.ndarray     # int64 [T, K]: global id in [0, G) or -1 (pads)
    weights: np.ndarray        # float32 [T, K]
    x: np.ndarray              # uint16 or float32 [T, H]
    real: np.ndarray           # bool [T]: row carries a token (not padding)
    w1: Optional[np.ndarray] = None   # [E, 2I, H]; rows [0, I) gate, [I, 2I) up
    w2: Optional[np.ndarray] = None   # [E, H, I]

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    nan = np.isnan(a)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16))
    r = r.astype(np.uint16)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, E: int):
    ss = np.random.SeedSequence(seed).spawn(3 + 2 * E)
    return ss[0], ss[1], ss[2], ss[3:3 + E], ss[3 + E:3 + 2 * E]


def _distinct_uniform(rng, n, G, K):
    # K distinct experts per row, uniform over G: first K of a random permutation.
    return np.argsort(rng.random((n, G)), axis=1, kind="stable")[:, :K]


def _distinct_weighted(rng, n, logp, K):
    # Weighted sampling of K distinct experts without replacement, drawn as the
    # top-K of log p + Gumbel noise (same law as drawing one at a time).
    keys = logp[None, :] + rng.gumbel(size=(n, logp.shape[0]))
    return np.argsort(-keys, axis=1, kind="stable")[:, :K]


def _route(spec: ConfigSpec, T: int, real: np.ndarray, rng) -> np.ndarray:
    """Global expert ids [T, K] for real rows; pad rows get -1."""
    K, G, E = spec.K, spec.G, spec.E
    gidx = np.full((T, K), -1, dtype=np.int64)
    rows = np.nonzero(real)[0]
    n = rows.size
    if n == 0:
        return gidx
    if spec.routing == "stride":
        # DeepEP issue #760 repro: topk ids k * (experts per rank), k = 0..15.
        gidx[rows] = np.arange(K, dtype=np.int64)[None, :] * E
        return gidx
    if spec.routing == "stride_random":
        draw = lambda m: _distinct_uniform(rng, m, G, K)
        need_local = True
    elif spec.routing == "stride_dense":
        # stress variant: all K slots of a real row name distinct local experts
        gidx[rows] = _distinct_uniform(rng, n, E, K)
        return gidx
    elif spec.routing == "uniform":
        draw = lambda m: _distinct_uniform(rng, m, G, K)
        need_local = spec.need_local
    elif spec.routing == "zipf":
        perm = rng.permutation(G)          # random popularity rank per expert
        p = (perm.astype(np.float64) + 1.0) ** (-spec.zipf_s)
        logp = np.log(p / p.sum())
        draw = lambda m: _distinct_weighted(rng, m, logp, K)
        need_local = spec.need_local
    else:
        raise ValueError(spec.routing)
    sel = draw(n).astype(np.int64)
    if need_local:
        while True:
            bad = ~((sel < E).any(axis=1))
            if not bad.any():
                break
            sel[bad] = draw(int(bad.sum()))
    gidx[rows] = sel
    return gidx


def make_workload(name: str, T: Optional[int] = None, seed: Optional[int] = None,
                  variant: str = "", with_weights: bool = False) -> Workload:
    """Routing, gate weights and x for a named workload.

    ``T`` overrides the row count (c3 uses T in {1, 2, 4, 8, 64}; the others
    accept a smaller T for quick checks: rows are drawn the same way).
    ``variant="random"`` selects the random routing variant of c3 and
    ``variant="dense"`` its stress variant (all 16 slots of a real row local);
    for c3 the default seed is 103 + T (+1000 random, +2000 dense).
    """
    spec = CONFIGS[name]
    if variant in ("random", "dense"):
        if name != "c3":
            raise ValueError(f"the {variant} variant exists for c3 only")
        spec = dataclasses.replace(spec, routing="stride_" + variant)
    T = spec.T if T is None else int(T)
    if seed is None:
        seed = spec.seed + (T if name == "c3" else 0) + {"": 0, "random": 1000, "dense": 2000}[variant]
    s_route, s_logit, s_x, _, _ = _streams(seed, spec.E)

    if name == "c3":
        real = (np.arange(T) % 8) == 0          # one real row in every 8
    elif name == "c4":
        real = np.zeros(T, dtype=bool)
        for j, c in enumerate(C4_WORKER_COUNTS):
            lo = j * C4_WORKER_ROWS
            real[lo:min(lo + c, T)] = True
    else:
        real = np.ones(T, dtype=bool)

    gidx = _route(spec, T, real, np.random.default_rng(s_route))

    K = spec.K
    if spec.routing in ("stride", "stride_random", "stride_dense"):
        weights = np.zeros((T, K), dtype=np.float32)
        weights[real] = np.float32(1.0 / K)
    else:
        logits = np.random.default_rng(s_logit).standard_normal((T, K), dtype=np.float32)
        z = logits.astype(np.float64)
        z = np.exp(z - z.max(axis=1, keepdims=True))
        weights = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
        weights[~real] = 0.0

    xf = np.random.default_rng(s_x).standard_normal((T, spec.H), dtype=np.float32)
    xf[~real] = 0.0
    x = f32_to_bf16_bits(xf) if spec.dtype == "bf16" else xf

    # Received form: ids local to this rank (expert_begin = 0) are kept, the
    # rest become -1.
    idx = np.where((gidx >= 0) & (gidx < spec.E), gidx, -1).astype(np.int64)

    wl = Workload(name=name, T=T, K=K, E=spec.E, G=spec.G, H=spec.H, I=spec.I,
                  dtype=spec.dtype, seed=seed, idx=idx, global_idx=gidx,
                  weights=weights, x=x, real=real)
    if with_weights:
        make_weights(wl)
    return wl


def _normal(stream, shape, std, dtype):
    a = np.random.default_rng(stream).standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def make_weights(wl: Workload, threads: Optional[int] = None) -> Workload:
    """W1[e] ~ N(0, 1/sqrt(H)) of shape [2I, H] and W2[e] ~ N(0, 1/sqrt(I)) of
    shape [H, I] for every local expert (standard deviation 1/sqrt(fan_in))."""
    _, _, _, s_w1, s_w2 = _streams(wl.seed, wl.E)
    E, H, I = wl.E, wl.H, wl.I
    dt = wl.np_dtype
    w1 = np.empty((E, 2 * I, H), dtype=dt)
    w2 = np.empty((E, H, I), dtype=dt)

    def job(e):
        w1[e] = _normal(s_w1[e], (2 * I, H), 1.0 / np.sqrt(H), wl.dtype)
        w2[e] = _normal(s_w2[e], (H, I), 1.0 / np.sqrt(I), wl.dtype)

    n = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=n) as ex:
        list(ex.map(job, range(E)))
    wl.w1, wl.w2 = w1, w2
    return wl


def make_expert_outputs(R: int, H: int, dtype: str, seed: int) -> np.ndarray:
    """Synthetic expert outputs O [R, H] ~ N(0, 1) for reduce-only checks."""
    a = np.random.default_rng(np.random.SeedSequence([seed, 7])).standard_normal((R, H), dtype=np.float32)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a
