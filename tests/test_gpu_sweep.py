"""A seeded sweep of small random workloads through moe_forward against the
oracle: every kernel family the shapes can reach (decode, small-batch and
per-expert streaming, tiled, any-shape bf16, fp32), the GEMM modes, padded
plans, int32 / int64 ids, global ids with expert_begin, and calls without
weights. Same bars as tests/test_gpu_path.py; rows that carry no token (or
route nowhere) must be +0."""

import numpy as np
import pytest
import torch

import gen
import oracle
import top_reduce_amd as tr
from tests._gpu import as_f64, host, say, torch_dtype, upload
from tests._util import max_err, tolerance

pytestmark = pytest.mark.gpu

N_CASES = 120


def _case(i):
    rng = np.random.default_rng(1000 + i)
    f32 = rng.random() < 0.25
    if f32:
        H = int(rng.integers(1, 48)) * 8
        I = int(rng.integers(4, 200))
    else:
        H = int(rng.choice([256, 512, 768, 264, 136, 1024, 2880 // 4 * 4]))
        I = int(rng.choice([128, 256, 384, 72, 70, 200, 640]))
    # sizes the oracle finishes quickly
    T = int(rng.choice([1, 2, 3, 5, 8, 17, 40, 64, 100, 257, 600]))
    K = int(rng.choice([1, 2, 4, 8, 8, 16, 32] if T <= 64 else [1, 2, 4, 8]))
    E = int(rng.integers(1, 40))
    G = E * int(rng.choice([1, 1, 2, 4]))
    K = min(K, G)
    zipf_s = float(rng.choice([0.0, 0.5, 1.2]))
    flags = int(rng.choice([0, 0, 0, tr.FLAG_GEMM_FORCE_TILED, tr.FLAG_GEMM_FORCE_STREAM]))
    idx32 = bool(rng.random() < 0.3)
    weights = bool(rng.random() < 0.8)
    shift = bool(G >= 2 * E and rng.random() < 0.5)
    padded = bool(rng.random() < 0.2 and T >= 4)
    return dict(f32=f32, H=H, I=I, T=T, K=K, E=E, G=G, zipf_s=zipf_s, flags=flags,
                idx32=idx32, weights=weights, shift=shift, padded=padded,
                seed=int(rng.integers(1, 1 << 30)), B=int(rng.integers(1, 9)))


@pytest.mark.parametrize("i", range(N_CASES))
def test_forward_random_workload(i):
    c = _case(i)
    say(f"sweep case {i}: {c}")
    name = f"sweep{i}"
    gen.custom_spec(name, T=c["T"], K=c["K"], E=c["E"], G=c["G"], H=c["H"], I=c["I"],
                    dtype="f32" if c["f32"] else "bf16", zipf_s=c["zipf_s"], need_local=False,
                    seed=c["seed"])
    wl = gen.make_workload(name, with_weights=True)
    d = upload(wl)
    T, K, E, G = wl.T, wl.K, wl.E, wl.G
    # the ids as the rank receives them: global ids, optionally seen by the
    # rank owning experts [E, 2E) (a shift that keeps the local view), and
    # int32 or int64
    eb = E if c["shift"] else 0
    g = wl.global_idx
    ids = np.where(g >= 0, (g + eb) % G, -1) if c["shift"] else g
    idx_t = torch.from_numpy(np.ascontiguousarray(ids)).to(
        torch.int32 if c["idx32"] else torch.int64).cuda()
    local = wl.idx.copy()
    carry = np.ones(T, bool)
    kw = {}
    if c["padded"]:
        B = c["B"]
        nb = -(-T // B)
        counts = np.random.default_rng(c["seed"]).integers(-1, B + 2, size=nb).astype(np.int32)
        carry = (np.arange(T) % B) < counts[np.arange(T) // B]
        kw = dict(block_rows=B, block_counts=torch.from_numpy(counts).cuda())
        local = np.where(carry[:, None], local, -1)
    p = tr.plan(idx_t, E=E, H=wl.H, I=wl.I, dtype=torch_dtype(wl), expert_begin=eb,
                flags=c["flags"], **kw)
    w = d["w"] if c["weights"] else None
    y = host(tr.forward(p, d["x"], w, d["w1"], d["w2"]))
    wref = wl.weights if c["weights"] else np.ones_like(wl.weights)
    ref = oracle.forward(wl.x, local, wref, wl.w1, wl.w2, E)
    err, tol = max_err(as_f64(y), ref), tolerance(ref, wl.dtype)
    say(f"  max|d|={err:.3e} tol={tol:.3e}")
    assert err <= tol, f"case {i}: max|d|={err} > tol={tol}"
    empty = ~(local >= 0).any(1)
    assert (y[empty] == 0).all(), "rows without a local route must be +0"
