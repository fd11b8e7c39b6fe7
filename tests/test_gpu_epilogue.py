"""The cross-rank combine epilogue (moe_combine_epilogue) through the C ABI
vs the oracle: element by element on random receive buffers (bf16 and fp32,
ragged hidden sizes, absent and repeated contributions), the DeepEP issue #760
combine-only repro emulated with 32 ranks on one GPU (exact 1 and 0), and the
edge cases. Bars: bf16 max|d| <= 1e-2 max|ref| + 1e-3, fp32 1e-5 max|ref|;
exact where the sums are exact."""

import numpy as np
import pytest
import torch

import gen
import oracle
import top_reduce_amd as tr
from tests._gpu import as_f64, dev, host, say
from tests._util import load_golden, max_err, tolerance

pytestmark = pytest.mark.gpu


def _recv(rng, N, H, dtype):
    f = rng.standard_normal((N, H)).astype(np.float32)
    return gen.f32_to_bf16_bits(f) if dtype == "bf16" else f


def _src(rng, T, J, N, p_absent=0.3):
    src = rng.integers(0, max(N, 1), (T, J)).astype(np.int32)
    src[rng.random((T, J)) < p_absent] = -1
    return src


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,J,N,H", [(1, 32, 32, 3584), (5, 16, 80, 7168), (64, 8, 300, 256),
                                     (300, 33, 1000, 520), (3, 1, 7, 8)])
def test_epilogue_matches_oracle(dtype, T, J, N, H):
    rng = np.random.default_rng(T * 1000 + J)
    recv = _recv(rng, N, H, dtype)
    src = _src(rng, T, J, N)
    say(f"epilogue {dtype} T={T} J={J} N={N} H={H}")
    y = tr.combine_epilogue(dev(src), dev(recv))
    torch.cuda.synchronize()
    ref = oracle.combine_epilogue(src, recv)
    got = as_f64(host(y))
    err, tol = max_err(got, ref), tolerance(ref, dtype)
    say(f"  max|d|={err:.3e} tol={tol:.3e}")
    assert err <= tol


def test_epilogue_deepep760_32_ranks():
    """The combine-only repro on one GPU: 32 destination ranks each run the
    route scan and the weighted reduce of their 28-expert range over the 32
    source rows with the repro's fake expert output (1 for every expanded
    row), then the epilogue sums the 32 rank partials of every source row.
    Real rows (TP rank 0 of each DP group) must come out exactly 1, padding
    rows exactly 0."""
    g = load_golden("deepep760_combine_only.txt")
    W, tp, topk, E, H = g["world_size"], g["tp_size"], g["topk"], g["local_experts"], g["hidden"]
    idx = -np.ones((W, topk), np.int64)
    w = np.zeros((W, topk), np.float32)
    real = np.array([r % tp == 0 for r in range(W)])
    idx[real] = np.arange(topk) * E
    w[real] = g["topk_weight"]
    idx_d, w_d = torch.from_numpy(idx).cuda(), torch.from_numpy(w).cuda()
    partials = torch.empty((W, W, H), dtype=torch.bfloat16, device="cuda")   # [rank, row, H]
    for rank in range(W):
        p = tr.plan(idx_d, E=E, H=H, I=128, expert_begin=rank * E)
        ones = torch.ones((W * topk, H), dtype=torch.bfloat16, device="cuda")
        tr.combine_reduce(p, w_d, y=partials[rank], expert_out=ones)
    src = (np.arange(W)[None, :] * W + np.arange(W)[:, None]).astype(np.int32)   # [row, rank]
    y = tr.combine_epilogue(dev(src), partials.view(W * W, H))
    torch.cuda.synchronize()
    got = host(y)
    one, zero = gen.f32_to_bf16_bits(np.float32(1.0)), np.uint16(0)
    assert np.all(got[real] == one), "real rows must combine to exactly 1"
    assert np.all(got[~real] == zero), "padding rows must combine to exactly +0"


def test_epilogue_absent_and_out_of_range_rows():
    """A token with no contribution is +0; rows at or past n_recv count as
    absent (the oracle sees them as -1)."""
    rng = np.random.default_rng(3)
    N, H = 40, 512
    recv = _recv(rng, N, H, "bf16")
    src = _src(rng, 12, 6, N)
    src[4] = -1
    src[7, :3] = [N, N + 5, 2 ** 30]
    y = host(tr.combine_epilogue(dev(src), dev(recv)))
    assert np.all(y[4] == 0)
    ref_src = np.where(src >= N, -1, src).astype(np.int32)
    ref = oracle.combine_epilogue(ref_src, recv)
    assert max_err(as_f64(y), ref) <= tolerance(ref, "bf16")


def test_epilogue_empty_and_deterministic():
    rng = np.random.default_rng(5)
    recv = dev(_recv(rng, 64, 3584, "bf16"))
    y0 = tr.combine_epilogue(torch.empty((0, 4), dtype=torch.int32, device="cuda"), recv)
    assert y0.shape == (0, 3584)
    src = dev(_src(rng, 8, 16, 64))
    a = tr.combine_epilogue(src, recv)
    b = tr.combine_epilogue(src, recv)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
