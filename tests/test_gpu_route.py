"""moe_route_scan on the GPU vs the oracle: bit-exact counts, offsets,
row_map, row_src, row_k, row_dst and stats, for every workload at full size and for
edge cases (empty, all padding, one hot expert, duplicates, foreign ids,
int32 ids, expert_begin, maximal E, ragged multi-block inputs)."""

import numpy as np
import pytest
import torch

import gen
import oracle
import top_reduce_amd as tr
from tests._gpu import say

pytestmark = pytest.mark.gpu


def _check(idx_np, E, eb=0, idx_dtype=torch.int64, H=256, I=128):
    T, K = idx_np.shape
    say(f"route T={T} K={K} E={E} eb={eb} idx={idx_dtype}")
    idx = torch.from_numpy(np.ascontiguousarray(idx_np)).to(idx_dtype).cuda()
    p = tr.plan(idx, E=E, H=H, I=I, dtype=torch.bfloat16, expert_begin=eb)
    stats = tr.plan_stats(p)
    v = p.views()
    ref = oracle.route(idx_np, E, eb)
    R = ref["R"]
    assert np.array_equal(v["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(v["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(v["row_map"].cpu().numpy(), ref["row_map"])
    assert np.array_equal(v["row_src"][:R].cpu().numpy(), ref["row_src"])
    assert np.array_equal(v["row_k"][:R].cpu().numpy(), ref["row_k"])
    # row_dst by its definition from the oracle's route: the slot of a
    # received row with exactly one local slot whose expert has more than 32
    # routes (the tiled GEMM's experts), -1 for every other row
    rm = ref["row_map"]
    n_loc = (rm >= 0).sum(1)
    want = np.full(R, -1, np.int64)
    tt, kk = np.nonzero((rm >= 0) & (n_loc[:, None] == 1))
    tiled = ref["counts"][idx_np[tt, kk] - eb] > 32
    tt, kk = tt[tiled], kk[tiled]
    want[rm[tt, kk]] = tt * K + kk
    assert np.array_equal(v["row_dst"][:R].cpu().numpy(), want)
    # tok_rest: every other received row, in ascending order
    rest = np.setdiff1d(np.arange(T), tt)
    n_rest = int(v["stats"][4])
    assert n_rest == rest.size
    assert np.array_equal(v["tok_rest"][:n_rest].cpu().numpy(), rest)
    local = (idx_np >= eb) & (idx_np < eb + E)
    assert stats == (R, int(local.any(1).sum()) if T else 0, int((~local).sum()),
                     int((ref["counts"] == 0).sum()))
    # experts of the streaming GEMM (1..32 routes) and of the tiled GEMM (> 32)
    c = ref["counts"]
    assert int(v["stats"][6]) == int(((c > 0) & (c <= 32)).sum())
    assert int(v["stats"][7]) == int((c > 32).sum())


@pytest.mark.parametrize("name,T", [("c1", None), ("c2", None), ("c3", 1), ("c3", 8), ("c3", 64),
                                    ("c4", None), ("c5", None)])
def test_route_configs(name, T):
    wl = gen.make_workload(name, T=T)
    _check(wl.idx, wl.E)


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_route_global_ids_and_int32(name):
    wl = gen.make_workload(name)
    _check(wl.global_idx, wl.E, idx_dtype=torch.int32)
    # the same routing as seen by the rank owning experts [3E, 4E)
    g = np.where(wl.global_idx >= 0, (wl.global_idx + 3 * wl.E) % wl.G, -1)
    _check(g, wl.E, eb=3 * wl.E)


def test_route_edge_cases():
    rng = np.random.default_rng(5)
    _check(np.zeros((0, 8), np.int64), 4)                          # T = 0
    _check(-np.ones((100, 8), np.int64), 16)                       # all padding
    _check(np.full((3000, 8), 5, np.int64), 16)                    # one expert, duplicates
    _check(np.zeros((777, 1), np.int64), 1)                        # K = 1, E = 1
    _check(rng.integers(-5, 40, size=(5000, 8)), 16)               # foreign ids on both sides
    _check(rng.integers(-1, 1024, size=(4099, 32)), 1024)          # max E and K, ragged blocks
    _check(rng.integers(-1, 3, size=(70000, 3)), 3)                # many blocks, few experts
    _check(rng.integers(0, 8, size=(513, 8)), 8, idx_dtype=torch.int32)
    # the partial sums of 32 < E <= 256 experts over ~254 blocks (batched
    # loads per thread) and of blocks with more slots than the LDS slot cache
    _check(rng.integers(-1, 64, size=(20000, 8)), 64)
    _check(rng.integers(-1, 256, size=(30000, 8)), 256)
    _check(rng.integers(-1, 48, size=(40000, 32)), 48)


def test_route_deterministic():
    wl = gen.make_workload("c5")
    idx = torch.from_numpy(wl.idx).cuda()
    a = tr.plan(idx, E=wl.E, H=256, I=128).views()
    b = tr.plan(idx, E=wl.E, H=256, I=128).views()
    R = int(a["stats"][0])
    for f in ("counts", "offsets", "row_map", "stats"):
        assert torch.equal(a[f], b[f]), f
    for f in ("row_src", "row_k"):          # defined for the first R rows only
        assert torch.equal(a[f][:R], b[f][:R]), f
