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


def _check(idx_np, E, eb=0, idx_dtype=torch.int64, H=256, I=128, flags=0):
    T, K = idx_np.shape
    say(f"route T={T} K={K} E={E} eb={eb} idx={idx_dtype} flags={flags}")
    idx = torch.from_numpy(np.ascontiguousarray(idx_np)).to(idx_dtype).cuda()
    p = tr.plan(idx, E=E, H=H, I=I, dtype=torch.bfloat16, expert_begin=eb, flags=flags)
    # fewest routes of an expert the tiled GEMM takes, per the plan's mode
    # (the automatic mode streams every expert of a batch of at most 128
    # expanded rows)
    lo = (1 if flags & tr.FLAG_GEMM_FORCE_TILED
          else np.iinfo(np.int64).max if flags & tr.FLAG_GEMM_FORCE_STREAM or T * K <= 128
          else 33)
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
    # received row with exactly one local slot whose expert the tiled GEMM
    # takes (more than 32 routes in the automatic mode), -1 for every other
    # row
    rm = ref["row_map"]
    n_loc = (rm >= 0).sum(1)
    want = np.full(R, -1, np.int64)
    tt, kk = np.nonzero((rm >= 0) & (n_loc[:, None] == 1))
    tiled = ref["counts"][idx_np[tt, kk] - eb] >= lo
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
    # experts of the streaming GEMM and of the tiled GEMM
    c = ref["counts"]
    assert int(v["stats"][6]) == int(((c > 0) & (c < lo)).sum())
    assert int(v["stats"][7]) == int((c >= lo).sum())


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


def test_route_small_batches():
    """The single-block kernel of T * K <= 1024 slots (decode batches): every
    expert count up to 1024, K = 1 .. 32, rows straddling waves (K = 3),
    one hot expert, and the GEMM modes."""
    rng = np.random.default_rng(6)
    _check(rng.integers(-1, 1024, size=(32, 32)), 1024)            # max slots, max E
    _check(rng.integers(-1, 1024, size=(2, 32)), 1024)             # 64 slots: one wave, 16 experts a thread
    _check(rng.integers(-1, 1024, size=(8, 32)), 1024)             # 256 slots: four waves
    _check(rng.integers(-1, 3, size=(60, 1)), 3)
    _check(rng.integers(-1, 20, size=(13, 5)), 17)                 # 65 slots
    _check(rng.integers(-2, 12, size=(341, 3)), 10)                # K = 3, 1023 slots
    _check(np.zeros((1, 1), np.int64), 1)                          # one slot
    _check(np.full((64, 16), 3, np.int64), 4)                      # one expert, 16 per row
    _check(rng.integers(0, 5, size=(1024, 1)), 5)                  # single-slot rows, tiled
    _check(rng.integers(-1, 40, size=(3, 7)), 40, idx_dtype=torch.int32)
    g = rng.integers(-1, 64, size=(100, 8))
    _check(np.where(g >= 0, g + 100, -1), 16, eb=108)             # expert_begin, foreign ids
    for fl in (tr.FLAG_GEMM_FORCE_TILED, tr.FLAG_GEMM_FORCE_STREAM):
        _check(rng.integers(-1, 6, size=(200, 4)), 6, flags=fl)
        _check(rng.integers(-1, 40, size=(1000, 1)), 40, flags=fl)
    # just past the single-block kernel: a few blocks of the general kernels
    _check(rng.integers(-1, 40, size=(1025, 1)), 40)
    _check(rng.integers(-1, 28, size=(256, 16)), 28)


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


@pytest.mark.parametrize("i", range(60))
def test_route_random_shapes(i):
    """Seeded random shapes on both sides of every kernel switch (one block
    of 64 / 256 / 1024 threads, the general single block, two kernels with
    few or many blocks; 1 to 1024 experts; K up to 32; int32 ids; foreign and
    shifted ids; every GEMM mode), bit-exact against the oracle."""
    rng = np.random.default_rng(2000 + i)
    K = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    T = int(rng.choice([1, 3, 16, 63, 100, 300, 1000, 3000, 20000, 60000]))
    T = max(1, min(T, 200000 // K))
    E = int(rng.choice([1, 2, 7, 28, 64, 100, 256, 1000, 1024]))
    lo, hi = -3, E + int(rng.integers(0, 3 * E + 1))
    idx = rng.integers(lo, hi, size=(T, K))
    eb = int(rng.choice([0, 0, 5, E]))
    flags = int(rng.choice([0, 0, tr.FLAG_GEMM_FORCE_TILED, tr.FLAG_GEMM_FORCE_STREAM]))
    dt = torch.int32 if rng.random() < 0.3 else torch.int64
    _check(np.where(idx >= 0, idx + eb, idx), E, eb=eb, idx_dtype=dt, flags=flags)
