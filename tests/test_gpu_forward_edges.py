"""moe_forward against the oracle on the edge cases of the method, through the
C ABI: every received row compared (or, where the oracle would take minutes, a
sample of at least 512 rows that includes every segment edge).

Cases: NaN in every non-local weight slot (never read: the bits equal the
finite run; DeepEP issue #760 repro masks routes below 0 before weighting),
T = 0, top-1 routing (every routed row then has one local slot, so GEMM2 writes
all outputs straight to y), a row naming the same local expert twice, global
ids with expert_begin = 3E (int32 and int64 ids), one expert holding every
route over more than two rounds of GEMM tiles, and y aliasing x on the
workloads whose GEMMs run as three launches (GEMM1's last round beside early
GEMM2 tiles). Bars: bf16 max|d| <= 1e-2 max|ref| + 1e-3; fp32 1e-5 max|ref|.
"""

import numpy as np
import pytest
import torch

import gen
import oracle
import top_reduce_amd as tr
from tests._gpu import as_f64, dev, host, sample_tokens, say, torch_dtype, upload
from tests._util import max_err, tolerance

pytestmark = pytest.mark.gpu

# several m-tiles with ragged tails on 8 experts (one round of tiles)
gen.custom_spec("edge_mid", T=1024, K=8, E=8, G=64, H=1024, I=512, zipf_s=1.0, seed=21)
# top-1: 8192 rows over 8 experts, ~4 m-tiles each; GEMM1 has 16 n-tiles per
# m-tile, about 576 tiles: two whole rounds of 256 blocks and a partial one,
# so the forward runs its three-launch GEMM schedule and every output row goes
# through GEMM2's y epilogue
gen.custom_spec("edge_k1_split", T=8192, K=1, E=8, G=8, H=512, I=2048, routing="uniform",
                seed=22)
# as in test_gpu_path: 17 m-tiles per expert, GEMM1 544 tiles (three-launch)
gen.custom_spec("edge_split", T=4200, K=8, E=8, G=8, H=2048, I=512, routing="uniform", seed=11)
gen.custom_spec("edge_f32", T=300, K=4, E=6, G=12, H=264, I=72, dtype="f32", zipf_s=0.5, seed=23)


def _check(y, ref, dtype, what):
    err, tol = max_err(y, ref), tolerance(ref, dtype)
    say(f"  {what}: max|d|={err:.3e} tol={tol:.3e} ratio={err / tol if tol else 0:.3f}")
    assert err <= tol, f"{what}: max|d|={err} > tol={tol}"


def _run(wl, idx=None, weights="wl", expert_begin=0, idx_dtype=torch.int64, flags=0,
         y_alias=False):
    idx = wl.idx if idx is None else idx
    d = upload(wl)
    d_idx = torch.from_numpy(np.ascontiguousarray(idx)).to(idx_dtype).cuda()
    w = d["w"] if isinstance(weights, str) else (None if weights is None else dev(weights))
    p = tr.plan(d_idx, E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl), expert_begin=expert_begin,
                flags=flags)
    y = tr.forward(p, d["x"], w, d["w1"], d["w2"], y=d["x"] if y_alias else None)
    torch.cuda.synchronize()
    return host(y)


def _oracle(wl, idx=None, weights="wl", expert_begin=0, tokens=None):
    idx = wl.idx if idx is None else idx
    w = wl.weights if isinstance(weights, str) else weights
    return oracle.forward(wl.x, idx, w, wl.w1, wl.w2, wl.E, expert_begin=expert_begin,
                          tokens=tokens)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("name", ["edge_mid", "edge_split", "edge_f32"])
def test_nan_in_non_local_weights(name):
    """Weights of slots that are not local are never read: NaN there gives the
    same bits as the finite run, and the oracle's values."""
    say(f"NaN non-local weights {name}")
    wl = gen.make_workload(name, with_weights=True)
    idx = wl.idx.copy()
    if not (idx < 0).any():
        # every slot local (G == E): hand a tenth of them to other ranks
        idx[np.random.default_rng(27).random(idx.shape) < 0.1] = -1
    wn = wl.weights.copy()
    wn[idx < 0] = np.nan
    assert np.isnan(wn).any()
    y_fin = _run(wl, idx=idx)
    y_nan = _run(wl, idx=idx, weights=wn)
    assert np.array_equal(_bits(y_nan), _bits(y_fin))
    route = oracle.route(idx, wl.E)
    toks = None if wl.T <= 1024 else sample_tokens(wl, route, 512)
    ref = _oracle(wl, idx=idx, weights=wn, tokens=toks)
    got = y_nan if toks is None else y_nan[toks]
    _check(as_f64(got), ref, wl.dtype, f"{name} y with NaN non-local weights")
    assert not np.isnan(as_f64(y_nan)).any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_rows(dtype):
    """T = 0: plan, forward and the stage entry points return TR_OK and the
    plan's statistics are zero (every expert empty)."""
    say(f"T=0 {dtype}")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H, I, E, K = 512, 256, 4, 2
    idx = torch.empty((0, K), dtype=torch.int64, device="cuda")
    p = tr.plan(idx, E=E, H=H, I=I, dtype=tdt)
    x = torch.empty((0, H), dtype=tdt, device="cuda")
    w = torch.empty((0, K), dtype=torch.float32, device="cuda")
    w1 = torch.zeros((E, 2 * I, H), dtype=tdt, device="cuda")
    w2 = torch.zeros((E, H, I), dtype=tdt, device="cuda")
    y = tr.forward(p, x, w, w1, w2)
    assert y.shape == (0, H)
    assert list(tr.plan_stats(p)) == [0, 0, 0, E]
    tr.combine_reduce(p, w)
    tr.grouped_gemm_up_x(p, x, w1)
    torch.cuda.synchronize()


def test_top1_all_rows_through_gemm2_epilogue():
    """K = 1 at a size whose GEMMs run as three launches: every routed row has
    one local slot, so GEMM2 writes every output row to y (no O, no reduce of
    routed rows). Every row compared with the oracle; NULL weights too."""
    say("top-1, three-launch GEMMs, every row")
    wl = gen.make_workload("edge_k1_split", with_weights=True)
    route = oracle.route(wl.idx, wl.E)
    assert route["R"] == wl.T
    y = _run(wl)
    _check(as_f64(y), _oracle(wl), wl.dtype, "top-1 y")
    y1 = _run(wl, weights=None)
    toks = sample_tokens(wl, route, 512)
    _check(as_f64(y1[toks]), _oracle(wl, weights=None, tokens=toks), wl.dtype, "top-1 y, w=1")


def test_duplicate_expert_in_one_row():
    """A row naming the same local expert in several slots gets one expanded
    row per slot and each contributes (weighted) to y."""
    say("duplicate ids")
    wl = gen.make_workload("edge_mid", with_weights=True)
    idx = wl.idx.copy()
    rng = np.random.default_rng(24)
    rows = rng.choice(wl.T, 300, replace=False)
    for t in rows[:200]:            # slot 1 repeats slot 0's expert
        e = int(rng.integers(0, wl.E))
        idx[t, 0] = idx[t, 1] = e
    for t in rows[200:]:            # every slot names one expert
        idx[t, :] = int(rng.integers(0, wl.E))
    route = oracle.route(idx, wl.E)
    assert route["R"] == int((idx >= 0).sum())
    y = _run(wl, idx=idx)
    _check(as_f64(y), _oracle(wl, idx=idx), wl.dtype, "duplicate ids y")
    # the rows whose slots all name one expert (K expanded rows of one
    # segment, summed in slot order) once more on their own bar
    t_all = np.sort(rows[200:])
    _check(as_f64(y[t_all]), _oracle(wl, idx=idx, tokens=t_all), wl.dtype,
           "rows with one expert in every slot")


@pytest.mark.parametrize("idx_dtype", [torch.int32, torch.int64])
@pytest.mark.parametrize("name", ["edge_mid", "edge_split"])
def test_global_ids_expert_begin(name, idx_dtype):
    """Global ids with expert_begin = 3E: this rank owns [3E, 4E); other
    ranks' ids on both sides of that range (and -1) are ignored. Same bits as
    the local-id run, and the oracle's values with the same global ids."""
    say(f"global ids {name} {idx_dtype}")
    wl = gen.make_workload(name, with_weights=True)
    eb = 3 * wl.E
    rng = np.random.default_rng(25)
    foreign = rng.integers(0, 8 * wl.E, size=wl.idx.shape)
    foreign = np.where((foreign >= eb) & (foreign < eb + wl.E), foreign + wl.E, foreign)
    foreign = np.where(rng.random(wl.idx.shape) < 0.2, -1, foreign)
    gidx = np.where(wl.idx >= 0, wl.idx + eb, foreign).astype(np.int64)
    assert ((gidx >= eb) & (gidx < eb + wl.E)).sum() == (wl.idx >= 0).sum()
    y_g = _run(wl, idx=gidx, expert_begin=eb, idx_dtype=idx_dtype)
    y_l = _run(wl)
    assert np.array_equal(_bits(y_g), _bits(y_l))
    route = oracle.route(gidx, wl.E, expert_begin=eb)
    toks = None if wl.T <= 1024 else sample_tokens(wl, route, 512)
    ref = _oracle(wl, idx=gidx, expert_begin=eb, tokens=toks)
    _check(as_f64(y_g if toks is None else y_g[toks]), ref, wl.dtype, f"{name} global ids y")


def test_one_expert_holds_every_route():
    """All local routes go to one expert (the others are empty): 8448 rows,
    33 m-tiles of that expert, 528 GEMM1 tiles, i.e. more than two rounds of
    the persistent grid on one expert's weights. Slot 1 is another rank's
    route. Every row compared with the oracle."""
    say("one expert, several rounds")
    gen.custom_spec("edge_one_expert", T=8448, K=2, E=8, G=8, H=256, I=2048,
                    routing="uniform", seed=26)
    wl = gen.make_workload("edge_one_expert", with_weights=True)
    idx = np.full_like(wl.idx, -1)
    idx[:, 0] = 5
    route = oracle.route(idx, wl.E)
    assert route["counts"][5] == wl.T and route["R"] == wl.T
    y = _run(wl, idx=idx)
    _check(as_f64(y), _oracle(wl, idx=idx), wl.dtype, "one expert y")
    y_t = _run(wl, idx=idx, flags=tr.FLAG_GEMM_FORCE_TILED)
    assert np.array_equal(_bits(y_t), _bits(y))


@pytest.mark.parametrize("name", ["edge_split", "edge_k1_split", "c5"])
def test_y_aliases_x_three_launch(name):
    """y may alias x on every path. On these workloads the forward's GEMMs
    run as three launches: early GEMM2 tiles write y while GEMM1's last round
    still gathers x. A row written there has its only local slot in an
    m-tile GEMM1 has finished, so no later GEMM1 tile reads it (except as a
    filler row past a segment, whose outputs are dropped). Same bits as the
    unaliased forward."""
    say(f"y aliases x {name}")
    wl = gen.make_workload(name, with_weights=True)
    y_sep = _run(wl)
    y_al = _run(wl, y_alias=True)
    assert np.array_equal(_bits(y_sep), _bits(y_al))


def test_split_against_oracle_sampled():
    """The three-launch workload against the oracle on 512 sampled rows
    (segment edges, first and last rows, random rows)."""
    say("split vs oracle, 512 rows")
    wl = gen.make_workload("edge_split", with_weights=True)
    route = oracle.route(wl.idx, wl.E)
    toks = sample_tokens(wl, route, 512)
    assert len(toks) >= 512
    y = _run(wl)
    _check(as_f64(y[toks]), _oracle(wl, tokens=toks), wl.dtype, "split y[512 rows]")
