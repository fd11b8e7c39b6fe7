"""Pins for the CPU oracle against facts that do not come from the oracle:
brute force by another formulation, closed forms, exact invariants and the
worked examples of the pages (tests/golden). Each test says which plausible
mistake it would catch."""

import itertools

import numpy as np
import pytest
from scipy.special import expit

import gen
from tests._util import load_golden

rng_seed = 20260


# --------------------------------------------------------------------------
# route scan
# --------------------------------------------------------------------------

def _route_by_sort(idx, E, eb):
    """Second formulation: sort the local (expert, token, slot) triples; the
    rank in that order is the expanded row."""
    T, K = idx.shape
    triples = sorted((int(idx[t, k]) - eb, t, k) for t in range(T) for k in range(K)
                     if 0 <= int(idx[t, k]) - eb < E)
    row_map = -np.ones((T, K), np.int64)
    for r, (e, t, k) in enumerate(triples):
        row_map[t, k] = r
    counts = np.array([sum(1 for tr in triples if tr[0] == e) for e in range(E)])
    return row_map, counts, [t for _, t, _ in triples], [k for _, _, k in triples]


@pytest.mark.parametrize("case", range(40))
def test_route_brute_force(oracle_mod, case):
    # catches: wrong stable order, off-by-one offsets, t/k index swaps
    rng = np.random.default_rng(rng_seed + case)
    T = int(rng.integers(0, 9))
    K = int(rng.integers(1, 5))
    E = int(rng.integers(1, 6))
    eb = int(rng.integers(-2, 3))
    idx = rng.integers(-3, E + eb + 3, size=(T, K))
    r = oracle_mod.route(idx, E, eb)
    row_map, counts, src, ks = _route_by_sort(idx, E, eb)
    assert np.array_equal(r["row_map"], row_map)
    assert np.array_equal(r["counts"], counts)
    assert r["offsets"][0] == 0 and np.array_equal(np.diff(r["offsets"]), counts)
    assert r["R"] == len(src)
    assert r["row_src"].tolist() == src and r["row_k"].tolist() == ks


def test_route_invariants_c2(oracle_mod):
    # catches: segments that do not match routing counts; non-bijective maps
    wl = gen.make_workload("c2", T=1024)
    r = oracle_mod.route(wl.idx, wl.E)
    local = wl.idx >= 0
    assert r["R"] == local.sum()                      # valid_recv_routes (issue #760)
    T_loc = int(local.any(1).sum())                   # valid_recv_rows (issue #760)
    assert T_loc == wl.T
    for e in range(wl.E):
        assert r["counts"][e] == (wl.idx == e).sum()
    rm = r["row_map"]
    assert np.array_equal(np.sort(rm[local]), np.arange(r["R"]))
    assert (rm[~local] == -1).all()
    t, k = np.nonzero(local)
    assert np.array_equal(r["row_src"][rm[t, k]], t) and np.array_equal(r["row_k"][rm[t, k]], k)
    # stable: inside each segment rows follow received order
    for e in range(wl.E):
        seg = r["row_src"][r["offsets"][e]:r["offsets"][e + 1]]
        assert (np.diff(seg) > 0).all()


def test_route_nonlocal_ids_ignored(oracle_mod):
    # catches: treating ids >= E (another rank's experts) as local
    wl = gen.make_workload("c2", T=256)
    a = oracle_mod.route(wl.idx, wl.E)
    b = oracle_mod.route(wl.global_idx, wl.E)
    for f in ("counts", "offsets", "row_map", "row_src", "row_k"):
        assert np.array_equal(a[f], b[f])
    # the same routing seen by rank 3 of 16 (ids shifted by 3 * 16)
    g = np.where(wl.global_idx >= 0, (wl.global_idx + 48) % 256, -1)
    c = oracle_mod.route(g, wl.E, expert_begin=48)
    assert np.array_equal(c["row_map"], a["row_map"])


def test_route_empty_and_all_pad(oracle_mod):
    r = oracle_mod.route(np.zeros((0, 4), np.int64), 5)
    assert r["R"] == 0 and (r["offsets"] == 0).all()
    r = oracle_mod.route(-np.ones((7, 3), np.int64), 5)
    assert r["R"] == 0 and (r["row_map"] == -1).all()


# --------------------------------------------------------------------------
# silu and the expert MLP
# --------------------------------------------------------------------------

def test_silu_values(oracle_mod):
    # textbook logistic values; catches z*sigmoid(-z) or a missing factor z
    assert oracle_mod.silu(1.0) == pytest.approx(0.7310585786300049, rel=1e-15)
    assert oracle_mod.silu(-1.0) == pytest.approx(-0.2689414213699951, rel=1e-15)
    assert oracle_mod.silu(2.0) == pytest.approx(1.7615941559557646, rel=1e-15)
    assert oracle_mod.silu(0.0) == 0.0
    for z in (0.3, 1.7, 5.0, 13.0):       # silu(z) - silu(-z) = z
        assert oracle_mod.silu(z) - oracle_mod.silu(-z) == pytest.approx(z, rel=1e-14)
    assert oracle_mod.silu(-800.0) == 0.0 and oracle_mod.silu(800.0) == 800.0


def _f32(a):
    return np.ascontiguousarray(a, np.float32)


def test_mlp_closed_form_orientation(oracle_mod):
    # W1 gate = a * P, W1 up = b * Q (P, Q selections of input coordinates),
    # W2 = S (a selection from I into H). With H != I a transposed operand,
    # swapped gate/up or a wrong W2 orientation changes the result.
    H, I = 6, 4
    rng = np.random.default_rng(7)
    x = _f32(rng.standard_normal(H))
    p = [4, 0, 5, 2]           # gate row i reads x[p[i]]
    q = [1, 3, 0, 4]           # up row i reads x[q[i]]
    s = [2, 0, 3, 1, 2, 0]     # output j reads h[s[j]]
    a, b = 1.5, -0.75
    w1 = np.zeros((2 * I, H), np.float32)
    for i in range(I):
        w1[i, p[i]] = a
        w1[I + i, q[i]] = b
    w2 = np.zeros((H, I), np.float32)
    for j in range(H):
        w2[j, s[j]] = 1.0
    out = oracle_mod.expert_mlp(w1, w2, x)
    xd = x.astype(np.float64)
    hv = [(a * xd[p[i]]) * expit(a * xd[p[i]]) * (b * xd[q[i]]) for i in range(I)]
    want = np.array([hv[s[j]] for j in range(H)])
    assert np.allclose(out, want, rtol=1e-12, atol=0)


def test_mlp_gate_zero_or_up_zero(oracle_mod):
    # catches: gate and up halves swapped (silu(0)=0 kills only the gate path)
    H, I = 8, 4
    rng = np.random.default_rng(8)
    x = _f32(rng.standard_normal(H))
    w2 = _f32(rng.standard_normal((H, I)))
    up = _f32(rng.standard_normal((I, H)))
    w1 = np.concatenate([np.zeros((I, H), np.float32), up])
    assert np.all(oracle_mod.expert_mlp(w1, w2, x) == 0.0)
    w1 = np.concatenate([up, np.zeros((I, H), np.float32)])
    assert np.all(oracle_mod.expert_mlp(w1, w2, x) == 0.0)


def _dense_gating_forward(x, idx, w, w1, w2, E, eb):
    """Second formulation of the layer: the classic dense-gating MoE
    y = sum_e G[:, e] * MLP_e(X) with G[t, e] the sum of the weights of the
    slots of t that point at local expert e; every expert runs on every token
    as matrix products (no scan, no expand, no per-route loop)."""
    T, K = idx.shape
    X = x.astype(np.float64)
    G = np.zeros((T, E))
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k]) - eb
            if 0 <= e < E:
                G[t, e] += 1.0 if w is None else float(w[t, k])
    I = w1.shape[1] // 2
    y = np.zeros((T, x.shape[1]))
    for e in range(E):
        W1 = w1[e].astype(np.float64)
        g = X @ W1[:I].T
        u = X @ W1[I:].T
        h = g * expit(g) * u
        y += G[:, e:e + 1] * (h @ w2[e].astype(np.float64).T)
    return y


@pytest.mark.parametrize("case", range(12))
def test_forward_vs_dense_gating(oracle_mod, case):
    # catches: wrong weight index (t*K+k), dropped or double-counted routes,
    # wrong expert offsets, a missing term of the MLP
    rng = np.random.default_rng(100 + case)
    T = int(rng.integers(1, 7))
    K = int(rng.integers(1, 4))
    E = int(rng.integers(1, 5))
    H = int(rng.choice([4, 6, 8]))
    I = int(rng.choice([2, 3, 4]))
    eb = int(rng.integers(0, 3))
    idx = rng.integers(-1, E + eb + 2, size=(T, K))
    w = _f32(rng.random((T, K)))
    x = _f32(rng.standard_normal((T, H)))
    w1 = _f32(rng.standard_normal((E, 2 * I, H)))
    w2 = _f32(rng.standard_normal((E, H, I)))
    if case % 3 == 0:
        w = None
    y = oracle_mod.forward(x, idx, w, w1, w2, E, expert_begin=eb)
    ref = _dense_gating_forward(x, idx, w, w1, w2, E, eb)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_forward_bf16_inputs_widened_exactly(oracle_mod):
    # bf16 bit patterns must be read as the float32 with those top 16 bits
    rng = np.random.default_rng(9)
    T, K, E, H, I = 3, 2, 2, 8, 4
    idx = np.array([[0, 1], [1, -1], [-1, 0]])
    w = _f32(rng.random((T, K)))
    xb = gen.f32_to_bf16_bits(rng.standard_normal((T, H)))
    w1b = gen.f32_to_bf16_bits(rng.standard_normal((E, 2 * I, H)))
    w2b = gen.f32_to_bf16_bits(rng.standard_normal((E, H, I)))
    y = oracle_mod.forward(xb, idx, w, w1b, w2b, E)
    yf = oracle_mod.forward(gen.bf16_bits_to_f32(xb), idx, w, gen.bf16_bits_to_f32(w1b),
                            gen.bf16_bits_to_f32(w2b), E)
    assert np.array_equal(y, yf)


def test_top1_unit_weight_is_single_expert_mlp(oracle_mod):
    # top-1 routing with weight 1 reproduces a dense SwiGLU MLP per token
    wl = gen.make_workload("c1", with_weights=True)
    idx = wl.idx[:, :1].copy()
    w = np.ones((wl.T, 1), np.float32)
    y = oracle_mod.forward(wl.x, idx, w, wl.w1, wl.w2, wl.E)
    for t in range(0, wl.T, 9):
        e = int(idx[t, 0])
        X = wl.x[t].astype(np.float64)
        W1 = wl.w1[e].astype(np.float64)
        g, u = W1[:wl.I] @ X, W1[wl.I:] @ X
        ref = wl.w2[e].astype(np.float64) @ (g * expit(g) * u)
        assert np.allclose(y[t], ref, rtol=1e-12, atol=1e-13)


def test_scaling_w2_doubles_exactly(oracle_mod):
    wl = gen.make_workload("c1", with_weights=True)
    y = oracle_mod.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E)
    y2 = oracle_mod.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2 * np.float32(2), wl.E)
    assert np.array_equal(y2, 2 * y)


def test_expert_relabel_invariance(oracle_mod):
    wl = gen.make_workload("c1", with_weights=True)
    perm = np.random.default_rng(3).permutation(wl.E)       # new label of expert e
    inv = np.argsort(perm)
    idx2 = np.where(wl.idx >= 0, perm[np.maximum(wl.idx, 0)], -1)
    y = oracle_mod.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E)
    y2 = oracle_mod.forward(wl.x, idx2, wl.weights, wl.w1[inv], wl.w2[inv], wl.E)
    assert np.array_equal(y, y2)


def test_nonlocal_weights_never_read(oracle_mod):
    wl = gen.make_workload("c1", with_weights=True)
    idx = wl.idx.copy()
    idx[::3, 1] = -1
    w = wl.weights.copy()
    w[idx < 0] = np.nan
    y = oracle_mod.forward(wl.x, idx, w, wl.w1, wl.w2, wl.E)
    assert np.isfinite(y).all()
    w0 = wl.weights.copy()
    w0[idx < 0] = 123.0
    assert np.array_equal(y, oracle_mod.forward(wl.x, idx, w0, wl.w1, wl.w2, wl.E))


def test_all_minus_one_gives_positive_zero(oracle_mod):
    wl = gen.make_workload("c1", with_weights=True)
    idx = -np.ones_like(wl.idx)
    y = oracle_mod.forward(wl.x, idx, wl.weights, wl.w1, wl.w2, wl.E)
    assert np.all(y == 0) and not np.signbit(y).any()


def test_expert_rows_match_forward(oracle_mod):
    wl = gen.make_workload("c1", with_weights=True)
    r = oracle_mod.route(wl.idx, wl.E)
    e_of_row = np.repeat(np.arange(wl.E), r["counts"])
    O = oracle_mod.expert_rows(e_of_row, r["row_src"], wl.x, wl.w1, wl.w2)
    for row in range(0, r["R"], 17):
        ref = oracle_mod.expert_mlp(wl.w1[e_of_row[row]], wl.w2[e_of_row[row]], wl.x[r["row_src"][row]])
        assert np.array_equal(O[row], ref)


# --------------------------------------------------------------------------
# expand and reduce
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_expand_is_row_gather(oracle_mod, dtype):
    wl = gen.make_workload("c2" if dtype == "bf16" else "c1", T=64)
    r = oracle_mod.route(wl.idx, wl.E)
    Xe = oracle_mod.expand(wl.x, r["row_src"])
    for row in range(r["R"]):
        assert np.array_equal(Xe[row].view(np.uint8), wl.x[r["row_src"][row]].view(np.uint8))


def test_combine_constant_expert(oracle_mod):
    # fake expert output 1 on every row (issue #760): y[t] = local weight sum
    wl = gen.make_workload("c4")
    r = oracle_mod.route(wl.idx, wl.E)
    O = np.ones((max(r["R"], 1), 5), np.float32)
    y = oracle_mod.combine(r["row_map"], wl.weights, O)
    for t in range(wl.T):
        s = sum(float(wl.weights[t, k]) for k in range(wl.K) if wl.idx[t, k] >= 0)
        assert np.all(y[t] == s)


def test_expand_reduce_round_trip(oracle_mod):
    # identity expert (O = Xe) and unit weights: y = (#local routes) * x;
    # with top-1 routing it is x itself, bit for bit
    wl = gen.make_workload("c2", T=128)
    r = oracle_mod.route(wl.idx, wl.E)
    Xe = oracle_mod.expand(wl.x, r["row_src"])
    y = oracle_mod.combine(r["row_map"], None, Xe)
    n_loc = (wl.idx >= 0).sum(1)
    assert np.array_equal(y, n_loc[:, None] * gen.bf16_bits_to_f32(wl.x).astype(np.float64))
    idx1 = wl.idx.copy()
    first = np.argmax(idx1 >= 0, axis=1)
    keep = np.zeros_like(idx1, dtype=bool)
    keep[np.arange(wl.T), first] = True
    idx1[~keep] = -1
    r1 = oracle_mod.route(idx1, wl.E)
    y1 = oracle_mod.combine(r1["row_map"], None, oracle_mod.expand(wl.x, r1["row_src"]))
    assert np.array_equal(gen.f32_to_bf16_bits(y1.astype(np.float32)), wl.x)


# --------------------------------------------------------------------------
# worked examples of the pages
# --------------------------------------------------------------------------

def test_deepep760_combine_only_emulated(oracle_mod):
    """Emulate the 32-rank combine-only repro on the CPU: every destination
    rank runs route + weighted reduce over its own expert range with a constant
    expert output; the cross-rank sum must give the repro's expected values."""
    g = load_golden("deepep760_combine_only.txt")
    W, tp, topk, E = g["world_size"], g["tp_size"], g["topk"], g["local_experts"]
    assert g["num_experts"] == W * E
    # one token per source rank; real only on TP rank 0 of each DP group
    idx = -np.ones((W, topk), np.int64)
    w = np.zeros((W, topk), np.float32)
    real = np.array([r % tp == 0 for r in range(W)])
    idx[real] = np.arange(topk) * E
    w[real] = g["topk_weight"]
    H = 16
    combined = np.zeros((W, H))
    for rank in range(W):
        r = oracle_mod.route(idx, E, expert_begin=rank * E)
        # valid_recv_routes / valid_recv_rows of the repro for this rank
        loc = (idx >= rank * E) & (idx < (rank + 1) * E)
        assert r["R"] == loc.sum()
        if r["R"] == 0:
            continue
        O = np.ones((r["R"], H), np.float32)
        combined += oracle_mod.combine(r["row_map"], w, O)
    assert np.all(combined[real] == g["expected_real"])
    assert np.all(combined[~real] == g["expected_pad"])


def test_deepep760_cross_rank_epilogue(oracle_mod):
    """The same repro with the cross-rank sum done by the epilogue oracle:
    the 32 rank partials are stacked into one receive buffer and every output
    token lists the rows of all ranks; the result must be the repro's
    expected 1 on real rows and 0 on padding rows, and must equal the plain
    sum of the partials."""
    g = load_golden("deepep760_combine_only.txt")
    W, tp, topk, E = g["world_size"], g["tp_size"], g["topk"], g["local_experts"]
    idx = -np.ones((W, topk), np.int64)
    w = np.zeros((W, topk), np.float32)
    real = np.array([r % tp == 0 for r in range(W)])
    idx[real] = np.arange(topk) * E
    w[real] = g["topk_weight"]
    H = 8
    partials = np.zeros((W, W, H), np.float32)       # [source rank, token, H]
    for rank in range(W):
        r = oracle_mod.route(idx, E, expert_begin=rank * E)
        if r["R"]:
            partials[rank] = oracle_mod.combine(r["row_map"], w, np.ones((r["R"], H), np.float32))
    recv = partials.reshape(W * W, H)
    src = (np.arange(W)[None, :] * W + np.arange(W)[:, None]).astype(np.int32)   # [token, rank]
    y = oracle_mod.combine_epilogue(src, recv)
    assert np.all(y[real] == g["expected_real"])
    assert np.all(y[~real] == g["expected_pad"])
    assert np.array_equal(y, partials.astype(np.float64).sum(axis=0))


def test_epilogue_one_hot_is_a_copy(oracle_mod):
    """One contribution per token (the rest -1): the output is that received
    row, exactly, for bf16 and fp32 rows."""
    rng = np.random.default_rng(7)
    for dt in ("bf16", "f32"):
        f = rng.standard_normal((20, 24)).astype(np.float32)
        recv = gen.f32_to_bf16_bits(f) if dt == "bf16" else f
        want = gen.bf16_bits_to_f32(recv) if dt == "bf16" else f
        src = -np.ones((9, 5), np.int32)
        rows = rng.integers(0, 20, 9)
        src[np.arange(9), rng.integers(0, 5, 9)] = rows
        y = oracle_mod.combine_epilogue(src, recv)
        assert np.array_equal(y, want[rows].astype(np.float64))
        assert np.all(oracle_mod.combine_epilogue(-np.ones((3, 4), np.int32), recv) == 0.0)


def test_epilogue_equals_count_matrix_product(oracle_mod):
    """Second formulation: y = S @ recv with S[t, r] the number of times row r
    is listed for token t (duplicates count twice, -1 never)."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        N, T, J, H = rng.integers(1, 30), rng.integers(1, 12), rng.integers(1, 9), rng.integers(1, 16)
        recv = rng.standard_normal((N, H)).astype(np.float32)
        src = rng.integers(-1, N, (T, J)).astype(np.int32)
        S = np.zeros((T, N))
        for t in range(T):
            for j in range(J):
                if src[t, j] >= 0:
                    S[t, src[t, j]] += 1
        y = oracle_mod.combine_epilogue(src, recv)
        np.testing.assert_allclose(y, S @ recv.astype(np.float64), rtol=1e-12, atol=1e-12)


def test_sglang6092_real_rows_in_padded_buffer():
    g = load_golden("sglang6092_dp_batch.txt")
    wl = gen.make_workload("c4")
    assert wl.T == g["padded_rows"] == 120 * g["workers"]
    assert int(wl.real.sum()) == g["real_rows"] == sum(g["worker_batch"])


# --------------------------------------------------------------------------
# DP-padded buffers (SGLang PR #6092 review thread)
# --------------------------------------------------------------------------

def _carrying(T, B, counts):
    """Rows that hold a query, listed block by block: the first counts[j]
    rows of block j (a count past the block's end means all of it)."""
    rows = []
    for j in range(-(-T // B)):
        for t in range(j * B, min(j * B + B, T)):
            if t - j * B < counts[j]:
                rows.append(t)
    return rows


@pytest.mark.parametrize("case", range(40))
def test_route_padded_brute_force(oracle_mod, case):
    # catches: block index and in-block offset swapped, <= for <, pad slots
    # counted, a count past the block's end spilling into the next block
    rng = np.random.default_rng(rng_seed + 500 + case)
    T = int(rng.integers(0, 13))
    K = int(rng.integers(1, 4))
    E = int(rng.integers(1, 5))
    B = int(rng.integers(1, 5))
    nb = -(-T // B)
    counts = rng.integers(-1, B + 2, size=nb).astype(np.int32)
    idx = rng.integers(-2, E + 2, size=(T, K))
    r = oracle_mod.route(idx, E, 0, block_rows=B, block_counts=counts)
    keep = _carrying(T, B, counts)
    masked = -np.ones_like(idx)
    masked[keep] = idx[keep]
    row_map, cnt, src, ks = _route_by_sort(masked, E, 0)
    assert np.array_equal(r["row_map"], row_map)
    assert np.array_equal(r["counts"], cnt)
    assert r["row_src"].tolist() == src and r["row_k"].tolist() == ks


def test_route_padded_full_blocks_is_plain_route(oracle_mod):
    # every row carries: identical to the plain route table
    rng = np.random.default_rng(rng_seed + 600)
    idx = rng.integers(-1, 6, size=(37, 3))
    a = oracle_mod.route(idx, 6)
    b = oracle_mod.route(idx, 6, block_rows=8, block_counts=np.full(5, 8, np.int32))
    c = oracle_mod.route(idx, 6, block_rows=8, block_counts=np.full(5, 1000, np.int32))
    for r in (b, c):
        assert r["R"] == a["R"] and np.array_equal(r["row_map"], a["row_map"])
        assert np.array_equal(r["row_src"], a["row_src"])
    z = oracle_mod.route(idx, 6, block_rows=8, block_counts=np.zeros(5, np.int32))
    assert z["R"] == 0 and (z["row_map"] == -1).all()


def test_sglang6092_compaction(oracle_mod):
    # the review thread's batch mix [120, 1, ..., 1] in a 960-row buffer: the
    # communication buffer holds 127 rows, the real rows of the c4 workload
    g = load_golden("sglang6092_dp_batch.txt")
    wl = gen.make_workload("c4")
    counts = np.array(g["worker_batch"], np.int32)
    B = g["padded_rows"] // g["workers"]
    x = wl.x
    comp, n = oracle_mod.compact_rows(x, B, counts)
    assert n == g["real_rows"] == comp.shape[0]
    assert np.array_equal(comp, x[np.nonzero(wl.real)[0]])
    assert np.array_equal(comp[120], x[120]) and np.array_equal(comp[126], x[840])
    back, n2 = oracle_mod.compact_rows(comp, B, counts, to_padded=True,
                                       dst=np.full_like(x, 7))
    assert n2 == n
    assert np.array_equal(back[wl.real], x[wl.real]) and (back[~wl.real] == 7).all()


def test_compaction_clamps_counts(oracle_mod):
    # negative counts carry nothing; counts past a block (or the buffer's
    # end) carry the whole block and nothing more
    src = np.arange(10 * 2, dtype=np.int32).reshape(10, 2)
    comp, n = oracle_mod.compact_rows(src, 4, np.array([-3, 9, 5], np.int32))
    assert n == 6 and comp[:, 0].tolist() == [8, 10, 12, 14, 16, 18]
    comp, n = oracle_mod.compact_rows(src, 4, np.array([2, 0, 1], np.int32))
    assert n == 3 and comp[:, 0].tolist() == [0, 2, 16]
