"""The HIP path through the C ABI vs the oracle.

Element-by-element at sizes the oracle finishes in seconds (several tiles and
ragged tails), and on sampled rows at the full workload sizes. Bars: expand is
a bit copy (bit-exact); outputs within max|d| <= 1e-2 max|ref| + 1e-3 for
bf16 and 1e-5 max|ref| for fp32."""

import numpy as np
import pytest
import torch

import gen
import oracle
import top_reduce_amd as tr
from tests._gpu import as_f64, dev, host, sample_tokens, say, torch_dtype, upload
from tests._util import max_err, tolerance

pytestmark = pytest.mark.gpu

# reduced shapes: several M tiles with ragged tails, several N tiles
gen.custom_spec("mid", T=1024, K=8, E=8, G=64, H=1024, I=512, zipf_s=1.0, seed=7)
gen.custom_spec("mid_small_experts", T=512, K=4, E=32, G=128, H=512, I=256, zipf_s=0.6, seed=8)
gen.custom_spec("mid_f32", T=300, K=4, E=6, G=12, H=264, I=72, dtype="f32", zipf_s=0.5, seed=9)
# fp32 with I not a multiple of 4 (ragged k tail of GEMM2, ragged output
# columns of GEMM1) and H not a multiple of 16
gen.custom_spec("odd_f32", T=200, K=3, E=5, G=9, H=136, I=70, dtype="f32", zipf_s=0.5, seed=12)
# bf16 shapes off the tiled kernel's 256 / 128 column grid (the any-shape
# kernel): H % 256 != 0 with I a multiple of 8; I not a multiple of 8 (GEMM2's
# k tail loaded element-wise, GEMM1's last output columns stored one by one);
# an H and I of a published expert shape's size class (2880 / 1440)
gen.custom_spec("odd_bf16", T=300, K=4, E=6, G=12, H=264, I=72, zipf_s=0.5, seed=13)
gen.custom_spec("odd_i_bf16", T=200, K=3, E=5, G=9, H=136, I=70, zipf_s=0.5, seed=14)
gen.custom_spec("wide_bf16", T=128, K=4, E=8, G=16, H=2880, I=1440, zipf_s=1.0, seed=15)
# every row routes to all 8 experts: 8 segments of 2080 rows, 9 m-tiles each
# (the last one 32 rows deep); 288 tiles per GEMM, more than one round of the
# persistent grid on 256 compute units.
gen.custom_spec("rounds", T=2080, K=8, E=8, G=8, H=1024, I=512, routing="uniform", seed=10)
# every row routed to all 8 experts: 17 m-tiles each, GEMM1 544 tiles (two
# rounds of 256 blocks plus 32), so the forward's hybrid launch runs GEMM1's
# last round beside early GEMM2 tiles
gen.custom_spec("split", T=4200, K=8, E=8, G=8, H=2048, I=512, routing="uniform", seed=11)


def _assert_close(got, ref, dtype, what):
    err, tol = max_err(got, ref), tolerance(ref, dtype)
    say(f"  {what}: max|d|={err:.3e} tol={tol:.3e} ratio={err / tol if tol else 0:.3f}")
    assert err <= tol, f"{what}: max|d|={err} > tol={tol}"


def _forward(wl, flags=0, y_alias=False, weights=True):
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl), flags=flags)
    y = d["x"] if y_alias else None
    y = tr.forward(p, d["x"], d["w"] if weights else None, d["w1"], d["w2"], y=y)
    torch.cuda.synchronize()
    return p, host(y)


@pytest.mark.parametrize("name,flags", [("c1", 0), ("mid_f32", 0), ("odd_f32", 0), ("mid", 0),
                                        ("rounds", 0),
                                        ("mid", tr.FLAG_GEMM_FORCE_TILED),
                                        ("mid", tr.FLAG_GEMM_FORCE_STREAM),
                                        ("mid_small_experts", 0),
                                        ("odd_bf16", 0), ("odd_i_bf16", 0), ("wide_bf16", 0),
                                        ("odd_bf16", tr.FLAG_GEMM_FORCE_TILED),
                                        ("odd_bf16", tr.FLAG_GEMM_FORCE_STREAM)])
def test_forward_full_compare(name, flags):
    say(f"forward {name} flags={flags}")
    wl = gen.make_workload(name, with_weights=True)
    _, y = _forward(wl, flags)
    ref = oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E)
    _assert_close(as_f64(y), ref, wl.dtype, f"{name} y")
    pad = ~(wl.idx >= 0).any(1)
    assert (y[pad] == 0).all()


@pytest.mark.parametrize("T", [1, 2, 4, 8, 64])
@pytest.mark.parametrize("variant", ["", "random", "dense"])
def test_forward_c3_decode(T, variant):
    say(f"forward c3 T={T} {variant}")
    wl = gen.make_workload("c3", T=T, variant=variant, with_weights=True)
    _, y = _forward(wl)
    ref = oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E)
    _assert_close(as_f64(y), ref, wl.dtype, f"c3 T={T} y")
    assert (y[~wl.real] == 0).all()


def test_forward_c4_all_rows():
    say("forward c4")
    wl = gen.make_workload("c4", with_weights=True)
    _, y = _forward(wl)
    rows = np.nonzero((wl.idx >= 0).any(1))[0]
    ref = oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E, tokens=rows)
    _assert_close(as_f64(y[rows]), ref, wl.dtype, "c4 y (rows with a local route)")
    others = np.setdiff1d(np.arange(wl.T), rows)
    assert (y[others] == 0).all()                       # exact +0 bits


@pytest.mark.parametrize("name", ["c2", "c5"])
def test_forward_full_size_sampled(name):
    say(f"forward {name} full size (sampled rows)")
    wl = gen.make_workload(name, with_weights=True)
    p, y = _forward(wl)
    route = oracle.route(wl.idx, wl.E)
    toks = sample_tokens(wl, route, 40)
    ref = oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E, tokens=toks)
    _assert_close(as_f64(y[toks]), ref, wl.dtype, f"{name} y[{len(toks)} rows]")


@pytest.mark.parametrize("name", ["mid", "c1", "rounds", "odd_i_bf16"])
def test_stages(name):
    """expand bit-exact; O rows vs the oracle's per-route MLP; reduce."""
    say(f"stages {name}")
    wl = gen.make_workload(name, with_weights=True)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl))
    route = oracle.route(wl.idx, wl.E)
    R = route["R"]
    tr.expand(p, d["x"])
    v = p.views()
    Xe = host(v["Xe"][:R])
    assert np.array_equal(Xe, oracle.expand(wl.x, route["row_src"]))
    tr.grouped_gemm(p, d["w1"], d["w2"])
    O = host(v["O"][:R])
    e_of_row = np.repeat(np.arange(wl.E), route["counts"])
    O_ref = oracle.expert_rows(e_of_row, route["row_src"], wl.x, wl.w1, wl.w2)
    _assert_close(as_f64(O), O_ref, wl.dtype, f"{name} O")
    y = host(tr.combine_reduce(p, d["w"]))
    _assert_close(as_f64(y), oracle.combine(route["row_map"], wl.weights, O), wl.dtype,
                  f"{name} reduce of the GPU's O")


@pytest.mark.parametrize("name", ["c5", "c4", "c1"])
def test_combine_synthetic_outputs(name):
    """Reduce alone on seeded expert outputs (not produced by the GPU)."""
    say(f"combine {name}")
    wl = gen.make_workload(name)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl))
    route = oracle.route(wl.idx, wl.E)
    O = gen.make_expert_outputs(wl.T * wl.K, wl.H, wl.dtype, seed=11)
    Od = dev(O)
    y = host(tr.combine_reduce(p, d["w"], expert_out=Od))
    rows = np.arange(wl.T) if wl.T <= 2048 else sample_tokens(wl, route, 512)
    ref = oracle.combine(route["row_map"][rows], wl.weights[rows], O)
    _assert_close(as_f64(y[rows]), ref, wl.dtype, f"{name} combine")
    # unit weights
    y1 = host(tr.combine_reduce(p, None, expert_out=Od))
    _assert_close(as_f64(y1[rows]), oracle.combine(route["row_map"][rows], None, O), wl.dtype,
                  f"{name} combine w=1")


def test_combine_closed_forms():
    say("combine closed forms")
    wl = gen.make_workload("c2", T=512)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I)
    route = oracle.route(wl.idx, wl.E)
    # expert output 1 everywhere: y[t] = local weight sum, rounded once to bf16
    ones = torch.ones((wl.T * wl.K, wl.H), dtype=torch.bfloat16, device="cuda")
    y = host(tr.combine_reduce(p, d["w"], expert_out=ones))
    wsum = np.where(wl.idx >= 0, wl.weights.astype(np.float64), 0).sum(1)
    assert np.abs(as_f64(y) - wsum[:, None]).max() <= 2 ** -8 * wsum.max()
    # identity expert + unit weight + top-1 routing: y == x bit for bit
    idx1 = np.where(np.arange(wl.K)[None, :] == np.argmax(wl.idx >= 0, axis=1)[:, None], wl.idx, -1)
    p1 = tr.plan(torch.from_numpy(idx1).cuda(), E=wl.E, H=wl.H, I=wl.I)
    tr.expand(p1, d["x"])
    y1 = tr.combine_reduce(p1, None, expert_out=p1.views()["Xe"])
    assert torch.equal(y1.view(torch.int16), d["x"].view(torch.int16))
    # non-local weights are never read (NaN there changes nothing)
    wn = wl.weights.copy()
    wn[wl.idx < 0] = np.nan
    y2 = tr.combine_reduce(p, dev(wn), expert_out=ones)
    assert torch.equal(y2.view(torch.int16), torch.from_numpy(y).view(torch.int16).cuda())


def test_all_padding_gives_positive_zero():
    say("all padding")
    wl = gen.make_workload("c3", T=8, with_weights=True)
    wl.idx[:] = -1
    _, y = _forward(wl)
    assert (y == 0).all()          # +0 bits


@pytest.mark.parametrize("name", ["mid", "odd_bf16"])
def test_y_aliases_x(name):
    say(f"y aliases x {name}")
    wl = gen.make_workload(name, with_weights=True)
    _, y_sep = _forward(wl)
    _, y_al = _forward(wl, y_alias=True)
    assert np.array_equal(y_sep, y_al)


def test_forward_deterministic():
    say("determinism")
    wl = gen.make_workload("mid", with_weights=True)
    _, a = _forward(wl)
    _, b = _forward(wl)
    assert np.array_equal(a, b)


def test_error_convention_on_device():
    wl = gen.make_workload("c1", with_weights=True)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch.float32)
    with pytest.raises(TypeError):
        tr.forward(p, d["x"].to(torch.bfloat16), d["w"], d["w1"], d["w2"])
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(tr.TopReduceError) as ei:
        tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch.float32, ws=small)
    assert ei.value.status == -3


@pytest.mark.parametrize("name,flags", [("mid", 0), ("mid", tr.FLAG_GEMM_FORCE_TILED),
                                        ("mid", tr.FLAG_GEMM_FORCE_STREAM),
                                        ("mid_small_experts", 0), ("mid_f32", 0), ("c1", 0),
                                        ("rounds", 0), ("odd_bf16", 0), ("odd_i_bf16", 0)])
def test_up_x_equals_expand_then_up(name, flags):
    """GEMM1 gathering the received rows through the route table computes the
    same h, bit for bit, as expand followed by GEMM1 over Xe: the same rows
    reach the same tile positions and the arithmetic order is unchanged (fp32
    gathers as well)."""
    say(f"up_x {name} flags={flags}")
    wl = gen.make_workload(name, with_weights=True)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl), flags=flags)
    R = oracle.route(wl.idx, wl.E)["R"]
    v = p.views()
    tr.expand(p, d["x"])
    tr.grouped_gemm_up(p, d["w1"])
    h_ref = v["h"][:R].clone()
    v["h"][:R].zero_()
    tr.grouped_gemm_up_x(p, d["x"], d["w1"])
    torch.cuda.synchronize()
    h_ref_b, h_b = host(h_ref), host(v["h"][:R])
    assert np.array_equal(h_b.view(np.uint8), h_ref_b.view(np.uint8)), "h differs"


@pytest.mark.parametrize("T", [1, 3, 64])
def test_up_x_decode(T):
    """Decode batches (weight-streaming kernel) gathering from x: h equals the
    expand route's."""
    say(f"up_x c3 T={T}")
    wl = gen.make_workload("c3", T=T, variant="random", with_weights=True)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl))
    R = oracle.route(wl.idx, wl.E)["R"]
    v = p.views()
    tr.expand(p, d["x"])
    tr.grouped_gemm_up(p, d["w1"])
    h_ref = host(v["h"][:R].clone())
    v["h"][:R].zero_()
    tr.grouped_gemm_up_x(p, d["x"], d["w1"])
    torch.cuda.synchronize()
    assert np.array_equal(host(v["h"][:R]).view(np.uint8), h_ref.view(np.uint8))


@pytest.mark.parametrize("name,flags,T", [("mid", 0, None), ("mid", tr.FLAG_GEMM_FORCE_TILED, None),
                                          ("mid", tr.FLAG_GEMM_FORCE_STREAM, None),
                                          ("mid_small_experts", 0, None), ("rounds", 0, None),
                                          ("split", 0, None),
                                          ("c3", 0, 1), ("c3", 0, 64), ("c4", 0, None),
                                          ("c2", 0, None), ("c5", 0, None),
                                          ("odd_bf16", 0, None), ("wide_bf16", 0, None),
                                          ("odd_i_bf16", tr.FLAG_GEMM_FORCE_TILED, None)])
def test_forward_fused_equals_stages(name, flags, T):
    """moe_forward (GEMM1 gathering x, GEMM2 writing rows of received rows
    with one local slot straight to y, the reduce for the rest) equals the
    unfused composition expand -> grouped GEMM -> reduce bit for bit, with
    and without weights; so do the fused stage entry points."""
    say(f"fused forward {name} flags={flags} T={T}")
    wl = gen.make_workload(name, T=T, variant="random" if name == "c3" else "", with_weights=True)
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl), flags=flags)
    for w in (d["w"], None):
        y_f = tr.forward(p, d["x"], w, d["w1"], d["w2"])
        tr.expand(p, d["x"])
        tr.grouped_gemm(p, d["w1"], d["w2"])
        y_s = tr.combine_reduce(p, w)
        y_3 = torch.full_like(y_s, float("nan"))
        tr.grouped_gemm_up_x(p, d["x"], d["w1"])
        tr.grouped_gemm_down_y(p, d["w2"], w, y_3)
        tr.combine_reduce_multi(p, w, y_3)
        torch.cuda.synchronize()
        assert torch.equal(y_f.view(torch.int16), y_s.view(torch.int16)), "forward != stages"
        assert torch.equal(y_3.view(torch.int16), y_s.view(torch.int16)), "fused stages != stages"


# decode batches (at most 32 expanded rows): the forward runs the reduce
# inside GEMM2; one local expert, several, every slot local (dense), K = 8
gen.custom_spec("decode_k8", T=4, K=8, E=12, G=24, H=512, I=256, zipf_s=0.3, seed=16)
# more than 64 local experts (the decode kernels' block-wide expert table)
gen.custom_spec("decode_e100", T=2, K=16, E=100, G=100, H=512, I=256, zipf_s=0.0, seed=19)


@pytest.mark.parametrize("name,T,variant", [("c3", 1, ""), ("c3", 2, ""), ("c3", 1, "random"),
                                            ("c3", 2, "random"), ("c3", 2, "dense"),
                                            ("decode_k8", None, ""), ("decode_e100", None, "")])
def test_decode_forward_equals_stages(name, T, variant):
    """A decode forward (GEMM2 with the reduce folded in) equals the unfused
    composition expand -> grouped GEMM -> reduce bit for bit, with and without
    weights, NaN in the non-local weights included."""
    say(f"decode forward {name} T={T} {variant}")
    wl = gen.make_workload(name, T=T, variant=variant, with_weights=True)
    assert wl.T * wl.K <= 32
    d = upload(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=torch_dtype(wl))
    wn = wl.weights.copy()
    wn[~((wl.idx >= 0) & (wl.idx < wl.E))] = np.nan
    for w in (d["w"], None, dev(wn)):
        y_f = tr.forward(p, d["x"], w, d["w1"], d["w2"])
        tr.expand(p, d["x"])
        tr.grouped_gemm(p, d["w1"], d["w2"])
        y_s = tr.combine_reduce(p, w)
        torch.cuda.synchronize()
        assert torch.equal(y_f.view(torch.int16), y_s.view(torch.int16)), "forward != stages"
    ref = oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E)
    y = host(tr.forward(p, d["x"], d["w"], d["w1"], d["w2"]))
    _assert_close(as_f64(y), ref, wl.dtype, f"{name} decode y")
    # y aliasing x (GEMM1 has read x before GEMM2 writes y)
    xa = d["x"].clone()
    y_al = tr.forward(p, xa, d["w"], d["w1"], d["w2"], y=xa)
    torch.cuda.synchronize()
    assert np.array_equal(host(y_al), y)


# fewer expanded rows than one 256-row m-tile, experts of many rows (the
# tiled kernel when forced, or in the automatic mode past 128 rows)
gen.custom_spec("few_rows_big_experts", T=64, K=2, E=2, G=2, H=512, I=256, zipf_s=0.0, seed=17)
gen.custom_spec("few_rows_192", T=96, K=2, E=2, G=2, H=512, I=256, zipf_s=0.0, seed=18)


@pytest.mark.parametrize("name,flags", [("few_rows_big_experts", 0),
                                        ("few_rows_big_experts", tr.FLAG_GEMM_FORCE_TILED),
                                        ("few_rows_192", 0),
                                        ("few_rows_192", tr.FLAG_GEMM_FORCE_TILED)])
def test_forward_fewer_rows_than_a_tile(name, flags):
    say(f"forward {name} flags={flags}")
    wl = gen.make_workload(name, with_weights=True)
    _, y = _forward(wl, flags)
    ref = oracle.forward(wl.x, wl.idx, wl.weights, wl.w1, wl.w2, wl.E)
    _assert_close(as_f64(y), ref, wl.dtype, f"{name} y")


def test_decode_forward_duplicates_and_padding():
    """Decode batches with the same local expert twice in one row, and a
    DP-padded plan whose padding rows hold stale local ids: the forward
    (reduce inside GEMM2) equals the stages bit for bit and the oracle on the
    carrying rows; padding rows are +0."""
    wl = gen.make_workload("decode_k8", with_weights=True)
    idx = wl.idx.copy()
    idx[0, :3] = 2                      # expert 2 three times in row 0
    idx[1, :] = -1                      # a row with no route
    idx[2, 1] = idx[2, 0] = 5
    d = upload(wl)
    di = dev(idx)
    p = tr.plan(di, E=wl.E, H=wl.H, I=wl.I)
    y_f = tr.forward(p, d["x"], d["w"], d["w1"], d["w2"])
    tr.expand(p, d["x"])
    tr.grouped_gemm(p, d["w1"], d["w2"])
    y_s = tr.combine_reduce(p, d["w"])
    torch.cuda.synchronize()
    assert torch.equal(y_f.view(torch.int16), y_s.view(torch.int16))
    ref = oracle.forward(wl.x, idx, wl.weights, wl.w1, wl.w2, wl.E)
    _assert_close(as_f64(host(y_f)), ref, wl.dtype, "decode duplicates y")
    # padded: blocks of 2 rows, the second block carries one row
    bc = torch.tensor([2, 1], dtype=torch.int32, device="cuda")
    stale = idx.copy()
    stale[3] = np.arange(wl.K) % wl.E   # padding row with local ids
    pp = tr.plan(dev(stale), E=wl.E, H=wl.H, I=wl.I, block_rows=2, block_counts=bc)
    y_p = host(tr.forward(pp, d["x"], d["w"], d["w1"], d["w2"]))
    carry = np.array([True, True, True, False])
    ref_p = oracle.forward(wl.x, np.where(carry[:, None], stale, -1), wl.weights, wl.w1, wl.w2,
                           wl.E)
    _assert_close(as_f64(y_p), ref_p, wl.dtype, "decode padded y")
    assert (y_p[~carry] == 0).all()


@pytest.mark.parametrize("name,flags,T", [("mid", 0, None), ("mid", tr.FLAG_GEMM_FORCE_TILED, None),
                                          ("mid", tr.FLAG_GEMM_FORCE_STREAM, None),
                                          ("mid_small_experts", 0, None), ("c3", 0, 1)])
def test_forward_without_xe_buffer(name, flags, T):
    """A plan made with FLAG_NO_XE has a workspace without the expanded rows
    (smaller by (T*K + 256) * H * 2 bytes, Xe NULL); moe_forward and
    moe_grouped_gemm_up_x on it give the same bits as on a full plan, and the
    entry points over Xe refuse it."""
    say(f"forward without Xe {name} flags={flags} T={T}")
    wl = gen.make_workload(name, T=T, variant="random" if name == "c3" else "", with_weights=True)
    d = upload(wl)
    dt = torch_dtype(wl)
    p_full = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=dt, flags=flags)
    p_lean = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=dt, flags=flags | tr.FLAG_NO_XE)
    assert p_lean.views()["Xe"] is None
    assert p_full.ws.numel() - p_lean.ws.numel() == (p_full.R_cap + 256) * wl.H * 2
    y_full = tr.forward(p_full, d["x"], d["w"], d["w1"], d["w2"])
    y_lean = tr.forward(p_lean, d["x"], d["w"], d["w1"], d["w2"])
    R = int(tr.plan_stats(p_lean)[0])
    tr.grouped_gemm_up_x(p_lean, d["x"], d["w1"])
    tr.grouped_gemm_up_x(p_full, d["x"], d["w1"])
    torch.cuda.synchronize()
    assert torch.equal(y_lean.view(torch.int16), y_full.view(torch.int16))
    assert torch.equal(p_lean.views()["h"][:R].view(torch.int16),
                       p_full.views()["h"][:R].view(torch.int16))
    for call in (lambda: tr.expand(p_lean, d["x"]), lambda: tr.grouped_gemm_up(p_lean, d["w1"]),
                 lambda: tr.grouped_gemm(p_lean, d["w1"], d["w2"])):
        with pytest.raises(tr.TopReduceError):
            call()


def test_forward_past_2gib_x_takes_the_expand_path():
    """x of more than 2 GiB is beyond the gathering GEMM's 32-bit buffer
    offsets: moe_forward and moe_grouped_gemm_up_x then expand first and run
    GEMM1 over Xe, and the reduce covers every row. Same bits as the stages,
    and the oracle on sampled rows. (150016 rows x 7168 bf16 = 2.15 GB; 2
    local experts, few routes, so the GEMMs are small.)"""
    T, K, E, H, I = 150016, 2, 2, 7168, 128
    say(f"forward past 2 GiB: T={T} H={H}")
    g = torch.Generator(device="cuda").manual_seed(17)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    rng = np.random.default_rng(17)
    idx = np.full((T, K), -1, np.int64)
    rows = rng.choice(T, 300, replace=False)
    idx[rows, 0] = rng.integers(0, E, rows.size)
    idx[rows[:100], 1] = 1 - idx[rows[:100], 0]
    w = rng.random((T, K)).astype(np.float32)
    w1 = (rng.standard_normal((E, 2 * I, H)) / np.sqrt(H)).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) / np.sqrt(I)).astype(np.float32)
    w1b, w2b = gen.f32_to_bf16_bits(w1), gen.f32_to_bf16_bits(w2)
    d_idx, d_w, d_w1, d_w2 = dev(idx), dev(w), dev(w1b), dev(w2b)
    p = tr.plan(d_idx, E=E, H=H, I=I)
    y_f = tr.forward(p, x, d_w, d_w1, d_w2)
    tr.expand(p, x)
    tr.grouped_gemm(p, d_w1, d_w2)
    y_s = tr.combine_reduce(p, d_w)
    torch.cuda.synchronize()
    assert torch.equal(y_f.view(torch.int16), y_s.view(torch.int16))
    v = p.views()
    R = int(tr.plan_stats(p)[0])
    h_ref = v["h"][:R].clone()
    tr.grouped_gemm_up_x(p, x, d_w1)           # falls back to expand + GEMM1
    torch.cuda.synchronize()
    assert torch.equal(v["h"][:R].view(torch.int16), h_ref.view(torch.int16))
    with pytest.raises(tr.TopReduceError):
        tr.grouped_gemm_down_y(p, d_w2, d_w, y_f)
    toks = np.sort(rows[:24])
    sel = torch.from_numpy(toks).cuda()
    ref = oracle.forward(host(x[sel]), idx[toks], w[toks], w1b, w2b, E)
    _assert_close(as_f64(host(y_f[sel])), ref, "bf16", "y (sampled rows)")
    others = torch.from_numpy(np.setdiff1d(np.arange(T), rows)[:1000]).cuda()
    assert (host(y_f[others]) == 0).all()
