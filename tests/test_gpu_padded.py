"""DP-padded received buffers on the GPU (SGLang PR #6092 review thread:
data-parallel workers' batches padded to one size; padding rows hold no query
and must cost no expert work; only effective rows go to the communication
buffer).

moe_plan_padded against the oracle's padded route table (bit-exact, with
padding rows holding stale expert ids that a plain plan would route), the
forward on such a plan (padding rows +0; carrying rows equal to the plain path
with the padding ids cleared, bit for bit, and to the oracle on sampled rows),
and moe_compact_rows in both directions against the oracle's compaction."""

import numpy as np
import pytest
import torch

import gen
import oracle
import top_reduce_amd as tr
from tests._gpu import as_f64, dev, host, say, upload
from tests._util import max_err, tolerance

pytestmark = pytest.mark.gpu


def _carrying_mask(T, B, counts):
    t = np.arange(T)
    return (t - (t // B) * B) < np.asarray(counts, np.int64)[t // B] if T else np.zeros(0, bool)


def _check_route(idx_np, E, B, counts, idx_dtype=torch.int64, flags=0):
    T, K = idx_np.shape
    say(f"padded route T={T} K={K} E={E} B={B} idx={idx_dtype}")
    idx = torch.from_numpy(np.ascontiguousarray(idx_np)).to(idx_dtype).cuda()
    bc = torch.from_numpy(np.asarray(counts, np.int32)).cuda()
    p = tr.plan(idx, E=E, H=256, I=128, block_rows=B, block_counts=bc, flags=flags)
    stats = tr.plan_stats(p)
    v = p.views()
    ref = oracle.route(idx_np, E, block_rows=B, block_counts=np.asarray(counts, np.int32))
    R = ref["R"]
    assert np.array_equal(v["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(v["offsets"].cpu().numpy(), ref["offsets"])
    assert np.array_equal(v["row_map"].cpu().numpy(), ref["row_map"])
    assert np.array_equal(v["row_src"][:R].cpu().numpy(), ref["row_src"])
    assert np.array_equal(v["row_k"][:R].cpu().numpy(), ref["row_k"])
    carry = _carrying_mask(T, B, counts)
    local = (idx_np >= 0) & (idx_np < E) & carry[:, None]
    foreign = ~((idx_np >= 0) & (idx_np < E)) & carry[:, None]
    assert stats == (R, int(local.any(1).sum()), int(foreign.sum()),
                     int((ref["counts"] == 0).sum()))
    assert int(v["stats"][5]) == int(carry.sum())
    # experts of the streaming and of the tiled GEMM, per the plan's mode
    c = ref["counts"]
    # (the automatic mode streams every expert of a batch of at most 128
    # expanded rows)
    lo = (1 if flags & tr.FLAG_GEMM_FORCE_TILED
          else np.iinfo(np.int64).max if flags & tr.FLAG_GEMM_FORCE_STREAM or T * K <= 128
          else 33)
    assert int(v["stats"][6]) == int(((c > 0) & (c < lo)).sum())
    assert int(v["stats"][7]) == int((c >= lo).sum())
    # padding rows are among the rows the reduce writes (as +0)
    n_rest = int(v["stats"][4])
    rest_rows = v["tok_rest"][:n_rest].cpu().numpy()
    assert np.all(np.diff(rest_rows) > 0)   # ascending row order
    rest = set(rest_rows.tolist())
    assert set(np.nonzero(~carry)[0].tolist()) <= rest
    return p


def _stale(idx, real, E, seed):
    """Padding rows given valid local ids (as a router run on zero inputs
    would leave them), so that only the padding information hides them."""
    rng = np.random.default_rng(seed)
    out = idx.copy()
    pads = np.nonzero(~real)[0]
    out[pads] = rng.integers(0, E, size=(pads.size, idx.shape[1]))
    return out


def test_padded_route_c4_stale_pad_ids():
    wl = gen.make_workload("c4")
    counts = gen.C4_WORKER_COUNTS
    stale = _stale(wl.idx, wl.real, wl.E, 1)
    _check_route(stale, wl.E, gen.C4_WORKER_ROWS, counts)
    _check_route(stale, wl.E, gen.C4_WORKER_ROWS, counts, idx_dtype=torch.int32)


def test_padded_route_edge_cases():
    rng = np.random.default_rng(11)
    # many scan blocks, counts clamped on both sides, last block partial
    T, B = 5000, 96
    _check_route(rng.integers(-1, 16, size=(T, 8)), 16, B,
                 rng.integers(-2, B + 20, size=-(-T // B)))
    # one scan block (T * K <= 4096), short blocks
    T, B = 1000, 7
    _check_route(rng.integers(-1, 6, size=(T, 4)), 6, B, rng.integers(0, 9, size=-(-T // B)))
    # every block empty: nothing routed whatever the ids
    _check_route(rng.integers(0, 8, size=(600, 8)), 8, 60, np.zeros(10, np.int32))
    # every row carries: the plain plan
    idx = rng.integers(-1, 8, size=(700, 8))
    _check_route(idx, 8, 100, np.full(7, 100, np.int32))
    # one-row blocks, the most blocks allowed
    T = 4096
    _check_route(rng.integers(-1, 32, size=(T, 2)), 32, 1, rng.integers(0, 2, size=T))
    # T = 0
    _check_route(np.zeros((0, 8), np.int64), 4, 10, np.zeros(0, np.int32))
    # 64 experts over ~254 scan blocks (batched partial sums)
    T, B = 20000, 96
    _check_route(rng.integers(-1, 64, size=(T, 8)), 64, B, rng.integers(0, B + 1, size=-(-T // B)))
    # small batches (the single-block kernel, T * K <= 1024): padding blocks
    # with counts below 0, inside and above the block, rows straddling waves
    T, B = 200, 16
    _check_route(rng.integers(-1, 10, size=(T, 4)), 10, B, rng.integers(-3, B + 4, size=-(-T // B)))
    T, B = 341, 5
    _check_route(rng.integers(-1, 7, size=(T, 3)), 7, B, rng.integers(-1, B + 2, size=-(-T // B)))
    _check_route(rng.integers(0, 3, size=(20, 8)), 3, 4, np.array([4, 0, 2, 9, 1], np.int32),
                 flags=tr.FLAG_GEMM_FORCE_TILED)
    # the GEMM modes' expert counts (experts with 1..32 and with more routes)
    T, B = 3000, 50
    idx = np.where(rng.random((T, 4)) < 0.02, rng.integers(0, 40, size=(T, 4)),
                   rng.integers(40, 48, size=(T, 4)))
    for fl in (0, tr.FLAG_GEMM_FORCE_TILED, tr.FLAG_GEMM_FORCE_STREAM):
        _check_route(idx, 48, B, rng.integers(0, B + 1, size=-(-T // B)), flags=fl)


@pytest.fixture(scope="module")
def c4():
    wl = gen.make_workload("c4", with_weights=True)
    return wl, upload(wl)


@pytest.mark.parametrize("flags", [0, tr.FLAG_GEMM_FORCE_TILED, tr.FLAG_GEMM_FORCE_STREAM])
def test_padded_forward_c4(c4, flags):
    """The forward over the padded c4 buffer with stale padding ids: padding
    rows are +0, the carrying rows equal the plain plan's forward with the
    padding ids cleared (bit for bit), and the oracle on sampled rows."""
    say(f"padded forward c4 flags={flags}")
    wl, d = c4
    stale = torch.from_numpy(_stale(wl.idx, wl.real, wl.E, 2)).cuda()
    w_stale = d["w"].clone()
    w_stale[torch.from_numpy(~wl.real).cuda()] = 0.5       # stale weights too
    bc = torch.tensor(gen.C4_WORKER_COUNTS, dtype=torch.int32, device="cuda")
    p_pad = tr.plan(stale, E=wl.E, H=wl.H, I=wl.I, flags=flags,
                    block_rows=gen.C4_WORKER_ROWS, block_counts=bc)
    p_plain = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, flags=flags)
    y_pad = tr.forward(p_pad, d["x"], w_stale, d["w1"], d["w2"])
    y_plain = tr.forward(p_plain, d["x"], d["w"], d["w1"], d["w2"])
    # the stage form on the padded plan: expand, GEMM over Xe, reduce
    tr.expand(p_pad, d["x"])
    tr.grouped_gemm(p_pad, d["w1"], d["w2"])
    y_st = tr.combine_reduce(p_pad, w_stale)
    torch.cuda.synchronize()
    s_pad, s_plain = tr.plan_stats(p_pad), tr.plan_stats(p_plain)
    n_pad_slots = int((~wl.real).sum()) * wl.K        # all -1 in the plain ids
    assert s_pad == (s_plain[0], s_plain[1], s_plain[2] - n_pad_slots, s_plain[3])
    assert torch.equal(y_pad.view(torch.int16), y_plain.view(torch.int16))
    assert torch.equal(y_st.view(torch.int16), y_plain.view(torch.int16))
    pads = torch.from_numpy(~wl.real).cuda()
    assert (y_pad[pads].view(torch.int16) == 0).all()
    toks = np.array([0, 57, 119, 120, 360, 840])
    ref = oracle.forward(wl.x[toks], wl.idx[toks], wl.weights[toks], wl.w1, wl.w2, wl.E)
    got = as_f64(host(y_pad[torch.from_numpy(toks).cuda()]))
    assert max_err(got, ref) <= tolerance(ref, "bf16")


def _compact_case(src_np, B, counts, seed):
    T = src_np.shape[0]
    say(f"compact T={T} row={src_np.shape[1:]} {src_np.dtype} B={B}")
    src = dev(src_np)
    bc = torch.from_numpy(np.asarray(counts, np.int32)).cuda()
    n = torch.full((1,), -5, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    tr.compact_rows(src, B, bc, dst=dst, n_out=n)
    ref, nref = oracle.compact_rows(src_np, B, np.asarray(counts, np.int32))
    torch.cuda.synchronize()
    assert int(n.item()) == nref
    assert np.array_equal(host(dst)[:nref].view(np.uint8), ref.view(np.uint8))
    # back to the padded layout over a buffer of junk: carrying rows restored,
    # padding rows untouched
    junk_np = np.random.default_rng(seed).integers(0, 255, size=src_np.nbytes,
                                                   dtype=np.uint8).view(src_np.dtype)
    junk_np = junk_np.reshape(src_np.shape)
    padded = dev(junk_np)
    tr.compact_rows(dst, B, bc, dst=padded, to_padded=True)
    ref_back, _ = oracle.compact_rows(ref, B, np.asarray(counts, np.int32), to_padded=True,
                                      dst=junk_np)
    torch.cuda.synchronize()
    assert np.array_equal(host(padded).view(np.uint8), ref_back.view(np.uint8))


def test_compact_rows_c4_buffers():
    """The c4 communication buffer: x (bf16, 16-byte copies), the ids (int64)
    and the weights (fp32) of the 127 effective rows out of 960."""
    wl = gen.make_workload("c4")
    B, counts = gen.C4_WORKER_ROWS, gen.C4_WORKER_COUNTS
    _compact_case(wl.x, B, counts, 1)
    _compact_case(wl.idx, B, counts, 2)
    _compact_case(wl.weights, B, counts, 3)


def test_compact_rows_edge_cases():
    rng = np.random.default_rng(12)
    # 12-byte rows (4-byte copies), clamped counts, a partial last block
    T, B = 1001, 50
    _compact_case(rng.random((T, 3), dtype=np.float32), B,
                  rng.integers(-3, 60, size=-(-T // B)), 4)
    # 4-byte rows, one-row blocks (most blocks allowed)
    T = 4096
    _compact_case(rng.integers(0, 1 << 30, size=(T, 1)).astype(np.int32), 1,
                  rng.integers(0, 2, size=T), 5)
    # wide rows spanning several wavefront slabs, and a ragged slab
    _compact_case(rng.integers(0, 1 << 16, size=(40, 7168 + 256), dtype=np.uint16), 8,
                  np.array([8, 0, 3, 9, 1]), 6)
    # nothing carries
    _compact_case(rng.random((64, 4), dtype=np.float32), 16, np.zeros(4, np.int32), 7)
    # T = 0 still reports n = 0
    n = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    tr.compact_rows(torch.zeros((0, 4), device="cuda"), 4,
                    torch.zeros(0, dtype=torch.int32, device="cuda"), n_out=n)
    torch.cuda.synchronize()
    assert int(n.item()) == 0


gen.custom_spec("pad_bf16", T=600, K=8, E=8, G=32, H=512, I=256, zipf_s=0.8, seed=21)
gen.custom_spec("pad_f32", T=300, K=4, E=6, G=12, H=264, I=72, dtype="f32", zipf_s=0.5, seed=22)


@pytest.mark.parametrize("name,flags,idx_dtype", [
    ("pad_bf16", 0, torch.int64), ("pad_bf16", tr.FLAG_NO_XE, torch.int32),
    ("pad_bf16", tr.FLAG_GEMM_FORCE_TILED | tr.FLAG_NO_XE, torch.int64),
    ("pad_f32", 0, torch.int32)])
def test_padded_forward_small(name, flags, idx_dtype):
    """Every row compared: a padded plan over rows whose padding holds stale
    ids gives the plain plan's output on the carrying rows (padding ids
    cleared) bit for bit, +0 on padding rows, and the oracle's values within
    tolerance; with and without the expanded buffer, for bf16 and fp32."""
    say(f"padded forward {name} flags={flags} idx={idx_dtype}")
    wl = gen.make_workload(name, with_weights=True)
    B = 64
    nb = -(-wl.T // B)
    counts = np.random.default_rng(wl.seed).integers(-3, B + 5, size=nb).astype(np.int32)
    carry = _carrying_mask(wl.T, B, counts)
    stale = _stale(wl.idx, carry, wl.E, 3)
    clean = np.where(carry[:, None], wl.idx, -1)
    d = upload(wl)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    p_pad = tr.plan(torch.from_numpy(stale).to(idx_dtype).cuda(), E=wl.E, H=wl.H, I=wl.I,
                    dtype=dt, flags=flags, block_rows=B,
                    block_counts=torch.from_numpy(counts).cuda())
    p_plain = tr.plan(torch.from_numpy(clean).cuda(), E=wl.E, H=wl.H, I=wl.I, dtype=dt,
                      flags=flags & ~tr.FLAG_NO_XE)
    y_pad = tr.forward(p_pad, d["x"], d["w"], d["w1"], d["w2"])
    y_plain = tr.forward(p_plain, d["x"], d["w"], d["w1"], d["w2"])
    torch.cuda.synchronize()
    bits = torch.int16 if dt == torch.bfloat16 else torch.int32
    assert torch.equal(y_pad.view(bits), y_plain.view(bits))
    assert (y_pad[torch.from_numpy(~carry).cuda()].view(bits) == 0).all()
    ref = oracle.forward(wl.x, clean, wl.weights, wl.w1, wl.w2, wl.E)
    assert max_err(as_f64(host(y_pad)), ref) <= tolerance(ref, wl.dtype)
