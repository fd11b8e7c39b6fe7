"""moe_forward_noalloc (plan + forward in the library's static workspace)
through the C ABI against moe_plan + moe_forward on a caller workspace: the
same bits, on two calls in a row where the second has a smaller batch (the
scratch keeps the first call's contents), on the weight-streaming decode
path, the tiled MFMA path and the fp32 path; and a batch past the scratch
size is refused with TR_EUNSUPPORTED."""

import numpy as np
import pytest
import torch

import gen
import top_reduce_amd as tr
from tests._gpu import say, torch_dtype, upload

pytestmark = pytest.mark.gpu

gen.custom_spec("noalloc_mid", T=1024, K=8, E=8, G=64, H=1024, I=512, zipf_s=1.0, seed=31)


def _pair(wl, flags=0):
    d = upload(wl)
    dt = torch_dtype(wl)
    p = tr.plan(d["idx"], E=wl.E, H=wl.H, I=wl.I, dtype=dt, flags=flags)
    y_ref = tr.forward(p, d["x"], d["w"], d["w1"], d["w2"])
    y = torch.full_like(y_ref, float("nan"))
    tr.forward_noalloc(d["idx"], d["x"], d["w"], d["w1"], d["w2"], y, E=wl.E, flags=flags)
    y1_ref = tr.forward(p, d["x"], None, d["w1"], d["w2"])
    y1 = torch.full_like(y_ref, float("nan"))
    tr.forward_noalloc(d["idx"], d["x"], None, d["w1"], d["w2"], y1, E=wl.E, flags=flags)
    torch.cuda.synchronize()
    iview = torch.int16 if dt == torch.bfloat16 else torch.int32
    assert torch.equal(y.view(iview), y_ref.view(iview)), "weighted forward differs"
    assert torch.equal(y1.view(iview), y1_ref.view(iview)), "unweighted forward differs"


@pytest.mark.parametrize("name,T_big,T_small,variant", [
    ("c3", 64, 8, "random"),          # weight-streaming GEMMs (decode)
    ("c3", 64, 1, "dense"),
    ("noalloc_mid", 1024, 300, ""),   # tiled MFMA GEMMs, fused GEMM2 epilogue
    ("c1", 64, 17, ""),               # fp32: expand, FMA GEMMs, full reduce
])
def test_noalloc_matches_forward_twice(name, T_big, T_small, variant):
    for T in (T_big, T_small):
        say(f"noalloc {name} T={T} {variant}")
        wl = gen.make_workload(name, T=T, variant=variant, with_weights=True)
        _pair(wl)


def test_noalloc_refuses_batch_past_scratch():
    wl = gen.make_workload("c3", T=8, with_weights=True)
    d = upload(wl)
    big_T = 1 << 16
    idx = torch.full((big_T, wl.K), -1, dtype=torch.int64, device="cuda")
    x = torch.zeros((big_T, wl.H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    with pytest.raises(tr.TopReduceError) as ei:
        tr.forward_noalloc(idx, x, None, d["w1"], d["w2"], y, E=wl.E)
    assert ei.value.status == -2
    assert "static scratch" in str(ei.value)
