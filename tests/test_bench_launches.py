"""bench.py times the forward's GEMM launches as moe_forward minus its reduce
launch, and names those launches; both follow from which kernels the library
picks for a shape. The committed rocprofv3 traces of the forward record the
kernels that actually ran: the names bench.py derives for each traced
workload must be exactly the `gemm_*` kernels of that trace."""

import os
import re

import pytest

import bench
import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MI355X_CUS = 256

# (profile, workload, received rows T)
TRACED = [
    ("kernels_c2_forward.md", "c2", None),
    ("kernels_c3_T1_forward.md", "c3", 1),
    ("kernels_c3_T64_forward.md", "c3", 64),
    ("kernels_c4_forward.md", "c4", None),
    ("kernels_c5_forward.md", "c5", None),
]


def _traced_gemms(fname):
    with open(os.path.join(ROOT, "profiles", fname)) as f:
        return {m.group(1) for m in re.finditer(r"^\| `(gemm_[^`]*)`", f.read(), re.M)}


@pytest.mark.parametrize("fname,cfg,T", TRACED)
def test_named_launches_match_trace(fname, cfg, T):
    c = gen.CONFIGS[cfg]
    T = c.T if T is None else T
    _, _, _, names = bench.forward_gemm_launches(c.dtype == "bf16", T, c.K, c.E, c.H, c.I,
                                                 MI355X_CUS)
    assert {n.split(" (")[0] for n in names} == _traced_gemms(fname)


def test_reduce_inside_gemm2_only_for_decode_batches():
    # the decode trace has no reduce kernel; the others have combine_rows
    with open(os.path.join(ROOT, "profiles", "kernels_c3_T1_forward.md")) as f:
        assert "combine_rows" not in f.read()
    with open(os.path.join(ROOT, "profiles", "kernels_c3_T64_forward.md")) as f:
        assert "combine_rows" in f.read()
    c = gen.CONFIGS["c3"]
    for T, folded in ((1, True), (2, True), (3, False), (8, False), (64, False)):
        assert bench.forward_gemm_launches(True, T, c.K, c.E, c.H, c.I, MI355X_CUS)[2] == folded
    # fp32 gathers in GEMM1 and always runs the full reduce
    c1 = gen.CONFIGS["c1"]
    assert bench.forward_gemm_launches(False, c1.T, c1.K, c1.E, c1.H, c1.I, MI355X_CUS)[:3] == \
        (True, False, False)
