"""Synthetic input generators: determinism and the structure each workload
must have (row patterns, locality rules, distinct experts, weights)."""

import numpy as np
import pytest

import gen


def _eq(a, b):
    return a.dtype == b.dtype and a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("name,T", [("c1", None), ("c2", 256), ("c3", 8), ("c4", None), ("c5", 512)])
def test_deterministic(name, T):
    a = gen.make_workload(name, T=T)
    b = gen.make_workload(name, T=T)
    for f in ("idx", "global_idx", "weights", "x", "real"):
        assert _eq(getattr(a, f), getattr(b, f)), f
    c = gen.make_workload(name, T=T, seed=a.seed + 1)
    assert not _eq(a.x, c.x)


def test_weights_deterministic_and_subset_independent():
    a = gen.make_workload("c1", with_weights=True)
    b = gen.make_workload("c1", with_weights=True)
    assert _eq(a.w1, b.w1) and _eq(a.w2, b.w2)
    assert a.w1.shape == (8, 256, 256) and a.w2.shape == (8, 256, 128)
    # std = 1/sqrt(fan_in)
    assert abs(a.w1.std() - 1 / 16) < 0.003 and abs(a.w2.std() - 1 / np.sqrt(128)) < 0.004


def test_bf16_rounding():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0, -0.0, np.inf, 3.0e38], np.float32)
    b = gen.f32_to_bf16_bits(f)
    back = gen.bf16_bits_to_f32(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: to even -> 1.0; 1 + 3*2^-8 -> 1 + 2^-6
    assert back.tolist()[:6] == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 0.0, -0.0]
    assert b[5] == 0x8000 and np.isinf(back[6])


def _distinct_rows(g):
    for row in g:
        v = row[row >= 0]
        assert len(set(v.tolist())) == len(v)


def test_c1_structure():
    wl = gen.make_workload("c1")
    assert wl.dtype == "f32" and wl.x.dtype == np.float32
    assert (wl.idx >= 0).all() and (wl.idx < 8).all()
    _distinct_rows(wl.idx)
    assert np.allclose(wl.weights.sum(1), 1.0, atol=1e-6)


def test_c2_structure():
    wl = gen.make_workload("c2", T=1024)
    assert (wl.global_idx >= 0).all() and (wl.global_idx < 256).all()
    _distinct_rows(wl.global_idx)
    assert ((wl.idx >= 0).any(1)).all()            # every row has a local route
    assert np.array_equal(wl.idx >= 0, wl.global_idx < 16)
    assert np.allclose(wl.weights.sum(1), 1.0, atol=1e-5)
    assert wl.x.dtype == np.uint16


@pytest.mark.parametrize("T", [1, 2, 4, 8, 64])
def test_c3_stride(T):
    wl = gen.make_workload("c3", T=T)
    real = np.arange(T) % 8 == 0
    assert np.array_equal(wl.real, real)
    # DeepEP issue #760 repro: ids k * 28, weights 1/16; only id 0 is local
    assert np.array_equal(wl.global_idx[real], np.tile(np.arange(16) * 28, (real.sum(), 1)))
    assert (wl.global_idx[~real] == -1).all()
    assert (wl.idx[real, 0] == 0).all() and (wl.idx[real, 1:] == -1).all()
    assert (wl.weights[real] == np.float32(1 / 16)).all() and (wl.weights[~real] == 0).all()
    assert (wl.x[~real] == 0).all() and (wl.x[real] != 0).any()


def test_c3_random_variant():
    wl = gen.make_workload("c3", T=64, variant="random")
    assert ((wl.idx[wl.real] >= 0).any(1)).all()
    _distinct_rows(wl.global_idx)
    assert (wl.idx[~wl.real] == -1).all()


def test_c4_dp_padding():
    wl = gen.make_workload("c4")
    assert wl.T == 960 and wl.real.sum() == 127       # SGLang PR #6092: [120,1,...,1]
    for j, c in enumerate([120, 1, 1, 1, 1, 1, 1, 1]):
        blk = wl.real[120 * j:120 * (j + 1)]
        assert blk[:c].all() and not blk[c:].any()
    assert (wl.idx[~wl.real] == -1).all() and (wl.x[~wl.real] == 0).all()
    counts = np.bincount(wl.idx[wl.idx >= 0], minlength=32)
    assert (counts == 0).sum() >= 3                   # skew leaves experts empty
    _distinct_rows(wl.global_idx)


def test_c5_zipf_skew():
    wl = gen.make_workload("c5", T=4096)
    assert ((wl.idx >= 0).any(1)).all()
    counts = np.bincount(wl.idx[wl.idx >= 0], minlength=32)
    assert counts.max() > 5 * counts.min() > 0
    _distinct_rows(wl.global_idx)
