"""Helpers for the GPU tests: move generator arrays to the device and back,
and run the library's path through the Python binding (C ABI)."""

import sys

import numpy as np
import torch

import gen


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype: str = None) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """cuda tensor -> numpy; bf16 comes back as uint16 bits."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return gen.bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def torch_dtype(wl) -> torch.dtype:
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def upload(wl, idx_dtype=torch.int64, global_ids=False):
    """Device tensors of a workload (weights only if generated)."""
    idx = wl.global_idx if global_ids else wl.idx
    d = dict(idx=torch.from_numpy(idx).to(idx_dtype).cuda(), w=dev(wl.weights), x=dev(wl.x))
    if wl.w1 is not None:
        d["w1"] = dev(wl.w1)
        d["w2"] = dev(wl.w2)
    return d


def sample_tokens(wl, route, n, seed=0):
    """A sample of received rows for full-size checks: the first and last rows,
    rows at the edges of expert segments, rows of the largest and smallest
    experts, rows without a local route, and random ones."""
    rng = np.random.default_rng(seed)
    picks = {0, wl.T - 1}
    off = route["offsets"]
    for e in range(wl.E):
        if route["counts"][e] > 0:
            picks.add(int(route["row_src"][off[e]]))
            picks.add(int(route["row_src"][off[e + 1] - 1]))
    nolocal = np.nonzero(~(wl.idx >= 0).any(1))[0]
    picks.update(int(t) for t in nolocal[:2])
    picks = sorted(picks)
    if len(picks) > n:
        picks = sorted(rng.choice(picks, n, replace=False).tolist())
    rest = np.setdiff1d(np.arange(wl.T), picks)
    extra = max(0, n - len(picks))
    if extra and rest.size:
        picks = sorted(picks + rng.choice(rest, min(extra, rest.size), replace=False).tolist())
    return np.array(picks, dtype=np.int64)
