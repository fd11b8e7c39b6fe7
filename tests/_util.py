"""Helpers shared by the tests (fixture parsing, tolerances)."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    """Parse a `key = value` fixture; numeric values become int/float, lists of
    numbers become lists."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            parts = v.split()

            def num(s):
                try:
                    return int(s)
                except ValueError:
                    return float(s)
            out[k] = num(parts[0]) if len(parts) == 1 else [num(p) for p in parts]
    return out


def tolerance(ref: np.ndarray, dtype: str) -> float:
    """Output bar: bf16 max|d| <= 1e-2 max|ref| + 1e-3; fp32 max|d| <= 1e-5 max|ref|."""
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    if dtype == "bf16":
        return 1e-2 * m + 1e-3
    return 1e-5 * m


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got.astype(np.float64) - ref.astype(np.float64))))
