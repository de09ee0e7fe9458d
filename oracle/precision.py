"""Rounding to a storage dtype, done directly from fp64.

The bf16 workloads keep q, k, v and the rotated q, k in bf16 tensors.  The
oracle computes in fp64 but models that storage: after the rotary embedding
the rotated q and k are rounded to the tensor dtype, exactly once, with
round-to-nearest-even on the fp64 value (no intermediate fp32 step, so no
double rounding).
"""

from __future__ import annotations

import numpy as np


def round_to(x, dtype: str | None) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    if dtype is None or dtype == "f64":
        return x
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        # bf16 keeps 8 significant bits; an fp64 has 53, so drop 45 low bits with RNE
        u = np.ascontiguousarray(x).view(np.uint64)
        lsb = (u >> np.uint64(45)) & np.uint64(1)
        r = (u + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
        return r.view(np.float64)
    raise ValueError(dtype)
