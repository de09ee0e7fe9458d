"""Oracle step 4: rotary position embedding at tree depth, fp64.

[DAG "Positions"]: the position of a token is its graph depth, so every
parent-child step has relative distance 1 wherever the two sit in the row.
With roots at depth 0 the depth of the t-th token of an unpacked sequence is
t, so the oracle rotates each unpacked sequence at positions 0..L-1.

Reading (the pages do not give the RoPE variant): rotate-half pairing of
dimensions i and i + D/2, frequency theta^(-2i/D) for i < D/2.
"""

from __future__ import annotations

import numpy as np


def rope(x, pos, theta: float = 10000.0) -> np.ndarray:
    """x [L, H, D] (any float), pos [L] -> rotated copy in fp64."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / D)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv_freq[None, :]     # [L, half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
