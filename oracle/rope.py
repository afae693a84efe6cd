"""Rotary position embedding at tree positions — TEST INFRASTRUCTURE (see ``oracle/__init__``).

[PTP] ("Prefix tree packing", furtherai.github.io): a packed row must reproduce every
unpacked sequence exactly.  For rotary attention that means each token turns by the angle of
its position in its own sequence: the plan's pos_ids (reading R14: position id = index in the
unpacked sequence), never the row offset.

The pages do not print a rotary formula; reading R22 takes the common rotate-half form: with
pairs (x[i], x[i + D/2]) for i < D/2 and angle a_i = pos * theta^(-2i/D), the pair turns by
a_i in its plane:  (x1, x2) -> (x1 cos a - x2 sin a, x2 cos a + x1 sin a).  float64 throughout.
"""
from __future__ import annotations

import numpy as np


def angles(pos, D: int, theta: float) -> np.ndarray:
    """a[..., i] = pos * theta^(-2i/D), float64, shape pos.shape + (D/2,)."""
    i = np.arange(D // 2, dtype=np.float64)
    inv_freq = np.power(float(theta), -2.0 * i / D)
    return np.asarray(pos, np.float64)[..., None] * inv_freq


def rotate(x, pos, theta: float = 10000.0, inverse: bool = False) -> np.ndarray:
    """Rotate x [..., H, D] (any float dtype; computed in float64) at positions pos [...]."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    a = angles(pos, D, theta)[..., None, :]          # broadcast over heads
    if inverse:
        a = -a
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)
