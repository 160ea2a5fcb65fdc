"""Worker side of the every-row parity check of whole workloads.

Each task is a block of whole (b, h) planes: the typed inputs of those planes,
their mask planes in the oracle's broadcast form, and the GPU's typed output.
The worker runs the float64 oracle on every row of the block and compares
element by element with ``tests.tolerance.compare``. No torch here, so the
worker processes start fast and never touch the GPU.
"""

import numpy as np

import oracle
from tests.tolerance import compare


def _merge(stats, s):
    for k, v in s.items():
        stats[k] = max(stats.get(k, 0.0), v)
    return stats


def forward_block(dt, x4, m4, got4, scale, causal, mask_kind, label):
    """x4, got4: typed [k, 1, Sq, Sk]; m4: broadcastable 4-D mask or None."""
    k, _, Sq, Sk = x4.shape
    ref = oracle.forward_rows(x4, dt, range(k * Sq), m4, scale, causal, mask_kind)
    got = oracle.decode(got4.reshape(k * Sq, Sk), dt)
    return compare(got, ref, dt, label, rowsum=True)


def backward_block(dt, y4, dy4, got4, scale, label):
    """y4, dy4, got4: typed [k, 1, Sq, Sk]."""
    k, _, Sq, Sk = y4.shape
    ref = oracle.backward_rows(y4, dy4, dt, range(k * Sq), scale)
    got = oracle.decode(got4.reshape(k * Sq, Sk), dt)
    return compare(got, ref, dt, label)


def mask_planes(m4, planes, H):
    """Mask of planes p = b*H + h in broadcast form [k or 1, 1, Sq or 1, Sk]."""
    if m4 is None:
        return None
    planes = np.asarray(planes)
    if m4.shape[0] == 1 and m4.shape[1] == 1:
        return m4
    b = planes // H if m4.shape[0] > 1 else np.zeros_like(planes)
    h = planes % H if m4.shape[1] > 1 else np.zeros_like(planes)
    return m4[b, h][:, None]


__all__ = ["forward_block", "backward_block", "mask_planes", "_merge"]
