"""GPU tensors to the oracle's typed numpy arrays, row gathering and sampling.

The tolerances and ``compare`` live in tests/tolerance.py (numpy only) and are
re-exported here.
"""

import numpy as np
import torch

import oracle
from tests.tolerance import F32_ABS, F32_ROWSUM, ULPS, compare, ulp  # noqa: F401

DTYPE_OF = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16",
            torch.float64: "f64"}


def to_np(t):
    """Typed numpy copy of a tensor for the oracle (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def decoded(t):
    """Exact float64 values of a GPU/CPU tensor."""
    return oracle.decode(to_np(t), DTYPE_OF[t.dtype])


def mask_4d(mask, mode):
    """The mask in the oracle's 4-D broadcast form (length-1 broadcast axes)."""
    if mask is None or mode == "none":
        return None
    m = to_np(mask)
    if mode == "sq_sk":
        return m.reshape((1, 1) + m.shape[-2:])
    if mode == "b_sq_sk":
        return m.reshape((m.shape[0], 1) + m.shape[-2:])
    if mode == "b_1_sk":
        return m.reshape(m.shape[0], 1, 1, m.shape[-1])
    return m


def sample_rows(n_rows, Sq, k=192, seed=0):
    """Row numbers to check one by one: ends, query positions 0, 1 and Sq-1,
    and a seeded uniform sample."""
    rng = np.random.default_rng(seed)
    fixed = {0, 1, n_rows - 1, n_rows - 2, Sq - 1, min(Sq, n_rows - 1), n_rows // 2}
    pick = rng.choice(n_rows, size=min(k, n_rows), replace=False)
    return sorted({int(r) for r in fixed if 0 <= r < n_rows} | {int(r) for r in pick})


def gather_rows(t, rows):
    """Rows (flat numbers over B*H*Sq) of a 4-D GPU tensor, as a typed numpy [n, Sk]."""
    B, H, Sq, Sk = t.shape
    idx = torch.as_tensor(rows, device=t.device, dtype=torch.long)
    q = idx % Sq
    h = (idx // Sq) % H
    b = idx // (Sq * H)
    return to_np(t[b, h, q, :])


def gather_mask_rows(mask, mode, shape, rows):
    """The mask row each flat row reads (typed numpy [n, Sk]), or None."""
    if mask is None:
        return None
    B, H, Sq, Sk = shape
    idx = torch.as_tensor(rows, device=mask.device, dtype=torch.long)
    q = idx % Sq
    h = (idx // Sq) % H
    b = idx // (Sq * H)
    if mode == "sq_sk":
        m = mask.reshape(Sq, Sk)[q]
    elif mode == "b_sq_sk":
        m = mask.reshape(B, Sq, Sk)[b, q]
    elif mode == "b_1_sk":
        m = mask.reshape(B, Sk)[b]
    else:
        m = mask[b, h, q]
    return to_np(m)
