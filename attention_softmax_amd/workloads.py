"""Seeded synthetic inputs for the fused scaled-masked softmax.

This module only draws random tensors; it holds none of the softmax
arithmetic. Both the HIP path (through the binding) and the float64 oracle are
fed from what it returns, so a parity check compares the two on the same
bytes.

The five workloads below are the attention-score tensors the operation is
measured on: fp32 [8,32,1024,1024] with a per-batch key-padding mask (the
~1 GB fp32 score tensor of lmnt.cn "Custom fused Softmax operator in CUDA,
wrapped into PyTorch", sec. 1.1), fp16 [4,32,2048,2048] causal, fp16
[4,32,4096,4096] causal with a per-sample mask (the B=4, H=32, S=4096 score
tensor of the pnsm.cn ScaledMaskSoftmax article, sec. 1.3), bf16
[16,16,1000,1000] with a broadcast mask, and a tiny fp32 [1,2,64,64] case.

Distributions: N(mu, sigma^2) notation, so "N(0,4)" has sigma = 2. Random
values are drawn in fp32 and rounded to the working dtype by round-to-nearest-
even (torch's ``Tensor.to``); fp64 tensors are drawn in fp64. Mask positions are independent Bernoulli draws.
"""

import math

import torch

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
               "f64": torch.float64}

# Mask broadcast modes, named by the mask's own shape.
MASK_SHAPES = {
    "none": None,
    "sq_sk": lambda B, H, Sq, Sk: (Sq, Sk),
    "b_sq_sk": lambda B, H, Sq, Sk: (B, Sq, Sk),
    "b_1_sk": lambda B, H, Sq, Sk: (B, 1, Sk),
    "full": lambda B, H, Sq, Sk: (B, H, Sq, Sk),
}

CONFIGS = {
    1: dict(name="fp32 [1,2,64,64] N(0,1), no mask, forward",
            dtype="f32", shape=(1, 2, 64, 64), scale=1.0 / math.sqrt(64), causal=False,
            mask="none", x_dist=("normal", 1.0), seed=0, backward=False),
    2: dict(name="fp32 [8,32,1024,1024] N(0,4), padding mask [8,1,1024], forward",
            dtype="f32", shape=(8, 32, 1024, 1024), scale=1.0 / math.sqrt(64), causal=False,
            mask="b_1_sk", mask_kind=("padding", 256, 1024, -10000.0),
            x_dist=("normal", 2.0), seed=1, backward=False),
    3: dict(name="fp16 [4,32,2048,2048] 8*N(0,1), causal, forward+backward",
            dtype="f16", shape=(4, 32, 2048, 2048), scale=1.0 / math.sqrt(128), causal=True,
            mask="none", x_dist=("normal", 8.0), seed=2, backward=True, dy_seed=102),
    4: dict(name="fp16 [4,32,4096,4096] 8*N(0,1), mask [4,4096,4096] 10% -inf, causal, forward",
            dtype="f16", shape=(4, 32, 4096, 4096), scale=1.0 / math.sqrt(128), causal=True,
            mask="b_sq_sk", mask_kind=("bernoulli_neginf", 0.10),
            x_dist=("normal", 8.0), seed=3, backward=False),
    5: dict(name="bf16 [16,16,1000,1000] U(-30,30), mask [1000,1000] 30% -inf, forward+backward",
            dtype="bf16", shape=(16, 16, 1000, 1000), scale=0.125, causal=False,
            mask="sq_sk", mask_kind=("bernoulli_neginf", 0.30),
            x_dist=("uniform", 30.0), seed=4, backward=True, dy_seed=104),
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def draw_x(shape, dtype, dist, seed, device):
    """x drawn in fp32 (fp64 for an fp64 ``dtype``) from ``dist``, then rounded
    to ``dtype``."""
    g = _gen(seed, device)
    kind, p = dist
    draw_dt = torch.float64 if dtype == "f64" else torch.float32
    if kind == "normal":
        v = torch.randn(shape, generator=g, device=device, dtype=draw_dt)
        if p != 1.0:
            v.mul_(p)
    elif kind == "uniform":
        v = torch.rand(shape, generator=g, device=device, dtype=draw_dt)
        v.mul_(2.0 * p).sub_(p)
    else:
        raise ValueError(kind)
    return v.to(TORCH_DTYPE[dtype])


def draw_mask(shape4, mode, dtype, kind, seed, device):
    """Additive mask in its own (broadcast) shape for ``mode``.

    kind = ("padding", lo, hi, value): per batch b a length L_b drawn uniformly
      from the integers lo..hi inclusive; 0 for keys k < L_b, ``value`` after.
      Only for mode "b_1_sk".
    kind = ("bernoulli_neginf", p): -inf with probability p at each position,
      0 elsewhere; the diagonal (key == query) is never masked.
    kind = ("normal", sigma): finite N(0, sigma^2) values (a generic additive bias).
    kind = ("bool", p): a boolean mask, True (key excluded) with probability p,
      the diagonal never excluded; ``dtype`` is ignored.
    """
    if mode == "none":
        return None
    B, H, Sq, Sk = shape4
    mshape = MASK_SHAPES[mode](B, H, Sq, Sk)
    g = _gen(seed, device)
    td = TORCH_DTYPE[dtype]
    if kind[0] == "padding":
        if mode != "b_1_sk":
            raise ValueError("padding masks are per batch: mode b_1_sk")
        _, lo, hi, value = kind
        lengths = torch.randint(lo, hi + 1, (B,), generator=g, device=device)
        k = torch.arange(Sk, device=device)
        keep = k.view(1, 1, Sk) < lengths.view(B, 1, 1)
        m = torch.full(mshape, value, dtype=torch.float32, device=device)
        m.masked_fill_(keep, 0.0)
        return m.to(td)
    if kind[0] == "bernoulli_neginf":
        p = kind[1]
        u = torch.rand(mshape, generator=g, device=device, dtype=torch.float32)
        m = torch.zeros(mshape, dtype=torch.float32, device=device)
        m.masked_fill_(u < p, -math.inf)
        if mode in ("sq_sk", "b_sq_sk", "full"):
            # query axis is mshape[-2]: keep the diagonal
            n = min(Sq, Sk)
            idx = torch.arange(n, device=device)
            m[..., idx, idx] = 0.0
        return m.to(td)
    if kind[0] == "normal":
        v = torch.randn(mshape, generator=g, device=device, dtype=torch.float32)
        return v.mul_(kind[1]).to(td)
    if kind[0] == "bool":
        # True (excluded) with probability p; the diagonal is never excluded.
        p = kind[1]
        u = torch.rand(mshape, generator=g, device=device, dtype=torch.float32)
        m = u < p
        if mode in ("sq_sk", "b_sq_sk", "full"):
            n = min(Sq, Sk)
            idx = torch.arange(n, device=device)
            m[..., idx, idx] = False
        return m
    raise ValueError(kind)


def draw_lengths(B, lo, hi, seed, device):
    """Per-batch key lengths, integers drawn uniformly from lo..hi inclusive (int32)."""
    g = _gen(seed, device)
    return torch.randint(lo, hi + 1, (B,), generator=g, device=device, dtype=torch.int64).to(
        torch.int32)


def draw_dy(shape, dtype, seed, device):
    """Upstream gradient dy ~ N(0,1), rounded to ``dtype``."""
    return draw_x(shape, dtype, ("normal", 1.0), seed, device)


def make_config(cfg_id, device, shape=None, with_dy=None):
    """Tensors of workload ``cfg_id`` (optionally at a smaller ``shape``).

    Returns a dict with x, mask (its own shape, or None), mode, scale, causal,
    dtype and, when the workload has a backward (or ``with_dy``), dy.
    """
    c = CONFIGS[cfg_id]
    shp = tuple(shape) if shape is not None else c["shape"]
    x = draw_x(shp, c["dtype"], c["x_dist"], c["seed"], device)
    mask = None
    if c["mask"] != "none":
        mask = draw_mask(shp, c["mask"], c["dtype"], c["mask_kind"], c["seed"] + 1000, device)
    out = dict(x=x, mask=mask, mode=c["mask"], scale=c["scale"], causal=c["causal"],
               dtype=c["dtype"], shape=shp)
    want_dy = c["backward"] if with_dy is None else with_dy
    if want_dy:
        out["dy"] = draw_dy(shp, c["dtype"], c.get("dy_seed", c["seed"] + 100), device)
    return out
