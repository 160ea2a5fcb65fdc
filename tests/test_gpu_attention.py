"""Fused attention forward (C ABI sms_attention_forward) against the float64
oracle (oracle.attention), element by element, with the tolerance derived in
tests/tolerance.py; masks, causal rules, grouped heads, tails, strides,
errors."""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from attention_softmax_amd import SmsError, sms_attention_forward
from attention_softmax_amd.workloads import TORCH_DTYPE, draw_lengths, draw_mask, draw_x
from tests.parity import DTYPE_OF, mask_4d, to_np
from tests.tolerance import compare_attention

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_mask(shape, mode, kind, dtype, seed):
    if kind == "none":
        return None
    if kind == "lengths":
        return draw_lengths(shape[0], 0, shape[3] + 2, seed, DEV)
    if kind == "bool":
        return draw_mask(shape, mode, dtype, ("bool", 0.3), seed, DEV)
    if kind == "neginf":
        return draw_mask(shape, mode, dtype, ("bernoulli_neginf", 0.25), seed, DEV)
    return draw_mask(shape, mode, dtype, ("normal", 2.0), seed, DEV)


def check(q, k, v, mask, mode, kind, scale, causal, what):
    dt = DTYPE_OF[q.dtype]
    o, lse = sms_attention_forward(q, k, v, mask, scale, causal, return_lse=True)
    torch.cuda.synchronize()
    okind = {"bool": "bool", "lengths": "lengths"}.get(kind, "additive")
    ref, ref_lse = oracle.attention.forward(
        to_np(q), to_np(k), to_np(v), dt,
        mask=None if kind in ("none", "lengths") else mask_4d(mask, mode), scale=scale,
        is_causal=causal, mask_kind=okind,
        key_lengths=to_np(mask) if kind == "lengths" else None)
    B, H, Sq, D = q.shape
    Hk = k.shape[1]
    vabs = np.abs(oracle.decode(to_np(v), dt)).max(axis=(2, 3))  # [B, Hk]
    vmax = np.repeat(vabs, H // Hk, axis=1)[:, :, None, None]
    return compare_attention(oracle.decode(to_np(o), dt), ref, vmax, dt, what,
                             to_np(lse), ref_lse)


SHAPES = [(1, 1), (37, 63), (128, 64), (129, 65), (200, 300), (64, 1000)]
MASKS = [("none", "none"), ("sq_sk", "additive"), ("b_sq_sk", "neginf"), ("b_1_sk", "neginf"),
         ("full", "additive"), ("b_sq_sk", "bool"), ("key_lengths", "lengths")]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Sk", SHAPES)
def test_attention_sweep(dtype, D, Sq, Sk):
    """Every mask shape and kind and causal rule on tails of both tile sizes
    (128 queries, 64 keys), with grouped heads (H = 4 over Hk = 2)."""
    say(f"attention dtype={dtype} D={D} Sq={Sq} Sk={Sk}")
    B, H, Hk = 2, 4, 2
    worst = 0.0
    for mode, kind in MASKS:
        for causal in (False, True, "bottom_right"):
            seed = zlib.crc32(f"a/{dtype}/{D}/{Sq}/{Sk}/{mode}/{kind}/{causal}".encode()) % 10000
            q = draw_x((B, H, Sq, D), dtype, ("normal", 1.0), seed, DEV)
            k = draw_x((B, Hk, Sk, D), dtype, ("normal", 1.0), seed + 1, DEV)
            v = draw_x((B, Hk, Sk, D), dtype, ("normal", 1.0), seed + 2, DEV)
            mask = make_mask((B, H, Sq, Sk), mode, kind, dtype, seed + 3)
            st = check(q, k, v, mask, mode, kind, D ** -0.5, causal,
                       f"{dtype} D={D} {Sq}x{Sk} {mode}/{kind} causal={causal}")
            worst = max(worst, st["max_err_over_tol"])
    say(f"  worst error / tolerance {worst:.3f}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_strided_and_large_scores(dtype):
    """Q, K, V as [B, S, H, D] storage viewed as [B, H, S, D] (strided heads),
    O written into a strided view, and scores of a few units (scale 1)."""
    say(f"attention strided dtype={dtype}")
    B, H, Sq, Sk, D = 2, 3, 150, 170, 64
    td = TORCH_DTYPE[dtype]
    q = draw_x((B, Sq, H, D), dtype, ("normal", 1.0), 1, DEV).permute(0, 2, 1, 3)
    k = draw_x((B, Sk, H, D), dtype, ("normal", 1.0), 2, DEV).permute(0, 2, 1, 3)
    v = draw_x((B, Sk, H, D), dtype, ("normal", 1.0), 3, DEV).permute(0, 2, 1, 3)
    obuf = torch.full((B, Sq, H, D), 5.0, dtype=td, device=DEV)
    o = obuf.permute(0, 2, 1, 3)
    sms_attention_forward(q, k, v, None, 0.25, True, o=o)
    torch.cuda.synchronize()
    ref, _ = oracle.attention.forward(to_np(q.contiguous()), to_np(k.contiguous()),
                                      to_np(v.contiguous()), dtype, scale=0.25, is_causal=True)
    vmax = np.abs(oracle.decode(to_np(v.contiguous()), dtype)).max(axis=(2, 3))[:, :, None, None]
    compare_attention(oracle.decode(to_np(o.contiguous()), dtype), ref, vmax, dtype, "strided")
    check(q.contiguous(), k.contiguous(), v.contiguous(), None, "none", "none", 1.0, False,
          "scale 1")


def test_attention_large_head_sampled():
    """fp16 [1, 2, 2048, 2048], D = 128, causal: every row of two heads."""
    say("attention 2048 x 2048")
    q = draw_x((1, 2, 2048, 128), "f16", ("normal", 1.0), 7, DEV)
    k = draw_x((1, 2, 2048, 128), "f16", ("normal", 1.0), 8, DEV)
    v = draw_x((1, 2, 2048, 128), "f16", ("normal", 1.0), 9, DEV)
    st = check(q, k, v, None, "none", "none", 128 ** -0.5, True, "2048 causal")
    say(f"  {st}")


def test_attention_errors():
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16, device=DEV)
    with pytest.raises(SmsError, match="SHAPE"):  # head dim 96
        z = torch.zeros(1, 1, 4, 96, dtype=torch.float16, device=DEV)
        sms_attention_forward(z, z, z)
    with pytest.raises(TypeError):
        f = torch.zeros(1, 1, 4, 64, device=DEV)
        sms_attention_forward(f, f, f)
    with pytest.raises(SmsError, match="SHAPE"):  # Hk does not divide H
        k3 = torch.zeros(1, 2, 4, 64, dtype=torch.float16, device=DEV)
        sms_attention_forward(torch.zeros(1, 3, 4, 64, dtype=torch.float16, device=DEV), k3, k3)
    with pytest.raises(SmsError, match="ALIGN"):  # rows not on 16-byte lines
        big = torch.zeros(1, 1, 4, 72, dtype=torch.float16, device=DEV)[..., 4:68]
        sms_attention_forward(big, q, q)
    empty = torch.zeros(1, 1, 0, 64, dtype=torch.float16, device=DEV)
    sms_attention_forward(empty, q, q)  # no query: a no-op
