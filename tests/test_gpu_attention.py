"""Fused attention forward and backward (C ABI sms_attention_forward /
sms_attention_backward) against the float64 oracle (oracle.attention), element
by element, with the tolerances derived in tests/tolerance.py; masks, causal
rules, grouped heads, tails, strides, empty sizes, autograd, errors."""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from attention_softmax_amd import (SmsError, attention, sms_attention_backward,
                                   sms_attention_forward, sms_attention_workspace_bytes)
from attention_softmax_amd.workloads import TORCH_DTYPE, draw_lengths, draw_mask, draw_x
from tests.parity import DTYPE_OF, mask_4d, to_np
from tests.tolerance import (attention_forward_bounds, attention_grad_tolerances,
                             compare_attention, compare_grads)

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


def fwd_bounds(qn, kn, vn, dt, o_ref, lse_ref, scale, **kw):
    """The forward's error bounds (tests/tolerance.py) from the oracle's
    probabilities of these typed inputs."""
    P, _ = oracle.attention.probabilities(qn, kn, dt, scale=scale, **kw)
    return attention_forward_bounds(P, lse_ref, *(oracle.decode(a, dt) for a in (qn, kn, vn)),
                                    o_ref, float(np.float32(scale)), dt)


def check(q, k, v, mask, mode, kind, scale, causal, what):
    dt = DTYPE_OF[q.dtype]
    o, lse = sms_attention_forward(q, k, v, mask, scale, causal, return_lse=True)
    torch.cuda.synchronize()
    okind = {"bool": "bool", "lengths": "lengths"}.get(kind, "additive")
    kw = dict(mask=None if kind in ("none", "lengths") else mask_4d(mask, mode),
              is_causal=causal, mask_kind=okind,
              key_lengths=to_np(mask) if kind == "lengths" else None)
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    ref, ref_lse = oracle.attention.forward(qn, kn, vn, dt, scale=scale, **kw)
    bounds = fwd_bounds(qn, kn, vn, dt, ref, ref_lse, scale, **kw)
    return compare_attention(oracle.decode(to_np(o), dt), ref, bounds, dt, what,
                             to_np(lse), ref_lse)


# (300, 100): bottom-right causal leaves the first 128-query tile without any key.
# (200, 136): additive masks as LDS tiles (Sk % 8 == 0) over two query tiles and
# a last key tile of 8 keys. (200, 144): boolean masks as LDS tiles too
# (Sk % 16 == 0), a last key tile of 16 keys.
SHAPES = [(1, 1), (37, 63), (128, 64), (129, 65), (200, 300), (64, 1000), (300, 100), (200, 136),
          (200, 144)]
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
    qn, kn, vn = (to_np(t.contiguous()) for t in (q, k, v))
    ref, ref_lse = oracle.attention.forward(qn, kn, vn, dtype, scale=0.25, is_causal=True)
    bounds = fwd_bounds(qn, kn, vn, dtype, ref, ref_lse, 0.25, is_causal=True)
    compare_attention(oracle.decode(to_np(o.contiguous()), dtype), ref, bounds, dtype, "strided")
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
    with pytest.raises(SmsError, match="STRIDE"):  # key rows more than 2^24 elements apart
        rs = (1 << 24) + 8
        kv = torch.zeros(rs + 64, dtype=torch.float16, device=DEV).as_strided(
            (1, 1, 2, 64), (2 * rs, 2 * rs, rs, 1))
        sms_attention_forward(torch.zeros(1, 1, 2, 64, dtype=torch.float16, device=DEV), kv, kv)
    empty = torch.zeros(1, 1, 0, 64, dtype=torch.float16, device=DEV)
    sms_attention_forward(empty, q, q)  # no query: a no-op


# ------------------------------------------------------------------ backward

def check_bwd(q, k, v, mask, mode, kind, scale, causal, what, seed, do=None, chain=False):
    """The GPU backward against the oracle's gradients; returns the worst
    elementwise error / tolerance over dQ, dK, dV.

    The backward is given the oracle's O rounded to the I/O dtype and its LSE
    rounded to fp32 (so the tolerance knows their deviation exactly), or with
    ``chain`` the GPU forward's O and LSE (tolerance from the forward's bound)."""
    dt = DTYPE_OF[q.dtype]
    okind = {"bool": "bool", "lengths": "lengths"}.get(kind, "additive")
    kw = dict(mask=None if kind in ("none", "lengths") else mask_4d(mask, mode),
              scale=scale, is_causal=causal, mask_kind=okind,
              key_lengths=to_np(mask) if kind == "lengths" else None)
    if do is None:
        do = draw_x(tuple(q.shape), dt, ("normal", 1.0), seed, DEV)
    qn, kn, vn, don = (to_np(t.contiguous()) for t in (q, k, v, do))
    refs = oracle.attention.backward(qn, kn, vn, don, dt, **kw)
    P, ref_lse = oracle.attention.probabilities(qn, kn, dt, **kw)
    o_ref, _ = oracle.attention.forward(qn, kn, vn, dt, **kw)
    if chain:
        o, lse = sms_attention_forward(q, k, v, mask, scale, causal, return_lse=True)
        o_in = lse_in = None
    else:
        o = torch.from_numpy(o_ref).to(DEV).to(q.dtype)
        lse = torch.from_numpy(ref_lse).to(DEV).to(torch.float32)
        o_in = oracle.decode(to_np(o), dt)
        lse_in = to_np(lse).astype(np.float64)
    dq, dk, dv = sms_attention_backward(q, k, v, o, lse, do, mask, scale, causal)
    torch.cuda.synchronize()
    qd, kd, vd, dod = (oracle.decode(a, dt) for a in (qn, kn, vn, don))
    B, H = q.shape[:2]
    group = H // k.shape[1]
    vrep = np.repeat(vd, group, axis=1)
    dP = dod @ np.swapaxes(vrep, 2, 3)
    vmax = np.abs(vrep).max(axis=(2, 3)) if vrep.size else np.zeros((B, H))
    tols, rms = attention_grad_tolerances(P, dP, qd, kd, dod, vmax, ref_lse,
                                          float(np.float32(scale)), dt, refs, o_in, o_ref, lse_in)
    worst = 0.0
    for name, got, ref, tol, rm in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs, tols, rms):
        worst = max(worst, compare_grads(oracle.decode(to_np(got.contiguous()), dt), ref, tol,
                                         f"{what} {name}", rm))
    return worst


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Sq,Sk", SHAPES)
def test_attention_backward_sweep(dtype, D, Sq, Sk):
    """dQ, dK, dV for every mask shape and kind and causal rule on tails of the
    tiles (128 queries of the dQ kernel, 128 keys of the dK/dV kernel, 64-key
    and 32-query inner tiles), grouped heads (H = 4 over Hk = 2)."""
    say(f"attention backward dtype={dtype} D={D} Sq={Sq} Sk={Sk}")
    B, H, Hk = 2, 4, 2
    worst = 0.0
    for mode, kind in MASKS:
        for causal in (False, True, "bottom_right"):
            seed = zlib.crc32(f"ab/{dtype}/{D}/{Sq}/{Sk}/{mode}/{kind}/{causal}".encode()) % 10000
            q = draw_x((B, H, Sq, D), dtype, ("normal", 1.0), seed, DEV)
            k = draw_x((B, Hk, Sk, D), dtype, ("normal", 1.0), seed + 1, DEV)
            v = draw_x((B, Hk, Sk, D), dtype, ("normal", 1.0), seed + 2, DEV)
            mask = make_mask((B, H, Sq, Sk), mode, kind, dtype, seed + 3)
            w = check_bwd(q, k, v, mask, mode, kind, D ** -0.5, causal,
                          f"bwd {dtype} D={D} {Sq}x{Sk} {mode}/{kind} causal={causal}", seed + 4)
            worst = max(worst, w)
    say(f"  worst error / tolerance {worst:.3f}")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_attention_backward_strided_mha_and_scale(dtype):
    """Q, K, V, dO as [B, S, H, D] storage viewed as [B, H, S, D], gradients
    written into strided views; plain multi-head (Hk = H) and 8 query heads on
    one key/value head; scale 1."""
    say(f"attention backward strided dtype={dtype}")
    B, H, Sq, Sk, D = 2, 3, 150, 170, 64
    td = TORCH_DTYPE[dtype]
    q = draw_x((B, Sq, H, D), dtype, ("normal", 1.0), 11, DEV).permute(0, 2, 1, 3)
    k = draw_x((B, Sk, H, D), dtype, ("normal", 1.0), 12, DEV).permute(0, 2, 1, 3)
    v = draw_x((B, Sk, H, D), dtype, ("normal", 1.0), 13, DEV).permute(0, 2, 1, 3)
    do = draw_x((B, Sq, H, D), dtype, ("normal", 1.0), 14, DEV).permute(0, 2, 1, 3)
    o, lse = sms_attention_forward(q, k, v, None, 0.25, True, return_lse=True)
    bufs = [torch.full((B, S, H, D), 7.0, dtype=td, device=DEV) for S in (Sq, Sk, Sk)]
    dq, dk, dv = (t.permute(0, 2, 1, 3) for t in bufs)
    sms_attention_backward(q, k, v, o, lse, do, None, 0.25, True, dq=dq, dk=dk, dv=dv)
    rq, rk, rv = sms_attention_backward(q.contiguous(), k.contiguous(), v.contiguous(),
                                        o.contiguous(), lse, do.contiguous(), None, 0.25, True)
    torch.cuda.synchronize()
    for a, b_, n in ((dq, rq, "dQ"), (dk, rk, "dK"), (dv, rv, "dV")):
        assert torch.equal(a.contiguous(), b_), f"strided {n} differs from contiguous"
    check_bwd(q.contiguous(), k.contiguous(), v.contiguous(), None, "none", "none", 0.25, True,
              "strided", 0, do=do.contiguous())
    q8 = draw_x((1, 8, 97, 128), dtype, ("normal", 1.0), 15, DEV)
    k1 = draw_x((1, 1, 300, 128), dtype, ("normal", 1.0), 16, DEV)
    v1 = draw_x((1, 1, 300, 128), dtype, ("normal", 1.0), 17, DEV)
    check_bwd(q8, k1, v1, None, "none", "none", 1.0, False, "8 heads on 1, scale 1", 18)


@pytest.mark.parametrize("kind,Sk", [("neginf", 1024), ("bool", 1024), ("none", 1000), ("lengths", 1000)])
def test_attention_backward_large_grid(kind, Sk):
    """D = 128 on a grid of 512 dK/dV workgroups (two per CU), where dK and dV
    run at two wavefronts per SIMD: as two launches with a per-score [B,Sq,Sk]
    mask (LDS tiles), as one launch with the V copy in LDS without one
    (smaller grids, as in the sweep, take one launch at one wavefront per
    SIMD). B = 2, 64 query heads over 32 key/value heads, 64 queries, 1024 or
    1000 keys (a last key block of 104), not causal and bottom-right causal."""
    say(f"attention backward large grid mask={kind} Sk={Sk}")
    B, H, Hk, Sq, D = 2, 64, 32, 64, 128
    worst = 0.0
    for causal in (False, "bottom_right"):
        seed = zlib.crc32(f"large/{kind}/{Sk}/{causal}".encode()) % 10000
        q = draw_x((B, H, Sq, D), "f16", ("normal", 1.0), seed, DEV)
        k = draw_x((B, Hk, Sk, D), "f16", ("normal", 1.0), seed + 1, DEV)
        v = draw_x((B, Hk, Sk, D), "f16", ("normal", 1.0), seed + 2, DEV)
        mode = {"none": "none", "lengths": "key_lengths"}.get(kind, "b_sq_sk")
        mask = make_mask((B, H, Sq, Sk), mode, kind, "f16", seed + 3)
        w = check_bwd(q, k, v, mask, mode, kind, D ** -0.5, causal,
                      f"large grid {kind} Sk={Sk} causal={causal}", seed + 4)
        worst = max(worst, w)
    say(f"  worst error / tolerance {worst:.3f}")


def test_attention_backward_long_causal():
    """fp16 [1, 2, 1024, 1024], D = 128, causal, every gradient element; once
    from the oracle's O and LSE, once from the GPU forward's."""
    say("attention backward 1024 x 1024")
    q = draw_x((1, 2, 1024, 128), "f16", ("normal", 1.0), 21, DEV)
    k = draw_x((1, 2, 1024, 128), "f16", ("normal", 1.0), 22, DEV)
    v = draw_x((1, 2, 1024, 128), "f16", ("normal", 1.0), 23, DEV)
    w = check_bwd(q, k, v, None, "none", "none", 128 ** -0.5, True, "1024 causal", 24)
    w2 = check_bwd(q, k, v, None, "none", "none", 128 ** -0.5, True, "1024 causal chain", 24,
                   chain=True)
    say(f"  worst error / tolerance {w:.3f}, from the GPU forward {w2:.3f}")


def test_attention_bench_workload_sampled():
    """The attention bench's workload at full size, in the launches the bench
    times: fp16 Q, K, V, dO [4, 32, 4096, 128] ~ N(0, 1) (the bench's seeds),
    causal, scale 1/sqrt(128); forward and backward over all 128 heads, then
    two (batch, head) pairs checked element by element against the oracle:
    O, LSE, dQ, dK and dV of those heads, the backward from the GPU
    forward's O and LSE."""
    B, H, S, D = 4, 32, 4096, 128
    sc = D ** -0.5
    say("attention bench workload fp16 [4,32,4096,128] causal")
    q, k, v, do = (draw_x((B, H, S, D), "f16", ("normal", 1.0), 11 + i, DEV) for i in range(4))
    o, lse = sms_attention_forward(q, k, v, None, sc, True, return_lse=True)
    dq, dk, dv = sms_attention_backward(q, k, v, o, lse, do, None, sc, True)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 31)):
        what = f"bench workload (b={b}, h={h})"
        say(f"  {what}")

        def head(t):
            return to_np(t[b:b + 1, h:h + 1].contiguous())

        qn, kn, vn, don = head(q), head(k), head(v), head(do)
        o_ref, lse_ref = oracle.attention.forward(qn, kn, vn, "f16", scale=sc, is_causal=True)
        vd = oracle.decode(vn, "f16")
        P, ref_lse = oracle.attention.probabilities(qn, kn, "f16", scale=sc, is_causal=True)
        qd, kd, dod = (oracle.decode(a, "f16") for a in (qn, kn, don))
        bounds = attention_forward_bounds(P, ref_lse, qd, kd, vd, o_ref, float(np.float32(sc)),
                                          "f16")
        st = compare_attention(oracle.decode(head(o), "f16"), o_ref, bounds, "f16", what + " O",
                               head(lse), lse_ref)
        say(f"    O: {st}")
        refs = oracle.attention.backward(qn, kn, vn, don, "f16", scale=sc, is_causal=True)
        dP = dod @ np.swapaxes(vd, 2, 3)
        tols, rms = attention_grad_tolerances(P, dP, qd, kd, dod, np.abs(vd).max(axis=(2, 3)),
                                              ref_lse, float(np.float32(sc)), "f16", refs, None,
                                              o_ref, None)
        for name, got, ref, tol, rm in zip(("dQ", "dK", "dV"), (dq, dk, dv), refs, tols, rms):
            compare_grads(oracle.decode(head(got), "f16"), ref, tol, f"{what} {name}", rm)


def test_attention_backward_empty_sides():
    """No key: dQ = 0 and nothing else; no query: dK = dV = 0."""
    say("attention backward empty sides")
    q = draw_x((1, 2, 40, 64), "bf16", ("normal", 1.0), 31, DEV)
    k0 = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    o, lse = sms_attention_forward(q, k0, k0, None, 0.125, False, return_lse=True)
    assert (o == 0).all() and (lse == -float("inf")).all()
    dq = torch.full_like(q, 3.0)
    sms_attention_backward(q, k0, k0, o, lse, q, None, 0.125, False, dq=dq)
    torch.cuda.synchronize()
    assert (dq == 0).all()
    k = draw_x((1, 2, 70, 64), "bf16", ("normal", 1.0), 32, DEV)
    q0 = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device=DEV)
    lse0 = torch.empty((1, 2, 0), dtype=torch.float32, device=DEV)
    dk, dv = torch.full_like(k, 3.0), torch.full_like(k, 3.0)
    sms_attention_backward(q0, k, k, q0, lse0, q0, None, 0.125, True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()


def test_attention_autograd():
    """attention() under autograd: the gradients are the backward entry
    point's, bit for bit, and agree with the oracle."""
    say("attention autograd")
    q = draw_x((2, 4, 77, 64), "f16", ("normal", 1.0), 41, DEV).requires_grad_()
    k = draw_x((2, 2, 90, 64), "f16", ("normal", 1.0), 42, DEV).requires_grad_()
    v = draw_x((2, 2, 90, 64), "f16", ("normal", 1.0), 43, DEV).requires_grad_()
    do = draw_x((2, 4, 77, 64), "f16", ("normal", 1.0), 44, DEV)
    lengths = torch.tensor([50, 90], dtype=torch.int64, device=DEV)
    o = attention(q, k, v, lengths, None, True)
    o.backward(do)
    o2, lse = sms_attention_forward(q.detach(), k.detach(), v.detach(),
                                    lengths.to(torch.int32), 64 ** -0.5, True, return_lse=True)
    gq, gk, gv = sms_attention_backward(q.detach(), k.detach(), v.detach(), o2, lse, do,
                                        lengths.to(torch.int32), 64 ** -0.5, True)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for a, b_ in ((q.grad, gq), (k.grad, gk), (v.grad, gv)):
        assert torch.equal(a, b_)
    check_bwd(q.detach(), k.detach(), v.detach(), lengths.to(torch.int32), "key_lengths",
              "lengths", 64 ** -0.5, True, "autograd case", 0, do=do, chain=True)


@pytest.mark.parametrize("dtype,D,mode,kind,causal", [
    ("f16", 128, "b_sq_sk", "additive", True),
    ("bf16", 64, "none", "none", False),
])
def test_attention_hip_graph_capture_and_replay(dtype, D, mode, kind, causal):
    """Forward + backward captured once into a HIP graph and replayed on new
    inputs copied into the static buffers, with eager work and synchronisation
    between replays: every replay equals the eager calls bit for bit, and the
    forward agrees with the oracle (the operator has no host-side control flow
    that would keep it out of a graph: pnsm.cn ScaledMaskSoftmax article,
    sec. 4.4)."""
    say(f"attention graph {dtype} D={D} mask={mode}/{kind} causal={causal}")
    B, H, Hk, Sq, Sk = 1, 4, 2, 200, 300
    scale = D ** -0.5
    shp_q, shp_k = (B, H, Sq, D), (B, Hk, Sk, D)

    def draw(seed):
        return (draw_x(shp_q, dtype, ("normal", 1.0), seed, DEV),
                draw_x(shp_k, dtype, ("normal", 1.0), seed + 1, DEV),
                draw_x(shp_k, dtype, ("normal", 1.0), seed + 2, DEV),
                draw_x(shp_q, dtype, ("normal", 1.0), seed + 3, DEV))

    q, k, v, do = draw(60)
    mask = make_mask((B, H, Sq, Sk), mode, kind, dtype, 64)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(sms_attention_workspace_bytes(B, H, Sq), dtype=torch.uint8, device=DEV)

    def run():
        sms_attention_forward(q, k, v, mask, scale, causal, o=o, lse=lse)
        sms_attention_backward(q, k, v, o, lse, do, mask, scale, causal, dq=dq, dk=dk, dv=dv,
                               workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the default stream
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        qn, kn, vn, don = draw(100 + 10 * rep)
        for dst, src in ((q, qn), (k, kn), (v, vn), (do, don)):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        oe, lse_e = sms_attention_forward(qn, kn, vn, mask, scale, causal, return_lse=True)
        gq, gk, gv = sms_attention_backward(qn, kn, vn, oe, lse_e, don, mask, scale, causal)
        torch.cuda.synchronize()
        for name, a, b_ in (("O", o, oe), ("LSE", lse, lse_e), ("dQ", dq, gq), ("dK", dk, gk),
                            ("dV", dv, gv)):
            assert torch.equal(a, b_), f"replay {rep}: {name} differs from the eager call"
        if rep == 0:
            check(qn, kn, vn, mask, mode, kind, scale, causal, f"graph replay {rep}")
    del g


def test_attention_backward_errors():
    q = torch.zeros(1, 1, 4, 64, dtype=torch.float16, device=DEV)
    lse = torch.zeros(1, 1, 4, dtype=torch.float32, device=DEV)
    assert sms_attention_workspace_bytes(2, 3, 5) == 4 * 2 * 3 * 5
    with pytest.raises(SmsError, match="WORKSPACE"):
        ws = torch.empty(8, dtype=torch.uint8, device=DEV)
        sms_attention_backward(q, q, q, q, lse, q, workspace=ws)
    with pytest.raises(SmsError, match="SHAPE"):  # head dim 96
        z = torch.zeros(1, 1, 4, 96, dtype=torch.float16, device=DEV)
        sms_attention_backward(z, z, z, z, lse, z)
    with pytest.raises(ValueError):  # lse of the wrong shape
        sms_attention_backward(q, q, q, q, lse[..., :3], q)
