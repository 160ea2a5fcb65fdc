"""CPU: the fused attention forward's parity checks are tight enough to catch
a wrong rounding of the probabilities.

The GPU kernel's arithmetic is simulated in float64 on the oracle's exact
probabilities: p~ = P / max P per row (the largest at 1), p~ rounded to the
I/O dtype for the P V product, the sum of the unrounded p~, O rounded to the
I/O dtype (round to nearest even) at the end. The correct simulation must pass
``compare_attention`` with room to spare; the same simulation with p~ rounded
to bf16 on the fp16 path, or truncated instead of rounded, must fail it.
Workload: one query head of the attention bench's recipe (Q, K, V ~ N(0, 1),
scale 1/sqrt(D), causal), at a length the CPU finishes in seconds."""

import numpy as np
import pytest

import oracle
from tests.tolerance import attention_forward_bounds, compare_attention

_PREC = {"f16": (11, -14), "bf16": (8, -126)}


def _round_bf16(x):
    """float64 -> nearest bf16 value (ties to even), through float32."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _round_nearest(x, dtype):
    if dtype == "f16":
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)
    return _round_bf16(x)


def _truncate(x, dtype):
    """float64 -> the dtype's value next toward zero (no rounding)."""
    p, emin = _PREC[dtype]
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    q = np.exp2(np.maximum(e, emin) - (p - 1))
    return np.sign(x) * np.floor(a / q) * q


def _inputs(dtype, S, D, seed):
    rng = np.random.default_rng(seed)
    t = np.float16 if dtype == "f16" else np.float32
    qkv = [rng.standard_normal((1, 1, S, D)).astype(t) for _ in range(3)]
    if dtype == "bf16":
        qkv = [(a.view(np.uint32) >> 16).astype(np.uint16) for a in qkv]
    return qkv


def _simulate(P, vd, dtype, round_p):
    pmax = P.max(axis=-1, keepdims=True)
    pt = P / np.where(pmax > 0, pmax, 1.0)
    L = pt.sum(axis=-1, keepdims=True)
    acc = round_p(pt) @ vd
    return _round_nearest(acc / np.where(L > 0, L, 1.0), dtype)


def _case(dtype, S, D, causal, seed):
    q, k, v = _inputs(dtype, S, D, seed)
    sc = float(np.float32(D ** -0.5))
    P, lse = oracle.attention.probabilities(q, k, dtype, scale=sc, is_causal=causal)
    o_ref, _ = oracle.attention.forward(q, k, v, dtype, scale=sc, is_causal=causal)
    qd, kd, vd = (oracle.decode(a, dtype) for a in (q, k, v))
    bounds = attention_forward_bounds(P, lse, qd, kd, vd, o_ref, sc, dtype)
    return P, vd, o_ref, bounds


CASES = [("f16", 1024, 128, True, 1), ("f16", 512, 64, False, 2), ("bf16", 1024, 128, True, 3)]


@pytest.mark.parametrize("dtype,S,D,causal,seed", CASES)
def test_correct_rounding_passes_with_margin(dtype, S, D, causal, seed):
    P, vd, o_ref, bounds = _case(dtype, S, D, causal, seed)
    got = _simulate(P, vd, dtype, lambda x: _round_nearest(x, dtype))
    st = compare_attention(got, o_ref, bounds, dtype, "round to nearest")
    assert st["max_err_over_tol"] < 0.5, st
    assert st["fro_over_bound"] < 0.5, st
    assert st["bias_over_bound"] < 0.5, st


@pytest.mark.parametrize("dtype,S,D,causal,seed", [c for c in CASES if c[0] == "f16"])
def test_bf16_probabilities_on_the_fp16_path_fail(dtype, S, D, causal, seed):
    P, vd, o_ref, bounds = _case(dtype, S, D, causal, seed)
    got = _simulate(P, vd, dtype, _round_bf16)
    with pytest.raises(AssertionError):
        compare_attention(got, o_ref, bounds, dtype, "P rounded to bf16")


@pytest.mark.parametrize("dtype,S,D,causal,seed", CASES)
def test_truncated_probabilities_fail(dtype, S, D, causal, seed):
    P, vd, o_ref, bounds = _case(dtype, S, D, causal, seed)
    got = _simulate(P, vd, dtype, lambda x: _truncate(x, dtype))
    with pytest.raises(AssertionError):
        compare_attention(got, o_ref, bounds, dtype, "P truncated")


def test_bounds_of_a_one_key_row():
    """One visible key: O is that key's value row, and the elementwise bound is
    the probability's unit roundoff plus 2 ulp of O, up to the fp32 terms."""
    from tests.tolerance import ulp
    q, k, v = _inputs("f16", 4, 64, 9)
    P, lse = oracle.attention.probabilities(q, k, "f16", scale=0.125, is_causal=True)
    o_ref, _ = oracle.attention.forward(q, k, v, "f16", scale=0.125, is_causal=True)
    b = attention_forward_bounds(P, lse, *(oracle.decode(a, "f16") for a in (q, k, v)), o_ref,
                                 0.125, "f16")
    v0 = oracle.decode(v, "f16")[0, 0, 0]
    assert (o_ref[0, 0, 0] == v0).all()     # query 0 sees key 0 alone
    want = 2 * 2.0 ** -11 * np.abs(v0) + 2 * ulp(v0, "f16")
    assert (b["tol"][0, 0, 0] >= want).all()
    assert (b["tol"][0, 0, 0] <= want * 1.1).all()   # the fp32 terms: a few per cent
