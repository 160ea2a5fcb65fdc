"""The float64 oracle against its pins (CPU only), and planted mistakes.

The second half plants plausible mistakes in a copy of the oracle (on the CPU,
through monkeypatch) and requires that at least one pin fails for each: that
is the evidence that the pins constrain every step of the oracle.
"""

import math

import numpy as np
import pytest

import oracle.softmax as S
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


# ----------------------------------------------------------- planted mistakes

_orig_fwd = S._forward_one_row
_orig_bwd = S._backward_one_row
_orig_decode = S.decode
_orig_mask_row = S._mask_row
_orig_row_index = S.row_index


def _fwd_generic(xrow, mrow, sc, causal, q, excluded=None, offset=0, *, use_scale=True,
                 causal_ge=False, mask_scaled=False, shift=True, full_mask="zeros",
                 causal_first_only=False):
    n = xrow.shape[0]
    s = xrow * (sc if use_scale else 1.0)
    if mrow is not None:
        s = s + (mrow * sc if mask_scaled else mrow)
    if excluded is not None:
        s = np.where(excluded, -math.inf, s)
    if causal:
        s = s.copy()
        k = np.arange(n)
        s[(k >= q + offset) if causal_ge else (k > q + offset)] = -math.inf
        if causal_first_only:
            s[k > q + offset + 1] = -math.inf
    m = s.max() if n else -math.inf
    if m == -math.inf:
        if full_mask == "zeros":
            return np.zeros(n)
        if full_mask == "uniform":
            return np.full(n, 1.0 / n)
        with np.errstate(invalid="ignore"):
            e = np.exp(s - m)
            return e / e.sum()
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(s - m) if shift else np.exp(s)
        return e / e.sum()


def _bwd_generic(y, dy, sc, *, use_scale=True, sign=1.0, use_dot=True, dot_sq=False):
    dot = float(np.dot(dy, y)) if use_dot else 0.0
    if dot_sq:
        dot = float(np.dot(y, y))
    return (sc if use_scale else 1.0) * y * (dy - sign * dot)


FWD_MUTANTS = {
    "scale dropped": dict(use_scale=False),
    "causal masks the diagonal too": dict(causal_ge=True),
    "causal mask one key late": dict(causal_first_only=False, causal_ge=False) | {"_late": True},
    "mask multiplied by scale": dict(mask_scaled=True),
    "no max subtraction": dict(shift=False),
    "fully masked row uniform": dict(full_mask="uniform"),
    "fully masked row NaN": dict(full_mask="nan"),
}

BWD_MUTANTS = {
    "backward scale dropped": dict(use_scale=False),
    "backward sign of dot flipped": dict(sign=-1.0),
    "backward dot dropped": dict(use_dot=False),
    "backward uses sum y^2": dict(dot_sq=True),
}


def _late_causal(xrow, mrow, sc, causal, q, excluded=None, offset=0):
    # keys up to q+1 kept (off by one in the other direction)
    return _orig_fwd(xrow, mrow, sc, causal, q + 1 if causal else q, excluded, offset)


def _run_all_pins():
    failures = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except AssertionError as e:
            failures.append((pin.__name__, str(e)[:80]))
        except (FloatingPointError, ValueError, IndexError) as e:
            failures.append((pin.__name__, repr(e)[:80]))
    return failures


@pytest.mark.parametrize("name", sorted(FWD_MUTANTS))
def test_planted_forward_mistake_is_caught(name, monkeypatch):
    kw = dict(FWD_MUTANTS[name])
    if kw.pop("_late", False):
        monkeypatch.setattr(S, "_forward_one_row", _late_causal)
    else:
        monkeypatch.setattr(S, "_forward_one_row",
                            lambda xr, mr, sc, c, q, ex=None, off=0:
                            _fwd_generic(xr, mr, sc, c, q, ex, off, **kw))
    assert _run_all_pins(), f"planted mistake '{name}' passed every pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_planted_backward_mistake_is_caught(name, monkeypatch):
    kw = BWD_MUTANTS[name]
    monkeypatch.setattr(S, "_backward_one_row", lambda y, dy, sc: _bwd_generic(y, dy, sc, **kw))
    assert _run_all_pins(), f"planted mistake '{name}' passed every pin"


def test_planted_indexing_mistakes_are_caught(monkeypatch):
    # mask broadcast taken along heads instead of batches
    def mask_row_h(maskd, b, h, q):
        return _orig_mask_row(maskd, h % maskd.shape[0], b % max(maskd.shape[1], 1), q)
    monkeypatch.setattr(S, "_mask_row", mask_row_h)
    assert _run_all_pins()
    monkeypatch.setattr(S, "_mask_row", _orig_mask_row)

    # row order (b, q, h) instead of (b, h, q)
    def row_index_swapped(shape, r):
        B, H, Sq, _ = shape
        return r // (Sq * H), r % H, (r // H) % Sq
    monkeypatch.setattr(S, "row_index", row_index_swapped)
    assert _run_all_pins()


def test_planted_decode_mistake_is_caught(monkeypatch):
    def decode_bad(a, dtype):
        if dtype == "bf16":
            a = np.asarray(a)
            return (a.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)
        return _orig_decode(a, dtype)
    monkeypatch.setattr(S, "decode", decode_bad)
    assert _run_all_pins()


_orig_backward_rows = S.backward_rows


def _backward_rows_mutant(kind):
    """A copy of the oracle's row gather with one plausible mistake planted."""
    def rows_fn(y, dy, dtype, rows, scale=1.0):
        y, dy = np.asarray(y), np.asarray(dy)
        B, H, Sq, Sk = y.shape
        sc = S._fp32(scale)
        out = np.empty((len(rows), Sk))
        for i, r in enumerate(rows):
            b, h, q = S.row_index(y.shape, int(r))
            yr, dyr = y[b, h, q, :], dy[b, h, q, :]
            if kind == "swap":            # y and dy exchanged
                yr, dyr = dyr, yr
            elif kind == "dy_bqh":        # dy read as if laid out [B, Sq, H, Sk]
                dyr = dy.reshape(B, Sq, H, Sk)[b, q, h, :]
            dec = S.decode
            if kind == "decode" and dtype == "bf16":   # bf16 bits taken as fp16 bits
                out[i] = S._backward_one_row(dec(yr.view(np.float16), "f16"),
                                             dec(dyr.view(np.float16), "f16"), sc)
                continue
            if kind == "decode" and dtype == "f16":    # fp16 bits taken as bf16 bits
                out[i] = S._backward_one_row(dec(yr.view(np.uint16), "bf16"),
                                             dec(dyr.view(np.uint16), "bf16"), sc)
                continue
            out[i] = S._backward_one_row(dec(yr, dtype), dec(dyr, dtype), sc)
        return out
    return rows_fn


@pytest.mark.parametrize("kind", ["swap", "dy_bqh", "decode"])
def test_planted_backward_gather_mistake_is_caught(kind, monkeypatch):
    """Mistakes in the tensor-level backward's row gather (y/dy swapped, dy
    from another (b, h, q), the wrong decoding of typed values): ``backward``
    goes through ``backward_rows``, so one planted copy covers both."""
    monkeypatch.setattr(S, "backward_rows", _backward_rows_mutant(kind))
    failures = _run_all_pins()
    assert any(n == "pin_backward_tensor_gather" for n, _ in failures), \
        f"planted gather mistake '{kind}' passed every pin"


def test_unplanted_backward_gather_copy_passes(monkeypatch):
    """The planting copy without a mistake passes every pin (so the failures
    above come from the mistakes, not from the copy)."""
    monkeypatch.setattr(S, "backward_rows", _backward_rows_mutant("none"))
    assert not _run_all_pins()


_orig_excluded = S._excluded
_orig_offset = S.causal_offset


def test_planted_mask_kind_mistakes_are_caught(monkeypatch):
    # boolean mask polarity inverted (zero taken as "excluded")
    def excluded_inverted(n, mrow_bool=None, key_len=None):
        if mrow_bool is not None:
            mrow_bool = (np.asarray(mrow_bool) == 0)
        return _orig_excluded(n, mrow_bool, key_len)
    monkeypatch.setattr(S, "_excluded", excluded_inverted)
    assert _run_all_pins()
    monkeypatch.setattr(S, "_excluded", _orig_excluded)

    # key length off by one (keys k > L excluded instead of k >= L)
    def excluded_len_late(n, mrow_bool=None, key_len=None):
        return _orig_excluded(n, mrow_bool, None if key_len is None else key_len + 1)
    monkeypatch.setattr(S, "_excluded", excluded_len_late)
    assert _run_all_pins()
    monkeypatch.setattr(S, "_excluded", _orig_excluded)

    # bottom-right offset with the wrong sign
    def offset_flipped(mode, Sq, Sk):
        o = _orig_offset(mode, Sq, Sk)
        return -o if o else o
    monkeypatch.setattr(S, "causal_offset", offset_flipped)
    assert _run_all_pins()


# ------------------------------------------------- planted attention mistakes

import oracle.attention as A  # noqa: E402

_orig_kv_head = A.kv_head
_orig_head_scores = A.head_scores
_orig_combine = A.combine
_orig_softmax_lse = S._softmax_and_lse


def _attention_pins_fail():
    """True if at least one attention pin fails."""
    for pin in P.ATTENTION_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


_orig_bwd_row = S._backward_one_row


@pytest.mark.parametrize("mistake", [
    "gqa_modulo", "scores_transposed", "probs_transposed", "values_unweighted",
    "lse_without_max", "no_scale", "softmax_backward_unscaled", "softmax_backward_no_dot",
])
def test_planted_attention_mistakes_are_caught(mistake, monkeypatch):
    if mistake == "gqa_modulo":  # query head h reads kv head h % Hk
        monkeypatch.setattr(A, "kv_head", lambda h, H, Hk: h % Hk)
    elif mistake == "scores_transposed":  # K Q^T in place of Q K^T
        monkeypatch.setattr(A, "head_scores", lambda qh, kh: (kh @ qh.T).T.T)
    elif mistake == "probs_transposed":  # P^T V
        monkeypatch.setattr(A, "combine", lambda P_, vh: P_.T @ vh)
    elif mistake == "values_unweighted":  # sum of V over the keys that survive
        monkeypatch.setattr(A, "combine", lambda P_, vh: (P_ > 0).astype(float) @ vh)
    elif mistake == "lse_without_max":  # log of the shifted sum only
        def lse_bad(s):
            p, lse = _orig_softmax_lse(s)
            m = s.max() if s.size else -math.inf
            return p, (lse - m) if m != -math.inf else lse
        monkeypatch.setattr(S, "_softmax_and_lse", lse_bad)
    elif mistake == "no_scale":
        monkeypatch.setattr(S, "_fp32", lambda v: 1.0)
    elif mistake == "softmax_backward_unscaled":  # dS without the scale factor
        monkeypatch.setattr(S, "_backward_one_row", lambda y, dy, sc: _orig_bwd_row(y, dy, 1.0))
    elif mistake == "softmax_backward_no_dot":  # dS = scale * P * dP
        monkeypatch.setattr(S, "_backward_one_row", lambda y, dy, sc: sc * y * dy)
    assert _attention_pins_fail(), mistake
