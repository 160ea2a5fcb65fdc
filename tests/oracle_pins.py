"""Checks that pin the float64 oracle to facts outside itself.

Each check raises AssertionError when the oracle disagrees with a closed form,
an invariant of the definition, a library routine on a special case, a brute
force second formulation, finite differences or the explicit Jacobian. The
checks call the oracle through ``oracle.softmax`` attributes at call time, so
``tests/test_oracle_pins.py`` can also run them against deliberately broken
copies of the oracle (planted on the CPU) and require that each is caught.

Sources of the facts: the operation's definition -- lmnt.cn "Custom fused
Softmax operator in CUDA, wrapped into PyTorch", sec. 1.2 (score = x*scale +
mask, softmax over keys; causal masks key j > query i), sec. 2.1 (max
subtraction leaves the result unchanged), sec. 3.3 (backward formula and its
Jacobian derivation); pnsm.cn ScaledMaskSoftmax article sec. 4.2/4.3 (a fully
masked row must not produce NaN; zeros chosen). For fused attention
(``oracle.attention``, the QK^T fusion of the pnsm.cn article's sec. 4.4):
closed forms of one and two keys and of equal scores, a second formulation by
brute force, invariances of attention under key permutation and key shift,
grouped-query head mapping, and reduction to the pinned softmax oracle when V
is the identity.
"""

import itertools
import math

import numpy as np

import oracle.attention as A
import oracle.softmax as S

F32, F16 = np.float32, np.float16
NINF = -math.inf


def _close(got, want, atol=0.0, rtol=1e-15, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    with np.errstate(invalid="ignore"):
        ok = (np.abs(got - want) <= atol + rtol * np.abs(want)) | (got == want)
    bad = ~ok  # NaN anywhere counts as a mismatch
    assert not bad.any(), f"{what}: got {got[bad][:4]} want {want[bad][:4]}"


def _logistic(a):
    """1 / (1 + e^-a), written so it never overflows."""
    if a >= 0:
        return 1.0 / (1.0 + math.exp(-a))
    ea = math.exp(a)
    return ea / (1.0 + ea)


# ---------------------------------------------------------------- forward pins

def pin_two_element_closed_form():
    """softmax([s0, s1]) = [logistic(s0-s1), logistic(s1-s0)] for any s0, s1."""
    vals = [-30.0, -7.25, -1.0, 0.0, 0.5, 3.0, 12.0, 40.0]
    for s0, s1 in itertools.product(vals, vals):
        y = S.forward_row(np.array([s0, s1], F32), "f32")
        _close(y, [_logistic(s0 - s1), _logistic(s1 - s0)], rtol=4e-16, what="two-element")
    # Large, equal-ish scores: the naive exp(1000) overflows; the definition does not.
    y = S.forward_row(np.array([1000.0, 1001.0], F32), "f32")
    _close(y, [1.0 / (1.0 + math.e), math.e / (1.0 + math.e)], rtol=4e-16, what="[1000,1001]")


def pin_hand_rows():
    """Rows worked by hand from the definition."""
    # [0, ln 3] -> [1/4, 3/4] up to the fp32 rounding of ln 3
    l3 = float(F32(math.log(3.0)))
    y = S.forward_row(np.array([0.0, l3], F32), "f32")
    _close(y, [1 / (1 + math.exp(l3)), math.exp(l3) / (1 + math.exp(l3))], rtol=4e-16)
    _close(y, [0.25, 0.75], rtol=2e-7, what="[0, ln3]")
    # constant row -> uniform, exactly
    for n in (1, 2, 3, 4, 7, 64, 1000):
        y = S.forward_row(np.full(n, 0.75, F32), "f32")
        _close(y, np.full(n, 1.0 / n), rtol=1e-15, what=f"uniform n={n}")
    # geometric row: s = [0.375, 0.125, -0.125] after scale 1/8; ratios r = e^0.25
    y = S.forward_row(np.array([3.0, 1.0, -1.0], F32), "f32", scale=0.125)
    r = math.exp(0.25)
    z = r * r + r + 1.0
    _close(y, [r * r / z, r / z, 1.0 / z], rtol=4e-16, what="geometric")
    # additive -inf mask entry is exactly 0 and the rest renormalise
    y = S.forward_row(np.array([2.0, 2.0, 5.0], F32), "f32", mrow=np.array([0, 0, NINF], F32))
    assert y.tolist() == [0.5, 0.5, 0.0], y
    # causal, query q=1: keys 2, 3 are masked (key j > query i), key 1 is kept
    y = S.forward_row(np.array([1.0, 2.0, 3.0, 4.0], F32), "f32", scale=0.5, is_causal=True, q=1)
    _close(y[:2], [_logistic(-0.5), _logistic(0.5)], rtol=4e-16, what="causal q=1")
    assert y[2] == 0.0 and y[3] == 0.0
    # causal q=0: only key 0 survives, its probability is exactly 1
    y = S.forward_row(np.array([9.0, -3.0, 1.0], F32), "f32", is_causal=True, q=0)
    assert y.tolist() == [1.0, 0.0, 0.0], y
    # fp16 row whose small probability is an fp16 subnormal: [0, -12]
    y = S.forward_row(np.array([0.0, -12.0], F16), "f16")
    _close(y, [_logistic(12.0), _logistic(-12.0)], rtol=4e-16, what="[0,-12]")


def pin_fully_masked_rows():
    """All keys masked (by the additive mask, by causality or both): all zeros."""
    n = 5
    y = S.forward_row(np.arange(n, dtype=F32), "f32", mrow=np.full(n, NINF, F32))
    assert y.tolist() == [0.0] * n and not np.isnan(y).any()
    m = np.zeros(n, F32)
    m[0] = NINF
    y = S.forward_row(np.arange(n, dtype=F32), "f32", mrow=m, is_causal=True, q=0)
    assert y.tolist() == [0.0] * n
    # one surviving key gets probability exactly 1
    m = np.full(n, NINF, F32)
    m[3] = 0.0
    y = S.forward_row(np.arange(n, dtype=F32), "f32", mrow=m)
    assert y.tolist() == [0.0, 0.0, 0.0, 1.0, 0.0]


def _rng(seed):
    return np.random.default_rng(seed)


def pin_invariants():
    """Sum to one; masked entries exactly zero; shift invariance; permutation."""
    rng = _rng(7)
    for trial in range(40):
        n = int(rng.integers(1, 300))
        x = (rng.standard_normal(n) * 4).astype(F32)
        m = np.where(rng.random(n) < 0.3, NINF, 0.0).astype(F32)
        q = int(rng.integers(0, n))
        causal = bool(trial % 2)
        y = S.forward_row(x, "f32", mrow=m, scale=0.3, is_causal=causal, q=q)
        dead = np.isinf(m) | ((np.arange(n) > q) if causal else False)
        assert (y[dead] == 0.0).all()
        if not dead.all():
            assert abs(math.fsum(y) - 1.0) < 1e-14
            assert (y[~dead] > 0).all()
        # shift: x + c with c a multiple of 2^-4 and |x| < 2^8 is exact in fp32
        xq = np.round(x * 16) / 16
        c = float(rng.integers(-64, 64)) / 16.0
        y0 = S.forward_row(xq.astype(F32), "f32", mrow=m, scale=1.0, is_causal=causal, q=q)
        y1 = S.forward_row((xq + c).astype(F32), "f32", mrow=m, scale=1.0, is_causal=causal, q=q)
        _close(y1, y0, atol=1e-15, rtol=1e-13, what="shift")
        # key permutation (no causal): output permutes with the input
        p = rng.permutation(n)
        ya = S.forward_row(x, "f32", mrow=m, scale=0.3)
        yb = S.forward_row(x[p], "f32", mrow=m[p], scale=0.3)
        _close(yb, ya[p], atol=1e-17, rtol=1e-14, what="permutation")
    # scale 0 -> uniform over the unmasked keys
    x = (rng.standard_normal(50) * 9).astype(F32)
    m = np.where(np.arange(50) % 3 == 0, NINF, 0.0).astype(F32)
    y = S.forward_row(x, "f32", mrow=m, scale=0.0)
    keep = ~np.isinf(m)
    _close(y[keep], np.full(keep.sum(), 1.0 / keep.sum()), rtol=1e-15, what="scale 0")
    # monotone: a larger score never gets a smaller probability
    x = (rng.standard_normal(200) * 3).astype(F32)
    y = S.forward_row(x, "f32", scale=0.7)
    o = np.argsort(x, kind="stable")
    assert (np.diff(y[o]) >= 0).all()


def pin_library_special_case():
    """No mask, no causal, scale 1: the library softmax in float64."""
    import scipy.special
    import torch
    rng = _rng(11)
    x = (rng.standard_normal((2, 3, 5, 37)) * 3).astype(F32)
    y = S.forward(x, "f32")
    _close(y, scipy.special.softmax(x.astype(np.float64), axis=-1), atol=1e-17, rtol=1e-14,
           what="scipy")
    t = torch.softmax(torch.from_numpy(x.astype(np.float64)), dim=-1).numpy()
    _close(y, t, atol=1e-17, rtol=1e-14, what="torch")


def _brute_row(svals):
    """Second formulation: exp(s_k) / sum_j exp(s_j) without the max shift,
    with math.fsum, on small scores only; masked keys are None."""
    keep = [v for v in svals if v is not None]
    if not keep:
        return [0.0] * len(svals)
    z = math.fsum(math.exp(v) for v in keep)
    return [0.0 if v is None else math.exp(v) / z for v in svals]


def pin_brute_force_exhaustive():
    """All 2^n mask patterns x causal x query position, n <= 6, on an exact grid."""
    rng = _rng(3)
    for n in range(1, 7):
        x = (rng.integers(-16, 17, n) * 0.25).astype(F32)  # exact grid in [-4, 4]
        for bits in range(1 << n):
            m = np.array([NINF if (bits >> k) & 1 else 0.0 for k in range(n)], F32)
            for causal in (False, True):
                for q in (range(n) if causal else [0]):
                    y = S.forward_row(x, "f32", mrow=m, scale=0.5, is_causal=causal, q=q)
                    s = [None if (np.isinf(m[k]) or (causal and k > q)) else 0.5 * float(x[k])
                         for k in range(n)]
                    _close(y, _brute_row(s), atol=1e-17, rtol=1e-14, what=f"brute n={n}")


def _mask_index(mode, b, h, q):
    return {"sq_sk": (0, 0, q), "b_sq_sk": (b, 0, q), "b_1_sk": (b, 0, 0),
            "full": (b, h, q)}[mode]


def pin_tensor_indexing():
    """Whole-tensor forward against an explicit per-(b,h,q) loop for every
    broadcast mode, with a mask that differs along every axis it has."""
    rng = _rng(5)
    B, H, Sq, Sk = 2, 3, 4, 6
    x = (rng.integers(-12, 13, (B, H, Sq, Sk)) * 0.25).astype(F32)
    shapes4 = {"sq_sk": (1, 1, Sq, Sk), "b_sq_sk": (B, 1, Sq, Sk), "b_1_sk": (B, 1, 1, Sk),
               "full": (B, H, Sq, Sk)}
    for mode, ms in shapes4.items():
        mask = (rng.integers(-8, 9, ms) * 0.5).astype(F32)
        mask[rng.random(ms) < 0.2] = NINF
        for causal in (False, True):
            y = S.forward(x, "f32", mask=mask, scale=0.75, is_causal=causal)
            for b, h, q in itertools.product(range(B), range(H), range(Sq)):
                mb, mh, mq = _mask_index(mode, b, h, q)
                s = []
                for k in range(Sk):
                    mv = float(mask[mb, mh, mq, k])
                    dead = math.isinf(mv) or (causal and k > q)
                    s.append(None if dead else 0.75 * float(x[b, h, q, k]) + mv)
                _close(y[b, h, q], _brute_row(s), atol=1e-17, rtol=1e-14,
                       what=f"indexing {mode} causal={causal} ({b},{h},{q})")
            # the row-subset entry point agrees with the whole-tensor one
            rows = [0, B * H * Sq - 1, 5]
            yr = S.forward_rows(x, "f32", rows, mask=mask, scale=0.75, is_causal=causal)
            for i, r in enumerate(rows):
                b, h, q = S.row_index(x.shape, r)
                assert (yr[i] == y[b, h, q]).all()


def pin_decode():
    """Exact decoding of typed inputs, from the formats' definitions."""
    bf = np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x8000, 0x7F80, 0xFF80, 0x4049, 0x0080],
                  np.uint16)
    want = [1.0, -2.0, 1.5, 2.0 ** -133, -0.0, math.inf, -math.inf,
            3.140625, 2.0 ** -126]
    got = S.decode(bf, "bf16")
    assert got.tolist() == want, got
    h = np.array([1.0, 2.0 ** -24, 65504.0, -0.5], F16)
    assert S.decode(h, "f16").tolist() == [1.0, 2.0 ** -24, 65504.0, -0.5]
    # the bf16 and fp32 paths of the oracle agree on bf16-representable rows
    v = np.array([0.5, -1.25, 3.0, 0.0], F32)
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    _close(S.forward_row(bits, "bf16", scale=0.9), S.forward_row(v, "f32", scale=0.9),
           rtol=0, what="bf16 vs f32")
    # fp64 values pass through unchanged, including those no fp32 holds
    d = np.array([0.1, 1.0 + 2.0 ** -52, -2.0 ** -1074, 1e300], np.float64)
    assert S.decode(d, "f64").tolist() == d.tolist()
    # the fp64 path is the same definition: the logistic closed form on a pair
    # of scores fp32 cannot hold, and equality with the f32 path where it can
    a, b = 0.1, 0.3
    y = S.forward_row(np.array([a, b]), "f64", scale=1.0)
    _close(y, [1 / (1 + math.exp(b - a)), 1 / (1 + math.exp(a - b))], rtol=1e-15, what="f64 pair")
    _close(S.forward_row(v.astype(np.float64), "f64", scale=0.9),
           S.forward_row(v, "f32", scale=0.9), rtol=0, what="f64 vs f32")
    try:
        S.decode(np.zeros(2, F32), "f64")
    except TypeError:
        pass
    else:
        raise AssertionError("f64 decode must reject float32 data")


def pin_scale_rounding():
    """scale enters as the fp32 value nearest to it."""
    s = 1.0 / math.sqrt(128.0)
    y = S.forward_row(np.array([0.0, 1.0], F32), "f32", scale=s)
    _close(y, [_logistic(-float(F32(s))), _logistic(float(F32(s)))], rtol=4e-16)


# --------------------------------------------------------------- backward pins

def _fd_grad(x, m, sc, causal, q, dy, h=1e-6):
    """Central differences of L(x) = sum_k dy_k * y_k(x) on the float64 forward core."""
    g = np.zeros_like(x)
    for j in range(x.size):
        hp = h * max(1.0, abs(x[j]))
        xp = x.copy()
        xm = x.copy()
        xp[j] += hp
        xm[j] -= hp
        lp = float(np.dot(dy, S._forward_one_row(xp, m, sc, causal, q)))
        lm = float(np.dot(dy, S._forward_one_row(xm, m, sc, causal, q)))
        g[j] = (lp - lm) / (2 * hp)
    return g


def pin_backward_finite_differences():
    rng = _rng(13)
    for trial in range(24):
        n = int(rng.integers(1, 17))
        x = rng.standard_normal(n) * 2.0
        m = np.where(rng.random(n) < 0.25, NINF, 0.0)
        causal = bool(trial % 3 == 0)
        q = int(rng.integers(0, n))
        sc = float(F32([0.125, 0.5, 1.0, 2.5][trial % 4]))
        dy = rng.standard_normal(n)
        y = S._forward_one_row(x, m, sc, causal, q)
        dx = S._backward_one_row(y, dy, sc)
        fd = _fd_grad(x, m, sc, causal, q, dy)
        _close(dx, fd, atol=2e-8, rtol=1e-6, what=f"FD trial {trial}")


def pin_backward_jacobian():
    """dx = scale * J^T dy with J = diag(y) - y y^T (the softmax Jacobian)."""
    rng = _rng(17)
    for n in (1, 2, 3, 8, 16):
        x = (rng.standard_normal(n) * 3).astype(F32)
        y = S.forward_row(x, "f32", scale=0.5).astype(F32)   # a typed y, as the op receives
        dy = rng.standard_normal(n).astype(F32)
        yd, dyd = y.astype(np.float64), dy.astype(np.float64)
        J = np.diag(yd) - np.outer(yd, yd)
        _close(S.backward_row(y, dy, "f32", scale=0.5), 0.5 * (J.T @ dyd), atol=1e-16,
               rtol=1e-12, what=f"Jacobian n={n}")
    # worked example: y = softmax([1,2,3]), dy = e_0, scale 1/2
    y = S._forward_one_row(np.array([1.0, 2.0, 3.0]), None, 1.0, False, 0)
    dx = S._backward_one_row(y, np.array([1.0, 0.0, 0.0]), 0.5)
    want = [0.5 * y[0] * (1 - y[0]), -0.5 * y[0] * y[1], -0.5 * y[0] * y[2]]
    _close(dx, want, rtol=1e-15, what="worked Jacobian")


def pin_backward_invariants():
    rng = _rng(19)
    for trial in range(20):
        n = int(rng.integers(2, 200))
        x = rng.standard_normal(n) * 2
        m = np.where(rng.random(n) < 0.3, NINF, 0.0)
        m[int(rng.integers(0, n))] = 0.0
        sc = 0.25 + trial * 0.1
        y = S._forward_one_row(x, m, sc, False, 0)
        dy = rng.standard_normal(n)
        dx = S._backward_one_row(y, dy, sc)
        assert abs(math.fsum(dx)) < 1e-14 * max(1.0, np.abs(dy).max())   # sum dx = 0
        assert (dx[y == 0.0] == 0.0).all()                               # masked -> 0
        dc = S._backward_one_row(y, np.full(n, 1.7), sc)                  # constant dy -> 0
        assert np.abs(dc).max() < 1e-15
        dyy = S._backward_one_row(y, y, sc)                               # dy = y
        _close(dyy, sc * y * (y - float(np.dot(y, y))), atol=1e-18, rtol=1e-12)
    # typed wrapper decodes y and dy before the formula
    y = np.array([0.25, 0.75], F16)
    dy = np.array([1.0, -1.0], F16)
    _close(S.backward_row(y, dy, "f16", scale=2.0), [2 * 0.25 * (1 - (-0.5)),
                                                     2 * 0.75 * (-1 - (-0.5))], rtol=0)


def _bf16_values_torch(bits):
    """bf16 bit patterns to float64 through torch's own bfloat16 type, a decoder
    that shares nothing with the oracle's."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def pin_backward_tensor_gather():
    """The whole-tensor backward (``backward``) and the row-subset one
    (``backward_rows``) against the softmax Jacobian applied row by row with
    explicit (b, h, q) indexing: y and dy differ in every row and along every
    axis, so a swap of y and dy, a row taken from another (b, h, q) or a wrong
    decoding of the typed values changes the result (lmnt.cn page sec. 3.3)."""
    rng = _rng(23)
    B, H, Sq, Sk = 2, 3, 4, 5
    for dtype in ("f32", "f16", "bf16"):
        # y: a distinct positive row per (b, h, q) (a probability-like row that
        # need not sum to 1: the formula does not assume it); dy: signed.
        yv = (rng.integers(1, 64, (B, H, Sq, Sk)) / 64.0
              + np.arange(B * H * Sq).reshape(B, H, Sq, 1) / 1024.0)
        dyv = rng.integers(-40, 41, (B, H, Sq, Sk)) / 16.0
        if dtype == "bf16":
            # values exact in bf16 (8 significant bits): multiples of 1/64 below 4
            yv = np.round(yv * 64) / 64
            y = (yv.astype(F32).view(np.uint32) >> 16).astype(np.uint16)
            dy = (dyv.astype(F32).view(np.uint32) >> 16).astype(np.uint16)
            yd, dyd = _bf16_values_torch(y), _bf16_values_torch(dy)
            assert (yd == yv).all() and (dyd == dyv).all()
        else:
            t = F32 if dtype == "f32" else F16
            y, dy = yv.astype(t), dyv.astype(t)
            yd, dyd = y.astype(np.float64), dy.astype(np.float64)
        sc = 0.75
        full = S.backward(y, dy, dtype, scale=sc)
        assert full.shape == (B, H, Sq, Sk)
        rows = [5, 0, B * H * Sq - 1, 13, 7]
        sub = S.backward_rows(y, dy, dtype, rows, scale=sc)
        for b, h, q in itertools.product(range(B), range(H), range(Sq)):
            yr, dyr = yd[b, h, q], dyd[b, h, q]
            J = np.diag(yr) - np.outer(yr, yr)      # d softmax / d s, symmetric
            want = sc * (J @ dyr)
            _close(full[b, h, q], want, atol=1e-15, rtol=1e-13,
                   what=f"backward {dtype} ({b},{h},{q})")
            r = (b * H + h) * Sq + q
            if r in rows:
                _close(sub[rows.index(r)], want, atol=1e-15, rtol=1e-13,
                       what=f"backward_rows {dtype} row {r}")


def pin_bool_masks():
    """Boolean masks: nonzero excludes the key (score -inf); exhaustive brute
    force over every pattern for n <= 6 and a hand row fixing the polarity."""
    y = S.forward_row(np.array([1.0, 2.0, 3.0], F32), "f32",
                      mrow=np.array([0, 1, 0], np.uint8), mask_kind="bool")
    _close(y, [_logistic(-2.0), 0.0, _logistic(2.0)], rtol=4e-16, what="bool polarity")
    assert y[1] == 0.0
    rng = _rng(23)
    for n in range(1, 7):
        x = (rng.integers(-16, 17, n) * 0.25).astype(F32)
        for bits in range(1 << n):
            m = np.array([(bits >> k) & 1 for k in range(n)], np.bool_)
            for causal in (False, True):
                for q in (range(n) if causal else [0]):
                    y = S.forward_row(x, "f32", mrow=m, scale=0.5, is_causal=causal, q=q,
                                      mask_kind="bool")
                    s = [None if (m[k] or (causal and k > q)) else 0.5 * float(x[k])
                         for k in range(n)]
                    _close(y, _brute_row(s), atol=1e-17, rtol=1e-14, what=f"bool brute n={n}")


def pin_key_lengths():
    """Key lengths: keys k >= L excluded; L = 0 gives zeros, L >= Sk nothing."""
    x = np.array([1.0, 2.0, 3.0, 4.0], F32)
    _close(S.forward_row(x, "f32", key_len=2), [_logistic(-1.0), _logistic(1.0), 0, 0],
           rtol=4e-16, what="L=2")
    assert S.forward_row(x, "f32", key_len=0).tolist() == [0.0] * 4
    assert S.forward_row(x, "f32", key_len=1).tolist() == [1.0, 0.0, 0.0, 0.0]
    _close(S.forward_row(x, "f32", key_len=9), S.forward_row(x, "f32"), rtol=0)
    # tensor level: one length per batch, against a per-row brute force
    rng = _rng(29)
    B, H, Sq, Sk = 3, 2, 3, 7
    xt = (rng.integers(-12, 13, (B, H, Sq, Sk)) * 0.25).astype(F32)
    lens = np.array([0, 3, 7])
    for causal in (False, True):
        y = S.forward(xt, "f32", scale=0.5, is_causal=causal, mask_kind="lengths",
                      key_lengths=lens)
        for b, h, q in itertools.product(range(B), range(H), range(Sq)):
            s = [None if (k >= lens[b] or (causal and k > q)) else 0.5 * float(xt[b, h, q, k])
                 for k in range(Sk)]
            _close(y[b, h, q], _brute_row(s), atol=1e-17, rtol=1e-14, what="lengths tensor")


def pin_causal_alignments():
    """Top-left: query q keeps keys 0..q. Bottom-right: keys 0..q+Sk-Sq, so the
    last query keeps every key; Sq > Sk leaves the first Sq-Sk rows empty."""
    x = np.zeros((1, 1, 2, 4), F32)  # equal scores: uniform over the kept keys
    y = S.forward(x, "f32", is_causal="bottom_right")
    _close(y[0, 0, 0], [1 / 3, 1 / 3, 1 / 3, 0], rtol=1e-15, what="BR q=0")
    _close(y[0, 0, 1], [0.25] * 4, rtol=1e-15, what="BR q=1")
    y = S.forward(x, "f32", is_causal="top_left")
    _close(y[0, 0, 0], [1, 0, 0, 0], rtol=0, what="TL q=0")
    _close(y[0, 0, 1], [0.5, 0.5, 0, 0], rtol=1e-15, what="TL q=1")
    x = np.zeros((1, 1, 4, 2), F32)
    y = S.forward(x, "f32", is_causal="bottom_right")
    assert y[0, 0, 0].tolist() == [0.0, 0.0] and y[0, 0, 1].tolist() == [0.0, 0.0]
    assert y[0, 0, 2].tolist() == [1.0, 0.0]
    _close(y[0, 0, 3], [0.5, 0.5], rtol=1e-15, what="BR Sq>Sk last")
    # square tensors: both rules agree
    xs = (_rng(31).standard_normal((1, 2, 5, 5)) * 2).astype(F32)
    _close(S.forward(xs, "f32", is_causal="bottom_right"), S.forward(xs, "f32", is_causal=True),
           rtol=0)


# ------------------------------------------------------------- attention pins

def _attn_brute(q, k, v, scale, causal_offset=None):
    """A second formulation for tiny float64 inputs without masks: loops over
    queries and keys, no max shift, exact sums (math.fsum)."""
    B, H, Sq, D = q.shape
    Hk, Sk = k.shape[1], k.shape[2]
    O = np.zeros((B, H, Sq, D))
    L = np.zeros((B, H, Sq))
    for b, h, i in itertools.product(range(B), range(H), range(Sq)):
        g = h // (H // Hk)
        keys = [j for j in range(Sk) if causal_offset is None or j <= i + causal_offset]
        w = [math.exp(scale * math.fsum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)))
             for j in keys]
        z = math.fsum(w)
        L[b, h, i] = math.log(z) if keys else NINF
        for d in range(D):
            O[b, h, i, d] = math.fsum(wj * v[b, g, j, d] for wj, j in zip(w, keys)) / z if keys else 0
    return O, L


def _ints(seed, shape, lo=-3, hi=4, dtype=F32):
    return _rng(seed).integers(lo, hi, size=shape).astype(dtype)


def pin_attention_one_and_two_keys():
    """One key: every query returns that key's value row and LSE = its score.
    Two keys: O = sigma v0 + (1 - sigma) v1 with sigma = logistic(s0 - s1) and
    LSE = log(e^s0 + e^s1), scores from integer vectors (exact)."""
    q, k, v = _ints(1, (1, 2, 3, 4)), _ints(2, (1, 2, 1, 4)), _ints(3, (1, 2, 1, 4))
    O, L = A.forward(q, k, v, "f32", scale=0.5)
    for h in range(2):
        _close(O[0, h], np.repeat(v[0, h].astype(np.float64), 3, axis=0), rtol=1e-15, what="one key O")
        _close(L[0, h], 0.5 * (q[0, h] @ k[0, h, 0]), rtol=1e-15, what="one key LSE")
    q, k, v = _ints(4, (1, 1, 3, 4)), _ints(5, (1, 1, 2, 4)), _ints(6, (1, 1, 2, 4))
    O, L = A.forward(q, k, v, "f32", scale=0.25)
    for i in range(3):
        s0 = 0.25 * float(q[0, 0, i] @ k[0, 0, 0])
        s1 = 0.25 * float(q[0, 0, i] @ k[0, 0, 1])
        sg = _logistic(s0 - s1)
        vd = v.astype(np.float64)
        _close(O[0, 0, i], sg * vd[0, 0, 0] + (1 - sg) * vd[0, 0, 1], rtol=1e-14, what="two keys O")
        _close(L[0, 0, i], max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), rtol=1e-15,
               what="two keys LSE")


def pin_attention_equal_scores():
    """Q = 0: every score is 0, so O is the mean of the value rows each query
    may see (all; the first i+1 under the causal rule; the first L_b with key
    lengths), LSE = log(count); no key at all gives zeros and -inf."""
    Sq = Sk = 5
    q = np.zeros((2, 1, Sq, 3), F32)
    k = _ints(7, (2, 1, Sk, 3))
    v = _ints(8, (2, 1, Sk, 3))
    vd = v.astype(np.float64)
    O, L = A.forward(q, k, v, "f32", scale=0.7)
    _close(O[:, 0], np.repeat(vd[:, 0].mean(axis=1, keepdims=True), Sq, axis=1), atol=1e-14,
           rtol=1e-14, what="mean of V")
    _close(L, np.full((2, 1, Sq), math.log(Sk)), rtol=1e-15, what="LSE log n")
    O, L = A.forward(q, k, v, "f32", is_causal=True)
    for i in range(Sq):
        _close(O[:, 0, i], vd[:, 0, :i + 1].mean(axis=1), atol=1e-14, rtol=1e-14,
               what="causal prefix mean")
        _close(L[:, 0, i], [math.log(i + 1)] * 2, rtol=1e-15, what="causal LSE")
    O, L = A.forward(q, k, v, "f32", mask_kind="lengths", key_lengths=[0, 2])
    assert (O[0] == 0).all() and (L[0] == NINF).all()
    _close(O[1, 0], np.repeat(vd[1, 0, :2].mean(axis=0, keepdims=True), Sq, axis=0), atol=1e-14,
           rtol=1e-14, what="length mean")


def pin_attention_brute_force():
    """Against the loop formulation on random tiny inputs: plain, top-left and
    bottom-right causal (Sq < Sk), and grouped heads (H = 4 over Hk = 2)."""
    r = _rng(9)
    for (B, H, Hk, Sq, Sk, D), causal in itertools.product(
            [(1, 2, 2, 3, 5, 4), (2, 4, 2, 4, 4, 3), (1, 1, 1, 1, 7, 2)],
            [False, True, "bottom_right"]):
        q = r.standard_normal((B, H, Sq, D)).astype(np.float64)
        k = r.standard_normal((B, Hk, Sk, D)).astype(np.float64)
        v = r.standard_normal((B, Hk, Sk, D)).astype(np.float64)
        off = S.causal_offset(causal, Sq, Sk)
        O, L = A.forward(q, k, v, "f64", scale=0.6, is_causal=causal)
        Ob, Lb = _attn_brute(q, k, v, float(np.float32(0.6)), off)
        _close(O, Ob, atol=1e-14, rtol=1e-12, what=f"brute O {causal}")
        _close(L, Lb, atol=1e-14, rtol=1e-12, what=f"brute LSE {causal}")
        # The probabilities themselves: P V is the brute-force output, the
        # log-sum-exp is the brute-force one, and every row sums to 1.
        P, LP = A.probabilities(q, k, "f64", scale=0.6, is_causal=causal)
        _close(LP, Lb, atol=1e-14, rtol=1e-12, what=f"probabilities LSE {causal}")
        _close(P.sum(axis=3), np.ones((B, H, Sq)), atol=1e-14, what="probability rows")
        PV = np.stack([np.stack([P[b, h] @ v[b, h // (H // Hk)] for h in range(H)])
                       for b in range(B)])
        _close(PV, Ob, atol=1e-14, rtol=1e-12, what=f"probabilities P V {causal}")


def pin_attention_invariants():
    """Permuting keys with their values leaves O unchanged (no causal rule);
    adding one vector c to every key adds scale*q.c to each row's scores, which
    leaves O unchanged and shifts LSE by exactly that (integer data: exact)."""
    q, k, v = _ints(10, (1, 2, 4, 3)), _ints(11, (1, 2, 6, 3)), _ints(12, (1, 2, 6, 3))
    O, L = A.forward(q, k, v, "f32", scale=0.5)
    perm = _rng(13).permutation(6)
    O2, L2 = A.forward(q, k[:, :, perm], v[:, :, perm], "f32", scale=0.5)
    _close(O2, O, rtol=1e-14, what="key permutation O")
    _close(L2, L, rtol=1e-14, what="key permutation LSE")
    c = np.array([1, -2, 3], F32)
    O3, L3 = A.forward(q, k + c, v, "f32", scale=0.5)
    _close(O3, O, atol=1e-14, rtol=1e-13, what="key shift O")
    _close(L3, L + 0.5 * (q.astype(np.float64) @ c.astype(np.float64)), rtol=1e-14,
           what="key shift LSE")


def pin_attention_heads_and_masks():
    """Grouped heads equal ordinary attention over repeated K/V; with V the
    identity (D = Sk) O equals the softmax oracle's rows of the scaled masked
    scores Q K^T (integer data: the scores are exact) for every mask kind and
    causal rule."""
    q, k, v = _ints(14, (2, 4, 3, 5)), _ints(15, (2, 2, 6, 5)), _ints(16, (2, 2, 6, 5))
    O, L = A.forward(q, k, v, "f32", scale=0.3)
    Or, Lr = A.forward(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), "f32", scale=0.3)
    _close(O, Or, rtol=0, what="GQA O")
    _close(L, Lr, rtol=0, what="GQA LSE")
    B, H, Sq, Sk = 2, 2, 4, 6
    q, k = _ints(17, (B, H, Sq, 3)), _ints(18, (B, H, Sk, 3))
    eye = np.broadcast_to(np.eye(Sk, dtype=F32), (B, H, Sk, Sk)).copy()
    S4 = (q.astype(np.float64) @ np.swapaxes(k.astype(np.float64), -1, -2)).astype(F32)
    add = (_rng(19).standard_normal((1, 1, Sq, Sk)) * 2).astype(F32)
    boolm = _rng(20).random((B, 1, Sq, Sk)) < 0.4
    lens = [2, 5]
    for causal in (False, True, "bottom_right"):
        for mask, kind, kl in ((None, "additive", None), (add, "additive", None),
                               (boolm, "bool", None), (None, "lengths", lens)):
            O, _ = A.forward(q, k, eye, "f32", mask=mask, scale=0.4, is_causal=causal,
                             mask_kind=kind, key_lengths=kl)
            want = S.forward(S4, "f32", mask=mask, scale=0.4, is_causal=causal, mask_kind=kind,
                             key_lengths=kl)
            _close(O, want, atol=1e-16, rtol=1e-14, what=f"V=I {kind} {causal}")


def pin_attention_backward_finite_differences():
    """dQ, dK, dV against central differences of L = sum(dO * O) computed with
    the forward oracle, on tiny float64 inputs: grouped heads (H = 2 over
    Hk = 1), an additive mask, a boolean mask with the causal rule, key lengths."""
    r = _rng(21)
    B, H, Hk, Sq, Sk, D = 1, 2, 1, 3, 4, 2
    q = r.standard_normal((B, H, Sq, D))
    k = r.standard_normal((B, Hk, Sk, D))
    v = r.standard_normal((B, Hk, Sk, D))
    do = r.standard_normal((B, H, Sq, D))
    add = r.standard_normal((1, 1, Sq, Sk))
    boolm = np.array([[[[0, 1, 0, 0], [0, 0, 1, 0], [1, 0, 0, 0]]]], bool)
    cases = [dict(), dict(mask=add), dict(mask=boolm, mask_kind="bool", is_causal=True),
             dict(mask_kind="lengths", key_lengths=[3], is_causal="bottom_right")]
    for kw in cases:
        def loss(qq, kk, vv):
            return float((A.forward(qq, kk, vv, "f64", scale=0.7, **kw)[0] * do).sum())
        dq, dk, dv = A.backward(q, k, v, do, "f64", scale=0.7, **kw)
        for arr, grad, name in ((q, dq, "dQ"), (k, dk, "dK"), (v, dv, "dV")):
            for idx in itertools.product(*[range(n) for n in arr.shape]):
                hstep = 1e-6
                a1, a2 = arr.copy(), arr.copy()
                a1[idx] += hstep
                a2[idx] -= hstep
                args1 = [a1 if x is arr else x for x in (q, k, v)]
                args2 = [a2 if x is arr else x for x in (q, k, v)]
                fd = (loss(*args1) - loss(*args2)) / (2 * hstep)
                _close(grad[idx], fd, atol=1e-8, rtol=1e-6, what=f"{name}{idx} {kw}")


def pin_attention_backward_structure():
    """Keys no query sees (key lengths) get dK = dV = 0; grouped heads sum
    their heads' gradients (equal to repeating K and V and adding the copies)."""
    q, k, v = _ints(22, (2, 2, 3, 4)), _ints(23, (2, 2, 5, 4)), _ints(24, (2, 2, 5, 4))
    do = _ints(25, (2, 2, 3, 4))
    dq, dk, dv = A.backward(q, k, v, do, "f32", scale=0.3, mask_kind="lengths", key_lengths=[2, 4])
    assert (dk[0, :, 2:] == 0).all() and (dv[0, :, 2:] == 0).all()
    assert (dk[1, :, 4:] == 0).all() and (dv[1, :, 4:] == 0).all()
    kq, vq = _ints(26, (2, 1, 5, 4)), _ints(27, (2, 1, 5, 4))
    dq1, dk1, dv1 = A.backward(q, kq, vq, do, "f32", scale=0.3)
    dq2, dk2, dv2 = A.backward(q, np.repeat(kq, 2, axis=1), np.repeat(vq, 2, axis=1), do, "f32",
                               scale=0.3)
    _close(dq1, dq2, rtol=0, what="GQA dQ")
    _close(dk1[:, 0], dk2.sum(axis=1), atol=1e-14, rtol=1e-14, what="GQA dK")
    _close(dv1[:, 0], dv2.sum(axis=1), atol=1e-14, rtol=1e-14, what="GQA dV")
    # No query: no gradient reaches K or V.
    dq0, dk0, dv0 = A.backward(q[:, :, :0], k, v, do[:, :, :0], "f32", scale=0.3)
    assert dq0.shape == (2, 2, 0, 4) and not dk0.any() and not dv0.any()


ATTENTION_PINS = [pin_attention_one_and_two_keys, pin_attention_equal_scores,
                  pin_attention_brute_force, pin_attention_invariants,
                  pin_attention_heads_and_masks, pin_attention_backward_finite_differences,
                  pin_attention_backward_structure]


FORWARD_PINS = [pin_two_element_closed_form, pin_hand_rows, pin_fully_masked_rows,
                pin_invariants, pin_library_special_case, pin_brute_force_exhaustive,
                pin_tensor_indexing, pin_decode, pin_scale_rounding, pin_bool_masks,
                pin_key_lengths, pin_causal_alignments]
BACKWARD_PINS = [pin_backward_finite_differences, pin_backward_jacobian,
                 pin_backward_invariants, pin_backward_tensor_gather]
ALL_PINS = FORWARD_PINS + BACKWARD_PINS + ATTENTION_PINS
