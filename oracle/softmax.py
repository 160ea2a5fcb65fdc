"""Plain float64 reference of y = softmax(x*scale + mask) and its backward.

TEST INFRASTRUCTURE ONLY (see the package docstring). Slow and obvious on
purpose: one row at a time, the definition written out, no blocking or fusion.

Conventions
-----------
* ``x`` has shape [B, H, Sq, Sk]; softmax runs over the last axis (keys).
* Typed inputs are numpy arrays: ``float32`` for fp32, ``float16`` for fp16,
  ``float64`` for fp64 and ``uint16`` holding the raw bit patterns for bf16
  (numpy has no bfloat16). The ``dtype`` argument ("f32", "f16", "bf16",
  "f64") says which. Every value converts to float64 exactly; for fp64 inputs
  the oracle computes at the inputs' own precision.
* ``mask`` is ``None`` or a 4-D array whose every axis has the length of the
  matching axis of ``x`` or length 1 (length 1 = broadcast over that axis).
  It holds additive values (0 keeps, a large negative value or -inf masks),
  in the same dtype as ``x`` -- lmnt.cn "Custom fused Softmax operator in CUDA,
  wrapped into PyTorch", sec. 2.2 (additive mask) and sec. 4.2 (mask passed with
  the input's element type).
* ``mask_kind="bool"``: the mask holds booleans (numpy bool or uint8); a
  nonzero entry excludes the key (its score is -inf), as in the pnsm.cn
  ScaledMaskSoftmax article, sec. 2.3 (mask value 1 marks an illegal position,
  handled inside the operator).
* ``mask_kind="lengths"``: ``key_lengths`` holds one integer per batch; keys
  k >= key_lengths[b] are excluded (key padding given as lengths).
* Causal: key k of query q is excluded when k > q + offset, with offset 0 for
  the top-left rule of lmnt.cn sec. 1.2 (key j > query i) and Sk - Sq for the
  bottom-right rule (the last query sees every key).
* ``scale`` is rounded to fp32 first, because the operation receives it as a
  32-bit float (same page, sec. 4.2: the wrapper casts it to float).
* Outputs are float64 arrays, unrounded.
"""

import math

import numpy as np

DTYPES = ("f32", "f16", "bf16", "f64")


def decode(a, dtype):
    """Exact float64 values of a typed array (bf16 given as uint16 bit patterns)."""
    a = np.asarray(a)
    if dtype == "f32":
        if a.dtype != np.float32:
            raise TypeError("f32 data must be a float32 array")
        return a.astype(np.float64)
    if dtype == "f16":
        if a.dtype != np.float16:
            raise TypeError("f16 data must be a float16 array")
        return a.astype(np.float64)
    if dtype == "f64":
        if a.dtype != np.float64:
            raise TypeError("f64 data must be a float64 array")
        return a.astype(np.float64)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be a uint16 array of bit patterns")
        # A bf16 value is the upper half of an IEEE binary32 value.
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _fp32(v):
    return float(np.float32(v))


def _check_mask_shape(mask, shape):
    if mask is None:
        return
    if mask.ndim != 4:
        raise ValueError("mask must be 4-D with length-1 axes for broadcast")
    for m, n in zip(mask.shape, shape):
        if m not in (1, n):
            raise ValueError(f"mask shape {mask.shape} does not broadcast to {shape}")


def row_index(shape, r):
    """Flat row number r -> (b, h, q) for x of shape [B, H, Sq, Sk]."""
    B, H, Sq, _ = shape
    if not 0 <= r < B * H * Sq:
        raise IndexError(r)
    q = r % Sq
    h = (r // Sq) % H
    b = r // (Sq * H)
    return b, h, q


def _mask_row(maskd, b, h, q):
    # Broadcast axes have length 1: index 0 there.
    mb = b if maskd.shape[0] > 1 else 0
    mh = h if maskd.shape[1] > 1 else 0
    mq = q if maskd.shape[2] > 1 else 0
    return maskd[mb, mh, mq, :]


def causal_offset(mode, Sq, Sk):
    """Offset of the causal bound: key k is excluded when k > q + offset."""
    if mode in (False, None, 0, "none"):
        return None
    if mode in (True, 1, "top_left"):
        return 0
    if mode in (2, "bottom_right"):
        return Sk - Sq
    raise ValueError(f"unknown causal mode {mode!r}")


def _scores_one_row(xrow, mrow, sc, causal, q, excluded=None, offset=0):
    """The scores of one row, in float64: x*scale + mask, -inf where a key is
    excluded (``excluded``: boolean mask, key lengths) or past the causal bound."""
    n = xrow.shape[0]
    # score_k = x_k*scale + mask_k
    s = xrow * sc
    if mrow is not None:
        s = s + mrow
    if excluded is not None:
        s = np.where(excluded, -math.inf, s)
    # Causal: keys after the bound are masked, after the additive mask.
    if causal:
        s = s.copy()
        s[np.arange(n) > q + offset] = -math.inf
    return s


def _softmax_and_lse(s):
    """softmax(s) and log(sum_k exp(s_k)) of one row of scores, in float64."""
    n = s.shape[0]
    m = s.max() if n else -math.inf
    if m == -math.inf:
        # Every key is masked: the row is all zeros (nothing to normalise).
        return np.zeros(n, dtype=np.float64), -math.inf
    e = np.exp(s - m)  # exp(-inf) is exactly 0
    z = e.sum()
    return e / z, m + math.log(z)


def _forward_one_row(xrow, mrow, sc, causal, q, excluded=None, offset=0):
    """Softmax of one row of scores, in float64. ``excluded`` is a boolean
    array of keys that take score -inf (boolean mask, key lengths)."""
    return _softmax_and_lse(_scores_one_row(xrow, mrow, sc, causal, q, excluded, offset))[0]


def _excluded(n, mrow_bool=None, key_len=None):
    ex = None
    if mrow_bool is not None:
        ex = np.asarray(mrow_bool) != 0
    if key_len is not None:
        lk = np.arange(n) >= int(key_len)
        ex = lk if ex is None else (ex | lk)
    return ex


def forward_row(xrow, dtype, mrow=None, scale=1.0, is_causal=False, q=0, mask_kind="additive",
                key_len=None, causal_offset=0):
    """Forward of one typed row of x (length Sk) with its mask row or None.

    ``q`` is the row's query position; with ``is_causal`` keys k > q +
    ``causal_offset`` are excluded. ``mask_kind`` is "additive" (``mrow`` typed
    like x) or "bool" (``mrow`` booleans, nonzero = excluded); ``key_len``
    excludes keys k >= key_len.
    """
    xd = decode(np.asarray(xrow), dtype)
    md, mb = None, None
    if mrow is not None:
        if mask_kind == "additive":
            md = decode(np.asarray(mrow), dtype)
        elif mask_kind == "bool":
            mb = np.asarray(mrow)
        else:
            raise ValueError(f"unknown mask kind {mask_kind!r}")
    if xd.ndim != 1 or any(m is not None and m.shape != xd.shape for m in (md, mb)):
        raise ValueError("rows must be 1-D and of one length")
    return _forward_one_row(xd, md, _fp32(scale), bool(is_causal), int(q),
                            _excluded(xd.shape[0], mb, key_len), int(causal_offset))


def forward_rows(x, dtype, rows, mask=None, scale=1.0, is_causal=False, mask_kind="additive",
                 key_lengths=None):
    """Forward on a list of flat row numbers; returns float64 [len(rows), Sk].

    ``is_causal``: False, True / "top_left" or "bottom_right". ``mask``: 4-D
    with length-1 broadcast axes (additive or boolean per ``mask_kind``).
    ``key_lengths``: one integer per batch, or None.
    """
    x = np.asarray(x)
    if x.ndim != 4:
        raise ValueError("x must be 4-D [B, H, Sq, Sk]")
    B, H, Sq, Sk = x.shape
    _check_mask_shape(mask, x.shape)
    off = causal_offset(is_causal, Sq, Sk)
    maskd = None
    if mask is not None:
        maskd = decode(mask, dtype) if mask_kind == "additive" else np.asarray(mask)
    if key_lengths is not None and len(key_lengths) != B:
        raise ValueError("key_lengths needs one entry per batch")
    sc = _fp32(scale)
    out = np.empty((len(rows), Sk), dtype=np.float64)
    for i, r in enumerate(rows):
        b, h, q = row_index(x.shape, int(r))
        xrow = decode(x[b, h, q, :], dtype)  # decoded per row: memory stays bounded
        mrow = _mask_row(maskd, b, h, q) if maskd is not None else None
        add = mrow if mask_kind == "additive" else None
        ex = _excluded(Sk, mrow if mask_kind == "bool" else None,
                       key_lengths[b] if key_lengths is not None else None)
        out[i] = _forward_one_row(xrow, add, sc, off is not None, q, ex, off or 0)
    return out


def forward(x, dtype, mask=None, scale=1.0, is_causal=False, mask_kind="additive",
            key_lengths=None):
    """Forward over the whole tensor; returns float64 of x's shape."""
    x = np.asarray(x)
    B, H, Sq, Sk = x.shape
    rows = range(B * H * Sq)
    return forward_rows(x, dtype, rows, mask, scale, is_causal, mask_kind,
                        key_lengths).reshape(B, H, Sq, Sk)


def _backward_one_row(yrow, dyrow, sc):
    # dot = sum_j dy_j * y_j ; dx_i = scale * y_i * (dy_i - dot)
    dot = float(np.dot(dyrow, yrow))
    return sc * yrow * (dyrow - dot)


def backward_row(yrow, dyrow, dtype, scale=1.0):
    """Backward of one typed row (y and dy of length Sk)."""
    yd = decode(np.asarray(yrow), dtype)
    dyd = decode(np.asarray(dyrow), dtype)
    if yd.ndim != 1 or yd.shape != dyd.shape:
        raise ValueError("rows must be 1-D and of one length")
    return _backward_one_row(yd, dyd, _fp32(scale))


def backward_rows(y, dy, dtype, rows, scale=1.0):
    """Backward on a list of flat row numbers; returns float64 [len(rows), Sk].

    ``y`` is the typed forward output the backward receives and ``dy`` the typed
    upstream gradient; neither the mask nor the causal flag enters the formula.
    """
    y = np.asarray(y)
    dy = np.asarray(dy)
    if y.shape != dy.shape or y.ndim != 4:
        raise ValueError("y and dy must be 4-D and of one shape")
    sc = _fp32(scale)
    out = np.empty((len(rows), y.shape[3]), dtype=np.float64)
    for i, r in enumerate(rows):
        b, h, q = row_index(y.shape, int(r))
        out[i] = _backward_one_row(decode(y[b, h, q, :], dtype),
                                   decode(dy[b, h, q, :], dtype), sc)
    return out


def backward(y, dy, dtype, scale=1.0):
    """Backward over the whole tensor; returns float64 of y's shape."""
    y = np.asarray(y)
    B, H, Sq, Sk = y.shape
    return backward_rows(y, dy, dtype, range(B * H * Sq), scale).reshape(B, H, Sq, Sk)
