"""Tolerances of the GPU outputs against the float64 oracle (numpy only).

* fp32: max |y - y_ref| <= 1e-6, and |sum_k y_k - 1| <= 1e-5 for every row
  with at least one unmasked key (sum taken in float64 over the fp32 outputs);
  the backward uses the same 1e-6 absolute bound.
* fp16 / bf16: |y - y_ref| <= 2 ulp of the output dtype at y_ref, per element,
  with ulp_T(v) = 2^(max(floor(log2|v|), e_min) - (p - 1)) (fp16: p = 11,
  e_min = -14; bf16: p = 8, e_min = -126). Same for the backward's dx.
* fp64 (computed in fp64 by the kernels): max |y - y_ref| <= 2^-36 and row
  sums within 2^-33 of 1; backward |dx - dx_ref| <= 2^-36. Derived from the
  arithmetic: the scores carry one rounding (relative 2^-52 of |s|), exp's
  argument s - max an absolute error of about 2^-51 * max|s|, the library exp
  one ulp, and the row sum at most n/256 + 8 sequential and tree additions
  (2^-41 relative for n = 2^20 keys); with |s| < 2^10 that is below 2^-39 of
  y <= 1, and the bound leaves 8x of margin.
* everywhere: where the oracle's value is exactly 0 (masked key, causal-future
  key, fully masked row) the GPU value must be exactly 0.

No torch here: worker processes that check whole workloads import this module.
"""

import numpy as np

F32_ABS = 1e-6
F32_ROWSUM = 1e-5
F64_ABS = 2.0 ** -36
F64_ROWSUM = 2.0 ** -33
ULPS = 2.0
_PREC = {"f16": (11, -14), "bf16": (8, -126)}


def ulp(ref, dtype):
    p, emin = _PREC[dtype]
    a = np.abs(ref)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.where(a > 0, np.maximum(e, emin), emin)
    return np.exp2(e - (p - 1))


def compare(got, ref, dtype, what="", rowsum=False, live_rows=None):
    """Raise AssertionError unless ``got`` (float64 of the typed GPU output)
    matches ``ref`` (oracle float64) to the dtype's tolerance. Returns stats."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite GPU output"
    zero = ref == 0.0
    nz_bad = int(np.count_nonzero(got[zero] != 0.0))
    assert nz_bad == 0, f"{what}: {nz_bad} elements must be exactly 0"
    err = np.abs(got - ref)
    stats = {"max_abs": float(err.max()) if err.size else 0.0}
    if dtype in ("f32", "f64"):
        abs_tol, sum_tol = (F32_ABS, F32_ROWSUM) if dtype == "f32" else (F64_ABS, F64_ROWSUM)
        bad = err > abs_tol
        assert not bad.any(), (f"{what}: max abs err {err.max():.3e} > {abs_tol} "
                               f"({int(bad.sum())} elements)")
        if rowsum and got.size:
            s = got.reshape(-1, got.shape[-1]).sum(axis=1)
            live = ref.reshape(-1, ref.shape[-1]).sum(axis=1) > 0 if live_rows is None else live_rows
            dev = np.abs(s[live] - 1.0)
            stats["max_rowsum_err"] = float(dev.max()) if dev.size else 0.0
            assert (dev <= sum_tol).all(), f"{what}: row sum off by {dev.max():.3e}"
    else:
        u = ulp(ref, dtype)
        r = err / u
        stats["max_ulp"] = float(r.max()) if r.size else 0.0
        bad = r > ULPS
        if bad.any():
            i = np.argmax(r)
            raise AssertionError(f"{what}: {int(bad.sum())} elements beyond {ULPS} ulp; worst "
                                 f"{r.flat[i]:.2f} ulp (got {got.flat[i]!r} want {ref.flat[i]!r})")
    return stats


# ------------------------------------------------------- fused attention
#
# O = sum_k p_k v_k / L with fp32 scores and sums, the probabilities rounded to
# the I/O dtype T (unit roundoff u_T = 2^-11 fp16, 2^-8 bf16) for the P V
# product while L sums them unrounded, and O rounded to T at the end. Per
# element: |O - O_ref| <= u_T * max_k |v_k| (the rounded probabilities) plus
# the fp32 score error (below 2^-20 relative for |scores| < 2^4) plus half an
# ulp of O; the bound allows twice that: 2 u_T max|v| + 2 ulp_T(O_ref). The
# log-sum-exp is fp32: |LSE - LSE_ref| <= 2^-18 (1 + |LSE_ref|). Rows with no
# visible key: O exactly 0 and LSE = -inf.

ATTN_U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def compare_attention(got_o, ref_o, vmax, dtype, what="", got_lse=None, ref_lse=None):
    """``vmax``: per output row, max |v| over the keys of its (batch, kv head),
    broadcastable to O's shape. Returns stats."""
    got = np.asarray(got_o, dtype=np.float64)
    ref = np.asarray(ref_o, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    tol = 2 * ATTN_U[dtype] * np.asarray(vmax, dtype=np.float64) + 2 * ulp(ref, dtype)
    err = np.abs(got - ref)
    bad = err > tol
    stats = {"max_abs": float(err.max()) if err.size else 0.0,
             "max_err_over_tol": float((err / tol).max()) if err.size else 0.0}
    if bad.any():
        i = np.argmax(err / tol)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond tolerance; worst at "
                             f"{np.unravel_index(i, got.shape)}: got {got.flat[i]!r} want "
                             f"{ref.flat[i]!r} tol {tol.flat[i]:.3g}")
    if got_lse is not None:
        gl = np.asarray(got_lse, dtype=np.float64)
        rl = np.asarray(ref_lse, dtype=np.float64)
        none = rl == -np.inf
        assert (gl[none] == -np.inf).all(), f"{what}: LSE of a row without keys must be -inf"
        assert (ref[none] == 0).all() and (got[none] == 0).all(), f"{what}: such a row is zeros"
        d = np.abs(gl[~none] - rl[~none])
        ltol = 2.0 ** -18 * (1 + np.abs(rl[~none]))
        assert (d <= ltol).all(), f"{what}: LSE off by {d.max():.3g}"
        stats["lse_max_abs"] = float(d.max()) if d.size else 0.0
    return stats
