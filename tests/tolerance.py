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
# The forward computes, per query row i, fp32 scores s_ik = scale q_i.k_k
# (+ mask), exponentials p~_ik = exp(s_ik - m_i) against a reference maximum
# m_i no larger than the row's maximum (so the largest p~ is >= 1), their fp32
# sum L_i, the product acc_id = sum_k RN_T(p~_ik) v_kd with the probabilities
# rounded to the I/O dtype T (unit roundoff u = 2^-11 fp16, 2^-8 bf16) and
# accumulated in fp32, and O_id = RN_T(acc_id / L_i). With the oracle's exact
# probabilities P_ik = p~_ik / L_i and output O, the first-order error terms:
#  * rounding p~ to T: relative u, or an absolute 2^(e_min - p) in the
#    subnormal range, which in units of P is at most u 2^e_min max_k P_ik
#    (because L_i >= 1); so u P'_ik with P'_ik = max(P_ik, 2^e_min max_k P_ik);
#  * the fp32 arithmetic of p~ (relative E_ik): the dot product over D,
#    (D + 4) 2^-24 scale (|q_i|.|k_k|), and the shifted exponent and the
#    exponential, 2^-22 (1 + |s_ik| + |m_i|);
#  * the fp32 accumulation of acc over n_i visible keys, (n_i + 4) 2^-24
#    (P|V|)_id, and of L (the same relative size on O);
#  * the division by L, 2^-22 |O|, and rounding O to T, half an ulp.
# Three checks, each of which a wrong kernel must pass to go unnoticed:
#  1. per element, twice the worst case of all terms aligned, plus 2 ulp;
#  2. the Frobenius norm of the error: the rounding errors of distinct
#     probabilities, sums and outputs are independent and zero-mean (round to
#     nearest), so E ||err||^2 <= sum sigma^2 with sigma^2 the squares of the
#     per-key terms summed over keys; the bound is (1.5 + 4/sqrt(N)) times
#     its root. Rounding the probabilities to a narrower type, or leaving out
#     their rounding's tie handling, moves this by its ratio of unit roundoffs;
#  3. the bias: sum err_id O_id / sum O_id^2 measures a common scaling of O.
#     Round to nearest leaves it at zero up to the noise (4 sigma); a
#     truncating rounding of P scales O by about 1 - 0.72 u. Allowed: u/8.
# The log-sum-exp is fp32: |LSE - LSE_ref| <= 2^-18 (1 + |LSE_ref|). Rows
# with no visible key: O exactly 0 and LSE = -inf.

ATTN_U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
_TMIN = {"f16": 2.0 ** -14, "bf16": 2.0 ** -126}


def attention_forward_bounds(P, lse, q, k, v, o_ref, scale, dtype):
    """Bounds of the fused attention forward's error against the oracle.

    P [B, H, Sq, Sk] and lse [B, H, Sq]: the oracle's probabilities and
    log-sum-exp; q [B, H, Sq, D], k and v [B, Hk, Sk, D(v)] decoded float64;
    o_ref [B, H, Sq, Dv]: the oracle's O. Returns a dict: ``tol`` (per
    element), ``var`` (per-element variance bound sigma^2), ``u``."""
    u = ATTN_U[dtype]
    B, H, Sq, Sk = P.shape
    Hk, D = k.shape[1], k.shape[3]
    group = H // Hk if Hk else 1
    o_ref = np.asarray(o_ref, dtype=np.float64)
    tol = np.zeros(o_ref.shape)
    var = np.zeros(o_ref.shape)
    aq, ak, av = np.abs(q), np.abs(k), np.abs(v)
    for b in range(B):
        for h in range(H):
            g = h // group
            p = P[b, h]
            if p.size == 0:
                continue
            live = p > 0
            fin = np.isfinite(lse[b, h])
            lf = np.where(fin, lse[b, h], 0.0)
            pmax = p.max(axis=1)
            pp = np.where(live, np.maximum(p, _TMIN[dtype] * pmax[:, None]), 0.0)
            logp = np.where(live, np.log(np.where(live, p, 1.0)), 0.0)
            s_abs = np.abs(logp + lf[:, None])              # |masked scaled score|
            m_abs = np.abs(lf + np.log(np.where(pmax > 0, pmax, 1.0)))   # |row maximum|
            E = (2.0 ** -22 * (1 + s_abs + m_abs[:, None])
                 + (D + 4) * 2.0 ** -24 * scale * (aq[b, h] @ ak[b, g].T))
            E = np.where(live, E, 0.0)
            n = live.sum(axis=1)[:, None]
            acc = (n + 4) * 2.0 ** -24
            pv = p @ av[b, g]
            pe = (p * E) @ av[b, g]
            ao = np.abs(o_ref[b, h])
            pE = (p * E).sum(axis=1)[:, None]
            tol[b, h] = 2 * (u * (pp @ av[b, g]) + pe + acc * pv
                             + ao * (pE + acc + 2.0 ** -22))
            var[b, h] = (u ** 2 * ((pp ** 2) @ (av[b, g] ** 2))
                         + ((p * E) ** 2) @ (av[b, g] ** 2)
                         + ao ** 2 * ((p * E) ** 2).sum(axis=1)[:, None]
                         + ((acc * pv) ** 2 + (acc * ao) ** 2) / np.maximum(n, 1)
                         + (2.0 ** -22 * ao) ** 2)
    half = 0.5 * ulp(o_ref, dtype)
    tol = tol + 2 * ulp(o_ref, dtype)
    var = var + half ** 2
    return {"tol": tol, "var": var, "u": u}


def compare_attention(got_o, ref_o, bounds, dtype, what="", got_lse=None, ref_lse=None):
    """Raise unless the GPU's O (float64 of the typed output) meets the three
    forward checks of ``attention_forward_bounds`` and, if given, its LSE the
    fp32 bound. Returns stats (each check's value over its bound)."""
    got = np.asarray(got_o, dtype=np.float64)
    ref = np.asarray(ref_o, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    tol, var, u = bounds["tol"], bounds["var"], bounds["u"]
    err = got - ref
    aerr = np.abs(err)
    bad = aerr > tol
    stats = {"max_abs": float(aerr.max()) if err.size else 0.0,
             "max_err_over_tol": float((aerr / tol).max()) if err.size else 0.0}
    if bad.any():
        i = np.argmax(aerr / tol)
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond tolerance; worst at "
                             f"{np.unravel_index(i, got.shape)}: got {got.flat[i]!r} want "
                             f"{ref.flat[i]!r} tol {tol.flat[i]:.3g}")
    nz = int(np.count_nonzero(var))
    if nz:
        fro = float(np.sqrt((err ** 2).sum()))
        fro_bound = (1.5 + 4.0 / np.sqrt(nz)) * float(np.sqrt(var.sum()))
        stats["fro_over_bound"] = fro / fro_bound
        assert fro <= fro_bound, (f"{what}: ||err||_F = {fro:.4g} above its bound "
                                  f"{fro_bound:.4g}")
        oo = float((ref ** 2).sum())
        if oo > 0:
            bias = float((err * ref).sum())
            allow = u / 8 * oo + 4.0 * float(np.sqrt((ref ** 2 * var).sum()))
            stats["bias"] = bias / oo
            stats["bias_over_bound"] = abs(bias) / allow
            assert abs(bias) <= allow, (f"{what}: O is scaled by 1 + {bias / oo:.3g} "
                                        f"(allowed {allow / oo:.3g})")
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


# -------------------------------------------------- fused attention backward
#
# The backward takes O (dtype T) and the fp32 LSE as inputs, recomputes
# P = exp(s*scale + mask - LSE) in fp32, takes delta_i = sum_d dO_id O_id,
# forms dS = P (dP - delta) with dP = dO V^T in fp32, rounds P and dS to T for
# the products dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q (fp32
# accumulation), and rounds the results to T once. Given O_in and LSE_in, the
# first-order error terms per element, with the oracle's exact P, dP, delta:
#  * P's relative error E_ij: the LSE input's deviation |LSE_in - LSE| plus
#    fp32 rounding of the exponent (2^-22 (1 + |LSE_i| + |z_ij|), z the masked
#    scaled score) and of the score sum (D 2^-24 scale (|Q||K|^T)_ij);
#  * delta's absolute error e_i: |sum_d dO_id (O_in - O)_id| plus the fp32
#    sums of delta and dP (D 2^-24 (|dO_i|.|O_in,i| + ||dO_i||_1 max|v|));
#  * rounding P or dS to T: relative u_T; fp32 accumulation over n terms:
#    n 2^-24 relative to the sum of absolute values (n = Sk for dQ,
#    Sq * group for dK and dV); the final rounding: half an ulp.
# Elementwise (worst case, every rounding error aligned), summed over the
# query heads that share a key/value head, the bound allows twice
#   dQ_id:  scale [ (u + gk) (|dS||K|)_id + ((|dS| o E)|K|)_id + e_i (P|K|)_id ]
#   dK_jd:  scale [ (u + gq) (|dS|^T|Q|)_jd + ((|dS| o E)^T|Q|)_jd + (P^T (e o |Q|))_jd ]
#   dV_jd:  (u + gq) (P^T|dO|)_jd + ((P o E)^T|dO|)_jd
# plus 2 ulp_T of the reference value. With cancellation in the sums this is
# loose (a 1% error in dQ can hide under it), so a second bound applies to
# the whole tensor: the rounding errors of P and dS are independent from
# element to element, so their contribution to ||err||_F is at most
# u sqrt(sum (dS^2 K^2)) (etc.) in expectation; the test allows three times
# the root-sum-square of that and of the final rounding (u |ref|), plus twice
# the Frobenius norm of the remaining (systematic) terms.


def attention_grad_tolerances(P, dP, q, k, do, vmax, lse, scale, dtype, refs, o_in=None,
                              o_ref=None, lse_in=None):
    """(elementwise tolerances (tol_dq, tol_dk, tol_dv), Frobenius bounds
    (rms_dq, rms_dk, rms_dv)) of the attention backward.

    P, dP [B, H, Sq, Sk] (oracle, float64; dP = dO V^T per query head),
    q/do [B, H, Sq, D], k [B, Hk, Sk, D], vmax [B, H] (max |v| over the head's
    keys), lse [B, H, Sq] (oracle), refs = oracle (dQ, dK, dV). o_in / lse_in:
    the O and LSE the backward was given, o_ref: the oracle's O; without them
    O_in is only known to satisfy the forward's bound 2 u max|v| + 2 ulp(O)
    (<= 6 u max|v|) and LSE_in its 2^-18 (1 + |LSE|)."""
    u = ATTN_U[dtype]
    B, H, Sq, Sk = P.shape
    Hk, D = k.shape[1], k.shape[3]
    group = H // Hk
    gk, gq = Sk * 2.0 ** -24, Sq * group * 2.0 ** -24
    aq, ak, ado = np.abs(q), np.abs(k), np.abs(do)
    shape_v = k.shape[:3] + (do.shape[3],)
    # w*: aligned rounding of P / dS (u times sums of absolute values);
    # s*: the other (systematic) terms; r*: expected squared rounding error.
    wq, sq_, rq = np.zeros(q.shape), np.zeros(q.shape), np.zeros(q.shape)
    wk, sk_, rk = np.zeros(k.shape), np.zeros(k.shape), np.zeros(k.shape)
    wv, sv_, rv = np.zeros(shape_v), np.zeros(shape_v), np.zeros(shape_v)
    for b in range(B):
        for h in range(H):
            g = h // group
            p = P[b, h]
            fin = np.isfinite(lse[b, h])
            lz = np.where(fin, np.abs(lse[b, h]), 0.0)
            lsef = np.where(fin, lse[b, h], 0.0)
            delta = (p * dP[b, h]).sum(axis=1)
            ads = p * np.abs(dP[b, h] - delta[:, None])
            live = p > 0
            z = np.where(live, np.abs(np.log(np.where(live, p, 1.0)) + lsef[:, None]), 0.0)
            qk = scale * (aq[b, h] @ ak[b, g].T)
            if lse_in is None:
                dl = 2.0 ** -18 * (1 + lz)
            else:
                dl = np.where(fin, np.abs(np.where(fin, lse_in[b, h], 0.0) - lsef), 0.0)
            E = (dl + 2.0 ** -22 * (1 + lz))[:, None] + 2.0 ** -22 * z + (D + 4) * 2.0 ** -24 * qk
            l1 = ado[b, h].sum(axis=1)
            if o_in is None:
                e = l1 * vmax[b, h] * (6 * u + 2 * D * 2.0 ** -24)
            else:
                e = (np.abs((do[b, h] * (o_in[b, h] - o_ref[b, h])).sum(axis=1))
                     + D * 2.0 ** -24 * ((ado[b, h] * np.abs(o_in[b, h])).sum(axis=1)
                                         + l1 * vmax[b, h]))
            wq[b, h] = u * scale * (ads @ ak[b, g])
            wk[b, g] += u * scale * (ads.T @ aq[b, h])
            wv[b, g] += u * (p.T @ ado[b, h])
            sq_[b, h] = scale * (gk * (ads @ ak[b, g]) + (ads * E) @ ak[b, g]
                                 + e[:, None] * (p @ ak[b, g]))
            sk_[b, g] += scale * (gq * (ads.T @ aq[b, h]) + (ads * E).T @ aq[b, h]
                                  + p.T @ (e[:, None] * aq[b, h]))
            sv_[b, g] += gq * (p.T @ ado[b, h]) + (p * E).T @ ado[b, h]
            rq[b, h] = (u * scale) ** 2 * ((ads ** 2) @ (ak[b, g] ** 2))
            rk[b, g] += (u * scale) ** 2 * ((ads ** 2).T @ (aq[b, h] ** 2))
            rv[b, g] += u ** 2 * ((p ** 2).T @ (ado[b, h] ** 2))
    refs = [np.asarray(r, dtype=np.float64) for r in refs]
    tols = tuple(2 * (w + s_) + 2 * ulp(r, dtype)
                 for w, s_, r in zip((wq, wk, wv), (sq_, sk_, sv_), refs))
    rms = tuple(3 * np.sqrt(rr.sum() + ((u * r) ** 2).sum()) + 2 * np.sqrt((s_ ** 2).sum())
                for rr, s_, r in zip((rq, rk, rv), (sq_, sk_, sv_), refs))
    return tols, rms


def compare_grads(got, ref, tol, what="", rms=None):
    """Raise unless |got - ref| <= tol everywhere and, if given, the Frobenius
    norm of got - ref is at most ``rms``; returns max(err / tol)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    r = err / tol
    if r.size and (r > 1).any():
        i = np.argmax(r)
        raise AssertionError(f"{what}: {int((r > 1).sum())} elements beyond tolerance; worst at "
                             f"{np.unravel_index(i, got.shape)}: got {got.flat[i]!r} want "
                             f"{ref.flat[i]!r} tol {tol.flat[i]:.3g}")
    if rms is not None:
        f = float(np.sqrt((err ** 2).sum()))
        assert f <= rms, f"{what}: ||err||_F = {f:.4g} above its bound {rms:.4g}"
    return float(r.max()) if r.size else 0.0
