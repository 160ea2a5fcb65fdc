"""Plain float64 reference of fused attention,

    O = softmax(Q K^T * scale + mask) V        (softmax over keys, per query row)

and of its log-sum-exp per row, and the backward (dQ, dK, dV for an upstream
gradient dO). TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources: the pnsm.cn ScaledMaskSoftmax article, sec. 4.4, proposes fusing the
QK^T product into the operator (FlashAttention-style tiling), which removes the
score tensor from memory; the 0539edu.com notes, fused-attention section, fold
the scale and the mask into the score right after the dot product, take the
softmax of each query's row and multiply by V. The step in the middle is
exactly the scaled-masked softmax of ``oracle.softmax`` applied to the rows of
S = Q K^T, so this module builds S and reuses that oracle's score rule
(``_scores_one_row``: scale, additive mask, boolean mask, key lengths, causal
rule) and its normalisation (``_softmax_and_lse``).

Conventions
-----------
* ``q`` [B, H, Sq, D], ``k`` [B, Hk, Sk, D], ``v`` [B, Hk, Sk, Dv] (Dv may
  differ from D) with Hk dividing H: query
  head h reads key/value head h // (H // Hk) (grouped-query attention; Hk = H
  is ordinary multi-head attention).
* Typed arrays and ``dtype`` as in ``oracle.softmax`` (every value decodes to
  float64 exactly); products and sums are float64.
* ``mask`` / ``mask_kind`` / ``key_lengths`` / ``is_causal``: as in
  ``oracle.softmax.forward_rows``, indexed by (b, h, query, key).
* Outputs: O float64 [B, H, Sq, Dv]; LSE float64 [B, H, Sq], the natural log of
  sum_k exp(score_k) over the keys that survive (-inf for a row with none; its
  O row is zeros, the softmax oracle's rule for fully masked rows).
"""


import numpy as np

from . import softmax as S


def kv_head(h, H, Hk):
    """Key/value head read by query head h."""
    if Hk < 1 or H % Hk:
        raise ValueError(f"Hk = {Hk} must divide H = {H}")
    return h // (H // Hk)


def head_scores(qh, kh):
    """S = Q K^T of one head: S[i, j] = q_i . k_j (float64)."""
    return qh @ kh.T


def combine(P, vh):
    """O = P V of one head: O[i] = sum_j P[i, j] v_j (float64)."""
    return P @ vh


def _decode4(a, dtype):
    a = np.asarray(a)
    if a.ndim != 4:
        raise ValueError("q, k and v must be 4-D")
    return S.decode(a, dtype)


def _prepare(q, k, v, dtype, mask, mask_kind):
    qd, kd, vd = _decode4(q, dtype), _decode4(k, dtype), _decode4(v, dtype)
    B, H, Sq, D = qd.shape
    Bk, Hk, Sk, Dk = kd.shape
    if vd.shape[:3] != kd.shape[:3] or Bk != B or Dk != D:
        raise ValueError(f"shapes q {qd.shape}, k {kd.shape}, v {vd.shape} do not match")
    S._check_mask_shape(mask, (B, H, Sq, Sk))
    maskd = None
    if mask is not None:
        maskd = S.decode(mask, dtype) if mask_kind == "additive" else np.asarray(mask)
    return qd, kd, vd, maskd


def _head_probabilities(qh, kh, maskd, b, h, sc, off, mask_kind, key_lengths):
    """(P, LSE) of one (batch, head): the scaled-masked softmax of each row of
    S = Q K^T, by the softmax oracle's score rule and normalisation."""
    scores = head_scores(qh, kh)  # [Sq, Sk]
    Sq, Sk = scores.shape
    P = np.empty((Sq, Sk), dtype=np.float64)
    LSE = np.empty(Sq, dtype=np.float64)
    for i in range(Sq):
        mrow = S._mask_row(maskd, b, h, i) if maskd is not None else None
        add = mrow if mask_kind == "additive" else None
        ex = S._excluded(Sk, mrow if mask_kind == "bool" else None,
                         key_lengths[b] if key_lengths is not None else None)
        s = S._scores_one_row(scores[i], add, sc, off is not None, i, ex, off or 0)
        P[i], LSE[i] = S._softmax_and_lse(s)
    return P, LSE


def probabilities(q, k, dtype, mask=None, scale=1.0, is_causal=False, mask_kind="additive",
                  key_lengths=None):
    """(P, LSE): P [B, H, Sq, Sk] = softmax(Q K^T * scale + mask) over keys, in
    float64, and its log-sum-exp [B, H, Sq]."""
    qd, kd = _decode4(q, dtype), _decode4(k, dtype)
    B, H, Sq, D = qd.shape
    Hk, Sk = kd.shape[1], kd.shape[2]
    if kd.shape[0] != B or kd.shape[3] != D:
        raise ValueError(f"shapes q {qd.shape}, k {kd.shape} do not match")
    S._check_mask_shape(mask, (B, H, Sq, Sk))
    maskd = None
    if mask is not None:
        maskd = S.decode(mask, dtype) if mask_kind == "additive" else np.asarray(mask)
    off = S.causal_offset(is_causal, Sq, Sk)
    sc = S._fp32(scale)
    P = np.empty((B, H, Sq, Sk), dtype=np.float64)
    LSE = np.empty((B, H, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            P[b, h], LSE[b, h] = _head_probabilities(qd[b, h], kd[b, kv_head(h, H, Hk)], maskd,
                                                     b, h, sc, off, mask_kind, key_lengths)
    return P, LSE


def forward(q, k, v, dtype, mask=None, scale=1.0, is_causal=False, mask_kind="additive",
            key_lengths=None):
    """(O, LSE) of the fused attention forward, in float64."""
    qd, kd, vd, maskd = _prepare(q, k, v, dtype, mask, mask_kind)
    B, H, Sq, D = qd.shape
    Hk, Sk, Dv = kd.shape[1], kd.shape[2], vd.shape[3]
    off = S.causal_offset(is_causal, Sq, Sk)
    sc = S._fp32(scale)
    O = np.zeros((B, H, Sq, Dv), dtype=np.float64)
    LSE = np.empty((B, H, Sq), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hk)
            P, LSE[b, h] = _head_probabilities(qd[b, h], kd[b, g], maskd, b, h, sc, off,
                                               mask_kind, key_lengths)
            O[b, h] = combine(P, vd[b, g])
    return O, LSE


def backward(q, k, v, do, dtype, mask=None, scale=1.0, is_causal=False, mask_kind="additive",
             key_lengths=None):
    """(dQ, dK, dV) of L = sum(dO * O), in float64.

    Chain rule through O = P V and P = softmax(S * scale + mask), S = Q K^T:
    dV = P^T dO; dP = dO V^T; the softmax backward of the softmax oracle gives
    dS = scale * P * (dP - sum_j dP_j P_j) row by row (lmnt.cn page sec. 3.3,
    the scale entering as the derivative of S * scale); dQ = dS K; dK = dS^T Q.
    Key/value heads shared by several query heads sum their contributions.
    """
    qd, kd, vd, maskd = _prepare(q, k, v, dtype, mask, mask_kind)
    dod = _decode4(do, dtype)
    B, H, Sq, D = qd.shape
    Hk, Sk = kd.shape[1], kd.shape[2]
    off = S.causal_offset(is_causal, Sq, Sk)
    sc = S._fp32(scale)
    dQ = np.zeros(qd.shape)
    dK = np.zeros(kd.shape)
    dV = np.zeros(vd.shape)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hk)
            P, _ = _head_probabilities(qd[b, h], kd[b, g], maskd, b, h, sc, off, mask_kind,
                                       key_lengths)
            dV[b, g] += P.T @ dod[b, h]
            dP = dod[b, h] @ vd[b, g].T
            dS = np.zeros((Sq, Sk))
            for i in range(Sq):
                dS[i] = S._backward_one_row(P[i], dP[i], sc)
            dQ[b, h] = dS @ kd[b, g]
            dK[b, g] += dS.T @ qd[b, h]
    return dQ, dK, dV
