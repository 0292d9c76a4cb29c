"""Plain float64 attention: the definition written out, one head at a time.

Test infrastructure only (see the package docstring).  Nothing here is blocked,
fused or reordered: S and P are built in full, as the unfused chain of
operators the pages contrast FlashAttention with (the CSDN post "Flash Attention1", "引言/动机": matmul,
scale, mask, softmax, matmul).

Conventions (the readings of the pages that this oracle fixes):

* S = scale * Q K^T.  The CSDN post "Flash Attention1" writes S = Q K^T; the scale is the
  ``sm_scale`` argument of the kernel call printed on the 51CTO FlashAttention V1/V2 notes ("Sequence
  Parallel"), and callers pass 1/sqrt(d).
* Causal mask: key j is visible to query row i iff j <= i + (Nk - Nq)
  (bottom-right alignment; for Nq == Nk this is the usual lower triangle that
  the 51CTO FlashAttention V1/V2 notes describes when it skips the upper-right blocks).  Masked scores are
  -inf, so they get probability exactly 0.
* L is the natural-log logsumexp of the scaled, masked score row.
* Additive bias (the "+ mask" of the method's formula, taken in general): an
  optional [nq, nk] matrix added to the scaled scores before the causal mask;
  -inf entries remove keys.  It is a constant of the computation (no
  gradient is formed for it).
* Dropout (optional): a multiplier matrix Z [nq, nk] (0 for a dropped score,
  1/keep-probability for a kept one, from ``oracle.philox``) applied to the
  normalised probabilities, O = (P * Z) V.  L stays the logsumexp of the
  scores: dropout acts after the softmax.
* All arithmetic is float64 on inputs converted exactly from bf16, fp16 or fp32.
"""

from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def causal_visible(nq: int, nk: int) -> np.ndarray:
    """Boolean [nq, nk] matrix: True where key j is visible to query row i.

    Bottom-right alignment: j <= i + (nk - nq).  The 51CTO FlashAttention V1/V2 notes ("FlashAttention V2 相比
    V1 有哪些改进") describes the causal case as skipping the blocks above the
    diagonal; for nq == nk the visible set is j <= i.
    """
    i = np.arange(nq)[:, None]
    j = np.arange(nk)[None, :]
    return j <= i + (nk - nq)


def scores(Q, K, scale: float, causal: bool, bias=None) -> np.ndarray:
    """S = scale * Q K^T (+ bias) with -inf at masked positions.  Q [nq, dk], K [nk, dk].

    The CSDN post "Flash Attention1", "Flash Attention" section, first line of the formula (S = Q K^T),
    with the softmax scale applied to the product and the additive mask term
    (``bias`` [nq, nk], optional) added to it.
    """
    Q = _as_f64(Q)
    K = _as_f64(K)
    S = scale * (Q @ K.T)
    if bias is not None:
        S = S + _as_f64(bias)
    if causal:
        S = np.where(causal_visible(Q.shape[0], K.shape[0]), S, -np.inf)
    return S


def softmax_with_lse(S) -> tuple[np.ndarray, np.ndarray]:
    """Row softmax P and natural-log logsumexp L of a score matrix S [nq, nk].

    Safe softmax (the 51CTO FlashAttention V1/V2 notes, "理解FlashAttention核心逻辑": softmax -> safe
    softmax): subtract the row maximum m before exponentiating, so
    P_ij = exp(S_ij - m_i) / l_i with l_i = sum_j exp(S_ij - m_i), and
    L_i = m_i + ln l_i.  Every row must hold at least one finite score.
    """
    S = _as_f64(S)
    m = S.max(axis=1, keepdims=True)
    if not np.all(np.isfinite(m)):
        raise ValueError("every score row needs at least one unmasked entry")
    e = np.exp(S - m)
    l = e.sum(axis=1, keepdims=True)
    P = e / l
    L = (m + np.log(l))[:, 0]
    return P, L


def attention_forward(Q, K, V, scale: float, causal: bool, bias=None, dropout=None):
    """Forward pass for one head: returns (O [nq, dv], L [nq]).

    The CSDN post "Flash Attention1", "Flash Attention" section: S = Q K^T, P = softmax(S), O = P V;
    L as defined in ``softmax_with_lse``.  With ``dropout`` (the multiplier
    matrix Z), O = (P * Z) V: the dropout on P of the V1 algorithm in the
    51CTO FlashAttention V1/V2 notes ("FlashAttention V2 相比 V1 有哪些改进").
    """
    S = scores(Q, K, scale, causal, bias)
    P, L = softmax_with_lse(S)
    if dropout is not None:
        P = P * _as_f64(dropout)
    O = P @ _as_f64(V)
    return O, L


def attention_forward_rows(Q, K, V, rows, scale: float, causal: bool, bias=None, dropout=None):
    """Forward pass for selected query rows of one head (same definition).

    Row i of O and L depends only on Q_i and all of K, V, so a sample of rows
    can be checked at sizes where the full S would be too large to hold.
    """
    Q = _as_f64(Q)
    K = _as_f64(K)
    V = _as_f64(V)
    nq, nk = Q.shape[0], K.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    S = scale * (Q[rows] @ K.T)
    if bias is not None:
        S = S + _as_f64(bias)[rows]
    if causal:
        vis = np.arange(nk)[None, :] <= (rows[:, None] + (nk - nq))
        S = np.where(vis, S, -np.inf)
    P, L = softmax_with_lse(S)
    if dropout is not None:
        P = P * _as_f64(dropout)[rows]
    return P @ V, L


def attention_backward(Q, K, V, dO, scale: float, causal: bool, return_aux: bool = False,
                       bias=None, dropout=None):
    """Gradients of f = sum(dO * O) for one head: returns (dQ, dK, dV).

    P is recomputed from the inputs (the Huawei Cloud post "FlashAttention", section 3: recomputation in the
    backward pass instead of storing the N x N intermediates).  The steps are
    the chain rule through O = P V and the row softmax; the pages name the
    per-row auxiliary D (the 51CTO FlashAttention V1/V2 notes, the ``D`` argument of the backward kernel
    call) but do not print its formula, which the softmax Jacobian fixes:

        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij
        dS = P * (dP - D)            (elementwise, D broadcast along rows)
        dQ = scale * dS K
        dK = scale * dS^T Q

    D is formed from P and dP, not from the shortcut dO_i . O_i that a kernel
    uses; the two agree because O_i = sum_j P_ij V_j.

    With ``dropout`` (Z), O = (P * Z) V, so the chain rule gives
    dV = (P * Z)^T dO and dP = (dO V^T) * Z (the gradient with respect to the
    undropped P); D, dS, dQ and dK then follow as above, and D_i still equals
    dO_i . O_i.
    With ``return_aux`` also returns a dict holding P, L, dP, D and dS.
    """
    Q = _as_f64(Q)
    K = _as_f64(K)
    V = _as_f64(V)
    dO = _as_f64(dO)
    S = scores(Q, K, scale, causal, bias)
    P, L = softmax_with_lse(S)
    Z = None if dropout is None else _as_f64(dropout)
    dV = (P if Z is None else P * Z).T @ dO
    dP = dO @ V.T
    if Z is not None:
        dP = dP * Z
    D = (P * dP).sum(axis=1, keepdims=True)
    dS = P * (dP - D)
    dQ = scale * (dS @ K)
    dK = scale * (dS.T @ Q)
    if return_aux:
        return dQ, dK, dV, {"P": P, "L": L, "dP": dP, "D": D[:, 0], "dS": dS}
    return dQ, dK, dV


def _heads(x):
    x = _as_f64(x)
    lead = x.shape[:-2]
    return x.reshape((-1,) + x.shape[-2:]), lead


def _head_bias(bias, lead):
    """Per-head view of a bias of shape [B or 1, H or 1, nq, nk] (None stays None)."""
    if bias is None:
        return None
    b = np.broadcast_to(_as_f64(bias), tuple(lead) + np.shape(bias)[-2:])
    return b.reshape((-1,) + b.shape[-2:])


def attention_forward_batched(Q, K, V, scale: float, causal: bool, heads=None, bias=None,
                              dropout=None):
    """``attention_forward`` over leading [B, H] dims, one head at a time.

    Q [B, H, nq, d], K and V [B, H, nk, d], bias (optional) [B or 1, H or 1,
    nq, nk], dropout (optional) Z [B, H, nq, nk].  ``heads`` (flat b*H + h
    indices) restricts the work to a sample
    of heads; the result then has shape [len(heads), nq, d] and [len(heads), nq].
    """
    q, lead = _heads(Q)
    k, _ = _heads(K)
    v, _ = _heads(V)
    bh = _head_bias(bias, lead)
    zh = _head_bias(dropout, lead)
    idx = range(q.shape[0]) if heads is None else list(heads)
    O = np.empty((len(idx), q.shape[1], v.shape[2]))
    L = np.empty((len(idx), q.shape[1]))
    for n, h in enumerate(idx):
        O[n], L[n] = attention_forward(q[h], k[h], v[h], scale, causal,
                                       None if bh is None else bh[h],
                                       None if zh is None else zh[h])
    if heads is None:
        return O.reshape(lead + O.shape[1:]), L.reshape(lead + L.shape[1:])
    return O, L


def attention_backward_batched(Q, K, V, dO, scale: float, causal: bool, heads=None, bias=None,
                               dropout=None):
    """``attention_backward`` over leading [B, H] dims, one head at a time."""
    q, lead = _heads(Q)
    k, _ = _heads(K)
    v, _ = _heads(V)
    do, _ = _heads(dO)
    bh = _head_bias(bias, lead)
    zh = _head_bias(dropout, lead)
    idx = range(q.shape[0]) if heads is None else list(heads)
    dQ = np.empty((len(idx),) + q.shape[1:])
    dK = np.empty((len(idx),) + k.shape[1:])
    dV = np.empty((len(idx),) + v.shape[1:])
    for n, h in enumerate(idx):
        dQ[n], dK[n], dV[n] = attention_backward(q[h], k[h], v[h], do[h], scale, causal,
                                                 bias=None if bh is None else bh[h],
                                                 dropout=None if zh is None else zh[h])
    if heads is None:
        return (dQ.reshape(lead + dQ.shape[1:]), dK.reshape(lead + dK.shape[1:]),
                dV.reshape(lead + dV.shape[1:]))
    return dQ, dK, dV
