"""Pins for the CPU oracle: checks that do not come from the oracle itself.

Each check below is written as a function of the oracle's entry points so that
``test_planted_mistakes_are_caught`` can run the same checks against copies of
the oracle with one plausible mistake planted (on the CPU only) and show that
some pin fails for every one of them.

Sources of truth used here:
* tests/golden/hand_derived_attention.json -- exact closed forms derived by
  hand from the CSDN "Flash Attention1" post's formula (the pages print no numeric example);
* the CSDN "Flash Attention1" post's online-softmax walk-through ("例子说明"), re-implemented
  independently as a running max / running sum recurrence;
* softmax identities: rows of P sum to 1, invariance under a per-row shift
  of the scores (the 51CTO FlashAttention V1/V2 notes, "理解FlashAttention核心逻辑": softmax -> safe softmax);
* central finite differences of f = sum(dO * O);
* torch's float64 scaled_dot_product_attention and autograd on the CPU;
* for the additive bias: a per-row constant only shifts L, a bias ln(w_j)
  weights key j by w_j (brute force with math.exp), and -inf entries are the
  same as removing those keys;
* for dropout: finite differences and torch's float64 autograd through
  softmax, the multiplier Z and the product with V; the expectation over
  masks drawn by the generator equals the attention without dropout; and the
  generator itself (Philox4x32-10) against the known-answer vectors published
  with its reference implementation (tests/golden/philox4x32_kat.json).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_derived_attention.json")
PHILOX_KAT = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_kat.json")


# --------------------------------------------------------------------------- helpers

def _val(t):
    a, b, c = (Fraction(s) for s in t)
    return float(a) + float(b) * math.log(2.0) + float(c) * math.log(3.0)


def _arr(x):
    if isinstance(x, list) and len(x) == 3 and all(isinstance(s, str) for s in x):
        return _val(x)
    return [_arr(e) for e in x]


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return a.shape == b.shape and np.all(np.abs(a - b) <= tol * (1.0 + np.abs(b)))


# --------------------------------------------------------------------------- checks
# Every check returns True when the implementation passes it.

def check_golden(fwd, bwd):
    ok = True
    for case in _golden_cases():
        Q, K, V = (np.array(_arr(case[n])) for n in ("Q", "K", "V"))
        scale = float(Fraction(case["scale"]))
        O, L = fwd(Q, K, V, scale, case["causal"])
        ok &= _close(O, _arr(case["O"]), 1e-13) and _close(L, _arr(case["L"]), 1e-13)
        if "dO" in case:
            dO = np.array(_arr(case["dO"]))
            dQ, dK, dV = bwd(Q, K, V, dO, scale, case["causal"])
            ok &= _close(dQ, _arr(case["dQ"]), 1e-13)
            ok &= _close(dK, _arr(case["dK"]), 1e-13)
            ok &= _close(dV, _arr(case["dV"]), 1e-13)
    return bool(ok)


def walkthrough_row(s, V):
    """The CSDN "Flash Attention1" post's 1 x N walk-through, written afresh: one key at a time, keep the
    running max and running sum, renormalise the accumulated output by
    old_sum / new_sum at every step (the page's accumulator is normalised at
    each step, not at the end)."""
    run_max = -math.inf
    run_sum = 0.0
    acc = np.zeros(V.shape[1])
    for j in range(len(s)):
        new_max = max(run_max, s[j])
        run_sum = run_sum * math.exp(run_max - new_max) if run_sum else 0.0
        new_sum = run_sum + math.exp(s[j] - new_max)
        acc = acc * (run_sum / new_sum) + (math.exp(s[j] - new_max) / new_sum) * V[j]
        run_max, run_sum = new_max, new_sum
    return acc, run_max + math.log(run_sum)


def check_walkthrough(fwd, bwd):
    ok = True
    for seed, (n, d) in enumerate([(4, 2), (1, 3), (7, 5), (64, 8), (33, 1)]):
        r = _rng(100 + seed)
        s = r.standard_normal(n) * 3.0
        V = r.standard_normal((n, d))
        acc, lse = walkthrough_row(s, V)
        # one query row whose scores are exactly s: Q = [[1]], K[:, 0] = s, scale 1
        O, L = fwd(np.ones((1, 1)), s[:, None], V, 1.0, False)
        ok &= _close(O[0], acc, 1e-12) and abs(L[0] - lse) <= 1e-12 * (1 + abs(lse))
    return bool(ok)


def check_shift_invariance(fwd, bwd):
    """K' = K + 1 u^T adds scale * Q_i . u to every score of row i: O unchanged,
    L_i shifted by exactly that amount (causal masks do not move)."""
    ok = True
    for causal in (False, True):
        r = _rng(7 + causal)
        Q, K, V = r.standard_normal((5, 4)), r.standard_normal((7, 4)), r.standard_normal((7, 3))
        u = r.standard_normal(4)
        scale = 0.37
        O, L = fwd(Q, K, V, scale, causal)
        O2, L2 = fwd(Q, K + u[None, :], V, scale, causal)
        ok &= _close(O2, O, 1e-12) and _close(L2, L + scale * (Q @ u), 1e-12)
    return bool(ok)


def check_closed_forms(fwd, bwd):
    ok = True
    r = _rng(11)
    # one key: O = V_0, L = S_00 (causal and not)
    for causal in (False, True):
        Q, K, V = r.standard_normal((1, 6)), r.standard_normal((1, 6)), r.standard_normal((1, 4))
        O, L = fwd(Q, K, V, 0.5, causal)
        ok &= _close(O, V, 1e-14) and _close(L, [0.5 * float(Q[0] @ K[0])], 1e-14)
    # causal row 0 with Nq == Nk sees only key 0
    Q, K, V = r.standard_normal((6, 3)), r.standard_normal((6, 3)), r.standard_normal((6, 2))
    O, L = fwd(Q, K, V, 0.8, True)
    ok &= _close(O[0], V[0], 1e-14) and _close(L[0], 0.8 * float(Q[0] @ K[0]), 1e-14)
    # all keys equal: uniform weights -> mean of V (non-causal), prefix means (causal)
    k = r.standard_normal(3)
    K = np.tile(k, (6, 1))
    O, L = fwd(Q, K, V, 0.8, False)
    ok &= _close(O, np.tile(V.mean(axis=0), (6, 1)), 1e-13)
    ok &= _close(L, 0.8 * (Q @ k) + math.log(6), 1e-13)
    O, L = fwd(Q, K, V, 0.8, True)
    prefix = np.cumsum(V, axis=0) / np.arange(1, 7)[:, None]
    ok &= _close(O, prefix, 1e-13) and _close(L, 0.8 * (Q @ k) + np.log(np.arange(1, 7)), 1e-13)
    return bool(ok)


def _f(fwd, Q, K, V, dO, scale, causal):
    O, _ = fwd(Q, K, V, scale, causal)
    return float((O * dO).sum())


def check_finite_differences(fwd, bwd):
    ok = True
    h = 1e-6
    shapes = [(1, 1, 2), (3, 3, 2), (5, 5, 3), (3, 5, 3), (2, 4, 2)]
    for causal in (False, True):
        for n, (nq, nk, d) in enumerate(shapes):
            if causal and nq > nk:
                continue
            r = _rng(200 + n + 10 * causal)
            Q, K, V, dO = (r.standard_normal(s) for s in ((nq, d), (nk, d), (nk, d), (nq, d)))
            scale = 0.6
            got = bwd(Q, K, V, dO, scale, causal)
            for which, X in enumerate((Q, K, V)):
                num = np.zeros_like(X)
                for idx in np.ndindex(X.shape):
                    args = [Q.copy(), K.copy(), V.copy()]
                    args[which][idx] += h
                    fp = _f(fwd, *args, dO, scale, causal)
                    args[which][idx] -= 2 * h
                    fm = _f(fwd, *args, dO, scale, causal)
                    num[idx] = (fp - fm) / (2 * h)
                g = np.asarray(got[which])
                if g.shape != num.shape:
                    return False
                err = np.abs(g - num).max() / max(np.abs(num).max(), 1e-30)
                ok &= err <= 1e-6
    return bool(ok)


def check_gradient_identities(fwd, bwd):
    ok = True
    for causal in (False, True):
        r = _rng(31 + causal)
        Q, K, V, dO = (r.standard_normal(s) for s in ((9, 4), (9, 4), (9, 3), (9, 3)))
        dQ, dK, dV = bwd(Q, K, V, dO, 0.5, causal)
        O, _ = fwd(Q, K, V, 0.5, causal)
        ok &= _close(dV.sum(axis=0), dO.sum(axis=0), 1e-12)       # sum_j dV_j = sum_i dO_i
        ok &= np.abs(dK.sum(axis=0)).max() <= 1e-12 * (1 + np.abs(dK).max())  # sum_j dK_j = 0
    return bool(ok)


def _lse_combine(parts):
    Ls = np.stack([p[1] for p in parts])
    M = Ls.max(axis=0)
    L = M + np.log(np.exp(Ls - M).sum(axis=0))
    O = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    return O, L


def check_split_combine(fwd, bwd):
    """Attention over key chunks, merged by their logsumexps, equals attention
    over all keys (the Flash-Decoding reduction of the 51CTO FlashAttention V1/V2 notes, "Sequence
    Parallel", final paragraph)."""
    ok = True
    r = _rng(41)
    Q, K, V = r.standard_normal((3, 5)), r.standard_normal((20, 5)), r.standard_normal((20, 4))
    O, L = fwd(Q, K, V, 0.45, False)
    for cuts in ([10], [1, 7, 19], [5, 10, 15]):
        edges = [0] + cuts + [20]
        parts = [fwd(Q, K[a:b], V[a:b], 0.45, False) for a, b in zip(edges[:-1], edges[1:])]
        Oc, Lc = _lse_combine(parts)
        ok &= _close(Oc, O, 1e-12) and _close(Lc, L, 1e-12)
    return bool(ok)


def _torch_ref(Q, K, V, dO, scale, causal):
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    mask = None
    if causal:
        nq, nk = q.shape[0], k.shape[0]
        mask = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None, None], k[None, None], v[None, None], attn_mask=mask, scale=scale)[0, 0]
    o.backward(torch.tensor(dO, dtype=torch.float64))
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def check_torch_library(fwd, bwd):
    ok = True
    for n, (nq, nk, d, causal) in enumerate([(8, 8, 16, False), (8, 8, 16, True), (5, 12, 8, True),
                                            (12, 5, 8, False), (33, 47, 4, True)]):
        r = _rng(300 + n)
        Q, K, V, dO = (r.standard_normal(s) for s in ((nq, d), (nk, d), (nk, d), (nq, d)))
        scale = 1.0 / math.sqrt(d)
        O_t, dQ_t, dK_t, dV_t = _torch_ref(Q, K, V, dO, scale, causal)
        O, _ = fwd(Q, K, V, scale, causal)
        dQ, dK, dV = bwd(Q, K, V, dO, scale, causal)
        ok &= _close(O, O_t, 1e-10) and _close(dQ, dQ_t, 1e-10)
        ok &= _close(dK, dK_t, 1e-10) and _close(dV, dV_t, 1e-10)
    return bool(ok)


def check_brute_force(fwd, bwd):
    """Plain Python loops with math.exp, no max shift, on tiny inputs."""
    ok = True
    for n, (nq, nk, d, causal) in enumerate([(3, 3, 2, True), (2, 5, 3, True), (4, 2, 2, False)]):
        r = _rng(400 + n)
        Q, K, V = r.standard_normal((nq, d)), r.standard_normal((nk, d)), r.standard_normal((nk, 2))
        O_ref = np.zeros((nq, 2))
        L_ref = np.zeros(nq)
        for i in range(nq):
            w = []
            for j in range(nk):
                if causal and j > i + (nk - nq):
                    w.append(0.0)
                else:
                    w.append(math.exp(0.7 * sum(Q[i, t] * K[j, t] for t in range(d))))
            tot = sum(w)
            L_ref[i] = math.log(tot)
            for j in range(nk):
                O_ref[i] += (w[j] / tot) * V[j]
        O, L = fwd(Q, K, V, 0.7, causal)
        ok &= _close(O, O_ref, 1e-13) and _close(L, L_ref, 1e-13)
    return bool(ok)


def check_bias_row_constant(fwd, bwd):
    """A bias constant along each row leaves O and the gradients unchanged and
    adds that constant to L (softmax is invariant to a per-row shift)."""
    ok = True
    for n, (nq, nk, causal) in enumerate([(6, 6, True), (4, 9, False), (5, 7, True)]):
        r = _rng(500 + n)
        Q, K, V, dO = r.standard_normal((nq, 4)), r.standard_normal((nk, 4)), \
            r.standard_normal((nk, 3)), r.standard_normal((nq, 3))
        c = r.standard_normal(nq) * 2.0
        bias = np.repeat(c[:, None], nk, axis=1)
        O0, L0 = fwd(Q, K, V, 0.6, causal)
        O1, L1 = fwd(Q, K, V, 0.6, causal, bias=bias)
        ok &= _close(O1, O0, 1e-12) and _close(L1, L0 + c, 1e-12)
        g0 = bwd(Q, K, V, dO, 0.6, causal)
        g1 = bwd(Q, K, V, dO, 0.6, causal, bias=bias)
        ok &= all(_close(a, b, 1e-11) for a, b in zip(g1, g0))
    return bool(ok)


def check_bias_log_weights(fwd, bwd):
    """bias_ij = ln w_j weights key j by w_j: brute force with math.exp."""
    ok = True
    for n, (nq, nk, causal) in enumerate([(3, 4, False), (4, 4, True), (2, 5, True)]):
        r = _rng(520 + n)
        Q, K, V = r.standard_normal((nq, 2)), r.standard_normal((nk, 2)), r.standard_normal((nk, 2))
        w = r.random(nk) + 0.1
        bias = np.tile(np.log(w)[None, :], (nq, 1))
        O_ref, L_ref = np.zeros((nq, 2)), np.zeros(nq)
        for i in range(nq):
            e = [0.0 if (causal and j > i + (nk - nq)) else
                 w[j] * math.exp(0.8 * sum(Q[i, t] * K[j, t] for t in range(2))) for j in range(nk)]
            L_ref[i] = math.log(sum(e))
            for j in range(nk):
                O_ref[i] += e[j] / sum(e) * V[j]
        O, L = fwd(Q, K, V, 0.8, causal, bias=bias)
        ok &= _close(O, O_ref, 1e-13) and _close(L, L_ref, 1e-13)
    return bool(ok)


def check_bias_neg_inf_drops_keys(fwd, bwd):
    """-inf bias entries on a set of keys give the attention over the other
    keys; the removed keys get zero dK and dV."""
    ok = True
    r = _rng(540)
    nq, nk = 5, 9
    Q, K, V, dO = r.standard_normal((nq, 4)), r.standard_normal((nk, 4)), r.standard_normal((nk, 3)), \
        r.standard_normal((nq, 3))
    keep = np.array([1, 0, 1, 1, 0, 0, 1, 0, 1], dtype=bool)
    bias = np.where(keep[None, :], 0.0, -np.inf) * np.ones((nq, 1))
    O, L = fwd(Q, K, V, 0.5, False, bias=bias)
    O_r, L_r = fwd(Q, K[keep], V[keep], 0.5, False)
    ok &= _close(O, O_r, 1e-12) and _close(L, L_r, 1e-12)
    dQ, dK, dV = bwd(Q, K, V, dO, 0.5, False, bias=bias)
    dQ_r, dK_r, dV_r = bwd(Q, K[keep], V[keep], dO, 0.5, False)
    ok &= _close(dQ, dQ_r, 1e-11) and _close(dK[keep], dK_r, 1e-11) and _close(dV[keep], dV_r, 1e-11)
    ok &= bool(np.all(dK[~keep] == 0) and np.all(dV[~keep] == 0))
    return bool(ok)


def _torch_ref_bias(Q, K, V, dO, scale, causal, bias):
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    m = torch.tensor(bias, dtype=torch.float64)
    if causal:
        nq, nk = q.shape[0], k.shape[0]
        vis = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
        m = m.masked_fill(~vis, float("-inf"))
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None, None], k[None, None], v[None, None], attn_mask=m[None, None], scale=scale)[0, 0]
    o.backward(torch.tensor(dO, dtype=torch.float64))
    return o.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def check_bias_torch_library(fwd, bwd):
    """torch's float64 attention with an additive float mask, and its autograd."""
    ok = True
    for n, (nq, nk, d, causal) in enumerate([(8, 8, 16, False), (8, 8, 16, True), (5, 12, 8, True)]):
        r = _rng(560 + n)
        Q, K, V, dO = (r.standard_normal(s) for s in ((nq, d), (nk, d), (nk, d), (nq, d)))
        bias = r.standard_normal((nq, nk)) * 1.5
        scale = 1.0 / math.sqrt(d)
        O_t, dQ_t, dK_t, dV_t = _torch_ref_bias(Q, K, V, dO, scale, causal, bias)
        O, _ = fwd(Q, K, V, scale, causal, bias=bias)
        dQ, dK, dV = bwd(Q, K, V, dO, scale, causal, bias=bias)
        ok &= _close(O, O_t, 1e-10) and _close(dQ, dQ_t, 1e-10)
        ok &= _close(dK, dK_t, 1e-10) and _close(dV, dV_t, 1e-10)
    return bool(ok)


def _mask(r, nq, nk, keep=0.6):
    """A dropout multiplier with both kept (1/keep) and dropped (0) entries."""
    return np.where(r.random((nq, nk)) < keep, 1.0 / keep, 0.0)


def check_dropout_finite_differences(fwd, bwd):
    """With the multiplier Z fixed, the backward is the gradient of sum(dO * O)."""
    ok = True
    h = 1e-6
    for n, (nq, nk, d, causal) in enumerate([(3, 3, 2, False), (4, 4, 2, True), (3, 5, 3, True)]):
        r = _rng(700 + n)
        Q, K, V, dO = (r.standard_normal(s) for s in ((nq, d), (nk, d), (nk, d), (nq, d)))
        Z = _mask(r, nq, nk)
        scale = 0.7
        got = bwd(Q, K, V, dO, scale, causal, dropout=Z)
        for which, X in enumerate((Q, K, V)):
            num = np.zeros_like(X)
            for idx in np.ndindex(X.shape):
                args = [Q.copy(), K.copy(), V.copy()]
                args[which][idx] += h
                fp = float((fwd(*args, scale, causal, dropout=Z)[0] * dO).sum())
                args[which][idx] -= 2 * h
                fm = float((fwd(*args, scale, causal, dropout=Z)[0] * dO).sum())
                num[idx] = (fp - fm) / (2 * h)
            err = np.abs(np.asarray(got[which]) - num).max() / max(np.abs(num).max(), 1e-30)
            ok &= err <= 1e-6
    return bool(ok)


def _torch_ref_dropout(Q, K, V, dO, scale, causal, Z):
    q, k, v = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    s = scale * (q @ k.T)
    if causal:
        nq, nk = s.shape
        vis = torch.ones(nq, nk, dtype=torch.bool).tril(diagonal=nk - nq)
        s = s.masked_fill(~vis, float("-inf"))
    lse = torch.logsumexp(s, dim=1)
    o = (torch.softmax(s, dim=1) * torch.tensor(Z, dtype=torch.float64)) @ v
    o.backward(torch.tensor(dO, dtype=torch.float64))
    return (o.detach().numpy(), lse.detach().numpy(), q.grad.numpy(), k.grad.numpy(),
            v.grad.numpy())


def check_dropout_torch_library(fwd, bwd):
    """torch's float64 softmax, the multiplier and the product with V, with autograd."""
    ok = True
    for n, (nq, nk, d, causal) in enumerate([(8, 8, 16, False), (8, 8, 16, True), (5, 12, 8, True)]):
        r = _rng(720 + n)
        Q, K, V, dO = (r.standard_normal(s) for s in ((nq, d), (nk, d), (nk, d), (nq, d)))
        Z = _mask(r, nq, nk, keep=0.75)
        scale = 1.0 / math.sqrt(d)
        O_t, L_t, dQ_t, dK_t, dV_t = _torch_ref_dropout(Q, K, V, dO, scale, causal, Z)
        O, L = fwd(Q, K, V, scale, causal, dropout=Z)
        dQ, dK, dV = bwd(Q, K, V, dO, scale, causal, dropout=Z)
        ok &= _close(O, O_t, 1e-10) and _close(L, L_t, 1e-10) and _close(dQ, dQ_t, 1e-10)
        ok &= _close(dK, dK_t, 1e-10) and _close(dV, dV_t, 1e-10)
    return bool(ok)


def check_dropout_expectation(fwd, bwd):
    """Averaged over masks drawn by the generator, O and the gradients are those
    without dropout (the multiplier 256/T makes each kept score unbiased)."""
    nq, nk, d, p, n = 4, 8, 3, 0.5, 4000
    r = _rng(740)
    Q, K, V, dO = (r.standard_normal(s) for s in ((nq, d), (nk, d), (nk, d), (nq, d)))
    Zs = np.stack([oracle.dropout_multiplier(nq, nk, p, seed=1234, offset=t, bh=0)
                   for t in range(n)])
    O0, L0 = fwd(Q, K, V, 0.5, False)
    g0 = bwd(Q, K, V, dO, 0.5, False)
    Os = np.stack([fwd(Q, K, V, 0.5, False, dropout=Z)[0] for Z in Zs])
    gs = [np.stack(x) for x in zip(*(bwd(Q, K, V, dO, 0.5, False, dropout=Z) for Z in Zs))]
    ok = True
    for mean_of, samples, exact in [(Os.mean(0), Os, O0)] + [(g.mean(0), g, e) for g, e in zip(gs, g0)]:
        sem = samples.std(0) / math.sqrt(n)  # standard error of the mean, per element
        ok &= bool(np.all(np.abs(mean_of - exact) <= 5.0 * sem + 1e-12))
    return bool(ok)


ALL_CHECKS = [check_golden, check_walkthrough, check_shift_invariance, check_closed_forms,
              check_finite_differences, check_gradient_identities, check_split_combine,
              check_torch_library, check_brute_force, check_bias_row_constant,
              check_bias_log_weights, check_bias_neg_inf_drops_keys, check_bias_torch_library,
              check_dropout_finite_differences, check_dropout_torch_library,
              check_dropout_expectation]


# --------------------------------------------------------------------------- tests

@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    assert check(oracle.attention_forward, oracle.attention_backward)


def test_walkthrough_matches_two_pass_softmax():
    """The CSDN post "Flash Attention1" walk-through (online, normalised per step) equals the two-pass
    softmax followed by the product with V, at N = 4, d = 2 as on the page."""
    r = _rng(5)
    s, V = r.random(4), r.random((4, 2))
    acc, _ = walkthrough_row(s, V)
    e = np.exp(s - s.max())
    assert np.allclose(acc, (e / e.sum()) @ V, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    r = _rng(9)
    Q, K = r.standard_normal((17, 8)), r.standard_normal((23, 8))
    P, L = oracle.softmax_with_lse(oracle.scores(Q, K, 0.35, causal))
    assert np.abs(P.sum(axis=1) - 1.0).max() <= 1e-12
    assert np.all(P >= 0)
    if causal:
        assert np.all(P[~oracle.causal_visible(17, 23)] == 0.0)


def test_softmax_row_shift_by_constant():
    r = _rng(10)
    S = r.standard_normal((6, 9))
    c = r.standard_normal((6, 1)) * 50
    P, L = oracle.softmax_with_lse(S)
    P2, L2 = oracle.softmax_with_lse(S + c)
    assert np.abs(P2 - P).max() <= 1e-12
    assert np.abs(L2 - (L + c[:, 0])).max() <= 1e-12 * 50


def test_softmax_rejects_fully_masked_row():
    S = np.array([[0.0, -np.inf], [-np.inf, -np.inf]])
    with pytest.raises(ValueError):
        oracle.softmax_with_lse(S)


def test_rows_and_batched_entry_points_agree_with_torch():
    r = _rng(12)
    B, H, N, d = 2, 3, 19, 8
    Q, K, V, dO = (r.standard_normal((B, H, N, d)) for _ in range(4))
    scale = 1 / math.sqrt(d)
    O, L = oracle.attention_forward_batched(Q, K, V, scale, True)
    dQ, dK, dV = oracle.attention_backward_batched(Q, K, V, dO, scale, True)
    for b in range(B):
        for h in range(H):
            O_t, dQ_t, dK_t, dV_t = _torch_ref(Q[b, h], K[b, h], V[b, h], dO[b, h], scale, True)
            assert _close(O[b, h], O_t, 1e-10) and _close(dQ[b, h], dQ_t, 1e-10)
            assert _close(dK[b, h], dK_t, 1e-10) and _close(dV[b, h], dV_t, 1e-10)
    heads = [4, 1]
    Os, Ls = oracle.attention_forward_batched(Q, K, V, scale, True, heads=heads)
    for n, hh in enumerate(heads):
        assert np.array_equal(Os[n], O.reshape(-1, N, d)[hh])
        assert np.array_equal(Ls[n], L.reshape(-1, N)[hh])
    rows = [0, 5, 18]
    Or, Lr = oracle.attention_forward_rows(Q[1, 2], K[1, 2], V[1, 2], rows, scale, True)
    O_t, *_ = _torch_ref(Q[1, 2], K[1, 2], V[1, 2], dO[1, 2], scale, True)
    assert _close(Or, O_t[rows], 1e-10) and _close(Lr, L[1, 2, rows], 1e-12)


def test_batched_bias_broadcasts_over_batch_and_heads():
    """Bias [1, H, nq, nk] and [B, 1, nq, nk] apply to every batch / head."""
    r = _rng(13)
    B, H, N, d = 2, 3, 7, 4
    Q, K, V, dO = (r.standard_normal((B, H, N, d)) for _ in range(4))
    for shape in ((1, H, N, N), (B, 1, N, N), (B, H, N, N)):
        bias = r.standard_normal(shape)
        O, L = oracle.attention_forward_batched(Q, K, V, 0.5, True, bias=bias)
        dQ, dK, dV = oracle.attention_backward_batched(Q, K, V, dO, 0.5, True, bias=bias)
        full = np.broadcast_to(bias, (B, H, N, N))
        for b in range(B):
            for h in range(H):
                Oh, Lh = oracle.attention_forward(Q[b, h], K[b, h], V[b, h], 0.5, True, bias=full[b, h])
                gh = oracle.attention_backward(Q[b, h], K[b, h], V[b, h], dO[b, h], 0.5, True,
                                               bias=full[b, h])
                assert np.array_equal(O[b, h], Oh) and np.array_equal(L[b, h], Lh)
                assert all(np.array_equal(g[b, h], e) for g, e in zip((dQ, dK, dV), gh))


# --------------------------------------------------------------------------- planted mistakes
# Copies of the oracle with one plausible mistake each.  Every one must fail at
# least one pin above.

def _mut_fwd(scale_in_scores=True, visible=None, lse_without_max=False, pv_transposed=False,
             bias_scaled=False, bias_transposed=False, drop_unscaled=False, drop_renormalised=False,
             drop_in_lse=False):
    def scores(Q, K, scale, causal, bias=None):
        S = (scale if scale_in_scores else 1.0) * (Q @ K.T)
        if bias is not None:
            b = np.asarray(bias, float)
            if bias_transposed and b.shape[0] == b.shape[1]:
                b = b.T
            S = S + (scale * b if bias_scaled else b)
        if causal:
            vis = (visible or A.causal_visible)(Q.shape[0], K.shape[0])
            S = np.where(vis, S, -np.inf)
        return S

    def fwd(Q, K, V, scale, causal, bias=None, dropout=None):
        S = scores(np.asarray(Q, float), np.asarray(K, float), scale, causal, bias)
        m = S.max(axis=1, keepdims=True)
        e = np.exp(S - m)
        l = e.sum(axis=1, keepdims=True)
        P = e / l
        L = np.log(l)[:, 0] if lse_without_max else (m + np.log(l))[:, 0]
        if dropout is not None:
            Z = np.asarray(dropout, float)
            if drop_unscaled:
                Z = (Z > 0).astype(float)
            P = P * Z
            if drop_renormalised:
                P = P / P.sum(axis=1, keepdims=True)
            if drop_in_lse:
                L = (m + np.log((e * Z).sum(axis=1, keepdims=True)))[:, 0]
        V = np.asarray(V, float)
        O = (P @ V) if not pv_transposed else (P @ V[::-1])
        return O, L
    return fwd, scores


def _mut_bwd(scores, dv_no_transpose=False, ds_sign=False, dq_no_scale=False,
             dk_wrong_operand=False, d_from_wrong_axis=False, bias_ignored=False,
             drop_not_in_dp=False, drop_not_in_dv=False):
    def bwd(Q, K, V, dO, scale, causal, bias=None, dropout=None):
        Q, K, V, dO = (np.asarray(x, float) for x in (Q, K, V, dO))
        S = scores(Q, K, scale, causal, None if bias_ignored else bias)
        P, _ = A.softmax_with_lse(S)
        Z = np.ones_like(P) if dropout is None else np.asarray(dropout, float)
        Pd = P if drop_not_in_dv else P * Z
        dV = (Pd @ dO) if dv_no_transpose and P.shape[0] == P.shape[1] else Pd.T @ dO
        dP = dO @ V.T
        if not drop_not_in_dp:
            dP = dP * Z
        D = (P * dP).sum(axis=0 if d_from_wrong_axis and P.shape[0] == P.shape[1] else 1,
                         keepdims=True)
        if d_from_wrong_axis and P.shape[0] == P.shape[1]:
            D = D.T
        dS = P * ((D - dP) if ds_sign else (dP - D))
        dQ = (1.0 if dq_no_scale else scale) * (dS @ K)
        dK = scale * ((dS @ Q) if dk_wrong_operand and dS.shape[0] == dS.shape[1] else dS.T @ Q)
        return dQ, dK, dV
    return bwd


def _top_left(nq, nk):
    return np.arange(nk)[None, :] <= np.arange(nq)[:, None]


def _off_by_one(nq, nk):
    return np.arange(nk)[None, :] < np.arange(nq)[:, None] + (nk - nq) + 2


def _mutants():
    f_ok, s_ok = _mut_fwd()
    yield "scale dropped from scores", _mut_fwd(scale_in_scores=False)[0], _mut_bwd(_mut_fwd(scale_in_scores=False)[1])
    f, s = _mut_fwd(visible=_top_left)
    yield "causal mask aligned top-left", f, _mut_bwd(s)
    f, s = _mut_fwd(visible=_off_by_one)
    yield "causal mask off by one", f, _mut_bwd(s)
    yield "logsumexp without the max", _mut_fwd(lse_without_max=True)[0], _mut_bwd(s_ok)
    yield "P V with rows of V permuted", _mut_fwd(pv_transposed=True)[0], _mut_bwd(s_ok)
    yield "dV = P dO (not P^T dO)", f_ok, _mut_bwd(s_ok, dv_no_transpose=True)
    yield "sign of dS flipped", f_ok, _mut_bwd(s_ok, ds_sign=True)
    yield "scale dropped from dQ", f_ok, _mut_bwd(s_ok, dq_no_scale=True)
    yield "dK = dS Q (not dS^T Q)", f_ok, _mut_bwd(s_ok, dk_wrong_operand=True)
    yield "D summed over the wrong axis", f_ok, _mut_bwd(s_ok, d_from_wrong_axis=True)
    f, s = _mut_fwd(bias_scaled=True)
    yield "bias multiplied by the scale", f, _mut_bwd(s)
    f, s = _mut_fwd(bias_transposed=True)
    yield "bias transposed", f, _mut_bwd(s)
    yield "bias left out of the backward", f_ok, _mut_bwd(s_ok, bias_ignored=True)
    yield "dropout mask not scaled by 1/keep", _mut_fwd(drop_unscaled=True)[0], _mut_bwd(s_ok)
    yield "probabilities renormalised after dropout", _mut_fwd(drop_renormalised=True)[0], _mut_bwd(s_ok)
    yield "logsumexp of the dropped probabilities", _mut_fwd(drop_in_lse=True)[0], _mut_bwd(s_ok)
    yield "dropout left out of dP", f_ok, _mut_bwd(s_ok, drop_not_in_dp=True)
    yield "dropout left out of dV", f_ok, _mut_bwd(s_ok, drop_not_in_dv=True)


def test_unmutated_copy_passes_every_pin():
    f, s = _mut_fwd()
    b = _mut_bwd(s)
    for check in ALL_CHECKS:
        assert check(f, b), check.__name__


@pytest.mark.parametrize("name,fwd,bwd", list(_mutants()), ids=[m[0] for m in _mutants()])
def test_planted_mistakes_are_caught(name, fwd, bwd):
    failed = []
    for check in ALL_CHECKS:
        try:
            passed = check(fwd, bwd)
        except Exception:  # a crash also counts as a failed pin
            passed = False
        if not passed:
            failed.append(check.__name__)
    assert failed, f"no pin caught the planted mistake: {name}"


# --------------------------------------------------------------------------- the dropout generator

def _kat_cases():
    with open(PHILOX_KAT) as f:
        rec = json.load(f)
    return [([int(x, 16) for x in c["counter"]], [int(x, 16) for x in c["key"]],
             [int(x, 16) for x in c["out"]]) for c in rec["cases"]]


def _philox_passes_kat(fn):
    for ctr, key, out in _kat_cases():
        got = [int(np.asarray(w)) for w in fn(ctr, key)]
        if got != out:
            return False
    return True


def test_philox_known_answer_vectors():
    assert _philox_passes_kat(oracle.philox4x32)


def test_philox_vectorised_over_counters():
    """A batch of counters gives what the counters give one at a time."""
    ctrs = [np.array([0, 5, 0xFFFFFFFF]), np.array([1, 2, 3]), np.array([7, 0, 9]), 4]
    batch = oracle.philox4x32(ctrs, (11, 12))
    for n in range(3):
        one = oracle.philox4x32([int(ctrs[0][n]), int(ctrs[1][n]), int(ctrs[2][n]), 4], (11, 12))
        assert [int(b[n]) for b in batch] == [int(np.asarray(w)) for w in one]


def _philox_mutant(kind):
    def fn(counter, key, rounds=10):
        c = [int(x) & 0xFFFFFFFF for x in counter]
        k0, k1 = int(key[0]), int(key[1])
        m0, m1 = (0xCD9E8D57, 0xD2511F53) if kind == "multipliers swapped" else (0xD2511F53, 0xCD9E8D57)
        for _ in range(rounds - (1 if kind == "nine rounds" else 0)):
            p0, p1 = m0 * c[0], m1 * c[2]
            hi0, lo0, hi1, lo1 = p0 >> 32, p0 & 0xFFFFFFFF, p1 >> 32, p1 & 0xFFFFFFFF
            if kind == "output words reordered":
                c = [hi0 ^ c[3] ^ k1, lo0, hi1 ^ c[1] ^ k0, lo1]
            else:
                c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
            if kind != "key not bumped":
                k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
        return c
    return fn


@pytest.mark.parametrize("kind", ["multipliers swapped", "nine rounds", "output words reordered",
                                  "key not bumped"])
def test_planted_generator_mistakes_fail_the_known_answers(kind):
    assert _philox_passes_kat(_philox_mutant("none"))
    assert not _philox_passes_kat(_philox_mutant(kind))


def test_dropout_bytes_follow_the_block_layout():
    """Score (i, j) takes byte j mod 4 of word i mod 4 of the call with counter
    (j div 4, i div 4, bh, offset), key (seed low, seed high)."""
    seed, offset, bh = 0x0123456789ABCDEF, 77, 5
    by = oracle.dropout_bytes(9, 11, seed, offset, bh)
    for i in range(9):
        for j in range(11):
            w = oracle.philox4x32([j // 4, i // 4, bh, offset], (seed & 0xFFFFFFFF, seed >> 32))
            assert int(by[i, j]) == (int(np.asarray(w[i % 4])) >> (8 * (j % 4))) & 0xFF


def test_keep_threshold():
    assert oracle.keep_threshold(0.0) == 256
    assert oracle.keep_threshold(0.5) == 128
    assert oracle.keep_threshold(0.1) == 230      # round(230.4)
    assert oracle.keep_threshold(0.998) == 1      # round(0.512)
    for bad in (-0.1, 1.0, 0.999, float("nan")):
        with pytest.raises(ValueError):
            oracle.keep_threshold(bad)


def test_dropout_bytes_are_uniform_and_the_keep_rate_is_t_over_256():
    by = oracle.dropout_bytes(256, 512, seed=42, offset=0, bh=3).ravel()
    n = by.size
    counts = np.bincount(by, minlength=256)
    chi2 = float(((counts - n / 256) ** 2 / (n / 256)).sum())
    assert 150 < chi2 < 370  # 255 degrees of freedom: mean 255, sd 22.6
    for p in (0.1, 0.3, 0.5):
        t = oracle.keep_threshold(p)
        frac = float((by < t).mean())
        q = t / 256
        assert abs(frac - q) <= 5 * math.sqrt(q * (1 - q) / n)
    Z = oracle.dropout_multiplier(256, 512, 0.3, seed=42, offset=0, bh=3)
    assert set(np.unique(Z)) == {0.0, 256.0 / oracle.keep_threshold(0.3)}


def test_dropout_masks_differ_across_heads_offsets_and_seeds():
    a = oracle.dropout_bytes(16, 16, 1, 0, 0)
    for other in (oracle.dropout_bytes(16, 16, 1, 0, 1), oracle.dropout_bytes(16, 16, 1, 1, 0),
                  oracle.dropout_bytes(16, 16, 2, 0, 0), oracle.dropout_bytes(16, 16, 1 << 32, 0, 0)):
        assert (a != other).mean() > 0.9


def test_batched_dropout_uses_the_flat_head_index():
    Z = oracle.dropout_multiplier_batched(2, 3, 5, 9, 0.25, seed=9, offset=4)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(Z[b, h], oracle.dropout_multiplier(5, 9, 0.25, 9, 4, b * 3 + h))
