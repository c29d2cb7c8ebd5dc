"""Exact brute force of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

This is the pin for the sequential oracle in ``gdr_oracle.c``.  It does not
follow the oracle's per-variant loops.  It writes every token's update as
the explicit dense affine map of the general gated delta rule,

    S_t = M_t S_{t-1} + k_t u_t^T,    M_t = (I - k_t a_t^T) D_t,
    o_t = S_t^T q_t,

and evaluates the whole sequence as the unrolled sum of products

    S_t = (M_t ... M_1) S_0 + sum_{s<=t} (M_t ... M_{s+1}) k_s u_s^T,

in exact rational arithmetic (``fractions.Fraction``), or in float64 numpy
for larger shapes.  The per-variant erase key a_t, written value u_t and
decay D_t come from the variant definitions:

  DeltaNet        D = I,             a = beta k,  u = beta v
  Gated DeltaNet  D = alpha I,       a = beta k,  u = beta v
  KDA             D = Diag(alpha),   a = beta k,  u = beta v
  GDN-2           D = Diag(alpha),   a = b (.) k, u = w (.) v
  KLA             D = alpha I,       a = beta k,  u = beta v,
                  beta = eta / (||k||^2 + eps)

("Linear Attention Architectures: Mechanisms, Trade-offs, and Cross-Layer
Routing": the four delta-rule mixers; "Gated DeltaNet-2: Decoupling Erase and
Write in Linear Attention": erase gate b_t on the key side and write gate w_t
on the value side, reducing to KDA when both collapse to one scalar;
"Kaczmarz Linear Attention": KLA update rule and step size.)
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _eye(n, one):
    zero = one - one
    return [[one if i == j else zero for j in range(n)] for i in range(n)]


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    zero = A[0][0] - A[0][0]
    out = [[zero for _ in range(p)] for _ in range(n)]
    for i in range(n):
        for l in range(m):
            a = A[i][l]
            if a == 0:
                continue
            row = B[l]
            o = out[i]
            for j in range(p):
                o[j] += a * row[j]
    return out


def _add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def _outer(x, y):
    return [[xi * yj for yj in y] for xi in x]


def token_terms(variant, t, q, k, v, alpha, beta, erase_b, write_w, eps):
    """Return (D, a, u) for token t of one head as Python lists."""
    kt = list(k[t])
    vt = list(v[t])
    dk = len(kt)
    one = kt[0] - kt[0] + 1
    if variant == "deltanet":
        D = _eye(dk, one)
        bt = beta[t]
        a = [bt * x for x in kt]
        u = [bt * x for x in vt]
    elif variant == "gated_deltanet":
        D = [[alpha[t] if i == j else one - one for j in range(dk)] for i in range(dk)]
        bt = beta[t]
        a = [bt * x for x in kt]
        u = [bt * x for x in vt]
    elif variant == "kda":
        D = [[alpha[t][i] if i == j else one - one for j in range(dk)] for i in range(dk)]
        bt = beta[t]
        a = [bt * x for x in kt]
        u = [bt * x for x in vt]
    elif variant == "gdn2":
        D = [[alpha[t][i] if i == j else one - one for j in range(dk)] for i in range(dk)]
        a = [erase_b[t][i] * kt[i] for i in range(dk)]
        u = [write_w[t][j] * vt[j] for j in range(len(vt))]
    elif variant == "kla":
        D = [[alpha[t] if i == j else one - one for j in range(dk)] for i in range(dk)]
        bt = beta[t] / (sum(x * x for x in kt) + eps)
        a = [bt * x for x in kt]
        u = [bt * x for x in vt]
    else:
        raise ValueError(variant)
    return D, a, u


def brute_force_head(variant, q, k, v, alpha=None, beta=None, erase_b=None,
                     write_w=None, eps=0, S0=None):
    """Unrolled-product evaluation for one head.

    Sequences are indexed by token: q[t], k[t] (length dk), v[t] (length dv),
    alpha[t] (scalar or length dk), beta[t], erase_b[t], write_w[t].  Works on
    Fractions (exact) or floats.  Returns (o [T][dv], S_T [dk][dv]).
    """
    T = len(k)
    dk, dv = len(k[0]), len(v[0])
    one = k[0][0] - k[0][0] + 1
    zero = one - one
    if S0 is None:
        S0 = [[zero] * dv for _ in range(dk)]
    Ms, writes = [], []
    for t in range(T):
        D, a, u = token_terms(variant, t, q, k, v, alpha, beta, erase_b, write_w, eps)
        E = _add(_eye(dk, one), [[-x for x in row] for row in _outer(list(k[t]), a)])
        Ms.append(_matmul(E, D))
        writes.append(_outer(list(k[t]), u))
    outs = []
    S_t = None
    for t in range(T):
        # S_t = (M_t..M_1) S0 + sum_s (M_t..M_{s+1}) k_s u_s^T
        prod = _eye(dk, one)
        acc = writes[t]
        for s in range(t - 1, -1, -1):
            prod = _matmul(prod, Ms[s + 1])
            acc = _add(acc, _matmul(prod, writes[s]))
        prod = _matmul(prod, Ms[0])
        S_t = _add(_matmul(prod, S0), acc)
        qt = list(q[t])
        outs.append([sum(S_t[i][j] * qt[i] for i in range(dk)) for j in range(dv)])
    return outs, S_t


def random_rational_head(rng, T, dk, dv, variant, denom=8):
    """Small exact rational inputs for one head (keys scaled into the stable
    region so that |1 - beta ||k||^2| < 1)."""
    def r(lo, hi):
        return Fraction(int(rng.integers(lo * denom, hi * denom + 1)), denom)

    q = [[r(-1, 1) for _ in range(dk)] for _ in range(T)]
    k = [[r(-1, 1) / 2 for _ in range(dk)] for _ in range(T)]
    v = [[r(-2, 2) for _ in range(dv)] for _ in range(T)]
    pos = lambda: Fraction(int(rng.integers(1, denom + 1)), denom)  # (0, 1]
    if variant in ("kda", "gdn2"):
        alpha = [[pos() for _ in range(dk)] for _ in range(T)]
    elif variant in ("gated_deltanet", "kla"):
        alpha = [pos() for _ in range(T)]
    else:
        alpha = None
    beta = [pos() for _ in range(T)] if variant != "gdn2" else None
    erase_b = [[pos() for _ in range(dk)] for _ in range(T)] if variant == "gdn2" else None
    write_w = [[pos() for _ in range(dv)] for _ in range(T)] if variant == "gdn2" else None
    S0 = [[r(-1, 1) for _ in range(dv)] for _ in range(dk)]
    eps = Fraction(1, 64) if variant == "kla" else Fraction(0)
    return dict(q=q, k=k, v=v, alpha=alpha, beta=beta, erase_b=erase_b,
                write_w=write_w, eps=eps, S0=S0)


def brute_force_numpy(variant, q, k, v, alpha=None, beta=None, erase_b=None,
                      write_w=None, eps=0.0, S0=None):
    """Float64 unrolled-product evaluation for one head with numpy arrays
    q [T,dk], k [T,dk], v [T,dv]; same maps as ``brute_force_head``."""
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, dtype=np.float64)
    Ms, W = [], []
    for t in range(T):
        if variant == "deltanet":
            D = np.eye(dk); a = beta[t] * k[t]; u = beta[t] * v[t]
        elif variant == "gated_deltanet":
            D = alpha[t] * np.eye(dk); a = beta[t] * k[t]; u = beta[t] * v[t]
        elif variant == "kda":
            D = np.diag(alpha[t]); a = beta[t] * k[t]; u = beta[t] * v[t]
        elif variant == "gdn2":
            D = np.diag(alpha[t]); a = erase_b[t] * k[t]; u = write_w[t] * v[t]
        elif variant == "kla":
            bt = beta[t] / (k[t] @ k[t] + eps)
            D = alpha[t] * np.eye(dk); a = bt * k[t]; u = bt * v[t]
        else:
            raise ValueError(variant)
        Ms.append((np.eye(dk) - np.outer(k[t], a)) @ D)
        W.append(np.outer(k[t], u))
    o = np.zeros((T, dv))
    S_t = S0
    for t in range(T):
        prod = np.eye(dk)
        acc = W[t].copy()
        for s in range(t - 1, -1, -1):
            prod = prod @ Ms[s + 1]
            acc += prod @ W[s]
        prod = prod @ Ms[0]
        S_t = prod @ S0 + acc
        o[t] = S_t.T @ q[t]
    return o, S_t
