"""Pins for the CPU oracle: each test checks the oracle against something fixed
by the pages or by mathematics, never against a retyped copy of its loops.

Sources: "Kaczmarz Linear Attention" (theoretical derivation: the update is the
orthogonal projection of the decayed state onto {S : S^T k = v}; key
properties: projection, exact line search, normalised gradient step; KLA
update rule), "Gated DeltaNet-2: Decoupling Erase and Write in Linear
Attention" (novelty: reduces to KDA when the erase and write gates collapse to
one scalar, and to Gated DeltaNet without channel-wise decay), "Linear
Attention Architectures ..." (the four delta-rule mixers), "What Matters in
Linearizing Language Models?" (additive and gated linear attention as the
no-erase family).
"""
import json
import os
import random

import numpy as np
import pytest

from oracle import exact, oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _head_arrays(d):
    """Exact-rational head dict -> batched float64 arrays [1,T,1,...]."""
    to = lambda x: None if x is None else np.array(x, dtype=object).astype(np.float64)
    q, k, v = to(d["q"]), to(d["k"]), to(d["v"])
    T = q.shape[0]
    out = dict(q=q[None, :, None], k=k[None, :, None], v=v[None, :, None])
    for g in ("alpha", "beta", "erase_b", "write_w"):
        a = to(d[g])
        out[g] = None if a is None else a.reshape((1, T, 1) + a.shape[1:])
    out["state_in"] = to(d["S0"])[None, None]
    out["eps"] = float(d["eps"])
    return out


def _rel(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _rand(rng, variant, T, dk, dv, unit_keys=True, S0=True):
    q = rng.standard_normal((1, T, 1, dk))
    k = rng.standard_normal((1, T, 1, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, T, 1, dv))
    g = dict(alpha=None, beta=None, erase_b=None, write_w=None)
    if variant in ("gated_deltanet", "kla"):
        g["alpha"] = rng.uniform(0.5, 1.0, (1, T, 1))
    if variant in ("kda", "gdn2"):
        g["alpha"] = rng.uniform(0.5, 1.0, (1, T, 1, dk))
    if variant != "gdn2":
        g["beta"] = rng.uniform(0.05, 1.0, (1, T, 1))
    else:
        g["erase_b"] = rng.uniform(0.0, 1.0, (1, T, 1, dk))
        g["write_w"] = rng.uniform(0.0, 1.0, (1, T, 1, dv))
    s0 = rng.standard_normal((1, 1, dk, dv)) if S0 else None
    return dict(q=q, k=k, v=v, state_in=s0, eps=1e-6 if variant == "kla" else 0.0, **g)


def _run(variant, d, lib=None):
    return oracle.forward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"],
                          beta=d["beta"], erase_b=d["erase_b"],
                          write_w=d["write_w"], eps=d["eps"],
                          state_in=d["state_in"], lib=lib)


def _steps(variant, d):
    """Run token by token through the state arguments; return the list of
    states S_0..S_T (float64 [dk,dv])."""
    T = d["q"].shape[1]
    S = [d["state_in"][0, 0]]
    for t in range(T):
        dt = {key: (val[:, t:t + 1] if isinstance(val, np.ndarray) and key != "state_in" else val)
              for key, val in d.items()}
        dt["state_in"] = S[-1][None, None]
        _, st = _run(variant, dt)
        S.append(st[0, 0])
    return S


# ---------------------------------------------------------------- P1 brute force

@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_exact_rational_brute_force(variant):
    """Oracle == exact unrolled products of the dense per-token affine maps
    (rational inputs, d_k=3 != d_v=2 so a transposed operand shows)."""
    rng = np.random.default_rng(7 + oracle.VARIANTS.index(variant))
    d = exact.random_rational_head(rng, T=6, dk=3, dv=2, variant=variant)
    o_ex, s_ex = exact.brute_force_head(variant, d["q"], d["k"], d["v"], d["alpha"],
                                        d["beta"], d["erase_b"], d["write_w"],
                                        d["eps"], d["S0"])
    arr = _head_arrays(d)
    o, s = _run(variant, arr)
    assert _rel(o[0, :, 0], np.array(o_ex, dtype=np.float64)) < 1e-13
    assert _rel(s[0, 0], np.array(s_ex, dtype=np.float64)) < 1e-13


def test_golden_exact_fixture():
    """Oracle == stored exact values written by tests/golden/make_golden.py."""
    with open(os.path.join(GOLDEN, "exact_rational_T6_dk3_dv2.json")) as f:
        cases = json.load(f)
    from fractions import Fraction
    assert set(c["variant"] for c in cases) == set(oracle.VARIANTS)
    for c in cases:
        F = lambda x: None if x is None else (
            [F(y) for y in x] if isinstance(x, list) else Fraction(x))
        d = {key: F(c["inputs"][key]) for key in c["inputs"]}
        arr = _head_arrays(d)
        o, s = _run(c["variant"], arr)
        o_ref = np.array([[float(Fraction(x)) for x in row] for row in c["o"]])
        s_ref = np.array([[float(Fraction(x)) for x in row] for row in c["S_T"]])
        assert _rel(o[0, :, 0], o_ref) < 1e-13, c["variant"]
        assert _rel(s[0, 0], s_ref) < 1e-13, c["variant"]


@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_numpy_brute_force_d128(variant):
    """Same unrolled products in float64 at the real head size (d_k=128,
    d_v=64), T=6, non-zero initial state."""
    rng = np.random.default_rng(11)
    d = _rand(rng, variant, T=6, dk=128, dv=64, unit_keys=variant != "kla")
    o, s = _run(variant, d)
    sq = lambda a: None if a is None else a[0, :, 0]
    o_ref, s_ref = exact.brute_force_numpy(variant, d["q"][0, :, 0], d["k"][0, :, 0],
                                           d["v"][0, :, 0], sq(d["alpha"]), sq(d["beta"]),
                                           sq(d["erase_b"]), sq(d["write_w"]), d["eps"],
                                           d["state_in"][0, 0])
    assert _rel(o[0, :, 0], o_ref) < 1e-12
    assert _rel(s[0, 0], s_ref) < 1e-12


# ---------------------------------------------------- P2-P4 Kaczmarz properties

def _decayed(variant, d, t, S_prev):
    a = d["alpha"]
    if variant in ("gated_deltanet", "kla"):
        return a[0, t, 0] * S_prev
    if variant in ("kda", "gdn2"):
        return a[0, t, 0][:, None] * S_prev
    return S_prev


def test_kaczmarz_projection_constraint_and_minimality():
    """eta=1, eps=0: S_t^T k_t = v_t exactly, and S_t is the closest state to
    the decayed one under that constraint (minimum-norm solution from lstsq)."""
    rng = np.random.default_rng(3)
    d = _rand(rng, "kla", T=8, dk=16, dv=8, unit_keys=False)
    d["beta"][:] = 1.0
    d["eps"] = 0.0
    S = _steps("kla", d)
    dk, dv = 16, 8
    for t in range(8):
        k, v = d["k"][0, t, 0], d["v"][0, t, 0]
        St = _decayed("kla", d, t, S[t])
        assert np.max(np.abs(S[t + 1].T @ k - v)) < 1e-12 * max(1, np.abs(v).max())
        # Constraint on vec(S) (row-major): for each column j, sum_i k_i S[i,j] = v_j.
        C = np.zeros((dv, dk * dv))
        for j in range(dv):
            C[j, j::dv] = k
        rhs = v - C @ St.reshape(-1)
        delta = np.linalg.lstsq(C, rhs, rcond=None)[0]  # minimum-norm correction
        assert _rel(S[t + 1], St + delta.reshape(dk, dv)) < 1e-12


@pytest.mark.parametrize("variant", ["deltanet", "gated_deltanet", "kda", "kla"])
def test_exact_line_search_residual_contraction(variant):
    """S_t^T k - v = (1 - beta ||k||^2) (S~^T k - v) for every token."""
    rng = np.random.default_rng(5)
    d = _rand(rng, variant, T=6, dk=12, dv=7, unit_keys=variant != "kla")
    S = _steps(variant, d)
    for t in range(6):
        k, v = d["k"][0, t, 0], d["v"][0, t, 0]
        beta = d["beta"][0, t, 0]
        if variant == "kla":
            beta = beta / (k @ k + d["eps"])
        St = _decayed(variant, d, t, S[t])
        lhs = S[t + 1].T @ k - v
        rhs = (1 - beta * (k @ k)) * (St.T @ k - v)
        assert np.max(np.abs(lhs - rhs)) < 1e-12


def test_normalised_gradient_step_and_rank_one_change():
    """eta=1, eps=0: S_t - S~ is rank one along k_t, equals minus the gradient
    of 1/2 ||S^T k - v||^2 at S~ (numerical gradient) divided by ||k||^2."""
    rng = np.random.default_rng(9)
    d = _rand(rng, "kla", T=4, dk=10, dv=6, unit_keys=False)
    d["beta"][:] = 1.0
    d["eps"] = 0.0
    S = _steps("kla", d)
    for t in range(4):
        k, v = d["k"][0, t, 0], d["v"][0, t, 0]
        St = _decayed("kla", d, t, S[t])
        diff = S[t + 1] - St
        P = np.eye(10) - np.outer(k, k) / (k @ k)
        assert np.max(np.abs(P @ diff)) < 1e-12
        loss = lambda X: 0.5 * np.sum((X.T @ k - v) ** 2)
        g = np.zeros_like(St)
        h = 1e-6
        for i in range(10):
            for j in range(6):
                E = np.zeros_like(St)
                E[i, j] = h
                g[i, j] = (loss(St + E) - loss(St - E)) / (2 * h)
        assert _rel(diff, -g / (k @ k)) < 1e-6


# ------------------------------------------------------------ P5 reductions

def test_variant_reductions():
    """GDN-2(b=w=beta) == KDA; KDA(alpha broadcast) == GDN; GDN(alpha=1) == DN;
    KLA(eta, eps) == GDN(beta = eta / (||k||^2 + eps))."""
    rng = np.random.default_rng(13)
    T, dk, dv = 40, 32, 24
    d = _rand(rng, "kda", T, dk, dv)
    beta = d["beta"]
    g2 = dict(d, beta=None, erase_b=np.repeat(beta[..., None], dk, -1),
              write_w=np.repeat(beta[..., None], dv, -1))
    o1, s1 = _run("kda", d)
    o2, s2 = _run("gdn2", g2)
    assert _rel(o2, o1) < 1e-12 and _rel(s2, s1) < 1e-12

    a_scalar = rng.uniform(0.5, 1.0, (1, T, 1))
    kda = dict(d, alpha=np.repeat(a_scalar[..., None], dk, -1))
    gdn = dict(d, alpha=a_scalar)
    o1, s1 = _run("kda", kda)
    o2, s2 = _run("gated_deltanet", gdn)
    assert _rel(o2, o1) < 1e-12 and _rel(s2, s1) < 1e-12

    o1, s1 = _run("gated_deltanet", dict(d, alpha=np.ones((1, T, 1))))
    o2, s2 = _run("deltanet", dict(d, alpha=None))
    assert _rel(o2, o1) < 1e-12 and _rel(s2, s1) < 1e-12

    kl = _rand(rng, "kla", T, dk, dv, unit_keys=False)
    k = kl["k"]
    beta = kl["beta"] / (np.sum(k * k, axis=-1) + kl["eps"])
    o1, s1 = _run("kla", kl)
    o2, s2 = _run("gated_deltanet", dict(kl, beta=beta, eps=0.0))
    assert _rel(o2, o1) < 1e-12 and _rel(s2, s1) < 1e-12


# --------------------------------------------------------- P6-P8 closed forms

@pytest.mark.parametrize("variant", ["gated_deltanet", "kda"])
def test_pure_decay(variant):
    """beta=0: S_t = Diag(prod alpha) S_0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(17)
    d = _rand(rng, variant, 20, 8, 5)
    d["beta"][:] = 0.0
    o, s = _run(variant, d)
    cum = np.cumprod(d["alpha"][0, :, 0], axis=0)
    S0 = d["state_in"][0, 0]
    for t in range(20):
        St = (cum[t] * S0) if variant == "gated_deltanet" else cum[t][:, None] * S0
        assert np.max(np.abs(o[0, t, 0] - St.T @ d["q"][0, t, 0])) < 1e-13
    assert _rel(s[0, 0], St) < 1e-13


def test_no_erase_is_gated_linear_attention():
    """GDN-2 with b=0 writes w.v without erasing: a masked, decayed q.k^T
    product (gated linear attention), computed here with einsum."""
    rng = np.random.default_rng(19)
    T, dk, dv = 24, 8, 6
    d = _rand(rng, "gdn2", T, dk, dv)
    d["erase_b"][:] = 0.0
    o, s = _run("gdn2", d)
    q, k, v = d["q"][0, :, 0], d["k"][0, :, 0], d["v"][0, :, 0]
    w, a = d["write_w"][0, :, 0], d["alpha"][0, :, 0]
    g = np.cumsum(np.log(a), axis=0)                 # [T, dk]
    decay = np.exp(g[:, None, :] - g[None, :, :])   # [t, s, i]
    mask = np.tril(np.ones((T, T)))
    scores = np.einsum("ti,si,tsi->ts", q, k, decay) * mask
    o_ref = scores @ (w * v) + np.einsum("ti,ij->tj", q * np.exp(g), d["state_in"][0, 0])
    assert _rel(o[0, :, 0], o_ref) < 1e-12
    # alpha = 1 as well: plain additive linear attention.
    d["alpha"][:] = 1.0
    o, _ = _run("gdn2", d)
    o_ref = (np.tril(q @ k.T)) @ (w * v) + q @ d["state_in"][0, 0]
    assert _rel(o[0, :, 0], o_ref) < 1e-12


def test_one_hot_keys_overwrite_rows():
    """DeltaNet, k_t = e_{i_t}, beta = 1: row i_t becomes v_t, the rest stay."""
    rng = np.random.default_rng(23)
    T, dk, dv = 12, 6, 4
    d = _rand(rng, "deltanet", T, dk, dv)
    idx = rng.integers(0, dk, T)
    d["k"][:] = 0.0
    d["k"][0, np.arange(T), 0, idx] = 1.0
    d["beta"][:] = 1.0
    S = _steps("deltanet", d)
    for t in range(T):
        expect = S[t].copy()
        expect[idx[t]] = d["v"][0, t, 0]
        assert np.array_equal(S[t + 1], expect)


def test_stability_long_sequence():
    """Unit keys and beta in (0,1): the erase factor's spectrum lies in
    [1 - beta, 1], so the state stays bounded over a long sequence."""
    rng = np.random.default_rng(29)
    d = _rand(rng, "deltanet", 3000, 16, 16, S0=False)
    o, s = _run("deltanet", d)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    # ||S||_2 grows by at most ||k u^T|| = beta ||v|| per token.
    bound = np.sum(d["beta"][0, :, 0] * np.linalg.norm(d["v"][0, :, 0], axis=-1))
    assert np.linalg.norm(s[0, 0], 2) <= bound
    assert np.max(np.abs(s)) < 50.0


# ------------------------------------------------------------ P10 chaining

@pytest.mark.parametrize("variant", oracle.VARIANTS)
def test_token_by_token_equals_full_sequence(variant):
    rng = np.random.default_rng(31)
    d = _rand(rng, variant, 9, 8, 5, unit_keys=variant != "kla")
    o, s = _run(variant, d)
    S = _steps(variant, d)
    assert _rel(S[-1], s[0, 0]) < 1e-14


def test_heads_are_independent_and_threaded():
    rng = np.random.default_rng(37)
    B, T, H, dk, dv = 2, 17, 3, 8, 4
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = rng.uniform(0, 1, (B, T, H))
    o, s = oracle.forward("deltanet", q, k, v, beta=beta, threads=4)
    for b in range(B):
        for h in range(H):
            o1, s1 = oracle.forward("deltanet", q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                    v[b:b + 1, :, h:h + 1], beta=beta[b:b + 1, :, h:h + 1],
                                    threads=1)
            assert np.array_equal(o[b, :, h], o1[0, :, 0])
            assert np.array_equal(s[b, h], s1[0, 0])
    o2, _ = oracle.forward("deltanet", q, k, v, beta=beta, heads=[(1, 2)])
    assert np.array_equal(o2[1, :, 2], o[1, :, 2]) and np.isnan(o2[0, 0, 0, 0])
