"""Pins of the oracle's input transforms (q/k L2 normalisation and gate
activations from pre-activations), against closed forms, library routines and
closed forms of the whole recurrence; and planted mistakes that they reject.

Each pin takes the front-end as a parameter, so the planted-mistake cases can
run the same pins on a copy of the module with one function changed.
"""
import types

import numpy as np
import pytest
import torch

from oracle import oracle

RNG = np.random.default_rng(8500)


def _fe(**over):
    """A namespace with the oracle's front-end functions, optionally replaced."""
    ns = types.SimpleNamespace(softplus=oracle.softplus, sigmoid=oracle.sigmoid,
                               l2normalize=oracle.l2normalize, frontend=oracle.frontend)
    for k, v in over.items():
        setattr(ns, k, v)
    return ns


# ---- pins of the pieces ---------------------------------------------------------

def pin_softplus(fe):
    x = np.concatenate([np.linspace(-30, 30, 241), RNG.normal(0, 5, 100)])
    ref = torch.nn.functional.softplus(torch.from_numpy(x), beta=1.0, threshold=1e9).numpy()
    assert np.max(np.abs(fe.softplus(x) - ref) / np.maximum(np.abs(ref), 1e-300)) < 1e-14
    assert abs(fe.softplus(0.0) - np.log(2.0)) < 1e-16
    # softplus(x) - softplus(-x) = x
    assert np.max(np.abs(fe.softplus(x) - fe.softplus(-x) - x)) < 1e-12
    # no overflow far out: softplus(1000) = 1000, softplus(-1000) = e^-1000 ~ 0
    assert fe.softplus(1000.0) == 1000.0 and 0.0 <= fe.softplus(-1000.0) < 1e-300


def pin_sigmoid(fe):
    x = np.concatenate([np.linspace(-40, 40, 321), RNG.normal(0, 5, 100)])
    ref = torch.sigmoid(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(fe.sigmoid(x) - ref)) < 1e-15
    assert fe.sigmoid(0.0) == 0.5
    assert np.max(np.abs(fe.sigmoid(x) + fe.sigmoid(-x) - 1.0)) < 1e-15
    # the derivative of softplus is the sigmoid (central differences)
    h = 1e-5
    xs = np.linspace(-6, 6, 49)
    fd = (oracle.softplus(xs + h) - oracle.softplus(xs - h)) / (2 * h)
    assert np.max(np.abs(fd - fe.sigmoid(xs))) < 1e-9


def pin_l2normalize(fe):
    assert np.allclose(fe.l2normalize(np.array([3.0, 4.0])),
                       np.array([3.0, 4.0]) / np.sqrt(25.0 + oracle.L2NORM_EPS), rtol=0, atol=1e-16)
    assert np.all(fe.l2normalize(np.zeros((2, 5))) == 0.0)
    x = RNG.normal(size=(3, 7, 2, 128)) * RNG.uniform(0.01, 10, size=(3, 7, 2, 1))
    y = fe.l2normalize(x)
    n2 = np.sum(x * x, axis=-1)
    # ||y||^2 = ||x||^2 / (||x||^2 + eps), and y is a positive multiple of x
    assert np.max(np.abs(np.sum(y * y, axis=-1) - n2 / (n2 + oracle.L2NORM_EPS))) < 1e-14
    ratio = y / x
    assert np.all(ratio > 0)
    assert np.max(np.ptp(ratio, axis=-1)) < 1e-15 * np.max(ratio)


# ---- pins of the composition with the recurrence ------------------------------------

def pin_normalised_one_hot_key(fe):
    """DeltaNet with QK_L2NORM and k_t = c e_i: k^ = g e_i with
    g = c / sqrt(c^2 + eps), so row i becomes (1 - beta g^2) S_i + beta g v and
    the other rows stay; the read-out uses q^ = q / sqrt(|q|^2 + eps)."""
    dk, dv, c, beta, i = 6, 3, 0.37, 0.8, 2
    S0 = RNG.normal(size=(1, 1, dk, dv))
    q = RNG.normal(size=(1, 1, 1, dk))
    k = np.zeros((1, 1, 1, dk))
    k[..., i] = c
    v = RNG.normal(size=(1, 1, 1, dv))
    b = np.full((1, 1, 1), beta)
    qn, kn, *_ = fe.frontend("deltanet", q, k, None, b, flags=oracle.QK_L2NORM)
    o, s = oracle.forward("deltanet", qn, kn, v, beta=b, state_in=S0)
    g = c / np.sqrt(c * c + oracle.L2NORM_EPS)
    S1 = S0[0, 0].copy()
    S1[i] = (1 - beta * g * g) * S0[0, 0, i] + beta * g * v[0, 0, 0]
    assert np.max(np.abs(s[0, 0] - S1)) < 1e-14
    qh = q[0, 0, 0] / np.sqrt(np.sum(q * q) + oracle.L2NORM_EPS)
    assert np.max(np.abs(o[0, 0, 0] - S1.T @ qh)) < 1e-14


def pin_raw_decay(fe):
    """With k = 0 nothing is written, so the state only decays:
    S_T = exp(-s sum_t softplus(x_t)) S_0 (softplus from torch)."""
    T, dk, dv, s_scale = 9, 4, 3, 0.37
    x = RNG.normal(size=(1, T, 1)) * 2
    S0 = RNG.normal(size=(1, 1, dk, dv))
    q = RNG.normal(size=(1, T, 1, dk))
    k = np.zeros((1, T, 1, dk))
    v = RNG.normal(size=(1, T, 1, dv))
    eta = RNG.normal(size=(1, T, 1))
    _, k2, a2, b2, *_ = fe.frontend("kla", q, k, x, eta, flags=oracle.RAW_GATES, decay_scale=s_scale)
    o, s = oracle.forward("kla", q, k2, v, alpha=a2, beta=b2, eps=1e-6, state_in=S0)
    sp = torch.nn.functional.softplus(torch.from_numpy(x), threshold=1e9).numpy()
    ref = np.exp(-s_scale * np.sum(sp)) * S0[0, 0]
    assert np.max(np.abs(s[0, 0] - ref)) < 1e-14


def pin_raw_step_size(fe):
    """Exact line search with an activated step: for Gated DeltaNet the
    residual after a token is (1 - sigmoid(x) |k|^2) times the residual before
    it (sigmoid from torch)."""
    dk, dv = 5, 3
    S0 = RNG.normal(size=(1, 1, dk, dv))
    k = RNG.normal(size=(1, 1, 1, dk)) * 0.4
    q = RNG.normal(size=(1, 1, 1, dk))
    v = RNG.normal(size=(1, 1, 1, dv))
    xa, xb = np.array([[[0.3]]]), np.array([[[-0.7]]])
    _, _, a2, b2, *_ = fe.frontend("gated_deltanet", q, k, xa, xb, flags=oracle.RAW_GATES,
                                   decay_scale=1.0)
    _, s = oracle.forward("gated_deltanet", q, k, v, alpha=a2, beta=b2, state_in=S0)
    alpha = float(torch.exp(-torch.nn.functional.softplus(torch.tensor(0.3, dtype=torch.float64))))
    beta = float(torch.sigmoid(torch.tensor(-0.7, dtype=torch.float64)))
    kk = k[0, 0, 0]
    before = (alpha * S0[0, 0]).T @ kk - v[0, 0, 0]
    after = s[0, 0].T @ kk - v[0, 0, 0]
    assert np.max(np.abs(after - (1 - beta * kk @ kk) * before)) < 1e-14


def pin_gdn2_gates(fe):
    """GDN-2 with raw erase and write gates equals GDN-2 on the torch-activated
    gates, and with x_b, x_w -> +inf (gates -> 1) it reduces to KDA with beta=1."""
    B, T, H, dk, dv = 1, 6, 1, 4, 3
    q, k = RNG.normal(size=(B, T, H, dk)), RNG.normal(size=(B, T, H, dk)) * 0.3
    v = RNG.normal(size=(B, T, H, dv))
    xa = RNG.normal(size=(B, T, H, dk))
    xb, xw = RNG.normal(size=(B, T, H, dk)), RNG.normal(size=(B, T, H, dv))
    _, _, a2, _, b2, w2 = fe.frontend("gdn2", q, k, xa, None, xb, xw, flags=oracle.RAW_GATES,
                                      decay_scale=0.5)
    sig = lambda z: torch.sigmoid(torch.from_numpy(z)).numpy()
    alpha = np.exp(-0.5 * torch.nn.functional.softplus(torch.from_numpy(xa), threshold=1e9).numpy())
    assert np.max(np.abs(a2 - alpha)) < 1e-15
    assert np.max(np.abs(b2 - sig(xb))) < 1e-15 and np.max(np.abs(w2 - sig(xw))) < 1e-15
    big = np.full_like(xb, 60.0)
    _, _, a3, _, b3, w3 = fe.frontend("gdn2", q, k, xa, None, big, np.full_like(xw, 60.0),
                                      flags=oracle.RAW_GATES, decay_scale=0.5)
    o1, s1 = oracle.forward("gdn2", q, k, v, alpha=a3, erase_b=b3, write_w=w3)
    o2, s2 = oracle.forward("kda", q, k, v, alpha=a3, beta=np.ones((B, T, H)))
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(s1 - s2)) < 1e-12


PINS = [pin_softplus, pin_sigmoid, pin_l2normalize, pin_normalised_one_hot_key, pin_raw_decay,
        pin_raw_step_size, pin_gdn2_gates]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_frontend_pin(pin):
    pin(_fe())


# ---- planted mistakes ---------------------------------------------------------------

def _frontend_with(**fns):
    """oracle.frontend with some of its helpers replaced."""
    def fe_fn(variant, q, k, alpha=None, beta=None, erase_b=None, write_w=None, flags=0,
              decay_scale=0.0):
        saved = {n: getattr(oracle, n) for n in fns}
        try:
            for n, f in fns.items():
                setattr(oracle, n, f)
            return oracle.frontend(variant, q, k, alpha, beta, erase_b, write_w, flags,
                                   decay_scale)
        finally:
            for n, f in saved.items():
                setattr(oracle, n, f)
    return fe_fn


def _bad_l2_no_eps(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _bad_l2_wrong_axis(x):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=0, keepdims=True) + oracle.L2NORM_EPS)


def _bad_frontend_q_only(variant, q, k, alpha=None, beta=None, erase_b=None, write_w=None,
                         flags=0, decay_scale=0.0):
    q2, k2, *rest = oracle.frontend(variant, q, k, alpha, beta, erase_b, write_w, flags,
                                    decay_scale)
    return (q2, oracle._f64(k), *rest) if flags & oracle.QK_L2NORM else (q2, k2, *rest)


def _bad_frontend_decay_sign(variant, q, k, alpha=None, beta=None, erase_b=None, write_w=None,
                             flags=0, decay_scale=0.0):
    out = list(oracle.frontend(variant, q, k, alpha, beta, erase_b, write_w, flags, decay_scale))
    if flags & oracle.RAW_GATES and alpha is not None:
        out[2] = np.exp(decay_scale * oracle.softplus(alpha))
    return tuple(out)


MISTAKES = [
    ("softplus_of_minus_x", dict(softplus=lambda x: oracle.softplus(-np.asarray(x, float)))),
    ("softplus_without_log1p", dict(softplus=lambda x: np.maximum(np.asarray(x, float), 0.0))),
    ("sigmoid_of_minus_x", dict(sigmoid=lambda x: oracle.sigmoid(-np.asarray(x, float)))),
    ("l2norm_without_eps", dict(l2normalize=_bad_l2_no_eps)),
    ("l2norm_over_wrong_axis", dict(l2normalize=_bad_l2_wrong_axis)),
    ("normalises_q_only", dict(frontend=_bad_frontend_q_only)),
    ("decay_with_wrong_sign", dict(frontend=_bad_frontend_decay_sign)),
]


def _caught(fe):
    for pin in PINS:
        try:
            pin(fe)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError):
            return True
    return False


@pytest.mark.parametrize("name,over", MISTAKES, ids=[m[0] for m in MISTAKES])
def test_frontend_mistake_is_caught(name, over):
    fe_over = dict(over)
    # helpers planted into the module are seen by oracle.frontend itself
    helpers = {k: v for k, v in fe_over.items() if k in ("softplus", "sigmoid", "l2normalize")}
    fe = _fe(**fe_over)
    if helpers:
        fe.frontend = _frontend_with(**helpers)
    with np.errstate(all="ignore"):
        assert _caught(fe), name
