"""Pins of the oracle's cross-layer routing quantities ("Linear Attention
Architectures: Mechanisms, Trade-offs, and Cross-Layer Routing", the
cross-layer routing section: a lower layer passes either its value target
(CLVR) or its error (CLER) up to a higher layer's write).

* delta_t, the residual token t writes (S_t = S~_t + k_t delta_t^T), is pinned
  by rebuilding every S_t from the deltas alone, S_t = D_t S_{t-1} + k_t
  delta_t^T, and checking the oracle's own outputs o_t = S_t^T q_t and S_T
  against it (the oracle computes those through its update, not from delta);
  and by the first token from a zero state, where delta = u (beta v, or w (.) v
  for GDN-2, with beta = eta / (|k|^2 + eps) for KLA).
* the routed value v_route enters only through u, and the recurrence is
  linear in (v, S_0) for fixed keys and gates: o(v + r, S_0) = o(v, S_0) +
  o(r, 0).
Planted mistakes in the delta bookkeeping are rejected.
"""
import os
import shutil

import numpy as np
import pytest

from oracle import oracle
from tests.test_oracle_mutations import _mutate
from tests.test_oracle_pins import _rand, _rel

VARIANTS = oracle.VARIANTS
SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")


def _decay(variant, d, t, dk):
    """D_t as a length-dk vector of row factors."""
    if d["alpha"] is None:
        return np.ones(dk)
    a = d["alpha"][0, t, 0]
    return np.full(dk, float(a)) if np.ndim(a) == 0 else np.asarray(a, dtype=np.float64)


def _rebuild(variant, d, delta):
    """States S_1..S_T from S_0 and the deltas alone; returns (o [T, dv], S_T)."""
    q, k = d["q"][0, :, 0], d["k"][0, :, 0]
    T, dk = k.shape
    S = np.array(d["state_in"][0, 0], dtype=np.float64)
    o = []
    for t in range(T):
        S = _decay(variant, d, t, dk)[:, None] * S + np.outer(k[t], delta[0, t, 0])
        o.append(S.T @ q[t])
    return np.array(o), S


def _run(variant, d, lib=None, **kw):
    return oracle.forward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                          erase_b=d["erase_b"], write_w=d["write_w"], eps=d.get("eps", 0.0),
                          state_in=d["state_in"], threads=1, lib=lib, **kw)


def _problem(variant, seed, T=9, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    d = _rand(rng, variant, T, dk, dv)
    d["eps"] = 0.25 if variant == "kla" else 0.0
    return d


def _delta_err(variant, lib=None, seed=7):
    d = _problem(variant, seed + VARIANTS.index(variant))
    o, s, delta = _run(variant, d, lib=lib, want_delta=True)
    o_rb, s_rb = _rebuild(variant, d, delta)
    return max(_rel(o_rb, o[0, :, 0]), _rel(s_rb, s[0, 0]))


@pytest.mark.parametrize("variant", VARIANTS)
def test_delta_rebuilds_every_state(variant):
    assert _delta_err(variant) < 1e-12


@pytest.mark.parametrize("variant", VARIANTS)
def test_first_delta_from_zero_state_is_the_write_value(variant):
    d = _problem(variant, 31)
    d["state_in"] = np.zeros_like(d["state_in"])
    _, _, delta = _run(variant, d, want_delta=True)
    v0, k0 = d["v"][0, 0, 0], d["k"][0, 0, 0]
    if variant == "gdn2":
        u = d["write_w"][0, 0, 0] * v0
    elif variant == "kla":
        u = d["beta"][0, 0, 0] / (k0 @ k0 + d["eps"]) * v0
    else:
        u = d["beta"][0, 0, 0] * v0
    assert _rel(delta[0, 0, 0], u) < 1e-14


@pytest.mark.parametrize("variant", VARIANTS)
def test_routed_value_is_linear(variant):
    d = _problem(variant, 53)
    r = np.random.default_rng(99).standard_normal(d["v"].shape)
    o_routed, s_routed = _run(variant, d, v_route=r)
    o_plain, s_plain = _run(variant, d)
    d0 = dict(d, v=r, state_in=np.zeros_like(d["state_in"]))
    o_r, s_r = _run(variant, d0)
    assert _rel(o_routed, o_plain + o_r) < 1e-12
    assert _rel(s_routed, s_plain + s_r) < 1e-12


# (name, variant, old text, new text, occurrence)
DELTA_MUTATIONS = [
    ("delta_without_beta", "deltanet", "record_delta(p, b, t, h, beta, v, NULL, kS);",
     "record_delta(p, b, t, h, 1.0, v, NULL, kS);", 0),
    ("delta_of_value_not_residual_gdn", "gated_deltanet", "record_delta(p, b, t, h, beta, v, NULL, kS);",
     "record_delta(p, b, t, h, beta, v, NULL, NULL);", 1),
    ("delta_without_write_gate", "gdn2", "record_delta(p, b, t, h, 1.0, v, ww, r);",
     "record_delta(p, b, t, h, 1.0, v, NULL, r);", 0),
    ("delta_sign_kla", "kla", "record_delta(p, b, t, h, beta, e, NULL, NULL);",
     "record_delta(p, b, t, h, -beta, e, NULL, NULL);", 0),
    ("delta_of_value_not_residual_kda", "kda", "record_delta(p, b, t, h, beta, v, NULL, kS);",
     "record_delta(p, b, t, h, beta, v, NULL, NULL);", 2),
]


@pytest.mark.parametrize("name,variant,old,new,occ", DELTA_MUTATIONS, ids=[m[0] for m in DELTA_MUTATIONS])
def test_planted_delta_mistake_is_caught(tmp_path, name, variant, old, new, occ):
    text = open(SRC).read()
    src = tmp_path / f"{name}.c"
    src.write_text(_mutate(text, old, new, occ))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / f"{name}.so")))
    assert _delta_err(variant, lib) > 1e-6, f"pin missed planted mistake {name}"


def test_unmutated_copy_passes_delta_pins(tmp_path):
    src = tmp_path / "o.c"
    shutil.copy(SRC, src)
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "lib.so")))
    for v in VARIANTS:
        assert _delta_err(v, lib) < 1e-12
