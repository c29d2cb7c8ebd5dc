"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a temporary copy of the oracle's C source
(on the CPU only), builds it, and checks that the exact rational brute-force
pin rejects it for the variant it touches.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import exact, oracle
from tests.test_oracle_pins import _head_arrays, _rel, _run

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

# (name, variant caught, old text, new text, occurrence index)
MUTATIONS = [
    ("sign_of_erase_deltanet", "deltanet",
     "- beta * k[i] * kS[j] + beta * k[i] * v[j]", "+ beta * k[i] * kS[j] + beta * k[i] * v[j]", 0),
    ("transposed_readout", "gated_deltanet",
     "acc += S[i * p->dv + j] * q[i];", "acc += S[j * p->dv + i] * q[i];", 0),
    ("dropped_decay_gdn", "gated_deltanet", "S[i] = alpha * S[i];", "(void)alpha;", 0),
    ("decay_on_value_axis_kda", "kda",
     "S[i * dv + j] = alpha[i] * S[i * dv + j];", "S[i * dv + j] = alpha[j] * S[i * dv + j];", 0),
    ("dropped_write_gate_gdn2", "gdn2", "k[i] * ww[j] * v[j]", "k[i] * v[j]", 0),
    ("erase_gate_on_wrong_side_gdn2", "gdn2",
     "acc += eb[i] * k[i] * S[i * dv + j];", "acc += k[i] * S[i * dv + j];", 0),
    ("dropped_eps_kla", "kla", "knorm2 + p->eps", "knorm2", 0),
    ("unsquared_norm_kla", "kla", "knorm2 += k[i] * k[i];", "knorm2 += k[i] < 0 ? -k[i] : k[i];", 0),
    ("ignored_initial_state", "kda", "if (p->state_in)", "if (0)", 0),
]


def _mutate(text, old, new, occurrence):
    start = -1
    for _ in range(occurrence + 1):
        start = text.index(old, start + 1)
    return text[:start] + new + text[start + len(old):]


def _exact_err(variant, lib):
    rng = np.random.default_rng(101 + oracle.VARIANTS.index(variant))
    d = exact.random_rational_head(rng, T=5, dk=3, dv=2, variant=variant)
    o_ex, s_ex = exact.brute_force_head(variant, d["q"], d["k"], d["v"], d["alpha"],
                                        d["beta"], d["erase_b"], d["write_w"],
                                        d["eps"], d["S0"])
    o, s = _run(variant, _head_arrays(d), lib=lib)
    return max(_rel(o[0, :, 0], np.array(o_ex, dtype=np.float64)),
               _rel(s[0, 0], np.array(s_ex, dtype=np.float64)))


def test_unmutated_copy_passes(tmp_path):
    src = tmp_path / "o.c"
    shutil.copy(SRC, src)
    lib = oracle.load(oracle.build(str(src), str(tmp_path / "lib.so")))
    for v in oracle.VARIANTS:
        assert _exact_err(v, lib) < 1e-13


@pytest.mark.parametrize("name,variant,old,new,occ", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, variant, old, new, occ):
    text = open(SRC).read()
    src = tmp_path / f"{name}.c"
    src.write_text(_mutate(text, old, new, occ))
    lib = oracle.load(oracle.build(str(src), str(tmp_path / f"{name}.so")))
    assert _exact_err(variant, lib) > 1e-6, f"pin missed planted mistake {name}"
