"""Write the exact-rational fixtures used by the oracle pins.

The values come only from ``oracle/exact.py`` (unrolled products of the dense
per-token affine maps, in exact rational arithmetic); nothing here touches the
GPU library.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import exact  # noqa: E402

VARIANTS = ("deltanet", "gated_deltanet", "kda", "gdn2", "kla")


def _s(x):
    if x is None:
        return None
    if isinstance(x, list):
        return [_s(y) for y in x]
    return str(x)


def main():
    cases = []
    for n, variant in enumerate(VARIANTS):
        rng = np.random.default_rng(2024 + n)
        d = exact.random_rational_head(rng, T=6, dk=3, dv=2, variant=variant)
        o, s = exact.brute_force_head(variant, d["q"], d["k"], d["v"], d["alpha"],
                                      d["beta"], d["erase_b"], d["write_w"],
                                      d["eps"], d["S0"])
        cases.append(dict(variant=variant, inputs={key: _s(val) for key, val in d.items()},
                          o=_s(o), S_T=_s(s)))
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                       "exact_rational_T6_dk3_dv2.json")
    with open(out, "w") as f:
        json.dump(cases, f, indent=1)
    print("wrote", out)


if __name__ == "__main__":
    main()
