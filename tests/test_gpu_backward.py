"""GPU parity of the gradient of the chunked forward (gdr_backward_chunked)
against the gradient oracle (reverse-mode differentiation of the token-by-token
recurrence in float64), on the same seeded inputs and upstream gradients.

Error measure and thresholds as for the forward: per head, max |x - ref| /
max |ref| over the head's entries; float32 inputs 1e-4, bfloat16 inputs 2e-2
(the bf16 path also rounds the chunk factors it reads in the reverse pass)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import VARIANTS, make_inputs, make_upstream_grads
from oracle import backward as oracle_bw
from tests.gpu_common import TOL, announce, rel_err, to_dev

pytestmark = pytest.mark.gpu

# head axes of each gradient: tokens-major inputs [B,T,H,...], state [B,H,dk,dv]
_AXES = dict(q=(0, 2), k=(0, 2), v=(0, 2), alpha=(0, 2), beta=(0, 2), erase_b=(0, 2),
             write_w=(0, 2), state_in=(0, 1))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    binding.lib()


def _check(variant, dtype, B=2, T=200, H=2, dk=128, dv=128, seed=0, state=True,
           d_o=True, d_state=True, heads=None, tol_scale=1.0):
    inp = make_inputs(variant, B, T, H, dk, dv, dtype, seed=seed,
                      state_scale=0.1 if state else 0.0)
    up = make_upstream_grads(B, T, H, dk, dv, dtype, seed=seed + 1000)
    if not d_o:
        up["d_o"] = None
    if not d_state:
        up["d_state_out"] = None
    d = to_dev(inp)
    du = to_dev(up)
    g = binding.backward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                         erase_b=d["erase_b"], write_w=d["write_w"], eps=d["eps"],
                         state_in=d["state_in"], d_o=du["d_o"], d_state_out=du["d_state_out"])
    torch.cuda.synchronize()
    ref = oracle_bw.backward(variant, inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                             beta=inp["beta"], erase_b=inp["erase_b"], write_w=inp["write_w"],
                             eps=inp["eps"], state_in=inp["state_in"], d_o=up["d_o"],
                             d_state_out=up["d_state_out"], heads=heads)
    tol = TOL[d["q"].dtype] * tol_scale
    errs = {}
    for name, r in ref.items():
        if r is None:
            assert g[name] is None, name
            continue
        x = g[name].cpu().numpy()
        ax = _AXES[name]
        if heads is None:
            errs[name] = rel_err(x, r, ax)
        else:
            sel = [(slice(b, b + 1), slice(None), slice(h, h + 1)) if ax == (0, 2)
                   else (slice(b, b + 1), slice(h, h + 1)) for b, h in heads]
            errs[name] = max(rel_err(x[s], r[s], ax) for s in sel)
    announce(f"grad {variant} {dtype} B={B} T={T} H={H} dk={dk} dv={dv}: " +
             " ".join(f"{n}={e:.1e}" for n, e in errs.items()) + f" (tol {tol})")
    bad = {n: e for n, e in errs.items() if not e < tol}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_backward_matches_oracle(variant, dtype):
    """Four chunks, the last one ragged; initial state and both upstream gradients."""
    _check(variant, dtype, seed=VARIANTS.index(variant) * 13 + (dtype == "bf16"))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("variant", ["gated_deltanet", "kda", "gdn2", "kla"])
def test_backward_head_sizes(variant, dk, dv):
    _check(variant, "fp32", B=1, T=130, H=3, dk=dk, dv=dv, seed=31)


@pytest.mark.parametrize("T", [1, 63, 64, 65])
@pytest.mark.parametrize("variant", ["deltanet", "kda", "kla"])
def test_backward_short_and_ragged(variant, T):
    _check(variant, "fp32", B=2, T=T, H=1, seed=40 + T)


@pytest.mark.parametrize("variant", ["gated_deltanet", "gdn2"])
def test_backward_upstream_variants(variant):
    """Zero initial state; only one of the two upstream gradients."""
    _check(variant, "fp32", T=100, state=False, d_state=False, seed=51)
    _check(variant, "fp32", T=100, state=False, d_o=False, seed=52)


@pytest.mark.parametrize("variant", ["kda", "kla"])
def test_backward_long_sampled_heads(variant):
    """A longer sequence (64 chunks) in bf16; the oracle checks sampled heads."""
    _check(variant, "bf16", B=1, T=4096 - 17, H=4, seed=61, heads=[(0, 0), (0, 3)])
