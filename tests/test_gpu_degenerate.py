"""GPU parity on the degenerate inputs of the delta rule, against the float64
oracle (whose closed forms for these cases are pinned in the CPU tests:
pure decay, one-hot keys, the reductions between variants).

  * zero keys on every third token: the token neither erases nor writes
    (for the Kaczmarz rule the step size eta / (|k|^2 + eps) is then 1e6 times
    eta, multiplying a zero key);
  * zero write strength (beta = 0, eta = 0, or GDN-2's b = w = 0): the state
    only decays, o_t = (Gamma_t S_0)^T q_t;
  * no decay (alpha = 1): the gated variants become the plain delta rule;
  * one-hot keys with beta = 1 (DeltaNet): each token replaces one row of
    the state by its value.

Each case runs the chunked forward (three full chunks and a ragged one, a
non-zero initial state) and one decode step, in bf16 and fp32, with the
normwise error and thresholds of the other parity tests."""
import numpy as np
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import VARIANTS, make_inputs
from tests.gpu_common import TOL, announce, gpu_forward, rel_err, run_oracle, to_dev

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def _zero_keys(variant, inp):
    inp["k"][:, ::3] = 0
    return inp


def _no_write(variant, inp):
    if variant == "gdn2":
        inp["erase_b"].zero_()
        inp["write_w"].zero_()
    else:
        inp["beta"].zero_()
    return inp


def _no_decay(variant, inp):
    if inp["alpha"] is not None:
        inp["alpha"].fill_(1.0)
    return inp


CASES = {"zero_keys": (_zero_keys, VARIANTS), "no_write": (_no_write, VARIANTS),
         "no_decay": (_no_decay, ("gated_deltanet", "kda", "gdn2", "kla"))}
PARAMS = [(c, v) for c, (_, vs) in CASES.items() for v in vs]


def _check_forward(variant, inp, dtype):
    o, s = gpu_forward(variant, to_dev(inp))
    o_ref, s_ref = run_oracle(variant, inp)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    tol = TOL[DT[dtype]]
    e_o = rel_err(o.float().cpu(), o_ref, (0, 2))
    e_s = rel_err(s.cpu(), s_ref, (0, 1))
    announce(f"  forward rel_err o={e_o:.3e} S={e_s:.3e}")
    assert e_o < tol and e_s < tol


def _check_decode(variant, inp, dtype):
    d = to_dev(inp)
    state = d["state_in"].clone()
    o = binding.decode_step(variant, d["q"], d["k"], d["v"], state, alpha=d["alpha"],
                            beta=d["beta"], erase_b=d["erase_b"], write_w=d["write_w"],
                            eps=d["eps"])
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(variant, inp)
    e_o = rel_err(o.float().cpu(), o_ref, (0, 2))
    e_s = rel_err(state.cpu(), s_ref, (0, 1))
    announce(f"  decode rel_err o={e_o:.3e} S={e_s:.3e}")
    assert e_o < TOL[DT[dtype]] and e_s < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case,variant", PARAMS)
def test_degenerate_forward(case, variant, dtype):
    announce(f"degenerate forward {case} {variant} {dtype}")
    inp = make_inputs(variant, 2, 3 * 64 + 29, 3, 128, 128, dtype, seed=950, state_scale=0.5)
    _check_forward(variant, CASES[case][0](variant, inp), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case,variant", PARAMS)
def test_degenerate_decode(case, variant, dtype):
    announce(f"degenerate decode {case} {variant} {dtype}")
    inp = make_inputs(variant, 3, 1, 4, 128, 128, dtype, seed=951, state_scale=0.5)
    if case == "zero_keys":
        inp["k"][1:] = 0   # the step's key is zero for batch rows 1 and 2
    else:
        inp = CASES[case][0](variant, inp)
    _check_decode(variant, inp, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_one_hot_keys_replace_rows(dtype):
    """DeltaNet, beta = 1, keys e_{i_t}: token t sets row i_t of S to v_t."""
    announce(f"one-hot keys {dtype}")
    B, T, H, d = 1, 2 * 64 + 17, 2, 128
    inp = make_inputs("deltanet", B, T, H, d, d, dtype, seed=952, state_scale=0.5)
    rng = np.random.default_rng(953)
    idx = rng.integers(0, d, size=(B, T, H))
    k = torch.zeros((B, T, H, d), dtype=torch.float32)
    k.scatter_(3, torch.from_numpy(idx)[..., None], 1.0)
    inp["k"] = k.to(inp["q"].dtype)
    inp["beta"].fill_(1.0)
    o, s = gpu_forward("deltanet", to_dev(inp))
    o_ref, s_ref = run_oracle("deltanet", inp)
    tol = TOL[DT[dtype]]
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < tol
    assert rel_err(s.cpu(), s_ref, (0, 1)) < tol
    # the closed form itself: the last token to touch a row set it to its value
    s_np = s.cpu().numpy()
    v = inp["v"].float().numpy()
    for h in range(H):
        for i in range(d):
            ts = np.nonzero(idx[0, :, h] == i)[0]
            if len(ts):
                assert np.allclose(s_np[0, h, i], v[0, ts[-1], h], rtol=tol, atol=tol)
