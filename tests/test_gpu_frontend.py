"""GPU parity of the on-load input transforms (q/k L2 normalisation; gates
from pre-activations) against the oracle's float64 front-end followed by its
recurrence, on the same seeded pre-activation inputs."""
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import VARIANTS, make_raw_inputs
from oracle import oracle
from tests.gpu_common import TOL, announce, rel_err, to_dev

pytestmark = pytest.mark.gpu

L2, RAW = binding.GDR_FLAG_QK_L2NORM, binding.GDR_FLAG_RAW_GATES


@pytest.fixture(scope="module", autouse=True)
def _lib():
    binding.lib()
    oracle.load()


def _scale(variant, flags):
    return 0.1 if (flags & RAW and variant != "deltanet") else 0.0


def _check_forward(variant, dtype, flags, B=2, T=200, H=2, dk=128, dv=128, seed=0, heads=None):
    inp = make_raw_inputs(variant, B, T, H, dk, dv, dtype, seed=seed)
    if not flags & L2:
        # stored keys must keep beta |k|^2 below 2: shrink them to norm ~ 0.7
        inp["k"] = (inp["k"].float() * 0.06).to(inp["k"].dtype)
    if not flags & RAW:
        # stored gates: map the draws into their ranges by hand-picked affine maps
        for key in ("beta", "erase_b", "write_w"):
            if inp[key] is not None:
                inp[key] = (inp[key] * 0.1 + 0.5).clamp(0.05, 0.95)
        if inp["alpha"] is not None:
            inp["alpha"] = (inp["alpha"] * 0.01 + 0.95).clamp(0.8, 1.0)
    ds = _scale(variant, flags)
    d = to_dev(inp)
    o, s = binding.forward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                           erase_b=d["erase_b"], write_w=d["write_w"], eps=d["eps"],
                           state_in=d["state_in"], flags=flags, decay_scale=ds)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward(variant, inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                                  beta=inp["beta"], erase_b=inp["erase_b"],
                                  write_w=inp["write_w"], eps=inp["eps"],
                                  state_in=inp["state_in"], heads=heads, flags=flags,
                                  decay_scale=ds)
    tol = TOL[d["q"].dtype]
    o_cpu, s_cpu = o.float().cpu().numpy(), s.cpu().numpy()
    if heads is None:
        e_o, e_s = rel_err(o_cpu, o_ref, (0, 2)), rel_err(s_cpu, s_ref, (0, 1))
    else:
        e_o = max(rel_err(o_cpu[b:b + 1, :, h:h + 1], o_ref[b:b + 1, :, h:h + 1], (0, 2))
                  for b, h in heads)
        e_s = max(rel_err(s_cpu[b:b + 1, h:h + 1], s_ref[b:b + 1, h:h + 1], (0, 1))
                  for b, h in heads)
    announce(f"{variant} {dtype} flags={flags} T={T}: rel_err o={e_o:.2e} S={e_s:.2e} (tol {tol})")
    assert e_o < tol and e_s < tol


@pytest.mark.parametrize("flags", [L2, RAW, L2 | RAW])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_forward_transforms_match_oracle(variant, dtype, flags):
    _check_forward(variant, dtype, flags, seed=VARIANTS.index(variant) * 7 + flags)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128)])
@pytest.mark.parametrize("variant", ["kda", "gdn2", "kla"])
def test_forward_transforms_head_sizes(variant, dk, dv):
    _check_forward(variant, "bf16", L2 | RAW, dk=dk, dv=dv, T=130, seed=11)


@pytest.mark.parametrize("H", [16, 4], ids=["pipelined", "segmented"])
@pytest.mark.parametrize("variant", ["kla", "kda", "gdn2"])
def test_forward_transforms_pipelined(variant, H):
    """514 chunks, sampled heads: at 16 heads the blocked path (one launch per
    block), at 4 heads the segmented one."""
    _check_forward(variant, "bf16", L2 | RAW, B=1, T=64 * 64 * 8 + 100, H=H, seed=21,
                   heads=[(0, 0), (0, H - 1)])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_decode_transforms_match_oracle(variant, dtype, dk, dv):
    flags = L2 | RAW
    B, H = 8, 3
    inp = make_raw_inputs(variant, B, 1, H, dk, dv, dtype, seed=31 + VARIANTS.index(variant))
    ds = _scale(variant, flags)
    d = to_dev(inp)
    state = d["state_in"].clone()
    o = binding.decode_step(variant, d["q"], d["k"], d["v"], state, alpha=d["alpha"],
                            beta=d["beta"], erase_b=d["erase_b"], write_w=d["write_w"],
                            eps=d["eps"], flags=flags, decay_scale=ds)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.forward(variant, inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                                  beta=inp["beta"], erase_b=inp["erase_b"],
                                  write_w=inp["write_w"], eps=inp["eps"],
                                  state_in=inp["state_in"], flags=flags, decay_scale=ds)
    tol = TOL[d["q"].dtype]
    e_o = rel_err(o.float().cpu().numpy(), o_ref, (0, 2))
    e_s = rel_err(state.cpu().numpy(), s_ref, (0, 1))
    announce(f"decode {variant} {dtype} {dk}x{dv}: rel_err o={e_o:.2e} S={e_s:.2e}")
    assert e_o < tol and e_s < tol
