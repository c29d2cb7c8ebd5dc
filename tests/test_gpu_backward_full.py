"""The gradient at the full workload sizes, in the configuration bench.py
times, through identities that hold at any size (the oracle cannot run these
lengths token by token).  For fixed keys and gates the forward's outputs
(o, S_T) are linear in (v, S_0), and o is linear in q (o_t = S_t^T q_t, S_t
independent of q); so for upstream gradients dO = o and dS_T = S_T

    <d_q, q> = |o|^2        <d_v, v> + <d_S0, S_0> = |o|^2 + |S_T|^2

with no cancellation on the right.  Both sides come from the GPU (forward,
then gradient) and agree up to rounding (about 1e-5 here); the bar, 1e-3,
is far below what a wrong term in d_q, d_v or d_S0 would leave."""
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import WORKLOADS, make_workload
from tests.gpu_common import announce

pytestmark = pytest.mark.gpu


def _dot(a, b):
    return float((a.double() * b.double()).sum())


@pytest.mark.parametrize("wid", [5, 3, 4])
def test_gradient_identities_full_size(wid):
    wl = WORKLOADS[wid]
    inp = make_workload(wl)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    g0 = torch.Generator(device="cpu").manual_seed(wl.seed + 9)
    s0 = (torch.randn((B, H, dk, dv), generator=g0) * 0.1).cuda()
    kw = dict(alpha=d["alpha"], beta=d["beta"], erase_b=d["erase_b"], write_w=d["write_w"],
              eps=d["eps"])
    o, s_T = binding.forward(wl.variant, d["q"], d["k"], d["v"], state_in=s0, **kw)
    g = binding.backward(wl.variant, d["q"], d["k"], d["v"], state_in=s0, d_o=o.contiguous(),
                         d_state_out=s_T.contiguous(), **kw)
    torch.cuda.synchronize()
    oo, ss = _dot(o, o), _dot(s_T, s_T)
    e_q = abs(_dot(g["q"], d["q"]) - oo) / oo
    e_v = abs(_dot(g["v"], d["v"]) + _dot(g["state_in"], s0) - (oo + ss)) / (oo + ss)
    announce(f"{wl.name}: <dq,q> vs |o|^2 rel {e_q:.2e}; <dv,v>+<dS0,S0> vs |o|^2+|S_T|^2 rel {e_v:.2e}")
    assert e_q < 1e-3 and e_v < 1e-3
