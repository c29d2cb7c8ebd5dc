"""GPU parity of the cross-layer routing input and output ("Linear Attention
Architectures: Mechanisms, Trade-offs, and Cross-Layer Routing", cross-layer
routing section): the routed value v_route (used as v + v_route) and the
per-token written residual delta_out, in the prefill and the decode step,
against the oracle on the same seeded inputs; and two stacked layers passing
the value target (CLVR) or the error (CLER) up, each side running its own
chain (the oracle chain takes no input from the GPU)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import VARIANTS, make_inputs, make_routed_value
from oracle import oracle
from tests.gpu_common import TOL, announce, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    binding.lib()
    oracle.load()


def _oracle(variant, inp, v_route=None, want_delta=True, heads=None, state_in=None):
    return oracle.forward(variant, inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                          beta=inp["beta"], erase_b=inp["erase_b"], write_w=inp["write_w"],
                          eps=inp["eps"], state_in=inp["state_in"] if state_in is None else state_in,
                          heads=heads, v_route=v_route, want_delta=want_delta)


def _gpu(variant, d, v_route=None, want_delta=True):
    out = binding.forward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                          erase_b=d["erase_b"], write_w=d["write_w"], eps=d["eps"],
                          state_in=d["state_in"], v_route=v_route, want_delta=want_delta)
    torch.cuda.synchronize()
    return out


def _errs(gpu, ref, heads=None):
    axes = [(0, 2), (0, 1), (0, 2)]
    out = []
    for x, r, ax in zip(gpu, ref, axes):
        x = x.float().cpu().numpy()
        if heads is None:
            out.append(rel_err(x, r, ax))
        else:
            sl = (lambda b, h: (slice(b, b + 1), slice(None), slice(h, h + 1))) if ax == (0, 2) \
                else (lambda b, h: (slice(b, b + 1), slice(h, h + 1)))
            out.append(max(rel_err(x[sl(b, h)], r[sl(b, h)], ax) for b, h in heads))
    return out


@pytest.mark.parametrize("routed", [False, True])
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_prefill_residual_and_routed_value(variant, dtype, routed):
    B, T, H, d = 2, 200, 2, 128
    seed = 300 + VARIANTS.index(variant) * 4 + 2 * (dtype == "bf16") + routed
    inp = make_inputs(variant, B, T, H, d, d, dtype, seed=seed, state_scale=0.1)
    vr = make_routed_value(B, T, H, d, dtype, seed=seed + 50) if routed else None
    dev = to_dev(inp)
    g = _gpu(variant, dev, None if vr is None else vr.cuda())
    ref = _oracle(variant, inp, vr)
    e_o, e_s, e_d = _errs(g, ref)
    tol = TOL[dev["q"].dtype]
    announce(f"{variant} {dtype} routed={routed}: o={e_o:.2e} S={e_s:.2e} delta={e_d:.2e} (tol {tol})")
    assert e_o < tol and e_s < tol and e_d < tol


@pytest.mark.parametrize("H", [16, 4], ids=["pipelined", "segmented"])
@pytest.mark.parametrize("variant", ["kla", "kda"])
def test_prefill_routing_pipelined(variant, H):
    """514 chunks in bf16, sampled heads: at 16 heads the blocked path (one
    launch per block), at 4 heads the segmented one."""
    B, T, d = 1, 64 * 64 * 8 + 77, 128
    inp = make_inputs(variant, B, T, H, d, d, "bf16", seed=41, state_scale=0.1)
    vr = make_routed_value(B, T, H, d, "bf16", seed=42, scale=0.5)
    heads = [(0, 0), (0, H - 1)]
    g = _gpu(variant, to_dev(inp), vr.cuda())
    ref = _oracle(variant, inp, vr, heads=heads)
    e = _errs(g, ref, heads)
    announce(f"{variant} pipelined T={T}: o={e[0]:.2e} S={e[1]:.2e} delta={e[2]:.2e}")
    assert max(e) < TOL[torch.bfloat16]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_residual_and_routed_value(variant, dtype):
    B, H, d = 8, 4, 128
    seed = 500 + VARIANTS.index(variant) * 2 + (dtype == "bf16")
    inp = make_inputs(variant, B, 1, H, d, d, dtype, seed=seed, state_scale=0.3)
    vr = make_routed_value(B, 1, H, d, dtype, seed=seed + 7)
    dev = to_dev(inp)
    state = dev["state_in"].clone()
    delta = torch.empty((B, 1, H, d), dtype=dev["q"].dtype, device="cuda")
    o = binding.decode_step(variant, dev["q"], dev["k"], dev["v"], state, alpha=dev["alpha"],
                            beta=dev["beta"], erase_b=dev["erase_b"], write_w=dev["write_w"],
                            eps=dev["eps"], v_route=vr.cuda(), delta_out=delta)
    torch.cuda.synchronize()
    ref = _oracle(variant, inp, vr)
    e_o, e_s, e_d = _errs((o, state, delta), ref)
    tol = TOL[dev["q"].dtype]
    announce(f"decode {variant} {dtype}: o={e_o:.2e} S={e_s:.2e} delta={e_d:.2e}")
    assert e_o < tol and e_s < tol and e_d < tol


def test_decode_residual_only_and_transforms():
    """delta_out without a routed value, with the on-load transforms on."""
    from gated_delta_rule_85_amd.inputs import make_raw_inputs
    L2, RAW = binding.GDR_FLAG_QK_L2NORM, binding.GDR_FLAG_RAW_GATES
    B, H, d = 8, 4, 128
    inp = make_raw_inputs("kla", B, 1, H, d, d, "bf16", seed=71)
    dev = to_dev(inp)
    state = dev["state_in"].clone()
    delta = torch.empty((B, 1, H, d), dtype=torch.bfloat16, device="cuda")
    o = binding.decode_step("kla", dev["q"], dev["k"], dev["v"], state, alpha=dev["alpha"],
                            beta=dev["beta"], eps=dev["eps"], flags=L2 | RAW, decay_scale=0.1,
                            delta_out=delta)
    torch.cuda.synchronize()
    ref = oracle.forward("kla", inp["q"], inp["k"], inp["v"], alpha=inp["alpha"], beta=inp["beta"],
                         eps=inp["eps"], state_in=inp["state_in"], flags=L2 | RAW, decay_scale=0.1,
                         want_delta=True)
    e = _errs((o, state, delta), ref)
    announce(f"decode kla transforms + delta: {e}")
    assert max(e) < TOL[torch.bfloat16]


@pytest.mark.parametrize("mode", ["clvr", "cler"])
@pytest.mark.parametrize("variant", ["gated_deltanet", "deltanet"])
def test_two_layer_routing(variant, mode):
    """Layer 2 receives layer 1's value target (CLVR) or its error (CLER) as
    v_route.  GPU and oracle each run the whole two-layer chain."""
    B, T, H, d = 1, 320, 2, 128
    l1 = make_inputs(variant, B, T, H, d, d, "bf16", seed=811)
    l2 = make_inputs(variant, B, T, H, d, d, "bf16", seed=812)
    # GPU chain
    d1, d2 = to_dev(l1), to_dev(l2)
    o1, s1, delta1 = _gpu(variant, d1)
    route_gpu = d1["v"] if mode == "clvr" else delta1
    g2 = _gpu(variant, d2, route_gpu.contiguous())
    # oracle chain
    ro1, rs1, rdelta1 = _oracle(variant, l1)
    route_ref = l1["v"] if mode == "clvr" else rdelta1
    r2 = _oracle(variant, l2, route_ref)
    e = _errs(g2, r2)
    announce(f"two-layer {mode} {variant}: o={e[0]:.2e} S={e[1]:.2e} delta={e[2]:.2e}")
    assert max(e) < TOL[torch.bfloat16]
