"""GPU parity under strong decay.  Channel-wise (Kimi Delta Attention, Gated
DeltaNet-2): a third of each head's key channels decay by a factor drawn from
[1e-3, 0.05] at every token, the rest as in the workloads.  Scalar (Gated
DeltaNet, Kaczmarz): a third of each head's tokens forget by such a factor.  The chunk form
splits a channel decay between the two operands of its Gram products; these
cases drive the split's factors far from 1, where a per-chunk reference would
overflow ("Gated DeltaNet-2", technical core: the channel decay is absorbed
into the asymmetric erase factor of the chunkwise WY algorithm).

Cases: forward in bf16 and fp32 in one pass, the pipelined bf16 forward
(>= 256 chunks), decays far below the chunk form's floor (e^{-10}, exact above
it; the oracle applies every decay exactly), gate pre-activations through the
on-load transforms, decode steps, and the gradient.  A scalar decay needs no
split: the chunk form only ever applies e^{g_r - g_s} with s <= r, e^{g_r}
and e^{g_C - g_r}, all at most 1, and it applies every decay exactly, so the
scalar cases take decays down to 1e-30 in every path, where e^{g} underflows
to zero within a chunk.  Errors are the normwise
per-head measure of ``gpu_common.rel_err`` against the same thresholds as
every other parity test (fp32 1e-4, bf16 2e-2)."""
import numpy as np
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import (make_inputs, make_raw_inputs, make_upstream_grads,
                                            with_strong_channel_decay, with_strong_scalar_decay)
from oracle import backward as oracle_bw
from oracle import oracle
from tests.gpu_common import TOL, announce, gpu_forward, rel_err, run_oracle, to_dev

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp32": torch.float32}
CHANNEL = ("kda", "gdn2")
SCALAR = ("gated_deltanet", "kla")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def _strong(variant, B, T, H, dtype, seed, lo=1e-3, hi=0.05, log=False, dk=128, dv=128):
    inp = make_inputs(variant, B, T, H, dk, dv, dtype, seed=seed, alpha_scale=0.05,
                      state_scale=0.3)
    strong = with_strong_scalar_decay if variant in SCALAR else with_strong_channel_decay
    return strong(inp, lo=lo, hi=hi, seed=seed + 1, log=log)


def _check_forward(variant, inp, dtype, heads=None, label=""):
    o, s = gpu_forward(variant, to_dev(inp))
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all(), "non-finite output"
    o_ref, s_ref = run_oracle(variant, inp, heads=heads)
    o_np, s_np = o.float().cpu().numpy(), s.cpu().numpy()
    if heads is not None:
        e_o = max(rel_err(o_np[b:b + 1, :, h:h + 1], o_ref[b:b + 1, :, h:h + 1], (0, 2))
                  for b, h in heads)
        e_s = max(rel_err(s_np[b:b + 1, h:h + 1], s_ref[b:b + 1, h:h + 1], (0, 1))
                  for b, h in heads)
    else:
        e_o, e_s = rel_err(o_np, o_ref, (0, 2)), rel_err(s_np, s_ref, (0, 1))
    tol = TOL[DT[dtype]]
    announce(f"  {label} rel_err o={e_o:.3e} S={e_s:.3e} (tol {tol})")
    assert e_o < tol and e_s < tol


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", CHANNEL)
def test_forward_strong_decay_one_pass(variant, dtype):
    """Three full chunks and a ragged one, a third of the channels at alpha in [1e-3, 0.05]."""
    announce(f"strong decay forward {variant} {dtype}")
    inp = _strong(variant, 2, 205, 3, dtype, seed=900)
    _check_forward(variant, inp, dtype, label=f"{variant} {dtype}")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("variant", CHANNEL)
def test_forward_strong_decay_head_sizes(variant, dk, dv):
    announce(f"strong decay forward sizes {variant} dk={dk} dv={dv}")
    inp = _strong(variant, 1, 150, 2, "bf16", seed=910, dk=dk, dv=dv)
    _check_forward(variant, inp, "bf16", label=f"{variant} dk={dk} dv={dv}")


@pytest.mark.parametrize("H", [16, 2], ids=["pipelined", "segmented"])
@pytest.mark.parametrize("variant", CHANNEL)
def test_forward_strong_decay_pipelined(variant, H):
    """257 chunks (the last ragged): at 16 heads the bf16 forward runs as
    blocks of 64 chunks with the prep of one block beside the scan of the
    previous one (three heads checked); at 2 heads as segments whose chains
    run side by side."""
    announce(f"strong decay long forward {variant} H={H}")
    inp = _strong(variant, 1, 256 * 64 + 37, H, "bf16", seed=920)
    heads = [(0, 0), (0, H // 2), (0, H - 1)] if H > 2 else None
    _check_forward(variant, inp, "bf16", heads=heads, label=f"{variant} pipelined")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", CHANNEL)
def test_forward_decay_below_floor(variant, dtype):
    """Decays from 1e-30 to 1e-6 (log-uniform) on a third of the channels: the
    chunk form applies them as e^{-10}, which lets at most 4.5e-5 of a
    channel's state through where less should pass; the result stays finite and
    within tolerance of the exact recurrence."""
    announce(f"decay below floor {variant} {dtype}")
    inp = _strong(variant, 1, 200, 2, dtype, seed=930, lo=1e-30, hi=1e-6, log=True)
    _check_forward(variant, inp, dtype, label=f"{variant} {dtype} floor")


@pytest.mark.parametrize("variant", CHANNEL)
def test_forward_raw_gates_strong_decay(variant):
    """Gate pre-activations with decay scale 1 and shifted up by 4: decays
    exp(-softplus(x)) down to ~e^{-8}, reached through the on-load transforms."""
    announce(f"raw gates strong decay {variant}")
    inp = make_raw_inputs(variant, 1, 200, 2, 128, 128, "bf16", seed=940)
    inp["alpha"] = inp["alpha"] + 4.0
    d = to_dev(inp)
    flags = binding.GDR_FLAG_QK_L2NORM | binding.GDR_FLAG_RAW_GATES
    o, s = binding.forward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                           erase_b=d["erase_b"], write_w=d["write_w"], eps=d["eps"],
                           state_in=d["state_in"], flags=flags, decay_scale=1.0)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    o_ref, s_ref = oracle.forward(variant, inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                                  beta=inp["beta"], erase_b=inp["erase_b"],
                                  write_w=inp["write_w"], eps=inp["eps"],
                                  state_in=inp["state_in"], flags=flags, decay_scale=1.0)
    e_o = rel_err(o.float().cpu(), o_ref, (0, 2))
    e_s = rel_err(s.cpu(), s_ref, (0, 1))
    announce(f"  rel_err o={e_o:.3e} S={e_s:.3e}")
    assert e_o < 2e-2 and e_s < 2e-2


@pytest.mark.parametrize("variant", CHANNEL)
def test_decode_strong_decay(variant):
    """Eight decode steps from a seeded state; decode applies each decay exactly."""
    announce(f"strong decay decode {variant}")
    inp = _strong(variant, 4, 8, 3, "bf16", seed=950, lo=1e-30, hi=0.05, log=True)
    d = to_dev(inp)
    state = d["state_in"].clone()
    outs = []
    for t in range(8):
        sl = {k: (v[:, t:t + 1].contiguous() if isinstance(v, torch.Tensor) and k != "state_in"
                  else v) for k, v in d.items()}
        outs.append(binding.decode_step(variant, sl["q"], sl["k"], sl["v"], state,
                                        alpha=sl["alpha"], beta=sl["beta"],
                                        erase_b=sl["erase_b"], write_w=sl["write_w"]))
    torch.cuda.synchronize()
    o = torch.cat(outs, 1)
    o_ref, s_ref = run_oracle(variant, inp)
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < 2e-2
    assert rel_err(state.cpu(), s_ref, (0, 1)) < 2e-2


_AXES = dict(q=(0, 2), k=(0, 2), v=(0, 2), alpha=(0, 2), beta=(0, 2), erase_b=(0, 2),
             write_w=(0, 2), state_in=(0, 1))


def _check_grad(variant, dtype, B, T, H, seed, lo=1e-3, hi=0.05, heads=None):
    inp = _strong(variant, B, T, H, dtype, seed=seed, lo=lo, hi=hi)
    up = make_upstream_grads(B, T, H, 128, 128, dtype, seed=seed + 7)
    d, du = to_dev(inp), to_dev(up)
    g = binding.backward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                         erase_b=d["erase_b"], write_w=d["write_w"], eps=d["eps"],
                         state_in=d["state_in"], d_o=du["d_o"], d_state_out=du["d_state_out"])
    torch.cuda.synchronize()
    ref = oracle_bw.backward(variant, inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                             beta=inp["beta"], erase_b=inp["erase_b"], write_w=inp["write_w"],
                             eps=inp["eps"], state_in=inp["state_in"], d_o=up["d_o"],
                             d_state_out=up["d_state_out"], heads=heads)
    errs = {}
    for name, r in ref.items():
        if r is None:
            continue
        x = g[name].cpu().numpy()
        assert np.isfinite(x).all(), f"non-finite gradient {name}"
        ax = _AXES[name]
        if heads is None:
            errs[name] = rel_err(x, r, ax)
        else:
            sel = [(slice(b, b + 1), slice(None), slice(h, h + 1)) if ax == (0, 2)
                   else (slice(b, b + 1), slice(h, h + 1)) for b, h in heads]
            errs[name] = max(rel_err(x[s], r[s], ax) for s in sel)
    tol = TOL[DT[dtype]]
    announce(f"  grad {variant} {dtype} T={T}: " +
             " ".join(f"{n}={e:.1e}" for n, e in errs.items()) + f" (tol {tol})")
    bad = {n: e for n, e in errs.items() if not e < tol}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", CHANNEL)
def test_backward_strong_decay(variant, dtype):
    announce(f"strong decay gradient {variant} {dtype}")
    _check_grad(variant, dtype, 2, 200, 2, seed=960)


@pytest.mark.parametrize("variant", CHANNEL)
def test_backward_strong_decay_long(variant):
    """64 chunks in bf16; the oracle checks sampled heads."""
    announce(f"strong decay gradient long {variant}")
    _check_grad(variant, "bf16", 1, 4096 - 17, 3, seed=970, heads=[(0, 0), (0, 2)])


# ------------------------------------------------- scalar forget gate near zero

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", SCALAR)
def test_forward_strong_scalar_decay_one_pass(variant, dtype):
    """Three full chunks and a ragged one, a third of the tokens at alpha in [1e-3, 0.05]."""
    announce(f"strong scalar decay forward {variant} {dtype}")
    inp = _strong(variant, 2, 205, 3, dtype, seed=1900)
    _check_forward(variant, inp, dtype, label=f"{variant} {dtype}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", SCALAR)
def test_forward_tiny_scalar_decay(variant, dtype):
    """A third of the tokens at alpha from 1e-30 to 1e-6 (log-uniform): e^{g}
    reaches zero within a chunk; the state before such a token is forgotten."""
    announce(f"tiny scalar decay forward {variant} {dtype}")
    inp = _strong(variant, 1, 200, 2, dtype, seed=1910, lo=1e-30, hi=1e-6, log=True)
    _check_forward(variant, inp, dtype, label=f"{variant} {dtype} tiny")


@pytest.mark.parametrize("H", [16, 4], ids=["pipelined", "segmented"])
@pytest.mark.parametrize("variant", SCALAR)
def test_forward_strong_scalar_decay_pipelined(variant, H):
    """513 chunks (the last ragged): at 16 heads the bf16 forward runs as
    blocks of 64 chunks with the prep of one block beside the scan of the
    previous one (three heads checked); at 4 heads as segments whose chains
    run side by side."""
    announce(f"strong scalar decay long forward {variant} H={H}")
    inp = _strong(variant, 1, 512 * 64 + 37, H, "bf16", seed=1920, lo=1e-30, hi=0.05, log=True)
    heads = [(0, 0), (0, H // 2), (0, H - 1)] if H > 4 else None
    _check_forward(variant, inp, "bf16", heads=heads, label=f"{variant} pipelined")


@pytest.mark.parametrize("variant", SCALAR)
def test_decode_strong_scalar_decay(variant):
    """Eight decode steps from a seeded state with scalar decays down to 1e-30."""
    announce(f"strong scalar decay decode {variant}")
    inp = _strong(variant, 4, 8, 3, "bf16", seed=1950, lo=1e-30, hi=0.05, log=True)
    d = to_dev(inp)
    state = d["state_in"].clone()
    outs = []
    for t in range(8):
        sl = {k: (v[:, t:t + 1].contiguous() if isinstance(v, torch.Tensor) and k != "state_in"
                  else v) for k, v in d.items()}
        outs.append(binding.decode_step(variant, sl["q"], sl["k"], sl["v"], state,
                                        alpha=sl["alpha"], beta=sl["beta"], eps=d["eps"]))
    torch.cuda.synchronize()
    o = torch.cat(outs, 1)
    o_ref, s_ref = run_oracle(variant, inp)
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < 2e-2
    assert rel_err(state.cpu(), s_ref, (0, 1)) < 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", SCALAR)
def test_backward_strong_scalar_decay(variant, dtype):
    """The gradient, d_alpha included (d log alpha / alpha, large where alpha is small)."""
    announce(f"strong scalar decay gradient {variant} {dtype}")
    _check_grad(variant, dtype, 2, 200, 2, seed=1960)
