"""The forward that keeps its records for the gradient, and the gradient that
reads them (gdr_forward_chunked_save, gdr_backward_chunked_saved).

The saving forward runs the gradient's first pass (every chunk's factors,
then the scan that records the state and residual entering each chunk) with
the scan also writing o and the final state.  The same kernels compute the
same values as gdr_forward_chunked and as gdr_backward_chunked's own first
pass, so o and state_out must equal the plain forward's bit for bit, and so
must every gradient the per-chunk gradient forms without atomic sums.  The
gradient accumulates some per-token sums (those of d_alpha, d_beta, and of
d_k for KLA) with atomic additions whose order varies from call to call, as
between two gdr_backward_chunked calls; those must agree to the rounding of
a float32 sum order (1e-5 normwise).  The plain gradient is itself checked
against the float64 oracle in test_gpu_backward.py; one case here also checks
the saved gradient against the oracle directly."""
import numpy as np
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import make_inputs, make_upstream_grads
from oracle import backward as oracle_bw
from tests.gpu_common import TOL, announce, rel_err, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = ("deltanet", "gated_deltanet", "kda", "gdn2", "kla")
ATOMIC_SUMS = {"alpha", "beta"}   # and k for KLA
DT = {"bf16": torch.bfloat16, "fp32": torch.float32}
AXES = dict(q=(0, 2), k=(0, 2), v=(0, 2), alpha=(0, 2), beta=(0, 2), erase_b=(0, 2),
            write_w=(0, 2), state_in=(0, 1))


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def _gates(d):
    return dict(alpha=d["alpha"], beta=d["beta"], erase_b=d["erase_b"], write_w=d["write_w"],
                eps=d["eps"], state_in=d["state_in"])


def _compare(variant, d, du):
    o_ref, s_ref = binding.forward(variant, d["q"], d["k"], d["v"], **_gates(d))
    g_ref = binding.backward(variant, d["q"], d["k"], d["v"], **_gates(d), d_o=du["d_o"],
                             d_state_out=du["d_state_out"])
    o, s, ws = binding.forward_save(variant, d["q"], d["k"], d["v"], **_gates(d))
    g = binding.backward(variant, d["q"], d["k"], d["v"], **_gates(d), d_o=du["d_o"],
                         d_state_out=du["d_state_out"], saved=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "o differs from gdr_forward_chunked"
    assert torch.equal(s, s_ref), "state_out differs from gdr_forward_chunked"
    for name, ref in g_ref.items():
        if ref is None:
            assert g[name] is None
            continue
        if name in ATOMIC_SUMS or (variant == "kla" and name == "k"):
            err = rel_err(g[name].cpu().numpy(), ref.cpu().numpy(), AXES[name])
            assert err < 1e-5, f"d_{name} differs from gdr_backward_chunked by {err:.1e}"
        else:
            assert torch.equal(g[name], ref), f"d_{name} differs from gdr_backward_chunked"
    return o, s, g, ws


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_saved_path_equals_recomputing_path(variant, dtype):
    """Two heads of two sequences, three full chunks and a ragged one."""
    announce(f"saved forward/gradient {variant} {dtype}")
    inp = make_inputs(variant, 2, 205, 2, 128, 128, dtype, seed=1300, state_scale=0.3)
    up = make_upstream_grads(2, 205, 2, 128, 128, dtype, seed=1301)
    _compare(variant, to_dev(inp), to_dev(up))


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_saved_path_head_sizes(dk, dv):
    announce(f"saved forward/gradient kla dk={dk} dv={dv}")
    inp = make_inputs("kla", 1, 150, 3, dk, dv, "bf16", seed=1310, state_scale=0.3)
    up = make_upstream_grads(1, 150, 3, dk, dv, "bf16", seed=1311)
    _compare("kla", to_dev(inp), to_dev(up))


@pytest.mark.parametrize("T", [1, 64, 65])
@pytest.mark.parametrize("variant", ["gdn2", "kla"])
def test_saved_path_short_sequences(variant, T):
    """One token, one full chunk, and a full chunk plus one token; d = 64."""
    announce(f"saved forward/gradient {variant} T={T}")
    inp = make_inputs(variant, 2, T, 2, 64, 64, "bf16", seed=1350 + T, state_scale=0.3)
    up = make_upstream_grads(2, T, 2, 64, 64, "bf16", seed=1351 + T)
    _compare(variant, to_dev(inp), to_dev(up))


def test_saving_forward_without_final_state():
    """state_out = NULL: the saving forward still keeps every record the
    gradient needs (the final state is not one of them)."""
    announce("saving forward without state_out")
    inp = make_inputs("gated_deltanet", 1, 140, 2, 128, 128, "bf16", seed=1360, state_scale=0.3)
    up = make_upstream_grads(1, 140, 2, 128, 128, "bf16", seed=1361)
    d, du = to_dev(inp), to_dev(up)
    o_ref, _ = binding.forward("gated_deltanet", d["q"], d["k"], d["v"], **_gates(d))
    g_ref = binding.backward("gated_deltanet", d["q"], d["k"], d["v"], **_gates(d), d_o=du["d_o"],
                             d_state_out=du["d_state_out"])
    o, s, ws = binding.forward_save("gated_deltanet", d["q"], d["k"], d["v"], **_gates(d),
                                    output_state=False)
    g = binding.backward("gated_deltanet", d["q"], d["k"], d["v"], **_gates(d), d_o=du["d_o"],
                         d_state_out=du["d_state_out"], saved=ws)
    torch.cuda.synchronize()
    assert s is None and torch.equal(o, o_ref)
    for name in ("q", "k", "v", "state_in"):
        assert torch.equal(g[name], g_ref[name]), name


@pytest.mark.parametrize("variant", ["kda", "gated_deltanet"])
def test_saved_path_where_the_plain_forward_is_pipelined(variant):
    """Long enough (257 / 513 chunks at 16 heads) that gdr_forward_chunked
    runs in 64-chunk blocks; the saving forward is one pass."""
    T = (256 if variant == "kda" else 512) * 64 + 37
    announce(f"saved path, pipelined plain forward: {variant} T={T}")
    inp = make_inputs(variant, 1, T, 16, 128, 128, "bf16", seed=1320, state_scale=0.3)
    up = make_upstream_grads(1, T, 16, 128, 128, "bf16", seed=1321)
    _compare(variant, to_dev(inp), to_dev(up))


@pytest.mark.parametrize("variant,H", [("kla", 4), ("kda", 4), ("gdn2", 8)])
def test_saved_path_where_the_forward_is_segmented(variant, H):
    """131 chunks at 4 or 8 heads: few enough heads that gdr_forward_chunked
    runs in segments whose chains run side by side; the saving forward and the
    gradient's own first pass take the same segments, so o, the final state
    and the gradients agree bit for bit as elsewhere."""
    T = 130 * 64 + 9
    announce(f"saved path, segmented forward: {variant} H={H} T={T}")
    inp = make_inputs(variant, 1, T, H, 128, 128, "bf16", seed=1325, state_scale=0.3)
    up = make_upstream_grads(1, T, H, 128, 128, "bf16", seed=1326)
    _compare(variant, to_dev(inp), to_dev(up))


def test_saved_gradient_against_oracle_and_workspace_reuse():
    """The saved gradient against the float64 oracle, then a second saving
    forward of other inputs in the same workspace: its gradient must follow
    the new inputs."""
    announce("saved gradient vs oracle, workspace reused")
    ws = None
    for seed in (1330, 1340):
        inp = make_inputs("kda", 1, 190, 2, 128, 128, "bf16", seed=seed, state_scale=0.3)
        up = make_upstream_grads(1, 190, 2, 128, 128, "bf16", seed=seed + 1)
        d, du = to_dev(inp), to_dev(up)
        _, _, ws = binding.forward_save("kda", d["q"], d["k"], d["v"], **_gates(d), workspace=ws)
        g = binding.backward("kda", d["q"], d["k"], d["v"], **_gates(d), d_o=du["d_o"],
                             d_state_out=du["d_state_out"], saved=ws)
        torch.cuda.synchronize()
        ref = oracle_bw.backward("kda", inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                                 beta=inp["beta"], erase_b=None, write_w=None, eps=0.0,
                                 state_in=inp["state_in"], d_o=up["d_o"],
                                 d_state_out=up["d_state_out"])
        errs = {n: rel_err(g[n].cpu().numpy(), r, AXES[n]) for n, r in ref.items() if r is not None}
        announce("  " + " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
        bad = {n: e for n, e in errs.items() if not e < TOL[torch.bfloat16]}
        assert not bad, bad
        assert all(np.isfinite(g[n].cpu().numpy()).all() for n in errs)
