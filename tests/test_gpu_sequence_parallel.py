"""The sequence-parallel forward against the float64 oracle.

With few heads (B * H * d_v / 16 column slices at most a quarter of the
compute units: B = 1 with H <= 8 at d_v = 128 on a 256-unit MI355X) the bf16
forward cuts the sequence into segments whose chains run side by side: every
segment but the last from S = 0 and from the identity (its local end state
and its transition), a serial combine of those from the initial state, then
every segment's scan from its start state.  The chunk map S -> M S + N is
affine in S, so the result is the same recurrence; these cases check o and
the final state (and the written residual with a routed value) element by
element on every head, for segment counts from 2 to 16 and a ragged last
segment and chunk.  The first test confirms from the workspace size that
these shapes take that path."""
import numpy as np
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import make_inputs, make_routed_value
from oracle import oracle
from tests.gpu_common import TOL, announce, gpu_forward, rel_err, run_oracle, to_dev

pytestmark = pytest.mark.gpu

FACTOR_BYTES = 2 * (64 * 128 * 4 + 64 * 64) + 4 * 128   # bf16 factors + e^{g_C} per chunk-head


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("H,T", [(8, 64 * 300 + 21), (4, 64 * 257 + 5), (2, 64 * 100 + 13),
                                 (1, 64 * 600)])
def test_few_heads_take_the_segmented_path(H, T):
    """The workspace holds every chunk's factors plus the segments' transition,
    end-state and start-state arrays (fp32, d_k x d_k and twice d_k x d_v per
    head and segment boundary)."""
    if 4 * H * 8 > _cus():
        pytest.skip("needs at least four times as many compute units as column slices")
    q = torch.empty((1, T, H, 128), dtype=torch.bfloat16, device="cuda")
    n = binding.workspace_bytes("kla", q, q, q)
    nc = (T + 63) // 64
    assert n > nc * H * FACTOR_BYTES + 7 * 256 + H * 3 * 128 * 128 * 4


CASES = [  # variant, H, T (chunks: 301, 258, 101, 600, 81)
    ("gdn2", 8, 64 * 300 + 21),
    ("kla", 4, 64 * 257 + 5),
    ("gated_deltanet", 2, 64 * 100 + 13),
    ("deltanet", 1, 64 * 600),
    ("kda", 4, 64 * 80 + 40),
    ("gdn2", 2, 64 * 100 + 13),
]


@pytest.mark.parametrize("variant,H,T", CASES)
def test_segmented_forward_matches_oracle(variant, H, T):
    announce(f"segmented forward {variant} B=1 H={H} T={T}")
    inp = make_inputs(variant, 1, T, H, 128, 128, "bf16", seed=960 + H, state_scale=0.3)
    o, s = gpu_forward(variant, to_dev(inp))
    o_ref, s_ref = run_oracle(variant, inp)
    e_o = rel_err(o.float().cpu(), o_ref, (0, 2))
    e_s = rel_err(s.cpu(), s_ref, (0, 1))
    announce(f"  rel_err o={e_o:.3e} S={e_s:.3e}")
    assert e_o < TOL[torch.bfloat16] and e_s < TOL[torch.bfloat16]


@pytest.mark.parametrize("B,H,dk,dv,T", [(1, 4, 128, 64, 64 * 64), (2, 2, 64, 64, 64 * 65 + 1),
                                         (1, 1, 128, 128, 64 * 64 + 1), (2, 1, 64, 128, 64 * 97 + 50)])
def test_segmented_forward_shapes(B, H, dk, dv, T):
    """Batch rows, head sizes and the smallest segmented lengths (64 chunks:
    four segments of 16; 65 chunks: 17, 17, 17 and 14)."""
    announce(f"segmented forward gated_deltanet B={B} H={H} dk={dk} dv={dv} T={T}")
    inp = make_inputs("gated_deltanet", B, T, H, dk, dv, "bf16", seed=980 + T % 97, state_scale=0.3)
    o, s = gpu_forward("gated_deltanet", to_dev(inp))
    o_ref, s_ref = run_oracle("gated_deltanet", inp)
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < TOL[torch.bfloat16]
    assert rel_err(s.cpu(), s_ref, (0, 1)) < TOL[torch.bfloat16]


def test_segmented_forward_zero_initial_state_and_head_sizes():
    """No initial state (the combine starts from zeros), d_k = 64, d_v = 128."""
    T = 64 * 150 + 7
    inp = make_inputs("kla", 1, T, 2, 64, 128, "bf16", seed=970, state_scale=0.0)
    o, s = gpu_forward("kla", to_dev(inp))
    o_ref, s_ref = run_oracle("kla", inp)
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < TOL[torch.bfloat16]
    assert rel_err(s.cpu(), s_ref, (0, 1)) < TOL[torch.bfloat16]


def test_segmented_forward_routed_value_and_residual():
    """A routed value added on load and the written residual of every token."""
    T = 64 * 130 + 3
    inp = make_inputs("kla", 1, T, 2, 128, 128, "bf16", seed=971, state_scale=0.3)
    vr = make_routed_value(1, T, 2, 128, "bf16", seed=972, scale=0.5)
    d = to_dev(inp)
    o, s, delta = binding.forward("kla", d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                                  eps=d["eps"], state_in=d["state_in"], v_route=vr.cuda(),
                                  want_delta=True)
    torch.cuda.synchronize()
    o_ref, s_ref, dl_ref = oracle.forward("kla", inp["q"], inp["k"], inp["v"], alpha=inp["alpha"],
                                          beta=inp["beta"], eps=inp["eps"],
                                          state_in=inp["state_in"], v_route=vr, want_delta=True)
    tol = TOL[torch.bfloat16]
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < tol
    assert rel_err(s.cpu(), s_ref, (0, 1)) < tol
    assert rel_err(delta.float().cpu(), dl_ref, (0, 2)) < tol


def test_segmented_forward_is_deterministic_and_replays_in_a_graph():
    """Two calls agree bit for bit, and a captured HIP graph of the call,
    replayed with other work in between, gives the same result."""
    T = 64 * 200 + 9
    inp = make_inputs("gated_deltanet", 1, T, 4, 128, 128, "bf16", seed=973, state_scale=0.3)
    d = to_dev(inp)
    o_ref, s_ref = gpu_forward("gated_deltanet", d)
    o = torch.empty_like(o_ref)
    s = torch.empty_like(s_ref)
    nbytes = binding.workspace_bytes("gated_deltanet", d["q"], d["k"], d["v"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def run():
        binding.forward("gated_deltanet", d["q"], d["k"], d["v"], alpha=d["alpha"],
                        beta=d["beta"], state_in=d["state_in"], o=o, state_out=s, workspace=ws)

    run()
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        o.zero_()
        s.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {i}: output differs"
        assert torch.equal(s, s_ref), f"replay {i}: state differs"


@pytest.mark.parametrize("T,H", [(65536, 8), (65536, 4), (131072, 2)])
def test_segmented_forward_at_full_length_sampled_heads(T, H):
    """The few-head Kaczmarz forwards the benchmark times (1,024 chunks in 4
    or 8 segments; 2,048 chunks in 16), on the same inputs (seed 85100 + H) and
    from a zero state with the workspace passed in, as timed there: every head
    runs on the GPU, the oracle recomputes the first and the last head over the
    whole sequence."""
    if 4 * H * 8 > _cus():
        pytest.skip("needs at least four times as many compute units as column slices")
    announce(f"segmented forward kla B=1 H={H} T={T} (full length), oracle on heads 0 and {H - 1}")
    inp = dict(make_inputs("kla", 1, T, H, 128, 128, "bf16", seed=85100 + H), state_in=None)
    d = to_dev(inp)
    ws = torch.empty(binding.workspace_bytes("kla", d["q"], d["k"], d["v"]), dtype=torch.uint8,
                     device="cuda")
    o, s = binding.forward("kla", d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                           eps=d["eps"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(s).all()
    heads = [(0, 0), (0, H - 1)]
    o_ref, s_ref = run_oracle("kla", inp, heads=heads)
    o_cpu, s_cpu = o.float().cpu().numpy(), s.cpu().numpy()
    for _, h in heads:
        e_o = rel_err(o_cpu[:, :, h:h + 1], o_ref[:, :, h:h + 1], (0, 2))
        e_s = rel_err(s_cpu[:, h:h + 1], s_ref[:, h:h + 1], (0, 1))
        announce(f"  head {h}: rel_err o={e_o:.3e} S={e_s:.3e}")
        assert e_o < TOL[torch.bfloat16] and e_s < TOL[torch.bfloat16]
