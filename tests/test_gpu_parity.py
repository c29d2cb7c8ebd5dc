"""GPU parity: the HIP kernels behind the C ABI against the CPU oracle, on the
same seeded inputs, element by element, with the normwise error of
``gpu_common.rel_err`` and its per-dtype threshold."""
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
    binding.lib()  # raises if the HIP library is missing


# ------------------------------------------------------------------- decode

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_decode_step_matches_oracle(variant, dtype, dk, dv):
    announce(f"decode {variant} {dtype} dk={dk} dv={dv}")
    inp = make_inputs(variant, 3, 1, 5, dk, dv, dtype, seed=100 + dk + dv, state_scale=0.5)
    d = to_dev(inp)
    state = d["state_in"].clone()
    o = binding.decode_step(variant, d["q"], d["k"], d["v"], state, alpha=d["alpha"],
                            beta=d["beta"], erase_b=d["erase_b"], write_w=d["write_w"],
                            eps=d["eps"])
    torch.cuda.synchronize()
    o_ref, s_ref = run_oracle(variant, inp)
    tol = TOL[DT[dtype]]
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < tol
    assert rel_err(state.cpu(), s_ref, (0, 1)) < (1e-5 if dtype == "fp32" else 1e-5)


def test_decode_separate_output_state():
    inp = make_inputs("kda", 2, 1, 3, 128, 128, "bf16", seed=7, state_scale=1.0)
    d = to_dev(inp)
    s_in = d["state_in"].clone()
    s_out = torch.full_like(s_in, float("nan"))
    binding.decode_step("kda", d["q"], d["k"], d["v"], s_in, alpha=d["alpha"],
                        beta=d["beta"], state_out=s_out)
    torch.cuda.synchronize()
    assert torch.equal(s_in, d["state_in"])       # input untouched
    _, s_ref = run_oracle("kda", inp)
    assert rel_err(s_out.cpu(), s_ref, (0, 1)) < 1e-5


# ------------------------------------------------------------------ forward

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_forward_matches_oracle(variant, dtype):
    """Several chunks plus a ragged tail (T = 3*64 + 13), non-zero S_0."""
    announce(f"forward {variant} {dtype}")
    inp = make_inputs(variant, 2, 205, 3, 128, 128, dtype, seed=200, state_scale=0.5)
    o, s = gpu_forward(variant, to_dev(inp))
    o_ref, s_ref = run_oracle(variant, inp)
    tol = TOL[DT[dtype]]
    e_o = rel_err(o.float().cpu(), o_ref, (0, 2))
    e_s = rel_err(s.cpu(), s_ref, (0, 1))
    announce(f"  rel_err o={e_o:.3e} S={e_s:.3e}")
    assert e_o < tol and e_s < tol


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("variant", VARIANTS)
def test_forward_head_sizes(variant, dtype, dk, dv):
    announce(f"forward sizes {variant} {dtype} dk={dk} dv={dv}")
    inp = make_inputs(variant, 1, 150, 2, dk, dv, dtype, seed=300, state_scale=0.3)
    o, s = gpu_forward(variant, to_dev(inp))
    o_ref, s_ref = run_oracle(variant, inp)
    tol = TOL[DT[dtype]]
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < tol
    assert rel_err(s.cpu(), s_ref, (0, 1)) < tol


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 128, 129])
def test_forward_lengths(T):
    announce(f"forward length T={T}")
    inp = make_inputs("gated_deltanet", 2, T, 2, 128, 128, "fp32", seed=400 + T,
                      state_scale=0.5)
    o, s = gpu_forward("gated_deltanet", to_dev(inp))
    o_ref, s_ref = run_oracle("gated_deltanet", inp)
    assert rel_err(o.cpu(), o_ref, (0, 2)) < 1e-4
    assert rel_err(s.cpu(), s_ref, (0, 1)) < 1e-4


def test_forward_without_state_output_and_zero_initial_state():
    inp = make_inputs("kla", 1, 100, 2, 128, 128, "bf16", seed=5)
    o, s = gpu_forward("kla", to_dev(inp), output_state=False)
    assert s is None
    o_ref, _ = run_oracle("kla", inp)
    assert rel_err(o.float().cpu(), o_ref, (0, 2)) < 2e-2


@pytest.mark.parametrize("variant", ["gated_deltanet", "gdn2"])
def test_split_resume_equals_one_pass(variant):
    """forward(T1) then forward(T2 from S_T1) == forward(T1 + T2)."""
    inp = make_inputs(variant, 2, 300, 2, 128, 128, "fp32", seed=17, state_scale=0.2)
    d = to_dev(inp)
    o_all, s_all = gpu_forward(variant, d)
    cut = 100
    first = {k: (v[:, :cut].contiguous() if isinstance(v, torch.Tensor) and k != "state_in" else v)
             for k, v in d.items()}
    second = {k: (v[:, cut:].contiguous() if isinstance(v, torch.Tensor) and k != "state_in" else v)
              for k, v in d.items()}
    o1, s1 = gpu_forward(variant, first)
    o2, s2 = gpu_forward(variant, second, state_in=s1)
    assert rel_err(torch.cat([o1, o2], 1).cpu(), o_all.cpu(), (0, 2)) < 1e-4
    assert rel_err(s2.cpu(), s_all.cpu(), (0, 1)) < 1e-4


@pytest.mark.parametrize("variant", VARIANTS)
def test_decode_steps_equal_forward(variant):
    """T decode steps from S_0 and the chunked forward over the same T tokens
    both match the oracle."""
    T = 40
    inp = make_inputs(variant, 2, T, 2, 128, 128, "bf16", seed=23, state_scale=0.3)
    d = to_dev(inp)
    o_fwd, s_fwd = gpu_forward(variant, d)
    state = d["state_in"].clone()
    outs = []
    for t in range(T):
        sl = lambda x: None if x is None else x[:, t:t + 1].contiguous()
        outs.append(binding.decode_step(variant, sl(d["q"]), sl(d["k"]), sl(d["v"]), state,
                                        alpha=sl(d["alpha"]), beta=sl(d["beta"]),
                                        erase_b=sl(d["erase_b"]), write_w=sl(d["write_w"]),
                                        eps=d["eps"]))
    torch.cuda.synchronize()
    o_dec = torch.cat(outs, 1)
    o_ref, s_ref = run_oracle(variant, inp)
    assert rel_err(o_dec.float().cpu(), o_ref, (0, 2)) < 2e-2
    assert rel_err(state.cpu(), s_ref, (0, 1)) < 1e-4
    assert rel_err(o_fwd.float().cpu(), o_ref, (0, 2)) < 2e-2
    assert rel_err(s_fwd.cpu(), s_ref, (0, 1)) < 2e-2


def test_forward_is_deterministic():
    inp = make_inputs("kda", 2, 333, 4, 128, 128, "bf16", seed=31, state_scale=0.5)
    d = to_dev(inp)
    o1, s1 = gpu_forward("kda", d)
    o2, s2 = gpu_forward("kda", d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_heads_and_batches_are_independent():
    """Permuting heads permutes outputs: no cross-head mixing."""
    inp = make_inputs("gdn2", 2, 130, 4, 128, 128, "bf16", seed=37, state_scale=0.5)
    d = to_dev(inp)
    o, s = gpu_forward("gdn2", d)
    perm = torch.tensor([2, 0, 3, 1], device="cuda")
    dp = {}
    for k, v in d.items():
        if isinstance(v, torch.Tensor) and k != "state_in":
            dp[k] = v.index_select(2, perm).contiguous()
        elif k == "state_in":
            dp[k] = v.index_select(1, perm).contiguous()
        else:
            dp[k] = v
    op, sp = gpu_forward("gdn2", dp)
    assert torch.equal(op, o.index_select(2, perm))
    assert torch.equal(sp, s.index_select(1, perm))


# ------------------------------------------------- pipelined (multi-block) forward

@pytest.mark.parametrize("H", [16, 2], ids=["H16", "H2_segmented"])
@pytest.mark.parametrize("T", [64 * 64 * 8 + 100, 64 * 64 * 8 + 1, 64 * 64 * 2 + 100],
                         ids=["pipelined", "pipelined_one_token_block", "one_pass"])
@pytest.mark.parametrize("variant", ["gdn2", "kla", "deltanet"])
def test_forward_pipelined_blocks(variant, T, H):
    """Long bf16 sequences at 16 heads: from 256 chunks on as blocks of 64
    chunks, one launch per block on the caller's stream (nine blocks here;
    with T = 32769 the last block is a single chunk holding one token), below
    that as one pass (130 chunks); three heads checked.  At 2 heads the same
    lengths run as segments whose chains run side by side (every head
    checked).  A ragged last chunk and a non-zero initial state."""
    announce(f"long forward {variant} T={T} H={H}")
    inp = make_inputs(variant, 1, T, H, 128, 128, "bf16", seed=77, state_scale=0.5)
    o, s = gpu_forward(variant, to_dev(inp))
    heads = sorted({(0, 0), (0, H // 2), (0, H - 1)})
    o_ref, s_ref = run_oracle(variant, inp, heads=heads)
    o_np, s_np = o.float().cpu().numpy(), s.cpu().numpy()
    e_o = max(rel_err(o_np[:, :, h:h + 1], o_ref[:, :, h:h + 1], (0, 2)) for _, h in heads)
    e_s = max(rel_err(s_np[:, h:h + 1], s_ref[:, h:h + 1], (0, 1)) for _, h in heads)
    announce(f"  rel_err o={e_o:.3e} S={e_s:.3e}")
    assert e_o < 2e-2 and e_s < 2e-2


@pytest.mark.parametrize("variant", ["kla", "gated_deltanet", "deltanet"])
def test_forward_wide_scan_slices(variant):
    """Batch 4 x 16 heads at d = 128 gives more 16-column scan slices than the
    chip has compute units, so a scalar-decay bf16 scan takes 32 columns per
    workgroup; a ragged last chunk and a non-zero initial state."""
    announce(f"wide scan slices {variant}")
    inp = make_inputs(variant, 4, 300, 16, 128, 128, "bf16", seed=83, state_scale=0.5)
    o, s = gpu_forward(variant, to_dev(inp))
    o_ref, s_ref = run_oracle(variant, inp)
    e_o = rel_err(o.float().cpu(), o_ref, (0, 2))
    e_s = rel_err(s.cpu(), s_ref, (0, 1))
    announce(f"  rel_err o={e_o:.3e} S={e_s:.3e}")
    assert e_o < 2e-2 and e_s < 2e-2


def test_forward_wide_scan_slices_pipelined():
    """The same wide slices in the pipelined forward (B = 4, H = 16, 514
    chunks), checked on sampled heads."""
    T = 64 * 513 + 37
    inp = make_inputs("kla", 4, T, 16, 128, 128, "bf16", seed=85, state_scale=0.3)
    o, s = gpu_forward("kla", to_dev(inp))
    heads = [(0, 0), (1, 7), (3, 15)]
    o_ref, s_ref = run_oracle("kla", inp, heads=heads)
    for b, h in heads:
        e_o = rel_err(o[b:b + 1, :, h:h + 1].float().cpu(), o_ref[b:b + 1, :, h:h + 1], (0, 2))
        e_s = rel_err(s[b:b + 1, h:h + 1].cpu(), s_ref[b:b + 1, h:h + 1], (0, 1))
        announce(f"  head ({b}, {h}): rel_err o={e_o:.3e} S={e_s:.3e}")
        assert e_o < 2e-2 and e_s < 2e-2


@pytest.mark.parametrize("variant", ["kda", "gdn2"])
def test_forward_channel_decay_pipelined_wide_scan(variant):
    """A channel decay's pipelined forward takes 32-column scan slices beside
    a prep on the units they leave free (B = 1, H = 16, 514 chunks), checked
    on sampled heads."""
    T = 64 * 513 + 37
    inp = make_inputs(variant, 1, T, 16, 128, 128, "bf16", seed=86, state_scale=0.3)
    o, s = gpu_forward(variant, to_dev(inp))
    heads = [(0, 0), (0, 9), (0, 15)]
    o_ref, s_ref = run_oracle(variant, inp, heads=heads)
    for b, h in heads:
        e_o = rel_err(o[b:b + 1, :, h:h + 1].float().cpu(), o_ref[b:b + 1, :, h:h + 1], (0, 2))
        e_s = rel_err(s[b:b + 1, h:h + 1].cpu(), s_ref[b:b + 1, h:h + 1], (0, 1))
        announce(f"  {variant} head ({b}, {h}): rel_err o={e_o:.3e} S={e_s:.3e}")
        assert e_o < 2e-2 and e_s < 2e-2


@pytest.mark.parametrize("variant,H", [("kda", 16), ("gdn2", 16), ("kla", 16), ("gated_deltanet", 16)])
def test_forward_pipelined_from_256_chunks(variant, H):
    """Pipelined from 256 chunks on (here 301: five blocks, the last one
    ragged): a channel decay always, a scalar decay when its scan takes half
    the compute units (B = 1, H = 16); checked on sampled heads."""
    T = 64 * 300 + 17
    inp = make_inputs(variant, 1, T, H, 128, 128, "bf16", seed=87, state_scale=0.3)
    o, s = gpu_forward(variant, to_dev(inp))
    heads = [(0, 0), (0, H - 1)]
    o_ref, s_ref = run_oracle(variant, inp, heads=heads)
    for b, h in heads:
        e_o = rel_err(o[b:b + 1, :, h:h + 1].float().cpu(), o_ref[b:b + 1, :, h:h + 1], (0, 2))
        e_s = rel_err(s[b:b + 1, h:h + 1].cpu(), s_ref[b:b + 1, h:h + 1], (0, 1))
        announce(f"  {variant} head ({b}, {h}): rel_err o={e_o:.3e} S={e_s:.3e}")
        assert e_o < 2e-2 and e_s < 2e-2


@pytest.mark.parametrize("H", [16, 2], ids=["pipelined", "segmented"])
def test_forward_pipelined_split_resume(H):
    """A long pass (576 chunks: pipelined at 16 heads, segmented at 2) equals
    the same sequence split in two calls, the second resuming from the
    first's final state."""
    T = 64 * 64 * 9
    inp = make_inputs("gated_deltanet", 1, T, H, 128, 128, "bf16", seed=79, state_scale=0.2)
    d = to_dev(inp)
    o_all, s_all = gpu_forward("gated_deltanet", d)
    cut = 64 * 64 * 4 + 64 * 5
    part = lambda a, b_: {k: (v[:, a:b_].contiguous() if isinstance(v, torch.Tensor) and k != "state_in"
                              else v) for k, v in d.items()}
    o1, s1 = gpu_forward("gated_deltanet", part(0, cut))
    o2, s2 = gpu_forward("gated_deltanet", part(cut, T), state_in=s1)
    assert rel_err(torch.cat([o1, o2], 1).float().cpu(), o_all.float().cpu(), (0, 2)) < 2e-2
    assert rel_err(s2.cpu(), s_all.cpu(), (0, 1)) < 2e-2


def test_forward_graph_capture_replays():
    """The pipelined forward (513 chunks, one launch per block) captured into a HIP graph
    and replayed several times, with other work in between, matches the eager
    result."""
    T = 64 * 64 * 8 + 64
    inp = make_inputs("kla", 1, T, 16, 128, 128, "bf16", seed=81, state_scale=0.3)
    d = to_dev(inp)
    o_ref, s_ref = gpu_forward("kla", d)
    o = torch.empty_like(o_ref)
    s = torch.empty_like(s_ref)
    nbytes = binding.workspace_bytes("kla", d["q"], d["k"], d["v"])
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def run():
        binding.forward("kla", d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                        eps=d["eps"], state_in=d["state_in"], o=o, state_out=s, workspace=ws)

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
        _ = (d["v"].float() * 2).sum().item()   # unrelated eager work between replays
