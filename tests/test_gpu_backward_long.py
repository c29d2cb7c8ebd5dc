"""Element-wise parity of the gradient at long lengths, against the
chunk-checkpointed float64 gradient oracle (``oracle.backward.
backward_head_checkpointed``: the token-by-token recurrence differentiated
segment by segment from stored states, equal to the plain gradient oracle).

* The benchmarked Kaczmarz prefill, B=1, H=16, T=65536 (1,024 chunks): every
  head's gradient on the GPU, every input's gradient of one sampled head
  compared entry by entry with the oracle.
* Kimi Delta Attention and Gated DeltaNet-2 at 257 chunks (the last one
  ragged), one sampled head each; with two heads both chains run in segments.
* The few-head Kaczmarz gradient, B=1, H=4, T=65536, and Kimi Delta
  Attention at 8 heads and 257 chunks, segmented likewise.

Error measure and thresholds as in the other gradient tests: per head,
max |x - ref| / max |ref|, bf16 inputs 2e-2."""
import numpy as np
import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import (WORKLOADS, make_inputs, make_upstream_grads,
                                            make_workload)
from oracle import backward as oracle_bw
from tests.gpu_common import announce, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def _check(variant, inp, up, b, h):
    d, du = to_dev(inp), to_dev(up)
    g = binding.backward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                         erase_b=d["erase_b"], write_w=d["write_w"], eps=d["eps"],
                         state_in=d["state_in"], d_o=du["d_o"], d_state_out=du["d_state_out"])
    torch.cuda.synchronize()
    got = {n: (None if x is None else (x[b, h] if n == "state_in" else x[b, :, h]).cpu().numpy())
           for n, x in g.items()}
    del g, d, du
    torch.cuda.empty_cache()
    sel = lambda x: None if x is None else x[b, :, h].double().numpy()
    s0 = inp["state_in"]
    ref = oracle_bw.backward_head_checkpointed(
        variant, sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["alpha"]), sel(inp["beta"]),
        sel(inp["erase_b"]), sel(inp["write_w"]), inp["eps"],
        None if s0 is None else s0[b, h].double().numpy(),
        sel(up["d_o"]), up["d_state_out"][b, h].double().numpy())
    errs = {}
    for n, r in ref.items():
        if r is None:
            assert got.get(n) is None, n
            continue
        assert np.isfinite(got[n]).all(), f"non-finite gradient {n}"
        errs[n] = rel_err(got[n][None], r[None], (0,))
    announce(f"  grad {variant} T={inp['q'].shape[1]} head ({b},{h}): " +
             " ".join(f"{n}={e:.1e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e < 2e-2}
    assert not bad, bad


def test_backward_benchmarked_prefill_sampled_head():
    """B=1, H=16, T=65536 Kaczmarz, bf16; 1,024 chunks in every pass."""
    wl = WORKLOADS[5]
    announce(f"gradient {wl.name} (full length), oracle on head 11")
    inp = make_workload(wl)
    up = make_upstream_grads(wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.dtype, seed=wl.seed + 1)
    _check("kla", inp, up, 0, 11)


@pytest.mark.parametrize("variant", ["kda", "gdn2"])
def test_backward_257_chunks_channel_decay(variant):
    T = 257 * 64 - 21
    announce(f"gradient {variant} T={T}, oracle on head 1")
    inp = make_inputs(variant, 1, T, 2, 128, 128, "bf16", seed=77, alpha_scale=0.05,
                      state_scale=0.1)
    up = make_upstream_grads(1, T, 2, 128, 128, "bf16", seed=78)
    _check(variant, inp, up, 0, 1)


def test_backward_few_heads_segmented_sampled_head():
    """The few-head Kaczmarz gradient the benchmark times (B=1, H=4,
    T=65536, its inputs and upstream gradients): 1,024 chunks, both the
    states pass and the reverse pass in 8 segments; head 3 against the
    oracle."""
    announce("gradient kla B=1 H=4 T=65536 (segmented), oracle on head 3")
    inp = make_inputs("kla", 1, 65536, 4, 128, 128, "bf16", seed=85104)
    up = make_upstream_grads(1, 65536, 4, 128, 128, "bf16", seed=85204)
    _check("kla", inp, up, 0, 3)


def test_backward_eight_heads_segmented_sampled_head():
    """Kimi Delta Attention at 8 heads (a quarter of the compute units in
    column slices: both chains in 4 segments), 257 chunks with a ragged last
    one; head 5 against the oracle."""
    T = 257 * 64 - 21
    announce(f"gradient kda B=1 H=8 T={T} (segmented), oracle on head 5")
    inp = make_inputs("kda", 1, T, 8, 128, 128, "bf16", seed=79, alpha_scale=0.05,
                      state_scale=0.1)
    up = make_upstream_grads(1, T, 8, 128, 128, "bf16", seed=80)
    _check("kda", inp, up, 0, 5)
