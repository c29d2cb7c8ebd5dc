"""Calls from several host threads at once (the header promises that the
entry points may be called concurrently).

Each thread runs pipelined forwards on a stream of its own.  A pipelined
forward runs each block's scan beside the next block's prep in one launch,
with grids sized from per-device caches (compute units, resident workgroups)
that the first calls fill.  ctypes releases the interpreter lock during a foreign call, so
the threads' calls and their device work overlap.  Every result must equal,
bit for bit, the same call made alone: the forward's arithmetic per chunk and
per column slice does not depend on which workgroup takes an item."""
import threading

import pytest
import torch

from gated_delta_rule_85_amd import binding
from gated_delta_rule_85_amd.inputs import make_inputs
from tests.gpu_common import announce, to_dev

pytestmark = pytest.mark.gpu

# (variant, B, T, H, seed): KDA from 256 chunks and Gated DeltaNet from 512
# chunks (at 16 heads) run pipelined, both with a ragged last chunk; KLA at 4
# heads runs as segments whose chains run side by side.
CASES = [("kda", 1, 300 * 64 + 17, 16, 910), ("gated_deltanet", 1, 520 * 64 + 5, 16, 911),
         ("kla", 1, 530 * 64, 4, 912)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.lib()


def _call(variant, d, stream):
    with torch.cuda.stream(stream):
        o, s = binding.forward(variant, d["q"], d["k"], d["v"], alpha=d["alpha"], beta=d["beta"],
                               erase_b=d["erase_b"], write_w=d["write_w"], eps=d["eps"],
                               state_in=d["state_in"], stream=stream)
    return o, s


def test_concurrent_pipelined_forwards_match_lone_calls():
    inputs = []
    for variant, B, T, H, seed in CASES:
        inp = make_inputs(variant, B, T, H, 128, 128, "bf16", seed=seed, state_scale=0.3)
        inputs.append((variant, to_dev(inp)))
    # the same calls made alone, one after another
    main = torch.cuda.current_stream()
    ref = [_call(variant, d, main) for variant, d in inputs]
    torch.cuda.synchronize()
    announce("lone calls done; starting one thread per case, 3 calls each")

    results, errors = {}, []

    def worker(i):
        try:
            variant, d = inputs[i]
            stream = torch.cuda.Stream()
            outs = [_call(variant, d, stream) for _ in range(3)]
            stream.synchronize()
            results[i] = outs
        except Exception as exc:   # reported in the main thread
            errors.append((i, repr(exc)))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(inputs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, (variant, _) in enumerate(inputs):
        o_ref, s_ref = ref[i]
        for n, (o, s) in enumerate(results[i]):
            assert torch.equal(o, o_ref), f"{variant} call {n}: o differs from the lone call"
            assert torch.equal(s, s_ref), f"{variant} call {n}: final state differs"
        announce(f"  {variant}: 3 concurrent calls equal the lone call")
