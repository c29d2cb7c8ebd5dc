"""Shared helpers of the GPU parity tests (no test cases here)."""
import numpy as np
import torch

from oracle import oracle

# Pass thresholds of the normwise error below: float32 inputs 1e-4, bfloat16
# inputs 2e-2 (bf16 rounding of the inputs to the matrix cores and of the
# output is ~2^-9 per element; the fp32 state keeps errors from growing).
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}

GATE_KEYS = ("alpha", "beta", "erase_b", "write_w", "state_in")


def to_dev(inp, device="cuda"):
    out = {}
    for key, val in inp.items():
        out[key] = val.to(device).contiguous() if isinstance(val, torch.Tensor) else val
    return out


def rel_err(x, ref, head_axes):
    """max over heads of max|x - ref| / max|ref| within the head.

    ``head_axes`` are the axes that index a head, e.g. (0, 2) for o [B,T,H,dv]
    and (0, 1) for a state [B,H,dk,dv]."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    other = tuple(a for a in range(x.ndim) if a not in head_axes)
    num = np.max(np.abs(x - ref), axis=other)
    den = np.maximum(np.max(np.abs(ref), axis=other), 1e-30)
    return float(np.max(num / den))


def run_oracle(variant, inp, heads=None, state_in=None):
    s0 = inp.get("state_in") if state_in is None else state_in
    return oracle.forward(variant, inp["q"], inp["k"], inp["v"], alpha=inp.get("alpha"),
                          beta=inp.get("beta"), erase_b=inp.get("erase_b"),
                          write_w=inp.get("write_w"), eps=inp.get("eps", 0.0),
                          state_in=s0, heads=heads)


def gpu_forward(variant, d, state_in=None, output_state=True):
    from gated_delta_rule_85_amd import binding
    o, s = binding.forward(variant, d["q"], d["k"], d["v"], alpha=d.get("alpha"),
                           beta=d.get("beta"), erase_b=d.get("erase_b"),
                           write_w=d.get("write_w"), eps=d.get("eps", 0.0),
                           state_in=d.get("state_in") if state_in is None else state_in,
                           output_state=output_state)
    torch.cuda.synchronize()
    return o, s


def announce(msg):
    print(msg, flush=True)
