"""Seeded synthetic inputs for the gated delta-rule forward pass.

This module only draws and stores random tensors; it holds none of the
method's arithmetic, so both the GPU path and the oracle can take their
inputs from it.

Distributions (one layer, one head group):
  * q ~ N(0,1) then L2-normalised over the key dimension of each (b, t, h);
  * k ~ N(0,1) then L2-normalised the same way, except for the Kaczmarz
    workload, whose keys keep their norm: k = N(0,1) * LogNormal(0, 0.5),
    one log-normal factor per (b, t, h) scaling the whole key vector;
  * v ~ N(0,1);
  * scalar decay alpha = exp(-softplus(N(0,1)) * s) per (b, t, h), or one such
    value per key channel for the channel-wise variants;
  * beta, eta, erase gate b and write gate w = sigmoid(N(0,1)).

Draw order from ``numpy.random.default_rng(seed)``: q, k (and the log-normal
key scale), v, then the gates in the order alpha, beta/eta, b, w.  Values are
drawn in float32; q, k, v are then stored in the requested dtype (bf16 by
round-to-nearest-even through torch) and gates stay float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

VARIANTS = ("deltanet", "gated_deltanet", "kda", "gdn2", "kla")


@dataclass(frozen=True)
class Workload:
    name: str
    variant: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str          # "fp32" or "bf16": storage type of q, k, v and o
    seed: int
    alpha_scale: float = 0.1
    eps: float = 0.0
    unnormalised_keys: bool = False
    decode: dict = field(default_factory=dict)


# The five layer shapes measured here.
WORKLOADS = {
    1: Workload("deltanet_fp32_B1_H2_T256_d64", "deltanet", 1, 2, 256, 64, 64,
                "fp32", 85001),
    2: Workload("gated_deltanet_bf16_B4_H8_T4096_d128", "gated_deltanet", 4, 8,
                4096, 128, 128, "bf16", 85002, alpha_scale=0.1),
    3: Workload("kda_bf16_B4_H8_T4096_d128", "kda", 4, 8, 4096, 128, 128,
                "bf16", 85003, alpha_scale=0.05),
    4: Workload("gdn2_bf16_B2_H16_T8192_d128", "gdn2", 2, 16, 8192, 128, 128,
                "bf16", 85004, alpha_scale=0.05),
    5: Workload("kla_bf16_B1_H16_T65536_d128_decode_B64x1024", "kla", 1, 16,
                65536, 128, 128, "bf16", 85005, alpha_scale=0.1, eps=1e-6,
                unnormalised_keys=True,
                decode=dict(B=64, steps=1024, seed=85105)),
    # Long-context efficiency shapes: prefill of a 131,072-token context, and
    # single-sequence decode from the state after a 32,768-token prefill, for
    # the Kaczmarz layer and its Gated DeltaNet counterpart (same shapes and
    # gates; only the step size differs).
    6: Workload("kla_bf16_B1_H16_T131072_d128_decode_at_32768", "kla", 1, 16,
                131072, 128, 128, "bf16", 85006, alpha_scale=0.1, eps=1e-6,
                unnormalised_keys=True,
                decode=dict(B=1, steps=256, seed=85106, position=32768)),
    7: Workload("gated_deltanet_bf16_B1_H16_T131072_d128_decode_at_32768", "gated_deltanet",
                1, 16, 131072, 128, 128, "bf16", 85007, alpha_scale=0.1,
                decode=dict(B=1, steps=256, seed=85107, position=32768)),
}


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def _l2norm_last(x):
    # Row by row in float64, in slices that stay in cache (same values as one
    # whole-array pass).
    flat = x.reshape(-1, x.shape[-1])
    out = np.empty(flat.shape, dtype=np.float32)
    step = 1 << 14
    for i in range(0, flat.shape[0], step):
        blk = flat[i:i + step]
        n = np.sqrt(np.sum(blk.astype(np.float64) ** 2, axis=-1, keepdims=True))
        out[i:i + step] = blk / np.maximum(n, 1e-30)
    return out.reshape(x.shape)


def _store(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def make_inputs(variant, B, T, H, dk, dv, dtype="bf16", seed=0,
                alpha_scale=0.1, eps=None, unnormalised_keys=None,
                state_scale=0.0):
    """Draw one problem.  Returns a dict of CPU torch tensors:
    q, k [B,T,H,dk], v [B,T,H,dv] in ``dtype``; alpha, beta, erase_b, write_w
    float32 (None where the variant has no such gate); eps (float); state_in
    float32 [B,H,dk,dv] drawn N(0,1)*state_scale, or None when state_scale==0.
    """
    if variant not in VARIANTS:
        raise ValueError(variant)
    if unnormalised_keys is None:
        unnormalised_keys = variant == "kla"
    if eps is None:
        eps = 1e-6 if variant == "kla" else 0.0
    rng = np.random.default_rng(seed)
    q = _l2norm_last(_normal(rng, (B, T, H, dk)))
    k = _normal(rng, (B, T, H, dk))
    if unnormalised_keys:
        scale = np.exp(0.5 * _normal(rng, (B, T, H, 1)))
        k = (k * scale).astype(np.float32)
    else:
        k = _l2norm_last(k)
    v = _normal(rng, (B, T, H, dv))
    out = dict(q=_store(q, dtype), k=_store(k, dtype), v=_store(v, dtype),
               alpha=None, beta=None, erase_b=None, write_w=None, eps=float(eps),
               state_in=None)
    if variant in ("gated_deltanet", "kla"):
        out["alpha"] = torch.from_numpy(
            np.exp(-_softplus(_normal(rng, (B, T, H))) * alpha_scale).astype(np.float32))
    elif variant in ("kda", "gdn2"):
        out["alpha"] = torch.from_numpy(
            np.exp(-_softplus(_normal(rng, (B, T, H, dk))) * alpha_scale).astype(np.float32))
    if variant != "gdn2":
        out["beta"] = torch.from_numpy(_sigmoid(_normal(rng, (B, T, H))).astype(np.float32))
    else:
        out["erase_b"] = torch.from_numpy(_sigmoid(_normal(rng, (B, T, H, dk))).astype(np.float32))
        out["write_w"] = torch.from_numpy(_sigmoid(_normal(rng, (B, T, H, dv))).astype(np.float32))
    if state_scale:
        out["state_in"] = torch.from_numpy(
            (_normal(rng, (B, H, dk, dv)) * state_scale).astype(np.float32))
    return out


def make_raw_inputs(variant, B, T, H, dk, dv, dtype="bf16", seed=0, state_scale=0.1):
    """Draw pre-activation inputs for the on-load transforms: q, k, v ~ N(0,1)
    (q and k not normalised), and every gate tensor ~ N(0,1) as a
    pre-activation (alpha per (b,t,h) or per key channel by variant).  Same
    dict layout as ``make_inputs``; the state_in is N(0,1) * state_scale."""
    if variant not in VARIANTS:
        raise ValueError(variant)
    rng = np.random.default_rng(seed)
    out = dict(q=_store(_normal(rng, (B, T, H, dk)), dtype),
               k=_store(_normal(rng, (B, T, H, dk)), dtype),
               v=_store(_normal(rng, (B, T, H, dv)), dtype),
               alpha=None, beta=None, erase_b=None, write_w=None,
               eps=1e-6 if variant == "kla" else 0.0, state_in=None)
    if variant in ("gated_deltanet", "kla"):
        out["alpha"] = torch.from_numpy(_normal(rng, (B, T, H)))
    elif variant in ("kda", "gdn2"):
        out["alpha"] = torch.from_numpy(_normal(rng, (B, T, H, dk)))
    if variant != "gdn2":
        out["beta"] = torch.from_numpy(_normal(rng, (B, T, H)))
    else:
        out["erase_b"] = torch.from_numpy(_normal(rng, (B, T, H, dk)))
        out["write_w"] = torch.from_numpy(_normal(rng, (B, T, H, dv)))
    if state_scale:
        out["state_in"] = torch.from_numpy((_normal(rng, (B, H, dk, dv)) * state_scale))
    return out


def with_strong_channel_decay(inp, frac=1 / 3, lo=1e-3, hi=0.05, seed=0, log=False):
    """Replace the per-channel decay of ``frac`` of the key channels of every
    head by values drawn uniformly from [lo, hi] (one draw per (b, t, h, i);
    with ``log``, uniformly in log(alpha) between log(lo) and log(hi)).
    The channels are drawn per (b, h).  Returns a new dict; the other tensors
    are shared.  Strong channel-wise decay is what sets the Kimi and Gated
    DeltaNet-2 variants apart from a scalar forget gate."""
    alpha = inp["alpha"]
    if alpha is None or alpha.dim() != 4:
        raise ValueError("needs a per-channel decay [B, T, H, dk]")
    rng = np.random.default_rng(seed)
    B, T, H, dk = alpha.shape
    pick = rng.random((B, 1, H, dk)) < frac
    if log:
        strong = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(B, T, H, dk)))
    else:
        strong = rng.uniform(lo, hi, size=(B, T, H, dk))
    a = np.where(pick, strong, alpha.numpy().astype(np.float64)).astype(np.float32)
    out = dict(inp)
    out["alpha"] = torch.from_numpy(a)
    return out


def with_strong_scalar_decay(inp, frac=1 / 3, lo=1e-3, hi=0.05, seed=0, log=False):
    """Replace the scalar decay of ``frac`` of the tokens of every (b, h) by
    values drawn uniformly from [lo, hi] (with ``log``, uniformly in log(alpha)
    between log(lo) and log(hi)).  Returns a new dict; the other tensors are
    shared.  For the variants whose forget gate is one scalar per head and
    token (Gated DeltaNet, Kaczmarz)."""
    alpha = inp["alpha"]
    if alpha is None or alpha.dim() != 3:
        raise ValueError("needs a scalar decay [B, T, H]")
    rng = np.random.default_rng(seed)
    pick = rng.random(tuple(alpha.shape)) < frac
    if log:
        strong = np.exp(rng.uniform(np.log(lo), np.log(hi), size=tuple(alpha.shape)))
    else:
        strong = rng.uniform(lo, hi, size=tuple(alpha.shape))
    a = np.where(pick, strong, alpha.numpy().astype(np.float64)).astype(np.float32)
    out = dict(inp)
    out["alpha"] = torch.from_numpy(a)
    return out


def make_routed_value(B, T, H, dv, dtype="bf16", seed=0, scale=1.0):
    """A value routed in from another layer, N(0,1) * scale [B,T,H,dv] in ``dtype``."""
    rng = np.random.default_rng(seed)
    return _store(_normal(rng, (B, T, H, dv)) * scale, dtype)


def make_upstream_grads(B, T, H, dk, dv, dtype="bf16", seed=0):
    """Upstream gradients of the forward's two outputs for a gradient check:
    d_o ~ N(0,1) [B,T,H,dv] stored in ``dtype`` and d_state_out ~ N(0,1)
    [B,H,dk,dv] float32, drawn in that order."""
    rng = np.random.default_rng(seed)
    d_o = _store(_normal(rng, (B, T, H, dv)), dtype)
    d_s = torch.from_numpy(_normal(rng, (B, H, dk, dv)))
    return dict(d_o=d_o, d_state_out=d_s)


def make_workload(wl: Workload, T=None, B=None, H=None):
    """Inputs of a named workload, optionally cut to a shorter sequence or
    fewer batch rows / heads (the draw keeps the workload's seed)."""
    return make_inputs(wl.variant, B or wl.B, T or wl.T, H or wl.H, wl.dk, wl.dv,
                       wl.dtype, wl.seed, alpha_scale=wl.alpha_scale,
                       eps=wl.eps, unnormalised_keys=wl.unnormalised_keys)


def make_decode_inputs(wl: Workload, steps=None, B=None):
    """Per-step decode inputs for a workload with a decode phase: tensors with
    a leading step axis, q, k [S,B,1,H,dk], v [S,B,1,H,dv], gates [S,B,1,H(,d)]."""
    d = wl.decode
    S = steps or d["steps"]
    Bd = B or d["B"]
    rng = np.random.default_rng(d["seed"])
    H, dk, dv = wl.H, wl.dk, wl.dv
    q = _l2norm_last(_normal(rng, (S, Bd, 1, H, dk)))
    k = _normal(rng, (S, Bd, 1, H, dk))
    if wl.unnormalised_keys:
        k = (k * np.exp(0.5 * _normal(rng, (S, Bd, 1, H, 1)))).astype(np.float32)
    else:
        k = _l2norm_last(k)
    v = _normal(rng, (S, Bd, 1, H, dv))
    out = dict(q=_store(q, wl.dtype), k=_store(k, wl.dtype), v=_store(v, wl.dtype),
               alpha=None, beta=None, erase_b=None, write_w=None, eps=float(wl.eps))
    variant = wl.variant
    if variant in ("gated_deltanet", "kla"):
        out["alpha"] = torch.from_numpy(
            np.exp(-_softplus(_normal(rng, (S, Bd, 1, H))) * wl.alpha_scale).astype(np.float32))
    elif variant in ("kda", "gdn2"):
        out["alpha"] = torch.from_numpy(
            np.exp(-_softplus(_normal(rng, (S, Bd, 1, H, dk))) * wl.alpha_scale).astype(np.float32))
    if variant != "gdn2":
        out["beta"] = torch.from_numpy(_sigmoid(_normal(rng, (S, Bd, 1, H))).astype(np.float32))
    else:
        out["erase_b"] = torch.from_numpy(_sigmoid(_normal(rng, (S, Bd, 1, H, dk))).astype(np.float32))
        out["write_w"] = torch.from_numpy(_sigmoid(_normal(rng, (S, Bd, 1, H, dv))).astype(np.float32))
    return out
