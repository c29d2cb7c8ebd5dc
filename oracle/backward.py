"""Parity oracle for the gradient of the gated delta-rule forward pass -- TEST
INFRASTRUCTURE ONLY (same rules as ``oracle.py``: only ``tests/`` may import it;
it shares no code with the GPU library).

The gradient is the plain definition: reverse-mode differentiation (torch
autograd, float64, CPU) of the sequential recurrence written token by token,
one function per variant, in the notation of the pages:

    decay first, S~ = D_t S_{t-1}; then the read along the erase key and the
    write of the residual, S_t = S~ - k_t (a_t^T S~) + k_t u_t^T; the output
    reads the updated state, o_t = S_t^T q_t

("Kaczmarz Linear Attention", KLA update rule: residual e_t = v_t - S~^T k_t
and step S_t = S~ + beta_t k_t e_t^T; "Gated DeltaNet-2", novelty section: the
channel-wise erase gate acts on the key side and the write gate on the value
side; "Linear Attention Architectures", the delta-rule family list.)

The loss whose gradient is returned is  L = sum(o * d_o) + sum(S_T * d_state_out)
for given upstream gradients d_o and d_state_out (either may be None = zero).

Parity status: pinned by central finite differences of the independent C
forward oracle (``gdr_oracle.c``) for every input of every variant, and by the
agreement of the forward pass written here with that oracle; see
``tests/test_oracle_backward.py``.
"""
from __future__ import annotations

import numpy as np
import torch

VARIANTS = ("deltanet", "gated_deltanet", "kda", "gdn2", "kla")


# ---- one token of each variant (S: [dk, dv]) -------------------------------------

def _step_deltanet(S, q, k, v, beta):
    S = S - beta * torch.outer(k, k @ S) + beta * torch.outer(k, v)
    return S, S.T @ q


def _step_gated_deltanet(S, q, k, v, alpha, beta):
    S = alpha * S
    S = S - beta * torch.outer(k, k @ S) + beta * torch.outer(k, v)
    return S, S.T @ q


def _step_kda(S, q, k, v, alpha, beta):
    S = alpha[:, None] * S                    # decay on the key rows
    S = S - beta * torch.outer(k, k @ S) + beta * torch.outer(k, v)
    return S, S.T @ q


def _step_gdn2(S, q, k, v, alpha, erase_b, write_w):
    S = alpha[:, None] * S
    r = (erase_b * k) @ S                      # read along the erase key b (.) k
    S = S - torch.outer(k, r) + torch.outer(k, write_w * v)
    return S, S.T @ q


def _step_kla(S, q, k, v, alpha, eta, eps):
    beta = eta / (k @ k + eps)                 # key-norm-normalised step size
    S = alpha * S
    e = v - S.T @ k                            # residual against the decayed state
    S = S + beta * torch.outer(k, e)
    return S, S.T @ q


def _head_forward(variant, q, k, v, alpha, beta, erase_b, write_w, eps, S):
    """Tokens of one head in order; q, k: [T, dk], v: [T, dv], gates per token."""
    outs = []
    for t in range(q.shape[0]):
        if variant == "deltanet":
            S, o = _step_deltanet(S, q[t], k[t], v[t], beta[t])
        elif variant == "gated_deltanet":
            S, o = _step_gated_deltanet(S, q[t], k[t], v[t], alpha[t], beta[t])
        elif variant == "kda":
            S, o = _step_kda(S, q[t], k[t], v[t], alpha[t], beta[t])
        elif variant == "gdn2":
            S, o = _step_gdn2(S, q[t], k[t], v[t], alpha[t], erase_b[t], write_w[t])
        else:
            S, o = _step_kla(S, q[t], k[t], v[t], alpha[t], beta[t], eps)
        outs.append(o)
    return torch.stack(outs), S


def _t64(x, grad=False):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu", torch.float64)
    else:
        x = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float64)))
    return x.clone().requires_grad_(grad)


def forward(variant, q, k, v, alpha=None, beta=None, erase_b=None, write_w=None,
            eps=0.0, state_in=None):
    """The recurrence in torch float64 (no gradient): (o [B,T,H,dv], S_T [B,H,dk,dv])."""
    with torch.no_grad():
        o, s, _ = _run(variant, q, k, v, alpha, beta, erase_b, write_w, eps, state_in, False)
    return o.numpy(), s.numpy()


def _run(variant, q, k, v, alpha, beta, erase_b, write_w, eps, state_in, grad, heads=None):
    if variant not in VARIANTS:
        raise ValueError(variant)
    ins = dict(q=_t64(q, grad), k=_t64(k, grad), v=_t64(v, grad), alpha=_t64(alpha, grad),
               beta=_t64(beta, grad), erase_b=_t64(erase_b, grad), write_w=_t64(write_w, grad),
               state_in=_t64(state_in, grad))
    B, T, H, dk = ins["q"].shape
    dv = ins["v"].shape[-1]
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float64)
    s_out = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float64)
    o_parts, s_parts = {}, {}
    for b, h in todo:
        g = lambda name: None if ins[name] is None else ins[name][b, :, h]
        S0 = (ins["state_in"][b, h] if ins["state_in"] is not None
              else torch.zeros(dk, dv, dtype=torch.float64))
        o_bh, s_bh = _head_forward(variant, g("q"), g("k"), g("v"), g("alpha"), g("beta"),
                                   g("erase_b"), g("write_w"), float(eps), S0)
        o_parts[(b, h)], s_parts[(b, h)] = o_bh, s_bh
    if not grad:
        for (b, h), x in o_parts.items():
            o[b, :, h] = x
            s_out[b, h] = s_parts[(b, h)]
    return (o, s_out, (ins, o_parts, s_parts)) if grad else (o, s_out, None)


def backward(variant, q, k, v, alpha=None, beta=None, erase_b=None, write_w=None, eps=0.0,
             state_in=None, d_o=None, d_state_out=None, heads=None):
    """Gradients of L = sum(o * d_o) + sum(S_T * d_state_out) with respect to every
    input, as float64 numpy arrays in a dict keyed q, k, v, alpha, beta, erase_b,
    write_w, state_in (None for inputs the variant does not take; the state_in
    gradient is returned even when state_in is None, i.e. for a zero initial
    state).  ``heads`` restricts the work to a list of (b, h); other heads'
    gradients are left as NaN."""
    if state_in is None:
        B, _, H, dk = np.shape(q)
        state_in = np.zeros((B, H, dk, np.shape(v)[-1]))
    _, _, (ins, o_parts, s_parts) = _run(variant, q, k, v, alpha, beta, erase_b, write_w, eps,
                                         state_in, True, heads)
    d_o = None if d_o is None else _t64(d_o)
    d_s = None if d_state_out is None else _t64(d_state_out)
    loss = torch.zeros((), dtype=torch.float64)
    for (b, h), o_bh in o_parts.items():
        if d_o is not None:
            loss = loss + torch.sum(o_bh * d_o[b, :, h])
        if d_s is not None:
            loss = loss + torch.sum(s_parts[(b, h)] * d_s[b, h])
    names = [n for n, t in ins.items() if t is not None]
    grads = torch.autograd.grad(loss, [ins[n] for n in names], allow_unused=True)
    out = {n: None for n in ins}
    sel = None
    if heads is not None:
        sel = np.zeros(ins["q"].shape[0:1] + ins["q"].shape[2:3], dtype=bool)
        for b, h in heads:
            sel[b, h] = True
    for n, gr in zip(names, grads):
        x = torch.zeros_like(ins[n]) if gr is None else gr
        x = x.numpy().copy()
        if sel is not None:
            if n == "state_in":
                x[~sel] = np.nan
            else:
                x[~sel[:, None, :].repeat(x.shape[1], axis=1)] = np.nan
        out[n] = x
    return out


def backward_head_checkpointed(variant, q, k, v, alpha=None, beta=None, erase_b=None,
                               write_w=None, eps=0.0, state_in=None, d_o=None, d_state_out=None,
                               every=64):
    """The same gradient as ``backward`` for one head, in bounded memory: one
    head's inputs q, k [T, dk], v [T, dv], gates [T] or [T, d], state_in
    [dk, dv] (None = zeros), upstream d_o [T, dv] and d_state_out [dk, dv].

    The recurrence runs forward once without a graph, keeping the state at
    every ``every``-th token.  Then, for each segment of ``every`` tokens from
    the last to the first, it runs the segment again from its stored state
    with autograd and takes the gradient of
        sum(o_seg * d_o_seg) + sum(S_end * G_end),
    where G_end is dL/dS at the segment's end (d_state_out for the last
    segment, else what the later segment returned for its start state).  This
    is the chain rule through the token-by-token recurrence, cut at the stored
    states; no chunk form is involved.  Returns a dict of float64 numpy
    arrays shaped like the inputs (None where the variant has no such input),
    with "state_in" always present."""
    prev = torch.get_num_threads()
    torch.set_num_threads(1)   # one head of small products: threads only add overhead
    try:
        return _backward_head_checkpointed(variant, q, k, v, alpha, beta, erase_b, write_w, eps,
                                           state_in, d_o, d_state_out, every)
    finally:
        torch.set_num_threads(prev)


def _backward_head_checkpointed(variant, q, k, v, alpha, beta, erase_b, write_w, eps, state_in,
                                d_o, d_state_out, every):
    T, dk = np.shape(q)[0], np.shape(q)[1]
    dv = np.shape(v)[1]
    raw = dict(q=q, k=k, v=v, alpha=alpha, beta=beta, erase_b=erase_b, write_w=write_w)
    ins = {n: _t64(x) for n, x in raw.items()}
    S = _t64(state_in) if state_in is not None else torch.zeros(dk, dv, dtype=torch.float64)
    d_o = None if d_o is None else _t64(d_o)
    G = (_t64(d_state_out) if d_state_out is not None
         else torch.zeros(dk, dv, dtype=torch.float64))
    starts = list(range(0, T, every))
    saved = []
    with torch.no_grad():
        for t0 in starts:
            saved.append(S.clone())
            sl = {n: (None if x is None else x[t0:t0 + every]) for n, x in ins.items()}
            _, S = _head_forward(variant, sl["q"], sl["k"], sl["v"], sl["alpha"], sl["beta"],
                                 sl["erase_b"], sl["write_w"], float(eps), S)
    out = {n: (None if x is None else np.zeros(tuple(x.shape))) for n, x in ins.items()}
    for t0, S0 in zip(reversed(starts), reversed(saved)):
        leaf = {n: (None if x is None else x[t0:t0 + every].clone().requires_grad_(True))
                for n, x in ins.items()}
        S0 = S0.clone().requires_grad_(True)
        o, S_end = _head_forward(variant, leaf["q"], leaf["k"], leaf["v"], leaf["alpha"],
                                 leaf["beta"], leaf["erase_b"], leaf["write_w"], float(eps), S0)
        loss = torch.sum(S_end * G)
        if d_o is not None:
            loss = loss + torch.sum(o * d_o[t0:t0 + every])
        names = [n for n, x in leaf.items() if x is not None]
        grads = torch.autograd.grad(loss, [leaf[n] for n in names] + [S0], allow_unused=True)
        for n, gr in zip(names, grads[:-1]):
            if gr is not None:
                out[n][t0:t0 + every] = gr.numpy()
        G = grads[-1].detach()
    out["state_in"] = G.numpy()
    return out
