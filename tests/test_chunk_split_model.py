"""CPU model of how the chunked forward splits a channel-wise decay, checked
against the exact Gram products and against the oracle.

Inside a chunk, with g the cumulative log decay per key channel, the Gram
products A[r][s] = sum_i a_r[i] k_s[i] e^{g_r[i] - g_s[i]} (and P with q for a)
need e^{g_r - g_s} <= 1 for s <= r.  The matrix cores take it as the product of
a left factor on the a/q row and a right factor on the k row.  The kernels use
one reference per 16-row block R, m_R = (g_{16R} + g_{16R+15}) / 2: rows are
stored as a e^{g - m_R}, q e^{g - m_R} and k e^{m_S - g} of their own blocks,
and an off-diagonal tile (R, S), S < R, multiplies its k rows by the middle
factor e^{m_R - m_S} <= 1.  With every token's log decay floored at -10, each
stored factor stays within e^{+-75}; the bf16 operands are rounded as the
kernel rounds them.  A single reference in the middle of the 64-row chunk
overflows once a channel decays by more than ~e^{-88} over half a chunk
("Gated DeltaNet-2", technical core: the decay sits in an asymmetric erase
factor of the chunkwise WY algorithm).

The second part runs the whole chunk form in float64 with and without the
floor and compares it with the token-by-token oracle: exact where no decay is
below e^{-10}, and within the float32 tolerance of the exact recurrence below
it.  No GPU code is involved."""
import numpy as np
import pytest
import torch

from oracle import oracle

C = 64
FLOOR = -10.0


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).double().numpy()


def _gram_exact(X, Y, g):
    n = X.shape[0]
    E = np.exp(np.minimum(g[:, None, :] - g[None, :, :], 0.0))   # s <= r entries are <= 0
    G = np.einsum("ri,si,rsi->rs", X, Y, E)
    return np.tril(G)


def _gram_blocks(X, Y, g):
    """The kernel's split: per-block references, middle factors off the diagonal,
    bf16 operands, fp32 exponentials.  Returns (G, max |stored factor|,
    max right factor of any off-diagonal tile)."""
    g = g.astype(np.float32)
    n = X.shape[0]
    blk = np.arange(n) // 16
    mu = np.stack([0.5 * (g[16 * R] + g[16 * R + 15]) for R in range(n // 16)]).astype(np.float32)
    fl = np.exp((g - mu[blk]).astype(np.float32))
    fr = np.exp((mu[blk] - g).astype(np.float32))
    L, K = _bf16(X * fl), _bf16(Y * fr)
    G = np.zeros((n, n))
    worst_off = 0.0
    for R in range(n // 16):
        for S in range(R + 1):
            Kt = K[16 * S:16 * S + 16]
            if S < R:
                m = np.exp((mu[R] - mu[S]).astype(np.float32))
                Kt = _bf16(Kt * m)
                worst_off = max(worst_off, float(np.max(np.exp(mu[R] - g[16 * S:16 * S + 16]))))
            G[16 * R:16 * R + 16, 16 * S:16 * S + 16] = L[16 * R:16 * R + 16] @ Kt.T
    return np.tril(G), float(max(fl.max(), fr.max())), worst_off


def _chunk_inputs(rng, lo, hi, log, dk=128):
    q = rng.standard_normal((C, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((C, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(C)))
    alpha = np.exp(-0.05 * np.log1p(np.exp(rng.standard_normal((C, dk)))))
    pick = rng.random(dk) < 1 / 3
    if log:
        alpha[:, pick] = np.exp(rng.uniform(np.log(lo), np.log(hi), (C, pick.sum())))
    else:
        alpha[:, pick] = rng.uniform(lo, hi, (C, pick.sum()))
    return _bf16(q), _bf16(k), beta, alpha


@pytest.mark.parametrize("lo,hi,log", [(0.8, 1.0, False), (1e-3, 0.05, False),
                                       (1e-5, 1e-3, True), (1e-30, 1e-8, True)])
def test_block_split_is_finite_and_matches_exact_gram(lo, hi, log):
    rng = np.random.default_rng(5)
    for _ in range(3):
        q, k, beta, alpha = _chunk_inputs(rng, lo, hi, log)
        lg = np.log(alpha.astype(np.float32)).astype(np.float64)
        g_exact = np.cumsum(lg, axis=0)
        g_floor = np.cumsum(np.maximum(lg, FLOOR), axis=0)
        a = beta[:, None] * k
        for X, strict in ((a, True), (q, False)):
            G, fmax, off = _gram_blocks(X, k, g_floor)
            ref = _gram_exact(X, k, g_exact)
            if strict:
                G, ref = np.tril(G, -1), np.tril(ref, -1)
            assert np.isfinite(G).all()
            assert fmax <= np.exp(75.0) * 1.0001       # within e^{7.5 * 10}
            assert off <= 1.0 + 1e-6                    # off-diagonal right factors <= 1
            # bf16 operands: ~2^-8 relative per entry, normwise over the chunk
            assert np.max(np.abs(G - ref)) / np.max(np.abs(ref)) < 1e-2


def test_single_reference_overflows_where_blocks_do_not():
    """The split the kernels used before: one reference g_{31} for the chunk."""
    rng = np.random.default_rng(6)
    q, k, beta, alpha = _chunk_inputs(rng, 0.01, 0.02, False)
    g = np.cumsum(np.log(alpha), axis=0).astype(np.float32)
    with np.errstate(over="ignore"):
        fl = np.exp(g - g[C // 2 - 1]).astype(np.float32)
    assert not np.isfinite(fl).all()
    G, _, _ = _gram_blocks(q, k, g)
    assert np.isfinite(G).all()


def _chunk_forward(q, k, v, alpha, beta, floor=None):
    """Kimi Delta Attention by the chunk form, float64, one head."""
    T, dk = q.shape
    S = np.zeros((dk, v.shape[1]))
    o = np.zeros((T, v.shape[1]))
    lg = np.log(alpha)
    if floor is not None:
        lg = np.maximum(lg, floor)
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        n = sl.stop - sl.start
        g = np.cumsum(lg[sl], axis=0)
        a, u = beta[sl, None] * k[sl], beta[sl, None] * v[sl]
        A = np.tril(_gram_exact(a, k[sl], g), -1)
        P = _gram_exact(q[sl], k[sl], g)
        Tm = np.linalg.inv(np.eye(n) + A)
        W, U = Tm @ (a * np.exp(g)), Tm @ u
        D = U - W @ S
        o[sl] = (q[sl] * np.exp(g)) @ S + P @ D
        S = np.exp(g[-1])[:, None] * S + (k[sl] * np.exp(g[-1] - g)).T @ D
    return o, S


@pytest.mark.parametrize("lo,hi,log,bound", [(1e-3, 0.05, False, 1e-12),
                                             (1e-6, 1e-4, True, 1e-4),
                                             (1e-30, 1e-10, True, 1e-4)])
def test_floored_chunk_form_against_oracle(lo, hi, log, bound):
    rng = np.random.default_rng(7)
    T, dk, dv = 200, 64, 32
    q = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    alpha = np.exp(-0.05 * np.log1p(np.exp(rng.standard_normal((T, dk)))))
    pick = rng.random(dk) < 1 / 3
    draw = (np.exp(rng.uniform(np.log(lo), np.log(hi), (T, pick.sum()))) if log
            else rng.uniform(lo, hi, (T, pick.sum())))
    alpha[:, pick] = draw
    o_ref, s_ref = oracle.forward("kda", q[None, :, None], k[None, :, None], v[None, :, None],
                                  alpha=alpha[None, :, None], beta=beta[None, :, None])
    o_ref, s_ref = o_ref[0, :, 0], s_ref[0, 0]
    exact_o, exact_s = _chunk_forward(q, k, v, alpha, beta)
    # the unfloored chunk form is the recurrence (an identity)
    assert np.max(np.abs(exact_o - o_ref)) / np.max(np.abs(o_ref)) < 1e-12
    assert np.max(np.abs(exact_s - s_ref)) / np.max(np.abs(s_ref)) < 1e-12
    o, s = _chunk_forward(q, k, v, alpha, beta, floor=FLOOR)
    assert np.max(np.abs(o - o_ref)) / np.max(np.abs(o_ref)) < bound
    assert np.max(np.abs(s - s_ref)) / np.max(np.abs(s_ref)) < bound
