"""Chunked (UT-transform) regrouping of the gated delta rule in fp64 numpy --
TEST INFRASTRUCTURE ONLY.

The Track L pull request (tessera #77, "What landed") and the
GatedDeltaRule.ixx File Reference ("Detailed Description") describe a second
form of the rule for prefill: it regroups the identical arithmetic of the
recurrence into chunks, with one forward substitution of (I + A) per chunk of
32 steps, and agrees with the recurrence up to float reassociation.  The pages
print the shape of that form but not its formulas; this module writes them out
from the recurrence itself (derivation below) so that the tests can check the
regrouping against ``oracle.fwd`` for many chunk sizes.  It is not the oracle
(the recurrence is) -- it is the pinned statement of the algebra that a
chunked kernel has to reproduce.

Derivation, one chunk of length c, state S0 at chunk entry, rows r = 1..c:
gamma_r = g_1 + ... + g_r (in-chunk cumulative log decay), Gamma_r = exp(gamma_r).
Unrolling S_r = alpha_r S_{r-1} + k_r delta_r^T gives
    S_r = Gamma_r S0 + sum_{i<=r} exp(gamma_r - gamma_i) k_i delta_i^T,
and putting that into delta_r = beta_r (v_r - (alpha_r S_{r-1})^T k_r) gives
    (I + A) Delta = diag(beta) V - diag(beta * Gamma) K S0,
    A[r, i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)      for i < r, else 0.
With T = (I + A)^-1 (unit lower triangular, by forward substitution):
    W = T diag(beta * Gamma) K,   U = T diag(beta) V,   Delta = U - W S0,
    P[r, i] = exp(gamma_r - gamma_i) (q_r . k_i)            for i <= r, else 0,
    O = diag(Gamma) Q S0 + P Delta,
    S_c = Gamma_c S0 + (diag(exp(gamma_c - gamma)) K)^T Delta.
Only differences gamma_r - gamma_i with i <= r are ever exponentiated, so no
factor exceeds 1 (the ratio form Gamma_r / Gamma_i overflows once gamma is
large and negative; ``ratio_form=True`` reproduces that mistake for a test).
"""
from __future__ import annotations

import numpy as np

from . import f64, gates, default_scale


def forward_substitution_inverse(A: np.ndarray) -> np.ndarray:
    """T = (I + A)^-1 for strictly lower triangular A, one row at a time:
    T[r, :] = e_r - sum_{i<r} A[r, i] T[i, :]."""
    c = A.shape[0]
    T = np.zeros_like(A)
    for r in range(c):
        T[r, r] = 1.0
        for i in range(r):
            T[r, :] -= A[r, i] * T[i, :]
    return T


def chunk_step(Q, K, V, g, beta, S0, ratio_form=False, dtype=np.float64):
    """One chunk: returns (O [c, d_v], S_c [d_k, d_v], T, W, U)."""
    Q, K, V, g, beta, S0 = (np.asarray(x, dtype=dtype) for x in (Q, K, V, g, beta, S0))
    c = K.shape[0]
    gam = np.cumsum(g)
    low_strict = np.tril(np.ones((c, c), dtype=bool), -1)
    low_incl = np.tril(np.ones((c, c), dtype=bool))
    if ratio_form:
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            E = np.exp(gam)[:, None] / np.exp(gam)[None, :]
    else:
        diff = np.where(low_incl, gam[:, None] - gam[None, :], 0.0)
        E = np.where(low_incl, np.exp(diff), 0.0)
    with np.errstate(over="ignore", invalid="ignore"):
        A = np.where(low_strict, beta[:, None] * E * (K @ K.T), 0.0).astype(dtype)
        T = forward_substitution_inverse(A)
        Gam = np.exp(gam)
        W = T @ ((beta * Gam)[:, None] * K)
        U = T @ (beta[:, None] * V)
        Delta = U - W @ S0
        P = np.where(low_incl, E * (Q @ K.T), 0.0)
        O = Gam[:, None] * (Q @ S0) + P @ Delta
        if ratio_form:
            tail = (np.exp(gam[-1]) / np.exp(gam))[:, None]
        else:
            tail = np.exp(gam[-1] - gam)[:, None]
        S = Gam[-1] * S0 + (tail * K).T @ Delta
    return O, S, T, W, U


def chunked_head(q_hat, k_hat, v, g, beta, S0, chunk, ratio_form=False, dtype=np.float64):
    """Chunked pass over one (sequence, value head): q_hat, k_hat [L, d_k]
    (already normalised, q_hat scaled), v [L, d_v], g, beta [L], S0 [d_k, d_v]."""
    L = k_hat.shape[0]
    S = np.array(S0, dtype=dtype)
    O = np.zeros((L, v.shape[1]), dtype=dtype)
    for s in range(0, L, chunk):
        e = min(s + chunk, L)
        O[s:e], S, _, _, _ = chunk_step(q_hat[s:e], k_hat[s:e], v[s:e], g[s:e], beta[s:e], S,
                                        ratio_form=ratio_form, dtype=dtype)
    return O, S


def fwd(q, k, v, a, b, A_log, dt_bias, chunk, initial_state=None, cu_seqlens=None,
        num_seqs=None, scale=None, l2_eps=1e-6, ratio_form=False, dtype=np.float64):
    """Chunked form over a whole batch, same arguments and layout as
    ``oracle.fwd``; chunks restart at every sequence start."""
    q, k, v = f64(q), f64(k), f64(v)
    total, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    G = H_v // H_k
    scale = default_scale(d_k) if scale is None or scale <= 0 else float(scale)
    q_hat, k_hat, g, beta = gates(q, k, a, b, A_log, dt_bias, scale=scale, l2_eps=l2_eps)
    if cu_seqlens is None:
        N = 1 if num_seqs is None else num_seqs
        cu = np.arange(N + 1) * (total // N)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        N = len(cu) - 1
    s0 = np.zeros((N, H_v, d_k, d_v)) if initial_state is None else f64(initial_state)
    o = np.zeros((total, H_v, d_v), dtype=dtype)
    S = np.zeros((N, H_v, d_k, d_v), dtype=dtype)
    for n in range(N):
        t0, t1 = cu[n], cu[n + 1]
        for h in range(H_v):
            hk = h // G
            o[t0:t1, h], S[n, h] = chunked_head(q_hat[t0:t1, hk], k_hat[t0:t1, hk], v[t0:t1, h],
                                                g[t0:t1, h], beta[t0:t1, h], s0[n, h], chunk,
                                                ratio_form=ratio_form, dtype=dtype)
    return o, S
