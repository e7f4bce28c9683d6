"""Oracle for the per-channel-decay variant of the rule (KDA) -- TEST
INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library never does, and this
module imports nothing from it.

The pages name the variant (the Mamba + KDA pull requests of the PLENA
compiler and simulator: a KDA functional core beside the Mamba-2 one, an fp32
recurrent state) but print no formula.  The reading taken here is the rule of
GatedDeltaRule.ixx File Reference ("Detailed Description") with its scalar
decay exp(g_t) replaced by one decay per key channel, i.e. a diagonal matrix
on the state's rows; everything else is the rule's:
    g_t[i] = -exp(A_log[h]) * softplus(a_t[i] + dt_bias[h, i])   (i < d_k)
    beta_t = sigmoid(b_t)
    S      <- diag(exp(g_t)) S
    delta  <- beta_t (v_t - k^_t^T S)
    S      <- S + k^_t (outer) delta
    o_t    <- q^_t^T S
with k^ = k / sqrt(|k|^2 + eps) and q^ = scale q / sqrt(|q|^2 + eps).
Shapes: q, k [total, H_k, d_k]; v [total, H_v, d_v]; a [total, H_v, d_k];
b [total, H_v]; A_log [H_v]; dt_bias [H_v, d_k]; states [S, H_v, d_k, d_v].

``kda`` is the sequential recurrence in that order, in fp64 numpy.
``kda_chunked`` regroups the same arithmetic into chunks (the UT-transform
form with channel-weighted Gram matrices); only the pins use it.
``MUTATION`` plants one mistake at a time for the tests that show each pin
can fail.
"""
from __future__ import annotations

import numpy as np

from . import f64

MUTATION = 0
_MUTATIONS = {
    1: "decay on the value columns",
    2: "dt_bias of channel 0 for every channel",
    3: "gate of channel 0 for every channel",
    4: "erase from the undecayed state",
    5: "output read before the write",
    6: "unnormalised k",
    7: "softplus replaced by exp",
}


def _softplus(x):
    if MUTATION == 7:
        return np.exp(x)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _cu(total, cu_seqlens, num_seqs):
    if cu_seqlens is not None:
        return [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    n = 1 if num_seqs is None else int(num_seqs)
    L = total // n if n else 0
    return [i * L for i in range(n + 1)]


def gates(a, b, A_log, dt_bias):
    """g [total, H_v, d_k] and beta [total, H_v] from the raw projections."""
    a, b, A_log, dt_bias = f64(a), f64(b), f64(A_log), f64(dt_bias)
    dtb = dt_bias
    if MUTATION == 2:
        dtb = np.repeat(dt_bias[:, :1], dt_bias.shape[1], axis=1)
    g = -np.exp(A_log)[None, :, None] * _softplus(a + dtb[None])
    if MUTATION == 3:
        g = np.repeat(g[:, :, :1], g.shape[2], axis=2)
    beta = 1.0 / (1.0 + np.exp(-b))
    return g, beta


def _norm(x, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def kda(q, k, v, a, b, A_log, dt_bias, initial_state=None, cu_seqlens=None, num_seqs=None,
        scale=None, l2_eps=1e-6, erase=True):
    """Sequential recurrence.  Returns (o [total, H_v, d_v], final [S, H_v, d_k, d_v]).
    ``erase=False`` drops the erase term (per-channel gated linear attention)."""
    q, k, v = f64(q), f64(k), f64(v)
    total, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    sc = 1.0 / np.sqrt(d_k) if scale is None or scale <= 0 else float(scale)
    g, beta = gates(a, b, A_log, dt_bias)
    kh = k if MUTATION == 6 else _norm(k, l2_eps)
    qh = sc * _norm(q, l2_eps)
    cu = _cu(total, cu_seqlens, num_seqs)
    S_n = len(cu) - 1
    s0 = np.zeros((S_n, H_v, d_k, d_v)) if initial_state is None else f64(initial_state)
    o = np.empty((total, H_v, d_v))
    final = np.empty((S_n, H_v, d_k, d_v))
    rep = H_v // H_k
    for n in range(S_n):
        for h in range(H_v):
            hk = h // rep
            S = s0[n, h].copy()
            for t in range(cu[n], cu[n + 1]):
                al = np.exp(g[t, h])
                kt, qt = kh[t, hk], qh[t, hk]
                if MUTATION == 5:
                    o[t, h] = qt @ S
                S_dec = S * al[None, :d_v] if MUTATION == 1 else al[:, None] * S
                if erase:
                    delta = beta[t, h] * (v[t, h] - kt @ (S if MUTATION == 4 else S_dec))
                else:
                    delta = beta[t, h] * v[t, h]
                S = S_dec + np.outer(kt, delta)
                if MUTATION != 5:
                    o[t, h] = qt @ S
            final[n, h] = S
    return o, final


def kda_chunked(q, k, v, a, b, A_log, dt_bias, initial_state=None, chunk=32, cu_seqlens=None,
                num_seqs=None, scale=None, l2_eps=1e-6):
    """The same map in chunks of ``chunk`` tokens.  Per chunk, with
    gam[r] = sum of g over rows 0..r of the chunk (per channel) and
    W[r, i] = exp(gam[r] - gam[i]) channel by channel (i <= r):
        A[r, i] = beta_r sum_c k_r[c] k_i[c] W[r, i][c]        (i < r)
        P[r, i] = sum_c q_r[c] k_i[c] W[r, i][c]               (i <= r)
        (I + A) Delta = diag(beta) (V - (K * exp(gam)) S)
        O  = (Q * exp(gam)) S + P Delta
        S' = diag(exp(gam[last])) S + (K * exp(gam[last] - gam))^T Delta
    with q, k normalised as in ``kda``."""
    q, k, v = f64(q), f64(k), f64(v)
    total, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    sc = 1.0 / np.sqrt(d_k) if scale is None or scale <= 0 else float(scale)
    g, beta = gates(a, b, A_log, dt_bias)
    kh = _norm(k, l2_eps)
    qh = sc * _norm(q, l2_eps)
    cu = _cu(total, cu_seqlens, num_seqs)
    S_n = len(cu) - 1
    s0 = np.zeros((S_n, H_v, d_k, d_v)) if initial_state is None else f64(initial_state)
    o = np.empty((total, H_v, d_v))
    final = np.empty((S_n, H_v, d_k, d_v))
    rep = H_v // H_k
    for n in range(S_n):
        for h in range(H_v):
            hk = h // rep
            S = s0[n, h].copy()
            for c0 in range(cu[n], cu[n + 1], chunk):
                c1 = min(c0 + chunk, cu[n + 1])
                K, Q, V = kh[c0:c1, hk], qh[c0:c1, hk], v[c0:c1, h]
                bt = beta[c0:c1, h]
                gam = np.cumsum(g[c0:c1, h], axis=0)
                L = c1 - c0
                W = np.exp(np.minimum(gam[:, None, :] - gam[None, :, :], 0.0))
                KK = np.einsum("rc,ic,ric->ri", K, K, W)
                QK = np.einsum("rc,ic,ric->ri", Q, K, W)
                A = np.tril(bt[:, None] * KK, -1)
                P = np.tril(QK)
                R = bt[:, None] * (V - (K * np.exp(gam)) @ S)
                D = np.linalg.solve(np.eye(L) + A, R)
                o[c0:c1, h] = (Q * np.exp(gam)) @ S + P @ D
                S = np.exp(gam[-1])[:, None] * S + (K * np.exp(gam[-1][None, :] - gam)).T @ D
            final[n, h] = S
    return o, final
