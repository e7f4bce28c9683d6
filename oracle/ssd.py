"""Oracle for the Mamba-2 SSD recurrence -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library never does, and this
module imports nothing from it.

The pages name the operation and its inputs but print no formula (Track L
pull request, "What landed": a selective_ssm op over x, A, B, C and delta with
an optional gate and an optional initial state, "SSD recurrence documented",
state h[D, N] carried for streaming decode; the hot-path scope lists it as the
same chunk scan with a scalar decay and no erase).  The plain reading taken
here, per head h of head dimension P, groups of heads sharing B and C
(head h reads group h // (H / G)), state h[N, P] in fp64:
    h_t = exp(delta_t A_h) h_{t-1} + B_t (delta_t x_t)^T
    y_t = h_t^T C_t                      (after the write, as the rule reads o)
    y_t <- y_t * SiLU(z_t)               (optional gate)
delta_t > 0 and A_h < 0 are given directly.  ``MUTATION`` plants one
mistake at a time for the tests that show each pin can fail.
"""
from __future__ import annotations

import numpy as np

from . import f64

MUTATION = 0
_MUTATIONS = {
    1: "output read before the write",
    2: "decay applied after the write",
    3: "delta missing from the write",
    4: "modulo group mapping",
    5: "gate sigmoid(z) instead of SiLU(z)",
    6: "B and C swapped",
    7: "decay exp(A) instead of exp(delta A)",
}


def _silu(x):
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def ssd(x, delta, A, B, C, initial_state=None, z=None, cu_seqlens=None, num_seqs=None):
    """x [total, H, P]; delta [total, H]; A [H]; B, C [total, G, N];
    initial_state [S, H, N, P] or None; z [total, H, P] or None.
    Returns (y [total, H, P], final_state [S, H, N, P])."""
    x, delta, A, B, C = f64(x), f64(delta), f64(A), f64(B), f64(C)
    total, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    assert H % G == 0 and C.shape == B.shape and delta.shape == (total, H) and A.shape == (H,)
    if cu_seqlens is not None:
        cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    else:
        n = 1 if num_seqs is None else int(num_seqs)
        L = total // n if n else 0
        cu = [i * L for i in range(n + 1)]
    S = len(cu) - 1
    h0 = np.zeros((S, H, N, P)) if initial_state is None else f64(initial_state)
    zz = None if z is None else f64(z)
    y = np.empty((total, H, P))
    final = np.empty((S, H, N, P))
    rep = H // G
    for s in range(S):
        for h in range(H):
            g = h % G if MUTATION == 4 else h // rep
            st = h0[s, h].copy()
            for t in range(cu[s], cu[s + 1]):
                bt, ct = (C[t, g], B[t, g]) if MUTATION == 6 else (B[t, g], C[t, g])
                decay = np.exp(A[h]) if MUTATION == 7 else np.exp(delta[t, h] * A[h])
                u = x[t, h] if MUTATION == 3 else delta[t, h] * x[t, h]
                if MUTATION == 1:
                    y[t, h] = st.T @ ct
                if MUTATION == 2:
                    st = (st + np.outer(bt, u)) * decay
                else:
                    st = decay * st + np.outer(bt, u)
                if MUTATION != 1:
                    y[t, h] = st.T @ ct
                if zz is not None:
                    gate = _sigmoid(zz[t, h]) if MUTATION == 5 else _silu(zz[t, h])
                    y[t, h] = y[t, h] * gate
            final[s, h] = st
    return y, final
