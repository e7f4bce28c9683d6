"""Oracle for the steps either side of the rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module; the GPU library never does, and this
module imports nothing from it.

The pages name these steps but print no formula for them (flashprove issue
"P1: Qwen3.8-27B port, tracking": the layer runs from the in_proj outputs
through a 4-tap conv1d, SiLU, the q/k L2 norm and the gates to the rule, and
ends in a gated RMSNorm of o; PLENA_Simulator pull request 113: the short
convolution has per-channel weights, an optional bias and a history carried
between calls as a ring buffer, kept in bf16 in the shipped configuration).
The plain readings taken here:

``short_conv_silu``
    depthwise causal convolution of width W over time, tap W-1 on the newest
    input, plus an optional per-channel bias, then SiLU(x) = x * sigmoid(x):
        y[t, c] = SiLU(bias[c] + sum_j w[c, j] * x[t - (W-1) + j, c]);
    inputs before a sequence's first token come from its carried history
    state[n, c, 0..W-2] (oldest first), zeros when there is none; the new
    history is the last W-1 inputs of the sequence (older history entries
    move up when the sequence is shorter than W-1).

``gated_rmsnorm``
    per (token, head) row of o:
        out = o / sqrt(mean(o^2) + eps) * w * SiLU(z).

Everything is computed in fp64 from exactly widened inputs.  ``MUTATION``
plants one mistake at a time for the tests that show each pin can fail.
"""
from __future__ import annotations

import numpy as np

from . import f64

MUTATION = 0
_MUTATIONS = {
    1: "history ignored (zeros before every sequence)",
    2: "history not shifted (new state = old state)",
    3: "taps reversed (tap 0 on the newest input)",
    4: "one weight row for every channel",
    5: "bias dropped",
    6: "sigmoid instead of SiLU after the convolution",
    7: "RMS over the sum of squares instead of the mean",
    8: "gate sigmoid(z) instead of SiLU(z)",
    9: "norm weight not applied",
    10: "RMS over the whole token row instead of per head",
}


def _silu(x):
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def _bounds(total, cu_seqlens, num_seqs):
    if cu_seqlens is not None:
        cu = [int(v) for v in np.asarray(cu_seqlens).reshape(-1)]
    else:
        n = int(num_seqs)
        L = total // n if n else 0
        cu = [i * L for i in range(n + 1)]
    assert cu[0] == 0 and cu[-1] == total and all(a <= b for a, b in zip(cu, cu[1:]))
    return cu


def short_conv_silu(x, weight, bias=None, conv_state=None, cu_seqlens=None, num_seqs=None):
    """x [total, C]; weight [C, W]; bias [C] or None; conv_state [N, C, W-1]
    (oldest first) or None.  Returns (y [total, C], new_state [N, C, W-1])."""
    x = f64(x)
    w = f64(weight)
    total, C = x.shape
    W = w.shape[1]
    assert w.shape == (C, W) and W >= 1
    if cu_seqlens is None and num_seqs is None:
        num_seqs = 1
    cu = _bounds(total, cu_seqlens, num_seqs)
    N = len(cu) - 1
    b = np.zeros(C) if bias is None or MUTATION == 5 else f64(bias)
    hist0 = np.zeros((N, C, W - 1)) if conv_state is None else f64(conv_state)
    assert hist0.shape == (N, C, W - 1)
    if MUTATION == 3:
        w = w[:, ::-1]
    if MUTATION == 4:
        w = np.broadcast_to(w[0], (C, W))
    y = np.empty((total, C))
    new_state = np.empty((N, C, W - 1))
    for n in range(N):
        t0, t1 = cu[n], cu[n + 1]
        hist = np.zeros((C, W - 1)) if MUTATION == 1 else hist0[n]
        # rows: W-1 history inputs (oldest first), then the sequence's inputs
        xx = np.concatenate([hist.T, x[t0:t1]], axis=0)
        for t in range(t1 - t0):
            window = xx[t:t + W]  # oldest .. newest, the newest is x[t0 + t]
            pre = b + np.einsum("jc,cj->c", window, w)
            y[t0 + t] = _sigmoid(pre) if MUTATION == 6 else _silu(pre)
        new_state[n] = hist0[n] if MUTATION == 2 else xx[xx.shape[0] - (W - 1):].T
    return y, new_state


def gated_rmsnorm(o, z, weight, eps=1e-6):
    """o, z [total, H, d]; weight [d].  Returns out [total, H, d]."""
    o = f64(o)
    z = f64(z)
    w = f64(weight)
    assert o.shape == z.shape and w.shape == (o.shape[-1],)
    if MUTATION == 10:
        ss = np.mean(o.reshape(o.shape[0], -1) ** 2, axis=-1)[:, None, None]
    elif MUTATION == 7:
        ss = np.sum(o ** 2, axis=-1, keepdims=True)
    else:
        ss = np.mean(o ** 2, axis=-1, keepdims=True)
    gate = _sigmoid(z) if MUTATION == 8 else _silu(z)
    out = o / np.sqrt(ss + eps) * gate
    return out if MUTATION == 9 else out * w
