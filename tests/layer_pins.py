"""Pins of the oracle for the steps either side of the rule (``oracle.layer``):
checks against facts that do not come from the oracle itself.

The two facts used throughout:
- SiLU(u) - SiLU(-u) = u for every u, since sigmoid(u) + sigmoid(-u) = 1.  A
  call on the negated inputs (and negated history and bias) therefore
  recovers the pre-activation exactly, whatever SiLU's own values are.
- textbook values of the logistic function (tests/golden/silu_values.json).

With one-hot taps the pre-activation is a known shifted copy of the input,
so the shift of the history, the per-channel weight rows and the bias each
get a pin of their own (PLENA_Simulator pull request 113 notes that an
identity newest tap without bias leaves all three unobserved).
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import layer

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def close(x, y, rtol=1e-12, atol=1e-12, what=""):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if x.shape != y.shape or not np.allclose(x, y, rtol=rtol, atol=atol):
        err = np.max(np.abs(x - y)) if x.shape == y.shape else "shape"
        raise AssertionError(f"{what}: mismatch (max abs err {err})")


def silu_points():
    with open(os.path.join(GOLDEN, "silu_values.json")) as f:
        return [tuple(p) for p in json.load(f)["points"]]


def _problem(seed, C=6, W=4, lengths=(7, 2, 0, 5)):
    rng = np.random.default_rng(seed)
    total = int(sum(lengths))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(x=rng.standard_normal((total, C)), state=rng.standard_normal((len(lengths), C, W - 1)),
                bias=rng.standard_normal(C), cu=cu, C=C, W=W, lengths=list(lengths))


def _expected_shift(p, tap_of_channel):
    """Pre-activation of one-hot taps: channel c reads the input
    W-1-tap(c) steps back, from the history before each sequence."""
    C, W, cu = p["C"], p["W"], p["cu"]
    out = np.zeros_like(p["x"])
    for n in range(len(cu) - 1):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for t in range(t0, t1):
            for c in range(C):
                back = W - 1 - tap_of_channel(c)
                src = t - back
                out[t, c] = p["x"][src, c] if src >= t0 else p["state"][n, c, W - 1 - (t0 - src)]
    return out


def _pre(p, w, bias=None, state=None):
    """Pre-activation through the oracle, from SiLU(u) - SiLU(-u) = u."""
    st = p["state"] if state is None else state
    y1, _ = layer.short_conv_silu(p["x"], w, bias, st, cu_seqlens=p["cu"])
    y2, _ = layer.short_conv_silu(-p["x"], w, None if bias is None else -bias, -st, cu_seqlens=p["cu"])
    return y1 - y2


# --------------------------------------------------------------- convolution
def pin_conv_silu_values():
    """Newest tap one, no bias, no history: y = SiLU(x) at textbook points."""
    pts = silu_points()
    x = np.array([[u, -u] for u, _ in pts])
    w = np.zeros((2, 4))
    w[:, 3] = 1.0
    y, _ = layer.short_conv_silu(x, w, None, None, num_seqs=1)
    close(y[:, 0], [v for _, v in pts], rtol=1e-15, atol=1e-16, what="SiLU values")
    close(y[:, 0] - y[:, 1], x[:, 0], what="SiLU(u) - SiLU(-u) = u")


def pin_conv_history_shift(seeds=range(3)):
    """Oldest tap one: the pre-activation is the input W-1 steps back, taken
    from the carried history before each sequence starts."""
    for s in seeds:
        p = _problem(s)
        w = np.zeros((p["C"], p["W"]))
        w[:, 0] = 1.0
        close(_pre(p, w), _expected_shift(p, lambda c: 0), what=f"oldest tap, seed {s}")


def pin_conv_per_channel_taps(seeds=range(3)):
    """Channel c one-hot at tap c % W: each channel has its own weight row."""
    for s in seeds:
        p = _problem(s, C=8)
        W = p["W"]
        w = np.zeros((p["C"], W))
        for c in range(p["C"]):
            w[c, c % W] = 1.0
        close(_pre(p, w), _expected_shift(p, lambda c: c % W), what=f"per-channel taps, seed {s}")


def pin_conv_bias(seeds=range(3)):
    """Zero weights: the pre-activation is the bias on every token."""
    for s in seeds:
        p = _problem(s)
        w = np.zeros((p["C"], p["W"]))
        pre = _pre(p, w, bias=p["bias"])
        close(pre, np.broadcast_to(p["bias"], pre.shape), what=f"bias, seed {s}")


def pin_conv_impulse_response(seeds=range(3)):
    """Zero history and bias, a unit impulse at (t, c): the pre-activation at
    t + j reads w[c, W-1-j] for j < W and is zero elsewhere."""
    for s in seeds:
        rng = np.random.default_rng(100 + s)
        C, W, T = 5, 4, 11
        w = rng.standard_normal((C, W))
        t, c = 3, 2
        x = np.zeros((T, C))
        x[t, c] = 1.0
        p = dict(x=x, state=np.zeros((1, C, W - 1)), cu=np.array([0, T]))
        pre = _pre(p, w)
        expect = np.zeros((T, C))
        for j in range(W):
            expect[t + j, c] = w[c, W - 1 - j]
        close(pre, expect, what=f"impulse response, seed {s}")


def pin_conv_new_history(seeds=range(3)):
    """The returned history is the last W-1 inputs of each sequence, older
    history entries moving up when the sequence is shorter than W-1."""
    for s in seeds:
        p = _problem(s, lengths=(7, 2, 0, 1, 5))
        rng = np.random.default_rng(s)
        w = rng.standard_normal((p["C"], p["W"]))
        _, st = layer.short_conv_silu(p["x"], w, p["bias"], p["state"], cu_seqlens=p["cu"])
        W, cu = p["W"], p["cu"]
        for n in range(len(cu) - 1):
            t0, t1 = int(cu[n]), int(cu[n + 1])
            for j in range(W - 1):  # entry j holds the input W-1-j steps before the end
                src = t1 - (W - 1) + j
                want = p["x"][src] if src >= t0 else p["state"][n, :, W - 1 - (t0 - src)]
                close(st[n, :, j], want, what=f"history seq {n} entry {j}, seed {s}")


def pin_conv_streaming(seeds=range(3)):
    """One call equals the same tokens split over calls with the history
    carried (split points inside the first W-1 tokens, and empty pieces)."""
    for s in seeds:
        rng = np.random.default_rng(200 + s)
        C, W, T = 6, 4, 13
        x = rng.standard_normal((T, C))
        w = rng.standard_normal((C, W))
        b = rng.standard_normal(C)
        s0 = rng.standard_normal((1, C, W - 1))
        y_all, st_all = layer.short_conv_silu(x, w, b, s0, num_seqs=1)
        ys, st = [], s0
        for a, e in ((0, 1), (1, 1), (1, 3), (3, 9), (9, 13)):
            y, st = layer.short_conv_silu(x[a:e], w, b, st, cu_seqlens=np.array([0, e - a]))
            ys.append(y)
        close(np.concatenate(ys), y_all, what=f"streaming outputs, seed {s}")
        close(st, st_all, what=f"streaming history, seed {s}")


# ------------------------------------------------------------ gated RMSNorm
def pin_gated_norm_hand_example():
    """o = [3, 4] has RMS sqrt(12.5); with z = 1 the difference of the calls
    at z and -z is o / RMS * w (eps = 0)."""
    o = np.array([[[3.0, 4.0]]])
    w = np.array([2.0, -0.5])
    d = layer.gated_rmsnorm(o, np.ones_like(o), w, eps=0.0) - layer.gated_rmsnorm(o, -np.ones_like(o), w, eps=0.0)
    r = np.sqrt(12.5)
    close(d, [[[3.0 / r * 2.0, 4.0 / r * -0.5]]], what="hand example")


def pin_gated_norm_gate_values():
    """With w = 1 and eps = 0, out / (o / RMS) is the gate SiLU(z)."""
    pts = silu_points()
    z = np.array([[[u for u, _ in pts]]])
    o = np.ones_like(z)  # RMS 1
    out = layer.gated_rmsnorm(o, z, np.ones(z.shape[-1]), eps=0.0)
    close(out[0, 0], [v for _, v in pts], rtol=1e-15, atol=1e-16, what="gate values")


def pin_gated_norm_rows(seeds=range(3)):
    """Each (token, head) row is normalised on its own: with z = 1 the
    difference of the calls at z and -z has RMS 1 per row (w = 1, eps = 0),
    scaling o leaves the output unchanged, and scaling one head's o leaves
    the other heads alone."""
    for s in seeds:
        rng = np.random.default_rng(300 + s)
        o = rng.standard_normal((5, 3, 8))
        one = np.ones_like(o)
        w = np.ones(8)
        d = layer.gated_rmsnorm(o, one, w, eps=0.0) - layer.gated_rmsnorm(o, -one, w, eps=0.0)
        close(np.sqrt(np.mean(d ** 2, axis=-1)), np.ones((5, 3)), what=f"row RMS, seed {s}")
        z = rng.standard_normal(o.shape)
        base = layer.gated_rmsnorm(o, z, rng.standard_normal(8), eps=0.0)
        w2 = rng.standard_normal(8)
        close(layer.gated_rmsnorm(3.7 * o, z, w2, eps=0.0), layer.gated_rmsnorm(o, z, w2, eps=0.0),
              what=f"scale invariance, seed {s}")
        o2 = o.copy()
        o2[:, 1] *= 5.0
        a = layer.gated_rmsnorm(o, z, w2, eps=1e-3)
        b = layer.gated_rmsnorm(o2, z, w2, eps=1e-3)
        close(a[:, 0], b[:, 0], what=f"heads independent, seed {s}")
        close(a[:, 2], b[:, 2], what=f"heads independent, seed {s}")
        assert base.shape == o.shape


def pin_gated_norm_eps():
    """eps enters as sqrt(mean(o^2) + eps): a row of zeros but one entry u has
    mean u^2/d, so with z = 1 the difference at z, -z is u / sqrt(u^2/d + eps)."""
    d, u, eps = 4, 0.3, 0.05
    o = np.zeros((1, 1, d))
    o[0, 0, 1] = u
    one = np.ones_like(o)
    diff = layer.gated_rmsnorm(o, one, np.ones(d), eps) - layer.gated_rmsnorm(o, -one, np.ones(d), eps)
    want = np.zeros(d)
    want[1] = u / np.sqrt(u * u / d + eps)
    close(diff[0, 0], want, what="eps")


CONV_PINS = [pin_conv_silu_values, pin_conv_history_shift, pin_conv_per_channel_taps, pin_conv_bias,
             pin_conv_impulse_response, pin_conv_new_history, pin_conv_streaming]
NORM_PINS = [pin_gated_norm_hand_example, pin_gated_norm_gate_values, pin_gated_norm_rows,
             pin_gated_norm_eps]
ALL_PINS = CONV_PINS + NORM_PINS
