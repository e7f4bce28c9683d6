"""Pins of the KDA oracle (``oracle.kda``): checks against facts that do not
come from its recurrence loop.

- a hand-worked two-channel example (tests/golden/kda_two_channel_example.json);
- gates equal across channels reduce it to the rule, whose oracle is pinned on
  its own (GatedDeltaRule.ixx File Reference, "Detailed Description");
- an independent per-step product with the explicit d_k x d_k matrix
  (I - beta k k^T) diag(alpha);
- with the erase term removed, the closed form of gated linear attention with
  one decay per channel, summed over earlier tokens;
- channel separability: without the erase term, channel c's gate moves only
  state row c;
- the chunked regrouping equals the recurrence at every chunk size;
- streaming over split calls.
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle
from oracle import kda

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def close(x, y, rtol=1e-11, atol=1e-12, what=""):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if x.shape != y.shape or not np.allclose(x, y, rtol=rtol, atol=atol):
        err = np.max(np.abs(x - y)) if x.shape == y.shape else "shape"
        raise AssertionError(f"{what}: mismatch (max abs err {err})")


def problem(seed, lens=(9,), H_k=2, H_v=4, d_k=4, d_v=3, init=True, a_mean=0.0):
    rng = np.random.default_rng(seed)
    T = int(sum(lens))
    return dict(q=rng.standard_normal((T, H_k, d_k)), k=rng.standard_normal((T, H_k, d_k)),
                v=rng.standard_normal((T, H_v, d_v)),
                a=a_mean + rng.standard_normal((T, H_v, d_k)),
                b=rng.standard_normal((T, H_v)), A_log=rng.uniform(-1.0, 1.0, H_v),
                dt_bias=0.5 * rng.standard_normal((H_v, d_k)),
                s0=rng.standard_normal((len(lens), H_v, d_k, d_v)) if init else None,
                cu=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))


def run(p, **kw):
    return kda.kda(p["q"], p["k"], p["v"], p["a"], p["b"], p["A_log"], p["dt_bias"], p["s0"],
                   cu_seqlens=p["cu"], **kw)


def ref_gates(p):
    """alpha [T, H_v, d_k] and beta [T, H_v] straight from the definitions."""
    x = p["a"] + p["dt_bias"][None]
    sp = np.log(1.0 + np.exp(x))
    alpha = np.exp(-np.exp(p["A_log"])[None, :, None] * sp)
    beta = 1.0 / (1.0 + np.exp(-p["b"]))
    return alpha, beta


def unit(x, eps=1e-6):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def pin_kda_two_channel_example():
    with open(os.path.join(GOLDEN, "kda_two_channel_example.json")) as f:
        g = json.load(f)
    T = len(g["v"])
    o, st = kda.kda(np.array(g["q"]).reshape(T, 1, 2), np.array(g["k"]).reshape(T, 1, 2),
                    np.array(g["v"]).reshape(T, 1, 1), np.array(g["a"]).reshape(T, 1, 2),
                    np.array(g["b"]).reshape(T, 1), np.zeros(1), np.zeros((1, 2)),
                    np.array(g["S0"]).reshape(1, 1, 2, 1), num_seqs=1, scale=1.0, l2_eps=0.0)
    close(o.reshape(-1), g["o"], rtol=1e-14, atol=1e-14, what="example outputs")
    close(st.reshape(-1), g["final"], rtol=1e-14, atol=1e-14, what="example state")


def pin_kda_reduces_to_rule(seeds=range(3)):
    for s in seeds:
        p = problem(100 + s, lens=(7, 0, 12))
        a1 = p["a"][:, :, :1]
        d1 = p["dt_bias"][:, :1]
        q = dict(p, a=np.repeat(a1, p["a"].shape[2], axis=2),
                 dt_bias=np.repeat(d1, p["dt_bias"].shape[1], axis=1))
        o, st = run(q)
        o_r, st_r = oracle.fwd(p["q"], p["k"], p["v"], a1[..., 0], p["b"], p["A_log"], d1[:, 0],
                               initial_state=p["s0"], cu_seqlens=p["cu"])
        close(o, o_r, what=f"uniform gates = rule, outputs, seed {s}")
        close(st, st_r, what=f"uniform gates = rule, state, seed {s}")


def brute(p, erase=True):
    """Per-step products with explicit matrices."""
    alpha, beta = ref_gates(p)
    T, H_k, d_k = p["q"].shape
    H_v, d_v = p["v"].shape[1:]
    kh, qh = unit(p["k"]), unit(p["q"]) / np.sqrt(d_k)
    cu = p["cu"]
    o = np.zeros((T, H_v, d_v))
    fin = np.zeros((len(cu) - 1, H_v, d_k, d_v))
    for n in range(len(cu) - 1):
        for h in range(H_v):
            hk = h // (H_v // H_k)
            S = p["s0"][n, h].copy() if p["s0"] is not None else np.zeros((d_k, d_v))
            for t in range(cu[n], cu[n + 1]):
                k = kh[t, hk][:, None]
                E = np.eye(d_k) - (beta[t, h] * (k @ k.T) if erase else 0.0)
                S = E @ np.diag(alpha[t, h]) @ S + beta[t, h] * k @ p["v"][t, h][None, :]
                o[t, h] = (qh[t, hk][None, :] @ S)[0]
            fin[n, h] = S
    return o, fin


def pin_kda_brute_force(seeds=range(4)):
    for s in seeds:
        p = problem(200 + s, lens=(6, 11), init=(s % 2 == 0))
        o, st = run(p)
        o_b, st_b = brute(p)
        close(o, o_b, what=f"brute force outputs, seed {s}")
        close(st, st_b, what=f"brute force state, seed {s}")


def pin_kda_erase_off_closed_form(seeds=range(2)):
    for s in seeds:
        p = problem(300 + s, lens=(10,))
        o, _ = run(p, erase=False)
        alpha, beta = ref_gates(p)
        T, H_k, d_k = p["q"].shape
        H_v = p["v"].shape[1]
        kh, qh = unit(p["k"]), unit(p["q"]) / np.sqrt(d_k)
        lg = np.cumsum(np.log(alpha), axis=0)  # lg[t] = sum of log-decays over steps 0..t
        want = np.zeros_like(o)
        for h in range(H_v):
            hk = h // (H_v // H_k)
            for t in range(T):
                want[t, h] = (qh[t, hk] * np.exp(lg[t, h])) @ p["s0"][0, h]
                for u in range(t + 1):
                    w = np.sum(qh[t, hk] * kh[u, hk] * np.exp(lg[t, h] - lg[u, h]))
                    want[t, h] += w * beta[u, h] * p["v"][u, h]
        close(o, want, what=f"erase-off closed form, seed {s}")


def pin_kda_channel_separability():
    p = problem(400, lens=(8,))
    _, st0 = run(p, erase=False)
    d_k = p["a"].shape[2]
    for c in range(d_k):
        for field in ("a", "dt_bias"):
            q = dict(p, **{field: p[field].copy()})
            if field == "a":
                q["a"][:, :, c] -= 1.5
            else:
                q["dt_bias"][:, c] -= 1.5
            _, st = run(q, erase=False)
            rows = [r for r in range(d_k) if r != c]
            close(st[:, :, rows], st0[:, :, rows], rtol=0, atol=0,
                  what=f"{field} channel {c}: other rows moved")
            assert not np.allclose(st[:, :, c], st0[:, :, c]), f"{field} channel {c}: row {c} did not move"


def pin_kda_chunked_equals_recurrent():
    for chunk in (1, 3, 8, 16, 32, 64):
        p = problem(500 + chunk, lens=(45, 1, 0, 17), d_k=8, d_v=5)
        o, st = run(p)
        o_c, st_c = kda.kda_chunked(p["q"], p["k"], p["v"], p["a"], p["b"], p["A_log"],
                                    p["dt_bias"], p["s0"], chunk=chunk, cu_seqlens=p["cu"])
        close(o_c, o, rtol=1e-10, atol=1e-11, what=f"chunked outputs, chunk {chunk}")
        close(st_c, st, rtol=1e-10, atol=1e-11, what=f"chunked state, chunk {chunk}")
    # strong decay (alpha down to ~1e-30 per step): the chunked form must not overflow
    p = problem(560, lens=(40,), a_mean=4.0)
    p["A_log"] = p["A_log"] + 2.5
    o, st = run(p)
    o_c, st_c = kda.kda_chunked(p["q"], p["k"], p["v"], p["a"], p["b"], p["A_log"], p["dt_bias"],
                                p["s0"], chunk=32, cu_seqlens=p["cu"])
    close(o_c, o, rtol=1e-10, atol=1e-11, what="chunked outputs, strong decay")
    close(st_c, st, rtol=1e-10, atol=1e-11, what="chunked state, strong decay")


def pin_kda_streaming():
    p = problem(600, lens=(15,))
    o_all, st_all = run(p)
    outs, st = [], p["s0"]
    for a, e in ((0, 1), (1, 6), (6, 6), (6, 15)):
        q = dict(p, q=p["q"][a:e], k=p["k"][a:e], v=p["v"][a:e], a=p["a"][a:e], b=p["b"][a:e],
                 s0=st, cu=np.array([0, e - a]))
        o, st = run(q)
        outs.append(o)
    close(np.concatenate(outs), o_all, rtol=0, atol=0, what="streamed outputs")
    close(st, st_all, rtol=0, atol=0, what="streamed state")


ALL_PINS = [pin_kda_two_channel_example, pin_kda_reduces_to_rule, pin_kda_brute_force,
            pin_kda_erase_off_closed_form, pin_kda_channel_separability,
            pin_kda_chunked_equals_recurrent, pin_kda_streaming]
