"""Pins of the SSD oracle (``oracle.ssd``): checks against facts that do not
come from the recurrence loop itself.

- a hand-worked scalar example (tests/golden/ssd_scalar_example.json);
- the quadratic (attention-like) form of the same map, the duality the SSD
  name refers to: y_t = sum_{s<=t} exp(A sum_{u=s+1..t} delta_u) delta_s
  (C_t . B_s) x_s + exp(A sum_{u<=t} delta_u) h0^T C_t, computed here from
  cumulative sums without a recurrence;
- the limits A = 0 (plain cumulative sums) and delta A -> -inf (no memory);
- streaming over split calls, the group mapping, and the gate through
  SiLU(u) - SiLU(-u) = u.
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import ssd

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def close(x, y, rtol=1e-12, atol=1e-12, what=""):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    if x.shape != y.shape or not np.allclose(x, y, rtol=rtol, atol=atol):
        err = np.max(np.abs(x - y)) if x.shape == y.shape else "shape"
        raise AssertionError(f"{what}: mismatch (max abs err {err})")


def problem(seed, T=9, H=4, G=2, N=3, P=2, init=True, A_scale=1.0):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((T, H, P)), delta=rng.uniform(0.05, 1.0, (T, H)),
                A=-A_scale * rng.uniform(0.1, 2.0, H), B=rng.standard_normal((T, G, N)),
                C=rng.standard_normal((T, G, N)),
                h0=rng.standard_normal((1, H, N, P)) if init else None)


def quadratic_form(p):
    """The SSD map as a weighted sum over earlier tokens (one sequence)."""
    x, dl, A, B, C, h0 = p["x"], p["delta"], p["A"], p["B"], p["C"], p["h0"]
    T, H, P = x.shape
    G = B.shape[1]
    y = np.zeros((T, H, P))
    for h in range(H):
        g = h // (H // G)
        cs = np.concatenate([[0.0], np.cumsum(dl[:, h])])  # cs[t+1] = sum_{u<=t} delta_u
        for t in range(T):
            for s in range(t + 1):
                w = np.exp(A[h] * (cs[t + 1] - cs[s + 1])) * dl[s, h] * (C[t, g] @ B[s, g])
                y[t, h] += w * x[s, h]
            if h0 is not None:
                y[t, h] += np.exp(A[h] * cs[t + 1]) * (h0[0, h].T @ C[t, g])
    return y


def run(p, **kw):
    return ssd.ssd(p["x"], p["delta"], p["A"], p["B"], p["C"], p["h0"], num_seqs=1, **kw)


def pin_ssd_scalar_example():
    with open(os.path.join(GOLDEN, "ssd_scalar_example.json")) as f:
        g = json.load(f)
    T = len(g["x"])
    y, st = ssd.ssd(np.array(g["x"]).reshape(T, 1, 1), np.array(g["delta"]).reshape(T, 1),
                    np.array([g["A"]]), np.array(g["B"]).reshape(T, 1, 1),
                    np.array(g["C"]).reshape(T, 1, 1), np.array(g["h0"]).reshape(1, 1, 1, 1))
    close(y.reshape(-1), g["y"], rtol=1e-14, atol=1e-14, what="scalar example outputs")
    close(st.reshape(-1), [g["final"]], rtol=1e-14, atol=1e-14, what="scalar example state")


def pin_ssd_quadratic_form(seeds=range(4)):
    for s in seeds:
        p = problem(10 + s)
        y, _ = run(p)
        close(y, quadratic_form(p), rtol=1e-10, atol=1e-12, what=f"quadratic form, seed {s}")


def pin_ssd_limits():
    # A = 0: no decay, the state is the plain sum of writes
    p = problem(20)
    p["A"] = np.zeros_like(p["A"])
    y, st = run(p)
    close(y, quadratic_form(p), what="A = 0 outputs")
    H, G = p["x"].shape[1], p["B"].shape[1]
    for h in range(H):
        g = h // (H // G)
        want = p["h0"][0, h] + sum(np.outer(p["B"][t, g], p["delta"][t, h] * p["x"][t, h])
                                   for t in range(p["x"].shape[0]))
        close(st[0, h], want, what=f"A = 0 state head {h}")
    # delta A -> -inf: no memory, y_t = delta_t (C_t . B_t) x_t
    p = problem(21, A_scale=1e4)
    y, _ = run(p)
    for h in range(H):
        g = h // (H // G)
        for t in range(p["x"].shape[0]):
            want = p["delta"][t, h] * (p["C"][t, g] @ p["B"][t, g]) * p["x"][t, h]
            close(y[t, h], want, what=f"no-memory limit t={t} h={h}")


def pin_ssd_streaming(seeds=range(3)):
    for s in seeds:
        p = problem(30 + s, T=14)
        y_all, st_all = run(p)
        ys, st = [], p["h0"]
        for a, e in ((0, 1), (1, 5), (5, 5), (5, 14)):
            q = dict(p, x=p["x"][a:e], delta=p["delta"][a:e], B=p["B"][a:e], C=p["C"][a:e], h0=st)
            y, st = run(q)
            ys.append(y)
        close(np.concatenate(ys), y_all, what=f"streaming outputs, seed {s}")
        close(st, st_all, what=f"streaming state, seed {s}")


def pin_ssd_groups():
    """Heads 2 and 3 of 4 read group 1 of 2: changing group 1's B leaves
    heads 0 and 1 alone."""
    p = problem(40)
    y1, _ = run(p)
    q = dict(p, B=p["B"].copy())
    q["B"][:, 1] += 1.0
    y2, _ = run(q)
    close(y1[:, :2], y2[:, :2], what="group 0 heads unchanged")
    assert not np.allclose(y1[:, 2:], y2[:, 2:]), "group 1 heads did not change"


def pin_ssd_gate():
    """y(z) - y(-z) = y_ungated * z since SiLU(u) - SiLU(-u) = u."""
    p = problem(50)
    z = np.random.default_rng(51).standard_normal(p["x"].shape)
    y0, _ = run(p)
    y1, _ = run(p, z=z)
    y2, _ = run(p, z=-z)
    close(y1 - y2, y0 * z, what="gate identity")


ALL_PINS = [pin_ssd_scalar_example, pin_ssd_quadratic_form, pin_ssd_limits, pin_ssd_streaming,
            pin_ssd_groups, pin_ssd_gate]
