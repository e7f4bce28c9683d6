"""Pins of the fp64 oracle: checks against facts that do not come from the
oracle itself (hand-worked closed forms, an independent brute force with the
explicit erase matrix, textbook special cases, invariants of the algebra).

Each pin is a function that raises AssertionError when the oracle disagrees;
``test_oracle_pins.py`` runs them and ``test_oracle_mutations.py`` plants a
mistake in the oracle and requires at least one pin to fail.
"""
from __future__ import annotations

import json
import os

import numpy as np
from scipy.special import expit

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def rand_problem(seed, T=12, H_k=2, H_v=4, d_k=6, d_v=6, N=1, init=True, lengths=None,
                 a_mean=0.0, b_mean=0.0):
    rng = np.random.default_rng(seed)
    total = T * N if lengths is None else int(sum(lengths))
    p = dict(
        q=rng.standard_normal((total, H_k, d_k)),
        k=rng.standard_normal((total, H_k, d_k)),
        v=rng.standard_normal((total, H_v, d_v)),
        a=rng.standard_normal((total, H_v)) + a_mean,
        b=rng.standard_normal((total, H_v)) + b_mean,
        A_log=rng.uniform(0.0, np.log(16.0), H_v),
        dt_bias=0.1 * rng.standard_normal(H_v),
    )
    nseq = N if lengths is None else len(lengths)
    p["initial_state"] = 0.1 * rng.standard_normal((nseq, H_v, d_k, d_v)) if init else None
    if lengths is not None:
        p["cu_seqlens"] = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    else:
        p["num_seqs"] = N
    return p


def run_oracle(p, **kw):
    args = {k: p[k] for k in ("q", "k", "v", "a", "b", "A_log", "dt_bias", "initial_state")}
    for key in ("cu_seqlens", "num_seqs"):
        if key in p:
            args[key] = p[key]
    args.update(kw)
    return oracle.fwd(**args)


def brute_force(q, k, v, a, b, A_log, dt_bias, S0, scale, eps):
    """Independent fp64 recurrence for one sequence with the explicit d_k x d_k
    erase matrix: S_t = alpha_t (I - beta_t k k^T) S_{t-1} + beta_t k v_t^T,
    o_t = S_t^T q  (Track L pull request, L1: the rule validated against an
    independent (I - beta k k^T) brute force).  Key heads are expanded to the
    value heads with np.repeat (value head h reads key head h // G).
    softplus and sigmoid come from numpy/scipy, not from the oracle."""
    T, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    G = H_v // H_k
    qv = np.repeat(q, G, axis=1)
    kv = np.repeat(k, G, axis=1)
    o = np.zeros((T, H_v, d_v))
    S_out = np.zeros((H_v, d_k, d_v))
    for h in range(H_v):
        S = np.zeros((d_k, d_v)) if S0 is None else S0[h].copy()
        for t in range(T):
            kk = kv[t, h] / np.sqrt(kv[t, h] @ kv[t, h] + eps)
            qq = qv[t, h] / np.sqrt(qv[t, h] @ qv[t, h] + eps) * scale
            beta = expit(b[t, h])
            g = -np.exp(A_log[h]) * np.logaddexp(0.0, a[t, h] + dt_bias[h])
            E = np.eye(d_k) - beta * np.outer(kk, kk)
            S = np.exp(g) * (E @ S) + beta * np.outer(kk, v[t, h])
            o[t, h] = S.T @ qq
        S_out[h] = S
    return o, S_out


def close(x, y, rtol=1e-12, atol=1e-12, what=""):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    assert np.all(np.isfinite(x)), f"{what}: non-finite values"
    err = np.max(np.abs(x - y)) if x.size else 0.0
    scale = max(np.max(np.abs(y)) if y.size else 0.0, 1.0)
    assert err <= atol + rtol * scale, f"{what}: max abs err {err:.3e} (scale {scale:.3e})"


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------- pins
def pin_e1_scalar_state():
    """Hand-worked scalar example (tests/golden/e1_scalar_state.json)."""
    e = load_golden("e1_scalar_state.json")
    args = dict(q=np.array(e["q"]), k=np.array(e["k"]), v=np.array(e["v"]), a=np.array(e["a"]),
                b=np.array(e["b"]), A_log=np.array(e["A_log"]), dt_bias=np.array(e["dt_bias"]),
                l2_eps=e["l2_eps"])
    o, S = oracle.fwd(**args)
    close(o[:, 0, 0], e["expected_o"], rtol=1e-14, what="E1 o")
    close(S.ravel(), [e["expected_final_state"]], rtol=1e-14, what="E1 S")
    o, S = oracle.fwd(**args, erase=False)
    close(o[:, 0, 0], e["expected_o_erase_off"], rtol=1e-14, what="E1 erase-off o")
    close(S.ravel(), [e["expected_final_state_erase_off"]], rtol=1e-14, what="E1 erase-off S")


def pin_e2_overwrite():
    """Hand-worked 2-d key example: the rule overwrites what is stored along a
    key (tests/golden/e2_overwrite.json)."""
    e = load_golden("e2_overwrite.json")
    args = dict(q=np.array(e["q"]), k=np.array(e["k"]), v=np.array(e["v"]), a=np.array(e["a"]),
                b=np.array(e["b"]), A_log=np.array(e["A_log"]), dt_bias=np.array(e["dt_bias"]),
                l2_eps=e["l2_eps"])
    o, S = oracle.fwd(**args)
    close(o[:, 0, 0], e["expected_o"], rtol=1e-14, atol=1e-14, what="E2 o")
    close(S[0, 0], e["expected_final_state"], rtol=1e-14, atol=1e-14, what="E2 S")
    o, S = oracle.fwd(**args, erase=False)
    close(o[:, 0, 0], e["expected_o_erase_off"], rtol=1e-14, what="E2 erase-off o")
    close(S[0, 0], e["expected_final_state_erase_off"], rtol=1e-14, what="E2 erase-off S")


def pin_brute_force(seeds=range(20)):
    """C1: the oracle equals the explicit erase-matrix brute force (GQA 4/2,
    square and non-square states, random initial state)."""
    for seed in seeds:
        rng = np.random.default_rng(seed)
        d_k = int(rng.integers(1, 9))
        d_v = d_k if seed % 2 == 0 else int(rng.integers(1, 9))
        T = int(rng.integers(1, 17))
        p = rand_problem(seed, T=T, H_k=2, H_v=4, d_k=d_k, d_v=d_v)
        scale = 1.0 / np.sqrt(d_k)
        o, S = run_oracle(p)
        ob, Sb = brute_force(p["q"], p["k"], p["v"], p["a"], p["b"], p["A_log"], p["dt_bias"],
                             p["initial_state"][0], scale, 1e-6)
        close(o, ob, what=f"C1 o seed {seed}")
        close(S[0], Sb, what=f"C1 S seed {seed}")


def pin_erase_off_closed_form(seeds=range(5)):
    """C2: with the erase term removed the rule is gated (decayed) linear
    attention, whose output has the closed form
    o_t = e^{G_t} q_t^T S0 + sum_{i<=t} e^{G_t - G_i} beta_i (q_t . k_i) v_i,
    G the cumulative sum of g over the sequence (Track L pull request,
    'The core finding (L0)')."""
    for seed in seeds:
        p = rand_problem(100 + seed, T=20, H_k=1, H_v=2, d_k=5, d_v=3)
        o, S = run_oracle(p, erase=False)
        qh, kh, g, beta = (np.asarray(x) for x in oracle.gates(
            p["q"], p["k"], p["a"], p["b"], p["A_log"], p["dt_bias"]))
        for h in range(2):
            G = np.cumsum(g[:, h])
            S0 = p["initial_state"][0, h]
            for t in range(20):
                ref = np.exp(G[t]) * (qh[t, 0] @ S0)
                for i in range(t + 1):
                    ref = ref + np.exp(G[t] - G[i]) * beta[i, h] * (qh[t, 0] @ kh[i, 0]) * p["v"][i, h]
                close(o[t, h], ref, what=f"C2 seed {seed} h {h} t {t}")


def pin_special_cases():
    """C4: (i) alpha = 0 (A_log = 50): o_t = beta_t (q_t . k_t) v_t;
    (ii) beta = 0 (b = -800): o_t = e^{G_t} S0^T q_t;
    (iii) q = k, beta = 1 (b = 40), l2_eps = 0: o_t = v_t / sqrt(d_k);
    (iv) gates: b = 0 -> beta = 1/2; A_log = 0, a + dt_bias = 0 -> g = -ln 2."""
    p = rand_problem(7, T=9, H_k=1, H_v=1, d_k=4, d_v=3)
    # (i)
    p1 = dict(p, A_log=np.array([50.0]))
    o, _ = run_oracle(p1)
    qh, kh, _, beta = oracle.gates(p["q"], p["k"], p["a"], p["b"], p1["A_log"], p["dt_bias"])
    ref = beta[:, 0, None] * np.sum(qh[:, 0] * kh[:, 0], axis=1)[:, None] * p["v"][:, 0]
    close(o[:, 0], ref, what="C4(i)")
    # (ii)
    p2 = dict(p, b=np.full_like(p["b"], -800.0))
    o, S = run_oracle(p2)
    _, _, g, _ = oracle.gates(p["q"], p["k"], p2["a"], p2["b"], p["A_log"], p["dt_bias"])
    G = np.cumsum(g[:, 0])
    ref = np.exp(G)[:, None] * (qh[:, 0] @ p["initial_state"][0, 0])
    close(o[:, 0], ref, what="C4(ii) o")
    close(S[0, 0], np.exp(G[-1]) * p["initial_state"][0, 0], what="C4(ii) S")
    # (iii)
    p3 = dict(p, q=p["k"].copy(), b=np.full_like(p["b"], 40.0))
    o, _ = run_oracle(p3, l2_eps=0.0)
    close(o[:, 0], p["v"][:, 0] / np.sqrt(4), what="C4(iii)")
    # (iv)
    a = np.array([[0.0, 1.5]])
    b = np.array([[0.0, -2.0]])
    _, _, g, beta = oracle.gates(np.ones((1, 1, 2)), np.ones((1, 1, 2)), a, b,
                                 np.array([0.0, 0.3]), np.array([0.0, -0.25]))
    close(beta[0, 0], 0.5, rtol=1e-15, what="C4(iv) beta")
    close(g[0, 0], -np.log(2.0), rtol=1e-15, what="C4(iv) g")
    close(beta[0, 1], 1.0 / (1.0 + np.exp(2.0)), rtol=1e-15, what="C4(iv) beta(-2)")
    close(g[0, 1], -np.exp(0.3) * np.log1p(np.exp(1.25)), rtol=1e-14, what="C4(iv) g(1.25)")


def pin_write_identity_and_contraction(seeds=range(4)):
    """C5: the per-step write identity
    k^T S_t = (1 - beta |k|^2) k^T (alpha S_{t-1}) + beta |k|^2 v^T,
    and the contraction bound |S_t[:, j]| <= alpha |S_{t-1}[:, j]| + beta |k| |v_j|
    (true because 0 <= beta |k|^2 <= 2 for normalised keys; Track L pull
    request, 'Numerics finding').  States are taken step by step by running
    the oracle one token at a time."""
    for seed in seeds:
        p = rand_problem(200 + seed, T=15, H_k=1, H_v=1, d_k=8, d_v=5)
        qh, kh, g, beta = oracle.gates(p["q"], p["k"], p["a"], p["b"], p["A_log"], p["dt_bias"])
        S_prev = p["initial_state"]
        for t in range(15):
            _, S_t = oracle.fwd(p["q"][t:t + 1], p["k"][t:t + 1], p["v"][t:t + 1],
                                p["a"][t:t + 1], p["b"][t:t + 1], p["A_log"], p["dt_bias"],
                                initial_state=S_prev)
            k_ = kh[t, 0]
            al = np.exp(g[t, 0])
            bt = beta[t, 0]
            kk = k_ @ k_
            lhs = k_ @ S_t[0, 0]
            rhs = (1 - bt * kk) * (k_ @ (al * S_prev[0, 0])) + bt * kk * p["v"][t, 0]
            close(lhs, rhs, what=f"C5 identity seed {seed} t {t}")
            bound = al * np.linalg.norm(S_prev[0, 0], axis=0) + bt * np.sqrt(kk) * np.abs(p["v"][t, 0])
            assert np.all(np.linalg.norm(S_t[0, 0], axis=0) <= bound * (1 + 1e-12) + 1e-15), \
                f"C5 contraction bound violated seed {seed} t {t}"
            S_prev = S_t


def pin_chunked_equals_recurrent():
    """C6: the chunked regrouping agrees with the recurrence for every chunk
    size, including ragged last chunks and chunk >= T (Track L pull request,
    L2: chunk == recurrent, chunk-size invariant; GatedDeltaRule.ixx File
    Reference: the two forms agree to float reassociation)."""
    p = rand_problem(300, T=70, H_k=2, H_v=4, d_k=8, d_v=6)
    o, S = run_oracle(p)
    for C in (1, 2, 3, 5, 8, 16, 32, 64, 70, 128):
        oc, Sc = chunked.fwd(p["q"], p["k"], p["v"], p["a"], p["b"], p["A_log"], p["dt_bias"], C,
                             initial_state=p["initial_state"])
        close(oc, o, rtol=1e-10, atol=1e-10, what=f"C6 o chunk {C}")
        close(Sc, S, rtol=1e-10, atol=1e-10, what=f"C6 S chunk {C}")
    # varlen with empty and one-token sequences, chunks restart at every start
    lens = [0, 1, 33, 5, 64, 31]
    p = rand_problem(301, H_k=1, H_v=3, d_k=4, d_v=4, lengths=lens)
    o, S = run_oracle(p)
    oc, Sc = chunked.fwd(p["q"], p["k"], p["v"], p["a"], p["b"], p["A_log"], p["dt_bias"], 16,
                         initial_state=p["initial_state"], cu_seqlens=p["cu_seqlens"])
    close(oc, o, rtol=1e-10, atol=1e-10, what="C6 varlen o")
    close(Sc, S, rtol=1e-10, atol=1e-10, what="C6 varlen S")


def pin_wy_transition(seeds=range(5)):
    """C7: Gamma_c I - K^T diag(e^{gamma_c - gamma}) T diag(beta Gamma) K equals
    the explicit product of alpha_r (I - beta_r k_r k_r^T), r = c..1; and T from
    forward substitution equals a dense inverse of (I + A)."""
    for seed in seeds:
        rng = np.random.default_rng(400 + seed)
        c, d = 7, 5
        K = rng.standard_normal((c, d))
        K /= np.linalg.norm(K, axis=1, keepdims=True)
        g = -np.abs(rng.standard_normal(c))
        beta = expit(rng.standard_normal(c))
        O, S, T, W, U = chunked.chunk_step(np.zeros((c, d)), K, np.zeros((c, 1)), g, beta,
                                           np.zeros((d, 1)))
        gam = np.cumsum(g)
        Kt = np.exp(gam[-1] - gam)[:, None] * K
        M = np.exp(gam[-1]) * np.eye(d) - Kt.T @ W
        ref = np.eye(d)
        for r in range(c):
            ref = np.exp(g[r]) * (np.eye(d) - beta[r] * np.outer(K[r], K[r])) @ ref
        close(M, ref, what=f"C7 WY seed {seed}")
        A = np.tril(beta[:, None] * np.exp(gam[:, None] - gam[None, :]) * (K @ K.T), -1)
        close(T, np.linalg.inv(np.eye(c) + A), what=f"C7 T seed {seed}")


def pin_linearity_and_structure():
    """C8: (i) outputs and final state are jointly linear in (V, S0);
    (ii) permuting the d_v columns of V and S0 permutes the outputs;
    (iii) a GQA run equals a run with q, k repeated to every value head;
    (iv) a packed varlen run equals each sequence run alone."""
    p = rand_problem(500, T=11, H_k=2, H_v=6, d_k=5, d_v=4)
    q_ = rand_problem(501, T=11, H_k=2, H_v=6, d_k=5, d_v=4)
    o1, S1 = run_oracle(p)
    o2, S2 = run_oracle(dict(p, v=q_["v"], initial_state=q_["initial_state"]))
    o3, S3 = run_oracle(dict(p, v=2 * p["v"] - 3 * q_["v"],
                             initial_state=2 * p["initial_state"] - 3 * q_["initial_state"]))
    close(o3, 2 * o1 - 3 * o2, what="C8(i) o")
    close(S3, 2 * S1 - 3 * S2, what="C8(i) S")
    perm = np.array([2, 0, 3, 1])
    o4, S4 = run_oracle(dict(p, v=p["v"][..., perm], initial_state=p["initial_state"][..., perm]))
    close(o4, o1[..., perm], what="C8(ii) o")
    close(S4, S1[..., perm], what="C8(ii) S")
    o5, S5 = run_oracle(dict(p, q=np.repeat(p["q"], 3, axis=1), k=np.repeat(p["k"], 3, axis=1)))
    close(o5, o1, rtol=0, atol=0, what="C8(iii) o")
    close(S5, S1, rtol=0, atol=0, what="C8(iii) S")
    lens = [4, 0, 9, 1, 6]
    pv = rand_problem(502, H_k=2, H_v=4, d_k=3, d_v=3, lengths=lens)
    o, S = run_oracle(pv)
    cu = pv["cu_seqlens"]
    for n in range(len(lens)):
        t0, t1 = cu[n], cu[n + 1]
        on, Sn = oracle.fwd(pv["q"][t0:t1], pv["k"][t0:t1], pv["v"][t0:t1], pv["a"][t0:t1],
                            pv["b"][t0:t1], pv["A_log"], pv["dt_bias"],
                            initial_state=pv["initial_state"][n:n + 1])
        close(o[t0:t1], on, rtol=0, atol=0, what=f"C8(iv) o seq {n}")
        close(S[n], Sn[0], rtol=0, atol=0, what=f"C8(iv) S seq {n}")


def pin_streaming_equals_recompute():
    """C9: carrying the state across calls is exactly one long call (Track L
    pull request, L3: streaming decode == full recompute): bitwise, since the
    sequential oracle performs the same operations in the same order."""
    p = rand_problem(600, T=40, H_k=1, H_v=2, d_k=6, d_v=5)
    o, S = run_oracle(p)
    rng = np.random.default_rng(601)
    cuts = sorted(set([0, 40] + list(rng.integers(1, 40, 5))))
    state = p["initial_state"]
    pieces = []
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        on, state = oracle.fwd(p["q"][t0:t1], p["k"][t0:t1], p["v"][t0:t1], p["a"][t0:t1],
                               p["b"][t0:t1], p["A_log"], p["dt_bias"], initial_state=state)
        pieces.append(on)
    assert np.array_equal(np.concatenate(pieces), o), "C9: split run differs from one run"
    assert np.array_equal(state, S), "C9: split final state differs"
    state = p["initial_state"]
    for t in range(40):
        on, state = oracle.fwd(p["q"][t:t + 1], p["k"][t:t + 1], p["v"][t:t + 1], p["a"][t:t + 1],
                               p["b"][t:t + 1], p["A_log"], p["dt_bias"], initial_state=state)
        assert np.array_equal(on[0], o[t]), f"C9: token-by-token output differs at {t}"
    assert np.array_equal(state, S), "C9: token-by-token final state differs"


def pin_segment_transition_map(seeds=range(3)):
    """The two-level scan's premise: over a segment the final state is affine
    in the entry state, S_out = M S_in + S_loc, where M is the segment run
    from S_in = I with v = 0 (d_k-wide values, so M is d_k x d_k) and S_loc
    the run from S_in = 0 (each step is alpha (I - beta k k^T) S + beta k v^T).
    Chaining the maps of consecutive segments, of equal or unequal length,
    reproduces the one long run, for d_k = d_v and d_k != d_v."""
    for s in seeds:
        p = rand_problem(800 + s, T=36, H_k=1, H_v=2, d_k=5, d_v=5)
        _, S_full = run_oracle(p)
        I = np.broadcast_to(np.eye(5), (1, 2, 5, 5)).copy()
        state = p["initial_state"]
        for t0, t1 in ((0, 12), (12, 24), (24, 36)):
            seg = {k: (p[k][t0:t1] if k in ("q", "k", "v", "a", "b") else p[k]) for k in p}
            _, M = oracle.fwd(seg["q"], seg["k"], np.zeros_like(seg["v"]), seg["a"], seg["b"],
                              p["A_log"], p["dt_bias"], initial_state=I)
            _, S_loc = oracle.fwd(seg["q"], seg["k"], seg["v"], seg["a"], seg["b"], p["A_log"],
                                  p["dt_bias"], initial_state=None)
            _, S_ref = oracle.fwd(seg["q"], seg["k"], seg["v"], seg["a"], seg["b"], p["A_log"],
                                  p["dt_bias"], initial_state=state)
            nxt = np.einsum("nhij,nhjk->nhik", M, state) + S_loc
            close(nxt, S_ref, rtol=1e-10, atol=1e-12, what=f"segment map, seed {s}, [{t0},{t1})")
            state = nxt
        close(state, S_full, rtol=1e-10, atol=1e-12, what=f"chained segment maps, seed {s}")
    # d_k != d_v and segments of unequal length (a packed sequence's last
    # segment is partial): M is d_k x d_k, the run from S_in = I with d_k-wide
    # zero values; S_loc and the states are d_k x d_v
    for s in seeds:
        p = rand_problem(810 + s, T=29, H_k=1, H_v=2, d_k=5, d_v=3)
        _, S_full = run_oracle(p)
        I = np.broadcast_to(np.eye(5), (1, 2, 5, 5)).copy()
        state = p["initial_state"]
        for t0, t1 in ((0, 8), (8, 16), (16, 24), (24, 29)):
            seg = {k: (p[k][t0:t1] if k in ("q", "k", "v", "a", "b") else p[k]) for k in p}
            zv = np.zeros(seg["v"].shape[:2] + (5,))
            _, M = oracle.fwd(seg["q"], seg["k"], zv, seg["a"], seg["b"], p["A_log"],
                              p["dt_bias"], initial_state=I)
            assert M.shape == (1, 2, 5, 5)
            _, S_loc = oracle.fwd(seg["q"], seg["k"], seg["v"], seg["a"], seg["b"], p["A_log"],
                                  p["dt_bias"], initial_state=None)
            state = np.einsum("nhij,nhjk->nhik", M, state) + S_loc
        close(state, S_full, rtol=1e-10, atol=1e-12, what=f"chained d_k x d_k maps, seed {s}")


def pin_constant_state():
    """C10: the state does not grow with context (GatedDeltaRule.ixx File
    Reference): final-state shape is independent of T."""
    shapes = set()
    for T in (1, 64, 4096):
        p = rand_problem(700, T=T, H_k=1, H_v=1, d_k=3, d_v=2)
        _, S = run_oracle(p)
        shapes.add(S.shape)
    assert len(shapes) == 1


ALL_PINS = [
    pin_e1_scalar_state,
    pin_e2_overwrite,
    pin_brute_force,
    pin_erase_off_closed_form,
    pin_special_cases,
    pin_write_identity_and_contraction,
    pin_chunked_equals_recurrent,
    pin_wy_transition,
    pin_linearity_and_structure,
    pin_streaming_equals_recompute,
    pin_segment_transition_map,
    pin_constant_state,
]
