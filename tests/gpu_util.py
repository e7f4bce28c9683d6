"""Helpers for the GPU parity tests: the error metric and oracle comparisons.

Error metric, per (sequence, value head) slice of the output (all tokens x d_v)
and of the final state (d_k x d_v): max |x - y| / max |y|, absolute error where
max |y| = 0; any NaN or Inf fails.  The reported value is the worst slice.
Bars: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32 state in both).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

TOL = {"f32": 1e-4, "bf16": 2e-2}


def slice_err(x, y) -> float:
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x)):
        return float("inf")
    num = float(np.max(np.abs(x - y)))
    den = float(np.max(np.abs(y)))
    return num / den if den > 0 else num


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().double().numpy()


def compare_full(o_gpu, S_gpu, o_ref, S_ref, cu, H_v):
    """Worst slice error over every (sequence, head) of full outputs."""
    o_gpu = to_np(o_gpu).reshape(o_ref.shape)
    worst_o = worst_s = 0.0
    for n in range(len(cu) - 1):
        for h in range(H_v):
            worst_o = max(worst_o, slice_err(o_gpu[cu[n]:cu[n + 1], h], o_ref[cu[n]:cu[n + 1], h]))
            if S_gpu is not None:
                worst_s = max(worst_s, slice_err(to_np(S_gpu[n, h]), S_ref[n, h]))
    return worst_o, worst_s


def compare_sampled(o_gpu, S_gpu, ref, cu):
    """Worst slice error over the sampled pairs; ``ref`` from oracle.fwd_sampled."""
    worst_o = worst_s = 0.0
    per = {}
    for (n, h), (o_r, S_r) in ref.items():
        eo = slice_err(to_np(o_gpu[cu[n]:cu[n + 1], h]), o_r)
        es = slice_err(to_np(S_gpu[n, h]), S_r) if S_gpu is not None else 0.0
        per[(n, h)] = (eo, es)
        worst_o, worst_s = max(worst_o, eo), max(worst_s, es)
    return worst_o, worst_s, per


def oracle_full(inp, cu, scale=None, l2_eps=1e-6):
    return oracle.fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                      inp["dt_bias"], initial_state=inp["initial_state"], cu_seqlens=cu,
                      scale=scale, l2_eps=l2_eps)


def oracle_pairs(inp, cu, pairs, initial_state=None, n_threads=0):
    s0 = inp["initial_state"] if initial_state is None else initial_state
    return oracle.fwd_sampled(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                              inp["dt_bias"], pairs, initial_state=s0, cu_seqlens=cu,
                              n_threads=n_threads)
