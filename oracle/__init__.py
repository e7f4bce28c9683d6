"""Oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and this
package never imports the GPU library: the two share no code.

``fwd`` is the plain fp64 sequential recurrence of the rule (the C file
``gdr_oracle.c``; GatedDeltaRule.ixx File Reference, "Detailed Description").
``gates`` derives beta, g and the normalised q, k the same way.
``chunked`` (module ``oracle.chunked``) is an fp64 numpy regrouping of the same
arithmetic into chunks (the UT-transform form of the Track L pull request,
"What landed"), pinned against ``fwd`` by the tests.
``oracle.ssd`` (the Mamba-2 SSD recurrence) and ``oracle.kda`` (the rule with
one decay per key channel) are the fp64 oracles of the two neighbouring
mixers, each pinned by its own tests.

Every function takes numpy arrays or CPU torch tensors of any float dtype and
widens them exactly to fp64; results are fp64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build(force=True)
            lib = ctypes.CDLL(_LIB_PATH)
            lib.gdr_oracle_fwd.restype = ctypes.c_int
            lib.gdr_oracle_fwd.argtypes = [
                ctypes.c_int64, _i64p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                ctypes.c_double, ctypes.c_double, ctypes.c_int,
                _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i64p, ctypes.c_int64, ctypes.c_int]
            lib.gdr_oracle_gates.restype = ctypes.c_int
            lib.gdr_oracle_gates.argtypes = [
                ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                ctypes.c_double, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
            lib.gdr_oracle_set_mutation.argtypes = [ctypes.c_int]
            lib.gdr_oracle_set_mutation.restype = None
            lib.gdr_oracle_get_mutation.restype = ctypes.c_int
            _lib = lib
    return _lib


def f64(x) -> np.ndarray:
    """Exact widening to a contiguous fp64 numpy array (bf16 and fp32 values
    are all exactly representable in fp64)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        if str(x.dtype) in ("torch.bfloat16", "torch.float16"):
            x = x.float()
        x = x.double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def set_mutation(m: int) -> None:
    """Plant mistake number ``m`` in the C recurrence (0 restores it).
    Used only by the tests that show every pin can fail."""
    _load().gdr_oracle_set_mutation(int(m))


def get_mutation() -> int:
    return int(_load().gdr_oracle_get_mutation())


def default_scale(d_k: int) -> float:
    # q is scaled by 1/sqrt(d_k) (GatedDeltaRule.ixx File Reference, "Detailed Description")
    return 1.0 / np.sqrt(d_k)


def gates(q, k, a, b, A_log, dt_bias, scale=None, l2_eps=1e-6):
    """beta = sigmoid(b), g = -exp(A_log)*softplus(a + dt_bias), and the
    L2-normalised q (times ``scale``) and k.

    q, k: [total, H_k, d_k]; a, b: [total, H_v]; A_log, dt_bias: [H_v].
    Returns (q_hat, k_hat, g, beta) as fp64 arrays.
    """
    q, k, a, b, A_log, dt_bias = map(f64, (q, k, a, b, A_log, dt_bias))
    total, H_k, d_k = q.shape
    H_v = a.shape[1]
    scale = default_scale(d_k) if scale is None or scale <= 0 else float(scale)
    q_hat = np.empty_like(q)
    k_hat = np.empty_like(k)
    g = np.empty((total, H_v))
    beta = np.empty((total, H_v))
    rc = _load().gdr_oracle_gates(total, H_k, H_v, d_k, scale, float(l2_eps), _ptr(q), _ptr(k),
                                  _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(q_hat),
                                  _ptr(k_hat), _ptr(g), _ptr(beta))
    if rc != 0:
        raise ValueError(f"gdr_oracle_gates: status {rc}")
    return q_hat, k_hat, g, beta


def _cu(cu_seqlens, total, num_seqs):
    if cu_seqlens is None:
        if num_seqs is None:
            num_seqs = 1
        assert total % num_seqs == 0, "dense batch: total must be a multiple of num_seqs"
        T = total // num_seqs
        return np.arange(num_seqs + 1, dtype=np.int64) * T
    if hasattr(cu_seqlens, "detach"):
        cu_seqlens = cu_seqlens.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))


def fwd(q, k, v, a, b, A_log, dt_bias, initial_state=None, cu_seqlens=None, num_seqs=None,
        scale=None, l2_eps=1e-6, erase=True, pairs=None, n_threads=0):
    """The sequential recurrence in fp64.

    q, k: [total, H_k, d_k]; v: [total, H_v, d_v]; a, b: [total, H_v];
    A_log, dt_bias: [H_v]; initial_state: [N, H_v, d_k, d_v] or None (zeros).
    Sequences are given by ``cu_seqlens`` ([N+1]) or, for a dense batch, by
    ``num_seqs`` equal-length sequences laid out one after another.
    ``pairs``: optional [(seq, value head), ...]; only those are computed
    (the rest of ``o`` and ``final_state`` is left zero).
    Returns (o [total, H_v, d_v], final_state [N, H_v, d_k, d_v]).
    """
    q, k, v, a, b, A_log, dt_bias = map(f64, (q, k, v, a, b, A_log, dt_bias))
    s0 = f64(initial_state)
    total, H_k, d_k = q.shape
    H_v, d_v = v.shape[1], v.shape[2]
    cu = _cu(cu_seqlens, total, num_seqs)
    N = len(cu) - 1
    assert cu[-1] == total, "cu_seqlens must end at the token count"
    scale = default_scale(d_k) if scale is None or scale <= 0 else float(scale)
    o = np.zeros((total, H_v, d_v))
    S = np.zeros((N, H_v, d_k, d_v))
    pr = None
    npairs = 0
    if pairs is not None:
        pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int64).reshape(-1, 2))
        npairs = pr.shape[0]
    rc = _load().gdr_oracle_fwd(N, cu.ctypes.data_as(_i64p), H_k, H_v, d_k, d_v, scale,
                                float(l2_eps), 1 if erase else 0, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias), _ptr(s0), _ptr(o),
                                _ptr(S), None if pr is None else pr.ctypes.data_as(_i64p), npairs,
                                int(n_threads))
    if rc != 0:
        raise ValueError(f"gdr_oracle_fwd: status {rc}")
    return o, S


def fwd_sampled(q, k, v, a, b, A_log, dt_bias, pairs, initial_state=None, cu_seqlens=None,
                num_seqs=None, scale=None, l2_eps=1e-6, n_threads=0):
    """The recurrence for selected (sequence, value head) pairs only, without
    widening the whole batch: each pair's token rows are cut out (value head h
    reads key head h // (H_v // H_k), the same grouping as ``fwd``) and the
    pairs are run together through ``fwd`` as a packed batch of one-head
    sequences, one OpenMP unit each.

    Inputs may be CPU torch tensors or numpy arrays of any float dtype.
    Returns {(n, h): (o [L, d_v], final_state [d_k, d_v])}.
    """
    total, H_k, d_k = q.shape
    H_v = v.shape[1]
    G = H_v // H_k
    cu = _cu(cu_seqlens, total, num_seqs)
    pairs = [(int(n), int(h)) for (n, h) in pairs]
    qs, ks, vs, as_, bs, s0s, lens = [], [], [], [], [], [], []
    A1 = f64(A_log)
    D1 = f64(dt_bias)
    for (n, h) in pairs:
        t0, t1 = int(cu[n]), int(cu[n + 1])
        hk = h // G
        qs.append(f64(q[t0:t1, hk:hk + 1]))
        ks.append(f64(k[t0:t1, hk:hk + 1]))
        vs.append(f64(v[t0:t1, h:h + 1]))
        as_.append(f64(a[t0:t1, h:h + 1]))
        bs.append(f64(b[t0:t1, h:h + 1]))
        if initial_state is not None:
            s0s.append(f64(initial_state[n:n + 1, h:h + 1]))
        lens.append(t1 - t0)
    if not pairs:
        return {}
    out = {}
    # group pairs by value head so that A_log/dt_bias stay per-head scalars
    by_head = {}
    for i, (n, h) in enumerate(pairs):
        by_head.setdefault(h, []).append(i)
    for h, idx in by_head.items():
        cu_h = np.zeros(len(idx) + 1, dtype=np.int64)
        cu_h[1:] = np.cumsum([lens[i] for i in idx])
        cat = lambda xs: np.concatenate([xs[i] for i in idx], axis=0)
        s0 = None
        if initial_state is not None:
            s0 = np.concatenate([s0s[i] for i in idx], axis=0)
        o1, S1 = fwd(cat(qs), cat(ks), cat(vs), cat(as_), cat(bs), A1[h:h + 1], D1[h:h + 1],
                     initial_state=s0, cu_seqlens=cu_h, scale=scale if scale else
                     default_scale(d_k), l2_eps=l2_eps, n_threads=n_threads)
        for j, i in enumerate(idx):
            out[pairs[i]] = (o1[cu_h[j]:cu_h[j + 1], 0], S1[j, 0])
    return out
