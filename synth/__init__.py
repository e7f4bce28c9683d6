"""Seeded synthetic inputs for the gated delta rule.

This module only draws random numbers in the shapes, dtypes and
distributions of the workloads; it holds none of the rule's arithmetic.  The
same tensors are handed to the GPU library and (widened to fp64) to the
oracle, so both sides see identical bits.

Distributions (per seed): q, k, v ~ N(0, 1); a, b ~ N(0, 1);
A_log ~ U(0, ln 16); dt_bias ~ N(0, 0.1); initial state, where a workload
carries one, ~ N(0, 0.01).  The second parameter of N is the standard
deviation.  bf16 workloads draw in fp32 and round to bf16 (round to nearest
even, torch's conversion).  The rule itself L2-normalises q and k, so raw
draws are passed in.

Workload shapes (value heads H_v share H_k key heads, state d_k x d_v):
  tiny      N=1, T=64,   H_v=H_k=2,   d=16,  fp32, chunk 16, zero state
  one_head  N=1, T=4096, H_v=H_k=1,   d=128, fp32, chunk 32, random state
  prefill   N=1, T=8192, H_v=48, H_k=16, d=128, bf16, chunk 32, zero state
  decode    N=256 sequences x 64 single-token steps, H_v=48, H_k=16, d=128,
            bf16, random state (inputs laid out step-major: [64, 256, ...])
  varlen    8 sequences, lengths ~ U[512, 32768] (per seed), packed with
            cu_seqlens, H_v=48, H_k=16, d=128, bf16, chunk 32, random state;
            sequences 6 and 7 are a stress slice with b ~ N(4, 1) (beta -> 1)
            and a ~ N(-6, 1) (g -> 0).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    H_k: int
    H_v: int
    d_k: int
    d_v: int
    dtype: str                      # "f32" or "bf16": dtype of q, k, v, a, b and o
    chunk: int = 32
    num_seqs: int = 1
    seq_len: int = 0                # dense batches: tokens per sequence
    lengths: Optional[Sequence[int]] = None   # varlen: per-sequence lengths
    init_state: bool = False
    stress_seqs: Sequence[int] = field(default_factory=tuple)
    steps: int = 0                  # decode: number of single-token steps

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def seq_lengths(self):
        if self.lengths is not None:
            return list(self.lengths)
        T = self.steps if self.steps else self.seq_len
        return [T] * self.num_seqs

    @property
    def total_tokens(self):
        return sum(self.seq_lengths)


WORKLOADS = {
    "tiny": Workload("tiny", H_k=2, H_v=2, d_k=16, d_v=16, dtype="f32", chunk=16, seq_len=64),
    "one_head": Workload("one_head", H_k=1, H_v=1, d_k=128, d_v=128, dtype="f32", chunk=32,
                         seq_len=4096, init_state=True),
    "prefill": Workload("prefill", H_k=16, H_v=48, d_k=128, d_v=128, dtype="bf16", chunk=32,
                        seq_len=8192),
    "decode": Workload("decode", H_k=16, H_v=48, d_k=128, d_v=128, dtype="bf16", num_seqs=256,
                       steps=64, init_state=True),
    "varlen": Workload("varlen", H_k=16, H_v=48, d_k=128, d_v=128, dtype="bf16", chunk=32,
                       num_seqs=8, init_state=True, stress_seqs=(6, 7)),
}


def varlen_lengths(seed: int, n: int = 8, lo: int = 512, hi: int = 32768):
    """Per-seed sequence lengths ~ U[lo, hi] (inclusive), drawn on the host."""
    g = torch.Generator(device="cpu").manual_seed(10_000 + seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def workload(name: str, seed: int = 0, **overrides) -> Workload:
    w = WORKLOADS[name]
    if name == "varlen" and w.lengths is None and "lengths" not in overrides:
        overrides["lengths"] = varlen_lengths(seed, w.num_seqs)
    return replace(w, **overrides) if overrides else w


def _normal(shape, gen, device, mean=0.0, std=1.0):
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(mean=mean, std=std, generator=gen)
    return x


def make_inputs(w: Workload, seed: int = 0, device="cpu"):
    """Draw one batch of inputs for workload ``w``.

    Returns a dict with q, k [total, H_k, d_k]; v [total, H_v, d_v];
    a, b [total, H_v] (all in w.dtype); A_log, dt_bias [H_v] fp32;
    initial_state [N, H_v, d_k, d_v] fp32 or None; cu_seqlens int32 [N+1]
    (on ``device``) or None for a dense batch; cu_host (list of ints).
    For a decode workload, q, k, v, a, b have a leading step axis
    [steps, N, ...] and the dense [N, steps] view is under "dense".
    """
    gen = torch.Generator(device=device).manual_seed(seed)
    lens = w.seq_lengths
    N = len(lens)
    total = sum(lens)
    dt = w.torch_dtype
    if w.steps:
        lead = (w.steps, N)
    else:
        lead = (total,)
    q = _normal(lead + (w.H_k, w.d_k), gen, device)
    k = _normal(lead + (w.H_k, w.d_k), gen, device)
    v = _normal(lead + (w.H_v, w.d_v), gen, device)
    a = _normal(lead + (w.H_v,), gen, device)
    b = _normal(lead + (w.H_v,), gen, device)
    if w.stress_seqs:
        cu = [0]
        for L in lens:
            cu.append(cu[-1] + L)
        for n in w.stress_seqs:
            t0, t1 = cu[n], cu[n + 1]
            b[t0:t1] = _normal((t1 - t0, w.H_v), gen, device, mean=4.0, std=1.0)
            a[t0:t1] = _normal((t1 - t0, w.H_v), gen, device, mean=-6.0, std=1.0)
    A_log = torch.empty(w.H_v, dtype=torch.float32, device=device).uniform_(
        0.0, math.log(16.0), generator=gen)
    dt_bias = _normal((w.H_v,), gen, device, std=0.1)
    s0 = None
    if w.init_state:
        s0 = _normal((N, w.H_v, w.d_k, w.d_v), gen, device, std=0.01)
    out = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), a=a.to(dt), b=b.to(dt), A_log=A_log,
               dt_bias=dt_bias, initial_state=s0)
    cu_host = [0]
    for L in lens:
        cu_host.append(cu_host[-1] + L)
    out["cu_host"] = cu_host
    out["cu_seqlens"] = (torch.tensor(cu_host, dtype=torch.int32, device=device)
                         if w.lengths is not None else None)
    if w.steps:
        # dense [N, steps] token order: sequence n's step s is row n*steps + s
        def dense(x):
            return x.transpose(0, 1).reshape((N * w.steps,) + tuple(x.shape[2:])).contiguous()
        out["dense"] = {kk: dense(out[kk]) for kk in ("q", "k", "v", "a", "b")}
    return out


def custom(H_k, H_v, d_k, d_v, dtype, lengths=None, seq_len=0, num_seqs=1, chunk=32,
           init_state=True, stress_seqs=()):
    """A workload of any shape (test sizes); same distributions."""
    return Workload("custom", H_k=H_k, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype, chunk=chunk,
                    num_seqs=num_seqs if lengths is None else len(lengths), seq_len=seq_len,
                    lengths=lengths, init_state=init_state, stress_seqs=tuple(stress_seqs))


def ssd_inputs(G, H, N, P, dtype, lengths=None, seq_len=0, num_seqs=1, seed=0, device="cpu",
               init_state=True, gate=False, delta_range=(1e-3, 1e-1)):
    """Inputs of the Mamba-2 SSD recurrence: x [total, H, P], delta [total, H],
    B, C [total, G, N], z [total, H, P] (when ``gate``) in ``dtype``; A [H]
    fp32; initial_state [S, H, N, P] fp32 or None.

    Distributions: x, B, C, z ~ N(0, 1); delta log-uniform on
    ``delta_range`` (the usual time-step range of Mamba-2 initialisation,
    1e-3 to 1e-1); A = -exp(U(0, ln 16)) (decay rates 1 to 16); initial
    state ~ N(0, 0.01).  Sequences are dense (``num_seqs`` x ``seq_len``)
    or packed with ``lengths`` (then cu_seqlens is on ``device``).
    """
    gen = torch.Generator(device=device).manual_seed(seed)
    lens = list(lengths) if lengths is not None else [seq_len] * num_seqs
    S = len(lens)
    total = sum(lens)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    x = _normal((total, H, P), gen, device)
    B = _normal((total, G, N), gen, device)
    C = _normal((total, G, N), gen, device)
    lo, hi = math.log(delta_range[0]), math.log(delta_range[1])
    delta = torch.empty((total, H), dtype=torch.float32, device=device).uniform_(
        lo, hi, generator=gen).exp()
    A = -torch.empty(H, dtype=torch.float32, device=device).uniform_(
        0.0, math.log(16.0), generator=gen).exp()
    z = _normal((total, H, P), gen, device) if gate else None
    s0 = _normal((S, H, N, P), gen, device, std=0.01) if init_state else None
    cu_host = [0]
    for L in lens:
        cu_host.append(cu_host[-1] + L)
    return dict(x=x.to(dt), delta=delta.to(dt), A=A, B=B.to(dt), C=C.to(dt),
                z=None if z is None else z.to(dt), initial_state=s0, cu_host=cu_host,
                cu_seqlens=(torch.tensor(cu_host, dtype=torch.int32, device=device)
                            if lengths is not None else None))


def kda_inputs(w: Workload, seed: int = 0, device="cpu", a_mean=0.0):
    """Inputs of the per-channel-decay variant for workload ``w``: those of
    ``make_inputs`` with a replaced by [..., H_v, d_k] ~ N(a_mean, 1) (in
    w.dtype) and dt_bias by [H_v, d_k] ~ N(0, 0.1) fp32, drawn from a second
    generator seeded seed + 7919 (so the other tensors equal make_inputs')."""
    out = make_inputs(w, seed, device=device)
    gen = torch.Generator(device=device).manual_seed(seed + 7919)
    lead = tuple(out["b"].shape)
    a = _normal(lead + (w.d_k,), gen, device, mean=a_mean)
    out["a"] = a.to(w.torch_dtype)
    out["dt_bias"] = _normal((w.H_v, w.d_k), gen, device, std=0.1)
    if w.steps:
        N = lead[1]
        out["dense"]["a"] = out["a"].transpose(0, 1).reshape((N * w.steps, w.H_v, w.d_k)).contiguous()
    return out


def coherent_keys(w: Workload, seed: int, eps: float, device="cpu"):
    """Keys that repeat a direction: k_t = u + eps * n_t, with u ~ N(0, I)
    drawn once per (sequence, key head) and n_t ~ N(0, I) per token, from a
    generator seeded seed + 4243 (the other tensors of make_inputs are left
    as they are).  At d_k = 128 the mean |cos| of two keys is about
    1 / (1 + eps^2): eps = 1 gives about 0.5, eps = 0.33 about 0.9, against
    about 0.07 for independent draws.  Shape and dtype of make_inputs' k
    (dense or packed batches; not the decode layout)."""
    gen = torch.Generator(device=device).manual_seed(seed + 4243)
    lens = w.seq_lengths
    u = _normal((len(lens), w.H_k, w.d_k), gen, device)
    n = _normal((sum(lens), w.H_k, w.d_k), gen, device)
    idx = torch.repeat_interleave(torch.arange(len(lens), device=device),
                                  torch.tensor(lens, device=device))
    return (u[idx] + eps * n).to(w.torch_dtype)
