"""A seeded random sweep of small problems through every forward entry point
of the library, each checked against its fp64 oracle (same metric and bars
as the other parity tests: 1e-4 for fp32 inputs, 2e-2 for bf16).

Each case draws, from its own seed: the key-head count and grouping, d_k and
d_v from {16, 32, 64, 128}, the dtype, the chunk size, 1-5 sequence lengths
in [0, 150] (zeros included), whether an initial state is given, and (for
the rule) a custom q scale and l2 epsilon.  The draws use numpy's seeded
generator only, so the cases are the same on every run."""
import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as gdr
import oracle
import synth
from oracle import kda, ssd
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DEV = "cuda"
DIMS = [16, 32, 64, 128]


def note(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.lib()
    yield
    torch.cuda.synchronize()


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    H_k = int(rng.integers(1, 4))
    H_v = H_k * int(rng.integers(1, 4))
    d_k, d_v = int(rng.choice(DIMS)), int(rng.choice(DIMS))
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    chunk = int(rng.choice([16, 32, 64]))
    lens = [int(x) for x in rng.integers(0, 151, size=int(rng.integers(1, 6)))]
    if rng.random() < 0.3:
        lens[int(rng.integers(0, len(lens)))] = 0
    init = bool(rng.random() < 0.7)
    scale = float(rng.uniform(0.05, 0.5)) if rng.random() < 0.3 else None
    eps = float(rng.choice([1e-6, 1e-3]))
    return dict(H_k=H_k, H_v=H_v, d_k=d_k, d_v=d_v, dtype=dtype, chunk=chunk, lens=lens,
                init=init, scale=scale, eps=eps)


def check(o, S, o_ref, S_ref, cu, H_v, dtype, what):
    eo, es = U.compare_full(o, S, o_ref, S_ref, cu, H_v)
    note(f"  {what}: o {eo:.2e} S {es:.2e}")
    assert eo <= U.TOL[dtype] and es <= U.TOL[dtype], (what, eo, es)


@pytest.mark.parametrize("seed", range(16))
def test_rule_random(seed):
    c = draw(seed)
    note(f"[rule sweep {seed}] {c}")
    w = synth.custom(c["H_k"], c["H_v"], c["d_k"], c["d_v"], c["dtype"], lengths=c["lens"],
                     chunk=c["chunk"], init_state=c["init"])
    inp = synth.make_inputs(w, 2000 + seed, device=DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])
    kw = dict(cu_seqlens=inp["cu_seqlens"], scale=c["scale"], l2_eps=c["eps"])
    o_ref, S_ref = U.oracle_full(inp, inp["cu_host"], scale=c["scale"], l2_eps=c["eps"])
    o1, S1 = gdr.recurrent_fwd(*args, **kw)
    o2, S2 = gdr.chunked_fwd(*args, chunk=c["chunk"], **kw)
    torch.cuda.synchronize()
    check(o1, S1, o_ref, S_ref, inp["cu_host"], w.H_v, c["dtype"], "recurrent")
    check(o2, S2, o_ref, S_ref, inp["cu_host"], w.H_v, c["dtype"], "chunked")


@pytest.mark.parametrize("seed", range(12))
def test_kda_random(seed):
    c = draw(100 + seed)
    chunk = c["chunk"] if c["chunk"] != 64 else 32  # KDA takes chunk 16 or 32
    note(f"[kda sweep {seed}] {c} chunk={chunk}")
    w = synth.custom(c["H_k"], c["H_v"], c["d_k"], c["d_v"], c["dtype"], lengths=c["lens"],
                     chunk=chunk, init_state=c["init"])
    inp = synth.kda_inputs(w, 3000 + seed, device=DEV)
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])
    o_ref, S_ref = kda.kda(*[t.cpu() if t is not None else None for t in args],
                           cu_seqlens=inp["cu_host"])
    o1, S1 = gdr.kda_recurrent_fwd(*args, cu_seqlens=inp["cu_seqlens"])
    o2, S2 = gdr.kda_chunked_fwd(*args, chunk=chunk, cu_seqlens=inp["cu_seqlens"])
    o3, S3 = gdr.kda_chunked_fwd(*args, chunk=chunk, cu_seqlens=inp["cu_seqlens"], fused=True)
    torch.cuda.synchronize()
    check(o1, S1, o_ref, S_ref, inp["cu_host"], w.H_v, c["dtype"], "kda recurrent")
    check(o2, S2, o_ref, S_ref, inp["cu_host"], w.H_v, c["dtype"], "kda chunked")
    check(o3, S3, o_ref, S_ref, inp["cu_host"], w.H_v, c["dtype"], "kda chunked, one launch")


@pytest.mark.parametrize("seed", range(12))
def test_ssd_random(seed):
    c = draw(200 + seed)
    note(f"[ssd sweep {seed}] {c}")
    gate = bool(seed % 2)
    inp = synth.ssd_inputs(c["H_k"], c["H_v"], c["d_k"], c["d_v"], c["dtype"], lengths=c["lens"],
                           seed=4000 + seed, device=DEV, init_state=c["init"], gate=gate)
    y_ref, S_ref = ssd.ssd(inp["x"].cpu(), inp["delta"].cpu(), inp["A"].cpu(), inp["B"].cpu(),
                           inp["C"].cpu(),
                           None if inp["initial_state"] is None else inp["initial_state"].cpu(),
                           None if inp["z"] is None else inp["z"].cpu(), cu_seqlens=inp["cu_host"])
    a = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], inp["initial_state"])
    y1, S1 = gdr.ssd_recurrent_fwd(*a, z=inp["z"], cu_seqlens=inp["cu_seqlens"])
    y2, S2 = gdr.ssd_chunked_fwd(*a, z=inp["z"], chunk=c["chunk"], cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    check(y1, S1, y_ref, S_ref, inp["cu_host"], c["H_v"], c["dtype"], "ssd recurrent")
    check(y2, S2, y_ref, S_ref, inp["cu_host"], c["H_v"], c["dtype"], "ssd chunked")
