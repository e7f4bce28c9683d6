"""Full-population GPU parity at the workload sizes: every (sequence, value
head) pair of configurations 3-5 against the fp64 oracle through the C ABI,
on every form that runs them, and sampled pairs of the per-channel-decay
variant's varlen batch.

  * prefill layer (1 x 8192 tokens, 48 value heads sharing 16 key heads,
    bf16, chunk 32): the cooperative chunked form (a workspace), the
    one-launch chunked form (none) and the recurrent form; all 48 heads;
  * batched decode (256 sequences x 48 heads, fp32 state carried in place
    over 64 single-token steps): every output of every step and every final
    state, and the same tokens as one chunked call;
  * varlen prefill (8 packed sequences of U[512, 32768] tokens, carried
    state, stress slice on sequences 6 and 7 as the workload defines it): all
    384 pairs on seeds 0, 1 and 2, chunked and recurrent forms.

The bar is max |gpu - oracle| / max |oracle| <= 2e-2 per (sequence, head)
slice of the outputs and of the final state (bf16 inputs, fp32 state).  The
worst slice of each case is printed.
"""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as gdr
import oracle
import synth
from oracle import kda as kda_oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = U.TOL["bf16"]


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.lib()
    yield
    torch.cuda.synchronize()


def args(inp):
    return (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])


def seq_kw(inp):
    if inp["cu_seqlens"] is not None:
        return dict(cu_seqlens=inp["cu_seqlens"])
    return dict(num_seqs=len(inp["cu_host"]) - 1)


def run_form(form, inp, w):
    if form == "recurrent":
        return gdr.recurrent_fwd(*args(inp), **seq_kw(inp))
    ws = "auto" if form == "chunked_coop" else None
    return gdr.chunked_fwd(*args(inp), chunk=w.chunk, workspace=ws, **seq_kw(inp))


@pytest.fixture(scope="module")
def prefill():
    w = synth.workload("prefill")
    inp = synth.make_inputs(w, 0, device=DEV)
    ref = U.oracle_full(inp, inp["cu_host"])
    return w, inp, ref


@pytest.mark.parametrize("form", ["chunked_coop", "chunked_one_launch", "recurrent"])
def test_prefill_layer_every_head(prefill, form):
    w, inp, ref = prefill
    if form == "chunked_coop":
        assert gdr.chunked_workspace_bytes(w.H_k, w.H_v, w.d_k, w.d_v, w.dtype) > 0
    o, S = run_form(form, inp, w)
    torch.cuda.synchronize()
    eo, es = U.compare_full(o, S, ref[0], ref[1], inp["cu_host"], w.H_v)
    note(f"[full] prefill layer, {form}, all {w.H_v} heads: worst o={eo:.3e} S={es:.3e}")
    assert eo <= TOL and es <= TOL, (eo, es)


def test_decode_every_pair_every_step():
    w = synth.workload("decode")
    inp = synth.make_inputs(w, 0, device=DEV)
    note(f"[full] decode {w.num_seqs} x {w.H_v} heads x {w.steps} steps")
    state = inp["initial_state"].clone()
    outs = []
    for s in range(w.steps):
        o, _ = gdr.recurrent_fwd(inp["q"][s], inp["k"][s], inp["v"][s], inp["a"][s],
                                 inp["b"][s], inp["A_log"], inp["dt_bias"], state,
                                 num_seqs=w.num_seqs, inplace=True)
        outs.append(o)
    torch.cuda.synchronize()
    o_all = torch.stack(outs, 1).reshape(w.num_seqs * w.steps, w.H_v, w.d_v)  # dense [N, steps]
    d = inp["dense"]
    cu = [i * w.steps for i in range(w.num_seqs + 1)]
    o_ref, S_ref = oracle.fwd(d["q"], d["k"], d["v"], d["a"], d["b"], inp["A_log"],
                              inp["dt_bias"], initial_state=inp["initial_state"], cu_seqlens=cu)
    eo, es = U.compare_full(o_all, state, o_ref, S_ref, cu, w.H_v)
    note(f"  recurrent, in place: worst o={eo:.3e} S={es:.3e}")
    assert eo <= TOL and es <= TOL, (eo, es)
    # the same tokens as one chunked call
    o_c, S_c = gdr.chunked_fwd(d["q"], d["k"], d["v"], d["a"], d["b"], inp["A_log"],
                               inp["dt_bias"], inp["initial_state"], chunk=32,
                               num_seqs=w.num_seqs)
    torch.cuda.synchronize()
    eo, es = U.compare_full(o_c, S_c, o_ref, S_ref, cu, w.H_v)
    note(f"  chunked, one call: worst o={eo:.3e} S={es:.3e}")
    assert eo <= TOL and es <= TOL, (eo, es)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_varlen_every_pair(seed):
    w = synth.workload("varlen", seed=seed)
    inp = synth.make_inputs(w, seed, device=DEV)
    note(f"[full] varlen seed {seed}: lengths {w.seq_lengths}, stress sequences "
         f"{list(w.stress_seqs)}")
    ref = U.oracle_full(inp, inp["cu_host"])
    for form in ("chunked_coop", "chunked_one_launch", "recurrent"):
        o, S = run_form(form, inp, w)
        torch.cuda.synchronize()
        eo, es = U.compare_full(o, S, ref[0], ref[1], inp["cu_host"], w.H_v)
        note(f"  {form}, all {len(w.seq_lengths) * w.H_v} pairs: worst o={eo:.3e} S={es:.3e}")
        assert eo <= TOL and es <= TOL, (form, eo, es)
        del o, S


def test_varlen_maximum_lengths_sampled():
    """The varlen workload at the top of its length range: 8 packed
    sequences of 32768 tokens (262,144 tokens, 48/16 heads, carried state,
    stress sequences 6 and 7), in the cooperative form the benchmark times
    and the one-launch form, against the oracle on two value heads of every
    sequence (byte offsets into v and o past 2^31)."""
    w = synth.workload("varlen", lengths=[32768] * 8)
    assert w.total_tokens * w.H_v * w.d_v * 2 > 2 ** 31
    inp = synth.make_inputs(w, 3, device=DEV)
    cu = inp["cu_host"]
    note(f"[full] varlen at the maximum lengths: {w.seq_lengths}")
    pairs = [(n, h) for n in range(w.num_seqs) for h in (5, 40)]
    ref = U.oracle_pairs(inp, cu, pairs)
    for form in ("chunked_coop", "chunked_one_launch"):
        o, S = run_form(form, inp, w)
        torch.cuda.synchronize()
        eo, es, per = U.compare_sampled(o, S, ref, cu)
        note(f"  {form}, {len(pairs)} pairs: worst o={eo:.3e} S={es:.3e}")
        assert eo <= TOL and es <= TOL, (form, per)
        del o, S


def test_kda_varlen_sampled_pairs():
    """The per-channel-decay variant on the varlen batch: both matrix-core
    forms against its fp64 oracle on sampled pairs (the oracle's per-token
    loop is too slow for all 384)."""
    w = synth.workload("varlen")
    inp = synth.kda_inputs(w, 73, device=DEV)
    cu = inp["cu_host"]
    G = w.H_v // w.H_k
    # the shortest sequences, the stress slice (6, 7) and spread heads
    order = sorted(range(w.num_seqs), key=lambda n: cu[n + 1] - cu[n])
    pairs = [(order[0], 0), (order[0], 47), (order[1], 20), (6, 5), (7, 33)]
    note(f"[full] kda varlen, pairs {pairs} of lengths "
         f"{[cu[n + 1] - cu[n] for n, _ in pairs]}")
    refs = {}
    for n, h in pairs:
        t0, t1, hk = cu[n], cu[n + 1], h // G
        cut = lambda x, lo, hi: x[t0:t1, lo:hi].cpu()
        s0 = None if inp["initial_state"] is None else inp["initial_state"][n:n + 1, h:h + 1].cpu()
        refs[(n, h)] = kda_oracle.kda(cut(inp["q"], hk, hk + 1), cut(inp["k"], hk, hk + 1),
                                      cut(inp["v"], h, h + 1), cut(inp["a"], h, h + 1),
                                      cut(inp["b"], h, h + 1), inp["A_log"][h:h + 1].cpu(),
                                      inp["dt_bias"][h:h + 1].cpu(), initial_state=s0,
                                      num_seqs=1)
    for fused in (False, True):
        o, S = gdr.kda_chunked_fwd(*args(inp), chunk=32, cu_seqlens=inp["cu_seqlens"],
                                   num_seqs=w.num_seqs, fused=fused)
        torch.cuda.synchronize()
        worst = 0.0
        for (n, h), (o_r, S_r) in refs.items():
            worst = max(worst, U.slice_err(U.to_np(o[cu[n]:cu[n + 1], h]), o_r[:, 0]),
                        U.slice_err(U.to_np(S[n, h]), S_r[0, 0]))
        note(f"  {'one-launch' if fused else 'two-launch'} form: worst {worst:.3e}")
        assert worst <= TOL, worst
