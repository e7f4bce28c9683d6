"""GPU checks of gdr_chunked_fwd_gated_rmsnorm, through the C ABI: the
chunked form followed by the gated RMSNorm of its output, against the fp64
oracle of the rule followed by the oracle's gated RMSNorm, on every
(sequence, value head) slice, at the bf16 bar of the rule; against the two
calls it stands for; without a workspace; and its alias check.
"""
import sys

import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as gdr
import synth
from oracle import layer
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = 1e-6


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


def gate_inputs(w, seed):
    """z [total, H_v, d_v] (bf16) and the norm weight [d_v] (fp32), seeded."""
    rng = np.random.default_rng(seed)
    total = int(sum(w.seq_lengths))
    z = torch.from_numpy(rng.standard_normal((total, w.H_v, w.d_v))).to(torch.bfloat16).to(DEV)
    nw = torch.from_numpy(1.0 + 0.1 * rng.standard_normal(w.d_v)).to(torch.float32).to(DEV)
    return z, nw


def rule_args(inp):
    return (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"])


def seqs(inp):
    return dict(cu_seqlens=inp["cu_seqlens"]) if inp["cu_seqlens"] is not None else \
        dict(num_seqs=len(inp["cu_host"]) - 1)


def one_call(inp, z, nw, ws):
    return gdr.chunked_fwd_gated_rmsnorm(*rule_args(inp), z, nw, inp["initial_state"],
                                         norm_eps=EPS, chunk=32, workspace=ws, **seqs(inp))


def two_calls(inp, z, nw, ws):
    o, S = gdr.chunked_fwd(*rule_args(inp), inp["initial_state"], chunk=32, workspace=ws,
                           **seqs(inp))
    return gdr.gated_rmsnorm(o, z, nw, EPS), S


def workspace_for(w):
    ws = gdr.chunked_workspace(w.H_k, w.H_v, w.d_k, w.d_v, "bf16", len(w.seq_lengths), device=DEV)
    assert ws is not None, "this shape should take the cooperative form"
    return ws


def oracle_out(inp, z, nw):
    o_ref, S_ref = U.oracle_full(inp, inp["cu_host"])
    return layer.gated_rmsnorm(o_ref, z, nw, EPS), S_ref


CASES = [
    # H_k, H_v, d_v, lengths
    (2, 6, 128, [200]),
    (2, 6, 64, [300, 1, 64, 0, 97]),
    (1, 3, 128, [300, 129, 0]),
    (8, 24, 128, [129] * 2),
]


def _id(c):
    return f"H{c[1]}/{c[0]}_dv{c[2]}_L{'-'.join(map(str, c[3]))}"


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_rule_then_norm_against_oracle(case):
    H_k, H_v, d_v, lens = case
    w = synth.custom(H_k, H_v, 128, d_v, "bf16", lengths=lens, chunk=32)
    note(f"[rule + norm] {_id(case)}")
    inp = synth.make_inputs(w, 61, device=DEV)
    z, nw = gate_inputs(w, 62)
    ws = workspace_for(w)
    out, S = one_call(inp, z, nw, ws)
    torch.cuda.synchronize()
    assert gdr.workspace_error(ws) == 0
    ref, S_ref = oracle_out(inp, z, nw)
    eo, es = U.compare_full(out, S, ref, S_ref, inp["cu_host"], w.H_v)
    note(f"  one call: max rel err out={eo:.3e} S={es:.3e}")
    assert eo <= U.TOL["bf16"] and es <= U.TOL["bf16"], (eo, es)
    # the two calls it stands for give the same bits
    out2, S2 = two_calls(inp, z, nw, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(S, S2)
    # no workspace: the one-launch form of the rule, then the norm
    out3, S3 = one_call(inp, z, nw, None)
    torch.cuda.synchronize()
    eo3, es3 = U.compare_full(out3, S3, ref, S_ref, inp["cu_host"], w.H_v)
    note(f"  without a workspace: max rel err out={eo3:.3e} S={es3:.3e}")
    assert eo3 <= U.TOL["bf16"] and es3 <= U.TOL["bf16"], (eo3, es3)


def test_rule_then_norm_prefill_layer():
    """The prefill layer (8192 tokens, 48 value heads sharing 16 key heads):
    every head of the normalised output against the oracle."""
    w = synth.workload("prefill")
    note("[rule + norm] prefill layer, all 48 heads")
    inp = synth.make_inputs(w, 0, device=DEV)
    z, nw = gate_inputs(w, 65)
    ws = workspace_for(w)
    out, S = one_call(inp, z, nw, ws)
    torch.cuda.synchronize()
    assert gdr.workspace_error(ws) == 0
    ref, S_ref = oracle_out(inp, z, nw)
    eo, es = U.compare_full(out, S, ref, S_ref, inp["cu_host"], w.H_v)
    note(f"  max rel err out={eo:.3e} S={es:.3e}")
    assert eo <= U.TOL["bf16"] and es <= U.TOL["bf16"], (eo, es)


def test_rule_then_norm_rejects_z_overlapping_out():
    w = synth.custom(1, 3, 128, 128, "bf16", lengths=[64], chunk=32)
    inp = synth.make_inputs(w, 66, device=DEV)
    z, nw = gate_inputs(w, 67)
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunked_fwd_gated_rmsnorm(*rule_args(inp), z, nw, inp["initial_state"], out=z,
                                      chunk=32, **seqs(inp))
    assert e.value.status == 7
