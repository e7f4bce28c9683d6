"""GPU parity at the contraction limit: keys that repeat a direction, under
long memory and beta -> 1, against the fp64 oracle through the C ABI.

Independent N(0, 1) keys at d_k = 128 are nearly orthogonal (mean |cos| of a
pair about 0.07), so the chunk matrix A stays small and (I + A)^-1 is close
to the identity.  Here every sequence draws its keys around one direction
(synth.coherent_keys: mean |cos| about 0.5 and about 0.9) with the stress
gates b ~ N(4, 1) (beta -> 1) and a ~ N(-6, 1) (g -> 0): the regime where the
erase term of the rule does the most work (GatedDeltaRule.ixx File
Reference, "Detailed Description"; Track L pull request, "Numerics
finding": the rule needs normalised keys and fp32 state to stay
well-conditioned) and where the triangular solve of the chunked form is
furthest from the identity.  Shapes are the prefill layer's heads: d = 128,
chunk 32, sequences of 2048 and more tokens.  Every (sequence, head) is
compared in full: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs.
"""
import sys

import pytest
import torch

import gated_delta_rule_68_amd as gdr
import synth
from oracle import kda as kda_oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DEV = "cuda"
EPS = [(1.0, "cos0.5"), (0.33, "cos0.9")]


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


def workload(dtype, lengths=(2048, 777)):
    return synth.custom(2, 6, 128, 128, dtype, lengths=list(lengths), chunk=32,
                        stress_seqs=tuple(range(len(lengths))))


def inputs(w, seed, eps, kda=False):
    inp = synth.kda_inputs(w, seed, device=DEV, a_mean=-6.0) if kda else \
        synth.make_inputs(w, seed, device=DEV)
    inp["k"] = synth.coherent_keys(w, seed, eps, device=DEV)
    return inp


def compare(tag, w, inp, o, S, ref):
    eo, es = U.compare_full(o, S, ref[0], ref[1], inp["cu_host"], w.H_v)
    tol = U.TOL[w.dtype]
    note(f"[coherent] {tag}: max rel err o={eo:.3e} S={es:.3e} (bar {tol:g})")
    assert eo <= tol and es <= tol, (eo, es)


def args(inp):
    return (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])


@pytest.mark.parametrize("eps,tag", EPS, ids=[t for _, t in EPS])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_coherent_keys_chunked(dtype, eps, tag):
    """gdr_chunked_fwd: the matrix-core kernels (bf16 and fp32 operands)."""
    w = workload(dtype)
    path = gdr.chunked_path(2, 6, 128, 128, dtype, 32)
    assert path == ("matrix_bf16" if dtype == "bf16" else "matrix_f32")
    note(f"[coherent] chunked {path} {tag} lens={w.seq_lengths}")
    inp = inputs(w, 41, eps)
    o, S = gdr.chunked_fwd(*args(inp), chunk=32, cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    compare(f"chunked {path} {tag}", w, inp, o, S, U.oracle_full(inp, inp["cu_host"]))


@pytest.mark.parametrize("eps,tag", EPS, ids=[t for _, t in EPS])
def test_coherent_keys_recurrent(eps, tag):
    w = workload("bf16")
    note(f"[coherent] recurrent {tag}")
    inp = inputs(w, 42, eps)
    o, S = gdr.recurrent_fwd(*args(inp), cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    compare(f"recurrent {tag}", w, inp, o, S, U.oracle_full(inp, inp["cu_host"]))


@pytest.mark.parametrize("eps,tag", EPS, ids=[t for _, t in EPS])
def test_coherent_keys_split(eps, tag):
    """gdr_chunked_fwd_split on the matrix cores: 4 segments of 512 tokens."""
    w = synth.custom(2, 6, 128, 128, "bf16", seq_len=2048, num_seqs=2, chunk=32,
                     stress_seqs=(0, 1))
    note(f"[coherent] split {tag}")
    inp = inputs(w, 43, eps)
    o, S = gdr.chunked_fwd_split(*args(inp), segment_len=512, chunk=32, num_seqs=2)
    torch.cuda.synchronize()
    compare(f"split {tag}", w, inp, o, S, U.oracle_full(inp, inp["cu_host"]))


@pytest.mark.parametrize("eps,tag", EPS, ids=[t for _, t in EPS])
@pytest.mark.parametrize("form", ["chunked", "chunked_fused"])
def test_coherent_keys_kda(form, eps, tag):
    """Both matrix-core forms of the per-channel-decay variant: the two-launch
    form (workspace) and the one-launch form."""
    w = workload("bf16")
    note(f"[coherent] kda {form} {tag}")
    inp = inputs(w, 44, eps, kda=True)
    o, S = gdr.kda_chunked_fwd(*args(inp), chunk=32, cu_seqlens=inp["cu_seqlens"],
                               num_seqs=w.num_seqs, fused=form == "chunked_fused")
    torch.cuda.synchronize()
    ref = kda_oracle.kda(*(x.cpu() for x in args(inp)), cu_seqlens=inp["cu_host"])
    compare(f"kda {form} {tag}", w, inp, o, S, ref)


@pytest.mark.parametrize("eps,tag", EPS, ids=[t for _, t in EPS])
def test_coherent_keys_split_packed(eps, tag):
    """gdr_chunked_fwd_split on a packed batch (the segment map formed on the
    device; the last segment of each sequence partial), its passes on the
    cooperative form, and the same for the KDA split."""
    w = workload("bf16", lengths=(2048, 777, 0, 1300))
    note(f"[coherent] split packed {tag}")
    inp = inputs(w, 45, eps)
    o, S = gdr.chunked_fwd_split(*args(inp), segment_len=512, chunk=32,
                                 cu_seqlens=inp["cu_seqlens"])
    torch.cuda.synchronize()
    compare(f"split packed {tag}", w, inp, o, S, U.oracle_full(inp, inp["cu_host"]))
    ik = inputs(w, 46, eps, kda=True)
    o, S = gdr.kda_chunked_fwd_split(*args(ik), segment_len=512, chunk=32,
                                     cu_seqlens=ik["cu_seqlens"])
    torch.cuda.synchronize()
    ref = kda_oracle.kda(*(x.cpu() for x in args(ik)), cu_seqlens=ik["cu_host"])
    compare(f"kda split packed {tag}", w, ik, o, S, ref)
