"""GPU parity of the per-channel-decay variant (KDA: gdr_kda_recurrent_fwd,
gdr_kda_chunked_fwd, through the C ABI) against the fp64 oracle in
``oracle.kda``.

Same metric and bars as the rule: per (sequence, value head) slice of o and
of the final state, max |x - y| / max |y|; 1e-4 for fp32 inputs, 2e-2 for
bf16 inputs (fp32 state; both kernels compute in fp32).  Inputs from
synth.kda_inputs: the rule's distributions with a [tokens, H_v, d_k] ~ N(0, 1)
and dt_bias [H_v, d_k] ~ N(0, 0.1); the strong-decay case draws a ~ N(4, 1)
(alpha down to about e^-60 per step), the long-memory case a ~ N(-6, 1).
"""
import pytest
import torch

import gated_delta_rule_68_amd as gdr
import synth
from oracle import kda
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

DEV = "cuda"


def note(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.lib()
    yield
    torch.cuda.synchronize()


def run(form, inp, w, chunk=32, **kw):
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])
    if form == "recurrent":
        return gdr.kda_recurrent_fwd(*args, cu_seqlens=inp["cu_seqlens"], num_seqs=w.num_seqs,
                                     **kw)
    # "chunked": the two-launch form (a workspace); "chunked_fused": the
    # one-launch form (none); both reach the vector kernel off their shapes
    return gdr.kda_chunked_fwd(*args, chunk=chunk, cu_seqlens=inp["cu_seqlens"],
                               num_seqs=w.num_seqs, fused=form == "chunked_fused", **kw)


def oracle_of(inp, heads=None):
    """The oracle over every value head, or over ``heads`` only (inputs cut
    to those heads and their key heads)."""
    q, k, v, a, b = inp["q"], inp["k"], inp["v"], inp["a"], inp["b"]
    A_log, dtb, s0 = inp["A_log"], inp["dt_bias"], inp["initial_state"]
    cu = inp["cu_host"]
    if heads is None:
        return kda.kda(q.cpu(), k.cpu(), v.cpu(), a.cpu(), b.cpu(), A_log.cpu(), dtb.cpu(),
                       None if s0 is None else s0.cpu(), cu_seqlens=cu)
    H_k, H_v = q.shape[1], v.shape[1]
    outs = [kda.kda(q[:, h // (H_v // H_k)][:, None].cpu(), k[:, h // (H_v // H_k)][:, None].cpu(),
                    v[:, h:h + 1].cpu(), a[:, h:h + 1].cpu(), b[:, h:h + 1].cpu(),
                    A_log[h:h + 1].cpu(), dtb[h:h + 1].cpu(),
                    None if s0 is None else s0[:, h:h + 1].cpu(), cu_seqlens=cu)
            for h in heads]
    import numpy as np
    return (np.concatenate([o for o, _ in outs], axis=1),
            np.concatenate([s for _, s in outs], axis=1))


def check(w, seed, form, chunk=32, heads=None, a_mean=0.0, tag=""):
    note(f"[kda] {tag} {form} chunk={chunk} H={w.H_v}/{w.H_k} d={w.d_k}x{w.d_v} {w.dtype} "
         f"lens={w.seq_lengths if len(w.seq_lengths) < 8 else len(w.seq_lengths)} seed={seed}")
    inp = synth.kda_inputs(w, seed, device=DEV, a_mean=a_mean)
    o, S = run(form, inp, w, chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_of(inp, heads)
    if heads is not None:
        o, S = o[:, heads], S[:, heads]
    eo, es = U.compare_full(o, S, o_ref, S_ref, inp["cu_host"], o_ref.shape[1])
    tol = U.TOL[w.dtype]
    note(f"  max rel err o={eo:.3e} S={es:.3e} (bar {tol:g})")
    assert eo <= tol and es <= tol, (eo, es)
    return inp, o, S


SHAPES = [
    # H_k, H_v, d_k, d_v, lengths
    (2, 6, 128, 128, [100, 0, 37]),
    (2, 4, 128, 64, [300, 1, 0, 64]),
    (1, 3, 64, 32, [0, 1, 31, 32, 33, 70]),
    (2, 2, 16, 64, [17, 64, 5]),
    (4, 8, 32, 16, [40, 9]),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"H{s[1]}/{s[0]}_d{s[2]}x{s[3]}")
@pytest.mark.parametrize("form,chunk", [("recurrent", None), ("chunked", 16), ("chunked", 32),
                                        ("chunked_fused", 32)])
def test_kda_small_shapes(dtype, shape, form, chunk):
    H_k, H_v, d_k, d_v, lens = shape
    w = synth.custom(H_k, H_v, d_k, d_v, dtype, lengths=lens, chunk=chunk or 32)
    check(w, 61, form, chunk or 32)


@pytest.mark.parametrize("form", ["chunked", "chunked_fused", "recurrent"])
@pytest.mark.parametrize("a_mean", [4.0, -6.0], ids=["strong_decay", "long_memory"])
def test_kda_gate_extremes(form, a_mean):
    """Strong decay: factors through a row inside a 16-row block would
    overflow, so this checks the exact diagonal blocks of the matrix-core
    kernel; long memory: the state carries across many chunks."""
    w = synth.custom(1, 2, 128, 128, "bf16", lengths=[200, 65], chunk=32)
    check(w, 62, form, 32, a_mean=a_mean, tag=f"a~N({a_mean},1)")


def test_kda_without_initial_state_dense():
    w = synth.custom(2, 4, 64, 64, "f32", seq_len=96, num_seqs=3, chunk=32, init_state=False)
    check(w, 63, "chunked", 32)
    check(w, 63, "recurrent")


def test_kda_chunked_equals_recurrent():
    w = synth.custom(2, 6, 128, 128, "bf16", lengths=[333, 64, 1], chunk=32)
    inp = synth.kda_inputs(w, 64, device=DEV)
    o1, S1 = run("chunked", inp, w, 32)
    o2, S2 = run("chunked", inp, w, 16)
    o3, S3 = run("recurrent", inp, w)
    torch.cuda.synchronize()
    cu = inp["cu_host"]
    worst = 0.0
    for o, S in ((o2, S2), (o3, S3)):
        for n in range(len(cu) - 1):
            for h in range(w.H_v):
                worst = max(worst, U.slice_err(U.to_np(o[cu[n]:cu[n + 1], h]),
                                               U.to_np(o1[cu[n]:cu[n + 1], h])),
                            U.slice_err(U.to_np(S[n, h]), U.to_np(S1[n, h])))
    note(f"  chunk 32 vs chunk 16 vs recurrent: {worst:.3e}")
    assert worst <= U.TOL["bf16"]  # fp32 arithmetic, but o is rounded to bf16


def test_kda_streaming_prefill_then_decode():
    """Prefill 96 tokens chunked, then 24 single-token steps in place: the
    oracle over all 120 tokens."""
    w = synth.custom(1, 3, 128, 128, "f32", lengths=[120], chunk=32)
    inp = synth.kda_inputs(w, 65, device=DEV)
    o_ref, S_ref = oracle_of(inp)
    args = lambda a, e: [inp[x][a:e] for x in ("q", "k", "v", "a", "b")] + [inp["A_log"],
                                                                             inp["dt_bias"]]
    o0, st = gdr.kda_chunked_fwd(*args(0, 96), inp["initial_state"], chunk=32, num_seqs=1)
    st = st.clone()
    outs = [o0]
    for t in range(96, 120):
        o, _ = gdr.kda_recurrent_fwd(*args(t, t + 1), st, num_seqs=1, inplace=True)
        outs.append(o)
    torch.cuda.synchronize()
    eo, es = U.compare_full(torch.cat(outs), st, o_ref, S_ref, [0, 120], 3)
    note(f"  streamed: o={eo:.3e} S={es:.3e}")
    assert eo <= U.TOL["f32"] and es <= U.TOL["f32"], (eo, es)


def test_kda_deterministic_and_inplace():
    w = synth.custom(2, 6, 128, 128, "bf16", lengths=[257, 31], chunk=32)
    inp = synth.kda_inputs(w, 66, device=DEV)
    a = run("chunked", inp, w, 32)
    b = run("chunked", inp, w, 32)
    st = inp["initial_state"].clone()
    c = run("chunked", dict(inp, initial_state=st), w, 32, inplace=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c[0], a[0]) and torch.equal(st, a[1])


@pytest.mark.parametrize("form", ["chunked", "chunked_fused"])
def test_kda_prefill_layer_sampled(form):
    """The prefill layer (8192 tokens, 48/16 heads, d = 128, bf16, chunk 32)
    in the launch configuration the benchmark times; the oracle checks three
    value heads."""
    w = synth.workload("prefill")
    check(w, 67, form, 32, heads=[0, 25, 47], tag="prefill")


@pytest.mark.parametrize("lens,d_v,with_state", [
    ([31, 0, 32, 33, 95, 1, 64], 128, True),
    ([31, 0, 32, 33, 95, 1, 64], 64, False),
    ([700, 5], 128, True),
], ids=["ragged_dv128", "ragged_dv64_nostate", "long_dv128"])
def test_kda_two_launch_vs_one_launch(lens, d_v, with_state):
    """The two-launch form against the one-launch form on the same inputs:
    ragged tails, empty and one-token sequences, with and without a carried
    state."""
    w = synth.custom(2, 6, 128, d_v, "bf16", lengths=lens, chunk=32)
    inp = synth.kda_inputs(w, 71, device=DEV)
    if not with_state:
        inp = dict(inp, initial_state=None)
    o1, S1 = run("chunked", inp, w, 32)
    o2, S2 = run("chunked_fused", inp, w, 32)
    torch.cuda.synchronize()
    cu = inp["cu_host"]
    worst = 0.0
    for n in range(len(cu) - 1):
        for h in range(w.H_v):
            if cu[n + 1] > cu[n]:
                worst = max(worst, U.slice_err(U.to_np(o1[cu[n]:cu[n + 1], h]),
                                               U.to_np(o2[cu[n]:cu[n + 1], h])))
            worst = max(worst, U.slice_err(U.to_np(S1[n, h]), U.to_np(S2[n, h])))
    note(f"  two-launch vs one-launch: {worst:.3e}")
    assert worst <= U.TOL["bf16"]


@pytest.mark.parametrize("d_v", [16, 32])
def test_kda_two_launch_other_widths(d_v):
    """Value widths that only the two-launch form runs on the matrix cores
    (the one-launch form takes 64 and 128)."""
    w = synth.custom(1, 2, 128, d_v, "bf16", lengths=[77, 32], chunk=32)
    check(w, 72, "chunked", 32, tag=f"d_v={d_v}")


def test_kda_decode_step_sampled():
    """One single-token step of the decode batch (256 sequences x 48/16
    heads, d = 128, bf16, random state), in place; the oracle checks every
    head of 4 sequences."""
    w = synth.workload("decode")
    inp = synth.kda_inputs(w, 68, device=DEV)
    st = inp["initial_state"].clone()
    x = [inp[n][0] for n in ("q", "k", "v", "a", "b")]
    o, _ = gdr.kda_recurrent_fwd(*x, inp["A_log"], inp["dt_bias"], st, num_seqs=256,
                                 inplace=True)
    torch.cuda.synchronize()
    worst = 0.0
    for n in (0, 77, 128, 255):
        o_r, S_r = kda.kda(*[t[n:n + 1].cpu() for t in x], inp["A_log"].cpu(),
                           inp["dt_bias"].cpu(), inp["initial_state"][n:n + 1].cpu(), num_seqs=1)
        eo, es = U.compare_full(o[n:n + 1], st[n:n + 1], o_r, S_r, [0, 1], w.H_v)
        worst = max(worst, eo, es)
    note(f"  decode step: {worst:.3e}")
    assert worst <= U.TOL["bf16"]


def test_kda_rejects_bad_arguments():
    w = synth.custom(1, 2, 64, 64, "bf16", lengths=[8])
    inp = synth.kda_inputs(w, 69, device=DEV)
    with pytest.raises(gdr.GdrError, match="UNSUPPORTED"):
        run("chunked", inp, w, 64)
    with pytest.raises(ValueError):  # a with one value per head is the rule's, not KDA's
        gdr.kda_recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["a"][..., 0].contiguous(),
                              inp["b"], inp["A_log"], inp["dt_bias"])


@pytest.mark.parametrize("lens", [[2048], [31, 32, 33, 95, 1]], ids=["T2048", "ragged"])
def test_kda_matrix_core_vs_vector_kernel(lens):
    """The bf16 matrix-core kernel (chunk 32) against the fp32 vector kernel
    (chunk 16) on the same inputs, over a long sequence and ragged tails."""
    w = synth.custom(2, 6, 128, 128, "bf16", lengths=lens, chunk=32)
    inp = synth.kda_inputs(w, 70, device=DEV)
    o1, S1 = run("chunked", inp, w, 32)
    o2, S2 = run("chunked", inp, w, 16)
    torch.cuda.synchronize()
    cu = inp["cu_host"]
    worst = 0.0
    for n in range(len(cu) - 1):
        for h in range(w.H_v):
            worst = max(worst, U.slice_err(U.to_np(o1[cu[n]:cu[n + 1], h]),
                                           U.to_np(o2[cu[n]:cu[n + 1], h])),
                        U.slice_err(U.to_np(S1[n, h]), U.to_np(S2[n, h])))
    note(f"  matrix-core vs vector kernel: {worst:.3e}")
    assert worst <= U.TOL["bf16"]


def test_kda_two_launch_on_the_varlen_batch():
    """The varlen workload (8 packed sequences, about 94k tokens, 48/16
    heads, carried state) through both matrix-core forms: the two-launch
    form's slot numbering and per-slot sequence lookup at full scale, the two
    forms against each other on every (sequence, head) and against the fp64
    oracle on one head of every sequence."""
    w = synth.workload("varlen")
    inp = synth.kda_inputs(w, 73, device=DEV)
    note(f"[kda] varlen two-launch vs one-launch lens={w.seq_lengths}")
    o1, S1 = run("chunked", inp, w, 32)
    o2, S2 = run("chunked_fused", inp, w, 32)
    torch.cuda.synchronize()
    cu = inp["cu_host"]
    worst = 0.0
    for n in range(len(cu) - 1):
        for h in range(w.H_v):
            worst = max(worst, U.slice_err(U.to_np(o1[cu[n]:cu[n + 1], h]),
                                           U.to_np(o2[cu[n]:cu[n + 1], h])),
                        U.slice_err(U.to_np(S1[n, h]), U.to_np(S2[n, h])))
    note(f"  two-launch vs one-launch on the varlen batch: {worst:.3e}")
    assert worst <= U.TOL["bf16"]
    # and both against the fp64 oracle on one value head of every sequence
    heads = [29]
    o_ref, S_ref = oracle_of(inp, heads)
    for name, (o, S) in (("two-launch", (o1, S1)), ("one-launch", (o2, S2))):
        eo, es = U.compare_full(o[:, heads], S[:, heads], o_ref, S_ref, cu, 1)
        note(f"  {name} vs oracle (head 29, every sequence): o={eo:.3e} S={es:.3e}")
        assert eo <= U.TOL["bf16"] and es <= U.TOL["bf16"], (name, eo, es)


@pytest.mark.parametrize("form", ["recurrent", "chunked", "chunked_fused"])
def test_kda_empty_batch(form):
    """Only empty sequences: the two-launch form's prep finds no chunk in any
    slot and its chains copy the initial state (or zeros) to the final one."""
    w = synth.custom(1, 2, 128, 64, "bf16", lengths=[0, 0, 0], chunk=32)
    inp = synth.kda_inputs(w, 74, device=DEV)
    o, S = run(form, inp, w)
    torch.cuda.synchronize()
    assert o.shape[0] == 0
    assert torch.equal(S, inp["initial_state"])
    o, S = run(form, dict(inp, initial_state=None), w)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0
