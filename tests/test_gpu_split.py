"""GPU parity of the segmented chunked form (gdr_chunked_fwd_split, a
two-level scan over segments of each sequence) against the fp64 oracle,
through the C ABI.  Same bars and metric as the other forms (1e-4 for fp32
inputs, 2e-2 for bf16 inputs with fp32 state; per (sequence, head) slice of
o and of the final state); with one segment it must give the bits of
gdr_chunked_fwd."""
import pytest
import torch

import gated_delta_rule_68_amd as gdr
import synth
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


def batch(w, inp):
    """The batch arguments: cu_seqlens for a packed workload, else num_seqs."""
    if w.lengths is not None:
        return dict(cu_seqlens=inp["cu_seqlens"])
    return dict(num_seqs=w.num_seqs)


def run_split(w, inp, seg, **kw):
    return gdr.chunked_fwd_split(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                                 inp["dt_bias"], inp["initial_state"], segment_len=seg,
                                 chunk=w.chunk, **batch(w, inp), **kw)


def check(w, seed, seg):
    note(f"[split] H={w.H_v}/{w.H_k} d_k={w.d_k} d_v={w.d_v} {w.dtype} N={w.num_seqs} "
         f"T={w.seq_len} lengths={w.lengths} chunk={w.chunk} segment={seg} seed={seed}")
    inp = synth.make_inputs(w, seed, device=DEV)
    o, S = run_split(w, inp, seg)
    torch.cuda.synchronize()
    o_ref, S_ref = U.oracle_full(inp, inp["cu_host"])
    eo, es = U.compare_full(o, S, o_ref, S_ref, inp["cu_host"], w.H_v)
    tol = U.TOL[w.dtype]
    note(f"  max rel err o={eo:.3e} S={es:.3e} (bar {tol:g})")
    assert eo <= tol and es <= tol, (eo, es)
    return inp, o, S


def test_split_one_head_real_state_f32():
    """The one-head workload (T = 4096, d = 128, fp32, chunk 32) in 8 segments."""
    w = synth.workload("one_head")
    check(w, 0, 512)


@pytest.mark.parametrize("seg", [64, 256, 1024])
def test_split_matrix_core_bf16(seg):
    w = synth.custom(1, 3, 128, 128, "bf16", seq_len=1024, num_seqs=2, chunk=32)
    check(w, 31, seg)


@pytest.mark.parametrize("d,dtype,chunk", [(16, "f32", 16), (32, "f32", 32), (64, "bf16", 64),
                                           (128, "f32", 16)])
def test_split_head_sizes(d, dtype, chunk):
    """Every head size (the combine pass has 1, 2 or 4 rows per thread)."""
    w = synth.custom(2, 4, d, d, dtype, seq_len=4 * chunk * 3, num_seqs=3, chunk=chunk)
    check(w, 32, chunk * 3)


def test_split_one_segment_is_the_direct_form():
    """One segment is gdr_chunked_fwd without a workspace (the one-launch
    form), bit for bit; the cooperative form, which a workspace selects,
    agrees with it only up to float reassociation."""
    w = synth.custom(1, 2, 128, 128, "bf16", seq_len=512, num_seqs=2, chunk=32)
    inp = synth.make_inputs(w, 33, device=DEV)
    o1, S1 = run_split(w, inp, 512)
    o2, S2 = gdr.chunked_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                             inp["dt_bias"], inp["initial_state"], chunk=32, num_seqs=2,
                             workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_split_in_place_and_without_initial_state():
    w = synth.custom(1, 2, 64, 64, "f32", seq_len=256, num_seqs=2, chunk=32)
    inp = synth.make_inputs(w, 34, device=DEV)
    o_ref, S_ref = U.oracle_full(inp, inp["cu_host"])
    st = inp["initial_state"].clone()
    o, S = run_split(w, dict(inp, initial_state=st), 64, inplace=True)
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr()
    eo, es = U.compare_full(o, S, o_ref, S_ref, inp["cu_host"], w.H_v)
    assert eo <= U.TOL["f32"] and es <= U.TOL["f32"], (eo, es)
    w0 = synth.custom(1, 2, 64, 64, "f32", seq_len=256, num_seqs=2, chunk=32, init_state=False)
    check(w0, 35, 128)


def test_split_long_single_head():
    """One bf16 head of 32768 tokens in 32 segments of 1024."""
    w = synth.custom(1, 1, 128, 128, "bf16", seq_len=32768, num_seqs=1, chunk=32)
    check(w, 36, 1024)


def test_split_long_memory_stress():
    """beta -> 1 and g -> 0 (b ~ N(4, 1), a ~ N(-6, 1)): the state carries
    across segments, so the segment maps M are far from zero."""
    w = synth.custom(1, 2, 128, 128, "bf16", seq_len=2048, num_seqs=2, chunk=32,
                     stress_seqs=(0, 1))
    check(w, 37, 256)
    wf = synth.custom(1, 2, 64, 64, "f32", seq_len=1024, num_seqs=1, chunk=32, stress_seqs=(0,))
    check(wf, 38, 128)


# ------------------------------------------- packed batches, d_k != d_v
# lengths with partial last segments, an empty sequence, one token, a length
# that is a whole number of segments and one shorter than a chunk
PACKED = [300, 0, 1, 128, 1000, 257, 33]


@pytest.mark.parametrize("d,dtype,chunk,seg", [(128, "bf16", 32, 128), (64, "f32", 16, 64),
                                               (32, "f32", 32, 96)])
def test_split_packed_ragged(d, dtype, chunk, seg):
    """A packed batch: every sequence cut into max(1, ceil(L / seg)) segments
    by the device-side segment map, the last one partial."""
    w = synth.custom(1, 3, d, d, dtype, lengths=PACKED, chunk=chunk)
    check(w, 50, seg)


def test_split_packed_without_initial_state_and_in_place():
    w = synth.custom(2, 4, 64, 64, "f32", lengths=[200, 65, 0, 96], chunk=32, init_state=False)
    check(w, 51, 64)
    w = synth.custom(2, 4, 64, 64, "f32", lengths=[200, 65, 0, 96], chunk=32)
    inp = synth.make_inputs(w, 52, device=DEV)
    o_ref, S_ref = U.oracle_full(inp, inp["cu_host"])
    st = inp["initial_state"].clone()
    o, S = run_split(w, dict(inp, initial_state=st), 64, inplace=True)
    torch.cuda.synchronize()
    assert S.data_ptr() == st.data_ptr()
    eo, es = U.compare_full(o, S, o_ref, S_ref, inp["cu_host"], w.H_v)
    assert eo <= U.TOL["f32"] and es <= U.TOL["f32"], (eo, es)


@pytest.mark.parametrize("dk,dv,dtype,chunk,seg,packed", [
    (128, 64, "bf16", 32, 256, False), (128, 64, "bf16", 32, 128, True),
    (64, 32, "f32", 16, 64, False), (32, 64, "f32", 32, 64, True)])
def test_split_key_and_value_widths_differ(dk, dv, dtype, chunk, seg, packed):
    """d_k != d_v: the segment maps M are d_k x d_k, from the kernels run with
    d_k-wide values into a workspace buffer rather than o."""
    if packed:
        w = synth.custom(1, 2, dk, dv, dtype, lengths=[500, 1, 260], chunk=chunk)
    else:
        w = synth.custom(1, 2, dk, dv, dtype, seq_len=4 * seg, num_seqs=2, chunk=chunk)
    check(w, 53, seg)


def test_split_packed_batch_in_one_segment_is_the_direct_form():
    """A packed batch of at most segment_len tokens runs gdr_chunked_fwd
    without a workspace (the one-launch form), bit for bit."""
    w = synth.custom(1, 2, 128, 128, "bf16", lengths=[40, 0, 23], chunk=32)
    inp = synth.make_inputs(w, 54, device=DEV)
    o1, S1 = run_split(w, inp, 64)
    o2, S2 = gdr.chunked_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                             inp["dt_bias"], inp["initial_state"], chunk=32,
                             cu_seqlens=inp["cu_seqlens"], workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_split_varlen_workload_sampled():
    """The varlen workload (8 packed sequences of U[512, 32768] tokens, 48/16
    heads, carried state, stress sequences 6 and 7) in segments of 2048
    tokens, against the oracle on two heads of every sequence."""
    w = synth.workload("varlen", seed=0)
    note(f"[split] varlen lengths={w.seq_lengths} segment=2048")
    inp = synth.make_inputs(w, 0, device=DEV)
    o, S = run_split(w, inp, 2048)
    torch.cuda.synchronize()
    cu = inp["cu_host"]
    pairs = [(n, h) for n in range(w.num_seqs) for h in (0, 29)]
    ref = U.oracle_pairs(inp, cu, pairs)
    eo, es, per = U.compare_sampled(o, S, ref, cu)
    note(f"  max rel err o={eo:.3e} S={es:.3e}")
    assert eo <= U.TOL["bf16"] and es <= U.TOL["bf16"], per


# ---------------------------------------------------------------- KDA segments
def check_kda(w, seed, seg, a_mean=0.0):
    from oracle import kda
    note(f"[kda split] H={w.H_v}/{w.H_k} d_k={w.d_k} d_v={w.d_v} {w.dtype} N={w.num_seqs} "
         f"T={w.seq_len} lengths={w.lengths} chunk={w.chunk} segment={seg} seed={seed}")
    inp = synth.kda_inputs(w, seed, device=DEV, a_mean=a_mean)
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])
    o, S = gdr.kda_chunked_fwd_split(*args, segment_len=seg, chunk=w.chunk, **batch(w, inp))
    torch.cuda.synchronize()
    o_ref, S_ref = kda.kda(*[t.cpu() if t is not None else None for t in args],
                           cu_seqlens=inp["cu_host"])
    eo, es = U.compare_full(o, S, o_ref, S_ref, inp["cu_host"], w.H_v)
    tol = U.TOL[w.dtype]
    note(f"  max rel err o={eo:.3e} S={es:.3e} (bar {tol:g})")
    assert eo <= tol and es <= tol, (eo, es)
    return inp, args, o, S


@pytest.mark.parametrize("dtype,chunk,seg", [("bf16", 32, 256), ("f32", 16, 64), ("bf16", 16, 128)])
def test_kda_split(dtype, chunk, seg):
    w = synth.custom(1, 2, 128, 128, dtype, seq_len=1024, num_seqs=2, chunk=chunk)
    check_kda(w, 40, seg)


def test_kda_split_one_segment_is_the_direct_form_and_long_memory():
    w = synth.custom(1, 2, 128, 128, "bf16", seq_len=512, num_seqs=1, chunk=32)
    inp, args, o1, S1 = check_kda(w, 41, 512)
    # one segment runs the one-launch chunked kernel (no workspace)
    o2, S2 = gdr.kda_chunked_fwd(*args, chunk=32, num_seqs=1, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    wl = synth.custom(1, 1, 64, 64, "f32", seq_len=2048, num_seqs=1, chunk=32)
    check_kda(wl, 42, 256, a_mean=-6.0)  # long memory: the segment maps carry the state


@pytest.mark.parametrize("dtype,chunk,seg,dv", [("bf16", 32, 256, 128), ("bf16", 32, 128, 64),
                                                ("f32", 16, 64, 128)])
def test_kda_split_packed(dtype, chunk, seg, dv):
    """KDA on packed batches (bf16 chunk 32: one prep over all segment slots
    serves the three chain passes), also with d_v != d_k."""
    w = synth.custom(1, 2, 128, dv, dtype, lengths=[700, 0, 65, 1024, 1], chunk=chunk)
    check_kda(w, 55, seg)
