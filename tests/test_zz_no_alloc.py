"""The allocation-free chunked entry point, gdr_chunked_fwd_noalloc, through
the C ABI: its cooperative workspace is the library's own per-device scratch
array.  Each call is held to gdr_chunked_fwd with a workspace the caller
allocated: the same cooperative kernel on the same inputs, so the outputs and
final states must agree bit for bit.  Two calls run in a row on the one
scratch, the second on a smaller batch, then the first again; a shape whose
workspace exceeds the scratch is refused with GDR_ERR_WORKSPACE."""
import sys

import pytest
import torch

import gated_delta_rule_68_amd as gdr
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


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


def check_against_workspace_call(w, seed):
    inp = synth.make_inputs(w, seed, device=DEV)
    ws = gdr.chunked_workspace(w.H_k, w.H_v, w.d_k, w.d_v, "bf16", len(w.seq_lengths), device=DEV)
    assert ws is not None and ws.numel() <= gdr.NOALLOC_SCRATCH_BYTES
    ref_o, ref_S = gdr.chunked_fwd(*args(inp), chunk=32, workspace=ws, **seq_kw(inp))
    o, S = torch.empty_like(ref_o), torch.empty_like(ref_S)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    gdr.chunked_fwd_noalloc(*args(inp), chunk=32, o=o, final_state=S, **seq_kw(inp))
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.equal(o, ref_o) and torch.equal(S, ref_S)


def test_noalloc_matches_workspace_calls():
    large = synth.workload("prefill")  # 8192 tokens, 16 key heads, 48 value heads
    small = synth.custom(2, 6, 128, 128, "bf16", lengths=[777, 64, 1], chunk=32)
    for tag, w, seed in (("prefill layer", large, 61), ("smaller batch", small, 62),
                         ("prefill layer again", large, 63)):
        note(f"[noalloc] {tag}: lengths {w.seq_lengths[:4]} H {w.H_v}/{w.H_k}")
        check_against_workspace_call(w, seed)


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    w = synth.custom(24, 72, 128, 64, "bf16", lengths=[64], chunk=32)
    assert gdr.chunked_workspace_bytes(24, 72, 128, 64, "bf16") > gdr.NOALLOC_SCRATCH_BYTES
    inp = synth.make_inputs(w, 64, device=DEV)
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunked_fwd_noalloc(*args(inp), chunk=32, **seq_kw(inp))
    assert e.value.status == 5
