"""GPU checks of the two launch forms of the matrix-core chunked kernel,
through the C ABI: the cooperative form (producer workgroups form each
chunk's triangular inverse, output mask and row factors once per value head
and hand them to the chain workgroups through the workspace) and the fused
form (every chain workgroup forms them itself).  Both are held to the fp64
oracle at the bf16 bar, and the cooperative form's workspace protocol is
checked: no wait runs out, the workspace is left zero-filled for the next
call, and repeated calls on one workspace give the same bits.
"""
import sys

import pytest
import torch

import gated_delta_rule_68_amd as gdr
import synth
from tests import gpu_util as U

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


def run(inp, w, workspace):
    kw = dict(cu_seqlens=inp["cu_seqlens"]) if inp["cu_seqlens"] is not None else \
        dict(num_seqs=len(inp["cu_host"]) - 1)
    return gdr.chunked_fwd(*args(inp), chunk=32, workspace=workspace, **kw)


def workspace_for(w):
    ws = gdr.chunked_workspace(w.H_k, w.H_v, w.d_k, w.d_v, "bf16", len(w.seq_lengths), device=DEV)
    assert ws is not None, "this shape should take the cooperative form"
    return ws


def check_clean(ws):
    """No wait ran out, and the counters and flags are back to zero."""
    torch.cuda.synchronize()
    assert gdr.workspace_error(ws) == 0
    head = ws[:2048].view(torch.int32).view(16, 32)
    assert int(head[:, 0].abs().sum()) == 0 and int(head[:, 1].abs().sum()) == 0


COOP_CASES = [
    # H_k, H_v, d_v, lengths
    (2, 6, 128, [200]),
    (2, 6, 128, [0, 64, 65, 5]),
    (1, 3, 128, [300, 129, 0]),
    (4, 4, 128, [97, 33]),
    (1, 1, 128, [31, 32, 33]),
    (2, 6, 64, [300, 1, 64, 0, 97]),
    (16, 48, 128, [70]),
    (2, 4, 128, [1000, 513]),     # two value heads per key head
    (8, 24, 128, [129] * 2),      # 16 groups: every slot of every XCD
]


def _id(c):
    return f"H{c[1]}/{c[0]}_dv{c[2]}_L{'-'.join(map(str, c[3]))}"


@pytest.mark.parametrize("case", COOP_CASES, ids=_id)
def test_cooperative_form_against_oracle(case):
    H_k, H_v, d_v, lens = case
    w = synth.custom(H_k, H_v, 128, d_v, "bf16", lengths=lens, chunk=32)
    note(f"[coop] {_id(case)}")
    inp = synth.make_inputs(w, 51, device=DEV)
    ws = workspace_for(w)
    o, S = run(inp, w, ws)
    check_clean(ws)
    ref = U.oracle_full(inp, inp["cu_host"])
    eo, es = U.compare_full(o, S, ref[0], ref[1], inp["cu_host"], w.H_v)
    note(f"  cooperative: max rel err o={eo:.3e} S={es:.3e}")
    assert eo <= U.TOL["bf16"] and es <= U.TOL["bf16"], (eo, es)
    # the fused form on the same inputs
    o2, S2 = run(inp, w, None)
    torch.cuda.synchronize()
    eo2, es2 = U.compare_full(o2, S2, ref[0], ref[1], inp["cu_host"], w.H_v)
    note(f"  fused:       max rel err o={eo2:.3e} S={es2:.3e}")
    assert eo2 <= U.TOL["bf16"] and es2 <= U.TOL["bf16"], (eo2, es2)


def test_cooperative_form_repeats_bitwise_on_one_workspace():
    """Back-to-back calls on one workspace, with a call on other inputs in
    between: the protocol state left by a call never leaks into the next."""
    w = synth.custom(2, 6, 128, 128, "bf16", lengths=[777, 64, 1], chunk=32)
    a = synth.make_inputs(w, 52, device=DEV)
    b = synth.make_inputs(w, 53, device=DEV)
    ws = workspace_for(w)
    first = run(a, w, ws)
    for i in range(4):
        if i == 1:
            run(b, w, ws)
        again = run(a, w, ws)
        torch.cuda.synchronize()
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1]), f"call {i + 1}"
    check_clean(ws)


def test_prefill_layer_cooperative_full():
    """The prefill layer (8192 tokens, 48 value heads sharing 16 key heads):
    every head against the oracle, on the cooperative form."""
    w = synth.workload("prefill")
    note("[coop] prefill layer, all 48 heads")
    inp = synth.make_inputs(w, 0, device=DEV)
    ws = workspace_for(w)
    o, S = run(inp, w, ws)
    check_clean(ws)
    ref = U.oracle_full(inp, inp["cu_host"])
    eo, es = U.compare_full(o, S, ref[0], ref[1], inp["cu_host"], w.H_v)
    note(f"  max rel err o={eo:.3e} S={es:.3e}")
    assert eo <= U.TOL["bf16"] and es <= U.TOL["bf16"], (eo, es)


def test_undersized_workspace_is_refused():
    w = synth.custom(1, 3, 128, 128, "bf16", lengths=[64], chunk=32)
    inp = synth.make_inputs(w, 54, device=DEV)
    ws = workspace_for(w)
    with pytest.raises(gdr.GdrError) as e:
        run(inp, w, ws[:-256])
    assert e.value.status == 5


BATCH_CASES = [
    # H_k, H_v, d_v, lengths, dense: batches whose groups do not fit one
    # launch, run as consecutive cooperative launches of the sequences that do
    (16, 48, 128, [1100, 1024, 1500], False),   # one sequence a launch, packed
    (16, 48, 128, [1056, 1056, 1056], True),    # the same, dense
    (2, 6, 128, [1030] * 9 + [2100] * 9, False),  # 8 sequences a launch, 3 launches
    (4, 8, 64, [1200] * 9, True),               # d_v 64, two value heads a key head
]


def _bid(c):
    return f"H{c[1]}/{c[0]}_dv{c[2]}_N{len(c[3])}_{'dense' if c[4] else 'packed'}"


@pytest.mark.parametrize("case", BATCH_CASES, ids=_bid)
def test_cooperative_batches_against_oracle(case):
    """More (sequence, key head) groups than one launch holds: consecutive
    launches on one workspace, each left clean for the next; every slice
    against the oracle, with initial states carried in."""
    H_k, H_v, d_v, lens, dense = case
    if dense:
        w = synth.custom(H_k, H_v, 128, d_v, "bf16", seq_len=lens[0], num_seqs=len(lens), chunk=32)
    else:
        w = synth.custom(H_k, H_v, 128, d_v, "bf16", lengths=lens, chunk=32)
    note(f"[coop batches] {_bid(case)}")
    inp = synth.make_inputs(w, 55, device=DEV)
    ws = workspace_for(w)
    # the workspace is sized for one launch, not for the whole batch
    assert ws.numel() < 2048 + len(lens) * H_k * (512 + (H_v // H_k) * 16 * 7168)
    o, S = run(inp, w, ws)
    check_clean(ws)
    ref = U.oracle_full(inp, inp["cu_host"])
    eo, es = U.compare_full(o, S, ref[0], ref[1], inp["cu_host"], w.H_v)
    note(f"  max rel err o={eo:.3e} S={es:.3e}")
    assert eo <= U.TOL["bf16"] and es <= U.TOL["bf16"], (eo, es)
    # the same bits again on the same workspace
    o2, S2 = run(inp, w, ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S, S2)
