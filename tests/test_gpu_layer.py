"""GPU parity of the layer's steps either side of the rule (gdr_conv_silu,
gdr_gated_rmsnorm, through the C ABI) against the fp64 oracle in
``oracle.layer``.

Tolerances: the oracle receives the inputs exactly and the kernels compute in
fp32 (SiLU from the hardware exp2 and reciprocal, about 1 ulp each), so the
error is the fp32 arithmetic (a few ulp, under 1e-6 relative) plus the
rounding of the output to its dtype: bf16 keeps 8 significant bits, so
round-to-nearest is off by at most 2^-8 = 3.9e-3 of |y|.  Bars, as
max |x - y| over max |y| per sequence (conv) or over the whole output
(norm): 1e-5 for fp32, 4.5e-3 for bf16.  The returned conv history is a copy of input values, so it
must match bit for bit.

Inputs: seeded numpy draws -- in_proj outputs and histories ~ N(0, 1),
weights ~ N(0, 1/width), bias ~ N(0, 0.1), o and z ~ N(0, 1), norm weight
1 + N(0, 0.1) -- in the shapes of the prefill layer (48 value heads sharing
16 key heads, d = 128) and of small ragged batches.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_68_amd as gdr
from oracle import layer

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 4.5e-3}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def note(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdr.lib()
    yield
    torch.cuda.synchronize()


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=dtype)


def to_np(t):
    return t.detach().float().cpu().double().numpy()


def conv_case(seed, H_k, H_v, d_k, d_v, lengths, width=4, dtype="bf16", bias=True, state=True):
    rng = np.random.default_rng(seed)
    C = 2 * H_k * d_k + H_v * d_v
    total, N = int(sum(lengths)), len(lengths)
    dt = TDT[dtype]
    x = to_dev(rng.standard_normal((total, C)), dt)
    w = to_dev(rng.standard_normal((C, width)) / np.sqrt(width), torch.float32)
    b = to_dev(0.1 * rng.standard_normal(C), torch.float32) if bias else None
    s0 = to_dev(rng.standard_normal((N, C, width - 1)), dt) if state else None
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=DEV)
    return dict(x=x, w=w, b=b, s0=s0, cu=cu, C=C, N=N, shape=(H_k, H_v, d_k, d_v), dtype=dtype)


def check_conv(c, q, k, v, st, what):
    H_k, H_v, d_k, d_v = c["shape"]
    y_ref, st_ref = layer.short_conv_silu(c["x"], c["w"], c["b"], c["s0"],
                                          cu_seqlens=c["cu"].cpu().numpy())
    total = y_ref.shape[0]
    y = np.concatenate([to_np(q).reshape(total, H_k * d_k), to_np(k).reshape(total, H_k * d_k),
                        to_np(v).reshape(total, H_v * d_v)], axis=1)
    cu = c["cu"].cpu().numpy()
    worst = 0.0
    for n in range(len(cu) - 1):
        a, e = int(cu[n]), int(cu[n + 1])
        if e > a:
            ref = y_ref[a:e]
            worst = max(worst, np.max(np.abs(y[a:e] - ref)) / max(np.max(np.abs(ref)), 1e-30))
    note(f"  {what}: conv max rel err {worst:.2e} (bar {TOL[c['dtype']]:g})")
    assert worst <= TOL[c["dtype"]], worst
    if st is not None:
        # the history holds input values: compare in the input dtype, bit for bit
        ref = torch.from_numpy(st_ref).to(TDT[c["dtype"]])
        assert torch.equal(st.cpu(), ref), "conv history differs"


CONV_CASES = [
    # seed, H_k, H_v, d_k, d_v, lengths, width, dtype, bias, state
    (1, 2, 6, 128, 128, [200, 3, 0, 77], 4, "bf16", True, True),
    (2, 2, 6, 128, 128, [200, 3, 0, 77], 4, "f32", True, True),
    (3, 1, 2, 16, 32, [1, 2, 0, 5, 64, 65], 4, "f32", False, True),
    (4, 1, 2, 16, 32, [1, 2, 0, 5, 64, 65], 3, "bf16", True, False),
    (5, 4, 8, 32, 16, [130, 1], 2, "bf16", True, True),
    (6, 1, 1, 64, 64, [0, 0], 4, "bf16", True, True),
    (7, 3, 3, 16, 16, [63, 64, 65, 129], 4, "f32", True, True),
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: f"seed{c[0]}_w{c[6]}_{c[7]}")
def test_conv_silu_parity(case):
    seed, H_k, H_v, d_k, d_v, lengths, width, dtype, bias, state = case
    note(f"[conv] seed={seed} H={H_v}/{H_k} d={d_k}x{d_v} lens={lengths} width={width} {dtype}")
    c = conv_case(seed, H_k, H_v, d_k, d_v, lengths, width, dtype, bias, state)
    q, k, v, st = gdr.conv_silu(c["x"], c["w"], H_k, H_v, d_k, d_v, bias=c["b"],
                                conv_state=c["s0"], cu_seqlens=c["cu"])
    torch.cuda.synchronize()
    check_conv(c, q, k, v, st, "packed")


def test_conv_silu_dense_batch_and_no_history_output():
    c = conv_case(8, 2, 4, 32, 32, [33] * 4, 4, "bf16", True, True)
    q, k, v, st = gdr.conv_silu(c["x"], c["w"], 2, 4, 32, 32, bias=c["b"], conv_state=c["s0"],
                                num_seqs=4, output_final_state=False)
    torch.cuda.synchronize()
    assert st is None
    check_conv(c, q, k, v, None, "dense")


def test_conv_silu_decode_steps_equal_one_call():
    """64 single-token steps per sequence with the history updated in place
    give the same outputs and history as one call over the 64 tokens."""
    H_k, H_v, d = 16, 48, 128
    N, T = 8, 64
    c = conv_case(9, H_k, H_v, d, d, [T] * N, 4, "bf16", True, True)
    x = c["x"].view(N, T, -1)
    hist = c["s0"].clone()
    outs = []
    for t in range(T):
        xt = x[:, t].contiguous()
        q, k, v, _ = gdr.conv_silu(xt, c["w"], H_k, H_v, d, d, bias=c["b"], conv_state=hist,
                                   num_seqs=N, inplace=True)
        outs.append(torch.cat([q.view(N, -1), k.view(N, -1), v.view(N, -1)], dim=1))
    q1, k1, v1, st1 = gdr.conv_silu(c["x"], c["w"], H_k, H_v, d, d, bias=c["b"],
                                    conv_state=c["s0"], cu_seqlens=c["cu"])
    torch.cuda.synchronize()
    y_steps = torch.stack(outs, dim=1).reshape(N * T, -1)
    y_one = torch.cat([q1.view(N * T, -1), k1.view(N * T, -1), v1.view(N * T, -1)], dim=1)
    assert torch.equal(y_steps, y_one), "decode steps differ from one call"
    assert torch.equal(hist, st1), "history after the steps differs"
    check_conv(c, q1, k1, v1, st1, "decode vs oracle")


def test_conv_silu_prefill_layer():
    """The prefill layer's shape: 8192 tokens, C = 2*16*128 + 48*128 = 10240."""
    c = conv_case(10, 16, 48, 128, 128, [8192], 4, "bf16", True, True)
    q, k, v, st = gdr.conv_silu(c["x"], c["w"], 16, 48, 128, 128, bias=c["b"],
                                conv_state=c["s0"], cu_seqlens=c["cu"])
    torch.cuda.synchronize()
    check_conv(c, q, k, v, st, "prefill layer")


NORM_CASES = [
    # seed, total, H_v, d_v, dtype
    (11, 37, 3, 16, "bf16"),
    (12, 37, 3, 16, "f32"),
    (13, 100, 6, 128, "bf16"),
    (14, 100, 6, 128, "f32"),
    (15, 5, 48, 64, "bf16"),
    (16, 1, 1, 32, "f32"),
    (17, 0, 4, 128, "bf16"),
]


@pytest.mark.parametrize("case", NORM_CASES, ids=lambda c: f"seed{c[0]}_T{c[1]}_d{c[3]}_{c[4]}")
def test_gated_rmsnorm_parity(case):
    seed, total, H, d, dtype = case
    note(f"[norm] seed={seed} T={total} H={H} d={d} {dtype}")
    rng = np.random.default_rng(seed)
    o = to_dev(rng.standard_normal((total, H, d)), TDT[dtype])
    z = to_dev(rng.standard_normal((total, H, d)), TDT[dtype])
    w = to_dev(1.0 + 0.1 * rng.standard_normal(d), torch.float32)
    out = gdr.gated_rmsnorm(o, z, w, 1e-6)
    torch.cuda.synchronize()
    if total == 0:
        assert out.numel() == 0
        return
    ref = layer.gated_rmsnorm(o, z, w, 1e-6)
    err = np.max(np.abs(to_np(out) - ref)) / np.max(np.abs(ref))
    note(f"  norm max rel err {err:.2e} (bar {TOL[dtype]:g})")
    assert err <= TOL[dtype], err
    # in place over o gives the same bits
    o2 = o.clone()
    gdr.gated_rmsnorm(o2, z, w, 1e-6, out=o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, out)


def test_gated_rmsnorm_prefill_layer():
    rng = np.random.default_rng(18)
    shape = (8192, 48, 128)
    o = to_dev(rng.standard_normal(shape), torch.bfloat16)
    z = to_dev(rng.standard_normal(shape), torch.bfloat16)
    w = to_dev(1.0 + 0.1 * rng.standard_normal(128), torch.float32)
    out = gdr.gated_rmsnorm(o, z, w, 1e-6)
    torch.cuda.synchronize()
    ref = layer.gated_rmsnorm(o, z, w, 1e-6)
    err = np.max(np.abs(to_np(out) - ref)) / np.max(np.abs(ref))
    note(f"  norm prefill layer max rel err {err:.2e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_layer_end_to_end(dtype):
    """conv + SiLU -> the rule (chunked) -> gated RMSNorm through the library,
    against the same chain of fp64 oracles (the conv oracle's outputs feed the
    rule's oracle directly, unrounded).  The chain's error is dominated by the
    rule's bar, so that is the bar here: per sequence and head, max |x - y| /
    max |y| of the normalised output within 2e-2 (bf16) or 1e-4 (fp32)."""
    import oracle
    H_k, H_v, d = 2, 6, 128
    lens = [130, 1, 64]
    note(f"[layer e2e] {dtype} H={H_v}/{H_k} d={d} lens={lens}")
    c = conv_case(21, H_k, H_v, d, d, lens, 4, dtype, True, True)
    rng = np.random.default_rng(22)
    total, N = int(sum(lens)), len(lens)
    dt = TDT[dtype]
    a = to_dev(rng.standard_normal((total, H_v)), dt)
    b = to_dev(rng.standard_normal((total, H_v)), dt)
    A_log = to_dev(rng.uniform(0.0, np.log(16.0), H_v), torch.float32)
    dt_bias = to_dev(0.1 * rng.standard_normal(H_v), torch.float32)
    s0 = to_dev(0.01 * rng.standard_normal((N, H_v, d, d)), torch.float32)
    z = to_dev(rng.standard_normal((total, H_v, d)), dt)
    nw = to_dev(1.0 + 0.1 * rng.standard_normal(d), torch.float32)
    q, k, v, _ = gdr.conv_silu(c["x"], c["w"], H_k, H_v, d, d, bias=c["b"], conv_state=c["s0"],
                               cu_seqlens=c["cu"])
    o, S = gdr.chunked_fwd(q, k, v, a, b, A_log, dt_bias, s0, chunk=32, cu_seqlens=c["cu"])
    out = gdr.gated_rmsnorm(o, z, nw, 1e-6)
    torch.cuda.synchronize()
    cu = c["cu"].cpu().numpy()
    y_ref, _ = layer.short_conv_silu(c["x"], c["w"], c["b"], c["s0"], cu_seqlens=cu)
    qr = y_ref[:, :H_k * d].reshape(total, H_k, d)
    kr = y_ref[:, H_k * d:2 * H_k * d].reshape(total, H_k, d)
    vr = y_ref[:, 2 * H_k * d:].reshape(total, H_v, d)
    o_ref, S_ref = oracle.fwd(qr, kr, vr, a, b, A_log, dt_bias, initial_state=s0, cu_seqlens=cu)
    out_ref = layer.gated_rmsnorm(o_ref, z, nw, 1e-6)
    from tests import gpu_util as U
    eo, es = U.compare_full(out, S, out_ref, S_ref, [int(x) for x in cu], H_v)
    bar = 2e-2 if dtype == "bf16" else 1e-4
    note(f"  end to end: out {eo:.3e}, state {es:.3e} (bar {bar:g})")
    assert eo <= bar and es <= bar, (eo, es)
