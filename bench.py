"""Benchmark of the gated delta rule hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one chunked prefill of the layer-shaped workload (T = 8192 tokens,
48 value heads sharing 16 key heads, d_k = d_v = 128, chunk 32, bf16 q/k/v/a/b,
fp32 state): gates and normalisation, chunk prologue, forward substitution,
WY factors, the inter-chunk state scan and the outputs, all inside one kernel
launch.  ``value`` is prefill tokens/s over the K timed steps.  The decode leg
(256 sequences x 48 heads, fp32 state 256x48x128x128 carried in place over 64
single-token recurrent steps) is timed in the same run and reported under
"decode" as achieved HBM GB/s.  Inputs are seeded synthetic tensors drawn on
the GPU; they are resident in HBM before the timed region starts.

Prints ONE JSON line (rank 0, N = 1).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (T=8192, 48 heads) + decode HBM GB/s, % of roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 peak (dense matrix cores and vector ALUs alike)
PREFILL_KERNEL = "chunked_coop_kernel"  # the prefill launch with a workspace


def prefill_flops(T, H_k, H_v, d_k, d_v, C):
    """Algorithmic matrix flops of the chunked form (lower triangles counted
    half, no redundant recompute): per chunk of c tokens
    H_v [c(c+1)(d_k + 2 d_v) + 6 c d_k d_v] + H_k [2 c^2 d_k]."""
    total = 0
    t = 0
    while t < T:
        c = min(C, T - t)
        total += H_v * (c * (c + 1) * (d_k + 2 * d_v) + 6 * c * d_k * d_v) + H_k * 2 * c * c * d_k
        t += c
    return total


def varlen_flops(lengths, H_k, H_v, d_k, d_v, C):
    """prefill_flops summed over the sequences of a packed batch (chunks
    restart at every sequence start)."""
    return sum(prefill_flops(L, H_k, H_v, d_k, d_v, C) for L in lengths)


def prefill_bytes(T, N, H_k, H_v, d_k, d_v, elem=2, s0=False):
    """Algorithmic HBM bytes of one fused pass: q, k, v, a, b read once, o
    written once in the input dtype, the fp32 state written (and read if given)."""
    per_tok = (2 * H_k * d_k + H_v * d_v + 2 * H_v) * elem + H_v * d_v * elem
    return T * per_tok + N * H_v * d_k * d_v * 4 * (2 if s0 else 1)


def decode_bytes(N, H_k, H_v, d_k, d_v, elem=2):
    """Algorithmic HBM bytes of one decode step: the fp32 state read and
    written once, q, k, v, a, b read, o written, A_log and dt_bias read."""
    return (N * H_v * d_k * d_v * 4 * 2 + N * (2 * H_k * d_k + H_v * d_v) * elem
            + N * H_v * 2 * elem + N * H_v * d_v * elem + 8 * H_v)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 100 untimed prefill launches (about 22 ms): after 3 the GPU has not yet
    # reached its full clock and a launch measures about 12 % slower, after
    # 50 still about 5 %
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=64)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (a known-size "
                         "reference for hardware byte counters under a profiler)")
    ap.add_argument("--cpu-heads", type=int, default=48,
                    help="value heads of the prefill workload the oracle runs for cpu_baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the rule runs without collectives and this build "
              "has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_68_amd as gdr
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ------------------------------------------------------------ prefill
    w = synth.workload("prefill")
    inp = synth.make_inputs(w, 0, device=dev)
    T, N = w.total_tokens, 1
    o = torch.empty((T, w.H_v, w.d_v), dtype=w.torch_dtype, device=dev)
    S = torch.empty((N, w.H_v, w.d_k, w.d_v), dtype=torch.float32, device=dev)
    # the cooperative form's workspace, allocated (zero-filled) once and kept
    # across launches, as a caller would
    ws = gdr.chunked_workspace(w.H_k, w.H_v, w.d_k, w.d_v, w.dtype, N, chunk=w.chunk, device=dev)

    def prefill_step(workspace=ws):
        gdr.chunked_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"],
                        inp["dt_bias"], None, chunk=w.chunk, num_seqs=1, o=o, final_state=S,
                        workspace=workspace)

    # the same launch with every cache cold: a 1 GiB write before each one
    # evicts the L2s and the last-level cache
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cold_ms = []
    for i in range(5):
        flush.fill_(float(i))
        ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ce[0].record(stream)
        prefill_step()
        ce[1].record(stream)
        torch.cuda.synchronize(dev)
        cold_ms.append(ce[0].elapsed_time(ce[1]))
    del flush
    # the one-launch form (no workspace: every chain workgroup forms its own
    # triangular inverses), for comparison
    for _ in range(10):
        prefill_step(None)
    torch.cuda.synchronize(dev)
    fe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    fe[0].record(stream)
    for _ in range(10):
        prefill_step(None)
    fe[1].record(stream)
    torch.cuda.synchronize(dev)
    fused_ms = fe[0].elapsed_time(fe[1]) / 10
    mfma_probe = mfma_rate_probe(gdr, dev, stream)
    norm_line = norm_fusion_leg(gdr, dev, stream, w, inp, ws, max(5, min(args.steps, 20)))

    # ------------------------------------------------------------ decode
    wd = synth.workload("decode")
    dinp = synth.make_inputs(wd, 0, device=dev)
    state = dinp["initial_state"].clone()
    od = torch.empty((wd.num_seqs, wd.H_v, wd.d_v), dtype=wd.torch_dtype, device=dev)
    nsteps = min(args.decode_steps, wd.steps)

    def decode_step(s):
        gdr.recurrent_fwd(dinp["q"][s], dinp["k"][s], dinp["v"][s], dinp["a"][s], dinp["b"][s],
                          dinp["A_log"], dinp["dt_bias"], state, num_seqs=wd.num_seqs, o=od,
                          inplace=True)

    for s in range(2):  # warm-up, then restore the initial state
        decode_step(s)
    state.copy_(dinp["initial_state"])
    torch.cuda.synchronize(dev)
    # one pair of events around the back-to-back steps, as for the prefill
    dev_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    dev_ev[0].record(stream)
    for s in range(nsteps):
        decode_step(s)
    dev_ev[1].record(stream)
    torch.cuda.synchronize(dev)
    dmean_ms = dev_ev[0].elapsed_time(dev_ev[1]) / nsteps
    # the same steps again with a pair of events around each one (from the
    # initial state), for the per-step median and spread
    state.copy_(dinp["initial_state"])
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(nsteps)]
    for s in range(nsteps):
        step_ev[s][0].record(stream)
        decode_step(s)
        step_ev[s][1].record(stream)
    torch.cuda.synchronize(dev)
    step_ms = sorted(a.elapsed_time(b) for a, b in step_ev)
    dmedian_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else \
        0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])
    dbytes = decode_bytes(wd.num_seqs, wd.H_k, wd.H_v, wd.d_k, wd.d_v, 2)
    dgbs = dbytes / (dmean_ms / 1e3) / 1e9

    # ------------------------------------------------------------ varlen prefill
    wv = synth.workload("varlen", seed=0)
    vinp = synth.make_inputs(wv, 0, device=dev)
    Tv, Nv = wv.total_tokens, wv.num_seqs
    ov = torch.empty((Tv, wv.H_v, wv.d_v), dtype=wv.torch_dtype, device=dev)
    Sv = torch.empty((Nv, wv.H_v, wv.d_k, wv.d_v), dtype=torch.float32, device=dev)

    def varlen_step():
        gdr.chunked_fwd(vinp["q"], vinp["k"], vinp["v"], vinp["a"], vinp["b"], vinp["A_log"],
                        vinp["dt_bias"], vinp["initial_state"], chunk=wv.chunk,
                        cu_seqlens=vinp["cu_seqlens"], o=ov, final_state=Sv)

    varlen_step()
    torch.cuda.synchronize(dev)
    vsteps = max(1, min(args.steps, 5))
    ve = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ve[0].record(stream)
    for _ in range(vsteps):
        varlen_step()
    ve[1].record(stream)
    torch.cuda.synchronize(dev)
    vms = ve[0].elapsed_time(ve[1]) / vsteps
    vflops = varlen_flops(wv.seq_lengths, wv.H_k, wv.H_v, wv.d_k, wv.d_v, wv.chunk)
    vbytes = prefill_bytes(Tv, Nv, wv.H_k, wv.H_v, wv.d_k, wv.d_v, 2, s0=True)
    del vinp, ov, Sv

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        torch.cuda.synchronize(dev)
        del src, dst

    # ------------------------------------ the layer's steps either side of the rule
    layer_line = layer_legs(gdr, dev, stream, max(1, min(args.steps, 10)))
    split_line = split_legs(gdr, dev, stream, max(1, min(args.steps, 5)))
    ssd_line = ssd_legs(gdr, dev, stream, max(1, min(args.steps, 10)))
    kda_line = kda_legs(gdr, dev, stream, max(1, min(args.steps, 5)))

    # ------------------------------------------------ the timed prefill launches
    # Timed after every other GPU leg above, so that the K launches run at the
    # clocks the GPU holds under sustained work: right after start-up or an
    # idle second, with 5 warm-up launches, a launch measures 190-210 us
    # against 166-168 us once the GPU has been busy for a while (the power
    # management raises the clocks over tens of milliseconds of load).  The
    # warm-up is still exactly W launches of this workload.
    for _ in range(args.warmup):
        prefill_step()
    torch.cuda.synchronize(dev)
    # one pair of events around the K launches: an event after every launch
    # would add about 4 us of gap per launch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        prefill_step()
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    total_ms = ev[0].elapsed_time(ev[1])
    per_launch_ms = [total_ms / args.steps]  # the average launch, back to back
    ms_per_step = total_ms / args.steps
    tokens_per_s = T * args.steps / (total_ms / 1e3)
    flops = prefill_flops(T, w.H_k, w.H_v, w.d_k, w.d_v, w.chunk)
    pbytes = prefill_bytes(T, N, w.H_k, w.H_v, w.d_k, w.d_v, 2, s0=False)
    avg_s = (sum(per_launch_ms) / len(per_launch_ms)) / 1e3
    achieved_tf = flops / avg_s / 1e12
    ws_error = gdr.workspace_error(ws) if ws is not None else 0
    if ws_error:
        raise RuntimeError(f"cooperative prefill: workspace error word {ws_error:#x}")


    # ------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, T, args.cpu_heads)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": gdr_chunked_dtype(gdr, w),
        "data": "synthetic",
        "config": {"workload": "prefill layer: 1 sequence x 8192 tokens, 48 value heads sharing "
                               "16 key heads, d_k=d_v=128, chunk 32, bf16 inputs, fp32 state",
                   "global_batch": 1, "seq_len": T, "H_v": w.H_v, "H_k": w.H_k, "d": w.d_k,
                   "chunk": w.chunk},
        "roofline": {"bound": "mfma", "achieved": achieved_tf, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved_tf / PEAK_BF16_TFLOPS,
                     "traffic": profiled_traffic(PREFILL_KERNEL),
                     "kernel": PREFILL_KERNEL if ws is not None else "chunked_mfma_kernel",
                     "flop_per_launch": flops,
                     "avg_launch_ms": avg_s * 1e3,
                     "cold_cache_launch_ms": sum(cold_ms) / len(cold_ms),
                     "one_launch_form_ms": fused_ms,
                     "measured_mfma_peak": mfma_probe,
                     "mfma_busy_profiled": {
                         "value": profiled_traffic(PREFILL_KERNEL, "mfma_busy_frac"),
                         "source": "profiles/traffic.json: hardware counters of a profiled run "
                                   "of this kernel's sources, not of this run"},
                     "hbm_view": {"bytes_per_launch": pbytes,
                                  "achieved_GBs": pbytes / avg_s / 1e9,
                                  "frac": pbytes / avg_s / 1e9 / PEAK_HBM_GBS}},
        "decode": {"workload": "256 sequences x 48 value heads (16 key heads), d_k=d_v=128, "
                               "fp32 state in place, bf16 inputs, single-token steps",
                   "steps": nsteps, "mean_step_ms": dmean_ms,
                   "per_step_events_ms": {"median": dmedian_ms, "min": step_ms[0],
                                          "max": step_ms[-1],
                                          "note": "a second pass of the same steps with a pair "
                                                  "of events around each step"},
                   "tokens_per_s": wd.num_seqs / (dmean_ms / 1e3),
                   "roofline": {"bound": "hbm", "achieved": dgbs, "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": dgbs / PEAK_HBM_GBS,
                                "traffic": profiled_traffic("recurrent_kernel"),
                                "bytes_per_launch": dbytes}},
        "varlen": {"workload": "8 packed sequences, lengths %s (seed 0), 48 value heads sharing "
                               "16 key heads, d_k=d_v=128, chunk 32, bf16, carried fp32 state"
                               % wv.seq_lengths,
                   "tokens": Tv, "steps": vsteps, "ms_per_step": vms,
                   "tokens_per_s": Tv / (vms / 1e3),
                   "roofline": {"bound": "mfma", "achieved": vflops / (vms / 1e3) / 1e12,
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": vflops / (vms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                                "flop_per_launch": vflops,
                                "hbm_GBs": vbytes / (vms / 1e3) / 1e9}},
        "layer": dict(layer_line, rule_then_gated_rmsnorm=norm_line),
        "split": split_line,
        "ssd": ssd_line,
        "kda": kda_line,
        "wall_s_prefill_timed": wall,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line))


def layer_legs(gdr, dev, stream, steps):
    """gdr_conv_silu and gdr_gated_rmsnorm at the prefill layer's shapes
    (8192 tokens; C = 2*16*128 + 48*128 = 10240 conv channels; o, z
    [8192, 48, 128]), bf16, synthetic N(0, 1) inputs resident in HBM.  Both
    are bound by HBM; the bytes are the algorithmic ones (every input read
    once, every output written once)."""
    import torch
    T, H_k, H_v, d = 8192, 16, 48, 128
    C, W = 2 * H_k * d + H_v * d, 4
    g = torch.Generator(device=dev).manual_seed(0)
    x = torch.randn((T, C), generator=g, device=dev).to(torch.bfloat16)
    w = torch.randn((C, W), generator=g, device=dev) / 2.0
    b = 0.1 * torch.randn((C,), generator=g, device=dev)
    hist = torch.randn((1, C, W - 1), generator=g, device=dev).to(torch.bfloat16)
    hist_out = torch.empty_like(hist)
    cu = torch.tensor([0, T], dtype=torch.int32, device=dev)
    o = torch.randn((T, H_v, d), generator=g, device=dev).to(torch.bfloat16)
    z = torch.randn((T, H_v, d), generator=g, device=dev).to(torch.bfloat16)
    nw = 1.0 + 0.1 * torch.randn((d,), generator=g, device=dev)
    out = torch.empty_like(o)

    def timed(fn):
        fn()
        torch.cuda.synchronize(dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(steps):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize(dev)
        return e[0].elapsed_time(e[1]) / steps

    conv_ms = timed(lambda: gdr.conv_silu(x, w, H_k, H_v, d, d, bias=b, conv_state=hist,
                                          cu_seqlens=cu, final_conv_state=hist_out))
    norm_ms = timed(lambda: gdr.gated_rmsnorm(o, z, nw, 1e-6, out=out))
    conv_bytes = 2 * T * C * 2 + C * W * 4 + C * 4 + 2 * C * (W - 1) * 2
    norm_bytes = 3 * T * H_v * d * 2 + d * 4

    def leg(workload, ms, nbytes, kernel):
        gbs = nbytes / (ms / 1e3) / 1e9
        return {"workload": workload, "steps": steps, "ms_per_launch": ms,
                "tokens_per_s": T / (ms / 1e3),
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                             "traffic": profiled_traffic(kernel), "bytes_per_launch": nbytes}}

    res = {
        "conv_silu": leg("short causal conv (width 4, bias, carried history) + SiLU over the "
                         "q|k|v channels of the in_proj output: 8192 tokens x 10240 channels, "
                         "bf16, split into q, k, v", conv_ms, conv_bytes, "conv_silu_kernel"),
        "gated_rmsnorm": leg("gated RMSNorm of o: 8192 tokens x 48 value heads x 128, bf16",
                             norm_ms, norm_bytes, "gated_rmsnorm_kernel"),
    }
    del x, w, b, hist, hist_out, o, z, out
    return res


def norm_fusion_leg(gdr, dev, stream, w, inp, ws, steps):
    """The rule followed by the gated RMSNorm of its output on the prefill
    layer (gdr_chunked_fwd_gated_rmsnorm: the cooperative launch, then the
    norm in place), back to back; z is N(0, 1), the weight 1 + 0.1 N(0, 1)."""
    import torch
    T = w.total_tokens
    g = torch.Generator(device=dev).manual_seed(1)
    z = torch.randn((T, w.H_v, w.d_v), generator=g, device=dev).to(w.torch_dtype)
    nw = 1.0 + 0.1 * torch.randn((w.d_v,), generator=g, device=dev)
    out = torch.empty((T, w.H_v, w.d_v), dtype=w.torch_dtype, device=dev)
    S = torch.empty((1, w.H_v, w.d_k, w.d_v), dtype=torch.float32, device=dev)

    def layer_tail():
        gdr.chunked_fwd_gated_rmsnorm(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                      inp["A_log"], inp["dt_bias"], z, nw, None, norm_eps=1e-6,
                                      chunk=w.chunk, num_seqs=1, out=out, final_state=S,
                                      workspace=ws)

    for _ in range(20):
        layer_tail()
    torch.cuda.synchronize(dev)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    e[0].record(stream)
    for _ in range(steps):
        layer_tail()
    e[1].record(stream)
    torch.cuda.synchronize(dev)
    ms = e[0].elapsed_time(e[1]) / steps
    if ws is not None and gdr.workspace_error(ws):
        raise RuntimeError("rule + norm: workspace error word set")
    del z, out, S
    return {"workload": "prefill layer (8192 tokens, 48 value heads, d 128, bf16): the rule and "
                        "the gated RMSNorm of its output, two launches per call",
            "steps": steps, "ms_per_call": ms, "tokens_per_s": T / (ms / 1e3)}


def split_legs(gdr, dev, stream, steps):
    """The segmented chunked form (two-level scan) against the direct form on
    long single-head prefill, where the direct form has one chain of chunks
    per (head, 32 columns): the one-head workload (4096 tokens, d = 128,
    fp32) and one bf16 head of 65536 tokens.  Work is counted as the direct
    form's algorithmic matrix flops; the split form does about three times
    that arithmetic."""
    import torch
    import synth

    def timed(fn):
        fn()
        torch.cuda.synchronize(dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(steps):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize(dev)
        return e[0].elapsed_time(e[1]) / steps

    res = {}
    cases = [("one_head", synth.workload("one_head"), 256),
             ("single_head_65536_bf16", synth.custom(1, 1, 128, 128, "bf16", seq_len=65536,
                                                     num_seqs=1, chunk=32), 2048)]
    for name, w, seg in cases:
        inp = synth.make_inputs(w, 0, device=dev)
        args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                inp["initial_state"])
        T = w.total_tokens
        direct_ms = timed(lambda: gdr.chunked_fwd(*args, chunk=w.chunk, num_seqs=w.num_seqs))
        split_ms = timed(lambda: gdr.chunked_fwd_split(*args, segment_len=seg, chunk=w.chunk,
                                                       num_seqs=w.num_seqs))
        flops = prefill_flops(T, w.H_k, w.H_v, w.d_k, w.d_v, w.chunk)
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        tf = flops / (split_ms / 1e3) / 1e12
        res[name] = {"workload": f"1 sequence x {T} tokens, {w.H_v} head, d_k=d_v={w.d_k}, "
                                 f"{w.dtype}, chunk {w.chunk}, {T // seg} segments of {seg}",
                     "direct_ms": direct_ms, "split_ms": split_ms, "speedup": direct_ms / split_ms,
                     "tokens_per_s": T / (split_ms / 1e3),
                     "roofline": {"bound": "mfma", "achieved": tf,
                                  "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
                                  "flop_per_launch": flops}}
        del inp, args
    # one GPU's share of the prefill layer sharded 8 ways by key-head groups
    # (6 value heads sharing 2 key heads, 8192 tokens): the direct forms fill
    # an eighth of the compute units, the segmented form all of them
    w = synth.custom(2, 6, 128, 128, "bf16", seq_len=8192, num_seqs=1, chunk=32)
    inp = synth.make_inputs(w, 0, device=dev)
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])
    T = w.total_tokens
    ws = gdr.chunked_workspace(w.H_k, w.H_v, w.d_k, w.d_v, w.dtype, 1, chunk=32, device=dev)
    coop_ms = timed(lambda: gdr.chunked_fwd(*args, chunk=32, num_seqs=1, workspace=ws))
    direct_ms = timed(lambda: gdr.chunked_fwd(*args, chunk=32, num_seqs=1))
    by_seg = {seg: timed(lambda: gdr.chunked_fwd_split(*args, segment_len=seg, chunk=32,
                                                       num_seqs=1))
              for seg in (512, 1024, 2048)}
    best = min(by_seg, key=by_seg.get)
    split_ms = by_seg[best]
    flops = prefill_flops(T, w.H_k, w.H_v, w.d_k, w.d_v, w.chunk)
    tf = flops / (split_ms / 1e3) / 1e12
    res["shard_8way_6v_2k_8192_bf16"] = {
        "workload": f"one GPU's share of the prefill layer sharded 8 ways by key-head groups: "
                    f"1 sequence x {T} tokens, 6 value heads sharing 2 key heads, d_k=d_v=128, "
                    f"bf16, chunk 32",
        "direct_ms": coop_ms, "one_launch_ms": direct_ms,
        "split_ms_by_segment": {str(k): v for k, v in by_seg.items()},
        "split_ms": split_ms, "segment_len": best, "speedup": coop_ms / split_ms,
        "tokens_per_s": T / (split_ms / 1e3),
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "flop_per_launch": flops}}
    del inp, args, ws
    # the per-channel-decay variant on one long head (its chunk step is slower
    # than the rule's, so the chain of chunks weighs more)
    w = synth.custom(1, 1, 128, 128, "bf16", seq_len=16384, num_seqs=1, chunk=32)
    seg = 1024
    inp = synth.kda_inputs(w, 0, device=dev)
    args = (inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
            inp["initial_state"])
    T = w.total_tokens
    direct_ms = timed(lambda: gdr.kda_chunked_fwd(*args, chunk=32, num_seqs=1))
    split_ms = timed(lambda: gdr.kda_chunked_fwd_split(*args, segment_len=seg, chunk=32,
                                                       num_seqs=1))
    flops = kda_prefill_flops(T, 1, 1, 128, 128, 32)
    tf = flops / (split_ms / 1e3) / 1e12
    res["kda_single_head_16384_bf16"] = {
        "workload": f"KDA, 1 sequence x {T} tokens, 1 head, d_k=d_v=128, bf16, chunk 32, "
                    f"{T // seg} segments of {seg}",
        "direct_ms": direct_ms, "split_ms": split_ms, "speedup": direct_ms / split_ms,
        "tokens_per_s": T / (split_ms / 1e3),
        "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "flop_per_launch": flops}}
    del inp, args
    return res


def ssd_flops(T, G, H, N, P, C):
    """Algorithmic matrix flops of the chunked SSD scan (lower triangles
    counted half): per chunk of c tokens G c(c+1) N for the C B^T products of
    each group and H [c(c+1) P + 4 c N P] per head (the masked outputs, C S
    and the state update B^T Delta)."""
    total = 0
    t = 0
    while t < T:
        c = min(C, T - t)
        total += G * c * (c + 1) * N + H * (c * (c + 1) * P + 4 * c * N * P)
        t += c
    return total


def ssd_bytes(T, S, G, H, N, P, elem=2, s0=False, gate=False):
    """Algorithmic HBM bytes of one SSD pass: x, delta, B, C (and z) read
    once, y written once in the input dtype, the fp32 state written (and
    read when given)."""
    per_tok = (H * P + H + 2 * G * N + H * P + (H * P if gate else 0)) * elem
    return T * per_tok + S * H * N * P * 4 * (2 if s0 else 1) + 4 * H


def ssd_legs(gdr, dev, stream, steps):
    """The Mamba-2 SSD recurrence on the same chunk scan: prefill of 8192
    tokens with 128 heads of P = 64 in 8 groups of B and C, state N = 128,
    chunk 32, bf16 (the chunked kernel, and the SiLU gate as its own launch),
    and decode of 256 sequences x 128 heads with the fp32 state carried in
    place (the recurrent kernel, 64 single-token steps).  Inputs from
    synth.ssd_inputs, resident in HBM."""
    import torch
    import synth

    def timed(fn, n):
        fn()
        torch.cuda.synchronize(dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(n):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize(dev)
        return e[0].elapsed_time(e[1]) / n

    T, G, H, N, P = 8192, 8, 128, 128, 64
    inp = synth.ssd_inputs(G, H, N, P, "bf16", seq_len=T, num_seqs=1, seed=0, device=dev,
                           init_state=False, gate=True)
    y = torch.empty((T, H, P), dtype=torch.bfloat16, device=dev)
    S = torch.empty((1, H, N, P), dtype=torch.float32, device=dev)
    args = (inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], None)
    scan_ms = timed(lambda: gdr.ssd_chunked_fwd(*args, chunk=32, num_seqs=1, y=y, final_state=S),
                    steps)
    gated_ms = timed(lambda: gdr.ssd_chunked_fwd(*args, z=inp["z"], chunk=32, num_seqs=1, y=y,
                                                 final_state=S), steps)
    flops = ssd_flops(T, G, H, N, P, 32)
    pbytes = ssd_bytes(T, 1, G, H, N, P)
    del inp, args, y, S

    Nd, steps_d = 256, 64
    dinp = synth.ssd_inputs(G, H, N, P, "bf16", seq_len=steps_d, num_seqs=Nd, seed=1,
                            device=dev, init_state=True)
    # step-major copies: step s of every sequence is one contiguous batch
    xs = dinp["x"].view(Nd, steps_d, H, P).transpose(0, 1).contiguous()
    ds = dinp["delta"].view(Nd, steps_d, H).transpose(0, 1).contiguous()
    Bs = dinp["B"].view(Nd, steps_d, G, N).transpose(0, 1).contiguous()
    Cs = dinp["C"].view(Nd, steps_d, G, N).transpose(0, 1).contiguous()
    state = dinp["initial_state"].clone()
    yd = torch.empty((Nd, H, P), dtype=torch.bfloat16, device=dev)
    box = [0]

    def dstep():
        s = box[0] % steps_d
        box[0] += 1
        gdr.ssd_recurrent_fwd(xs[s], ds[s], dinp["A"], Bs[s], Cs[s], state, num_seqs=Nd, y=yd,
                              inplace=True)

    dec_ms = timed(dstep, steps_d)
    dbytes = Nd * H * N * P * 4 * 2 + Nd * (2 * H * P + H + 2 * G * N) * 2 + 4 * H
    del dinp, xs, ds, Bs, Cs, state, yd
    tf = flops / (scan_ms / 1e3) / 1e12
    gbs = pbytes / (scan_ms / 1e3) / 1e9
    dgbs = dbytes / (dec_ms / 1e3) / 1e9
    return {
        "prefill": {"workload": f"1 sequence x {T} tokens, {H} heads of P={P} in {G} groups "
                                f"of B and C, N={N}, chunk 32, bf16 inputs, fp32 state",
                    "steps": steps, "ms_per_launch": scan_ms, "tokens_per_s": T / (scan_ms / 1e3),
                    "with_gate_ms": gated_ms,
                    "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                 "bytes_per_launch": pbytes,
                                 "mfma_view": {"flop_per_launch": flops, "achieved_TFs": tf,
                                               "frac": tf / PEAK_BF16_TFLOPS}}},
        "decode": {"workload": f"{Nd} sequences x {H} heads of P={P} ({G} groups), N={N}, "
                               "fp32 state in place, bf16 inputs, single-token steps",
                   "steps": steps_d, "mean_step_ms": dec_ms, "tokens_per_s": Nd / (dec_ms / 1e3),
                   "roofline": {"bound": "hbm", "achieved": dgbs, "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": dgbs / PEAK_HBM_GBS,
                                "bytes_per_launch": dbytes}},
    }


def kda_prefill_flops(T, H_k, H_v, d_k, d_v, C):
    """Algorithmic flops of the chunked KDA form: the rule's contractions
    (prefill_flops) plus, for the channel-weighted Gram matrices, one more
    multiply per channel of every (row, earlier row) pair, per value head:
    H_v c(c+1)/2 d_k x 2 (the A and P sums share the weight).  The
    exponentials of the weights are not counted."""
    extra = 0
    t = 0
    while t < T:
        c = min(C, T - t)
        extra += H_v * c * (c + 1) // 2 * d_k * 2
        t += c
    return prefill_flops(T, H_k, H_v, d_k, d_v, C) + extra


def kda_legs(gdr, dev, stream, steps):
    """The per-channel-decay variant (KDA) at the rule's shapes: decode of
    256 sequences x 48 value heads (16 key heads), d = 128, fp32 state in
    place, 64 single-token steps (recurrent kernel, HBM-bound); the prefill
    layer (8192 tokens, chunk 32, bf16) on the two-launch chunked form, with
    the one-launch form timed beside it; and the varlen workload (8 packed
    sequences, carried state) on the two-launch form.  Inputs from
    synth.kda_inputs, resident in HBM."""
    import torch
    import synth

    def timed(fn, n):
        fn()
        torch.cuda.synchronize(dev)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(stream)
        for _ in range(n):
            fn()
        e[1].record(stream)
        torch.cuda.synchronize(dev)
        return e[0].elapsed_time(e[1]) / n

    wd = synth.workload("decode")
    d = synth.kda_inputs(wd, 0, device=dev)
    state = d["initial_state"].clone()
    od = torch.empty((wd.num_seqs, wd.H_v, wd.d_v), dtype=wd.torch_dtype, device=dev)
    box = [0]

    def dstep():
        s = box[0] % wd.steps
        box[0] += 1
        gdr.kda_recurrent_fwd(d["q"][s], d["k"][s], d["v"][s], d["a"][s], d["b"][s], d["A_log"],
                              d["dt_bias"], state, num_seqs=wd.num_seqs, o=od, inplace=True)

    dec_ms = timed(dstep, wd.steps)
    N, H_k, H_v, dk, dv = wd.num_seqs, wd.H_k, wd.H_v, wd.d_k, wd.d_v
    dbytes = (N * H_v * dk * dv * 4 * 2 + N * (2 * H_k * dk + H_v * dv) * 2
              + N * H_v * (dk + 1) * 2 + N * H_v * dv * 2 + 4 * H_v * (dk + 1))
    del d, state, od

    w = synth.workload("prefill")
    inp = synth.kda_inputs(w, 0, device=dev)
    o = torch.empty((w.total_tokens, w.H_v, w.d_v), dtype=w.torch_dtype, device=dev)
    S = torch.empty((1, w.H_v, w.d_k, w.d_v), dtype=torch.float32, device=dev)

    def pre(fused):
        return lambda: gdr.kda_chunked_fwd(inp["q"], inp["k"], inp["v"], inp["a"], inp["b"],
                                           inp["A_log"], inp["dt_bias"], None, chunk=32,
                                           num_seqs=1, o=o, final_state=S, fused=fused)

    pre_ms = timed(pre(False), steps)  # prep + chains (the library's workspace form)
    one_ms = timed(pre(True), steps)   # the one-launch form, for comparison
    T = w.total_tokens
    flops = kda_prefill_flops(T, w.H_k, w.H_v, w.d_k, w.d_v, 32)
    del inp, o, S

    # the varlen workload (8 packed sequences, carried state) on the same form
    wv = synth.workload("varlen")
    vin = synth.kda_inputs(wv, 0, device=dev)
    vo = torch.empty((wv.total_tokens, wv.H_v, wv.d_v), dtype=wv.torch_dtype, device=dev)
    vS = torch.empty_like(vin["initial_state"])
    var_ms = timed(lambda: gdr.kda_chunked_fwd(vin["q"], vin["k"], vin["v"], vin["a"], vin["b"],
                                               vin["A_log"], vin["dt_bias"], vin["initial_state"],
                                               chunk=32, cu_seqlens=vin["cu_seqlens"], o=vo,
                                               final_state=vS), steps)
    var_flops = sum(kda_prefill_flops(L, wv.H_k, wv.H_v, wv.d_k, wv.d_v, 32) for L in wv.seq_lengths)
    var_tokens = wv.total_tokens
    var_lens = list(wv.seq_lengths)
    del vin, vo, vS
    dgbs = dbytes / (dec_ms / 1e3) / 1e9
    tf = flops / (pre_ms / 1e3) / 1e12
    return {
        "decode": {"workload": "256 sequences x 48 value heads (16 key heads), d_k=d_v=128, "
                               "per-channel gates a [256, 48, 128], fp32 state in place, bf16 "
                               "inputs, single-token steps",
                   "steps": wd.steps, "mean_step_ms": dec_ms, "tokens_per_s": N / (dec_ms / 1e3),
                   "roofline": {"bound": "hbm", "achieved": dgbs, "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": dgbs / PEAK_HBM_GBS,
                                "bytes_per_launch": dbytes}},
        "prefill": {"workload": "prefill layer: 1 sequence x 8192 tokens, 48 value heads sharing "
                                "16 key heads, d_k=d_v=128, chunk 32, bf16 inputs, fp32 state; "
                                "two launches (per-chunk prep over the batch, then the chains)",
                    "steps": steps, "ms_per_launch": pre_ms, "tokens_per_s": T / (pre_ms / 1e3),
                    "one_launch_ms": one_ms,
                    "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                                 "flop_per_launch": flops,
                                 "mfma_busy": {"prep": profiled_traffic("kda_prep_kernel", "mfma_busy_frac"),
                                               "chain": profiled_traffic("kda_chain_kernel", "mfma_busy_frac")}}},
        "varlen": {"workload": f"{len(var_lens)} packed sequences, lengths {var_lens} (seed 0), "
                               "48 value heads sharing 16 key heads, d_k=d_v=128, per-channel "
                               "gates, chunk 32, bf16, carried fp32 state; two launches",
                   "tokens": var_tokens, "steps": steps, "ms_per_launch": var_ms,
                   "tokens_per_s": var_tokens / (var_ms / 1e3),
                   "roofline": {"bound": "mfma", "achieved": var_flops / (var_ms / 1e3) / 1e12,
                                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                "frac": var_flops / (var_ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                                "flop_per_launch": var_flops}},
    }


def mfma_rate_probe(gdr, dev, stream):
    """The dense bf16 matrix-core rate this GPU sustains on back-to-back
    independent v_mfma_f32_16x16x32_bf16 (libgdr_probe.so), in TFLOP/s, beside
    the published peak."""
    import ctypes
    import torch
    path = os.path.join(os.path.dirname(gdr.library_path()), "libgdr_probe.so")
    if not os.path.exists(path):
        return None
    probe = ctypes.CDLL(path)
    probe.gdr_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    probe.gdr_probe_mfma_bf16.restype = ctypes.c_int
    probe.gdr_probe_mfma_bf16_flop.argtypes = [ctypes.c_int, ctypes.c_int]
    probe.gdr_probe_mfma_bf16_flop.restype = ctypes.c_double
    blocks, iters, reps = 1024, 2000, 5  # four workgroups of four waves per CU
    out = torch.empty(blocks, dtype=torch.float32, device=dev)
    h = ctypes.c_void_p(stream.cuda_stream)
    for _ in range(2):
        if probe.gdr_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), h) != 0:
            return None
    torch.cuda.synchronize(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        probe.gdr_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), h)
    ev[1].record(stream)
    torch.cuda.synchronize(dev)
    s = ev[0].elapsed_time(ev[1]) / reps / 1e3
    tf = probe.gdr_probe_mfma_bf16_flop(blocks, iters) / s / 1e12
    return {"value": tf, "unit": "TFLOP/s", "frac_of_published": tf / PEAK_BF16_TFLOPS,
            "kernel": "independent v_mfma_f32_16x16x32_bf16, 8 accumulators a wave, "
                      "16 waves a CU"}


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, inp, T, cpu_heads):
    """The fp64 oracle timed on this host: the prefill layer (the bench
    workload) on `threads` threads, plus every configuration's oracle time
    (bounded samples, scaled) and 1-thread times for configurations 1-3."""
    import oracle
    import synth
    # one GPU's share of the host's cores: 16 a GPU on an eight-GPU host,
    # whatever count the process sees
    threads = min(16, os.cpu_count() or 1)

    def run(wl, x, pairs=None, n_threads=threads, dense=None):
        src = dense if dense is not None else x
        q, k, v, a, b = (oracle.f64(src[n]) for n in ("q", "k", "v", "a", "b"))
        A, D = oracle.f64(x["A_log"]), oracle.f64(x["dt_bias"])
        s0 = None if x["initial_state"] is None else oracle.f64(x["initial_state"])
        cu = x["cu_host"] if x["cu_seqlens"] is not None else None
        N = len(x["cu_host"]) - 1
        t0 = time.perf_counter()
        if dense is not None:
            oracle.fwd(q, k, v, a, b, A, D, initial_state=s0, num_seqs=N, pairs=pairs,
                       n_threads=n_threads)
        else:
            oracle.fwd(q, k, v, a, b, A, D, initial_state=s0, cu_seqlens=cu,
                       num_seqs=None if cu else N, pairs=pairs, n_threads=n_threads)
        return time.perf_counter() - t0

    heads = max(1, min(cpu_heads, w.H_v))
    pairs = [(0, h) for h in range(heads)]
    c_s = run(w, inp, pairs)
    layer_s = c_s * w.H_v / heads
    table = []

    def entry(name, wl, x, n_threads, frac_pairs=1.0, dense=None, tokens=None):
        N = len(x["cu_host"]) - 1
        all_pairs = [(n, h) for n in range(N) for h in range(wl.H_v)]
        npairs = max(1, int(round(len(all_pairs) * frac_pairs)))
        sel = all_pairs[:: max(1, len(all_pairs) // npairs)][:npairs]
        sec = run(wl, x, sel if npairs < len(all_pairs) else None, n_threads, dense)
        scale = len(all_pairs) / len(sel)
        toks = tokens if tokens is not None else x["cu_host"][-1]
        table.append({"config": name, "threads": n_threads, "pairs_run": len(sel),
                      "pairs": len(all_pairs), "seconds_run": sec,
                      "seconds_full": sec * scale, "tokens_per_s_full": toks / (sec * scale)})

    for cfg, name in ((1, "tiny"), (2, "one_head")):
        wl = synth.workload(name)
        x = synth.make_inputs(wl, 0)
        for th in (1, threads):
            entry(cfg, wl, x, th)
    entry(3, w, inp, threads)
    entry(3, w, inp, 1, frac_pairs=4 / w.H_v)
    wd = synth.workload("decode")
    xd = synth.make_inputs(wd, 0)
    entry(4, wd, xd, threads, dense=xd["dense"], tokens=wd.num_seqs * wd.steps)
    wv = synth.workload("varlen", seed=0)
    xv = synth.make_inputs(wv, 0)
    entry(5, wv, xv, threads, frac_pairs=0.25)
    return {"value": T / layer_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": f"fp64 sequential oracle (plain C, OpenMP over (sequence, head) pairs) "
                      f"on {heads} of {w.H_v} value heads x {T} tokens of the prefill "
                      f"workload ({c_s:.2f} s wall on {threads} threads), scaled to the "
                      f"{w.H_v}-head layer",
            "per_config": table}


def profiled_traffic(kernel, field="traffic_bytes"):
    """A hardware-counter figure of `kernel` from the committed profile: by
    default its HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, scaled by a
    plain copy of known size); `mfma_busy_frac` is the share of SIMD-cycles
    its matrix pipes were busy.  None when that kernel's sources changed
    after the counters were taken (the recorded sha256 no longer matches)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))["kernels"][kernel]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        value = rec[field]
    except (OSError, KeyError, ValueError):
        return None
    return value if h.hexdigest() == rec["sha256"] else None


def gdr_chunked_dtype(gdr, w):
    """Arithmetic type of the chunked kernel the library picks for ``w``:
    bf16 matrix operands (fp32 accumulation and state) or fp32 throughout."""
    path = gdr.chunked_path(w.H_k, w.H_v, w.d_k, w.d_v, w.dtype, w.chunk)
    return "bf16" if path == "matrix_bf16" else "f32"


if __name__ == "__main__":
    main()
