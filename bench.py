"""Benchmark of the SDM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_context]

The default workload is the largest layer that fits one GPU: the
long-context prefill (B = 1, H = 16, T = 1,048,576 tokens, N = 2^20 slots
per head, d_v = 128, k' = W = R = 32).  One step is one pass of the whole
hot path over one batch of synthetic input of the named layer: copy the
learned M0 into every sequence (on a second stream, concurrently with the
addressing, which does not touch the state), PKM addressing of all B*T*H
token-heads (write and read), the prefill scan over the T tokens, and one
decode step (a new token for every sequence).  The "decode" workload
instead times 1024 consecutive decode steps of 32 sequences.

Prints one JSON line: whole-step tokens/s, the roofline of the dominant
kernel (the scan; HBM-bound) measured with HIP events on the launch stream,
a per-kernel breakdown, and the CPU oracle timed on the host as a baseline.
After the timed region it also times the steps either side of the path (the
gates, and the read-out's norm and output gate, and the backward of both)
on the same layer, reported under "layer_edges" and not counted in the step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure

PREFILL_WORKLOADS = ("tiny", "small", "prefill_1p4b", "long_context")
KERNEL_SOURCES = ("sdm_scan.hip", "sdm_scan_lanes.hip", "scan_prep.hip", "scan_lanes.h", "lanes_common.h",
                  "device_common.h", "kernels.h")


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="long_context",
                   choices=list(PREFILL_WORKLOADS) + ["decode", "gdn_1p4b", "train_small", "train_1p4b",
                                                      "row_traffic"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="minimum CPU time spent on the oracle baseline (0 disables it)")
    p.add_argument("--decode-steps", type=int, default=1024, help="decode steps per step (decode workload)")
    p.add_argument("--chunks", type=int, default=None,
                   help="prefill pipelined over this many equal chunks of tokens (the addressing of chunk c + 1 "
                        "overlapping the scan of chunk c); default for one-sequence layers: chunks growing from "
                        "16,384 tokens by 1.5x up to 131,072 (sdm.prefill_chunks); 1 = no pipelining")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one plain 1 GiB device copy (for counter calibration) and exit")
    return p.parse_args()


# sources of the scan's backward (its counter summaries carry their hash)
BACKWARD_SOURCES = ("sdm_scan_bwd_lanes.hip", "sdm_scan_backward.hip", "scan_lanes.h", "lanes_common.h",
                    "device_common.h", "kernels.h")


def scan_source_hash(files=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_memory_linear_pkm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, backward: bool = False, launches: int = 1):
    """HBM bytes per launch of the scan (or of the scan's backward) from the
    committed counter summary, if it was taken on the current kernel source
    (and, for a step of several launches, with the same number of launches
    per step: the average per launch); else None."""
    stem = "sdm_scan_backward" if backward else "sdm_scan"
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    key = "backward_source_sha256_16" if backward else "scan_source_sha256_16"
    if kv.get(key) != scan_source_hash(BACKWARD_SOURCES if backward else KERNEL_SOURCES):
        return None
    try:
        if launches > 1:
            if int(kv["launches_per_step"]) != launches:
                return None
            return float(kv["hbm_bytes_per_step"]) / launches
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def device_inputs(name, d, seed):
    import numpy as np
    import torch
    import sdm_synth as synth
    p = synth.PRESETS[name]
    if d.B * d.T * d.H <= 1 << 20 and d.H * d.N * d.d_v <= 1 << 28:
        x = synth.make_inputs(d, seed, reuse_frac=p.reuse_frac, recall_frac=p.recall_frac)

        def dev(a):
            a = np.ascontiguousarray(a)
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
            return torch.from_numpy(a).cuda()
        return {k: dev(v) for k, v in x.items()}, x
    return synth.make_inputs_torch(d, seed, reuse_frac=p.reuse_frac, recall_frac=p.recall_frac), None


def cpu_baseline(name, d, host_x, seed, min_seconds):
    """The oracle (as it stands) on the host cores, whole steps of the same
    workload (or a stated sample of it), reported in tokens/s."""
    import numpy as np
    import oracle
    import sdm_synth as synth
    threads = oracle.default_threads()
    if name == "decode":
        # 8 (b, h) pairs x a few hundred steps: the 137 GB state does not fit host RAM
        ds = d.replace(B=1, H=8, T=256)
        x = synth.make_inputs(ds, seed)
        sample = f"decode: 1 sequence x 8 heads x {ds.T} steps of the decode layer (N=1,048,576)"
        tokens = ds.T
    elif host_x is not None:
        ds, x = d, host_x
        sample = f"full step of the {name} workload (B={d.B}, T={d.T}, H={d.H})"
        tokens = d.B * d.T + d.B
    else:
        # a prefix of one sequence on a subset of the heads, so that the
        # sample's M0 and state fit host memory (2 heads of the long-context
        # layer: 1 GiB each); heads are independent and identically shaped,
        # so the rate is reported per token of all H heads
        Ts = min(d.T, 2048)
        Hs = max(1, min(d.H, (1 << 28) // (d.N * d.d_v)))
        ds = d.replace(B=1, T=Ts, H=Hs)
        x = synth.make_inputs(ds, seed)
        sample = (f"{name}: 1 sequence x {Ts} tokens x {Hs} of the {d.H} heads (prefix of the workload; "
                  f"rate scaled to all {d.H} heads: token-heads/s / {d.H})")
        tokens = Ts * Hs / d.H
    total_tokens, elapsed, reps = 0, 0.0, 0
    while elapsed < min_seconds or reps == 0:
        t0 = time.perf_counter()
        M = oracle.state_init(x["M0"], ds)
        ad = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], ds, nthreads=threads)
        oracle.scan(M, *ad, x["v"], x["a"], x["b"], ds, nthreads=threads)
        if name != "decode" and host_x is not None:
            k1 = np.ascontiguousarray(x["k"][:, -1])
            q1 = np.ascontiguousarray(x["q"][:, -1])
            v1 = np.ascontiguousarray(x["v"][:, -1])
            oracle.decode_step(M, k1, q1, x["C_w"], x["C_r"], v1, x["a"][:, -1].copy(),
                               x["b"][:, -1].copy(), ds, nthreads=threads)
        elapsed += time.perf_counter() - t0
        total_tokens += tokens
        reps += 1
        if reps >= 50:
            break
    return {"value": total_tokens / elapsed, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample}; {reps} repetition(s), {elapsed:.1f} s"}


def layer_edges(sdm, synth, torch, d, dims, o, stream, seed, reps=20):
    """The steps either side of the path, timed after the timed region (they
    are not part of the step): the gates from their pre-activations, the norm
    and output gate of the scan's read-out o, and the backward of both for
    given upstream gradients.  Per-launch time from HIP events on the launch
    stream, against the HBM peak."""
    x = synth.make_layer_edge_inputs_torch(d, seed)
    a = torch.empty_like(x["a_raw"])
    b = torch.empty_like(x["b_raw"])
    y = torch.empty(o.shape, dtype=x["g"].dtype, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(seed + 3)
    da = torch.randn(a.shape, generator=gen, dtype=torch.float32, device="cuda")
    db = torch.randn(a.shape, generator=gen, dtype=torch.float32, device="cuda")
    dy = torch.randn(o.shape, generator=gen, dtype=torch.float32, device="cuda")
    da_raw, db_raw = torch.empty_like(a), torch.empty_like(b)
    dA, ddt = torch.empty_like(x["A"]), torch.empty_like(x["A"])
    do, dg, dgamma = torch.empty_like(o), torch.empty_like(o), torch.empty_like(x["gamma"])
    nws_bytes = sdm.sdm_output_norm_gate_backward_workspace_size(dims)
    nws = torch.empty(max(nws_bytes, 1), dtype=torch.uint8, device="cuda")
    gws_bytes = sdm.sdm_gates_backward_workspace_size(dims)
    gws = torch.empty(max(gws_bytes, 1), dtype=torch.uint8, device="cuda")
    calls = [
        ("sdm_gates", lambda: sdm.sdm_gates(x["a_raw"], x["b_raw"], x["A"], x["dt_bias"], dims, a, b, stream)),
        ("sdm_output_norm_gate", lambda: sdm.sdm_output_norm_gate(o, x["g"], x["gamma"], 1e-5, dims, y, stream)),
        ("sdm_gates_backward", lambda: sdm.sdm_gates_backward(x["a_raw"], x["b_raw"], x["A"], x["dt_bias"], da, db,
                                                               dims, da_raw, db_raw, dA, ddt, gws, gws_bytes,
                                                               stream)),
        ("sdm_output_norm_gate_backward", lambda: sdm.sdm_output_norm_gate_backward(
            o, x["g"], x["gamma"], 1e-5, dy, dims, do, dg, dgamma, nws, nws_bytes, stream)),
    ]
    for _, f in calls:
        f()
    torch.cuda.synchronize()
    nc = len(calls)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range((nc + 1) * reps)]
    for r in range(reps):
        ev[(nc + 1) * r].record(stream)
        for c, (_, f) in enumerate(calls):
            f()
            ev[(nc + 1) * r + c + 1].record(stream)
    torch.cuda.synchronize()
    ms = [sum(ev[(nc + 1) * r + c].elapsed_time(ev[(nc + 1) * r + c + 1]) for r in range(reps)) / reps
          for c in range(nc)]
    th = d.B * d.T * d.H
    esz = 2 if d.in_dtype == "bf16" else 4
    nbytes = {
        "sdm_gates": th * 16 + d.H * 8,                                     # a_raw, b_raw read; a, b written
        "sdm_output_norm_gate": th * d.d_v * (4 + 2 * esz) + d.d_v * 4,     # o, g read; y written
        "sdm_gates_backward": th * 24,   # a_raw, b_raw, da, db read; da_raw, db_raw written
        "sdm_output_norm_gate_backward": th * d.d_v * (4 + esz + 4 + 8) + d.d_v * 4,   # o, g, dy read; do, dg written
    }
    out = {}
    for (name, _), t in zip(calls, ms):
        nb = nbytes[name]
        gbs = nb / (t * 1e-3) / 1e9
        out[name] = {"bound": "hbm", "ms": t, "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nb}
    return out


def decode_batches(sdm, torch, dx, per, M, o, dims1, d, nsteps, stream):
    """After the timed region: one batch of `nsteps` decode steps from the
    learned initial state, two ways.  Plain: sdm_state_init copies M0 into
    every sequence (B x |M0| bytes), then the steps.  Copy-on-write: the
    bitmap is cleared, then sdm_decode_step_cow reads every row a sequence
    has not written from M0.  Times from HIP events on the launch stream;
    the state buffer M is reused."""
    touched = torch.empty(sdm.sdm_cow_bitmap_bytes(dims1) // 4, dtype=torch.int32, device="cuda")
    ev = {n: torch.cuda.Event(enable_timing=True) for n in ("p0", "p1", "p2", "c0", "c1", "c2")}

    def steps(cow):
        for t in range(nsteps):
            args = (per["k"][t], per["q"][t], dx["C_w"], dx["C_r"], per["v"][t], per["a"][t], per["b"][t], o,
                    None, None, dims1, stream)
            if cow:
                sdm.sdm_decode_step_cow(M, dx["M0"], touched, *args)
            else:
                sdm.sdm_decode_step(M, *args)

    ev["p0"].record(stream)
    sdm.sdm_state_init(M, dx["M0"], dims1, stream)
    ev["p1"].record(stream)
    steps(False)
    ev["p2"].record(stream)
    ev["c0"].record(stream)
    sdm.sdm_cow_reset(touched, dims1, stream)
    ev["c1"].record(stream)
    steps(True)
    ev["c2"].record(stream)
    torch.cuda.synchronize()
    el = lambda a, b: ev[a].elapsed_time(ev[b])
    return {"steps": nsteps,
            "plain": {"state_init_ms": el("p0", "p1"), "steps_ms": el("p1", "p2"), "batch_ms": el("p0", "p2")},
            "copy_on_write": {"bitmap_reset_ms": el("c0", "c1"), "steps_ms": el("c1", "c2"),
                              "batch_ms": el("c0", "c2"), "bitmap_bytes": touched.numel() * 4},
            "batch_tokens_per_s_plain": d.B * nsteps / (el("p0", "p2") * 1e-3),
            "batch_tokens_per_s_cow": d.B * nsteps / (el("c0", "c2") * 1e-3)}


FP32_VECTOR_PEAK_TFLOPS = 157.3   # MI355X fp32 vector (packed) peak, vendor figure


def bench_gdn(args, sdm, synth, torch):
    """The dense Gated DeltaNet recurrence at the 1.4B layer's shape (B, T, H,
    d_k = d_v = 128, bf16 inputs): the rule the sparse memory reduces to with
    every slot selected.  One step = reset the state from S0 + one
    sdm_gdn_dense_forward over all B*T tokens."""
    import oracle
    base = synth.PRESETS["prefill_1p4b"].dims
    d = base.replace(n_sub=8, k_prime=8, W=64, R=64)
    x = synth.make_gdn_inputs_torch(d, args.seed)
    dims = sdm.dims_from(d)
    S = torch.empty_like(x["S0"])
    o = torch.empty((d.B, d.T, d.H, d.d_v), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = []

    def step(timed):
        S.copy_(x["S0"])
        e0 = torch.cuda.Event(enable_timing=True); e0.record(stream)
        sdm.sdm_gdn_dense_forward(S, x["k"], x["q"], x["v"], x["a"], x["b"], o, dims, stream)
        e1 = torch.cuda.Event(enable_timing=True); e1.record(stream)
        if timed:
            ev.append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True); end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(True)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / args.steps
    k_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    th = d.B * d.T * d.H
    flops = th * 6 * d.d_k * d.d_v          # k.s, the rank-1 update, q.s: 2 flops per state entry each
    tflops = flops / (k_ms * 1e-3) / 1e12
    result = {
        "metric": "dense Gated DeltaNet layer tokens/sec (the sparse memory with every slot selected)",
        "value": d.B * d.T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": "gdn_1p4b", "B": d.B, "T": d.T, "H": d.H, "d_k": d.d_k, "d_v": d.d_v,
                   "inputs": d.in_dtype, "state": "fp32",
                   "step": "state reset from S0 + sdm_gdn_dense_forward over B*T tokens"},
        "wall_s_timed_region": wall,
        "kernels_ms": {"sdm_gdn_dense_forward": k_ms},
        "roofline": {"kernel": "sdm_gdn_dense_kernel", "bound": "alu", "achieved": tflops,
                     "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tflops / FP32_VECTOR_PEAK_TFLOPS,
                     "traffic": None, "algorithmic_flops_per_launch": flops, "avg_launch_ms": k_ms},
    }
    if args.cpu_seconds > 0:
        ds = d.replace(B=1, T=2048)
        hx = synth.make_gdn_inputs(ds, args.seed)
        threads = oracle.default_threads()
        elapsed, reps = 0.0, 0
        while elapsed < args.cpu_seconds or reps == 0:
            S0 = hx["S0"].copy()
            t0 = time.perf_counter()
            oracle.gdn_dense(S0, hx["k"], hx["q"], hx["v"], hx["a"], hx["b"], ds, nthreads=threads)
            elapsed += time.perf_counter() - t0
            reps += 1
            if reps >= 50:
                break
        result["cpu_baseline"] = {"value": reps * ds.T / elapsed, "unit": "tokens/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"1 sequence x {ds.T} tokens x {ds.H} heads; {reps} repetition(s), "
                                            f"{elapsed:.1f} s"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def bench_train(args, sdm, synth, torch, name):
    """Forward with saving and the backward of a whole prefill layer between
    its projections (small or 1.4B).  One step = state init + the gates from
    their pre-activations + PKM addressing + the scan with its rows saved +
    the output norm and gate; then, for a given dL/dy (dL/dM_T = 0), the
    norm's backward + the backward scan + the addressing's backward (into k,
    q and the shared codebook) + the gates' backward.  The state copy and the
    zeroing of dL/dM_T run on a second stream beside the gates and the
    addressing."""
    layer = {"train_small": "small", "train_1p4b": "prefill_1p4b"}[name]
    d = synth.PRESETS[layer].dims
    dx, _ = device_inputs(layer, d, args.seed)
    ex = synth.make_layer_edge_inputs_torch(d, seed=args.seed + 7)
    dims = sdm.dims_from(d)
    B, T, H, N = d.B, d.T, d.H, d.N
    f32 = dict(dtype=torch.float32, device="cuda")
    M = torch.empty((B, H, N, d.d_v), **f32)
    dM = torch.empty_like(M)
    widx = torch.empty((B, T, H, d.W), dtype=torch.int32, device="cuda")
    wwt = torch.empty((B, T, H, d.W), **f32)
    ridx = torch.empty((B, T, H, d.R), dtype=torch.int32, device="cuda")
    rwt = torch.empty((B, T, H, d.R), **f32)
    a = torch.empty((B, T, H), **f32)
    b = torch.empty((B, T, H), **f32)
    o = torch.empty((B, T, H, d.d_v), **f32)
    y = torch.empty((B, T, H, d.d_v), dtype=ex["g"].dtype, device="cuda")
    xs = torch.empty((B, H, T, d.d_v // 4, d.W, 4), **f32)
    zs = torch.empty((B, H, T, d.d_v // 4, d.R, 4), **f32)
    dy = torch.randn((B, T, H, d.d_v), generator=torch.Generator(device="cuda").manual_seed(args.seed + 1), **f32)
    do = torch.empty((B, T, H, d.d_v), **f32)
    dg = torch.empty_like(do)
    dgamma = torch.empty(d.d_v, **f32)
    grads = [torch.empty((B, T, H, d.d_v), **f32), torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32),
             torch.empty((B, T, H, d.W), **f32), torch.empty((B, T, H, d.R), **f32)]
    da_raw, db_raw = torch.empty((B, T, H), **f32), torch.empty((B, T, H), **f32)
    dA, ddt = torch.empty(H, **f32), torch.empty(H, **f32)
    ws_bytes = sdm.sdm_scan_workspace_size(dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    aws_bytes = sdm.sdm_address_backward_workspace_size(dims)
    aws = torch.empty(max(aws_bytes, 1), dtype=torch.uint8, device="cuda")
    bws_bytes = sdm.sdm_scan_backward_workspace_size(dims)
    bws = torch.empty(max(bws_bytes, 1), dtype=torch.uint8, device="cuda")
    nws_bytes = sdm.sdm_output_norm_gate_backward_workspace_size(dims)
    nws = torch.empty(max(nws_bytes, 1), dtype=torch.uint8, device="cuda")
    gws_bytes = sdm.sdm_gates_backward_workspace_size(dims)
    gws = torch.empty(max(gws_bytes, 1), dtype=torch.uint8, device="cuda")
    dk = torch.empty((B, T, H, d.d_k), **f32)
    dq = torch.empty_like(dk)
    dC = torch.empty((H, 2, d.n_sub, d.d_k // 2), **f32)
    stream = torch.cuda.current_stream()
    eps = 1e-5
    names = ["init+gates+address", "sdm_scan_forward_save", "sdm_output_norm_gate",
             "sdm_output_norm_gate_backward", "sdm_scan_backward", "sdm_address_backward", "sdm_gates_backward"]
    timers = []

    # the state copy and the zeroing of dL/dM_T (two HBM streams) are
    # independent of the gates and the addressing (VALU-bound): they run on a
    # second stream, concurrently, and the forward scan waits for them
    side = torch.cuda.Stream()

    def step(timed):
        ev = [torch.cuda.Event(enable_timing=timed) for _ in range(len(names) + 1)]
        side_done = torch.cuda.Event()
        ev[0].record(stream)
        side.wait_event(ev[0])
        sdm.sdm_state_init(M, dx["M0"], dims, side)
        with torch.cuda.stream(side):
            dM.zero_()
        side_done.record(side)
        sdm.sdm_gates(ex["a_raw"], ex["b_raw"], ex["A"], ex["dt_bias"], dims, a, b, stream)
        sdm.sdm_pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims, widx, wwt, ridx, rwt, stream)
        stream.wait_event(side_done)
        ev[1].record(stream)
        sdm.sdm_scan_forward_save(M, widx, wwt, ridx, rwt, dx["v"], a, b, o, xs, zs, ws, ws_bytes, dims, stream)
        ev[2].record(stream)
        sdm.sdm_output_norm_gate(o, ex["g"], ex["gamma"], eps, dims, y, stream)
        ev[3].record(stream)
        sdm.sdm_output_norm_gate_backward(o, ex["g"], ex["gamma"], eps, dy, dims, do, dg, dgamma, nws, nws_bytes,
                                          stream)
        ev[4].record(stream)
        sdm.sdm_scan_backward(dM, widx, wwt, ridx, rwt, dx["v"], a, b, do, xs, zs, *grads, bws, bws_bytes, dims,
                              stream)
        ev[5].record(stream)
        # the codebook is shared by both kinds: one gradient buffer receives both sums
        sdm.sdm_address_backward(dx["k"], dx["q"], dx["C_w"], dx["C_r"], widx, wwt, ridx, rwt, grads[3], grads[4],
                                 dims, dk, dq, dC, dC, aws, aws_bytes, stream)
        ev[6].record(stream)
        sdm.sdm_gates_backward(ex["a_raw"], ex["b_raw"], ex["A"], ex["dt_bias"], grads[1], grads[2], dims, da_raw,
                               db_raw, dA, ddt, gws, gws_bytes, stream)
        ev[7].record(stream)
        if timed:
            timers.append(ev)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True); end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(True)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = start.elapsed_time(end) / args.steps
    kms = {n: sum(ev[i].elapsed_time(ev[i + 1]) for ev in timers) / len(timers) for i, n in enumerate(names)}
    fwd_ms, bwd_ms = kms["sdm_scan_forward_save"], kms["sdm_scan_backward"]
    th = B * T * H
    bwd_bytes = th * 3 * (d.W + d.R) * d.d_v * 4   # G rows in and out, saved rows in
    fwd_bytes = th * (2 * d.W + d.R + d.W + d.R) * d.d_v * 4   # the scan's rows plus the saved rows written
    # norm backward: o, g, dy read, do and dg written
    nbwd_bytes = th * d.d_v * (4 + (2 if d.in_dtype == "bf16" else 4) + 4 + 4 + 4)
    gbs = bwd_bytes / (bwd_ms * 1e-3) / 1e9
    result = {
        "metric": "SDM layer training tokens/sec (gates + addressing + scan forward with saved rows + output norm "
                  "and gate, and the backward of each)",
        "value": B * T / (ms_per_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
        "config": {"workload": name, "B": B, "T": T, "H": H, "N": N, "d_v": d.d_v, "W": d.W, "R": d.R,
                   "step": "state init and dL/dM_T zeroing (second stream, concurrent with the gates and the "
                           "addressing) + sdm_gates + addressing + sdm_scan_forward_save + sdm_output_norm_gate + "
                           "sdm_output_norm_gate_backward + sdm_scan_backward + sdm_address_backward + "
                           "sdm_gates_backward"},
        "wall_s_timed_region": wall,
        "kernels_ms": kms,
        "roofline": {"kernel": "sdm_scan_backward_kernel", "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(name, backward=True),
                     "algorithmic_bytes_per_launch": bwd_bytes, "avg_launch_ms": bwd_ms},
        "forward_save": {"GB/s": fwd_bytes / (fwd_ms * 1e-3) / 1e9, "algorithmic_bytes_per_launch": fwd_bytes},
        "norm_backward": {"GB/s": nbwd_bytes / (kms["sdm_output_norm_gate_backward"] * 1e-3) / 1e9,
                          "algorithmic_bytes_per_launch": nbwd_bytes},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def bench_row_traffic(args, torch):
    """What the MI355X delivers for the scan's memory-access pattern: the
    random row-segment gathers (write rows and read rows) and the stores of
    the write rows, in the scan's instruction form and workgroup layout, with
    no arithmetic and no dependence between steps (libsdm_bench.so).  Run on
    the long-context layer's table (16 chains of 2^20 rows of 512 bytes) with
    the segment sizes the scan can use (32, 64, 128 bytes: 2, 4, 8 waves per
    workgroup); with 4x or 2x the waves per workgroup, each extra group moving
    its own rows (more requests in flight per CU); with the same bytes split
    over 4x and 16x the chains at 32 bytes; and on a 16 GiB table split into
    32, 64 and 128 chains at 128 bytes (more CUs each moving whole lines).
    On the long-context table at 32 and 128 bytes also three variants: the
    gathers alone (the stores issued past the buffer range), and the gathers
    non-temporal or at device scope (bypassing the CU's L1).  Bytes per
    workgroup and step: 64 rows x 3 x segment per token group (x 2 for the
    gathers alone)."""
    import ctypes
    path = os.path.join(ROOT, "sparse_memory_linear_pkm_amd", "libsdm_bench.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m sparse_memory_linear_pkm_amd.build`")
    lib = ctypes.CDLL(path)
    fn = lib.sdm_bench_row_traffic
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.c_int, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    row_bytes = 512
    M = torch.zeros(128 * (1 << 18) * row_bytes // 4, dtype=torch.float32, device="cuda")   # 16 GiB
    stream = torch.cuda.current_stream()
    # (chains, log2 rows per chain, segment bytes, token groups, variant)
    configs = [(16, 20, 32, 1, 0), (16, 20, 64, 1, 0), (16, 20, 128, 1, 0), (16, 20, 32, 4, 0), (16, 20, 128, 2, 0),
               (64, 18, 32, 1, 0), (256, 16, 32, 1, 0), (32, 20, 128, 1, 0), (64, 19, 128, 1, 0),
               (128, 18, 128, 1, 0), (16, 20, 32, 1, 1), (16, 20, 32, 1, 2), (16, 20, 32, 1, 3),
               (16, 20, 128, 1, 1), (16, 20, 128, 1, 2), (16, 20, 128, 1, 3)]
    variants = {0: "scan form", 1: "gathers only", 2: "gathers non-temporal", 3: "gathers at device scope"}
    steps = max(1024, args.steps * 1024)
    out = []
    for chains, lg, seg, tg, var in configs:
        wgs = chains * row_bytes // seg
        nbytes = wgs * tg * steps * 64 * (2 if var == 1 else 3) * seg
        rc = fn(M.data_ptr(), chains, lg, row_bytes, seg, tg, var, 1024, 1, stream.cuda_stream)
        assert rc == 0, rc
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = fn(M.data_ptr(), chains, lg, row_bytes, seg, tg, var, steps, 7, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        assert rc == 0, rc
        ms = e0.elapsed_time(e1)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out.append({"chains": chains, "rows_per_chain": 1 << lg, "segment_bytes": seg, "token_groups": tg,
                    "variant": variants[var],
                    "workgroups": wgs, "waves": wgs * seg // 16 * tg, "steps": steps, "bytes": nbytes, "ms": ms,
                    "GB/s": gbs, "GB/s_per_workgroup": gbs / wgs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS})
    print(json.dumps({"metric": "scan access-pattern bandwidth (random row-segment gathers and stores, no arithmetic)",
                      "unit": "GB/s", "n_gpus": 1, "peak": HBM_PEAK_GBS, "data": "synthetic",
                      "config": {"workload": "row_traffic", "row_bytes": row_bytes,
                                 "per_step": "64 write-row and 64 read-row segments gathered, 64 stored, "
                                             "per token group"},
                      "results": out}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (every (sequence, head) chain is "
              "independent, so heads or sequences would shard with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sdm_synth as synth
    import sparse_memory_linear_pkm_amd as sdm

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    sdm.load_library()

    if args.copy_calibration:
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "copy_calibration_bytes_written": 4 * n}))
        return

    name = args.workload
    if name == "row_traffic":
        bench_row_traffic(args, torch)
        return
    if name == "gdn_1p4b":
        bench_gdn(args, sdm, synth, torch)
        return
    if name.startswith("train_"):
        bench_train(args, sdm, synth, torch, name)
        return
    d = synth.PRESETS[name].dims
    decode_mode = name == "decode"
    dx, host_x = device_inputs(name, d, args.seed)
    N = d.N
    stream = torch.cuda.current_stream()

    if decode_mode:
        d1 = d.replace(T=1)
        dims1 = sdm.dims_from(d1)
        M = torch.empty((d.B, d.H, N, d.d_v), dtype=torch.float32, device="cuda")
        sdm.state_init(dx["M0"], dims1, M=M)
        o = torch.empty((d.B, d.H, d.d_v), dtype=torch.float32, device="cuda")
        per = {key: [dx[key][:, t].contiguous() for t in range(d.T)] for key in ("k", "q", "v", "a", "b")}
        nsteps = min(args.decode_steps, d.T)

        def step(timers=None):
            ev = []
            for t in range(nsteps):
                if timers is not None and t == 0:
                    e = torch.cuda.Event(enable_timing=True); e.record(stream); ev.append(e)
                sdm.sdm_decode_step(M, per["k"][t], per["q"][t], dx["C_w"], dx["C_r"], per["v"][t], per["a"][t],
                                    per["b"][t], o, None, None, dims1, stream)
            if timers is not None:
                e = torch.cuda.Event(enable_timing=True); e.record(stream); ev.append(e)
                timers.append(ev)
        tokens_per_step = d.B * nsteps
    else:
        dims = sdm.dims_from(d)
        d1 = d.replace(T=1)
        dims1 = sdm.dims_from(d1)
        B, T, H = d.B, d.T, d.H
        M = torch.empty((B, H, N, d.d_v), dtype=torch.float32, device="cuda")
        widx = torch.empty((B, T, H, d.W), dtype=torch.int32, device="cuda")
        wwt = torch.empty((B, T, H, d.W), dtype=torch.float32, device="cuda")
        ridx = torch.empty((B, T, H, d.R), dtype=torch.int32, device="cuda")
        rwt = torch.empty((B, T, H, d.R), dtype=torch.float32, device="cuda")
        o = torch.empty((B, T, H, d.d_v), dtype=torch.float32, device="cuda")
        o1 = torch.empty((B, H, d.d_v), dtype=torch.float32, device="cuda")
        ws_bytes = sdm.sdm_scan_workspace_size(dims)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        # the decode token of each step: the last prefill token's inputs reused
        dec = {key: dx[key][:, -1].contiguous() for key in ("k", "q", "v", "a", "b")}

        # Chunked prefill (one sequence: a chunk of tokens is a contiguous
        # slice of every [B,T,H,...] array): the addressing of chunk c + 1 runs
        # on a second stream with at most one workgroup per CU
        # (sdm_pkm_address_overlapped), overlapping the scan of chunk c on the
        # main stream, whose workgroups take one CU each with room to spare.
        # The scan over consecutive chunks gives the same bits as one call.
        # Default: chunks growing from 16,384 tokens (sdm.prefill_chunks);
        # --chunks N: N equal chunks.
        if args.chunks is not None:
            nc = args.chunks
            if nc < 1 or T % nc != 0 or (nc > 1 and B != 1):
                raise SystemExit(f"--chunks {nc}: needs B == 1 and T divisible by the chunk count")
            chunks = [T // nc] * nc
        else:
            chunks = sdm.prefill_chunks(T) if B == 1 and T > 0 else [T]
        nc = len(chunks)
        bounds = [(sum(chunks[:c]), sum(chunks[:c + 1])) for c in range(nc)]
        dimsc = [sdm.dims_from(d.replace(T=n)) for n in chunks]
        wsc_bytes = max(sdm.sdm_scan_workspace_size(x) for x in dimsc)
        wsc = ws if nc == 1 else torch.empty(max(wsc_bytes, 1), dtype=torch.uint8, device="cuda")
        addr_stream = torch.cuda.Stream()

        def step_chunked(timers=None):
            E = lambda: torch.cuda.Event(enable_timing=timers is not None)
            ev = {k: E() for k in ("start", "init0", "init1", "scan1", "dec1")}
            ea = [(E(), E()) for _ in range(nc)]
            es = [(E(), E()) for _ in range(nc)]
            ev["start"].record(stream)
            addr_stream.wait_event(ev["start"])
            ev["init0"].record(stream)
            sdm.sdm_state_init(M, dx["M0"], dims, stream)
            ev["init1"].record(stream)
            for c, (t0, t1) in enumerate(bounds):
                sl = slice(t0, t1)
                ea[c][0].record(addr_stream)
                sdm.sdm_pkm_address_overlapped(dx["k"][:, sl], dx["q"][:, sl], dx["C_w"], dx["C_r"], dimsc[c],
                                               widx[:, sl], wwt[:, sl], ridx[:, sl], rwt[:, sl], addr_stream)
                ea[c][1].record(addr_stream)
            for c, (t0, t1) in enumerate(bounds):
                sl = slice(t0, t1)
                stream.wait_event(ea[c][1])
                es[c][0].record(stream)
                sdm.sdm_scan_forward(M, widx[:, sl], wwt[:, sl], ridx[:, sl], rwt[:, sl], dx["v"][:, sl],
                                     dx["a"][:, sl], dx["b"][:, sl], o[:, sl], wsc, wsc_bytes, dimsc[c], stream)
                es[c][1].record(stream)
            ev["scan1"].record(stream)
            sdm.sdm_decode_step(M, dec["k"], dec["q"], dx["C_w"], dx["C_r"], dec["v"], dec["a"], dec["b"], o1,
                                None, None, dims1, stream)
            ev["dec1"].record(stream)
            if timers is not None:
                timers.append((ev, ea, es))

        # state init and addressing are independent (one writes M, the other
        # reads k, q and the codebooks): the copy runs on a second stream,
        # concurrently with the addressing, and the scan waits for both
        init_stream = torch.cuda.Stream()

        def step_whole(timers=None):
            E = lambda: torch.cuda.Event(enable_timing=timers is not None)
            ev = {k: E() for k in ("start", "init0", "init1", "addr1", "scan0", "scan1", "dec1")}
            ev["start"].record(stream)
            init_stream.wait_event(ev["start"])
            ev["init0"].record(init_stream)
            sdm.sdm_state_init(M, dx["M0"], dims, init_stream)
            ev["init1"].record(init_stream)
            sdm.sdm_pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims, widx, wwt, ridx, rwt, stream)
            ev["addr1"].record(stream)
            stream.wait_event(ev["init1"])
            ev["scan0"].record(stream)
            sdm.sdm_scan_forward(M, widx, wwt, ridx, rwt, dx["v"], dx["a"], dx["b"], o, ws, ws_bytes, dims,
                                 stream)
            ev["scan1"].record(stream)
            sdm.sdm_decode_step(M, dec["k"], dec["q"], dx["C_w"], dx["C_r"], dec["v"], dec["a"], dec["b"], o1,
                                None, None, dims1, stream)
            ev["dec1"].record(stream)
            if timers is not None:
                timers.append(ev)
        step = step_chunked if nc > 1 else step_whole
        tokens_per_step = B * T + B

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timers = []
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step(timers)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    value = tokens_per_step / (ms_per_step / 1e3)

    result = {
        "metric": "SDM layer tokens/sec (prefill scan + decode) and % of HBM roofline",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": name, "B": d.B, "T": d.T, "H": d.H, "d_k": d.d_k, "n_sub": d.n_sub, "N": N,
                   "d_v": d.d_v, "k_prime": d.k_prime, "W": d.W, "R": d.R, "inputs": d.in_dtype,
                   "state": "fp32", "tokens_per_step": tokens_per_step,
                   "step": ("1024 decode steps" if decode_mode else
                            (f"state init + PKM addressing + prefill scan over {nc} chunks of "
                             f"{', '.join(str(n) for n in chunks)} tokens "
                             "(addressing of chunk c + 1 on a second stream, one workgroup per CU, overlapping "
                             "the scan of chunk c) + 1 decode token per sequence" if nc > 1 else
                             "state init (second stream, concurrent with the addressing) + PKM addressing + "
                             "prefill scan + 1 decode token per sequence"))},
        "wall_s_timed_region": wall,
    }

    if decode_mode:
        per_step_ms = [ev[0].elapsed_time(ev[1]) for ev in timers]
        avg = sum(per_step_ms) / len(per_step_ms)
        dec_ms = avg / nsteps
        bytes_per_launch = d.B * d.H * (2 * d.W + d.R) * d.d_v * 4
        achieved = bytes_per_launch / (dec_ms * 1e-3) / 1e9
        result["kernels_ms"] = {"sdm_decode_step": dec_ms}
        result["roofline"] = {"kernel": "sdm_decode_kernel", "bound": "hbm", "achieved": achieved,
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                              "traffic": None, "algorithmic_bytes_per_launch": bytes_per_launch,
                              "avg_launch_ms": dec_ms}
        result["copy_on_write"] = decode_batches(sdm, torch, dx, per, M, o, dims1, d, nsteps, stream)
    else:
        if nc > 1:
            # per call, summed over the chunks of a step (the addressing's
            # chunks run on the second stream, overlapped with the scan)
            def per_step(t):
                ev, ea, es = t
                return {"sdm_state_init": ev["init0"].elapsed_time(ev["init1"]),
                        "sdm_pkm_address_overlapped": sum(a.elapsed_time(b) for a, b in ea),
                        "sdm_scan_forward": sum(a.elapsed_time(b) for a, b in es),
                        "sdm_decode_step": ev["scan1"].elapsed_time(ev["dec1"])}
            rows_ = [per_step(t) for t in timers]
            avg = {k: sum(r[k] for r in rows_) / len(rows_) for k in rows_[0]}
        else:
            spans = {"sdm_state_init": ("init0", "init1"), "sdm_pkm_address": ("start", "addr1"),
                     "sdm_scan_forward": ("scan0", "scan1"), "sdm_decode_step": ("scan1", "dec1")}
            avg = {n: sum(ev[a].elapsed_time(ev[b]) for ev in timers) / len(timers) for n, (a, b) in spans.items()}
        result["kernels_ms"] = avg
        th = d.B * d.T * d.H
        scan_bytes = th * (2 * d.W + d.R) * d.d_v * 4
        scan_s = avg["sdm_scan_forward"] * 1e-3
        achieved = scan_bytes / scan_s / 1e9
        # per launch of sdm_scan_forward: one chunk of the sequence on average
        # (the whole sequence when nc = 1); the counter summary holds the bytes
        # per launch, or per step of nc launches
        traffic = measured_traffic(name, launches=nc)
        result["roofline"] = {"kernel": "sdm_scan_forward (scan_prep_kernel + sdm_scan_lanes_kernel)",
                              "bound": "hbm", "achieved": achieved,
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                              "traffic": traffic, "algorithmic_bytes_per_launch": scan_bytes / nc,
                              "avg_launch_ms": avg["sdm_scan_forward"] / nc, "launches_per_step": nc}
        # the addressing alone, after the timed region (in the step it shares
        # the chip with the state copy on the second stream)
        reps = max(3, min(20, args.steps))
        ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        torch.cuda.synchronize()
        ev_a[0].record(stream)
        for r in range(reps):
            sdm.sdm_pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims, widx, wwt, ridx, rwt, stream)
            ev_a[r + 1].record(stream)
        torch.cuda.synchronize()
        addr_alone = sum(ev_a[r].elapsed_time(ev_a[r + 1]) for r in range(reps)) / reps
        flops = th * 4 * d.n_sub * d.d_k
        addr_tflops = flops / (addr_alone * 1e-3) / 1e12
        result["pkm_scoring"] = {"kernel": "pkm_score_topk", "bound": "mfma", "achieved": addr_tflops,
                                 "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                                 "frac": addr_tflops / BF16_DENSE_PEAK_TFLOPS,
                                 "algorithmic_flops_per_launch": flops, "avg_launch_ms": addr_alone,
                                 "timed": f"sdm_pkm_address alone, {reps} launches after the timed region"}
        init_bytes = (1 + d.B) * d.H * N * d.d_v * 4
        result["state_init"] = {"GB/s": init_bytes / (avg["sdm_state_init"] * 1e-3) / 1e9,
                                "bytes_per_launch": init_bytes}
        result["scan_tokens_per_s"] = d.B * d.T / scan_s
        result["layer_edges"] = layer_edges(sdm, synth, torch, d, dims, o, stream, args.seed)

    if args.cpu_seconds > 0:
        result["cpu_baseline"] = cpu_baseline(name, d, host_x, args.seed, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
