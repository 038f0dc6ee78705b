"""The C-ABI calls under HIP graph capture: one whole step (state init,
addressing, prefill scan, decode step) captured once and replayed several
times, with eager work and synchronisations between the replays; every
replay must reproduce the eager step bit for bit (the library allocates
nothing, clears nothing with memsets and never synchronises, so the calls
are capturable as they are)."""
import numpy as np
import pytest

import sdm_synth as synth
from sdm_synth import Dims

from gpu_helpers import note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available()
    return _t


@pytest.fixture(scope="module")
def sdm():
    import sparse_memory_linear_pkm_amd as _s
    _s.load_library()
    return _s


def test_graph_capture_replays_match_eager(sdm, torch):
    d = Dims(B=3, T=70, H=2, d_k=128, n_sub=32, d_v=64, k_prime=8, W=8, R=6)
    note(f"graph capture {d}")
    x = synth.make_inputs_torch(d, seed=21)
    dims = sdm.dims_from(d)
    dims1 = sdm.dims_from(d.replace(T=1))
    B, T, H = d.B, d.T, d.H
    dev = "cuda"
    M = torch.empty((B, H, d.N, d.d_v), dtype=torch.float32, device=dev)
    widx = torch.empty((B, T, H, d.W), dtype=torch.int32, device=dev)
    wwt = torch.empty((B, T, H, d.W), dtype=torch.float32, device=dev)
    ridx = torch.empty((B, T, H, d.R), dtype=torch.int32, device=dev)
    rwt = torch.empty((B, T, H, d.R), dtype=torch.float32, device=dev)
    o = torch.empty((B, T, H, d.d_v), dtype=torch.float32, device=dev)
    o1 = torch.empty((B, H, d.d_v), dtype=torch.float32, device=dev)
    wo = torch.empty((B, H, d.W), dtype=torch.int32, device=dev)
    ro = torch.empty((B, H, d.R), dtype=torch.int32, device=dev)
    ws_bytes = sdm.sdm_scan_workspace_size(dims)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    dec = {k: x[k][:, -1].contiguous() for k in ("k", "q", "v", "a", "b")}

    def step():
        sdm.sdm_state_init(M, x["M0"], dims)
        sdm.sdm_pkm_address(x["k"], x["q"], x["C_w"], x["C_r"], dims, widx, wwt, ridx, rwt)
        sdm.sdm_scan_forward(M, widx, wwt, ridx, rwt, x["v"], x["a"], x["b"], o, ws, ws_bytes, dims)
        sdm.sdm_decode_step(M, dec["k"], dec["q"], x["C_w"], x["C_r"], dec["v"], dec["a"], dec["b"], o1, wo, ro,
                            dims1)

    outs = (M, widx, wwt, ridx, rwt, o, o1, wo, ro)
    step()
    torch.cuda.synchronize()
    ref = [to_host(t).copy() for t in outs]

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:   # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("M", "widx", "wwt", "ridx", "rwt", "o", "o1", "wo", "ro"), outs, ref):
            np.testing.assert_array_equal(to_host(t), r, err_msg=f"replay {rep}: {name}")


def test_graph_capture_training_step_and_layer_edges(sdm, torch):
    """The other entry points under capture: gates, the scan with its rows
    saved, the backward scan, the output norm and gate, the backward of the
    norm and of the gates, the addressing's backward, and the dense
    recurrence; three replays, each bit-identical to the eager run."""
    d = Dims(B=2, T=40, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=8, R=8)
    note(f"graph capture, training step {d}")
    x = synth.make_inputs(d, seed=31)
    ad = synth.random_addressing(d, seed=31, hazard_slots=40)
    e = synth.make_layer_edge_inputs(d, seed=31)
    g = synth.make_gdn_inputs(d.replace(d_k=64), seed=31)
    dims, gdims = sdm.dims_from(d), sdm.dims_from(d.replace(d_k=64))
    T = torch
    dev = {k: to_dev(v) for k, v in ad.items()}
    M0 = to_dev(np.repeat(x["M0"][None], d.B, axis=0).copy())
    M = T.empty_like(M0)
    dM = T.empty_like(M0)
    o = T.empty((d.B, d.T, d.H, d.d_v), dtype=T.float32, device="cuda")
    xs = T.empty((d.B, d.H, d.T, d.d_v // 4, d.W, 4), dtype=T.float32, device="cuda")
    zs = T.empty((d.B, d.H, d.T, d.d_v // 4, d.R, 4), dtype=T.float32, device="cuda")
    dout = to_dev(np.random.default_rng(2).normal(0, 1, (d.B, d.T, d.H, d.d_v)).astype(np.float32))
    grads = [T.empty((d.B, d.T, d.H, d.d_v), dtype=T.float32, device="cuda"),
             T.empty((d.B, d.T, d.H), dtype=T.float32, device="cuda"),
             T.empty((d.B, d.T, d.H), dtype=T.float32, device="cuda"),
             T.empty((d.B, d.T, d.H, d.W), dtype=T.float32, device="cuda"),
             T.empty((d.B, d.T, d.H, d.R), dtype=T.float32, device="cuda")]
    a_g = T.empty((d.B, d.T, d.H), dtype=T.float32, device="cuda")
    b_g = T.empty_like(a_g)
    y = T.empty((d.B, d.T, d.H, d.d_v), dtype=T.bfloat16, device="cuda")
    S0 = to_dev(g["S0"])
    S = T.empty_like(S0)
    og = T.empty((d.B, d.T, d.H, d.d_v), dtype=T.float32, device="cuda")
    ws_bytes = sdm.sdm_scan_workspace_size(dims)
    ws = T.empty(max(ws_bytes, 1), dtype=T.uint8, device="cuda")
    inp = {k: to_dev(v) for k, v in e.items()}
    gin = {k: to_dev(v) for k, v in g.items() if k != "S0"}
    xv = to_dev(x["v"])
    do_n, dg_n = T.empty_like(o), T.empty_like(o)
    dgamma = T.empty(d.d_v, dtype=T.float32, device="cuda")
    gb = [T.empty((d.B, d.T, d.H), dtype=T.float32, device="cuda") for _ in range(2)]
    gb += [T.empty(d.H, dtype=T.float32, device="cuda") for _ in range(2)]
    nws_bytes = sdm.sdm_output_norm_gate_backward_workspace_size(dims)
    nws = T.empty(max(nws_bytes, 1), dtype=T.uint8, device="cuda")
    gws_bytes = sdm.sdm_gates_backward_workspace_size(dims)
    gws = T.empty(max(gws_bytes, 1), dtype=T.uint8, device="cuda")
    aws_bytes = sdm.sdm_address_backward_workspace_size(dims)
    aws = T.empty(max(aws_bytes, 1), dtype=T.uint8, device="cuda")
    bws_bytes = sdm.sdm_scan_backward_workspace_size(dims)
    bws = T.empty(max(bws_bytes, 1), dtype=T.uint8, device="cuda")
    kx, qx, Cw = to_dev(x["k"]), to_dev(x["q"]), to_dev(x["C_w"])
    dk = T.empty((d.B, d.T, d.H, d.d_k), dtype=T.float32, device="cuda")
    dq = T.empty_like(dk)
    dC = T.empty((d.H, 2, d.n_sub, d.d_k // 2), dtype=T.float32, device="cuda")

    def step():
        sdm.sdm_gates(inp["a_raw"], inp["b_raw"], inp["A"], inp["dt_bias"], dims, a_g, b_g)
        M.copy_(M0)
        dM.zero_()
        sdm.sdm_scan_forward_save(M, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], xv, a_g, b_g, o, xs, zs, ws,
                                  ws_bytes, dims)
        sdm.sdm_scan_backward(dM, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], xv, a_g, b_g, dout, xs, zs,
                              *grads, bws, bws_bytes, dims)
        sdm.sdm_output_norm_gate(o, inp["g"], inp["gamma"], 1e-5, dims, y)
        sdm.sdm_output_norm_gate_backward(o, inp["g"], inp["gamma"], 1e-5, dout, dims, do_n, dg_n, dgamma, nws,
                                          nws_bytes)
        sdm.sdm_gates_backward(inp["a_raw"], inp["b_raw"], inp["A"], inp["dt_bias"], grads[1], grads[2], dims,
                               *gb, gws, gws_bytes)
        sdm.sdm_address_backward(kx, qx, Cw, Cw, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], grads[3], grads[4],
                                 dims, dk, dq, dC, dC, aws, aws_bytes)
        S.copy_(S0)
        sdm.sdm_gdn_dense_forward(S, gin["k"], gin["q"], gin["v"], gin["a"], gin["b"], og, gdims)

    outs = (a_g, b_g, M, dM, o, xs, zs, *grads, y, do_n, dg_n, dgamma, *gb, dk, dq, dC, S, og)
    step()
    T.cuda.synchronize()
    ref = [to_host(t).copy() for t in outs]
    gr = T.cuda.CUDAGraph()
    side = T.cuda.Stream()
    side.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(side):
        with T.cuda.graph(gr):
            step()
    T.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.zero_()
        T.cuda.synchronize()
        gr.replay()
        T.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            np.testing.assert_array_equal(to_host(t), r, err_msg=f"replay {rep}: output {i}")


def test_graph_capture_copy_on_write_decode(sdm, torch):
    """A batch of copy-on-write decode steps under capture: bitmap reset,
    four steps, materialize; three replays (with the state and bitmap
    overwritten in between), each bit-identical to the eager run."""
    d = Dims(B=3, T=4, H=2, d_k=128, n_sub=32, d_v=64, k_prime=8, W=8, R=6)
    note(f"graph capture, copy-on-write decode {d}")
    x = synth.make_inputs_torch(d, seed=22)
    dims1 = sdm.dims_from(d.replace(T=1))
    T = torch
    M = T.empty((d.B, d.H, d.N, d.d_v), dtype=T.float32, device="cuda")
    touched = T.empty(sdm.sdm_cow_bitmap_bytes(dims1) // 4, dtype=T.int32, device="cuda")
    per = [{k: x[k][:, t].contiguous() for k in ("k", "q", "v", "a", "b")} for t in range(d.T)]
    o1 = [T.empty((d.B, d.H, d.d_v), dtype=T.float32, device="cuda") for _ in range(d.T)]
    wo = [T.empty((d.B, d.H, d.W), dtype=T.int32, device="cuda") for _ in range(d.T)]

    def step():
        sdm.sdm_cow_reset(touched, dims1)
        for t in range(d.T):
            p = per[t]
            sdm.sdm_decode_step_cow(M, x["M0"], touched, p["k"], p["q"], x["C_w"], x["C_r"], p["v"], p["a"], p["b"],
                                    o1[t], wo[t], None, dims1)
        sdm.sdm_cow_materialize(M, x["M0"], touched, dims1)

    outs = (M, touched, *o1, *wo)
    M.fill_(float("nan"))
    step()
    T.cuda.synchronize()
    ref = [to_host(t).copy() for t in outs]
    g = T.cuda.CUDAGraph()
    side = T.cuda.Stream()
    side.wait_stream(T.cuda.current_stream())
    with T.cuda.stream(side):
        with T.cuda.graph(g):
            step()
    T.cuda.synchronize()
    for rep in range(3):
        M.fill_(float("nan"))
        touched.fill_(-1)
        for t in o1 + wo:
            t.zero_()
        T.cuda.synchronize()
        g.replay()
        T.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outs, ref)):
            np.testing.assert_array_equal(to_host(t), r, err_msg=f"replay {rep}: output {i}")
