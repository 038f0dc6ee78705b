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

from gpu_helpers import note, to_host

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
