"""The prefill pipelined over chunks of tokens, as the long-context bench
step runs it: the addressing of each chunk on a second stream with at most
one workgroup per CU (sdm_pkm_address_overlapped), the scan of each chunk on
the main stream once its addressing is done.  Every output must equal the
one-call prefill (sdm_pkm_address, then sdm_scan_forward over all tokens)
bit for bit: the addressing is per token-head, and the scan over
consecutive chunks performs the same operations in the same order."""
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


@pytest.mark.parametrize("d,nc", [
    (Dims(B=1, T=4096, H=8, d_k=128, n_sub=256, d_v=64, k_prime=16, W=16, R=16), 8),
    (Dims(B=1, T=2048, H=4, d_k=128, n_sub=1024, d_v=128, k_prime=32, W=32, R=32), 16),
], ids=["n256_dv64", "n1024_dv128"])
def test_chunked_pipelined_prefill_equals_one_call(sdm, torch, d, nc):
    note(f"pipelined prefill {d}, {nc} chunks")
    T = torch
    x = synth.make_inputs_torch(d, seed=19, recall_frac=0.01)
    dims = sdm.dims_from(d)
    Tc = d.T // nc
    dimsc = sdm.dims_from(d.replace(T=Tc))
    B, H = d.B, d.H

    def bufs():
        return (T.empty((B, d.T, H, d.W), dtype=T.int32, device="cuda"),
                T.empty((B, d.T, H, d.W), dtype=T.float32, device="cuda"),
                T.empty((B, d.T, H, d.R), dtype=T.int32, device="cuda"),
                T.empty((B, d.T, H, d.R), dtype=T.float32, device="cuda"))

    # one call each
    w1, ww1, r1, rw1 = bufs()
    main = T.cuda.current_stream()
    sdm.sdm_pkm_address(x["k"], x["q"], x["C_w"], x["C_r"], dims, w1, ww1, r1, rw1, main)
    M1 = sdm.state_init(x["M0"], dims)
    o1 = sdm.scan_forward(M1, w1, ww1, r1, rw1, x["v"], x["a"], x["b"], dims)
    # the pipelined form
    w2, ww2, r2, rw2 = bufs()
    M2 = sdm.state_init(x["M0"], dims)
    o2 = T.empty_like(o1)
    ws_bytes = sdm.sdm_scan_workspace_size(dimsc)
    ws = T.empty(max(ws_bytes, 1), dtype=T.uint8, device="cuda")
    side = T.cuda.Stream()
    start = T.cuda.Event()
    start.record(main)
    side.wait_event(start)
    done = []
    for c in range(nc):
        sl = slice(c * Tc, (c + 1) * Tc)
        sdm.sdm_pkm_address_overlapped(x["k"][:, sl], x["q"][:, sl], x["C_w"], x["C_r"], dimsc,
                                       w2[:, sl], ww2[:, sl], r2[:, sl], rw2[:, sl], side)
        e = T.cuda.Event()
        e.record(side)
        done.append(e)
    for c in range(nc):
        sl = slice(c * Tc, (c + 1) * Tc)
        main.wait_event(done[c])
        sdm.sdm_scan_forward(M2, w2[:, sl], ww2[:, sl], r2[:, sl], rw2[:, sl], x["v"][:, sl], x["a"][:, sl],
                             x["b"][:, sl], o2[:, sl], ws, ws_bytes, dimsc, main)
    T.cuda.synchronize()
    for name, a, b in (("widx", w1, w2), ("wwt", ww1, ww2), ("ridx", r1, r2), ("rwt", rw1, rw2), ("o", o1, o2),
                       ("M", M1, M2)):
        assert np.array_equal(to_host(a), to_host(b)), name


@pytest.mark.parametrize("n_sub,kp", [(1024, 32), (1024, 8), (512, 32), (2048, 32)])
def test_overlapped_addressing_equals_address(sdm, torch, n_sub, kp):
    """sdm_pkm_address_overlapped (one workgroup per CU, the one-part
    selection) returns the same slots and weights, bit for bit, as
    sdm_pkm_address (for 1024 or more sub-keys per half the selection in parts
    of 512 and their merges)."""
    d = Dims(B=2, T=300, H=3, d_k=128, n_sub=n_sub, d_v=32, k_prime=kp, W=32, R=kp)
    note(f"overlapped vs plain addressing {d}")
    x = synth.make_inputs_torch(d, seed=23, m0=False)
    dims = sdm.dims_from(d)
    a = sdm.pkm_address(x["k"], x["q"], x["C_w"], x["C_r"], dims)
    b = [torch.empty_like(t) for t in a]
    sdm.sdm_pkm_address_overlapped(x["k"], x["q"], x["C_w"], x["C_r"], dims, *b)
    torch.cuda.synchronize()
    for ta, tb, name in zip(a, b, ("widx", "wwt", "ridx", "rwt")):
        np.testing.assert_array_equal(to_host(ta), to_host(tb), err_msg=name)
