"""The whole layer between its projections, forward and backward, chained
through the C ABI as the training bench runs it, against the same chain of
oracle functions: gates -> addressing -> scan (rows saved) -> output norm and
gate; then, for a given dL/dy, the norm's backward -> the scan's backward ->
the addressing's backward (one codebook for both kinds) -> the gates'
backward.  This checks how the calls compose (what each hands the next);
each one is checked on its own elsewhere.  The slot lists are the GPU's
(the oracle's selection is compared separately, with its near-tie rule).

Bar: every final gradient within 2e-3 x RMS of the oracle chain's.
"""
import numpy as np
import pytest

import oracle
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


def close_rms(got, ref, what, bar=2e-3):
    ref = np.asarray(ref, np.float64)
    scale = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref)))
    note(f"{what}: max |err| / RMS = {err / max(scale, 1e-30):.2e}")
    assert err <= bar * scale, f"{what}: max error {err:.3g} > {bar} x RMS {scale:.3g}"


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_layer_forward_backward_chain(sdm, torch, in_dtype):
    T = torch
    d = Dims(B=2, T=96, H=3, d_k=128, n_sub=16, d_v=64, k_prime=8, W=8, R=8, in_dtype=in_dtype)
    note(f"layer chain {d}")
    x = synth.make_inputs(d, seed=51)
    e = synth.make_layer_edge_inputs(d, seed=52)
    gr = synth.make_layer_edge_grads(d, seed=53)
    eps = 1e-5
    dims = sdm.dims_from(d)
    dx = {k: to_dev(v) for k, v in x.items()}
    de = {k: to_dev(v) for k, v in e.items()}
    # GPU chain
    a, b = sdm.gates(de["a_raw"], de["b_raw"], de["A"], de["dt_bias"], dims)
    widx, wwt, ridx, rwt = sdm.pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_w"], dims)
    M = sdm.state_init(dx["M0"], dims)
    o, xs, zs = sdm.scan_forward_save(M, widx, wwt, ridx, rwt, dx["v"], a, b, dims)
    y = sdm.output_norm_gate(o, de["g"], de["gamma"], eps, dims)
    do, dg, dgamma = sdm.output_norm_gate_backward(o, de["g"], de["gamma"], eps, to_dev(gr["dy"]), dims)
    dM = T.zeros_like(M)
    dv, da, db, dw, dr = sdm.scan_backward(dM, widx, wwt, ridx, rwt, dx["v"], a, b, do, xs, zs, dims)
    dk, dq, dC, _ = sdm.address_backward(dx["k"], dx["q"], dx["C_w"], dx["C_w"], widx, wwt, ridx, rwt, dw, dr, dims,
                                         shared_codebook_grad=True)
    da_raw, db_raw, dA, ddt = sdm.gates_backward(de["a_raw"], de["b_raw"], de["A"], de["dt_bias"], da, db, dims)
    T.cuda.synchronize()
    # oracle chain (on the GPU's slot lists and weights)
    hw, hww, hr, hrw = (to_host(t) for t in (widx, wwt, ridx, rwt))
    oa, ob = oracle.gates(e["a_raw"], e["b_raw"], e["A"], e["dt_bias"], d)
    M0 = np.repeat(x["M0"][None], d.B, axis=0).copy()
    oo = oracle.scan(M0.copy(), hw, hww, hr, hrw, x["v"], oa, ob, d)
    oy = oracle.output_norm_gate(oo.astype(np.float32), e["g"], e["gamma"], eps, d)
    odo, odg, odgamma = oracle.output_norm_gate_backward(oo.astype(np.float32), e["g"], e["gamma"], eps, gr["dy"], d)
    g = oracle.scan_backward(M0, hw, hww, hr, hrw, x["v"], oa, ob, odo, d)
    odk, odq, oCw, oCr = oracle.address_backward(x["k"], x["q"], x["C_w"], x["C_w"], hw, hww, hr, hrw, g["dw"],
                                                 g["dr"], d)
    oda_raw, odb_raw, odA, oddt = oracle.gates_backward(e["a_raw"], e["b_raw"], e["A"], e["dt_bias"], g["da"],
                                                        g["db"], d)
    if in_dtype == "bf16":
        # rounded to bf16 from an fp32 value within 2e-3 x RMS of the exact
        # one: one of the two bf16 neighbours of the exact value, or its
        # rounding of a slightly different value
        yh = synth.bf16_bits_to_f32(to_host(y)).astype(np.float64)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(oy), 2.0 ** -126))) - 7)
        tol = ulp + 2e-3 * np.sqrt(np.mean(oy ** 2))
        assert np.all(np.abs(yh - oy) <= tol), f"y: {int((np.abs(yh - oy) > tol).sum())} out of tolerance"
    else:
        close_rms(to_host(y), oy, "y")
    for name, got, ref in (("do", do, odo), ("dg", dg, odg), ("dgamma", dgamma, odgamma), ("dM0", dM, g["dM"]),
                           ("dv", dv, g["dv"]), ("da", da, g["da"]), ("db", db, g["db"]), ("dw", dw, g["dw"]),
                           ("dr", dr, g["dr"]), ("dk", dk, odk), ("dq", dq, odq),
                           ("dC", dC, oCw.astype(np.float64) + oCr), ("da_raw", da_raw, oda_raw),
                           ("db_raw", db_raw, odb_raw), ("dA", dA, odA), ("ddt_bias", ddt, oddt)):
        close_rms(to_host(got), ref, name)
