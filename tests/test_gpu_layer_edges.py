"""GPU parity of the steps either side of the path, through the C ABI:
sdm_gates (forget and input gates from their pre-activations) and
sdm_output_norm_gate (RMS norm of the read-out with the output gate),
element by element against the oracle.

Tolerances follow from the fp32 arithmetic of the kernels (u = 2^-24):
  a = exp(-A softplus(z)): the sum z = a_raw + dt_bias is rounded once
    (relative u, amplified by A |z| in the exponent), softplus, the product
    and exp each add a few u of relative error to ln a, so
    |a_gpu - a| <= a (A |z| 2u + (|ln a| + 1) 8u).
  b = 1 / (1 + exp(-b_raw)): |b_gpu - b| <= 8u b.
  The oracle's fp32 values add their own rounding (u relative), and results
  in the fp32 subnormal range may be off by a few subnormal steps.
  y (fp32): the sum of squares of d_v terms (per-lane chains of d_v/8 terms
    and an 8-lane tree), the mean, sqrt, reciprocal, three products and silu:
    |y_gpu - y| <= (d_v/8 + 24) u |y|.
  y (bf16): the fp32 value above rounded to bf16, which lands on one of the
    two bf16 neighbours of the exact value: |y_gpu - y| <= one bf16 ulp of |y|.
"""
import numpy as np
import pytest

import oracle
import sdm_synth as synth
from sdm_synth import Dims

from gpu_helpers import note, to_dev, to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
SUBNORMAL = 2.0 ** -149
MIN_NORMAL = 2.0 ** -126


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


def check_gates(a_gpu, b_gpu, a_raw, b_raw, A, dt, d):
    a_o, b_o = oracle.gates(a_raw, b_raw, A, dt, d)
    a_o64, b_o64 = a_o.astype(np.float64), b_o.astype(np.float64)
    # the oracle's values are the exact ones rounded once to fp32 (half an ulp more)
    z = np.abs(a_raw.astype(np.float64) + dt.astype(np.float64)[None, None, :])
    Ah = A.astype(np.float64)[None, None, :]
    lna = np.where(a_o64 > 0, -np.log(np.maximum(a_o64, 1e-300)), 0.0)
    tol_a = a_o64 * (Ah * z * 2 * U + (lna + 1.0) * 8 * U + U) + 4 * SUBNORMAL
    err_a = np.abs(a_gpu.astype(np.float64) - a_o64)
    assert np.all(err_a <= tol_a), (f"a: {int((err_a > tol_a).sum())} out of tolerance, worst excess "
                                    f"{np.max(err_a - tol_a):.3g}")
    tol_b = 9 * U * b_o64 + 4 * SUBNORMAL
    err_b = np.abs(b_gpu.astype(np.float64) - b_o64)
    assert np.all(err_b <= tol_b), f"b: {int((err_b > tol_b).sum())} out of tolerance"


def bf16_ulp(y):
    ay = np.abs(y)
    e = np.floor(np.log2(np.maximum(ay, MIN_NORMAL)))
    return np.exp2(e - 7)


def check_norm(y_gpu, y_orc, d):
    y_orc = y_orc.astype(np.float64)
    if d.in_dtype == "bf16":
        yg = synth.bf16_bits_to_f32(y_gpu).astype(np.float64)
        tol = bf16_ulp(y_orc) + 2.0 ** -133
    else:
        yg = y_gpu.astype(np.float64)
        tol = (d.d_v / 8 + 24) * U * np.abs(y_orc) + SUBNORMAL
    err = np.abs(yg - y_orc)
    assert np.all(err <= tol), (f"y: {int((err > tol).sum())} elements out of tolerance; worst excess "
                                f"{np.max(err - tol):.3g} at {np.unravel_index(np.argmax(err - tol), err.shape)}")


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (3, 77, 5), (2, 1000, 16), (4, 0, 3)])
def test_gates_match_oracle(sdm, torch, B, T, H):
    d = Dims(B=B, T=T, H=H, d_k=8, n_sub=4, d_v=32, k_prime=4, W=4, R=4, in_dtype="f32")
    note(f"gates B={B} T={T} H={H}")
    x = synth.make_layer_edge_inputs(d, seed=B * 100 + T + H)
    a_raw, b_raw = x["a_raw"] * 3.0, x["b_raw"] * 3.0
    # extremes: large pre-activations of both signs, and the softplus branch point
    ext_a = np.array([40.0, -40.0, 90.0, -90.0, 0.0, 1e-7], np.float32)
    ext_b = np.array([40.0, -40.0, 100.0, -100.0], np.float32)
    fa, fb = a_raw.reshape(-1), b_raw.reshape(-1)
    fa[:min(fa.size, ext_a.size)] = ext_a[:min(fa.size, ext_a.size)]
    fb[:min(fb.size, ext_b.size)] = ext_b[:min(fb.size, ext_b.size)]
    dims = sdm.dims_from(d)
    a_d, b_d = sdm.gates(to_dev(a_raw), to_dev(b_raw), to_dev(x["A"]), to_dev(x["dt_bias"]), dims)
    torch.cuda.synchronize()
    check_gates(to_host(a_d), to_host(b_d), a_raw, b_raw, x["A"], x["dt_bias"], d)


def test_gates_in_place(sdm, torch):
    d = Dims(B=2, T=33, H=4, d_k=8, n_sub=4, d_v=32, k_prime=4, W=4, R=4, in_dtype="f32")
    note("gates in place")
    x = synth.make_layer_edge_inputs(d, seed=5)
    dims = sdm.dims_from(d)
    a_t, b_t = to_dev(x["a_raw"]), to_dev(x["b_raw"])
    sdm.sdm_gates(a_t, b_t, to_dev(x["A"]), to_dev(x["dt_bias"]), dims, a_t, b_t)
    torch.cuda.synchronize()
    check_gates(to_host(a_t), to_host(b_t), x["a_raw"], x["b_raw"], x["A"], x["dt_bias"], d)


@pytest.mark.parametrize("d", [
    Dims(B=2, T=150, H=3, d_k=128, n_sub=16, d_v=64, k_prime=8, W=16, R=16),
    Dims(B=1, T=77, H=2, d_k=32, n_sub=8, d_v=32, k_prime=8, W=8, R=5, in_dtype="f32"),
    Dims(B=8, T=64, H=16, d_k=128, n_sub=32, d_v=128, k_prime=32, W=32, R=32),
], ids=["small_bf16", "f32_W8_R5", "dv128_W32"])
def test_gated_scan_equals_gates_then_scan(sdm, torch, d):
    """sdm_scan_forward_gated (the gates applied in the scan's preparation
    pass) gives the results of sdm_gates followed by sdm_scan_forward bit for
    bit, also with extreme pre-activations; and both match the oracle's
    gates followed by the oracle's scan."""
    note(f"gated scan {d}")
    x = synth.make_inputs(d, seed=13)
    ad = synth.random_addressing(d, seed=13, hazard_slots=4 * max(d.W, d.R))
    e = synth.make_layer_edge_inputs(d, seed=13)
    a_raw, b_raw = e["a_raw"] * 3.0, e["b_raw"] * 3.0
    fa, fb = a_raw.reshape(-1), b_raw.reshape(-1)
    fa[:6] = [40.0, -40.0, 90.0, -90.0, 0.0, 1e-7]
    fb[:4] = [40.0, -40.0, 100.0, -100.0]
    dims = sdm.dims_from(d)
    dev = {k: to_dev(v) for k, v in ad.items()}
    M0 = np.repeat(x["M0"][None], d.B, axis=0).copy()
    ar, br, Ad, dtd = to_dev(a_raw), to_dev(b_raw), to_dev(e["A"]), to_dev(e["dt_bias"])
    a_d, b_d = sdm.gates(ar, br, Ad, dtd, dims)
    M1 = to_dev(M0)
    o1 = sdm.scan_forward(M1, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], to_dev(x["v"]), a_d, b_d, dims)
    M2 = to_dev(M0)
    o2 = torch.empty_like(o1)
    need = sdm.sdm_scan_workspace_size(dims)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    sdm.sdm_scan_forward_gated(M2, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], to_dev(x["v"]), ar, br, Ad, dtd,
                               o2, ws, need, dims)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(o1), to_host(o2))
    assert np.array_equal(to_host(M1), to_host(M2))
    # against the oracle (gates, then the scan), the scan's bar
    a_o, b_o = oracle.gates(a_raw, b_raw, e["A"], e["dt_bias"], d)
    Mo = M0.copy()
    oo = oracle.scan(Mo, ad["widx"], ad["wwt"], ad["ridx"], ad["rwt"], x["v"], a_o, b_o, d)
    for name, got, ref in (("o", to_host(o2), oo), ("M", to_host(M2), Mo)):
        ref = ref.astype(np.float64)
        scale = float(np.sqrt(np.mean(ref ** 2)))
        err = float(np.max(np.abs(got.astype(np.float64) - ref)))
        note(f"{name}: max |err| / RMS = {err / scale:.2e}")
        assert err <= 2e-3 * scale


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d_v,B,T,H", [(32, 1, 1, 1), (64, 2, 45, 3), (96, 1, 19, 2), (128, 3, 50, 4),
                                       (256, 1, 9, 5), (1024, 1, 3, 2), (128, 2, 0, 3)])
def test_output_norm_gate_matches_oracle(sdm, torch, in_dtype, d_v, B, T, H):
    d = Dims(B=B, T=T, H=H, d_k=8, n_sub=4, d_v=d_v, k_prime=4, W=4, R=4, in_dtype=in_dtype)
    note(f"output norm gate {in_dtype} d_v={d_v} B={B} T={T} H={H}")
    x = synth.make_layer_edge_inputs(d, seed=d_v + T)
    o = x["o"]
    if o.size:
        o.reshape(-1, d_v)[0] = 0.0                 # a zero row stays zero
        if o.shape[0] * o.shape[1] * o.shape[2] > 2:
            o.reshape(-1, d_v)[1] *= 1e15           # large and tiny magnitudes
            o.reshape(-1, d_v)[2] *= 1e-15
    eps = 1e-5
    dims = sdm.dims_from(d)
    y = sdm.output_norm_gate(to_dev(o), to_dev(x["g"]), to_dev(x["gamma"]), eps, dims)
    torch.cuda.synchronize()
    check_norm(to_host(y), oracle.output_norm_gate(o, x["g"], x["gamma"], eps, d), d)


def test_output_norm_gate_eps_zero_constant_rows(sdm, torch):
    # eps = 0: a constant row normalises to +-1 exactly in exact arithmetic
    d = Dims(B=1, T=40, H=1, d_k=8, n_sub=4, d_v=128, k_prime=4, W=4, R=4, in_dtype="f32")
    note("output norm gate eps=0 constant rows")
    x = synth.make_layer_edge_inputs(d, seed=9)
    o = np.repeat(np.linspace(-3, 3, 40, dtype=np.float32)[:, None], 128, axis=1).reshape(1, 40, 1, 128)
    dims = sdm.dims_from(d)
    y = sdm.output_norm_gate(to_dev(o), to_dev(x["g"]), to_dev(x["gamma"]), 0.0, dims)
    torch.cuda.synchronize()
    check_norm(to_host(y), oracle.output_norm_gate(o, x["g"], x["gamma"], 0.0, d), d)


@pytest.mark.parametrize("name", ["small", "prefill_1p4b"])
def test_full_size_layer_edges(sdm, torch, name):
    """The benchmarked layers at full size, every element checked."""
    d = synth.PRESETS[name].dims
    note(f"layer edges full size {name} B={d.B} T={d.T} H={d.H} d_v={d.d_v}")
    x = synth.make_layer_edge_inputs(d, seed=11)
    dims = sdm.dims_from(d)
    a_d, b_d = sdm.gates(to_dev(x["a_raw"]), to_dev(x["b_raw"]), to_dev(x["A"]), to_dev(x["dt_bias"]), dims)
    y = sdm.output_norm_gate(to_dev(x["o"]), to_dev(x["g"]), to_dev(x["gamma"]), 1e-5, dims)
    torch.cuda.synchronize()
    check_gates(to_host(a_d), to_host(b_d), x["a_raw"], x["b_raw"], x["A"], x["dt_bias"], d)
    check_norm(to_host(y), oracle.output_norm_gate(x["o"], x["g"], x["gamma"], 1e-5, d), d)
