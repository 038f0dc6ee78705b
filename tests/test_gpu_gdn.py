"""GPU parity of the dense Gated DeltaNet recurrence (sdm_gdn_dense_forward)
against the oracle, and against the sparse scan with every slot selected
(the reduction of [P] Sec. 3.1 "Connection to GDN"), both on the GPU.

Bar: o and the final state within 2e-3 x RMS of the oracle's (the scan's
bar); the maximum relative error is printed for each case.
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


def gdn_dims(**kw):
    base = dict(B=2, T=50, H=3, d_k=64, n_sub=8, d_v=20, k_prime=8, W=64, R=64, in_dtype="bf16")
    base.update(kw)
    return Dims(**base)


def close_rms(got, ref, what, bar=2e-3):
    scale = float(np.sqrt(np.mean(ref.astype(np.float64) ** 2))) if ref.size else 1.0
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if ref.size else 0.0
    note(f"{what}: max |err| / RMS = {err / max(scale, 1e-30):.2e}")
    assert err <= bar * scale, f"{what}: max error {err:.3g} > {bar} x RMS {scale:.3g}"


def run_gdn(sdm, torch, x, d):
    S = to_dev(x["S0"])
    o = sdm.gdn_dense_forward(S, to_dev(x["k"]), to_dev(x["q"]), to_dev(x["v"]), to_dev(x["a"]), to_dev(x["b"]),
                              sdm.dims_from(d))
    torch.cuda.synchronize()
    return to_host(S), to_host(o)


CASES = {
    "dk16_dv1": dict(d_k=16, d_v=1, T=33),
    "dk32_dv5_f32": dict(d_k=32, d_v=5, T=40, in_dtype="f32"),
    "dk64_dv20": dict(d_k=64, d_v=20),
    "dk128_dv33": dict(d_k=128, d_v=33, T=70),
    "dk128_dv128_f32": dict(d_k=128, d_v=128, T=30, B=1, in_dtype="f32"),
    "dk256_dv16": dict(d_k=256, d_v=16, T=25, H=2),
    "dk256_dv24_f32": dict(d_k=256, d_v=24, T=9, in_dtype="f32"),
    "T1": dict(d_k=128, d_v=64, T=1),
    "T_not_multiple_of_8": dict(d_k=64, d_v=16, T=13),
}


@pytest.mark.parametrize("case", list(CASES))
def test_gdn_matches_oracle(sdm, torch, case):
    d = gdn_dims(**CASES[case])
    note(f"gdn {case} {d}")
    x = synth.make_gdn_inputs(d, seed=len(case))
    S_g, o_g = run_gdn(sdm, torch, x, d)
    S_o = x["S0"].copy()
    o_o = oracle.gdn_dense(S_o, x["k"], x["q"], x["v"], x["a"], x["b"], d)
    close_rms(o_g, o_o, f"{case} o")
    close_rms(S_g, S_o, f"{case} S")


def test_gdn_equals_sparse_scan_with_every_slot_selected(sdm, torch):
    """Both GPU paths on the same function: the scan with W = R = N = d_k = 64,
    slot lists 0..63 and the key and query as weights."""
    d = gdn_dims(B=2, T=60, H=2, d_k=64, n_sub=8, d_v=32, W=64, R=64, in_dtype="bf16")
    note(f"gdn vs sparse scan {d}")
    x = synth.make_gdn_inputs(d, seed=12)
    S_g, o_g = run_gdn(sdm, torch, x, d)
    idx = np.broadcast_to(np.arange(64, dtype=np.int32), (d.B, d.T, d.H, 64)).copy()
    wk = synth.bf16_bits_to_f32(x["k"]).astype(np.float32)
    wq = synth.bf16_bits_to_f32(x["q"]).astype(np.float32)
    M = to_dev(x["S0"])
    o_s = sdm.scan_forward(M, to_dev(idx), to_dev(wk), to_dev(idx), to_dev(wq), to_dev(x["v"]), to_dev(x["a"]),
                           to_dev(x["b"]), sdm.dims_from(d))
    torch.cuda.synchronize()
    close_rms(o_g, to_host(o_s).astype(np.float64), "gdn vs scan o", bar=1e-4)
    close_rms(S_g, to_host(M).astype(np.float64), "gdn vs scan S", bar=1e-4)


def test_gdn_empty(sdm, torch):
    d = gdn_dims(T=0)
    S = torch.randn((d.B, d.H, d.d_k, d.d_v), device="cuda")
    before = to_host(S).copy()
    e = lambda *shape, dt=torch.bfloat16: torch.empty(shape, dtype=dt, device="cuda")
    o = sdm.gdn_dense_forward(S, e(d.B, 0, d.H, d.d_k), e(d.B, 0, d.H, d.d_k), e(d.B, 0, d.H, d.d_v),
                              e(d.B, 0, d.H, dt=torch.float32), e(d.B, 0, d.H, dt=torch.float32), sdm.dims_from(d))
    torch.cuda.synchronize()
    assert o.numel() == 0 and np.array_equal(to_host(S), before)


def test_gdn_full_size_1p4b_shape(sdm, torch):
    """The dense recurrence at the 1.4B layer's shape (B=8, T=8192, H=16,
    d_k = d_v = 128), every output and state element checked."""
    base = synth.PRESETS["prefill_1p4b"].dims
    d = base.replace(n_sub=8, k_prime=8, W=64, R=64)
    note(f"gdn full size {d}")
    x = synth.make_gdn_inputs(d, seed=13)
    S_g, o_g = run_gdn(sdm, torch, x, d)
    S_o = x["S0"].copy()
    o_o = oracle.gdn_dense(S_o, x["k"], x["q"], x["v"], x["a"], x["b"], d)
    close_rms(o_g, o_o, "full o")
    close_rms(S_g, S_o, "full S")
