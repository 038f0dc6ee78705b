"""GPU parity of the addressing gradients (sdm_address_backward, through
the C ABI) against the oracle's, the selected slots held fixed.

Bar: dk, dq and the codebook gradients within 2e-3 x RMS of the oracle's;
a second run is bit-identical (every sum has a fixed order).
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
    ref = ref.astype(np.float64)
    scale = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 1.0
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if ref.size else 0.0
    note(f"{what}: max |err| / RMS = {err / max(scale, 1e-30):.2e}")
    assert err <= bar * scale, f"{what}: max error {err:.3g} > {bar} x RMS {scale:.3g}"


def run_case(sdm, torch, d, seed, shared, hot=0):
    """hot > 0: the first `hot` sub-keys of every half get 8x the norm, so
    most tokens select them (a few very large buckets in the sort)."""
    x = synth.make_inputs(d, seed=seed, separate_read_codebook=not shared, m0=False)
    if hot:
        for name in ("C_w", "C_r"):
            C = synth.bf16_bits_to_f32(x[name]) if d.in_dtype == "bf16" else x[name].copy()
            C[:, :, :hot] *= 8.0
            x[name] = synth.f32_to_bf16_bits(C) if d.in_dtype == "bf16" else C
    dims = sdm.dims_from(d)
    k, q, Cw, Cr = (to_dev(x[n]) for n in ("k", "q", "C_w", "C_r"))
    if shared:
        Cr = Cw
    widx, wwt, ridx, rwt = sdm.pkm_address(k, q, Cw, Cr, dims)
    rng = np.random.default_rng(seed)
    dw = rng.normal(0, 1, (d.B, d.T, d.H, d.W)).astype(np.float32)
    dr = rng.normal(0, 1, (d.B, d.T, d.H, d.R)).astype(np.float32)
    out = sdm.address_backward(k, q, Cw, Cr, widx, wwt, ridx, rwt, to_dev(dw), to_dev(dr), dims,
                               shared_codebook_grad=shared)
    out2 = sdm.address_backward(k, q, Cw, Cr, widx, wwt, ridx, rwt, to_dev(dw), to_dev(dr), dims,
                                shared_codebook_grad=shared)
    torch.cuda.synchronize()
    g = [to_host(t) for t in out]
    for a, b in zip(g, (to_host(t) for t in out2)):
        assert np.array_equal(a, b), "two runs differ"
    hw, hr = to_host(widx), to_host(ridx)
    ok, oq, oCw, oCr = oracle.address_backward(x["k"], x["q"], x["C_w"], x["C_r"] if not shared else x["C_w"], hw,
                                               to_host(wwt), hr, to_host(rwt), dw, dr, d)
    close_rms(g[0], ok, "dk")
    close_rms(g[1], oq, "dq")
    if shared:
        close_rms(g[2], oCw.astype(np.float64) + oCr, "dC (shared)")
    else:
        close_rms(g[2], oCw, "dC_w")
        close_rms(g[3], oCr, "dC_r")


CASES = {
    "bf16_small_shape": (Dims(B=2, T=100, H=3, d_k=128, n_sub=64, d_v=32, k_prime=16, W=16, R=16), False),
    "bf16_shared": (Dims(B=2, T=77, H=2, d_k=128, n_sub=32, d_v=32, k_prime=8, W=8, R=12), True),
    "f32_dk48": (Dims(B=1, T=50, H=2, d_k=48, n_sub=20, d_v=32, k_prime=6, W=5, R=3, in_dtype="f32"), False),
    "bf16_two_ranges": (Dims(B=1, T=64, H=2, d_k=128, n_sub=300, d_v=32, k_prime=32, W=32, R=32), True),
    "bf16_dk256": (Dims(B=1, T=40, H=1, d_k=256, n_sub=128, d_v=32, k_prime=64, W=64, R=1), False),
    # the dx pass in its wide form (16-byte codebook pieces): 8 pieces per row
    # (8 entry groups), one piece group per row (d_k = 512: one entry group),
    # and fp32 with 8 and 2 pieces per row
    "bf16_dk64": (Dims(B=1, T=50, H=2, d_k=64, n_sub=40, d_v=32, k_prime=16, W=16, R=9), False),
    "bf16_dk512": (Dims(B=1, T=24, H=1, d_k=512, n_sub=24, d_v=32, k_prime=8, W=8, R=8), True),
    "f32_dk32": (Dims(B=1, T=60, H=2, d_k=32, n_sub=24, d_v=32, k_prime=8, W=8, R=5, in_dtype="f32"), False),
    "f32_dk8": (Dims(B=2, T=33, H=1, d_k=8, n_sub=10, d_v=32, k_prime=4, W=4, R=7, in_dtype="f32"), True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_address_backward_matches_oracle(sdm, torch, case):
    d, shared = CASES[case]
    note(f"address backward {case} {d}")
    run_case(sdm, torch, d, seed=len(case), shared=shared)


@pytest.mark.parametrize("shared", [True, False], ids=["shared", "separate"])
def test_address_backward_hot_subkeys(sdm, torch, shared):
    d = Dims(B=2, T=600, H=2, d_k=128, n_sub=64, d_v=32, k_prime=16, W=16, R=16)
    note(f"address backward hot sub-keys {d}")
    run_case(sdm, torch, d, seed=9, shared=shared, hot=3)


def test_address_backward_full_size_1p4b(sdm, torch):
    """The 1.4B training shape at full size (B=8, T=8192, H=16, n_sub=512,
    W=R=32, one codebook for both kinds, as the training bench runs it):
    every element of dk, dq and the codebook gradient."""
    d = synth.PRESETS["prefill_1p4b"].dims
    note(f"address backward full size {d}")
    run_case(sdm, torch, d, seed=43, shared=True)


def test_address_backward_full_size_small_layer(sdm, torch):
    d = synth.PRESETS["small"].dims
    note(f"address backward full size {d}")
    run_case(sdm, torch, d, seed=41, shared=True)


def test_address_backward_unaligned_outputs(sdm, torch):
    """dk and dq 4 bytes past a 16-byte boundary (the C ABI asks only for 4):
    the dx pass then takes its element-wise form, with the same results up
    to the order of the sums."""
    d = Dims(B=2, T=70, H=2, d_k=128, n_sub=48, d_v=32, k_prime=16, W=16, R=16)
    note(f"address backward, unaligned dk/dq {d}")
    x = synth.make_inputs(d, seed=5, separate_read_codebook=True, m0=False)
    dims = sdm.dims_from(d)
    k, q, Cw, Cr = (to_dev(x[n]) for n in ("k", "q", "C_w", "C_r"))
    widx, wwt, ridx, rwt = sdm.pkm_address(k, q, Cw, Cr, dims)
    rng = np.random.default_rng(5)
    dw = rng.normal(0, 1, (d.B, d.T, d.H, d.W)).astype(np.float32)
    dr = rng.normal(0, 1, (d.B, d.T, d.H, d.R)).astype(np.float32)
    nx = d.B * d.T * d.H * d.d_k
    big = torch.zeros(2 * nx + 8, dtype=torch.float32, device="cuda")
    dk, dq = big[1:1 + nx], big[nx + 5:2 * nx + 5]     # 4 bytes past 16-byte boundaries
    assert dk.data_ptr() % 16 == 4 and dq.data_ptr() % 16 == 4
    dCw = torch.empty((d.H, 2, d.n_sub, d.d_k // 2), dtype=torch.float32, device="cuda")
    dCr = torch.empty_like(dCw)
    need = sdm.sdm_address_backward_workspace_size(dims)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    sdm.sdm_address_backward(k, q, Cw, Cr, widx, wwt, ridx, rwt, to_dev(dw), to_dev(dr), dims, dk, dq, dCw, dCr,
                             ws, need)
    torch.cuda.synchronize()
    ok, oq, _, _ = oracle.address_backward(x["k"], x["q"], x["C_w"], x["C_r"], to_host(widx), to_host(wwt),
                                           to_host(ridx), to_host(rwt), dw, dr, d)
    close_rms(to_host(dk).reshape(ok.shape), ok, "dk")
    close_rms(to_host(dq).reshape(oq.shape), oq, "dq")
