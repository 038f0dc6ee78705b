"""GPU parity of the scan's gradients (sdm_scan_forward_save +
sdm_scan_backward, through the C ABI) against the oracle's, and checks of
the saved rows.

Bar: every gradient (dM, dv, da, db, dw, dr) within 2e-3 x RMS of the
oracle's, the scan's own bar; the forward with saving is bit-identical to
the forward without.  Both backward paths are checked: the lane-parallel one
(with a workspace, what the training step runs) and the token-serial one
(no workspace); the lane-parallel one gives the same bits on a second run.
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


def serial_backward(sdm, dM, ad_dev, v, a, b, dout, xs, zs, dims, d, torch):
    """sdm_scan_backward without a workspace: the token-serial kernels."""
    dev = dM.device
    dv = torch.empty((d.B, d.T, d.H, d.d_v), dtype=torch.float32, device=dev)
    da = torch.empty((d.B, d.T, d.H), dtype=torch.float32, device=dev)
    db = torch.empty_like(da)
    dw = torch.empty((d.B, d.T, d.H, d.W), dtype=torch.float32, device=dev)
    dr = torch.empty((d.B, d.T, d.H, d.R), dtype=torch.float32, device=dev)
    sdm.sdm_scan_backward(dM, ad_dev["widx"], ad_dev["wwt"], ad_dev["ridx"], ad_dev["rwt"], v, a, b, dout, xs, zs,
                          dv, da, db, dw, dr, None, 0, dims)
    return dv, da, db, dw, dr


def run_case(sdm, torch, d, x, ad, seed, serial=True):
    dims = sdm.dims_from(d)
    rng = np.random.default_rng(seed)
    M0 = np.repeat(x["M0"][None], d.B, axis=0).copy()
    dout = rng.normal(0, 1, (d.B, d.T, d.H, d.d_v)).astype(np.float32)
    dMT = rng.normal(0, 1, M0.shape).astype(np.float32)
    dev = {k: to_dev(v) for k, v in ad.items()}
    M = to_dev(M0)
    o, xs, zs = sdm.scan_forward_save(M, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], to_dev(x["v"]),
                                      to_dev(x["a"]), to_dev(x["b"]), dims)
    # the forward with saving gives the forward's results bit for bit
    M2 = to_dev(M0)
    o2 = sdm.scan_forward(M2, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], to_dev(x["v"]), to_dev(x["a"]),
                          to_dev(x["b"]), dims)
    dM = to_dev(dMT)
    note(f"lane-parallel backward, workspace {sdm.sdm_scan_backward_workspace_size(dims)} bytes")
    assert sdm.sdm_scan_backward_workspace_size(dims) > 0
    grads = sdm.scan_backward(dM, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], to_dev(x["v"]),
                              to_dev(x["a"]), to_dev(x["b"]), to_dev(dout), xs, zs, dims)
    torch.cuda.synchronize()
    # a second run gives the same bits (every sum in a fixed order)
    dM2 = to_dev(dMT)
    grads2 = sdm.scan_backward(dM2, dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], to_dev(x["v"]),
                               to_dev(x["a"]), to_dev(x["b"]), to_dev(dout), xs, zs, dims)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dM), to_host(dM2))
    for g1, g2 in zip(grads, grads2):
        assert np.array_equal(to_host(g1), to_host(g2))
    dv, da, db, dw, dr = grads
    assert np.array_equal(to_host(o), to_host(o2)) and np.array_equal(to_host(M), to_host(M2))
    # o is the read weights applied to the saved read rows
    zh = to_host(zs)                                     # [B,H,T,d_v/4,R,4]
    zh = zh.transpose(0, 1, 2, 4, 3, 5).reshape(d.B, d.H, d.T, d.R, d.d_v)
    o_from_z = np.einsum("bthr,bhtrc->bthc", ad["rwt"].astype(np.float64), zh.astype(np.float64))
    close_rms(to_host(o), o_from_z, "o from zsave", bar=1e-5)
    g = oracle.scan_backward(M0, ad["widx"], ad["wwt"], ad["ridx"], ad["rwt"], x["v"], x["a"], x["b"], dout, d,
                             dM_final=dMT)
    for name, got in (("dM", dM), ("dv", dv), ("da", da), ("db", db), ("dw", dw), ("dr", dr)):
        close_rms(to_host(got), g[name], name)
    if serial:
        note("token-serial backward")
        dM3 = to_dev(dMT)
        s = serial_backward(sdm, dM3, dev, to_dev(x["v"]), to_dev(x["a"]), to_dev(x["b"]), to_dev(dout), xs, zs,
                            dims, d, torch)
        torch.cuda.synchronize()
        for name, got in zip(("dM", "dv", "da", "db", "dw", "dr"), (dM3, *s)):
            close_rms(to_host(got), g[name], name + " (token-serial)")


CASES = {
    "bf16_dv64_W16_hazards": (Dims(B=2, T=150, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=16, R=16), 40),
    "f32_dv32_W8_R5": (Dims(B=3, T=97, H=1, d_k=32, n_sub=8, d_v=32, k_prime=8, W=8, R=5, in_dtype="f32"), 20),
    "bf16_dv128_W32": (Dims(B=1, T=64, H=3, d_k=128, n_sub=32, d_v=128, k_prime=32, W=32, R=32), None),
    "bf16_dv96_W4_R12": (Dims(B=2, T=33, H=2, d_k=128, n_sub=8, d_v=96, k_prime=8, W=4, R=12), 16),
    "bf16_dv256_W64_R1": (Dims(B=1, T=20, H=2, d_k=128, n_sub=16, d_v=256, k_prime=16, W=64, R=1), 100),
    "T1": (Dims(B=5, T=1, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=16, R=16), None),
    # Q = 4 (16 sub-tokens, 8 tokens per step of the lane-parallel pass), ragged T
    "f32_dv32_W3_R4": (Dims(B=2, T=77, H=1, d_k=32, n_sub=8, d_v=32, k_prime=8, W=3, R=4, in_dtype="f32"), 12),
    # Q = 64 (one sub-token per step), W < R
    "bf16_dv64_W20_R40": (Dims(B=1, T=41, H=2, d_k=128, n_sub=16, d_v=64, k_prime=16, W=20, R=40), 90),
}


@pytest.mark.parametrize("case", list(CASES))
def test_scan_backward_matches_oracle(sdm, torch, case):
    d, pool = CASES[case]
    note(f"scan backward {case} {d}")
    x = synth.make_inputs(d, seed=17)
    ad = synth.random_addressing(d, seed=17, hazard_slots=pool)
    run_case(sdm, torch, d, x, ad, seed=3)


def test_scan_backward_repeated_read_slots(sdm, torch):
    """A read slot listed at several positions of one token (allowed: only
    write slots must be distinct) adds every position's r_i do into G; the
    lane-per-position backward merges such positions.  Every third token
    repeats position 1 at positions 3 and 7, every fifth repeats position 0
    at the last position; the slots come from a small pool, so the repeated
    rows are also written and read by nearby tokens."""
    for d in (Dims(B=2, T=120, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=16, R=16),
              Dims(B=1, T=90, H=3, d_k=128, n_sub=32, d_v=128, k_prime=32, W=32, R=32)):
        note(f"scan backward repeated read slots {d}")
        x = synth.make_inputs(d, seed=29)
        ad = synth.random_addressing(d, seed=29, hazard_slots=60)
        r = ad["ridx"]
        r[:, 0::3, :, 3] = r[:, 0::3, :, 1]
        r[:, 0::3, :, 7] = r[:, 0::3, :, 1]
        r[:, 0::5, :, d.R - 1] = r[:, 0::5, :, 0]
        assert any(len(set(r[b, t, h])) < d.R for b in range(d.B) for t in range(d.T) for h in range(d.H))
        run_case(sdm, torch, d, x, ad, seed=5)


@pytest.mark.parametrize("d", [
    Dims(B=2, T=70, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=16, R=16),             # Q = 16: 2 tokens per step
    Dims(B=1, T=60, H=2, d_k=128, n_sub=32, d_v=128, k_prime=32, W=32, R=32),           # Q = 32: 1 token per step
    Dims(B=2, T=50, H=1, d_k=32, n_sub=8, d_v=32, k_prime=4, W=4, R=4, in_dtype="f32"),  # Q = 4: 8 tokens per step
], ids=["Q16", "Q32", "Q4"])
def test_scan_backward_sub_token_dependencies(sdm, torch, d):
    """Sub-tokens of one step of the lane-parallel backward that update the
    same rows: every third token reads exactly the slots it writes (its write
    part then takes the rows its read part just updated), every fourth reads
    the slots the next token writes, every fifth writes the slots the
    previous token reads (dependencies across the two tokens of a step and
    across steps), the rest from a small pool."""
    note(f"scan backward sub-token dependencies {d}")
    x = synth.make_inputs(d, seed=41)
    ad = synth.random_addressing(d, seed=41, hazard_slots=3 * max(d.W, d.R))
    w, r = ad["widx"], ad["ridx"]
    n = min(d.W, d.R)
    r[:, 0::3, :, :n] = w[:, 0::3, :, :n]
    r[:, 0:-1:4, :, :n] = w[:, 1::4, :, :n][:, :r[:, 0:-1:4].shape[1]]
    w[:, 5::5, :, :n] = r[:, 4:-1:5, :, :n][:, :w[:, 5::5].shape[1]]
    # write slots of one token stay distinct
    for bb in range(d.B):
        for t in range(d.T):
            for h in range(d.H):
                assert len(set(w[bb, t, h])) == d.W
    run_case(sdm, torch, d, x, ad, seed=6)


def test_scan_backward_with_pkm_addressing(sdm, torch):
    """Slot lists and weights from the GPU addressing of the small layer's
    shape (T shortened)."""
    d = synth.PRESETS["small"].dims.replace(B=2, T=300)
    note(f"scan backward with PKM addressing {d}")
    x = synth.make_inputs(d, seed=23)
    widx, wwt, ridx, rwt = sdm.pkm_address(to_dev(x["k"]), to_dev(x["q"]), to_dev(x["C_w"]), to_dev(x["C_r"]),
                                           sdm.dims_from(d))
    torch.cuda.synchronize()
    ad = dict(widx=to_host(widx), wwt=to_host(wwt), ridx=to_host(ridx), rwt=to_host(rwt))
    run_case(sdm, torch, d, x, ad, seed=4)


def test_scan_backward_full_size_small_layer(sdm, torch):
    """The small layer at full size (B=4, T=4096, H=8, N=65,536, d_v=64),
    random slot lists, every gradient element checked."""
    d = synth.PRESETS["small"].dims
    note(f"scan backward full size {d}")
    x = synth.make_inputs(d, seed=29)
    ad = synth.random_addressing(d, seed=29)
    run_case(sdm, torch, d, x, ad, seed=5)


def test_scan_backward_full_size_1p4b_sampled(sdm, torch):
    """The 1.4B training shape at full size (B=8, T=8192, H=16, N=262,144,
    d_v=128, W=R=32) in the training bench's launch configuration: slot
    lists from the GPU addressing, the forward with saving, the backward for
    a random dL/do with dL/dM_T = 0.  Two sampled chains (sequence, head),
    every gradient of each, against the oracle run on that chain alone
    (chains do not interact)."""
    T = torch
    d = synth.PRESETS["prefill_1p4b"].dims
    note(f"scan backward full size 1.4B, sampled chains {d}")
    x = synth.make_inputs_torch(d, seed=31)
    dims = sdm.dims_from(d)
    widx, wwt, ridx, rwt = sdm.pkm_address(x["k"], x["q"], x["C_w"], x["C_r"], dims)
    M = sdm.state_init(x["M0"], dims)
    o, xs, zs = sdm.scan_forward_save(M, widx, wwt, ridx, rwt, x["v"], x["a"], x["b"], dims)
    del M, o
    dout = T.randn((d.B, d.T, d.H, d.d_v), generator=T.Generator(device="cuda").manual_seed(7), device="cuda")
    dM = T.zeros((d.B, d.H, d.N, d.d_v), dtype=T.float32, device="cuda")
    dv, da, db, dw, dr = sdm.scan_backward(dM, widx, wwt, ridx, rwt, x["v"], x["a"], x["b"], dout, xs, zs, dims)
    T.cuda.synchronize()
    del xs, zs
    d1 = d.replace(B=1, H=1)
    for b, h in ((0, 0), (d.B - 1, d.H - 1)):
        note(f"chain b={b} h={h}")
        sl = lambda t: to_host(t[b:b + 1, :, h:h + 1].contiguous())
        g = oracle.scan_backward(to_host(x["M0"][h:h + 1]).reshape(1, 1, d.N, d.d_v), sl(widx), sl(wwt), sl(ridx),
                                 sl(rwt), sl(x["v"]), sl(x["a"]), sl(x["b"]), sl(dout), d1)
        close_rms(to_host(dM[b:b + 1, h:h + 1]), g["dM"], f"dM[{b},{h}]")
        for name, got in (("dv", dv), ("da", da), ("db", db), ("dw", dw), ("dr", dr)):
            close_rms(sl(got), g[name], f"{name}[{b},{h}]")
