"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle
on the same seeded inputs.

Bars: slot indices bit-exact except oracle near-ties (score gap < 1e-5);
weights within 1e-6 where the lists agree; o and the written rows of M within
2e-3 x RMS of the oracle's; rows never written bit-identical to M0.
"""
import numpy as np
import pytest

import oracle
import sdm_synth as synth
from sdm_synth import Dims

from gpu_helpers import (assert_close_rms, check_weights, compare_slot_lists, gpu_dims, note, replay_weights,
                         to_dev, to_host, written_mask)

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


def run_address(sdm, torch, x, d):
    dims = gpu_dims(d)
    out = sdm.pkm_address(to_dev(x["k"]), to_dev(x["q"]), to_dev(x["C_w"]), to_dev(x["C_r"]), dims)
    torch.cuda.synchronize()
    return [to_host(t) for t in out]


def check_address(x, d, gpu, max_tie_frac=0.01):
    gw, gww, gr, grw = gpu
    ow, oww, orr, orw = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    rw_diff, nw = compare_slot_lists(gw, ow, x["k"], x["C_w"], d)
    rr_diff, nr = compare_slot_lists(gr, orr, x["q"], x["C_r"], d)
    rows = rw_diff.size
    assert rw_diff.sum() <= max_tie_frac * rows + 1, f"{rw_diff.sum()} of {rows} write lists differ"
    assert rr_diff.sum() <= max_tie_frac * rows + 1, f"{rr_diff.sum()} of {rows} read lists differ"
    # every row's weights, near-tie rows against the oracle's softmax over the GPU's own list
    check_weights(gw, gww, ow, oww, x["k"], x["C_w"], d)
    check_weights(gr, grw, orr, orw, x["q"], x["C_r"], d)
    return (ow, oww, orr, orw), (rw_diff.reshape(gww.shape[:-1]), rr_diff.reshape(grw.shape[:-1]))


# ---------------------------------------------------------------------------
def test_state_init_bit_exact(sdm, torch):
    d = Dims(B=3, T=1, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=8, R=8)
    note("state_init B=3 H=2 N=256 d_v=64")
    M0 = np.random.default_rng(0).standard_normal((d.H, d.N, d.d_v)).astype(np.float32)
    M = sdm.state_init(to_dev(M0), gpu_dims(d))
    torch.cuda.synchronize()
    got = to_host(M)
    for b in range(d.B):
        np.testing.assert_array_equal(got[b], M0)


ADDRESS_CASES = {
    "tiny_full": (synth.PRESETS["tiny"].dims, {}),
    "small_T61": (synth.PRESETS["small"].dims.replace(B=1, T=61, H=3), {}),
    "prefill_T45": (synth.PRESETS["prefill_1p4b"].dims.replace(B=2, T=23, H=2), {}),
    "decode_dims": (synth.PRESETS["decode"].dims.replace(B=1, T=17, H=2), {}),
    "sep_codebook": (Dims(B=2, T=19, H=3, d_k=64, n_sub=40, d_v=32, k_prime=12, W=9, R=30), dict(sep=True)),
    "kprime_below_W": (Dims(B=1, T=33, H=2, d_k=128, n_sub=64, d_v=32, k_prime=5, W=20, R=25), {}),
    "fp32_wide": (Dims(B=1, T=40, H=2, d_k=24, n_sub=50, d_v=32, k_prime=10, W=7, R=3, in_dtype="f32"), {}),
    # 1024 sub-keys per half: the two-part selection, with k' below 32 and
    # below W (the PKM approximation), and separate codebooks
    "split_kp16_W20": (Dims(B=1, T=33, H=2, d_k=128, n_sub=1024, d_v=32, k_prime=16, W=20, R=9), {}),
    "split_kp5_sep": (Dims(B=2, T=21, H=1, d_k=128, n_sub=1024, d_v=32, k_prime=5, W=3, R=25), dict(sep=True)),
}


@pytest.mark.parametrize("case", list(ADDRESS_CASES))
def test_address_parity(sdm, torch, case):
    d, opt = ADDRESS_CASES[case]
    note(f"address {case} {d}")
    x = synth.make_inputs(d, seed=101, m0=False, separate_read_codebook=opt.get("sep", False))
    check_address(x, d, run_address(sdm, torch, x, d))


def test_address_identity_codebook_bit_exact(sdm, torch):
    """C = I: the half scores are the bf16 inputs exactly, so the lists (ties
    included, broken to the lower index) must match bit for bit."""
    d = Dims(B=2, T=30, H=2, d_k=128, n_sub=64, d_v=32, k_prime=16, W=16, R=5)
    note("address identity codebook")
    x = synth.make_inputs(d, seed=7, m0=False)
    eye = synth.f32_to_bf16_bits(np.broadcast_to(np.eye(64, dtype=np.float32), (d.H, 2, 64, 64)).copy())
    # coarse inputs so that many scores tie exactly
    for kk in ("k", "q"):
        f = synth.bf16_bits_to_f32(x[kk])
        x[kk] = synth.f32_to_bf16_bits(np.round(f * 4) / 4)
    x["C_w"] = x["C_r"] = eye
    gw, gww, gr, grw = run_address(sdm, torch, x, d)
    ow, oww, orr, orw = oracle.address(x["k"], x["q"], eye, eye, d)
    np.testing.assert_array_equal(gw, ow)
    np.testing.assert_array_equal(gr, orr)
    np.testing.assert_allclose(gww, oww, rtol=0, atol=1e-6)
    np.testing.assert_allclose(grw, orw, rtol=0, atol=1e-6)


@pytest.mark.parametrize("n_sub,kp", [(1024, 32), (512, 32), (1024, 12), (2048, 32), (1536, 20)])
def test_address_integer_scores_bit_exact(sdm, torch, n_sub, kp):
    """Codebook and inputs in {-1, 0, 1}: every half score is a small integer,
    exact in fp32 whatever the summation order, so scores tie very often and
    the lists (ties to the lower index, at both levels) must equal the
    oracle's bit for bit.  n_sub = 1024, 1536 and 2048 exercise the selection
    of each half in two, three and four parts of 512 sub-keys and their
    merges; 512 the one-part form."""
    d = Dims(B=1, T=40, H=2, d_k=128, n_sub=n_sub, d_v=32, k_prime=kp, W=32, R=kp)
    note(f"address integer scores n_sub={n_sub} k'={kp}")
    g = np.random.default_rng(11)
    tern = lambda shape: synth.f32_to_bf16_bits(g.integers(-1, 2, size=shape).astype(np.float32))
    x = {"k": tern((d.B, d.T, d.H, d.d_k)), "q": tern((d.B, d.T, d.H, d.d_k))}
    x["C_w"] = x["C_r"] = tern((d.H, 2, d.n_sub, d.d_k // 2))
    gw, gww, gr, grw = run_address(sdm, torch, x, d)
    ow, oww, orr, orw = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    np.testing.assert_array_equal(gw, ow)
    np.testing.assert_array_equal(gr, orr)
    np.testing.assert_allclose(gww, oww, rtol=0, atol=1e-6)
    np.testing.assert_allclose(grw, orw, rtol=0, atol=1e-6)


# ---------------------------------------------------------------------------
SCAN_CASES = {
    # name: (dims, hazard slot pool or None)
    "f32_dv32_W4": (Dims(B=1, T=256, H=1, d_k=32, n_sub=32, d_v=32, k_prime=4, W=4, R=4, in_dtype="f32"), 64),
    "bf16_dv64_W16": (Dims(B=2, T=300, H=3, d_k=128, n_sub=64, d_v=64, k_prime=16, W=16, R=16), 200),
    "bf16_dv128_W32": (Dims(B=2, T=129, H=2, d_k=128, n_sub=128, d_v=128, k_prime=32, W=32, R=32), 300),
    "ragged_lists": (Dims(B=3, T=77, H=1, d_k=128, n_sub=32, d_v=96, k_prime=8, W=5, R=3), 40),
    "W64_R1": (Dims(B=1, T=50, H=2, d_k=128, n_sub=64, d_v=32, k_prime=8, W=64, R=1), 500),
    "no_hazard_pool": (Dims(B=2, T=200, H=2, d_k=128, n_sub=256, d_v=64, k_prime=16, W=16, R=16), None),
    "W8_R8_f32": (Dims(B=2, T=90, H=2, d_k=32, n_sub=16, d_v=64, k_prime=8, W=8, R=8, in_dtype="f32"), 60),
    "W64_R64": (Dims(B=1, T=70, H=2, d_k=128, n_sub=64, d_v=64, k_prime=8, W=64, R=64), 400),
    "W32_T1": (Dims(B=3, T=1, H=2, d_k=128, n_sub=64, d_v=128, k_prime=32, W=32, R=32), None),
    "W32_T17_dv32": (Dims(B=2, T=17, H=1, d_k=128, n_sub=64, d_v=32, k_prime=32, W=32, R=32), 100),
    # moderate collision rates: steps of concurrent tokens mixed with steps
    # whose tokens depend on each other, and reads of the token's own writes
    "mixed_W16": (Dims(B=5, T=500, H=2, d_k=128, n_sub=64, d_v=64, k_prime=16, W=16, R=16), 3000),
    "mixed_W32": (Dims(B=3, T=300, H=3, d_k=128, n_sub=128, d_v=128, k_prime=32, W=32, R=32), 6000),
    "mixed_W4_K16": (Dims(B=9, T=700, H=1, d_k=32, n_sub=32, d_v=32, k_prime=4, W=4, R=4, in_dtype="f32"), 300),
    "mixed_W12_R7": (Dims(B=2, T=333, H=5, d_k=128, n_sub=64, d_v=160, k_prime=8, W=12, R=7), 1500),
    # B*H*d_v/4 column chunks select the workgroup shape of the scan: >= 4096
    # (8 waves per workgroup, depth 2), >= 2048 (8 waves, depth 4), >= 1024
    # (4 waves, depth 4); the cases above run 2 waves per workgroup, depth 4
    "shape_g8_d2": (Dims(B=4, T=45, H=8, d_k=128, n_sub=16, d_v=512, k_prime=16, W=32, R=32), 120),
    "shape_g8_d4": (Dims(B=2, T=70, H=8, d_k=128, n_sub=16, d_v=512, k_prime=16, W=16, R=16), 100),
    "shape_g4_d4": (Dims(B=2, T=90, H=4, d_k=128, n_sub=32, d_v=512, k_prime=8, W=8, R=8), 200),
    "shape_g8_d4_f32": (Dims(B=2, T=70, H=8, d_k=32, n_sub=16, d_v=512, k_prime=8, W=8, R=8, in_dtype="f32"), 100),
    "shape_g8_d2_f32": (Dims(B=4, T=40, H=8, d_k=32, n_sub=16, d_v=512, k_prime=4, W=4, R=3, in_dtype="f32"), 50),
}


def run_scan(sdm, torch, d, x, ad, M0_full=None):
    dims = gpu_dims(d)
    M = to_dev(M0_full if M0_full is not None else np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy())
    o = sdm.scan_forward(M, to_dev(ad["widx"]), to_dev(ad["wwt"]), to_dev(ad["ridx"]), to_dev(ad["rwt"]),
                         to_dev(x["v"]), to_dev(x["a"]), to_dev(x["b"]), dims)
    torch.cuda.synchronize()
    return to_host(o), to_host(M)


def check_scan(d, x, ad, o_gpu, M_gpu):
    M = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    M0 = M.copy()
    o_ref = oracle.scan(M, ad["widx"], ad["wwt"], ad["ridx"], ad["rwt"], x["v"], x["a"], x["b"], d)
    assert_close_rms(o_gpu, o_ref, what="o")
    wm = written_mask(ad["widx"], d)
    assert_close_rms(M_gpu[wm], M[wm], what="M written rows")
    np.testing.assert_array_equal(M_gpu[~wm], M0[~wm])


@pytest.mark.parametrize("case", list(SCAN_CASES))
def test_scan_parity(sdm, torch, case):
    d, pool = SCAN_CASES[case]
    note(f"scan {case} {d} pool={pool}")
    x = synth.make_inputs(d, seed=202)
    ad = synth.random_addressing(d, seed=202, hazard_slots=pool)
    o, M = run_scan(sdm, torch, d, x, ad)
    check_scan(d, x, ad, o, M)


def test_scan_memory_above_1gib(sdm, torch):
    """One (sequence, head) memory of 1.125 GiB (n_sub = 1536, d_v = 128):
    rows at byte offsets past 1 GiB are gathered, updated and stored, and
    writes superseded within the pipeline window are dropped, exactly as
    below 1 GiB.  Half of the slots of a frequently colliding pool are moved
    past 2^21 (row offset >= 1 GiB), so both ranges and their hazards mix."""
    d = Dims(B=1, T=300, H=1, d_k=128, n_sub=1536, d_v=128, k_prime=32, W=32, R=32)
    assert d.N * d.d_v * 4 >= (1 << 30) + (1 << 27)
    note(f"scan memory above 1 GiB {d}")
    x = synth.make_inputs(d.replace(n_sub=4), seed=211, m0=False)
    g = np.random.default_rng(211)
    x["M0"] = (g.standard_normal((d.H, d.N, d.d_v), dtype=np.float32) * np.float32(np.sqrt(0.02)))
    ad = synth.random_addressing(d, seed=211, hazard_slots=2000)
    base = d.N - 4096
    for key in ("widx", "ridx"):
        sl = ad[key]
        ad[key] = np.where(sl % 2 == 0, sl + base, sl).astype(np.int32)
    assert (ad["widx"] >= (1 << 21)).mean() > 0.4
    o, M = run_scan(sdm, torch, d, x, ad)
    check_scan(d, x, ad, o, M)


def test_scan_b_zero_decay_bit_exact(sdm, torch):
    d = Dims(B=2, T=60, H=2, d_k=128, n_sub=8, d_v=64, k_prime=8, W=6, R=4)
    note("scan b=0")
    x = synth.make_inputs(d, seed=5)
    ad = synth.random_addressing(d, seed=5, hazard_slots=20)
    x["b"] = np.zeros_like(x["b"])
    _, M = run_scan(sdm, torch, d, x, ad)
    ref = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    for b in range(d.B):
        for h in range(d.H):
            for t in range(d.T):
                for s in ad["widx"][b, t, h]:
                    ref[b, h, s] = np.float32(x["a"][b, t, h]) * ref[b, h, s]
    np.testing.assert_array_equal(M, ref)


def test_scan_write_then_read_exact(sdm, torch):
    """a = b = 1, W = R = 1, read slot = write slot: o_t = v_t exactly on
    dyadic data (every fp32 operation is exact)."""
    d = Dims(B=2, T=64, H=2, d_k=32, n_sub=8, d_v=32, k_prime=4, W=1, R=1, in_dtype="f32")
    note("scan write-then-read")
    g = np.random.default_rng(3)
    x = synth.make_inputs(d, seed=3)
    x["M0"] = (g.integers(-1000, 1000, x["M0"].shape) / 256).astype(np.float32)
    x["v"] = (g.integers(-1000, 1000, x["v"].shape) / 256).astype(np.float32)
    x["a"] = np.ones_like(x["a"])
    x["b"] = np.ones_like(x["b"])
    slots = g.integers(0, 12, (d.B, d.T, d.H, 1)).astype(np.int32)
    ad = dict(widx=slots, ridx=slots.copy(), wwt=np.ones((d.B, d.T, d.H, 1), np.float32),
              rwt=np.ones((d.B, d.T, d.H, 1), np.float32))
    o, _ = run_scan(sdm, torch, d, x, ad)
    np.testing.assert_array_equal(o, x["v"])


def test_scan_hazard_closed_form(sdm, torch):
    """Same slots and weights for every token, r = w: per column
    p_{n+1} = a p_n + b |w|^2 (v - a p_n) and o_n = p_{n+1}."""
    d = Dims(B=1, T=200, H=1, d_k=128, n_sub=16, d_v=64, k_prime=8, W=8, R=8)
    note("scan hazard closed form")
    x = synth.make_inputs(d, seed=9)
    g = np.random.default_rng(9)
    slots = g.permutation(d.N)[:d.W].astype(np.int32)
    w = g.random(d.W) + 0.1
    w = (w / w.sum()).astype(np.float32)
    widx = np.broadcast_to(slots, (1, d.T, 1, d.W)).copy()
    wwt = np.broadcast_to(w, (1, d.T, 1, d.W)).copy()
    ad = dict(widx=widx, wwt=wwt, ridx=widx.copy(), rwt=wwt.copy())
    o, _ = run_scan(sdm, torch, d, x, ad)
    p = (w.astype(np.float64)[:, None] * x["M0"][0, slots].astype(np.float64)).sum(0)
    w2 = float((w.astype(np.float64) ** 2).sum())
    vf = synth.bf16_bits_to_f32(x["v"]).astype(np.float64)
    ref = []
    for t in range(d.T):
        at, bt = float(x["a"][0, t, 0]), float(x["b"][0, t, 0])
        p = at * p + bt * w2 * (vf[0, t, 0] - at * p)
        ref.append(p.copy())
    ref = np.array(ref)
    np.testing.assert_allclose(o[0, :, 0], ref, rtol=0, atol=1e-5 * np.abs(ref).max())


def test_scan_split_and_determinism(sdm, torch):
    d = Dims(B=2, T=150, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=8, R=8)
    note("scan split + determinism")
    x = synth.make_inputs(d, seed=12)
    ad = synth.random_addressing(d, seed=12, hazard_slots=40)
    o_full, M_full = run_scan(sdm, torch, d, x, ad)
    o_again, M_again = run_scan(sdm, torch, d, x, ad)
    np.testing.assert_array_equal(o_full, o_again)
    np.testing.assert_array_equal(M_full, M_again)
    T1 = 61
    M = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    outs = []
    for lo, hi in ((0, T1), (T1, d.T)):
        dd = d.replace(T=hi - lo)
        sl = lambda z: np.ascontiguousarray(z[:, lo:hi])
        o, M = run_scan(sdm, torch, dd, {**x, "v": sl(x["v"]), "a": sl(x["a"]), "b": sl(x["b"])},
                        {k: sl(v) for k, v in ad.items()}, M0_full=M)
        outs.append(o)
    np.testing.assert_array_equal(np.concatenate(outs, 1), o_full)
    np.testing.assert_array_equal(M, M_full)


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "small_sub"])
def test_end_to_end_prefill(sdm, torch, name):
    if name == "tiny":
        d = synth.PRESETS["tiny"].dims
    else:
        d = synth.PRESETS["small"].dims.replace(B=2, T=256, H=3)
    note(f"end-to-end {name} {d}")
    x = synth.make_inputs(d, seed=0)
    dims = gpu_dims(d)
    dx = {k: to_dev(v) for k, v in x.items()}
    widx, wwt, ridx, rwt = sdm.pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims)
    M = sdm.state_init(dx["M0"], dims)
    o = sdm.scan_forward(M, widx, wwt, ridx, rwt, dx["v"], dx["a"], dx["b"], dims)
    torch.cuda.synchronize()
    gpu = [to_host(t) for t in (widx, wwt, ridx, rwt)]
    check_address(x, d, gpu)
    # the oracle scan on the GPU's own (validated) lists, with the oracle's
    # weights for them, so a near-tie swap does not end the comparison
    gw, _, gr, _ = gpu
    ow, oww, orr, orw = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    ww = replay_weights(gw, ow, oww, x["k"], x["C_w"], d)
    rw = replay_weights(gr, orr, orw, x["q"], x["C_r"], d)
    Mo = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    o_ref = oracle.scan(Mo, gw, ww, gr, rw, x["v"], x["a"], x["b"], d)
    o_gpu, M_gpu = to_host(o), to_host(M)
    assert_close_rms(o_gpu, o_ref, what="o")
    wm = written_mask(gw, d)
    assert_close_rms(M_gpu[wm], Mo[wm], what="M written rows")
    M0b = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape)
    np.testing.assert_array_equal(M_gpu[~wm], M0b[~wm])


def _full_path(sdm, torch, d, x):
    """Addressing, state init and prefill scan of host inputs x; host outputs."""
    dims = gpu_dims(d)
    dx = {k: to_dev(v) for k, v in x.items()}
    lists = sdm.pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims)
    M = sdm.state_init(dx["M0"], dims)
    o = sdm.scan_forward(M, *lists, dx["v"], dx["a"], dx["b"], dims)
    torch.cuda.synchronize()
    return [to_host(t) for t in lists], to_host(o), to_host(M)


def test_gpu_power_of_two_homogeneity_bit_exact(sdm, torch):
    """Scaling M0 and v by 2 scales o and M by 2 exactly (every operation of
    the update is exact under a power-of-two scale); the slots do not move."""
    d = Dims(B=2, T=150, H=2, d_k=128, n_sub=32, d_v=64, k_prime=8, W=8, R=8)
    note(f"homogeneity {d}")
    x = synth.make_inputs(d, seed=41)
    x2 = dict(x)
    x2["M0"] = x["M0"] * np.float32(2)
    x2["v"] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(x["v"]) * np.float32(2))
    l1, o1, M1 = _full_path(sdm, torch, d, x)
    l2, o2, M2 = _full_path(sdm, torch, d, x2)
    for a, b in zip(l1, l2):
        np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(o2, o1 * np.float32(2))
    np.testing.assert_array_equal(M2, M1 * np.float32(2))


def test_gpu_permuting_sequences_permutes_outputs(sdm, torch):
    """Sequences are independent: permuting the batch permutes every output
    bit for bit (addressing tiles mix sequences, but each score depends only
    on its own row)."""
    d = Dims(B=5, T=37, H=3, d_k=128, n_sub=32, d_v=32, k_prime=8, W=8, R=5)
    note(f"permutation {d}")
    x = synth.make_inputs(d, seed=42)
    perm = np.array([3, 0, 4, 2, 1])
    xp = dict(x)
    for k in ("k", "q", "v", "a", "b"):
        xp[k] = np.ascontiguousarray(x[k][perm])
    l1, o1, M1 = _full_path(sdm, torch, d, x)
    l2, o2, M2 = _full_path(sdm, torch, d, xp)
    for a, b in zip(l1, l2):
        np.testing.assert_array_equal(b, a[perm])
    np.testing.assert_array_equal(o2, o1[perm])
    np.testing.assert_array_equal(M2, M1[perm])


def test_gpu_superposition(sdm, torch):
    """For fixed slots, weights and gates the scan is linear in (M0, v):
    scan(M0, v) = scan(M0, 0) + scan(0, v) within the o/M tolerance."""
    d = Dims(B=2, T=120, H=2, d_k=128, n_sub=32, d_v=64, k_prime=8, W=8, R=8)
    note(f"superposition {d}")
    x = synth.make_inputs(d, seed=43)
    ad = synth.random_addressing(d, seed=43, hazard_slots=100)
    zero_v = synth.f32_to_bf16_bits(np.zeros(x["v"].shape, np.float32))
    M0b = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    o_full, M_full = run_scan(sdm, torch, d, x, ad, M0b)
    o_m, M_m = run_scan(sdm, torch, d, dict(x, v=zero_v), ad, M0b)
    o_v, M_v = run_scan(sdm, torch, d, x, ad, np.zeros_like(M0b))
    assert_close_rms(o_m + o_v, o_full, what="o superposition")
    assert_close_rms(M_m + M_v, M_full, what="M superposition")


def test_decode_reads_own_writes(sdm, torch):
    """Tokens whose read slots are their own write slots (q = k with one
    shared codebook): the read must see the new rows.  B = 5 also leaves a
    partly filled tile of sequences.  Against the oracle and, bit for bit,
    against the prefill of the same tokens."""
    d = Dims(B=5, T=4, H=3, d_k=128, n_sub=32, d_v=96, k_prime=8, W=8, R=6)
    note(f"decode own writes {d}")
    x = synth.make_inputs(d, seed=34)
    x["C_r"] = x["C_w"].copy()
    x["q"][:, 0::2] = x["k"][:, 0::2]
    d1 = d.replace(T=1)
    dims1 = gpu_dims(d1)
    dx = {k: to_dev(v) for k, v in x.items()}
    M = sdm.state_init(dx["M0"], dims1)
    outs, widxs, ridxs = [], [], []
    import torch as T
    for t in range(d.T):
        wo = T.empty((d.B, d.H, d.W), dtype=T.int32, device="cuda")
        ro = T.empty((d.B, d.H, d.R), dtype=T.int32, device="cuda")
        args = [dx[k][:, t].contiguous() for k in ("k", "q")]
        rest = [dx[k][:, t].contiguous() for k in ("v", "a", "b")]
        outs.append(sdm.decode_step(M, *args, dx["C_w"], dx["C_r"], *rest, dims1, widx_out=wo, ridx_out=ro))
        widxs.append(wo)
        ridxs.append(ro)
    T.cuda.synchronize()
    o_dec = np.stack([to_host(o) for o in outs], 1)
    w_dec = np.stack([to_host(w) for w in widxs], 1)
    r_dec = np.stack([to_host(r) for r in ridxs], 1)
    # every even token reads R of its own W write slots
    assert all(np.isin(r_dec[b, t, h], w_dec[b, t, h]).all()
               for b in range(d.B) for t in range(0, d.T, 2) for h in range(d.H))
    ow, oww, orr, orw = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    compare_slot_lists(w_dec, ow, x["k"], x["C_w"], d)
    compare_slot_lists(r_dec, orr, x["q"], x["C_r"], d)
    # the oracle scan replayed on the decode step's own lists
    Mo = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    o_ref = oracle.scan(Mo, w_dec, replay_weights(w_dec, ow, oww, x["k"], x["C_w"], d), r_dec,
                        replay_weights(r_dec, orr, orw, x["q"], x["C_r"], d), x["v"], x["a"], x["b"], d)
    assert_close_rms(o_dec, o_ref, what="decode o")
    dims = gpu_dims(d)
    widx, wwt, ridx, rwt = sdm.pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims)
    M2 = sdm.state_init(dx["M0"], dims)
    o2 = sdm.scan_forward(M2, widx, wwt, ridx, rwt, dx["v"], dx["a"], dx["b"], dims)
    T.cuda.synchronize()
    np.testing.assert_array_equal(w_dec, to_host(widx))
    np.testing.assert_array_equal(r_dec, to_host(ridx))
    np.testing.assert_array_equal(o_dec, to_host(o2))
    np.testing.assert_array_equal(to_host(M), to_host(M2))


def test_decode_matches_oracle_and_prefill(sdm, torch):
    d = Dims(B=4, T=6, H=2, d_k=128, n_sub=64, d_v=64, k_prime=8, W=8, R=8)
    note(f"decode {d}")
    x = synth.make_inputs(d, seed=33)
    d1 = d.replace(T=1)
    dims1 = gpu_dims(d1)
    dx = {k: to_dev(v) for k, v in x.items()}
    M = sdm.state_init(dx["M0"], dims1)
    Mo = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    outs, widxs, ridxs = [], [], []
    import torch as T
    for t in range(d.T):
        wo = T.empty((d.B, d.H, d.W), dtype=T.int32, device="cuda")
        ro = T.empty((d.B, d.H, d.R), dtype=T.int32, device="cuda")
        k = dx["k"][:, t].contiguous()
        q = dx["q"][:, t].contiguous()
        v = dx["v"][:, t].contiguous()
        a = dx["a"][:, t].contiguous()
        b = dx["b"][:, t].contiguous()
        o = sdm.decode_step(M, k, q, dx["C_w"], dx["C_r"], v, a, b, dims1, widx_out=wo, ridx_out=ro)
        outs.append(o)
        widxs.append(wo)
        ridxs.append(ro)
    T.cuda.synchronize()
    o_dec = np.stack([to_host(o) for o in outs], 1)
    w_dec = np.stack([to_host(w) for w in widxs], 1)
    r_dec = np.stack([to_host(r) for r in ridxs], 1)
    M_dec = to_host(M)
    # against the oracle (decode = addressing + one scan step per token)
    ow, oww, orr, orw = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    compare_slot_lists(w_dec, ow, x["k"], x["C_w"], d)
    compare_slot_lists(r_dec, orr, x["q"], x["C_r"], d)
    # the oracle scan replayed on the decode step's own lists
    o_ref = oracle.scan(Mo, w_dec, replay_weights(w_dec, ow, oww, x["k"], x["C_w"], d), r_dec,
                        replay_weights(r_dec, orr, orw, x["q"], x["C_r"], d), x["v"], x["a"], x["b"], d)
    assert_close_rms(o_dec, o_ref, what="decode o")
    wm = written_mask(w_dec, d)
    assert_close_rms(M_dec[wm], Mo[wm], what="decode M")
    np.testing.assert_array_equal(M_dec[~wm], np.broadcast_to(x["M0"][None], M_dec.shape)[~wm])
    # against the GPU prefill of the same tokens: bit-identical
    dims = gpu_dims(d)
    widx, wwt, ridx, rwt = sdm.pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims)
    M2 = sdm.state_init(dx["M0"], dims)
    o2 = sdm.scan_forward(M2, widx, wwt, ridx, rwt, dx["v"], dx["a"], dx["b"], dims)
    T.cuda.synchronize()
    np.testing.assert_array_equal(w_dec, to_host(widx))
    np.testing.assert_array_equal(r_dec, to_host(ridx))
    np.testing.assert_array_equal(o_dec, to_host(o2))
    np.testing.assert_array_equal(M_dec, to_host(M2))


def test_empty_inputs_touch_nothing(sdm, torch):
    """No tokens (T = 0) or no sequences (B = 0): every call succeeds on the
    empty tensors and leaves the state as it was, bit for bit."""
    d = Dims(B=2, T=0, H=3, d_k=128, n_sub=16, d_v=32, k_prime=8, W=8, R=8)
    note(f"empty inputs {d}")
    T = torch
    dims = gpu_dims(d)
    M = T.randn((d.B, d.H, d.N, d.d_v), dtype=T.float32, device="cuda")
    M_before = to_host(M).copy()
    x = synth.make_inputs(d.replace(T=1), seed=3)
    e = lambda *shape, dt=T.float32: T.empty(shape, dtype=dt, device="cuda")
    k = e(d.B, 0, d.H, d.d_k, dt=T.bfloat16)
    widx, wwt, ridx, rwt = sdm.pkm_address(k, k, to_dev(x["C_w"]), to_dev(x["C_r"]), dims)
    assert widx.numel() == 0 and rwt.numel() == 0
    o = sdm.scan_forward(M, widx, wwt, ridx, rwt, e(d.B, 0, d.H, d.d_v, dt=T.bfloat16), e(d.B, 0, d.H),
                         e(d.B, 0, d.H), dims)
    assert o.numel() == 0
    a, b = sdm.gates(e(d.B, 0, d.H), e(d.B, 0, d.H), to_dev(np.ones(d.H, np.float32)),
                     to_dev(np.zeros(d.H, np.float32)), dims)
    y = sdm.output_norm_gate(o, e(d.B, 0, d.H, d.d_v, dt=T.bfloat16), to_dev(np.ones(d.d_v, np.float32)), 1e-5,
                             dims)
    d0 = d.replace(B=0, T=1)
    dims0 = gpu_dims(d0)
    M0 = to_dev(x["M0"])
    sdm.state_init(M0, dims0, M=e(0, d.H, d.N, d.d_v))
    sdm.decode_step(e(0, d.H, d.N, d.d_v), e(0, d.H, d.d_k, dt=T.bfloat16), e(0, d.H, d.d_k, dt=T.bfloat16),
                    to_dev(x["C_w"]), to_dev(x["C_r"]), e(0, d.H, d.d_v, dt=T.bfloat16), e(0, d.H), e(0, d.H), dims0)
    T.cuda.synchronize()
    assert np.array_equal(to_host(M), M_before)
    assert a.numel() == 0 and y.numel() == 0
