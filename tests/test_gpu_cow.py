"""GPU tests of the copy-on-write decode state (sdm_cow_reset,
sdm_decode_step_cow, sdm_cow_materialize, through the C ABI).

The copy-on-write state reads every row a sequence has not written from the
shared M0 instead of a per-sequence copy.  It must give the same slots,
outputs and written rows, bit for bit, as sdm_state_init followed by the
plain decode steps, and sdm_cow_materialize must turn it into exactly that
plain state.  The plain path is itself checked against the oracle and
against the prefill scan (test_gpu_parity); one case here compares with the
oracle directly.
"""
import numpy as np
import pytest

import oracle
import sdm_synth as synth
from sdm_synth import Dims

from gpu_helpers import compare_slot_lists, note, replay_weights, to_dev, to_host

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


def run_steps(sdm, T, d, dx, cow, steps, M=None, touched=None):
    """`steps` decode steps from M0 (plain: state init + sdm_decode_step;
    cow: bitmap reset + sdm_decode_step_cow).  Returns (outputs per step,
    M, touched)."""
    d1 = d.replace(T=1)
    dims1 = sdm.dims_from(d1)
    if M is None:
        M = T.empty((d.B, d.H, d.N, d.d_v), dtype=T.float32, device="cuda")
        if cow:
            M.fill_(float("nan"))   # rows never written must not be read from M
            touched = T.empty(sdm.sdm_cow_bitmap_bytes(dims1) // 4, dtype=T.int32, device="cuda")
            sdm.sdm_cow_reset(touched, dims1)
        else:
            sdm.state_init(dx["M0"], dims1, M=M)
    outs = []
    for t in steps:
        wo = T.empty((d.B, d.H, d.W), dtype=T.int32, device="cuda")
        ro = T.empty((d.B, d.H, d.R), dtype=T.int32, device="cuda")
        o = T.empty((d.B, d.H, d.d_v), dtype=T.float32, device="cuda")
        args = [dx[k][:, t].contiguous() for k in ("k", "q")] + [dx["C_w"], dx["C_r"]] + \
               [dx[k][:, t].contiguous() for k in ("v", "a", "b")]
        if cow:
            sdm.sdm_decode_step_cow(M, dx["M0"], touched, *args, o, wo, ro, dims1)
        else:
            sdm.sdm_decode_step(M, *args, o, wo, ro, dims1)
        outs.append((o, wo, ro))
    return outs, M, touched


def host_outs(outs):
    return [[to_host(x) for x in step] for step in outs]


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("own", [False, True], ids=["random", "reads_own_writes"])
def test_cow_decode_equals_plain(sdm, torch, in_dtype, own):
    """B = 5 (a partly filled tile of sequences), 6 steps; with q = k and one
    codebook the tokens read the rows they write, and repeated tokens
    rewrite rows written by earlier steps."""
    T = torch
    d = Dims(B=5, T=6, H=3, d_k=128, n_sub=32, d_v=96, k_prime=8, W=8, R=6, in_dtype=in_dtype)
    note(f"cow decode vs plain own={own} {d}")
    x = synth.make_inputs(d, seed=41)
    if own:
        x["C_r"] = x["C_w"].copy()
        x["q"][:, 0::2] = x["k"][:, 0::2]
        x["k"][:, 3] = x["k"][:, 1]      # token 3 writes the rows token 1 wrote
    dx = {k: to_dev(v) for k, v in x.items()}
    plain, Mp, _ = run_steps(sdm, T, d, dx, False, range(d.T))
    cow, Mc, tb = run_steps(sdm, T, d, dx, True, range(d.T))
    T.cuda.synchronize()
    hp, hc = host_outs(plain), host_outs(cow)
    for t in range(d.T):
        for i, name in enumerate(("o", "widx", "ridx")):
            np.testing.assert_array_equal(hc[t][i], hp[t][i], err_msg=f"step {t} {name}")
    # the rows written are the plain state's rows; the bitmap marks exactly them
    Mp_h, Mc_h = to_host(Mp), to_host(Mc)
    w = np.stack([s[1] for s in hp], 1)                  # [B, T, H, W]
    written = np.zeros((d.B, d.H, d.N), bool)
    for b in range(d.B):
        for h in range(d.H):
            written[b, h, np.unique(w[b, :, h])] = True
    np.testing.assert_array_equal(Mc_h[written], Mp_h[written])
    bits = np.unpackbits(to_host(tb).view(np.uint8), bitorder="little").reshape(d.B, d.H, -1)[:, :, :d.N]
    np.testing.assert_array_equal(bits.astype(bool), written)
    # made plain, the state is the plain path's, bit for bit
    sdm.sdm_cow_materialize(Mc, dx["M0"], tb, sdm.dims_from(d.replace(T=1)))
    T.cuda.synchronize()
    np.testing.assert_array_equal(to_host(Mc), Mp_h)
    assert (to_host(tb) == -1).all()


def test_cow_decode_matches_oracle(sdm, torch):
    T = torch
    d = Dims(B=3, T=4, H=2, d_k=128, n_sub=64, d_v=64, k_prime=8, W=8, R=8)
    note(f"cow decode vs oracle {d}")
    x = synth.make_inputs(d, seed=42)
    dx = {k: to_dev(v) for k, v in x.items()}
    cow, _, _ = run_steps(sdm, T, d, dx, True, range(d.T))
    T.cuda.synchronize()
    hc = host_outs(cow)
    w_dec = np.stack([s[1] for s in hc], 1)
    r_dec = np.stack([s[2] for s in hc], 1)
    o_dec = np.stack([s[0] for s in hc], 1)
    ow, oww, orr, orw = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    compare_slot_lists(w_dec, ow, x["k"], x["C_w"], d)
    compare_slot_lists(r_dec, orr, x["q"], x["C_r"], d)
    # the oracle scan replayed on the decode step's own lists (near-tie swaps included)
    Mo = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    o_ref = oracle.scan(Mo, w_dec, replay_weights(w_dec, ow, oww, x["k"], x["C_w"], d), r_dec,
                        replay_weights(r_dec, orr, orw, x["q"], x["C_r"], d), x["v"], x["a"], x["b"], d)
    err = np.max(np.abs(o_dec.astype(np.float64) - o_ref))
    scale = np.sqrt(np.mean(o_ref ** 2))
    assert err <= 1e-4 * scale, (err, scale)


def test_cow_reset_and_continue(sdm, torch):
    """Reset starts a new batch from M0 whatever M holds; materialize then
    plain steps continue exactly like plain steps all along."""
    T = torch
    d = Dims(B=2, T=6, H=2, d_k=64, n_sub=24, d_v=32, k_prime=8, W=8, R=8)
    note(f"cow reset / continue {d}")
    x = synth.make_inputs(d, seed=43)
    dx = {k: to_dev(v) for k, v in x.items()}
    dims1 = sdm.dims_from(d.replace(T=1))
    # a first batch of 3 steps, then reset and run all 6: equals a fresh run
    _, Mc, tb = run_steps(sdm, T, d, dx, True, range(3))
    sdm.sdm_cow_reset(tb, dims1)
    again, Mc, tb = run_steps(sdm, T, d, dx, True, range(d.T), M=Mc, touched=tb)
    plain, Mp, _ = run_steps(sdm, T, d, dx, False, range(d.T))
    T.cuda.synchronize()
    for a, b in zip(host_outs(again), host_outs(plain)):
        for u, v in zip(a, b):
            np.testing.assert_array_equal(u, v)
    # 3 copy-on-write steps, materialize, 3 plain steps = 6 plain steps
    first, Mc2, tb2 = run_steps(sdm, T, d, dx, True, range(3))
    sdm.sdm_cow_materialize(Mc2, dx["M0"], tb2, dims1)
    rest, Mc2, _ = run_steps(sdm, T, d, dx, False, range(3, 6), M=Mc2)
    T.cuda.synchronize()
    mixed = host_outs(first) + host_outs(rest)
    for a, b in zip(mixed, host_outs(plain)):
        for u, v in zip(a, b):
            np.testing.assert_array_equal(u, v)
    np.testing.assert_array_equal(to_host(Mc2), to_host(Mp))


def test_cow_decode_layer_shape(sdm, torch):
    """The decode layer's shape (n_sub = 1024: N = 1M slots of d_v = 128 per
    head, 8 heads, k' = W = R = 32) with 2 sequences and 8 steps: outputs
    bit-identical to the plain path, and the written rows (gathered on the
    GPU) equal."""
    T = torch
    base = synth.PRESETS["decode"].dims
    d = base.replace(B=2, T=8)
    note(f"cow decode layer shape {d}")
    x = synth.make_inputs_torch(d, seed=44)
    plain, Mp, _ = run_steps(sdm, T, d, x, False, range(d.T))
    cow, Mc, _ = run_steps(sdm, T, d, x, True, range(d.T))
    T.cuda.synchronize()
    hp, hc = host_outs(plain), host_outs(cow)
    for t in range(d.T):
        for i in range(3):
            np.testing.assert_array_equal(hc[t][i], hp[t][i], err_msg=f"step {t} output {i}")
    w = T.stack([s[1] for s in plain], 1).long()          # [B, T, H, W]
    for b in range(d.B):
        for h in range(d.H):
            rows = T.unique(w[b, :, h])
            assert T.equal(Mc[b, h, rows], Mp[b, h, rows])


@pytest.mark.parametrize("B", [64, 127], ids=["TS2", "TS4_ragged"])
def test_decode_tiled_sequences(sdm, torch, B):
    """Enough sequences that a decode workgroup takes 2 (B = 64) or 4
    (B = 127, the last tile partly filled) of them, H = 8: the plain decode
    reproduces the prefill of the same tokens bit for bit, and the
    copy-on-write decode the plain one."""
    T = torch
    d = Dims(B=B, T=3, H=8, d_k=128, n_sub=16, d_v=32, k_prime=8, W=8, R=8)
    note(f"decode with tiled sequences {d}")
    x = synth.make_inputs(d, seed=45)
    dx = {k: to_dev(v) for k, v in x.items()}
    plain, Mp, _ = run_steps(sdm, T, d, dx, False, range(d.T))
    cow, Mc, tb = run_steps(sdm, T, d, dx, True, range(d.T))
    dims = sdm.dims_from(d)
    widx, wwt, ridx, rwt = sdm.pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims)
    M2 = sdm.state_init(dx["M0"], dims)
    o2 = sdm.scan_forward(M2, widx, wwt, ridx, rwt, dx["v"], dx["a"], dx["b"], dims)
    T.cuda.synchronize()
    hp, hc = host_outs(plain), host_outs(cow)
    np.testing.assert_array_equal(np.stack([s[0] for s in hp], 1), to_host(o2))
    np.testing.assert_array_equal(np.stack([s[1] for s in hp], 1), to_host(widx))
    np.testing.assert_array_equal(np.stack([s[2] for s in hp], 1), to_host(ridx))
    np.testing.assert_array_equal(to_host(Mp), to_host(M2))
    for t in range(d.T):
        for i in range(3):
            np.testing.assert_array_equal(hc[t][i], hp[t][i], err_msg=f"step {t} output {i}")
    sdm.sdm_cow_materialize(Mc, dx["M0"], tb, sdm.dims_from(d.replace(T=1)))
    T.cuda.synchronize()
    np.testing.assert_array_equal(to_host(Mc), to_host(Mp))


@pytest.mark.parametrize("d_k,shared", [(64, False), (128, False), (256, True), (256, False)],
                         ids=["dk64_separate", "dk128_separate", "dk256_shared", "dk256_separate"])
def test_decode_scoring_routes(sdm, torch, d_k, shared):
    """The decode step's other scoring routes (separate read codebook: one
    kind at a time; d_k = 256: the generic tile): plain decode against the
    prefill of the same tokens and copy-on-write against plain, bit for bit."""
    T = torch
    d = Dims(B=3, T=3, H=2, d_k=d_k, n_sub=16, d_v=64, k_prime=8, W=8, R=6)
    note(f"decode scoring route d_k={d_k} shared={shared} {d}")
    x = synth.make_inputs(d, seed=46, separate_read_codebook=not shared)
    dx = {k: to_dev(v) for k, v in x.items()}
    plain, Mp, _ = run_steps(sdm, T, d, dx, False, range(d.T))
    cow, Mc, tb = run_steps(sdm, T, d, dx, True, range(d.T))
    dims = sdm.dims_from(d)
    widx, wwt, ridx, rwt = sdm.pkm_address(dx["k"], dx["q"], dx["C_w"], dx["C_r"], dims)
    M2 = sdm.state_init(dx["M0"], dims)
    o2 = sdm.scan_forward(M2, widx, wwt, ridx, rwt, dx["v"], dx["a"], dx["b"], dims)
    T.cuda.synchronize()
    hp, hc = host_outs(plain), host_outs(cow)
    np.testing.assert_array_equal(np.stack([s[1] for s in hp], 1), to_host(widx))
    np.testing.assert_array_equal(np.stack([s[2] for s in hp], 1), to_host(ridx))
    np.testing.assert_array_equal(np.stack([s[0] for s in hp], 1), to_host(o2))
    np.testing.assert_array_equal(to_host(Mp), to_host(M2))
    for t in range(d.T):
        for i in range(3):
            np.testing.assert_array_equal(hc[t][i], hp[t][i], err_msg=f"step {t} output {i}")
