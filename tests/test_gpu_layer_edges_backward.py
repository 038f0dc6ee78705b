"""GPU parity of the gradients of the steps either side of the path, through
the C ABI: sdm_gates_backward and sdm_output_norm_gate_backward, element by
element against the oracle (whose values are the exact ones rounded once to
fp32).

Tolerances follow from the fp32 arithmetic of the kernels (u = 2^-24); the
magnitudes they scale are computed here in float64 from the inputs.
  gates: a carries the forward's relative error e_a = A |z| 2u + (|ln a| + 1) 8u
    (z = a_raw + dt_bias, rounded once); sigmoid(z) adds |z| u (the rounding
    of z) and a few u; the products a few u more:
      da_raw: |err| <= (e_a + |z| u + 16u) |da_raw|
      db_raw = db e / (1 + e)^2, e = exp(-|b_raw|): |err| <= 12u |db_raw|
    dA and ddt_bias are sums over the B*T tokens of terms with the relative
    error above (for dA: e_a + |z| u + 16u as well, softplus included), taken
    as at most 512 parts (each a chain of its tokens), then 2-term chains
    and an 8-level tree: |err| <= (e_term + (B*T/parts + 12) u) * sum |term|
    (parts >= 1: bounded by B*T + 12).
  norm: with inv = 1/sqrt(mean(o^2) + eps) (relative error e_i =
    ((d_v/8 + 3)/2 + 4) u: a d_v/8-term chain and a 3-level butterfly of
    squares, the mean, sqrt, reciprocal), n = o inv, s = sigmoid(g),
    q = dy gamma g s and P = sum_c |q n| per row:
      do = inv (q - n <q, n>/d_v): every rounding is a multiple of u times
        inv |q| or inv |n| P / d_v, at most (d_v/8 + 40) of them:
        |err| <= (d_v/8 + 40) u inv (|q| + |n| P / d_v)
      dg = dy gamma n s (1 + g (1 - s)): the bracket may cancel (g near -1.28),
        so its absolute error |g| (4s + 2) u + 2u counts against
        |dy gamma n s|, the rest relatively:
        |err| <= u |dy gamma n s| (|g| (4s + 2) + 3) + (e_i/u + 16) u |dg|
      dgamma = sum over rows of dy n g s, taken as per-slot chains of
        tiles/blocks terms, 32 slots in order, then 1024 / 256-term chains and
        an 8-level tree: |err| <= (e_i/u + 12 + L) u sum |term|, L the length.
"""
import numpy as np
import pytest

import oracle
import sdm_synth as synth
from sdm_synth import Dims

from gpu_helpers import note, to_dev, to_host

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
TINY = 2.0 ** -126


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


def _softplus(z):
    return np.logaddexp(0.0, z)


def _sig(z):
    return 0.5 * (1.0 + np.tanh(0.5 * z))


def _assert_within(name, got, want, tol):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = err > tol
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} out of tolerance; worst excess "
                           f"{np.max(err - tol):.3g} at {np.unravel_index(np.argmax(err - tol), err.shape)}")


def check_gates_backward(got, x, g, d):
    da_raw, db_raw, dA, ddt = got
    o_da_raw, o_db_raw, o_dA, o_ddt = oracle.gates_backward(x["a_raw"], x["b_raw"], x["A"], x["dt_bias"],
                                                            g["da"], g["db"], d)
    z = x["a_raw"].astype(np.float64) + x["dt_bias"].astype(np.float64)[None, None, :]
    Ah = x["A"].astype(np.float64)[None, None, :]
    sp = _softplus(z)
    a = np.exp(-Ah * sp)
    lna = Ah * sp
    e_t = Ah * np.abs(z) * 2 * U + (lna + 1.0) * 8 * U + np.abs(z) * U + 16 * U
    _assert_within("da_raw", da_raw, o_da_raw, e_t * np.abs(o_da_raw) + U * np.abs(o_da_raw) + TINY)
    _assert_within("db_raw", db_raw, o_db_raw, 13 * U * np.abs(o_db_raw) + TINY)
    bt = d.B * d.T
    rows = 256 // min(1 << max(d.H - 1, 0).bit_length(), 256)
    parts = max(1, min(512, -(-bt // (rows * 4))))
    chain = (-(-bt // parts) + 12) * U
    da = g["da"].astype(np.float64)
    term_A = np.abs(da * a * sp)
    term_d = np.abs(da * a * Ah * _sig(z))
    tol_A = ((e_t + chain) * term_A).sum(axis=(0, 1)) + U * np.abs(o_dA) + TINY
    tol_d = ((e_t + chain) * term_d).sum(axis=(0, 1)) + U * np.abs(o_ddt) + TINY
    _assert_within("dA", dA, o_dA, tol_A)
    _assert_within("ddt_bias", ddt, o_ddt, tol_d)


def check_norm_backward(got, x, gr, eps, d, rows=None):
    """rows: a sample of row indices to check do and dg on (None: all)."""
    dout, dg, dgamma = got
    o_do, o_dg, o_dgamma = oracle.output_norm_gate_backward(x["o"], x["g"], x["gamma"], eps, gr["dy"], d)
    dv = d.d_v
    o2 = x["o"].reshape(-1, dv)
    g2 = x["g"].reshape(-1, dv)
    dy2 = gr["dy"].reshape(-1, dv)
    if d.in_dtype == "bf16":
        g2 = synth.bf16_bits_to_f32(g2)
    gm = x["gamma"].astype(np.float64)[None, :]
    e_i = ((dv / 8 + 3) / 2 + 4) * U
    # dgamma: the sum of |dy n g s| over all rows, accumulated in row blocks
    nrows = o2.shape[0]
    tiles = (nrows + 31) // 32
    nblk = min(tiles, 1024)
    L = -(-tiles // nblk) + 32 + -(-nblk // 256) + 8 + 2
    mag = np.zeros(dv)
    for r0 in range(0, nrows, 1 << 16):
        ob = o2[r0:r0 + (1 << 16)].astype(np.float64)
        inv = 1.0 / np.sqrt((ob * ob).mean(axis=1, keepdims=True) + eps)
        gb = g2[r0:r0 + (1 << 16)].astype(np.float64)
        mag += np.abs(dy2[r0:r0 + (1 << 16)] * ob * inv * gb * _sig(gb)).sum(axis=0)
    _assert_within("dgamma", dgamma, o_dgamma, (e_i + (12 + L) * U) * mag + U * np.abs(o_dgamma) + TINY)
    sel = np.arange(nrows) if rows is None else rows
    ob = o2[sel].astype(np.float64)
    gb = g2[sel].astype(np.float64)
    dyb = dy2[sel].astype(np.float64)
    inv = 1.0 / np.sqrt((ob * ob).mean(axis=1, keepdims=True) + eps)
    n = ob * inv
    s = _sig(gb)
    q = dyb * gm * gb * s
    P = np.abs(q * n).sum(axis=1, keepdims=True)
    want_do = o_do.reshape(-1, dv)[sel]
    want_dg = o_dg.reshape(-1, dv)[sel]
    tol_do = (dv / 8 + 40) * U * inv * (np.abs(q) + np.abs(n) * P / dv) + U * np.abs(want_do) + TINY
    _assert_within("do", dout.reshape(-1, dv)[sel], want_do, tol_do)
    base = np.abs(dyb * gm * n * s)
    tol_dg = U * base * (np.abs(gb) * (4 * s + 2) + 3) + (e_i + 17 * U) * np.abs(want_dg) + TINY
    _assert_within("dg", dg.reshape(-1, dv)[sel], want_dg, tol_dg)


@pytest.mark.parametrize("B,T,H", [(1, 1, 1), (3, 77, 5), (2, 1000, 16), (1, 300, 1)])
def test_gates_backward_matches_oracle(sdm, torch, B, T, H):
    d = Dims(B=B, T=T, H=H, d_k=8, n_sub=4, d_v=32, k_prime=4, W=4, R=4, in_dtype="f32")
    note(f"gates backward B={B} T={T} H={H}")
    x = synth.make_layer_edge_inputs(d, seed=B * 100 + T + H)
    gr = synth.make_layer_edge_grads(d, seed=B + T)
    x["a_raw"] *= 3.0
    x["b_raw"] *= 3.0
    # extremes: large pre-activations of both signs (b near 0 and 1, a near 1)
    fa, fb = x["a_raw"].reshape(-1), x["b_raw"].reshape(-1)
    ext = np.array([40.0, -40.0, 90.0, -90.0, 0.0, 1e-7], np.float32)
    fa[:min(fa.size, ext.size)] = ext[:min(fa.size, ext.size)]
    fb[:min(fb.size, ext.size)] = ext[:min(fb.size, ext.size)]
    dims = sdm.dims_from(d)
    dev = {k: to_dev(v) for k, v in list(x.items()) + list(gr.items()) if k in
           ("a_raw", "b_raw", "A", "dt_bias", "da", "db")}
    got = sdm.gates_backward(dev["a_raw"], dev["b_raw"], dev["A"], dev["dt_bias"], dev["da"], dev["db"], dims)
    torch.cuda.synchronize()
    check_gates_backward([to_host(t) for t in got], x, gr, d)


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d_v,B,T,H", [(32, 1, 1, 1), (64, 2, 45, 3), (96, 1, 19, 2), (128, 3, 50, 4),
                                       (256, 1, 9, 5), (1024, 1, 3, 2), (128, 4, 2100, 5)])
def test_output_norm_gate_backward_matches_oracle(sdm, torch, in_dtype, d_v, B, T, H):
    """Ragged row counts (tails of a 32-row tile), every register layout
    (d_v/32 = 1, 2, 4 and the generic path), and more tiles than workgroups
    (the last case: 1313 tiles over 1024 workgroups)."""
    d = Dims(B=B, T=T, H=H, d_k=8, n_sub=4, d_v=d_v, k_prime=4, W=4, R=4, in_dtype=in_dtype)
    note(f"output norm gate backward {in_dtype} d_v={d_v} B={B} T={T} H={H}")
    x = synth.make_layer_edge_inputs(d, seed=d_v + T)
    gr = synth.make_layer_edge_grads(d, seed=d_v * 3 + T)
    o = x["o"]
    if o.shape[0] * o.shape[1] * o.shape[2] > 2:
        o.reshape(-1, d_v)[1] *= 1e15           # large and tiny magnitudes
        o.reshape(-1, d_v)[2] *= 1e-15
    eps = 1e-5
    dims = sdm.dims_from(d)
    got = sdm.output_norm_gate_backward(to_dev(o), to_dev(x["g"]), to_dev(x["gamma"]), eps, to_dev(gr["dy"]), dims)
    torch.cuda.synchronize()
    check_norm_backward([to_host(t) for t in got], x, gr, eps, d)


def test_output_norm_gate_backward_zero_row_and_determinism(sdm, torch):
    """A zero row with eps > 0 gives do = dy gamma silu(g) / sqrt(eps) and
    dg = 0; two calls give the same bits (fixed summation order)."""
    d = Dims(B=2, T=600, H=3, d_k=8, n_sub=4, d_v=64, k_prime=4, W=4, R=4, in_dtype="bf16")
    note("output norm gate backward zero row, determinism")
    x = synth.make_layer_edge_inputs(d, seed=3)
    gr = synth.make_layer_edge_grads(d, seed=4)
    x["o"].reshape(-1, 64)[5] = 0.0
    dims = sdm.dims_from(d)
    args = (to_dev(x["o"]), to_dev(x["g"]), to_dev(x["gamma"]), 1e-5, to_dev(gr["dy"]), dims)
    r1 = [to_host(t) for t in sdm.output_norm_gate_backward(*args)]
    r2 = [to_host(t) for t in sdm.output_norm_gate_backward(*args)]
    torch.cuda.synchronize()
    check_norm_backward(r1, x, gr, 1e-5, d)
    for a, b in zip(r1, r2):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.all(r1[1].reshape(-1, 64)[5] == 0.0)


@pytest.mark.parametrize("name", ["small", "prefill_1p4b"])
def test_full_size_layer_edges_backward(sdm, torch, name):
    """The benchmarked layers at full size: every gate gradient, dgamma, and
    do and dg on a sample of 50,000 rows (every row for the small layer)."""
    d = synth.PRESETS[name].dims
    note(f"layer edges backward full size {name} B={d.B} T={d.T} H={d.H} d_v={d.d_v}")
    x = synth.make_layer_edge_inputs(d, seed=11)
    gr = synth.make_layer_edge_grads(d, seed=12)
    dims = sdm.dims_from(d)
    got = sdm.gates_backward(to_dev(x["a_raw"]), to_dev(x["b_raw"]), to_dev(x["A"]), to_dev(x["dt_bias"]),
                             to_dev(gr["da"]), to_dev(gr["db"]), dims)
    torch.cuda.synchronize()
    check_gates_backward([to_host(t) for t in got], x, gr, d)
    del got
    got = sdm.output_norm_gate_backward(to_dev(x["o"]), to_dev(x["g"]), to_dev(x["gamma"]), 1e-5,
                                        to_dev(gr["dy"]), dims)
    torch.cuda.synchronize()
    host = [to_host(t) for t in got]
    del got
    nrows = d.B * d.T * d.H
    rows = None if nrows <= 200_000 else np.sort(np.random.default_rng(0).choice(nrows, 50_000, replace=False))
    check_norm_backward(host, x, gr, 1e-5, d, rows=rows)
