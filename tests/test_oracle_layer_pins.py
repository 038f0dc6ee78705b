"""Pins for the oracle's gates (before the path) and output norm and gate
(after it): closed forms, special cases, and library routines on an
independent formulation (numpy's logaddexp for softplus, scipy's expit for
the sigmoid, torch's rms_norm and silu).

A plausible slip (the time-step bias added outside the softplus, the decay
applied without its minus sign, the wrong head's parameters, the mean
replaced by a sum, eps outside the square root, the gain indexed by head
instead of by feature, the gate's sigmoid without the factor g) fails at
least one of these.
"""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
import sdm_synth as synth
from sdm_synth import Dims


def dims(**kw):
    base = dict(B=1, T=4, H=1, d_k=8, n_sub=4, d_v=4, k_prime=4, W=4, R=4, in_dtype="f32")
    base.update(kw)
    return Dims(**base)


def f32_ulp(x):
    return np.spacing(np.abs(np.asarray(x, np.float32)))


# ---------------------------------------------------------------------------
# gates
# ---------------------------------------------------------------------------
def test_gates_closed_forms():
    d = dims(B=1, T=4, H=3)
    dt = np.array([0.25, -1.5, 3.0], np.float32)
    A = np.array([1.0, 2.0, 0.0], np.float32)
    # a_raw + dt_bias = 0 on every head: softplus(0) = ln 2, so a = 2^-A
    a_raw = np.broadcast_to(-dt, (1, 4, 3)).copy()
    b_raw = np.zeros((1, 4, 3), np.float32)
    a, b = oracle.gates(a_raw, b_raw, A, dt, d)
    assert np.array_equal(a, np.broadcast_to(np.array([0.5, 0.25, 1.0], np.float32), a.shape))
    assert np.all(b == 0.5)
    # A = 0 never decays, whatever the input
    rng = np.random.default_rng(1)
    a_raw = rng.normal(0, 5, (1, 4, 3)).astype(np.float32)
    a, _ = oracle.gates(a_raw, b_raw, np.zeros(3, np.float32), dt, d)
    assert np.all(a == 1.0)


def test_gates_match_library_routines():
    d = dims(B=3, T=50, H=5)
    rng = np.random.default_rng(2)
    a_raw = rng.normal(0, 3, (3, 50, 5)).astype(np.float32)
    b_raw = rng.normal(0, 3, (3, 50, 5)).astype(np.float32)
    A = rng.uniform(0.0, 16.0, 5).astype(np.float32)
    dt = rng.normal(-3, 1, 5).astype(np.float32)
    a, b = oracle.gates(a_raw, b_raw, A, dt, d)
    z = a_raw.astype(np.float64) + dt.astype(np.float64)[None, None, :]
    a_ref = np.exp(-A.astype(np.float64)[None, None, :] * np.logaddexp(0.0, z)).astype(np.float32)
    b_ref = scipy.special.expit(b_raw.astype(np.float64)).astype(np.float32)
    # both sides round an fp64 value once: equal up to the last bit of the fp64 work
    assert np.all(np.abs(a - a_ref) <= f32_ulp(a_ref))
    assert np.all(np.abs(b - b_ref) <= f32_ulp(b_ref))
    # decay strictly decreases with the forget pre-activation where it is representable
    order = np.argsort(a_raw[:, :, 0], axis=None)
    aa = a[:, :, 0].ravel()[order]
    assert np.all(np.diff(aa.astype(np.float64)) <= 0)


def test_gates_extreme_inputs():
    d = dims(B=1, T=6, H=1)
    a_raw = np.array([[[80.0], [-80.0], [1e30], [-1e30], [30.0], [-30.0]]], np.float32)
    b_raw = np.array([[[80.0], [-80.0], [1e30], [-1e30], [30.0], [-30.0]]], np.float32)
    a, b = oracle.gates(a_raw, b_raw, np.ones(1, np.float32), np.zeros(1, np.float32), d)
    a = a.ravel(); b = b.ravel()
    assert a[0] == np.float32(np.exp(-80.0)) and a[2] == 0.0
    assert a[3] == 1.0 and a[1] == np.float32(np.exp(-np.log1p(np.exp(-80.0))))
    assert a[4] == np.float32(np.exp(-(30.0 + np.log1p(np.exp(-30.0)))))
    assert b[0] == 1.0 and b[2] == 1.0 and b[3] == 0.0
    assert b[1] == np.float32(np.exp(-80.0) / (1.0 + np.exp(-80.0)))
    assert b[4] + b[5] == pytest.approx(1.0, abs=1e-7)


def test_gates_reject_bad_parameters():
    d = dims(B=1, T=2, H=1)
    z = np.zeros((1, 2, 1), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.gates(z, z, np.array([-1.0], np.float32), np.zeros(1, np.float32), d)
    with pytest.raises(oracle.OracleError):
        oracle.gates(z + np.nan, z, np.ones(1, np.float32), np.zeros(1, np.float32), d)


# ---------------------------------------------------------------------------
# output norm and gate
# ---------------------------------------------------------------------------
def test_norm_gate_constant_rows_and_eps():
    d = dims(B=1, T=3, H=1, d_v=4)
    gamma = np.array([1.0, -2.0, 0.5, 3.0], np.float32)
    g = np.array([[[[0.0, 1.0, -1.0, 4.0]]] * 3], np.float32).reshape(1, 3, 1, 4)
    silu = lambda x: x / (1.0 + np.exp(-x))
    o = np.stack([np.full(4, 7.0), np.full(4, -0.25), np.array([3.0, 4.0, 0.0, 0.0])]).astype(np.float32)
    o = o.reshape(1, 3, 1, 4)
    y = oracle.output_norm_gate(o, g, gamma, 0.0, d).reshape(3, 4)
    gg = g.reshape(3, 4).astype(np.float64)
    np.testing.assert_allclose(y[0], gamma * silu(gg[0]), rtol=1e-15)      # RMS of a constant row
    np.testing.assert_allclose(y[1], -gamma * silu(gg[1]), rtol=1e-15)
    # [3, 4, 0, 0]: mean square 25/4; with eps = 25/4 the divisor is sqrt(12.5)
    y = oracle.output_norm_gate(o, g, gamma, 6.25, d).reshape(3, 4)
    np.testing.assert_allclose(y[2], np.array([3.0, 4.0, 0, 0]) / np.sqrt(12.5) * gamma * silu(gg[2]), rtol=1e-15)
    # a zero row stays zero (eps > 0)
    z = np.zeros_like(o)
    assert np.all(oracle.output_norm_gate(z, g, gamma, 1e-5, d) == 0.0)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_norm_gate_matches_torch(in_dtype):
    d = dims(B=2, T=9, H=3, d_v=32, in_dtype=in_dtype)
    rng = np.random.default_rng(3)
    o = rng.normal(0, 0.3, (2, 9, 3, 32)).astype(np.float32)
    g32 = rng.normal(0, 2, (2, 9, 3, 32)).astype(np.float32)
    g = synth.f32_to_bf16_bits(g32) if in_dtype == "bf16" else g32
    gdec = synth.bf16_bits_to_f32(g) if in_dtype == "bf16" else g32
    gamma = rng.normal(1, 0.5, 32).astype(np.float32)
    eps = 1e-5
    y = oracle.output_norm_gate(o, g, gamma, eps, d)
    ref = F.rms_norm(torch.from_numpy(o).double(), (32,), torch.from_numpy(gamma).double(), eps) * \
        F.silu(torch.from_numpy(gdec).double())
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-300)


def test_norm_gate_rows_independent():
    d = dims(B=1, T=5, H=2, d_v=8)
    rng = np.random.default_rng(4)
    o = rng.normal(0, 1, (1, 5, 2, 8)).astype(np.float32)
    g = rng.normal(0, 1, (1, 5, 2, 8)).astype(np.float32)
    gamma = rng.normal(1, 0.1, 8).astype(np.float32)
    y = oracle.output_norm_gate(o, g, gamma, 1e-6, d)
    perm = rng.permutation(10)
    yp = oracle.output_norm_gate(o.reshape(10, 8)[perm].reshape(1, 5, 2, 8),
                                 g.reshape(10, 8)[perm].reshape(1, 5, 2, 8), gamma, 1e-6, d)
    assert np.array_equal(yp.reshape(10, 8), y.reshape(10, 8)[perm])


# ---------------------------------------------------------------------------
# gradients of the gates and of the output norm and gate: central differences
# of the forward definitions written here in numpy (fp64)
# ---------------------------------------------------------------------------
def _gates64(a_raw, b_raw, A, dt):
    z = a_raw + dt[None, None, :]
    return np.exp(-A[None, None, :] * np.logaddexp(0.0, z)), scipy.special.expit(b_raw)


def test_gates_gradients_match_central_differences():
    d = dims(B=2, T=7, H=3)
    rng = np.random.default_rng(21)
    a_raw = rng.normal(0, 2, (2, 7, 3)).astype(np.float32)
    b_raw = rng.normal(0, 2, (2, 7, 3)).astype(np.float32)
    A = rng.uniform(0.5, 4, 3).astype(np.float32)
    dt = rng.normal(-1, 1, 3).astype(np.float32)
    da = rng.normal(0, 1, (2, 7, 3)).astype(np.float32)
    db = rng.normal(0, 1, (2, 7, 3)).astype(np.float32)
    g = oracle.gates_backward(a_raw, b_raw, A, dt, da, db, d)
    base = dict(a_raw=a_raw.astype(np.float64), b_raw=b_raw.astype(np.float64), A=A.astype(np.float64),
                dt=dt.astype(np.float64))

    def loss(**over):
        y = {k: over.get(k, v) for k, v in base.items()}
        a, b = _gates64(y["a_raw"], y["b_raw"], y["A"], y["dt"])
        return float(np.sum(da * a) + np.sum(db * b))

    for name, gr in zip(("a_raw", "b_raw", "A", "dt"), g):
        delta = rng.normal(0, 1, base[name].shape)
        h = 1e-6
        fd = (loss(**{name: base[name] + h * delta}) - loss(**{name: base[name] - h * delta})) / (2 * h)
        an = float(np.sum(gr.astype(np.float64) * delta))
        assert abs(fd - an) <= 1e-6 * (abs(fd) + np.sqrt(np.sum(gr.astype(np.float64) ** 2))), (name, fd, an)


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_norm_gate_gradients_match_central_differences(in_dtype):
    d = dims(B=2, T=5, H=2, d_v=16, in_dtype=in_dtype)
    rng = np.random.default_rng(22)
    o = rng.normal(0, 0.5, (2, 5, 2, 16)).astype(np.float32)
    g32 = rng.normal(0, 1.5, (2, 5, 2, 16)).astype(np.float32)
    g = synth.f32_to_bf16_bits(g32) if in_dtype == "bf16" else g32
    gdec = (synth.bf16_bits_to_f32(g) if in_dtype == "bf16" else g32).astype(np.float64)
    gamma = rng.normal(1, 0.3, 16).astype(np.float32)
    dy = rng.normal(0, 1, (2, 5, 2, 16)).astype(np.float32)
    eps = 1e-3
    do, dg, dgamma = oracle.output_norm_gate_backward(o, g, gamma, eps, dy, d)
    base = dict(o=o.astype(np.float64), g=gdec, gamma=gamma.astype(np.float64))

    def loss(**over):
        y = {k: over.get(k, v) for k, v in base.items()}
        ref = (F.rms_norm(torch.from_numpy(y["o"]), (16,), torch.from_numpy(y["gamma"]), eps) *
               F.silu(torch.from_numpy(y["g"]))).numpy()
        return float(np.sum(dy * ref))

    for name, gr in (("o", do), ("g", dg), ("gamma", dgamma)):
        delta = rng.normal(0, 1, base[name].shape)
        h = 1e-6
        fd = (loss(**{name: base[name] + h * delta}) - loss(**{name: base[name] - h * delta})) / (2 * h)
        an = float(np.sum(gr.astype(np.float64) * delta))
        assert abs(fd - an) <= 1e-6 * (abs(fd) + np.sqrt(np.sum(gr.astype(np.float64) ** 2))), (name, fd, an)


def test_gates_gradient_tails():
    """Far in the sigmoid's tails its derivative is e^-|x| to within a
    relative 2 e^-|x| (the leading term of e^-|x| / (1 + e^-|x|)^2), so
    db_raw for db = 1 must be that exponential, not a difference of two
    numbers near 1 rounded to 0."""
    xs = np.array([40.0, -40.0, 60.0, -60.0, 100.0, -100.0], np.float32)
    d = dims(B=1, T=6, H=1)
    z = np.zeros((1, 6, 1), np.float32)
    _, db_raw, _, _ = oracle.gates_backward(z, xs.reshape(1, 6, 1), np.ones(1, np.float32),
                                            np.zeros(1, np.float32), z, np.ones((1, 6, 1), np.float32), d)
    want = np.exp(-np.abs(xs.astype(np.float64)))
    got = db_raw.reshape(-1).astype(np.float64)
    ulp = np.spacing(want.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - want) <= ulp), (got, want)
