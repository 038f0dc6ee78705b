"""Pins for the oracle's scan gradients: central differences of an
independent fp64 forward written here (numpy, per token), along random
directions in every input (the initial state, v, a, b, both weight lists),
with frequent slot collisions between tokens and reads of rows the same
token writes; linearity in the incoming gradients; and the b = 0 case.

A plausible slip in the backward (the read gradient added after the write
rows are processed, the prediction term of dw or da dropped, G[s_j]
replaced without the w_j dp term, the decay missing from dX, a sign error
in dp) fails the difference checks.
"""
import numpy as np
import pytest

import oracle
import sdm_synth as synth
from sdm_synth import Dims


def small_dims(**kw):
    base = dict(B=2, T=12, H=2, d_k=8, n_sub=3, d_v=4, k_prime=3, W=3, R=2, in_dtype="f32")
    base.update(kw)
    return Dims(**base)


def forward64(M0, widx, wwt, ridx, rwt, v, a, b):
    """The scan in fp64 with no rounding: returns o and the final state."""
    M = M0.astype(np.float64).copy()
    B, T, H, W = widx.shape
    o = np.zeros(v.shape, np.float64)
    for bb in range(B):
        for h in range(H):
            Mc = M[bb, h]
            for t in range(T):
                wi, ri = widx[bb, t, h], ridx[bb, t, h]
                w, r = wwt[bb, t, h].astype(np.float64), rwt[bb, t, h].astype(np.float64)
                p = w @ Mc[wi]
                u = v[bb, t, h] - a[bb, t, h] * p
                Mc[wi] = a[bb, t, h] * Mc[wi] + b[bb, t, h] * np.outer(w, u)
                o[bb, t, h] = r @ Mc[ri]
    return o, M


def inputs(d, seed, pool):
    x = synth.make_inputs(d, seed)
    ad = synth.random_addressing(d, seed, hazard_slots=pool)
    M0 = np.repeat(x["M0"][None], d.B, axis=0).astype(np.float64)
    M0 += np.random.default_rng(seed).normal(0, 0.1, M0.shape)     # sequences start from different states
    return dict(M0=M0.astype(np.float32), v=x["v"].astype(np.float64), a=x["a"], b=x["b"], **ad)


@pytest.mark.parametrize("pool", [9, 5])
def test_scan_gradients_match_central_differences(pool):
    d = small_dims()
    x = inputs(d, 3, pool)
    rng = np.random.default_rng(7)
    dout = rng.normal(0, 1, (d.B, d.T, d.H, d.d_v))
    dMT = rng.normal(0, 1, x["M0"].shape)
    g = oracle.scan_backward(x["M0"], x["widx"], x["wwt"], x["ridx"], x["rwt"], x["v"].astype(np.float32),
                             x["a"], x["b"], dout.astype(np.float32), d, dM_final=dMT.astype(np.float32))
    dout32, dMT32 = dout.astype(np.float32).astype(np.float64), dMT.astype(np.float32).astype(np.float64)

    def loss(**over):
        y = {k: over.get(k, x[k]) for k in ("M0", "wwt", "rwt", "v", "a", "b")}
        o, MT = forward64(y["M0"], x["widx"], y["wwt"], x["ridx"], y["rwt"], y["v"], y["a"], y["b"])
        return float(np.sum(dout32 * o) + np.sum(dMT32 * MT))

    grads = dict(M0=g["dM"], v=g["dv"], a=g["da"], b=g["db"], wwt=g["dw"], rwt=g["dr"])
    for name, gr in grads.items():
        base = x[name].astype(np.float64)
        delta = rng.normal(0, 1, base.shape)
        h = 1e-5
        fd = (loss(**{name: base + h * delta}) - loss(**{name: base - h * delta})) / (2 * h)
        an = float(np.sum(gr.astype(np.float64) * delta))
        assert abs(fd - an) <= 2e-5 * (abs(fd) + np.sqrt(np.sum(gr.astype(np.float64) ** 2))), \
            f"{name}: difference quotient {fd:.9g} vs gradient {an:.9g}"


def test_scan_gradients_linear_in_incoming_gradient():
    d = small_dims(T=9)
    x = inputs(d, 4, 9)
    rng = np.random.default_rng(8)
    dout = rng.normal(0, 1, (d.B, d.T, d.H, d.d_v)).astype(np.float32)
    args = (x["M0"], x["widx"], x["wwt"], x["ridx"], x["rwt"], x["v"].astype(np.float32), x["a"], x["b"])
    g1 = oracle.scan_backward(*args, dout, d)
    g2 = oracle.scan_backward(*args, 2 * dout, d)
    for k in g1:
        assert np.array_equal(g2[k], 2 * g1[k]), k


def test_scan_gradients_b_zero():
    # b = 0: the writes only decay their rows, so v never reaches the output
    d = small_dims()
    x = inputs(d, 5, 9)
    b0 = np.zeros_like(x["b"])
    rng = np.random.default_rng(9)
    dout = rng.normal(0, 1, (d.B, d.T, d.H, d.d_v)).astype(np.float32)
    g = oracle.scan_backward(x["M0"], x["widx"], x["wwt"], x["ridx"], x["rwt"], x["v"].astype(np.float32),
                             x["a"], b0, dout, d)
    assert np.all(g["dv"] == 0.0)
    # with b = 0 the write weights act only through the prediction, which b scales away
    assert np.all(g["dw"] == 0.0)
