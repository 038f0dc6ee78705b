"""Pins for the oracle's addressing gradients: central differences of an
independent fp64 forward written here (the selected slots held fixed: slot
score = first-half score + second-half score, softmax over the list), for
keys, queries and both codebooks, with separate and with shared codebooks;
the one-slot list (weight 1, zero gradient) and a constant weight gradient
(softmax invariance).

A plausible slip (the softmax Jacobian without its mean term, the halves'
codebook rows swapped, the slot split as i2 * n_sub + i1, the codebook
gradient taken from the wrong kind's input) fails the difference checks.
"""
import numpy as np
import pytest

import oracle
import sdm_synth as synth
from sdm_synth import Dims


def dims(**kw):
    base = dict(B=2, T=5, H=2, d_k=8, n_sub=5, d_v=4, k_prime=3, W=4, R=3, in_dtype="f32")
    base.update(kw)
    return Dims(**base)


def weights64(x, C, idx, d):
    """softmax over the selected slots of fp64 two-half scores; x [B,T,H,d_k], C [H,2,n_sub,half]."""
    half = d.d_k // 2
    i1, i2 = idx // d.n_sub, idx % d.n_sub
    B, T, H, n = idx.shape
    hh = np.broadcast_to(np.arange(H)[None, None, :, None], idx.shape)
    s0 = np.einsum("bthe,bthne->bthn", x[..., :half], C[hh, 0, i1])
    s1 = np.einsum("bthe,bthne->bthn", x[..., half:], C[hh, 1, i2])
    sc = s0 + s1
    e = np.exp(sc - sc.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


@pytest.mark.parametrize("shared", [False, True])
def test_address_gradients_match_central_differences(shared):
    d = dims()
    x = synth.make_inputs(d, seed=11, separate_read_codebook=not shared)
    widx, wwt, ridx, rwt = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    rng = np.random.default_rng(12)
    dw = rng.normal(0, 1, wwt.shape).astype(np.float32)
    dr = rng.normal(0, 1, rwt.shape).astype(np.float32)
    dk, dq, dCw, dCr = oracle.address_backward(x["k"], x["q"], x["C_w"], x["C_r"], widx, wwt, ridx, rwt, dw, dr, d)
    base = {n: x[n].astype(np.float64) for n in ("k", "q", "C_w", "C_r")}

    def loss(**over):
        y = {n: over.get(n, base[n]) for n in base}
        if shared:
            y["C_r"] = y["C_w"]
        return float(np.sum(dw * weights64(y["k"], y["C_w"], widx, d)) +
                     np.sum(dr * weights64(y["q"], y["C_r"], ridx, d)))

    grads = {"k": dk, "q": dq, "C_w": dCw + dCr if shared else dCw}
    if not shared:
        grads["C_r"] = dCr
    for name, gr in grads.items():
        delta = rng.normal(0, 1, base[name].shape)
        h = 1e-6
        fd = (loss(**{name: base[name] + h * delta}) - loss(**{name: base[name] - h * delta})) / (2 * h)
        an = float(np.sum(gr.astype(np.float64) * delta))
        assert abs(fd - an) <= 1e-5 * (abs(fd) + np.sqrt(np.sum(gr.astype(np.float64) ** 2))), \
            f"{name}: difference quotient {fd:.9g} vs gradient {an:.9g}"


def test_address_gradients_single_slot_and_constant_gradient():
    d = dims(W=1, R=2)
    x = synth.make_inputs(d, seed=13)
    widx, wwt, ridx, rwt = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    dw = np.full(wwt.shape, 3.0, np.float32)
    dr = np.full(rwt.shape, -2.0, np.float32)
    dk, dq, dCw, dCr = oracle.address_backward(x["k"], x["q"], x["C_w"], x["C_r"], widx, wwt, ridx, rwt, dw, dr, d)
    assert np.all(dk == 0.0)                  # one slot: weight 1 whatever its score
    # a constant weight gradient moves nothing (the weights sum to one)
    assert np.max(np.abs(dq)) <= 1e-6 and np.max(np.abs(dCr)) <= 1e-6
