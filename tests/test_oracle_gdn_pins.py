"""Pins for the oracle's dense Gated DeltaNet recurrence ([P] Sec. 2 Eq. 2;
Sec. 3.1 "Connection to GDN"): the literal matrix form in numpy, the SDM
scan oracle with every slot selected (the reduction the paper states), and
closed forms (pure decay; a unit key overwrites one row).

A plausible slip (the prediction taken after the rows change, a missing
decay on the prediction, the read before the write, k and q swapped, the
state transposed) fails at least one of these.
"""
import numpy as np
import pytest

import oracle
import sdm_synth as synth
from sdm_synth import Dims


def gdn_dims(**kw):
    base = dict(B=2, T=20, H=2, d_k=16, n_sub=4, d_v=6, k_prime=4, W=16, R=16, in_dtype="f32")
    base.update(kw)
    return Dims(**base)


def dec(x, d):
    return synth.bf16_bits_to_f32(x) if d.in_dtype == "bf16" else np.asarray(x, np.float32)


def matrix_form(S0_T, ks, qs, vs, a, b):
    """S <- a S (I - b k k^T) + b v k^T on S [d_v, d_k]; o = S q."""
    S = S0_T.T.astype(np.float64).copy()
    I = np.eye(S.shape[1])
    outs = []
    for t in range(len(ks)):
        k = ks[t][:, None]
        S = a[t] * S @ (I - b[t] * (k @ k.T)) + b[t] * (vs[t][:, None] @ k.T)
        outs.append(S @ qs[t])
    return np.array(outs), S.T


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_gdn_matches_matrix_form(in_dtype):
    d = gdn_dims(in_dtype=in_dtype)
    x = synth.make_gdn_inputs(d, seed=4)
    S = x["S0"].copy()
    o = oracle.gdn_dense(S, x["k"], x["q"], x["v"], x["a"], x["b"], d)
    kf, qf, vf = (dec(x[n], d).astype(np.float64) for n in ("k", "q", "v"))
    for bb in range(d.B):
        for h in range(d.H):
            ro, rS = matrix_form(x["S0"][bb, h], kf[bb, :, h], qf[bb, :, h], vf[bb, :, h],
                                 x["a"][bb, :, h].astype(np.float64), x["b"][bb, :, h].astype(np.float64))
            np.testing.assert_allclose(o[bb, :, h], ro, rtol=0, atol=1e-6 * np.sqrt(np.mean(ro ** 2)))
            np.testing.assert_allclose(S[bb, h], rS, rtol=0, atol=1e-6 * np.sqrt(np.mean(rS ** 2)))


@pytest.mark.parametrize("in_dtype", ["f32", "bf16"])
def test_gdn_equals_sdm_scan_with_every_slot_selected(in_dtype):
    """W = R = N = d_k with slot lists 0..N-1 and the dense key and query as
    weights: the SDM scan and the dense recurrence are the same function
    (same operations in the same order here, so bit-identical)."""
    d = gdn_dims(in_dtype=in_dtype)
    x = synth.make_gdn_inputs(d, seed=5)
    S = x["S0"].copy()
    o = oracle.gdn_dense(S, x["k"], x["q"], x["v"], x["a"], x["b"], d)
    N = d.d_k
    idx = np.broadcast_to(np.arange(N, dtype=np.int32), (d.B, d.T, d.H, N)).copy()
    wk = dec(x["k"], d).astype(np.float32)
    wq = dec(x["q"], d).astype(np.float32)
    M = x["S0"].copy()
    o2 = oracle.scan(M, idx, wk, idx, wq, x["v"], x["a"], x["b"], d)
    assert np.array_equal(o, o2)
    assert np.array_equal(S, M)


def test_gdn_closed_forms():
    d = gdn_dims(B=1, H=1, T=5, d_k=8, n_sub=2, d_v=3, W=4, R=4)
    x = synth.make_gdn_inputs(d, seed=6)
    # b = 0: pure decay, each step one fp32 product per element
    S = x["S0"].copy()
    b0 = np.zeros_like(x["b"])
    oracle.gdn_dense(S, x["k"], x["q"], x["v"], x["a"], b0, d)
    ref = x["S0"].copy()
    for t in range(d.T):
        ref = (np.float64(x["a"][0, t, 0]) * ref.astype(np.float64)).astype(np.float32)
    assert np.array_equal(S, ref)
    # a = b = 1 and a unit key e_j: row j of the state becomes v_t exactly, the
    # other rows are unchanged, and the query e_j reads v_t back
    k = np.zeros((1, d.T, 1, d.d_k), np.float32)
    j = np.array([3, 0, 7, 3, 5])
    k[0, np.arange(d.T), 0, j] = 1.0
    ones = np.ones((1, d.T, 1), np.float32)
    S = x["S0"].copy()
    o = oracle.gdn_dense(S, k, k, x["v"], ones, ones, d)
    assert np.array_equal(o[0, :, 0], x["v"][0, :, 0])
    assert np.array_equal(S[0, 0, [3, 0, 7, 5]], x["v"][0, [3, 1, 2, 4], 0])
    untouched = [1, 2, 4, 6]
    assert np.array_equal(S[0, 0, untouched], x["S0"][0, 0, untouched])
