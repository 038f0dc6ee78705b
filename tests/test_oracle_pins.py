"""Pins for the CPU oracle: each test checks it against something other than
itself -- brute force over all N slots, a special case with a closed form, a
library routine on an independent formulation, or a hand-worked example.

A plausible slip anywhere in the oracle (a dropped term, a wrong sign or
index, a transposed operand, the read taken before the write, sequential
instead of simultaneous row updates) fails at least one of these.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import sdm_synth as synth
from sdm_synth import Dims

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# independent helpers (numpy; no oracle code)
# ---------------------------------------------------------------------------
def dec(x, d):
    return synth.bf16_bits_to_f32(x) if d.in_dtype == "bf16" else np.asarray(x, np.float32)


def brute_scores(x_row, C_h, d):
    """All N fp32 slot scores of one token-head: fp32 half scores via an fp64
    matmul, then the fp32 outer sum, flat slot = i1*n_sub + i2."""
    half = d.d_k // 2
    xs = dec(x_row, d).astype(np.float64)
    Cs = dec(C_h, d).astype(np.float64)           # [2, n_sub, half]
    s1 = (Cs[0] @ xs[:half]).astype(np.float32)
    s2 = (Cs[1] @ xs[half:]).astype(np.float32)
    return (s1[:, None] + s2[None, :]).reshape(-1)  # float32 + float32 -> float32


def brute_topn(scores, n):
    order = np.lexsort((np.arange(scores.size), -scores.astype(np.float64)))
    return order[:n].astype(np.int32), scores[order[:n]]


def dims(**kw):
    base = dict(B=1, T=8, H=1, d_k=8, n_sub=4, d_v=4, k_prime=4, W=4, R=4, in_dtype="f32")
    base.update(kw)
    return Dims(**base)


# ---------------------------------------------------------------------------
# addressing
# ---------------------------------------------------------------------------
def test_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_example.json")))
    d = Dims(B=1, T=3, H=1, d_k=2, n_sub=2, d_v=2, k_prime=2, W=1, R=1, in_dtype="f32")
    C = np.array([[[1.0], [-1.0]], [[1.0], [-1.0]]], np.float32)[None]  # [H,2,n_sub,half]
    k = np.array(g["k"], np.float32)[None, :, None, :]
    q = np.array(g["q"], np.float32)[None, :, None, :]
    v = np.array(g["v"], np.float32)[None, :, None, :]
    a = np.array(g["a"], np.float32)[None, :, None]
    b = np.array(g["b"], np.float32)[None, :, None]
    widx, wwt, ridx, rwt = oracle.address(k, q, C, C, d)
    assert widx.ravel().tolist() == g["expect_widx"]
    assert ridx.ravel().tolist() == g["expect_ridx"]
    assert np.all(wwt == 1.0) and np.all(rwt == 1.0)
    M = np.array(g["M0"], np.float32)[None, None]
    o = oracle.scan(M, widx, wwt, ridx, rwt, v, a, b, d)
    np.testing.assert_array_equal(o[0, :, 0], np.array(g["expect_o"], np.float32))
    np.testing.assert_array_equal(M[0, 0], np.array(g["expect_M"], np.float32))
    # tie rule: equal scores go to the lower slot index
    d2 = d.replace(T=1, W=2)
    kt = np.array(g["tie_k"], np.float32)[None, None, None, :]
    widx2, wwt2, _, _ = oracle.address(kt, kt, C, C, d2)
    assert widx2.ravel().tolist() == g["tie_expect_widx"]
    e = math.e
    np.testing.assert_allclose(wwt2.ravel(), [e / (1 + e), 1 / (1 + e)], rtol=1e-7)


@pytest.mark.parametrize("name,rows", [("tiny", None), ("small", 96)])
def test_pkm_equals_brute_force(name, rows):
    """With k' >= W the cartesian merge of the per-half top-k' lists is the exact
    top-W over all N slots (the 'no need to materialise all scores' claim)."""
    p = synth.PRESETS[name]
    d = p.dims
    if rows is not None:
        d = d.replace(B=1, T=rows // d.H if rows >= d.H else 1)
    x = synth.make_inputs(d, seed=3)
    widx, wwt, ridx, rwt, wsc, rsc = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d, scores=True)
    mism = 0
    for bb in range(d.B):
        for t in range(d.T):
            for h in range(d.H):
                for kind, xin, C, idx, sc, n in (("w", x["k"], x["C_w"], widx, wsc, d.W),
                                                 ("r", x["q"], x["C_r"], ridx, rsc, d.R)):
                    s = brute_scores(xin[bb, t, h], C[h], d)
                    bi, bs = brute_topn(s, n)
                    np.testing.assert_array_equal(sc[bb, t, h], bs)
                    if not np.array_equal(idx[bb, t, h], bi):
                        # only an exact fp32 rounding tie may reorder; the scores agree
                        mism += 1
                        assert np.array_equal(np.sort(s[idx[bb, t, h]]), np.sort(bs))
    assert mism == 0


def test_pkm_bruteforce_with_larger_kprime():
    d = dims(B=2, T=16, H=3, d_k=16, n_sub=12, k_prime=7, W=5, R=3)
    x = synth.make_inputs(d, seed=11)
    widx, _, ridx, _ = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    for bb in range(d.B):
        for t in range(d.T):
            for h in range(d.H):
                bi, _ = brute_topn(brute_scores(x["k"][bb, t, h], x["C_w"][h], d), d.W)
                assert widx[bb, t, h].tolist() == bi.tolist()
                bi, _ = brute_topn(brute_scores(x["q"][bb, t, h], x["C_r"][h], d), d.R)
                assert ridx[bb, t, h].tolist() == bi.tolist()


def test_pkm_approximation_when_kprime_below_w():
    """k' < W is the PKM approximation: every selected slot comes from the
    per-half top-k' lists, and the list is the best W of those k'^2 pairs."""
    d = dims(B=1, T=12, H=2, d_k=8, n_sub=10, k_prime=3, W=7, R=9)
    x = synth.make_inputs(d, seed=5)
    widx, _, _, _ = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    for t in range(d.T):
        for h in range(d.H):
            s = brute_scores(x["k"][0, t, h], x["C_w"][h], d)
            half = d.d_k // 2
            xs = dec(x["k"][0, t, h], d).astype(np.float64)
            Cs = dec(x["C_w"][h], d).astype(np.float64)
            h1 = (Cs[0] @ xs[:half]).astype(np.float32)
            h2 = (Cs[1] @ xs[half:]).astype(np.float32)
            t1 = np.lexsort((np.arange(d.n_sub), -h1.astype(np.float64)))[:d.k_prime]
            t2 = np.lexsort((np.arange(d.n_sub), -h2.astype(np.float64)))[:d.k_prime]
            allowed = {int(i1 * d.n_sub + i2) for i1 in t1 for i2 in t2}
            assert set(widx[0, t, h].tolist()) <= allowed
            cand = np.array(sorted(allowed))
            bi, _ = brute_topn(s[cand], d.W)
            assert widx[0, t, h].tolist() == cand[bi].tolist()


def test_identity_codebook_half_scores_exact():
    """With n_sub = d_k/2 and C = I the half scores are the input halves
    exactly, which pins the half split and the codebook layout."""
    d = Dims(B=2, T=5, H=3, d_k=32, n_sub=16, d_v=8, k_prime=4, W=1, R=3, in_dtype="bf16")
    x = synth.make_inputs(d, seed=2)
    eye = synth.f32_to_bf16_bits(np.broadcast_to(np.eye(16, dtype=np.float32), (d.H, 2, 16, 16)).copy())
    hs = oracle.half_scores(x["k"], eye, d)
    kf = synth.bf16_bits_to_f32(x["k"])
    np.testing.assert_array_equal(hs[..., 0, :], kf[..., :16])
    np.testing.assert_array_equal(hs[..., 1, :], kf[..., 16:])
    widx, wwt, _, _ = oracle.address(x["k"], x["q"], eye, eye, d)
    # W = 1: the best slot is argmax of each half; weight exactly 1
    expect = np.argmax(kf[..., :16], -1) * 16 + np.argmax(kf[..., 16:], -1)
    np.testing.assert_array_equal(widx[..., 0], expect)
    assert np.all(wwt == 1.0)


def test_half_scores_match_fp64_matmul():
    d = synth.PRESETS["small"].dims.replace(B=1, T=8)
    x = synth.make_inputs(d, seed=9)
    hs = oracle.half_scores(x["k"], x["C_w"], d)
    kf = synth.bf16_bits_to_f32(x["k"]).astype(np.float64)
    Cf = synth.bf16_bits_to_f32(x["C_w"]).astype(np.float64)
    half = d.d_k // 2
    ref0 = np.einsum("bthe,hue->bthu", kf[..., :half], Cf[:, 0]).astype(np.float32)
    ref1 = np.einsum("bthe,hue->bthu", kf[..., half:], Cf[:, 1]).astype(np.float32)
    np.testing.assert_array_equal(hs[..., 0, :], ref0)
    np.testing.assert_array_equal(hs[..., 1, :], ref1)


@pytest.mark.parametrize("in_dtype,sep", [("bf16", False), ("bf16", True), ("f32", True)])
def test_slot_scores_equal_brute_force(in_dtype, sep):
    """oracle.slot_scores (the near-tie classifier of the GPU parity tests)
    equals the brute-force fp32 score s1[i1] + s2[i2] of the named slot, with
    i1 = slot // n_sub taken from the first half of the key and
    i2 = slot % n_sub from the second ([P] Sec. 2, product keys), for random
    token-head rows of several heads, both codebooks and both input dtypes.
    n_sub is not a power of two and the rows span heads, so a swapped split,
    a transposed codebook or a wrong head fails."""
    d = Dims(B=2, T=7, H=3, d_k=64 if in_dtype == "bf16" else 24, n_sub=37, d_v=8, k_prime=5, W=3, R=2,
             in_dtype=in_dtype)
    x = synth.make_inputs(d, seed=17, m0=False, separate_read_codebook=sep)
    g = np.random.default_rng(23)
    n = 400
    rows = g.integers(0, d.B * d.T * d.H, n)
    slots = g.integers(0, d.N, n).astype(np.int32)
    for xk, ck in (("k", "C_w"), ("q", "C_r")):
        xf = x[xk].reshape(d.B * d.T * d.H, d.d_k)
        got = oracle.slot_scores(x[xk], x[ck], d, rows, slots)
        full = [brute_scores(xf[r], x[ck][r % d.H], d) for r in rows]
        want = np.array([f[s] for f, s in zip(full, slots)], np.float32)
        np.testing.assert_array_equal(got, want)
        # the pin is sensitive to the slot split: the swapped split gives other scores
        i1, i2 = slots // d.n_sub, slots % d.n_sub
        swapped = np.array([f[b * d.n_sub + a] for f, a, b in zip(full, i1, i2)], np.float32)
        assert np.mean(swapped != want) > 0.9
    if sep:
        # the two codebooks give different scores for the same input
        assert np.mean(oracle.slot_scores(x["k"], x["C_w"], d, rows, slots)
                       != oracle.slot_scores(x["k"], x["C_r"], d, rows, slots)) > 0.9


def test_softmax_weights():
    d = dims(B=2, T=20, H=2, d_k=16, n_sub=9, k_prime=6, W=6, R=1)
    x = synth.make_inputs(d, seed=4)
    widx, wwt, ridx, rwt = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    assert np.all(rwt == 1.0)                       # one selected slot -> weight exactly 1
    np.testing.assert_allclose(wwt.sum(-1), 1.0, atol=1e-6)
    assert np.all(np.diff(wwt, axis=-1) <= 0)       # lists are score-descending
    for bb in range(d.B):
        for t in range(d.T):
            for h in range(d.H):
                s = brute_scores(x["k"][bb, t, h], x["C_w"][h], d)
                ref = scipy.special.softmax(s[widx[bb, t, h]].astype(np.float64))
                np.testing.assert_allclose(wwt[bb, t, h], ref, rtol=2e-7, atol=1e-9)


# ---------------------------------------------------------------------------
# scan
# ---------------------------------------------------------------------------
def _dense_gdn(M0_h, ks, qs, vs, a, b):
    """Textbook Gated DeltaNet recurrence on a dense state S [d_v, N]:
    S <- a S (I - b k k^T) + b v k^T ; o = S q."""
    S = M0_h.T.astype(np.float64).copy()
    N = S.shape[1]
    outs = []
    I = np.eye(N)
    for t in range(len(ks)):
        k = ks[t][:, None]
        S = a[t] * S @ (I - b[t] * (k @ k.T)) + b[t] * (vs[t][:, None] @ k.T)
        outs.append(S @ qs[t])
    return np.array(outs), S.T


@pytest.mark.parametrize("n_sub,in_dtype", [(4, "f32"), (8, "f32"), (4, "bf16")])
def test_dense_reduction_to_gated_deltanet(n_sub, in_dtype):
    """W = R = N (every slot selected, dense softmax keys) must reproduce the
    Gated DeltaNet update exactly (up to rounding)."""
    N = n_sub * n_sub
    d = Dims(B=2, T=24, H=2, d_k=8, n_sub=n_sub, d_v=5, k_prime=n_sub, W=N, R=N, in_dtype=in_dtype)
    x = synth.make_inputs(d, seed=21)
    widx, wwt, ridx, rwt = oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d)
    M = synth.make_inputs(d, seed=21)["M0"][None].repeat(d.B, 0).copy()
    M0 = M.copy()
    o = oracle.scan(M, widx, wwt, ridx, rwt, x["v"], x["a"], x["b"], d)
    vf = dec(x["v"], d).astype(np.float64)
    for bb in range(d.B):
        for h in range(d.H):
            ks, qs = [], []
            for t in range(d.T):
                sk = brute_scores(x["k"][bb, t, h], x["C_w"][h], d).astype(np.float64)
                sq = brute_scores(x["q"][bb, t, h], x["C_r"][h], d).astype(np.float64)
                ks.append(scipy.special.softmax(sk))
                qs.append(scipy.special.softmax(sq))
            ro, rM = _dense_gdn(M0[bb, h], ks, qs, vf[bb, :, h], x["a"][bb, :, h].astype(np.float64),
                                x["b"][bb, :, h].astype(np.float64))
            scale = np.sqrt(np.mean(ro ** 2))
            np.testing.assert_allclose(o[bb, :, h], ro, rtol=0, atol=2e-6 * scale + 1e-9)
            np.testing.assert_allclose(M[bb, h], rM, rtol=0, atol=2e-6 * np.sqrt(np.mean(rM ** 2)))


def _scan_inputs(d, seed, hazard_slots=None):
    x = synth.make_inputs(d, seed)
    addr = synth.random_addressing(d, seed, hazard_slots=hazard_slots)
    return x, addr


def test_unselected_rows_bit_unchanged_and_b_zero_decay():
    d = dims(B=2, T=40, H=2, n_sub=6, W=3, R=2, d_v=7)
    x, ad = _scan_inputs(d, 8, hazard_slots=20)
    M = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    M0 = M.copy()
    bz = np.zeros_like(x["b"])
    oracle.scan(M, ad["widx"], ad["wwt"], ad["ridx"], ad["rwt"], x["v"], x["a"], bz, d)
    # replay: every written row is multiplied by a_t in token order (fp32 product,
    # correctly rounded); rows never written stay bit-identical
    ref = M0.copy()
    for bb in range(d.B):
        for h in range(d.H):
            for t in range(d.T):
                for s in ad["widx"][bb, t, h]:
                    ref[bb, h, s] = np.float32(x["a"][bb, t, h]) * ref[bb, h, s]
    np.testing.assert_array_equal(M, ref)
    written = np.zeros((d.B, d.H, d.N), bool)
    for bb in range(d.B):
        for h in range(d.H):
            written[bb, h, np.unique(ad["widx"][bb, :, h])] = True
    assert (~written).any()
    np.testing.assert_array_equal(M[~written], M0[~written])


def test_write_then_read_returns_v():
    """a = b = 1, W = R = 1, q = k: the read returns v_t exactly."""
    d = Dims(B=2, T=30, H=3, d_k=16, n_sub=8, d_v=6, k_prime=4, W=1, R=1, in_dtype="f32")
    x = synth.make_inputs(d, 13)
    widx, wwt, ridx, rwt = oracle.address(x["k"], x["k"], x["C_w"], x["C_w"], d)
    np.testing.assert_array_equal(widx, ridx)
    M = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    one = np.ones_like(x["a"])
    o = oracle.scan(M, widx, wwt, ridx, rwt, x["v"], one, one, d)
    np.testing.assert_array_equal(o, x["v"])


def test_hazard_closed_form():
    """The same (slots, weights) written and read for consecutive tokens with
    r = w: per column p_{n+1} = a_n p_n + b_n |w|^2 (v_n - a_n p_n), o_n = p_{n+1}."""
    d = dims(B=1, T=50, H=1, n_sub=8, W=5, R=5, d_v=6)
    x = synth.make_inputs(d, 17)
    g = np.random.default_rng(1)
    slots = g.permutation(d.N)[:d.W].astype(np.int32)
    w = g.random(d.W).astype(np.float32) + 0.1
    w = (w / w.sum()).astype(np.float32)
    widx = np.broadcast_to(slots, (1, d.T, 1, d.W)).copy()
    wwt = np.broadcast_to(w, (1, d.T, 1, d.W)).copy()
    M = x["M0"][None].copy()
    p = (w.astype(np.float64)[:, None] * M[0, 0, slots].astype(np.float64)).sum(0)
    o = oracle.scan(M, widx, wwt, widx, wwt, x["v"], x["a"], x["b"], d)
    w2 = float((w.astype(np.float64) ** 2).sum())
    ref = []
    for t in range(d.T):
        at, bt = float(x["a"][0, t, 0]), float(x["b"][0, t, 0])
        p = at * p + bt * w2 * (x["v"][0, t, 0].astype(np.float64) - at * p)
        ref.append(p.copy())
    np.testing.assert_allclose(o[0, :, 0], np.array(ref), rtol=0, atol=1e-5 * np.abs(ref).max())


def test_superposition_and_power_of_two_homogeneity():
    d = dims(B=2, T=30, H=2, n_sub=6, W=3, R=4, d_v=5)
    x, ad = _scan_inputs(d, 31, hazard_slots=12)
    M0 = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    args = (ad["widx"], ad["wwt"], ad["ridx"], ad["rwt"])

    def run(M, v):
        M = M.copy()
        return oracle.scan(M, *args, v, x["a"], x["b"], d), M

    o_full, M_full = run(M0, x["v"])
    o_m, M_m = run(M0, np.zeros_like(x["v"]))
    o_v, M_v = run(np.zeros_like(M0), x["v"])
    sc = np.abs(o_full).max()
    np.testing.assert_allclose(o_full, o_m + o_v, rtol=0, atol=1e-6 * sc)
    np.testing.assert_allclose(M_full, M_m + M_v, rtol=0, atol=1e-6 * np.abs(M_full).max())
    o2, M2 = run(2 * M0, 2 * x["v"])
    np.testing.assert_array_equal(o2, 2 * o_full)
    np.testing.assert_array_equal(M2, 2 * M_full)


def test_split_scan_equals_full_scan():
    d = dims(B=1, T=37, H=2, n_sub=5, W=3, R=3, d_v=4)
    x, ad = _scan_inputs(d, 41, hazard_slots=10)
    M = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    Mf = M.copy()
    o_full = oracle.scan(Mf, ad["widx"], ad["wwt"], ad["ridx"], ad["rwt"], x["v"], x["a"], x["b"], d)
    T1 = 15
    outs = []
    for lo, hi in ((0, T1), (T1, d.T)):
        dd = d.replace(T=hi - lo)
        sl = lambda z: np.ascontiguousarray(z[:, lo:hi])
        outs.append(oracle.scan(M, sl(ad["widx"]), sl(ad["wwt"]), sl(ad["ridx"]), sl(ad["rwt"]),
                                sl(x["v"]), sl(x["a"]), sl(x["b"]), dd))
    np.testing.assert_array_equal(np.concatenate(outs, 1), o_full)
    np.testing.assert_array_equal(M, Mf)


def test_permuting_sequences_permutes_outputs():
    d = dims(B=3, T=12, H=2, n_sub=5, W=2, R=3, d_v=4)
    x, ad = _scan_inputs(d, 51, hazard_slots=9)
    M = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    perm = [2, 0, 1]
    Mp = M[perm].copy()
    o = oracle.scan(M, ad["widx"], ad["wwt"], ad["ridx"], ad["rwt"], x["v"], x["a"], x["b"], d)
    P = lambda z: np.ascontiguousarray(z[perm])
    op = oracle.scan(Mp, P(ad["widx"]), P(ad["wwt"]), P(ad["ridx"]), P(ad["rwt"]), P(x["v"]),
                     P(x["a"]), P(x["b"]), d)
    np.testing.assert_array_equal(op, o[perm])
    np.testing.assert_array_equal(Mp, M[perm])


def test_state_init_copies_m0():
    d = dims(B=3, H=2, n_sub=4, d_v=3)
    M0 = np.random.default_rng(0).standard_normal((d.H, d.N, d.d_v)).astype(np.float32)
    M = oracle.state_init(M0, d)
    for bb in range(d.B):
        np.testing.assert_array_equal(M[bb], M0)


def test_oracle_rejects_bad_inputs():
    d = dims(B=1, T=2, H=1, n_sub=4, W=2, R=2, d_v=2)
    x, ad = _scan_inputs(d, 1)
    M = np.zeros((1, 1, d.N, d.d_v), np.float32)
    bad = ad["widx"].copy()
    bad[0, 1, 0, 1] = bad[0, 1, 0, 0]          # repeated write slot within a token
    with pytest.raises(oracle.OracleError):
        oracle.scan(M, bad, ad["wwt"], ad["ridx"], ad["rwt"], x["v"], x["a"], x["b"], d)
    bad = ad["ridx"].copy()
    bad[0, 0, 0, 0] = d.N
    with pytest.raises(oracle.OracleError):
        oracle.scan(M, ad["widx"], ad["wwt"], bad, ad["rwt"], x["v"], x["a"], x["b"], d)
    with pytest.raises(oracle.OracleError):
        oracle.address(x["k"], x["q"], x["C_w"], x["C_r"], d.replace(k_prime=5))
