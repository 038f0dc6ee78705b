"""GPU parity at the full sizes of the benchmarked layers, in the launch
configuration bench.py times.

The whole hot path runs on the GPU over the full layer; the oracle then
checks sampled outputs it can compute one by one: every (sequence, head)
chain of the scan is an independent recurrence and every token's addressing
is independent, so whole chains (or a chain's token prefix) and sampled
token rows are exact sub-problems.  The scan chains are replayed by the
oracle on the GPU's own slot lists and weights, so the scan check does not
depend on addressing near-ties.  Same bars as test_gpu_parity.
"""
import gc

import numpy as np
import pytest

import oracle
import sdm_synth as synth

from gpu_helpers import assert_close_rms, check_weights, compare_slot_lists, note, replay_weights, to_host

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


def _free(torch):
    gc.collect()
    torch.cuda.empty_cache()


def _sample_address(sdm, torch, x, d, gpu_lists, tsel):
    """Addressing of tokens tsel (all sequences and heads) against the oracle."""
    gw, gww, gr, grw = (to_host(t[:, tsel]) for t in gpu_lists)
    idx = torch.as_tensor(tsel, device="cuda")
    hx = {k: to_host(x[k].index_select(1, idx).contiguous()) for k in ("k", "q")}
    hx["C_w"], hx["C_r"] = to_host(x["C_w"]), to_host(x["C_r"])
    ds = d.replace(T=len(tsel))
    ow, oww, orr, orw = oracle.address(hx["k"], hx["q"], hx["C_w"], hx["C_r"], ds)
    rw, _ = compare_slot_lists(gw, ow, hx["k"], hx["C_w"], ds)
    rr, _ = compare_slot_lists(gr, orr, hx["q"], hx["C_r"], ds)
    rows = rw.size
    assert rw.sum() <= 0.01 * rows + 1 and rr.sum() <= 0.01 * rows + 1
    # every row's weights, near-tie rows against the oracle's softmax over the GPU's own list
    check_weights(gw, gww, ow, oww, hx["k"], hx["C_w"], ds)
    check_weights(gr, grw, orr, orw, hx["q"], hx["C_r"], ds)


def _replay_chain(x, d, lists, M_gpu, o_gpu, b, h, T):
    """The oracle scan of chain (b, h) over tokens [0, T) on the GPU's lists."""
    d1 = d.replace(B=1, H=1, T=T)
    sl = lambda t: np.ascontiguousarray(to_host(t[b:b + 1, :T, h:h + 1]))
    widx, wwt, ridx, rwt = (sl(t) for t in lists)
    M1 = np.ascontiguousarray(to_host(x["M0"][h])[None, None])
    o_ref = oracle.scan(M1, widx, wwt, ridx, rwt, sl(x["v"]), sl(x["a"]), sl(x["b"]), d1)
    assert_close_rms(o_gpu, o_ref[0, :, 0], what=f"o chain ({b},{h})")
    rows = np.unique(widx.ravel())
    assert_close_rms(M_gpu[rows], M1[0, 0][rows], what=f"M chain ({b},{h})")
    untouched = np.ones(d.N, bool)
    untouched[rows] = False
    return rows, untouched


@pytest.mark.parametrize("name", ["small", "prefill_1p4b"])
def test_fullsize_prefill_layer(sdm, torch, name):
    p = synth.PRESETS[name]
    d = p.dims
    note(f"full-size {name} {d}")
    x = synth.make_inputs_torch(d, seed=3, reuse_frac=p.reuse_frac, recall_frac=p.recall_frac)
    dims = sdm.dims_from(d)
    lists = sdm.pkm_address(x["k"], x["q"], x["C_w"], x["C_r"], dims)
    M = sdm.state_init(x["M0"], dims)
    o = sdm.scan_forward(M, *lists, x["v"], x["a"], x["b"], dims)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    _sample_address(sdm, torch, x, d, lists, np.sort(rng.choice(d.T, size=24, replace=False)))
    for b, h in ((0, 0), (d.B - 1, d.H - 1)):
        Mg = to_host(M[b, h])
        rows, untouched = _replay_chain(x, d, lists, Mg, to_host(o[b, :, h]), b, h, d.T)
        np.testing.assert_array_equal(Mg[untouched], to_host(x["M0"][h])[untouched])
    del x, lists, M, o
    _free(torch)


def test_fullsize_long_context_prefix(sdm, torch):
    """The 1M-token layer on the GPU; the oracle replays a 65,536-token prefix
    of two chains (a prefix of the recurrence is itself exact), and the
    benchmark's pipelined form of the whole step (sdm.prefill_chunks) equals
    the one-call prefill bit for bit."""
    p = synth.PRESETS["long_context"]
    d = p.dims
    note(f"full-size long_context {d}")
    x = synth.make_inputs_torch(d, seed=4, reuse_frac=p.reuse_frac, recall_frac=p.recall_frac)
    dims = sdm.dims_from(d)
    lists = sdm.pkm_address(x["k"], x["q"], x["C_w"], x["C_r"], dims)
    rng = np.random.default_rng(2)
    _sample_address(sdm, torch, x, d, lists, np.sort(rng.choice(d.T, size=8, replace=False)))
    # scan only the prefix (a separate call of T = 65,536 on the same lists),
    # then the whole layer, whose prefix outputs must agree exactly
    Tp = 65536
    dp = d.replace(T=Tp)
    pre = lambda t: t[:, :Tp].contiguous()
    Mp = sdm.state_init(x["M0"], sdm.dims_from(dp))
    op = sdm.scan_forward(Mp, *(pre(t) for t in lists), pre(x["v"]), pre(x["a"]), pre(x["b"]),
                          sdm.dims_from(dp))
    torch.cuda.synchronize()
    for h in (0, d.H - 1):
        _replay_chain(x, d, lists, to_host(Mp[0, h]), to_host(op[0, :, h]), 0, h, Tp)
    del Mp
    _free(torch)
    M = sdm.state_init(x["M0"], dims)
    o = sdm.scan_forward(M, *lists, x["v"], x["a"], x["b"], dims)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(o[:, :Tp]), to_host(op))
    del op
    _free(torch)
    # the step as the benchmark runs it: the chunks of sdm.prefill_chunks
    # (growing from 16,384 tokens), each chunk's addressing on a second
    # stream with at most one workgroup per CU (sdm_pkm_address_overlapped),
    # each chunk's scan on the main stream once its addressing is done; every
    # output equals the one-call prefill's
    chunks = sdm.prefill_chunks(d.T)
    note(f"full-size long_context pipelined over {len(chunks)} chunks")
    bounds = [(sum(chunks[:c]), sum(chunks[:c + 1])) for c in range(len(chunks))]
    dimsc = [sdm.dims_from(d.replace(T=n)) for n in chunks]
    lists2 = tuple(torch.empty_like(t) for t in lists)
    M2 = sdm.state_init(x["M0"], dims)
    o2 = torch.empty_like(o)
    ws_bytes = max(sdm.sdm_scan_workspace_size(dc) for dc in dimsc)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    start = torch.cuda.Event()
    start.record(main)
    side.wait_event(start)
    done = []
    for c, (t0, t1) in enumerate(bounds):
        sl = slice(t0, t1)
        sdm.sdm_pkm_address_overlapped(x["k"][:, sl], x["q"][:, sl], x["C_w"], x["C_r"], dimsc[c],
                                       *(t[:, sl] for t in lists2), side)
        e = torch.cuda.Event()
        e.record(side)
        done.append(e)
    for c, (t0, t1) in enumerate(bounds):
        sl = slice(t0, t1)
        main.wait_event(done[c])
        sdm.sdm_scan_forward(M2, *(t[:, sl] for t in lists2), x["v"][:, sl], x["a"][:, sl], x["b"][:, sl],
                             o2[:, sl], ws, ws_bytes, dimsc[c], main)
    torch.cuda.synchronize()
    for name, a, b in zip(("widx", "wwt", "ridx", "rwt"), lists, lists2):
        assert torch.equal(a, b), name
    assert torch.equal(o, o2), "o"
    assert torch.equal(M, M2), "M"
    del x, lists, lists2, M, M2, o, o2, ws
    _free(torch)


def test_fullsize_decode_layer(sdm, torch):
    """16 decode steps of all 32 x 8 chains of the decode layer (N = 2^20
    slots per head, 137 GB of state); eight chains are replayed by the oracle
    on the decode step's own slot lists."""
    p = synth.PRESETS["decode"]
    d = p.dims.replace(T=16)
    note(f"full-size decode {d}")
    x = synth.make_inputs_torch(d, seed=5)
    d1 = d.replace(T=1)
    dims1 = sdm.dims_from(d1)
    M = sdm.state_init(x["M0"], dims1)
    outs, wl, rl = [], [], []
    for t in range(d.T):
        wo = torch.empty((d.B, d.H, d.W), dtype=torch.int32, device="cuda")
        ro = torch.empty((d.B, d.H, d.R), dtype=torch.int32, device="cuda")
        o = sdm.decode_step(M, *(x[k][:, t].contiguous() for k in ("k", "q")), x["C_w"], x["C_r"],
                            *(x[k][:, t].contiguous() for k in ("v", "a", "b")), dims1, widx_out=wo, ridx_out=ro)
        outs.append(o)
        wl.append(wo)
        rl.append(ro)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    chains = [(0, 0), (d.B - 1, d.H - 1)] + [(int(rng.integers(d.B)), int(rng.integers(d.H))) for _ in range(6)]
    for b, h in chains:
        dc = d.replace(B=1, H=1)
        sl = lambda k: np.ascontiguousarray(to_host(x[k][b:b + 1, :, h:h + 1]))
        hx = {k: sl(k) for k in ("k", "q", "v", "a", "b")}
        for k in ("C_w", "C_r"):
            hx[k] = np.ascontiguousarray(to_host(x[k][h:h + 1]))
        ow, oww, orr, orw = oracle.address(hx["k"], hx["q"], hx["C_w"], hx["C_r"], dc)
        gw = np.stack([to_host(w[b, h]) for w in wl])[None, :, None]
        gr = np.stack([to_host(r[b, h]) for r in rl])[None, :, None]
        compare_slot_lists(gw, ow, hx["k"], hx["C_w"], dc)
        compare_slot_lists(gr, orr, hx["q"], hx["C_r"], dc)
        # the oracle scan replayed on the GPU's own lists (near-tie swaps included)
        ww = replay_weights(gw, ow, oww, hx["k"], hx["C_w"], dc)
        rw = replay_weights(gr, orr, orw, hx["q"], hx["C_r"], dc)
        M1 = np.ascontiguousarray(to_host(x["M0"][h])[None, None])
        o_ref = oracle.scan(M1, gw, ww, gr, rw, hx["v"], hx["a"], hx["b"], dc)
        o_dec = np.stack([to_host(o[b, h]) for o in outs])
        assert_close_rms(o_dec, o_ref[0, :, 0], what=f"decode o ({b},{h})")
        rows = np.unique(gw.ravel())
        Mg = to_host(M[b, h])
        assert_close_rms(Mg[rows], M1[0, 0][rows], what=f"decode M ({b},{h})")
        sample = rng.choice(d.N, size=4096, replace=False)
        sample = sample[~np.isin(sample, rows)]
        np.testing.assert_array_equal(Mg[sample], to_host(x["M0"][h])[sample])
    del x, M, outs
    _free(torch)
