"""Shared helpers for the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import numpy as np

import oracle
import sdm_synth as synth

NEAR_TIE = 1e-5   # oracle fp32 score gap below which two slots may swap


def to_dev(x: np.ndarray):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def to_host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def note(msg: str):
    print(f"[case] {msg}", flush=True)


def compare_slot_lists(gpu_idx: np.ndarray, orc_idx: np.ndarray, x: np.ndarray, C: np.ndarray, d,
                       tol: float = NEAR_TIE):
    """Index parity: the GPU list must equal the oracle list except at
    positions where the two slots' oracle fp32 scores differ by < tol.

    Returns (row_mask_differs, n_positions_differing).  Raises AssertionError
    on a difference that is not a near-tie or on a repeated slot."""
    n = gpu_idx.shape[-1]
    g = gpu_idx.reshape(-1, n)
    o = orc_idx.reshape(-1, n)
    # validity: distinct slots in range
    srt = np.sort(g, axis=1)
    assert (srt[:, 1:] != srt[:, :-1]).all(), "GPU list holds a repeated slot"
    assert (g >= 0).all() and (g < d.N).all(), "GPU slot out of range"
    diff = g != o
    rows_differ = diff.any(axis=1)
    if not diff.any():
        return rows_differ, 0
    rr, jj = np.nonzero(diff)
    sg = oracle.slot_scores(x, C, d, rr, g[rr, jj])
    so = oracle.slot_scores(x, C, d, rr, o[rr, jj])
    gap = np.abs(sg.astype(np.float64) - so.astype(np.float64))
    bad = gap >= tol
    assert not bad.any(), (f"{int(bad.sum())} slot differences are not near-ties; first at row "
                           f"{int(rr[bad][0])} pos {int(jj[bad][0])}: gpu {int(g[rr[bad][0], jj[bad][0]])} "
                           f"orc {int(o[rr[bad][0], jj[bad][0]])} gap {float(gap[bad][0]):.3g}")
    return rows_differ, int(diff.sum())


def list_weights(x: np.ndarray, C: np.ndarray, d, idx: np.ndarray, rows=None) -> np.ndarray:
    """The oracle's weights for given slot lists: the softmax, in fp64, of the
    oracle's fp32 slot scores of each list (what the oracle would return had
    it selected these slots).  idx [..., n] holds the lists of the flat
    token-head rows `rows` (default: every row of x, in order)."""
    n = idx.shape[-1]
    flat = np.ascontiguousarray(idx).reshape(-1, n)
    if rows is None:
        rows = np.arange(flat.shape[0])
    rows = np.asarray(rows, np.int64)
    if flat.shape[0] == 0:
        return np.zeros(idx.shape, np.float32)
    s = oracle.slot_scores(x, C, d, np.repeat(rows, n), flat.ravel()).reshape(-1, n).astype(np.float64)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32).reshape(idx.shape)


def replay_weights(gpu_idx: np.ndarray, orc_idx: np.ndarray, orc_wt: np.ndarray, x: np.ndarray, C: np.ndarray,
                   d) -> np.ndarray:
    """Weights of the GPU's own lists as the oracle defines them: the oracle's
    weights where the lists agree, the oracle's softmax over the GPU list's
    slot scores where a near-tie selected other slots."""
    n = gpu_idx.shape[-1]
    g = gpu_idx.reshape(-1, n)
    w = np.array(orc_wt, np.float32).reshape(-1, n)
    differ = np.nonzero((g != orc_idx.reshape(-1, n)).any(axis=1))[0]
    if differ.size:
        w[differ] = list_weights(x, C, d, g[differ], rows=differ)
    return w.reshape(gpu_idx.shape)


def check_weights(gpu_idx, gpu_wt, orc_idx, orc_wt, x, C, d, atol: float = 1e-6):
    """GPU weights within atol of the oracle's weights for the GPU's lists, on
    every row (near-tie rows included)."""
    ref = replay_weights(gpu_idx, orc_idx, orc_wt, x, C, d)
    np.testing.assert_allclose(gpu_wt, ref, rtol=0, atol=atol)


def rms(x: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.asarray(x, np.float64) ** 2)))


def assert_close_rms(got: np.ndarray, ref: np.ndarray, rel: float = 2e-3, what: str = ""):
    scale = rms(ref)
    err = float(np.max(np.abs(got.astype(np.float64) - ref.astype(np.float64)))) if got.size else 0.0
    assert err <= rel * scale + 1e-30, f"{what}: max abs err {err:.3g} > {rel} x RMS {scale:.3g}"
    return err, scale


def written_mask(widx: np.ndarray, d) -> np.ndarray:
    """[B,H,N] mask of slots written at least once."""
    m = np.zeros((d.B, d.H, d.N), bool)
    for b in range(d.B):
        for h in range(d.H):
            m[b, h, np.unique(widx[b, :, h].ravel())] = True
    return m


def device_inputs(x: dict):
    return {k: to_dev(v) for k, v in x.items()}


def gpu_dims(d, **kw):
    import sparse_memory_linear_pkm_amd as sdm
    return sdm.dims_from(d, **kw)
