"""The allocation-free scan entry point (sdm_scan_forward_noalloc, the
library's static scratch in place of a workspace) against sdm_scan_forward
on the same inputs, through the C ABI: bit for bit, on two calls in a row,
the second with a smaller input (the scratch keeps the first call's bytes)."""
import numpy as np
import pytest

import sdm_synth as synth
from sdm_synth import Dims

from gpu_helpers import note, to_dev, to_host

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


def _both(sdm, torch, d, seed, pool):
    x = synth.make_inputs(d, seed=seed)
    ad = synth.random_addressing(d, seed=seed, hazard_slots=pool)
    dims = sdm.dims_from(d)
    assert 0 < sdm.sdm_scan_workspace_size(dims) <= sdm.SDM_NOALLOC_SCRATCH_BYTES
    M0 = np.broadcast_to(x["M0"][None], (d.B,) + x["M0"].shape).copy()
    dev = {k: to_dev(v) for k, v in ad.items()}
    args = [dev["widx"], dev["wwt"], dev["ridx"], dev["rwt"], to_dev(x["v"]), to_dev(x["a"]), to_dev(x["b"])]
    M_ref = to_dev(M0)
    o_ref = sdm.scan_forward(M_ref, *args, dims)
    M_na = to_dev(M0)
    o_na = sdm.scan_forward_noalloc(M_na, *args, dims)
    torch.cuda.synchronize()
    return (to_host(o_ref), to_host(M_ref)), (to_host(o_na), to_host(M_na))


def test_noalloc_scan_matches_scan_forward_twice(sdm, torch):
    cases = [
        (Dims(B=3, T=300, H=4, d_k=128, n_sub=64, d_v=128, k_prime=32, W=32, R=32), 2000),
        (Dims(B=1, T=77, H=2, d_k=128, n_sub=32, d_v=64, k_prime=16, W=16, R=12), 300),
    ]
    for i, (d, pool) in enumerate(cases):
        note(f"noalloc scan call {i} {d}")
        (o_ref, M_ref), (o_na, M_na) = _both(sdm, torch, d, seed=61 + i, pool=pool)
        np.testing.assert_array_equal(o_na, o_ref)
        np.testing.assert_array_equal(M_na, M_ref)


def test_noalloc_scan_rejects_dims_beyond_the_scratch(sdm, torch):
    d = Dims(B=4, T=4096, H=16, d_k=128, n_sub=16, d_v=128, k_prime=16, W=32, R=32)
    dims = sdm.dims_from(d)
    assert sdm.sdm_scan_workspace_size(dims) > sdm.SDM_NOALLOC_SCRATCH_BYTES
    st = sdm.sdm_scan_forward_noalloc(1 << 40, 1 << 41, 1 << 42, 3 << 41, 1 << 43, 5 << 41, 3 << 42, 7 << 41,
                                      1 << 44, dims, stream=0, check=False)
    assert st == sdm.SDM_ERR_UNSUPPORTED
    assert "scratch" in sdm.sdm_last_error()
