"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/sdm.h declares, and rejects bad arguments on the host
before anything reaches the device."""
import ctypes
import os
import re

import pytest

import sparse_memory_linear_pkm_amd as sdm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdm_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = sdm.load_library()
    names = declared_functions()
    assert {"sdm_state_init", "sdm_pkm_address", "sdm_scan_forward", "sdm_decode_step",
            "sdm_scan_workspace_size", "sdm_status_string", "sdm_last_error", "sdm_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    nm = os.popen(f"nm -D --defined-only {sdm.lib_path()}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", nm), f"{n} not exported"


def test_status_strings_and_version():
    assert sdm.sdm_status_string(sdm.SDM_OK) == "ok"
    assert "invalid" in sdm.sdm_status_string(sdm.SDM_ERR_INVALID_ARG)
    assert "unsupported" in sdm.sdm_status_string(sdm.SDM_ERR_UNSUPPORTED)
    assert "HIP" in sdm.sdm_status_string(sdm.SDM_ERR_HIP)
    assert sdm.sdm_version() >= 10000


def good_dims(**kw):
    base = dict(B=2, T=8, H=2, d_k=128, n_sub=16, d_v=64, k_prime=8, W=8, R=8, in_dtype="bf16")
    base.update(kw)
    return sdm.dims_from(**base)


FAKE = 1 << 40  # never dereferenced: every case below fails validation first


def addr(dims, **ptrs):
    p = dict(k=FAKE, q=FAKE, C_w=FAKE, C_r=FAKE, widx=FAKE, wwt=FAKE + (1 << 30), ridx=FAKE + (2 << 30),
             rwt=FAKE + (3 << 30))
    p.update(ptrs)
    return sdm.sdm_pkm_address(p["k"], p["q"], p["C_w"], p["C_r"], dims, p["widx"], p["wwt"], p["ridx"],
                               p["rwt"], stream=0, check=False)


@pytest.mark.parametrize("kw,status", [
    (dict(d_k=127), sdm.SDM_ERR_INVALID_ARG),
    (dict(k_prime=17), sdm.SDM_ERR_INVALID_ARG),        # k' > n_sub
    (dict(W=65, k_prime=16), sdm.SDM_ERR_UNSUPPORTED),  # W <= k'^2 but above the kernel cap
    (dict(W=0), sdm.SDM_ERR_INVALID_ARG),
    (dict(R=100, k_prime=8), sdm.SDM_ERR_INVALID_ARG),  # R > k'^2
    (dict(d_v=48), sdm.SDM_ERR_UNSUPPORTED),
    (dict(d_k=96), sdm.SDM_ERR_UNSUPPORTED),            # bf16 MFMA needs d_k/2 % 32 == 0
    (dict(in_dtype=7), sdm.SDM_ERR_INVALID_ARG),
    (dict(reserved=1), sdm.SDM_ERR_INVALID_ARG),
    (dict(H=0), sdm.SDM_ERR_INVALID_ARG),
])
def test_address_rejects_bad_dims(kw, status):
    assert addr(good_dims(**kw)) == status
    assert sdm.sdm_last_error() != ""


def test_address_rejects_null_and_misaligned():
    assert addr(good_dims(), k=None) == sdm.SDM_ERR_INVALID_ARG
    assert addr(good_dims(), q=FAKE + 2) == sdm.SDM_ERR_INVALID_ARG
    # overlapping outputs
    assert addr(good_dims(), ridx=FAKE) == sdm.SDM_ERR_INVALID_ARG


def test_address_overlapped_validates_like_address():
    """sdm_pkm_address_overlapped shares sdm_pkm_address's checks."""
    def call(dims, k=FAKE, q=FAKE + (1 << 32), widx=FAKE + (2 << 32), ridx=FAKE + (3 << 32)):
        return sdm.sdm_pkm_address_overlapped(k, q, FAKE + (4 << 32), FAKE + (5 << 32), dims, widx,
                                              FAKE + (6 << 32), ridx, FAKE + (7 << 32), stream=0, check=False)
    assert call(good_dims(), k=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), q=FAKE + 2) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ridx=FAKE + (2 << 32)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(W=65, k_prime=16)) == sdm.SDM_ERR_UNSUPPORTED
    assert sdm.sdm_pkm_address_overlapped(None, None, None, None, good_dims(T=0), None, None, None, None, stream=0,
                                          check=False) == sdm.SDM_OK


def scan(dims, **ptrs):
    base = FAKE
    step = 1 << 34
    p = dict(M=base, widx=base + step, wwt=base + 2 * step, ridx=base + 3 * step, rwt=base + 4 * step,
             v=base + 5 * step, a=base + 6 * step, b=base + 7 * step, o=base + 8 * step, ws=None, ws_bytes=0)
    p.update(ptrs)
    return sdm.sdm_scan_forward(p["M"], p["widx"], p["wwt"], p["ridx"], p["rwt"], p["v"], p["a"], p["b"],
                                p["o"], p["ws"], p["ws_bytes"], dims, stream=0, check=False)


def test_scan_rejects_bad_arguments():
    d = good_dims()
    assert scan(d, o=FAKE + 64) == sdm.SDM_ERR_INVALID_ARG          # o overlaps M
    assert scan(d, M=None) == sdm.SDM_ERR_INVALID_ARG
    assert scan(d, M=FAKE + 4) == sdm.SDM_ERR_INVALID_ARG           # misaligned M
    assert scan(good_dims(W=70)) == sdm.SDM_ERR_UNSUPPORTED
    assert scan(good_dims(T=-1)) == sdm.SDM_ERR_INVALID_ARG
    assert scan(good_dims(n_sub=46341)) == sdm.SDM_ERR_INVALID_ARG
    # one (b, h) memory must stay below 4 GiB for 32-bit buffer offsets
    assert scan(good_dims(n_sub=4096, d_v=128)) == sdm.SDM_ERR_UNSUPPORTED
    need = sdm.sdm_scan_workspace_size(d)
    if need:
        assert scan(d, ws=None, ws_bytes=0) == sdm.SDM_ERR_INVALID_ARG


def test_decode_rejects_bad_arguments():
    d = good_dims(T=2)
    st = sdm.sdm_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + (1 << 36), None, None, d,
                             stream=0, check=False)
    assert st == sdm.SDM_ERR_INVALID_ARG
    d = good_dims(T=1)
    st = sdm.sdm_decode_step(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + (1 << 36), None, None, d,
                             stream=0, check=False)
    assert st == sdm.SDM_ERR_INVALID_ARG


def test_state_init_rejects_overlap():
    d = good_dims()
    assert sdm.sdm_state_init(FAKE, FAKE + 16, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG
    assert sdm.sdm_state_init(None, FAKE, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG
    big = good_dims(B=1 << 31)
    assert sdm.sdm_state_init(FAKE, FAKE + (1 << 40), big, stream=0, check=False) == sdm.SDM_ERR_UNSUPPORTED


def test_workspace_size_is_host_only():
    assert sdm.sdm_scan_workspace_size(good_dims()) >= 0
    bad = good_dims(W=0)
    assert sdm.sdm_scan_workspace_size(bad) == 0


def test_binding_raises_with_detail():
    with pytest.raises(sdm.SdmError) as ei:
        sdm.sdm_pkm_address(None, FAKE, FAKE, FAKE, good_dims(), FAKE, FAKE, FAKE, FAKE, stream=0)
    assert ei.value.status == sdm.SDM_ERR_INVALID_ARG
    assert "NULL" in str(ei.value)


def gates_call(dims, **ptrs):
    p = dict(a_raw=FAKE, b_raw=FAKE + (1 << 30), A=FAKE + (2 << 30), dt=FAKE + (3 << 30), a=FAKE + (4 << 30),
             b=FAKE + (5 << 30))
    p.update(ptrs)
    return sdm.sdm_gates(p["a_raw"], p["b_raw"], p["A"], p["dt"], dims, p["a"], p["b"], stream=0, check=False)


def test_gates_rejects_bad_arguments():
    assert gates_call(good_dims(H=0)) == sdm.SDM_ERR_INVALID_ARG
    assert gates_call(good_dims(T=-1)) == sdm.SDM_ERR_INVALID_ARG
    assert gates_call(good_dims(reserved=1)) == sdm.SDM_ERR_INVALID_ARG
    assert gates_call(good_dims(), A=None) == sdm.SDM_ERR_INVALID_ARG
    assert gates_call(good_dims(), a=FAKE + (4 << 30) + 2) == sdm.SDM_ERR_INVALID_ARG
    # a may be a_raw exactly (in place), not a shifted view of it, and never b
    assert gates_call(good_dims(), a=FAKE + 4) == sdm.SDM_ERR_INVALID_ARG
    assert gates_call(good_dims(), b=FAKE + (4 << 30)) == sdm.SDM_ERR_INVALID_ARG
    assert gates_call(good_dims(), a=FAKE + (1 << 30)) == sdm.SDM_ERR_INVALID_ARG   # a over b_raw
    # nothing to do: validation passes and no kernel is launched
    assert gates_call(good_dims(B=0)) == sdm.SDM_OK


def norm_call(dims, eps=1e-5, **ptrs):
    p = dict(o=FAKE, g=FAKE + (1 << 30), gamma=FAKE + (2 << 30), y=FAKE + (3 << 30))
    p.update(ptrs)
    return sdm.sdm_output_norm_gate(p["o"], p["g"], p["gamma"], eps, dims, p["y"], stream=0, check=False)


@pytest.mark.parametrize("kw,eps,status", [
    (dict(d_v=48), 1e-5, sdm.SDM_ERR_UNSUPPORTED),
    (dict(d_v=2048), 1e-5, sdm.SDM_ERR_UNSUPPORTED),
    (dict(in_dtype=3), 1e-5, sdm.SDM_ERR_INVALID_ARG),
    (dict(H=0), 1e-5, sdm.SDM_ERR_INVALID_ARG),
    (dict(), -1.0, sdm.SDM_ERR_INVALID_ARG),
    (dict(), float("nan"), sdm.SDM_ERR_INVALID_ARG),
    (dict(), float("inf"), sdm.SDM_ERR_INVALID_ARG),
])
def test_norm_gate_rejects_bad_dims(kw, eps, status):
    assert norm_call(good_dims(**kw), eps) == status


def test_norm_gate_rejects_null_misaligned_overlap():
    assert norm_call(good_dims(), g=None) == sdm.SDM_ERR_INVALID_ARG
    assert norm_call(good_dims(), o=FAKE + 8) == sdm.SDM_ERR_INVALID_ARG
    assert norm_call(good_dims(), y=FAKE + (3 << 30) + 4) == sdm.SDM_ERR_INVALID_ARG
    assert norm_call(good_dims(), y=FAKE + 64) == sdm.SDM_ERR_INVALID_ARG   # y inside o
    assert norm_call(good_dims(B=0)) == sdm.SDM_OK


def test_calls_without_work_accept_null_and_do_nothing():
    # zero-sized work: valid dims, NULL buffers (what empty tensors give), nothing launched
    assert sdm.sdm_state_init(None, None, good_dims(B=0), stream=0, check=False) == sdm.SDM_OK
    assert addr(good_dims(T=0), k=None, q=None, widx=None) == sdm.SDM_OK
    assert sdm.sdm_scan_forward(None, None, None, None, None, None, None, None, None, None, 0, good_dims(T=0),
                                stream=0, check=False) == sdm.SDM_OK
    assert sdm.sdm_decode_step(None, None, None, None, None, None, None, None, None, None, None,
                               good_dims(B=0, T=1), stream=0, check=False) == sdm.SDM_OK
    assert gates_call(good_dims(T=0), a_raw=None, a=None) == sdm.SDM_OK
    assert norm_call(good_dims(B=0), o=None, y=None) == sdm.SDM_OK
    # invalid dims are still rejected when there is no work
    assert addr(good_dims(T=0, d_k=127)) == sdm.SDM_ERR_INVALID_ARG
    assert norm_call(good_dims(T=0), eps=-1.0) == sdm.SDM_ERR_INVALID_ARG


def test_gdn_rejects_bad_arguments():
    def call(dims, **ptrs):
        p = dict(S=FAKE, k=FAKE + (1 << 30), q=FAKE + (2 << 30), v=FAKE + (3 << 30), a=FAKE + (4 << 30),
                 b=FAKE + (5 << 30), o=FAKE + (6 << 30))
        p.update(ptrs)
        return sdm.sdm_gdn_dense_forward(p["S"], p["k"], p["q"], p["v"], p["a"], p["b"], p["o"], dims, stream=0,
                                         check=False)
    assert call(good_dims(d_k=48)) == sdm.SDM_ERR_UNSUPPORTED
    assert call(good_dims(d_k=512)) == sdm.SDM_ERR_UNSUPPORTED
    assert call(good_dims(H=0)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(in_dtype=5)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), k=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), q=FAKE + (2 << 30) + 8) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), o=FAKE + 4) == sdm.SDM_ERR_INVALID_ARG          # o over S
    assert call(good_dims(T=0), S=None, k=None) == sdm.SDM_OK


def test_scan_backward_rejects_bad_arguments():
    def call(dims, **ptrs):
        names = ("dM", "widx", "wwt", "ridx", "rwt", "v", "a", "b", "dout", "xs", "zs", "dv", "da", "db", "dw", "dr",
                 "ws")
        p = {n: FAKE + (i << 30) for i, n in enumerate(names)}
        ws_bytes = ptrs.pop("ws_bytes", 1 << 29)
        p.update(ptrs)
        return sdm.sdm_scan_backward(*(p[n] for n in names), ws_bytes, dims, stream=0, check=False)
    assert call(good_dims(d_v=512)) == sdm.SDM_ERR_UNSUPPORTED
    assert call(good_dims(W=65, k_prime=16)) == sdm.SDM_ERR_UNSUPPORTED
    assert call(good_dims(W=0)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), xs=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dv=FAKE + (11 << 30) + 4) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), da=FAKE + (11 << 30)) == sdm.SDM_ERR_INVALID_ARG   # da over dv
    # outputs over inputs: dv over v, dw over the saved write rows, dM over dout
    assert call(good_dims(), dv=FAKE + (5 << 30)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dw=FAKE + (9 << 30) + 64) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dM=FAKE + (8 << 30)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(T=0), dM=None) == sdm.SDM_OK
    # the lane-parallel path's workspace: its size, too small, misaligned, over dM, an output or an input
    need = sdm.sdm_scan_backward_workspace_size(good_dims())
    assert need > 0
    assert call(good_dims(), ws_bytes=need - 1) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws=None, ws_bytes=need) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws=FAKE + (16 << 30) + 4) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws=FAKE + 64) == sdm.SDM_ERR_INVALID_ARG            # over dM
    assert call(good_dims(), ws=FAKE + (14 << 30)) == sdm.SDM_ERR_INVALID_ARG    # over dw
    assert call(good_dims(), ws=FAKE + (9 << 30)) == sdm.SDM_ERR_INVALID_ARG     # over xsave
    # beyond the lane-parallel path's 2 GiB ranges the size is 0 (token-serial kernels)
    assert sdm.sdm_scan_backward_workspace_size(good_dims(T=1 << 22)) == 0
    assert sdm.sdm_scan_backward_workspace_size(good_dims(d_v=512)) == 0


def test_scan_noalloc_rejects_beyond_scratch_on_the_host():
    """The allocation-free scan refuses dims whose preparation streams exceed
    its static scratch before touching the device, and a call without work
    succeeds on NULL buffers."""
    big = good_dims(B=4, T=4096, H=16, d_v=128, W=32, R=32, k_prime=16)
    assert sdm.sdm_scan_workspace_size(big) > sdm.SDM_NOALLOC_SCRATCH_BYTES
    args = [FAKE + (i << 30) for i in range(9)]
    assert sdm.sdm_scan_forward_noalloc(*args, big, stream=0, check=False) == sdm.SDM_ERR_UNSUPPORTED
    assert "scratch" in sdm.sdm_last_error()
    assert sdm.sdm_scan_forward_noalloc(*args, good_dims(W=0), stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG
    assert sdm.sdm_scan_forward_noalloc(*([None] * 9), good_dims(T=0), stream=0, check=False) == sdm.SDM_OK


def test_gated_scan_rejects_bad_arguments():
    def call(dims, **ptrs):
        names = ("M", "widx", "wwt", "ridx", "rwt", "v", "a_raw", "b_raw", "A", "dt", "o", "ws")
        p = {n: FAKE + (i << 30) for i, n in enumerate(names)}
        p.update(ptrs)
        return sdm.sdm_scan_forward_gated(*(p[n] for n in names), 1 << 29, dims, stream=0, check=False)
    assert call(good_dims(), A=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dt=FAKE + (9 << 30) + 2) == sdm.SDM_ERR_INVALID_ARG    # misaligned
    assert call(good_dims(), A=FAKE + 64) == sdm.SDM_ERR_INVALID_ARG                # A inside M
    assert call(good_dims(), dt=FAKE + (10 << 30) + 16) == sdm.SDM_ERR_INVALID_ARG  # dt_bias inside o
    assert call(good_dims(), dt=FAKE + (11 << 30)) == sdm.SDM_ERR_INVALID_ARG       # dt_bias over the workspace
    assert call(good_dims(W=0)) == sdm.SDM_ERR_INVALID_ARG
    assert sdm.sdm_scan_forward_gated(*([None] * 12), 0, good_dims(T=0), stream=0, check=False) == sdm.SDM_OK


def test_scan_forward_save_needs_both_buffers():
    dims = good_dims()
    args = [FAKE + (i << 30) for i in range(9)]
    st = sdm.sdm_scan_forward_save(*args, None, FAKE + (10 << 30), FAKE + (11 << 30), 1 << 40, dims, stream=0,
                                   check=False)
    assert st == sdm.SDM_ERR_INVALID_ARG


def test_address_backward_rejects_bad_arguments():
    def call(dims, ws_bytes=1 << 40, **ptrs):
        names = ("k", "q", "Cw", "Cr", "widx", "wwt", "ridx", "rwt", "dw", "dr")
        p = {n: FAKE + (i << 30) for i, n in enumerate(names)}
        outs = {"dk": FAKE + (10 << 30), "dq": FAKE + (11 << 30), "dCw": FAKE + (12 << 30), "dCr": FAKE + (13 << 30),
                "ws": FAKE + (14 << 30)}
        p.update(outs)
        p.update(ptrs)
        return sdm.sdm_address_backward(*(p[n] for n in names), dims, p["dk"], p["dq"], p["dCw"], p["dCr"], p["ws"],
                                        ws_bytes, stream=0, check=False)
    assert call(good_dims(d_k=127)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dk=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws_bytes=16) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dq=FAKE + (10 << 30) + 256) == sdm.SDM_ERR_INVALID_ARG    # dq inside dk
    # outputs or workspace over inputs: dk over k, the workspace over C_w, dC_w over dw
    assert call(good_dims(), dk=FAKE) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws=FAKE + (2 << 30) + 16) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dCw=FAKE + (8 << 30)) == sdm.SDM_ERR_INVALID_ARG
    assert sdm.sdm_address_backward_workspace_size(good_dims()) > 0
    assert call(good_dims(T=0), k=None) == sdm.SDM_OK


def test_gates_backward_rejects_bad_arguments():
    def call(dims, ws_bytes=1 << 40, **ptrs):
        names = ("a_raw", "b_raw", "A", "dt", "da", "db", "da_raw", "db_raw", "dA", "ddt", "ws")
        p = {n: FAKE + (i << 30) for i, n in enumerate(names)}
        p.update(ptrs)
        return sdm.sdm_gates_backward(*(p[n] for n in names[:6]), dims, *(p[n] for n in names[6:]), ws_bytes,
                                      stream=0, check=False)
    assert call(good_dims(H=0)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(reserved=1)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), da=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dA=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), db_raw=FAKE + (7 << 30) + 2) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), da_raw=FAKE + (4 << 30)) == sdm.SDM_ERR_INVALID_ARG      # in place over da
    assert call(good_dims(), ddt=FAKE + (8 << 30) + 4) == sdm.SDM_ERR_INVALID_ARG     # ddt over dA
    assert call(good_dims(), ws=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws_bytes=4) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws=FAKE + (6 << 30) + 64) == sdm.SDM_ERR_INVALID_ARG    # workspace inside da_raw
    assert call(good_dims(T=0), a_raw=None, dA=None, ws=None) == sdm.SDM_OK
    # per head, two sums for each part of the tokens
    assert sdm.sdm_gates_backward_workspace_size(good_dims(B=2, T=8, H=2)) == 2 * 1 * 2 * 4
    assert sdm.sdm_gates_backward_workspace_size(good_dims(B=8, T=8192, H=16)) == 2 * 512 * 16 * 4
    assert sdm.sdm_gates_backward_workspace_size(good_dims(T=0)) == 0


def test_norm_gate_backward_rejects_bad_arguments():
    def call(dims, eps=1e-5, ws_bytes=1 << 40, **ptrs):
        names = ("o", "g", "gamma", "dy", "dout", "dg", "dgamma", "ws")
        p = {n: FAKE + (i << 30) for i, n in enumerate(names)}
        p.update(ptrs)
        return sdm.sdm_output_norm_gate_backward(p["o"], p["g"], p["gamma"], eps, p["dy"], dims, p["dout"], p["dg"],
                                                 p["dgamma"], p["ws"], ws_bytes, stream=0, check=False)
    assert call(good_dims(d_v=48)) == sdm.SDM_ERR_UNSUPPORTED
    assert call(good_dims(d_v=2048)) == sdm.SDM_ERR_UNSUPPORTED
    assert call(good_dims(in_dtype=3)) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), eps=float("nan")) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dy=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws=None) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), ws_bytes=16) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dout=FAKE + (4 << 30) + 8) == sdm.SDM_ERR_INVALID_ARG
    assert call(good_dims(), dg=FAKE + (3 << 30)) == sdm.SDM_ERR_INVALID_ARG           # dg over dy
    assert call(good_dims(), ws=FAKE + (4 << 30) + 256) == sdm.SDM_ERR_INVALID_ARG     # workspace inside dout
    assert call(good_dims(B=0), o=None, ws=None) == sdm.SDM_OK
    # one partial row of d_v floats per workgroup, at most 1024 workgroups
    assert sdm.sdm_output_norm_gate_backward_workspace_size(good_dims(B=2, T=8, H=2)) == 4 * 64
    big = good_dims(B=4, T=4096, H=16, d_v=128)
    assert sdm.sdm_output_norm_gate_backward_workspace_size(big) == 4 * 1024 * 128
    assert sdm.sdm_output_norm_gate_backward_workspace_size(good_dims(d_v=48)) == 0


def test_cow_calls_reject_bad_arguments():
    d = good_dims(T=1)
    nb = sdm.sdm_cow_bitmap_bytes(d)
    assert nb == 4 * d.B * d.H * ((d.n_sub * d.n_sub + 31) // 32)
    assert sdm.sdm_cow_bitmap_bytes(good_dims(H=0)) == 0
    assert sdm.sdm_cow_reset(None, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG
    assert sdm.sdm_cow_reset(FAKE + 2, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG
    assert sdm.sdm_cow_reset(None, good_dims(B=0, T=1), stream=0, check=False) == sdm.SDM_OK
    M, M0, tb = FAKE, FAKE + (1 << 36), FAKE + (2 << 36)
    assert sdm.sdm_cow_materialize(M, None, tb, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG
    assert sdm.sdm_cow_materialize(M, M + 64, tb, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG   # M0 in M
    assert sdm.sdm_cow_materialize(M, M0, M0 + 16, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG  # bitmap in M0
    assert sdm.sdm_cow_materialize(M, M0 + 8, tb, d, stream=0, check=False) == sdm.SDM_ERR_INVALID_ARG   # misaligned
    ins = [FAKE + ((3 + i) << 36) for i in range(8)]   # k, q, C_w, C_r, v, a, b, o
    step = lambda M_, M0_, tb_, dims=d: sdm.sdm_decode_step_cow(M_, M0_, tb_, *ins, None, None, dims, stream=0,
                                                                check=False)
    assert step(M, None, tb) == sdm.SDM_ERR_INVALID_ARG
    assert step(M, M0, None) == sdm.SDM_ERR_INVALID_ARG
    assert step(M, M0, ins[7]) == sdm.SDM_ERR_INVALID_ARG                       # bitmap over o
    assert step(M, M0, tb, dims=good_dims(T=2)) == sdm.SDM_ERR_INVALID_ARG     # T must be 1
    assert step(None, None, None, dims=good_dims(B=0, T=1)) == sdm.SDM_OK
