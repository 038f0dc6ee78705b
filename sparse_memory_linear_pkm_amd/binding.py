"""ctypes binding of the C ABI declared in ``include/sdm.h``.

Low-level functions carry the C names and take raw device pointers (ints) or
torch tensors; the convenience wrappers (``state_init``, ``pkm_address``,
``scan_forward``, ``decode_step``) allocate outputs with torch and check
shapes, dtypes and devices before calling the library.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libsdm.so"

SDM_OK, SDM_ERR_INVALID_ARG, SDM_ERR_UNSUPPORTED, SDM_ERR_HIP = 0, -1, -2, -3
SDM_F32, SDM_BF16 = 0, 1
SDM_NOALLOC_SCRATCH_BYTES = 134217728   # static scratch of sdm_scan_forward_noalloc (include/sdm.h)


class SdmError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"{what}: {sdm_status_string(status)} ({status}): {detail}")
        self.status = status


class SdmDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "T", "H", "d_k", "n_sub", "d_v", "k_prime", "W", "R")] + \
               [("in_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


def lib_path() -> str:
    return os.environ.get("SDM_LIBRARY", os.path.join(HERE, _LIB_NAME))


_lib = None


def load_library():
    """Load libsdm.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m sparse_memory_linear_pkm_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32 = ctypes.c_void_p, ctypes.c_int
    D = ctypes.POINTER(SdmDims)
    sigs = {
        "sdm_state_init": [P, P, D, P],
        "sdm_pkm_address": [P, P, P, P, D, P, P, P, P, P],
        "sdm_pkm_address_overlapped": [P, P, P, P, D, P, P, P, P, P],
        "sdm_scan_forward": [P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, D, P],
        "sdm_decode_step": [P, P, P, P, P, P, P, P, P, P, P, D, P],
        "sdm_gates": [P, P, P, P, D, P, P, P],
        "sdm_output_norm_gate": [P, P, P, ctypes.c_float, D, P, P],
        "sdm_gdn_dense_forward": [P, P, P, P, P, P, P, D, P],
        "sdm_scan_forward_save": [P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, D, P],
        "sdm_scan_forward_noalloc": [P, P, P, P, P, P, P, P, P, D, P],
        "sdm_scan_forward_gated": [P] * 12 + [ctypes.c_size_t, D, P],
        "sdm_scan_backward": [P] * 17 + [ctypes.c_size_t, D, P],
        "sdm_address_backward": [P] * 10 + [D, P, P, P, P, P, ctypes.c_size_t, P],
        "sdm_gates_backward": [P] * 6 + [D, P, P, P, P, P, ctypes.c_size_t, P],
        "sdm_cow_reset": [P, D, P],
        "sdm_decode_step_cow": [P] * 13 + [D, P],
        "sdm_cow_materialize": [P, P, P, D, P],
        "sdm_output_norm_gate_backward": [P, P, P, ctypes.c_float, P, D, P, P, P, P, ctypes.c_size_t, P],
    }
    for name, args in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = I32
    lib.sdm_cow_bitmap_bytes.argtypes = [D]
    lib.sdm_cow_bitmap_bytes.restype = ctypes.c_size_t
    lib.sdm_scan_workspace_size.argtypes = [D]
    lib.sdm_scan_workspace_size.restype = ctypes.c_size_t
    lib.sdm_scan_backward_workspace_size.argtypes = [D]
    lib.sdm_scan_backward_workspace_size.restype = ctypes.c_size_t
    lib.sdm_address_backward_workspace_size.argtypes = [D]
    lib.sdm_address_backward_workspace_size.restype = ctypes.c_size_t
    lib.sdm_gates_backward_workspace_size.argtypes = [D]
    lib.sdm_gates_backward_workspace_size.restype = ctypes.c_size_t
    lib.sdm_output_norm_gate_backward_workspace_size.argtypes = [D]
    lib.sdm_output_norm_gate_backward_workspace_size.restype = ctypes.c_size_t
    lib.sdm_status_string.argtypes = [I32]
    lib.sdm_status_string.restype = ctypes.c_char_p
    lib.sdm_last_error.argtypes = []
    lib.sdm_last_error.restype = ctypes.c_char_p
    lib.sdm_version.argtypes = []
    lib.sdm_version.restype = I32
    _lib = lib
    return lib


def dims_from(d=None, **kw) -> SdmDims:
    """SdmDims from an object with B, T, H, d_k, n_sub, d_v, k_prime, W, R and
    in_dtype ("bf16"/"f32" or SDM_BF16/SDM_F32) attributes, or keywords."""
    vals = {}
    for n in ("B", "T", "H", "d_k", "n_sub", "d_v", "k_prime", "W", "R", "in_dtype"):
        if n in kw:
            vals[n] = kw[n]
        elif d is not None:
            vals[n] = getattr(d, n)
        else:
            raise TypeError(f"missing dimension {n}")
    dt = vals["in_dtype"]
    if isinstance(dt, str):
        dt = {"bf16": SDM_BF16, "f32": SDM_F32}[dt]
    out = SdmDims(*(int(vals[n]) for n in ("B", "T", "H", "d_k", "n_sub", "d_v", "k_prime", "W", "R")),
                  int(dt), int(kw.get("reserved", 0)))
    return out


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, what: str):
    if status != SDM_OK:
        raise SdmError(status, what, sdm_last_error())


# ---------------------------------------------------------------------------
# the C calls, same names
# ---------------------------------------------------------------------------
def sdm_status_string(status: int) -> str:
    return load_library().sdm_status_string(int(status)).decode()


def sdm_last_error() -> str:
    return load_library().sdm_last_error().decode()


def sdm_version() -> int:
    return load_library().sdm_version()


def sdm_scan_workspace_size(dims: SdmDims) -> int:
    return int(load_library().sdm_scan_workspace_size(ctypes.byref(dims)))


def sdm_state_init(M, M0, dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_state_init(_ptr(M), _ptr(M0), ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_state_init")
    return st


def sdm_pkm_address(k, q, C_w, C_r, dims: SdmDims, widx, wwt, ridx, rwt, stream=None, *,
                    check: bool = True) -> int:
    st = load_library().sdm_pkm_address(_ptr(k), _ptr(q), _ptr(C_w), _ptr(C_r), ctypes.byref(dims),
                                        _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt), _stream(stream))
    if check:
        _check(st, "sdm_pkm_address")
    return st


def sdm_pkm_address_overlapped(k, q, C_w, C_r, dims: SdmDims, widx, wwt, ridx, rwt, stream=None, *,
                               check: bool = True) -> int:
    st = load_library().sdm_pkm_address_overlapped(_ptr(k), _ptr(q), _ptr(C_w), _ptr(C_r), ctypes.byref(dims),
                                                   _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt), _stream(stream))
    if check:
        _check(st, "sdm_pkm_address_overlapped")
    return st


def sdm_scan_forward(M, widx, wwt, ridx, rwt, v, a, b, o, workspace, workspace_bytes: int,
                     dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_scan_forward(_ptr(M), _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt), _ptr(v),
                                         _ptr(a), _ptr(b), _ptr(o), _ptr(workspace),
                                         int(workspace_bytes), ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_scan_forward")
    return st


def sdm_scan_forward_noalloc(M, widx, wwt, ridx, rwt, v, a, b, o, dims: SdmDims, stream=None, *,
                             check: bool = True) -> int:
    st = load_library().sdm_scan_forward_noalloc(_ptr(M), _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt), _ptr(v),
                                                 _ptr(a), _ptr(b), _ptr(o), ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_scan_forward_noalloc")
    return st


def sdm_decode_step(M, k, q, C_w, C_r, v, a, b, o, widx_out, ridx_out, dims: SdmDims, stream=None, *,
                    check: bool = True) -> int:
    st = load_library().sdm_decode_step(_ptr(M), _ptr(k), _ptr(q), _ptr(C_w), _ptr(C_r), _ptr(v), _ptr(a),
                                        _ptr(b), _ptr(o), _ptr(widx_out), _ptr(ridx_out),
                                        ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_decode_step")
    return st


def sdm_cow_bitmap_bytes(dims: SdmDims) -> int:
    return int(load_library().sdm_cow_bitmap_bytes(ctypes.byref(dims)))


def sdm_cow_reset(touched, dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_cow_reset(_ptr(touched), ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_cow_reset")
    return st


def sdm_decode_step_cow(M, M0, touched, k, q, C_w, C_r, v, a, b, o, widx_out, ridx_out, dims: SdmDims, stream=None,
                        *, check: bool = True) -> int:
    st = load_library().sdm_decode_step_cow(_ptr(M), _ptr(M0), _ptr(touched), _ptr(k), _ptr(q), _ptr(C_w), _ptr(C_r),
                                            _ptr(v), _ptr(a), _ptr(b), _ptr(o), _ptr(widx_out), _ptr(ridx_out),
                                            ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_decode_step_cow")
    return st


def sdm_cow_materialize(M, M0, touched, dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_cow_materialize(_ptr(M), _ptr(M0), _ptr(touched), ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_cow_materialize")
    return st


def sdm_gates(a_raw, b_raw, A, dt_bias, dims: SdmDims, a, b, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_gates(_ptr(a_raw), _ptr(b_raw), _ptr(A), _ptr(dt_bias), ctypes.byref(dims), _ptr(a),
                                  _ptr(b), _stream(stream))
    if check:
        _check(st, "sdm_gates")
    return st


def sdm_output_norm_gate(o, g, gamma, eps: float, dims: SdmDims, y, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_output_norm_gate(_ptr(o), _ptr(g), _ptr(gamma), float(eps), ctypes.byref(dims),
                                             _ptr(y), _stream(stream))
    if check:
        _check(st, "sdm_output_norm_gate")
    return st


def sdm_gates_backward_workspace_size(dims: SdmDims) -> int:
    return int(load_library().sdm_gates_backward_workspace_size(ctypes.byref(dims)))


def sdm_gates_backward(a_raw, b_raw, A, dt_bias, da, db, dims: SdmDims, da_raw, db_raw, dA, ddt_bias, workspace,
                       workspace_bytes: int, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_gates_backward(_ptr(a_raw), _ptr(b_raw), _ptr(A), _ptr(dt_bias), _ptr(da), _ptr(db),
                                           ctypes.byref(dims), _ptr(da_raw), _ptr(db_raw), _ptr(dA),
                                           _ptr(ddt_bias), _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "sdm_gates_backward")
    return st


def sdm_output_norm_gate_backward_workspace_size(dims: SdmDims) -> int:
    return int(load_library().sdm_output_norm_gate_backward_workspace_size(ctypes.byref(dims)))


def sdm_output_norm_gate_backward(o, g, gamma, eps: float, dy, dims: SdmDims, dout, dg, dgamma, workspace,
                                  workspace_bytes: int, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_output_norm_gate_backward(_ptr(o), _ptr(g), _ptr(gamma), float(eps), _ptr(dy),
                                                      ctypes.byref(dims), _ptr(dout), _ptr(dg), _ptr(dgamma),
                                                      _ptr(workspace), int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "sdm_output_norm_gate_backward")
    return st


def sdm_scan_forward_gated(M, widx, wwt, ridx, rwt, v, a_raw, b_raw, A, dt_bias, o, workspace, workspace_bytes: int,
                           dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_scan_forward_gated(_ptr(M), _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt), _ptr(v),
                                               _ptr(a_raw), _ptr(b_raw), _ptr(A), _ptr(dt_bias), _ptr(o),
                                               _ptr(workspace), int(workspace_bytes), ctypes.byref(dims),
                                               _stream(stream))
    if check:
        _check(st, "sdm_scan_forward_gated")
    return st


def sdm_scan_forward_save(M, widx, wwt, ridx, rwt, v, a, b, o, xsave, zsave, workspace, workspace_bytes: int,
                          dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_scan_forward_save(_ptr(M), _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt), _ptr(v),
                                              _ptr(a), _ptr(b), _ptr(o), _ptr(xsave), _ptr(zsave), _ptr(workspace),
                                              int(workspace_bytes), ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_scan_forward_save")
    return st


def sdm_scan_backward_workspace_size(dims: SdmDims) -> int:
    return int(load_library().sdm_scan_backward_workspace_size(ctypes.byref(dims)))


def sdm_scan_backward(dM, widx, wwt, ridx, rwt, v, a, b, dout, xsave, zsave, dv, da, db, dw, dr, workspace,
                      workspace_bytes: int, dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_scan_backward(_ptr(dM), _ptr(widx), _ptr(wwt), _ptr(ridx), _ptr(rwt), _ptr(v), _ptr(a),
                                          _ptr(b), _ptr(dout), _ptr(xsave), _ptr(zsave), _ptr(dv), _ptr(da),
                                          _ptr(db), _ptr(dw), _ptr(dr), _ptr(workspace), int(workspace_bytes),
                                          ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_scan_backward")
    return st


def sdm_address_backward_workspace_size(dims: SdmDims) -> int:
    return int(load_library().sdm_address_backward_workspace_size(ctypes.byref(dims)))


def sdm_address_backward(k, q, C_w, C_r, widx, wwt, ridx, rwt, dw, dr, dims: SdmDims, dk, dq, dC_w, dC_r,
                         workspace, workspace_bytes: int, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_address_backward(_ptr(k), _ptr(q), _ptr(C_w), _ptr(C_r), _ptr(widx), _ptr(wwt),
                                             _ptr(ridx), _ptr(rwt), _ptr(dw), _ptr(dr), ctypes.byref(dims),
                                             _ptr(dk), _ptr(dq), _ptr(dC_w), _ptr(dC_r), _ptr(workspace),
                                             int(workspace_bytes), _stream(stream))
    if check:
        _check(st, "sdm_address_backward")
    return st


def sdm_gdn_dense_forward(S, k, q, v, a, b, o, dims: SdmDims, stream=None, *, check: bool = True) -> int:
    st = load_library().sdm_gdn_dense_forward(_ptr(S), _ptr(k), _ptr(q), _ptr(v), _ptr(a), _ptr(b), _ptr(o),
                                              ctypes.byref(dims), _stream(stream))
    if check:
        _check(st, "sdm_gdn_dense_forward")
    return st


# ---------------------------------------------------------------------------
# torch conveniences (allocation + shape checks only)
# ---------------------------------------------------------------------------
def _expect(t, shape, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} dtype {t.dtype} != {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _in_dtype(d: SdmDims):
    import torch
    return torch.bfloat16 if d.in_dtype == SDM_BF16 else torch.float32


def state_init(M0, dims: SdmDims, M=None, stream=None):
    import torch
    N = dims.n_sub * dims.n_sub
    _expect(M0, (dims.H, N, dims.d_v), torch.float32, "M0")
    if M is None:
        M = torch.empty((dims.B, dims.H, N, dims.d_v), dtype=torch.float32, device=M0.device)
    _expect(M, (dims.B, dims.H, N, dims.d_v), torch.float32, "M")
    sdm_state_init(M, M0, dims, stream)
    return M


def pkm_address(k, q, C_w, C_r, dims: SdmDims, out=None, stream=None):
    import torch
    dt = _in_dtype(dims)
    B, T, H = dims.B, dims.T, dims.H
    for n, t in (("k", k), ("q", q)):
        _expect(t, (B, T, H, dims.d_k), dt, n)
    for n, t in (("C_w", C_w), ("C_r", C_r)):
        _expect(t, (H, 2, dims.n_sub, dims.d_k // 2), dt, n)
    if out is None:
        dev = k.device
        out = (torch.empty((B, T, H, dims.W), dtype=torch.int32, device=dev),
               torch.empty((B, T, H, dims.W), dtype=torch.float32, device=dev),
               torch.empty((B, T, H, dims.R), dtype=torch.int32, device=dev),
               torch.empty((B, T, H, dims.R), dtype=torch.float32, device=dev))
    widx, wwt, ridx, rwt = out
    sdm_pkm_address(k, q, C_w, C_r, dims, widx, wwt, ridx, rwt, stream)
    return widx, wwt, ridx, rwt


def scan_forward(M, widx, wwt, ridx, rwt, v, a, b, dims: SdmDims, o=None, workspace=None, stream=None):
    import torch
    B, T, H = dims.B, dims.T, dims.H
    N = dims.n_sub * dims.n_sub
    _expect(M, (B, H, N, dims.d_v), torch.float32, "M")
    _expect(widx, (B, T, H, dims.W), torch.int32, "widx")
    _expect(wwt, (B, T, H, dims.W), torch.float32, "wwt")
    _expect(ridx, (B, T, H, dims.R), torch.int32, "ridx")
    _expect(rwt, (B, T, H, dims.R), torch.float32, "rwt")
    _expect(v, (B, T, H, dims.d_v), _in_dtype(dims), "v")
    _expect(a, (B, T, H), torch.float32, "a")
    _expect(b, (B, T, H), torch.float32, "b")
    if o is None:
        o = torch.empty((B, T, H, dims.d_v), dtype=torch.float32, device=M.device)
    _expect(o, (B, T, H, dims.d_v), torch.float32, "o")
    need = sdm_scan_workspace_size(dims)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=M.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sdm_scan_forward(M, widx, wwt, ridx, rwt, v, a, b, o, workspace, ws_bytes, dims, stream)
    return o


def scan_forward_noalloc(M, widx, wwt, ridx, rwt, v, a, b, dims: SdmDims, o=None, stream=None):
    """scan_forward through the allocation-free entry point (the library's
    static scratch instead of a workspace); o is allocated here if None."""
    import torch
    B, T, H = dims.B, dims.T, dims.H
    N = dims.n_sub * dims.n_sub
    _expect(M, (B, H, N, dims.d_v), torch.float32, "M")
    _expect(widx, (B, T, H, dims.W), torch.int32, "widx")
    _expect(wwt, (B, T, H, dims.W), torch.float32, "wwt")
    _expect(ridx, (B, T, H, dims.R), torch.int32, "ridx")
    _expect(rwt, (B, T, H, dims.R), torch.float32, "rwt")
    _expect(v, (B, T, H, dims.d_v), _in_dtype(dims), "v")
    _expect(a, (B, T, H), torch.float32, "a")
    _expect(b, (B, T, H), torch.float32, "b")
    if o is None:
        o = torch.empty((B, T, H, dims.d_v), dtype=torch.float32, device=M.device)
    _expect(o, (B, T, H, dims.d_v), torch.float32, "o")
    sdm_scan_forward_noalloc(M, widx, wwt, ridx, rwt, v, a, b, o, dims, stream)
    return o


def decode_step(M, k, q, C_w, C_r, v, a, b, dims: SdmDims, o=None, widx_out=None, ridx_out=None,
                stream=None):
    import torch
    B, H = dims.B, dims.H
    N = dims.n_sub * dims.n_sub
    dt = _in_dtype(dims)
    _expect(M, (B, H, N, dims.d_v), torch.float32, "M")
    _expect(k, (B, H, dims.d_k), dt, "k")
    _expect(q, (B, H, dims.d_k), dt, "q")
    _expect(C_w, (H, 2, dims.n_sub, dims.d_k // 2), dt, "C_w")
    _expect(C_r, (H, 2, dims.n_sub, dims.d_k // 2), dt, "C_r")
    _expect(v, (B, H, dims.d_v), dt, "v")
    _expect(a, (B, H), torch.float32, "a")
    _expect(b, (B, H), torch.float32, "b")
    if o is None:
        o = torch.empty((B, H, dims.d_v), dtype=torch.float32, device=M.device)
    sdm_decode_step(M, k, q, C_w, C_r, v, a, b, o, widx_out, ridx_out, dims, stream)
    return o


def gates(a_raw, b_raw, A, dt_bias, dims: SdmDims, a=None, b=None, stream=None):
    import torch
    B, T, H = dims.B, dims.T, dims.H
    _expect(a_raw, (B, T, H), torch.float32, "a_raw")
    _expect(b_raw, (B, T, H), torch.float32, "b_raw")
    _expect(A, (H,), torch.float32, "A")
    _expect(dt_bias, (H,), torch.float32, "dt_bias")
    if a is None:
        a = torch.empty((B, T, H), dtype=torch.float32, device=a_raw.device)
    if b is None:
        b = torch.empty((B, T, H), dtype=torch.float32, device=a_raw.device)
    _expect(a, (B, T, H), torch.float32, "a")
    _expect(b, (B, T, H), torch.float32, "b")
    sdm_gates(a_raw, b_raw, A, dt_bias, dims, a, b, stream)
    return a, b


def output_norm_gate(o, g, gamma, eps: float, dims: SdmDims, y=None, stream=None):
    import torch
    shp = (dims.B, dims.T, dims.H, dims.d_v)
    dt = _in_dtype(dims)
    _expect(o, shp, torch.float32, "o")
    _expect(g, shp, dt, "g")
    _expect(gamma, (dims.d_v,), torch.float32, "gamma")
    if y is None:
        y = torch.empty(shp, dtype=dt, device=o.device)
    _expect(y, shp, dt, "y")
    sdm_output_norm_gate(o, g, gamma, eps, dims, y, stream)
    return y


def gdn_dense_forward(S, k, q, v, a, b, dims: SdmDims, o=None, stream=None):
    import torch
    B, T, H = dims.B, dims.T, dims.H
    dt = _in_dtype(dims)
    _expect(S, (B, H, dims.d_k, dims.d_v), torch.float32, "S")
    _expect(k, (B, T, H, dims.d_k), dt, "k")
    _expect(q, (B, T, H, dims.d_k), dt, "q")
    _expect(v, (B, T, H, dims.d_v), dt, "v")
    _expect(a, (B, T, H), torch.float32, "a")
    _expect(b, (B, T, H), torch.float32, "b")
    if o is None:
        o = torch.empty((B, T, H, dims.d_v), dtype=torch.float32, device=S.device)
    _expect(o, (B, T, H, dims.d_v), torch.float32, "o")
    sdm_gdn_dense_forward(S, k, q, v, a, b, o, dims, stream)
    return o


def scan_forward_save(M, widx, wwt, ridx, rwt, v, a, b, dims: SdmDims, o=None, workspace=None, stream=None):
    """scan_forward that also returns the saved rows (xsave, zsave) for scan_backward."""
    import torch
    B, T, H = dims.B, dims.T, dims.H
    dev = M.device
    if o is None:
        o = torch.empty((B, T, H, dims.d_v), dtype=torch.float32, device=dev)
    xsave = torch.empty((B, H, T, dims.d_v // 4, dims.W, 4), dtype=torch.float32, device=dev)
    zsave = torch.empty((B, H, T, dims.d_v // 4, dims.R, 4), dtype=torch.float32, device=dev)
    need = sdm_scan_workspace_size(dims)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sdm_scan_forward_save(M, widx, wwt, ridx, rwt, v, a, b, o, xsave, zsave, workspace, ws_bytes, dims, stream)
    return o, xsave, zsave


def scan_backward(dM, widx, wwt, ridx, rwt, v, a, b, dout, xsave, zsave, dims: SdmDims, workspace=None,
                  stream=None):
    """Gradients of the scan; dM is updated in place (dL/dM after -> before the
    call).  Returns (dv, da, db, dw, dr).  The workspace is allocated here if
    None and the dims need one."""
    import torch
    B, T, H = dims.B, dims.T, dims.H
    dev = dM.device
    _expect(dout, (B, T, H, dims.d_v), torch.float32, "dout")
    _expect(xsave, (B, H, T, dims.d_v // 4, dims.W, 4), torch.float32, "xsave")
    _expect(zsave, (B, H, T, dims.d_v // 4, dims.R, 4), torch.float32, "zsave")
    dv = torch.empty((B, T, H, dims.d_v), dtype=torch.float32, device=dev)
    da = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    db = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dw = torch.empty((B, T, H, dims.W), dtype=torch.float32, device=dev)
    dr = torch.empty((B, T, H, dims.R), dtype=torch.float32, device=dev)
    need = sdm_scan_backward_workspace_size(dims)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sdm_scan_backward(dM, widx, wwt, ridx, rwt, v, a, b, dout, xsave, zsave, dv, da, db, dw, dr, workspace, ws_bytes,
                      dims, stream)
    return dv, da, db, dw, dr


def address_backward(k, q, C_w, C_r, widx, wwt, ridx, rwt, dw, dr, dims: SdmDims, shared_codebook_grad=False,
                     stream=None):
    """Gradients of the addressing (selection held fixed).  Returns (dk, dq,
    dC_w, dC_r); with shared_codebook_grad one buffer receives both sums and
    is returned twice."""
    import torch
    B, T, H = dims.B, dims.T, dims.H
    dev = k.device
    dk = torch.empty((B, T, H, dims.d_k), dtype=torch.float32, device=dev)
    dq = torch.empty_like(dk)
    dC_w = torch.empty((H, 2, dims.n_sub, dims.d_k // 2), dtype=torch.float32, device=dev)
    dC_r = dC_w if shared_codebook_grad else torch.empty_like(dC_w)
    need = sdm_address_backward_workspace_size(dims)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    sdm_address_backward(k, q, C_w, C_r, widx, wwt, ridx, rwt, dw, dr, dims, dk, dq, dC_w, dC_r, ws, need, stream)
    return dk, dq, dC_w, dC_r


def gates_backward(a_raw, b_raw, A, dt_bias, da, db, dims: SdmDims, workspace=None, stream=None):
    """Gradients of gates(): returns (da_raw, db_raw [B,T,H], dA, ddt_bias [H])."""
    import torch
    B, T, H = dims.B, dims.T, dims.H
    for name, x, shp in (("a_raw", a_raw, (B, T, H)), ("b_raw", b_raw, (B, T, H)), ("A", A, (H,)),
                         ("dt_bias", dt_bias, (H,)), ("da", da, (B, T, H)), ("db", db, (B, T, H))):
        _expect(x, shp, torch.float32, name)
    dev = a_raw.device
    da_raw = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    db_raw = torch.empty_like(da_raw)
    dA = torch.empty(H, dtype=torch.float32, device=dev)
    ddt = torch.empty_like(dA)
    need = sdm_gates_backward_workspace_size(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    sdm_gates_backward(a_raw, b_raw, A, dt_bias, da, db, dims, da_raw, db_raw, dA, ddt, workspace, ws_bytes, stream)
    return da_raw, db_raw, dA, ddt


def output_norm_gate_backward(o, g, gamma, eps: float, dy, dims: SdmDims, workspace=None, stream=None):
    """Gradients of output_norm_gate() for dL/dy = dy: returns (do, dg
    [B,T,H,d_v], dgamma [d_v]), all float32."""
    import torch
    shp = (dims.B, dims.T, dims.H, dims.d_v)
    _expect(o, shp, torch.float32, "o")
    _expect(g, shp, _in_dtype(dims), "g")
    _expect(gamma, (dims.d_v,), torch.float32, "gamma")
    _expect(dy, shp, torch.float32, "dy")
    dev = o.device
    dout = torch.empty(shp, dtype=torch.float32, device=dev)
    dg = torch.empty_like(dout)
    dgamma = torch.empty(dims.d_v, dtype=torch.float32, device=dev)
    need = sdm_output_norm_gate_backward_workspace_size(dims)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    sdm_output_norm_gate_backward(o, g, gamma, eps, dy, dims, dout, dg, dgamma, workspace, ws_bytes, stream)
    return dout, dg, dgamma
