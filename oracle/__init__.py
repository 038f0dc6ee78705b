"""CPU oracle for the Sparse Delta Memory hot path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its binding) never imports, links or calls it, and it shares no code with
that path.

The arithmetic lives in ``sdm_oracle.c`` (plain C, fp64 accumulation, scalar
loops, OpenMP only across independent rows or sequences); this module builds
it with gcc and marshals numpy arrays.  Function-level citations of the pages
are in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sdm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


class OracleError(RuntimeError):
    pass


class _Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("B", "T", "H", "d_k", "n_sub", "d_v", "k_prime", "W", "R")] + \
               [("in_bf16", ctypes.c_int32), ("pad_", ctypes.c_int32)]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", "-Wextra", "-o", _LIB + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.orc_address.argtypes = [P, P, P, P, ctypes.POINTER(_Dims), P, P, P, P, P, P, I32]
        lib.orc_half_scores.argtypes = [P, P, ctypes.POINTER(_Dims), P, I32]
        lib.orc_slot_scores.argtypes = [P, P, ctypes.POINTER(_Dims), I64, P, P, P]
        lib.orc_scan.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.POINTER(_Dims), I32]
        lib.orc_state_init.argtypes = [P, P, ctypes.POINTER(_Dims)]
        lib.orc_gates.argtypes = [P, P, P, P, ctypes.POINTER(_Dims), P, P]
        lib.orc_output_norm_gate.argtypes = [P, P, P, ctypes.c_double, ctypes.POINTER(_Dims), P]
        lib.orc_gdn_dense.argtypes = [P, P, P, P, P, P, P, ctypes.POINTER(_Dims), I32]
        lib.orc_scan_backward.argtypes = [P] * 15 + [ctypes.POINTER(_Dims), I32]
        lib.orc_address_backward.argtypes = [P] * 10 + [ctypes.POINTER(_Dims), P, P, P, P]
        lib.orc_gates_backward.argtypes = [P] * 6 + [ctypes.POINTER(_Dims), P, P, P, P]
        lib.orc_output_norm_gate_backward.argtypes = [P, P, P, ctypes.c_double, P, ctypes.POINTER(_Dims), P, P, P]
        for f in (lib.orc_address, lib.orc_half_scores, lib.orc_slot_scores, lib.orc_scan,
                  lib.orc_state_init, lib.orc_gates, lib.orc_output_norm_gate, lib.orc_gdn_dense,
                  lib.orc_scan_backward, lib.orc_address_backward, lib.orc_gates_backward,
                  lib.orc_output_norm_gate_backward):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _dims(d) -> _Dims:
    return _Dims(d.B, d.T, d.H, d.d_k, d.n_sub, d.d_v, d.k_prime, d.W, d.R,
                 1 if d.in_dtype == "bf16" else 0, 0)


def _in(x: np.ndarray, d) -> np.ndarray:
    want = np.uint16 if d.in_dtype == "bf16" else np.float32
    if x.dtype != want:
        raise TypeError(f"expected {want} input, got {x.dtype}")
    return np.ascontiguousarray(x)


def _p(x: Optional[np.ndarray]):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count() or 1)


def address(k, q, C_w, C_r, d, *, scores: bool = False, nthreads: Optional[int] = None):
    """Top-W write and top-R read slots with softmax weights for every token-head.

    Returns (widx, wwt, ridx, rwt) shaped [B,T,H,W] / [B,T,H,R]; with
    ``scores=True`` also the selected fp32 slot scores (wsc, rsc).
    """
    lib = _load()
    k, q, C_w, C_r = (_in(x, d) for x in (k, q, C_w, C_r))
    shp = (d.B, d.T, d.H)
    widx = np.empty(shp + (d.W,), np.int32)
    wwt = np.empty(shp + (d.W,), np.float32)
    ridx = np.empty(shp + (d.R,), np.int32)
    rwt = np.empty(shp + (d.R,), np.float32)
    wsc = np.empty(shp + (d.W,), np.float32) if scores else None
    rsc = np.empty(shp + (d.R,), np.float32) if scores else None
    dm = _dims(d)
    rc = lib.orc_address(_p(k), _p(q), _p(C_w), _p(C_r), ctypes.byref(dm), _p(widx), _p(wwt),
                         _p(ridx), _p(rwt), _p(wsc), _p(rsc), nthreads or default_threads())
    _check(rc, "orc_address")
    if scores:
        return widx, wwt, ridx, rwt, wsc, rsc
    return widx, wwt, ridx, rwt


def half_scores(x, C, d, *, nthreads: Optional[int] = None) -> np.ndarray:
    """fp32 half scores [B,T,H,2,n_sub] of x against codebook C."""
    lib = _load()
    x, C = _in(x, d), _in(C, d)
    out = np.empty((d.B, d.T, d.H, 2, d.n_sub), np.float32)
    dm = _dims(d)
    _check(lib.orc_half_scores(_p(x), _p(C), ctypes.byref(dm), _p(out), nthreads or default_threads()),
           "orc_half_scores")
    return out


def slot_scores(x, C, d, rows: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """fp32 slot scores for flat token-head rows and slots (same length)."""
    lib = _load()
    x, C = _in(x, d), _in(C, d)
    rows = np.ascontiguousarray(rows, dtype=np.int64).ravel()
    slots = np.ascontiguousarray(slots, dtype=np.int32).ravel()
    if rows.shape != slots.shape:
        raise ValueError("rows and slots differ in length")
    out = np.empty(rows.shape, np.float32)
    dm = _dims(d)
    _check(lib.orc_slot_scores(_p(x), _p(C), ctypes.byref(dm), rows.size, _p(rows), _p(slots), _p(out)),
           "orc_slot_scores")
    return out


def scan(M, widx, wwt, ridx, rwt, v, a, b, d, *, nthreads: Optional[int] = None) -> np.ndarray:
    """Run the scan in place on M [B,H,N,d_v] (float32); returns o [B,T,H,d_v]."""
    lib = _load()
    if M.dtype != np.float32 or not M.flags.c_contiguous:
        raise TypeError("M must be a C-contiguous float32 array")
    if M.shape != (d.B, d.H, d.N, d.d_v):
        raise ValueError(f"M shape {M.shape} != {(d.B, d.H, d.N, d.d_v)}")
    widx = np.ascontiguousarray(widx, np.int32)
    ridx = np.ascontiguousarray(ridx, np.int32)
    wwt = np.ascontiguousarray(wwt, np.float32)
    rwt = np.ascontiguousarray(rwt, np.float32)
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    v = _in(v, d)
    for name, arr, shp in (("widx", widx, (d.B, d.T, d.H, d.W)), ("ridx", ridx, (d.B, d.T, d.H, d.R)),
                           ("wwt", wwt, (d.B, d.T, d.H, d.W)), ("rwt", rwt, (d.B, d.T, d.H, d.R)),
                           ("v", v, (d.B, d.T, d.H, d.d_v)), ("a", a, (d.B, d.T, d.H)),
                           ("b", b, (d.B, d.T, d.H))):
        if arr.shape != shp:
            raise ValueError(f"{name} shape {arr.shape} != {shp}")
    o = np.empty((d.B, d.T, d.H, d.d_v), np.float32)
    dm = _dims(d)
    rc = lib.orc_scan(_p(M), _p(widx), _p(wwt), _p(ridx), _p(rwt), _p(v), _p(a), _p(b), _p(o),
                      ctypes.byref(dm), nthreads or default_threads())
    _check(rc, "orc_scan")
    return o


def state_init(M0: np.ndarray, d) -> np.ndarray:
    """M [B,H,N,d_v] with every sequence set to M0 [H,N,d_v]."""
    lib = _load()
    M0 = np.ascontiguousarray(M0, np.float32)
    if M0.shape != (d.H, d.N, d.d_v):
        raise ValueError("M0 shape")
    M = np.empty((d.B, d.H, d.N, d.d_v), np.float32)
    dm = _dims(d)
    _check(lib.orc_state_init(_p(M), _p(M0), ctypes.byref(dm)), "orc_state_init")
    return M


def decode_step(M, k, q, C_w, C_r, v, a, b, d, *, nthreads: Optional[int] = None
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One single-token step for every sequence: addressing then one scan step.

    k, q [B,H,d_k]; v [B,H,d_v]; a, b [B,H]; M updated in place.
    Returns (o [B,H,d_v], widx [B,H,W], ridx [B,H,R]).
    """
    d1 = d.replace(T=1)
    ex = lambda x: np.ascontiguousarray(x)[:, None]
    widx, wwt, ridx, rwt = address(ex(k), ex(q), C_w, C_r, d1, nthreads=nthreads)
    o = scan(M, widx, wwt, ridx, rwt, ex(v), ex(a), ex(b), d1, nthreads=nthreads)
    return o[:, 0], widx[:, 0], ridx[:, 0]


def gates(a_raw, b_raw, A, dt_bias, d) -> Tuple[np.ndarray, np.ndarray]:
    """Forget and input gates (a, b) [B,T,H] fp32 from their pre-activations
    a_raw, b_raw [B,T,H] and the per-head decay A and time-step bias [H]."""
    lib = _load()
    a_raw, b_raw = (np.ascontiguousarray(x, np.float32) for x in (a_raw, b_raw))
    A, dt_bias = (np.ascontiguousarray(x, np.float32) for x in (A, dt_bias))
    if a_raw.shape != (d.B, d.T, d.H) or b_raw.shape != (d.B, d.T, d.H):
        raise ValueError("a_raw / b_raw shape")
    if A.shape != (d.H,) or dt_bias.shape != (d.H,):
        raise ValueError("A / dt_bias shape")
    a = np.empty((d.B, d.T, d.H), np.float32)
    b = np.empty((d.B, d.T, d.H), np.float32)
    dm = _dims(d)
    _check(lib.orc_gates(_p(a_raw), _p(b_raw), _p(A), _p(dt_bias), ctypes.byref(dm), _p(a), _p(b)), "orc_gates")
    return a, b


def output_norm_gate(o, g, gamma, eps: float, d) -> np.ndarray:
    """y [B,T,H,d_v] float64 (exact, before rounding to the output precision):
    RMS norm of each o row with gain gamma [d_v], times silu(g)."""
    lib = _load()
    o = np.ascontiguousarray(o, np.float32)
    g = _in(g, d)
    gamma = np.ascontiguousarray(gamma, np.float32)
    shp = (d.B, d.T, d.H, d.d_v)
    if o.shape != shp or g.shape != shp or gamma.shape != (d.d_v,):
        raise ValueError("o / g / gamma shape")
    y = np.empty(shp, np.float64)
    dm = _dims(d)
    _check(lib.orc_output_norm_gate(_p(o), _p(g), _p(gamma), float(eps), ctypes.byref(dm), _p(y)),
           "orc_output_norm_gate")
    return y


def gdn_dense(S, k, q, v, a, b, d, *, nthreads: Optional[int] = None) -> np.ndarray:
    """The dense Gated DeltaNet recurrence, in place on S [B,H,d_k,d_v]
    (float32, the state transposed: row j belongs to key dimension j).
    k, q [B,T,H,d_k]; v [B,T,H,d_v] (input dtype); a, b [B,T,H].
    Returns o [B,T,H,d_v] float32."""
    lib = _load()
    if S.dtype != np.float32 or not S.flags.c_contiguous:
        raise TypeError("S must be a C-contiguous float32 array")
    if S.shape != (d.B, d.H, d.d_k, d.d_v):
        raise ValueError(f"S shape {S.shape} != {(d.B, d.H, d.d_k, d.d_v)}")
    k, q, v = _in(k, d), _in(q, d), _in(v, d)
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    for name, arr, shp in (("k", k, (d.B, d.T, d.H, d.d_k)), ("q", q, (d.B, d.T, d.H, d.d_k)),
                           ("v", v, (d.B, d.T, d.H, d.d_v)), ("a", a, (d.B, d.T, d.H)), ("b", b, (d.B, d.T, d.H))):
        if arr.shape != shp:
            raise ValueError(f"{name} shape {arr.shape} != {shp}")
    o = np.empty((d.B, d.T, d.H, d.d_v), np.float32)
    dm = _dims(d)
    _check(lib.orc_gdn_dense(_p(S), _p(k), _p(q), _p(v), _p(a), _p(b), _p(o), ctypes.byref(dm),
                             nthreads or default_threads()), "orc_gdn_dense")
    return o


def scan_backward(M, widx, wwt, ridx, rwt, v, a, b, dout, d, dM_final=None, *, nthreads: Optional[int] = None):
    """Gradients of the scan for dL/do = dout [B,T,H,d_v] and dL/dM_T =
    dM_final (zeros when None).  M [B,H,N,d_v] is the state before the call
    (not modified).  Returns a dict: dM (dL/dM before the call), dv, da, db,
    dw [B,T,H,W], dr [B,T,H,R] (float32)."""
    lib = _load()
    M = np.ascontiguousarray(M, np.float32)
    if M.shape != (d.B, d.H, d.N, d.d_v):
        raise ValueError("M shape")
    widx, ridx = (np.ascontiguousarray(x, np.int32) for x in (widx, ridx))
    wwt, rwt, a, b = (np.ascontiguousarray(x, np.float32) for x in (wwt, rwt, a, b))
    dout = np.ascontiguousarray(dout, np.float32)
    v = _in(v, d)
    if dout.shape != (d.B, d.T, d.H, d.d_v):
        raise ValueError("dout shape")
    dM = np.zeros_like(M) if dM_final is None else np.array(dM_final, np.float32, copy=True, order="C")
    shp = (d.B, d.T, d.H)
    out = dict(dM=dM, dv=np.empty(shp + (d.d_v,), np.float32), da=np.empty(shp, np.float32),
               db=np.empty(shp, np.float32), dw=np.empty(shp + (d.W,), np.float32),
               dr=np.empty(shp + (d.R,), np.float32))
    dm = _dims(d)
    _check(lib.orc_scan_backward(_p(M), _p(widx), _p(wwt), _p(ridx), _p(rwt), _p(v), _p(a), _p(b), _p(dout),
                                 _p(out["dM"]), _p(out["dv"]), _p(out["da"]), _p(out["db"]), _p(out["dw"]),
                                 _p(out["dr"]), ctypes.byref(dm), nthreads or default_threads()),
           "orc_scan_backward")
    return out


def address_backward(k, q, C_w, C_r, widx, wwt, ridx, rwt, dw, dr, d):
    """Gradients of the addressing with the selected slots held fixed, for
    dL/dwwt = dw and dL/drwt = dr.  Returns (dk, dq, dC_w, dC_r), float32."""
    lib = _load()
    k, q, C_w, C_r = (_in(x, d) for x in (k, q, C_w, C_r))
    widx, ridx = (np.ascontiguousarray(x, np.int32) for x in (widx, ridx))
    wwt, rwt, dw, dr = (np.ascontiguousarray(x, np.float32) for x in (wwt, rwt, dw, dr))
    dk = np.empty((d.B, d.T, d.H, d.d_k), np.float32)
    dq = np.empty_like(dk)
    dCw = np.empty((d.H, 2, d.n_sub, d.d_k // 2), np.float32)
    dCr = np.empty_like(dCw)
    dm = _dims(d)
    _check(lib.orc_address_backward(_p(k), _p(q), _p(C_w), _p(C_r), _p(widx), _p(wwt), _p(ridx), _p(rwt), _p(dw),
                                    _p(dr), ctypes.byref(dm), _p(dk), _p(dq), _p(dCw), _p(dCr)),
           "orc_address_backward")
    return dk, dq, dCw, dCr


def gates_backward(a_raw, b_raw, A, dt_bias, da, db, d):
    """Gradients of gates(): returns (da_raw, db_raw [B,T,H], dA, ddt_bias [H]), float32."""
    lib = _load()
    a_raw, b_raw, A, dt_bias, da, db = (np.ascontiguousarray(x, np.float32) for x in (a_raw, b_raw, A, dt_bias, da, db))
    shp = (d.B, d.T, d.H)
    out = (np.empty(shp, np.float32), np.empty(shp, np.float32), np.empty(d.H, np.float32), np.empty(d.H, np.float32))
    dm = _dims(d)
    _check(lib.orc_gates_backward(_p(a_raw), _p(b_raw), _p(A), _p(dt_bias), _p(da), _p(db), ctypes.byref(dm),
                                  *(_p(x) for x in out)), "orc_gates_backward")
    return out


def output_norm_gate_backward(o, g, gamma, eps: float, dy, d):
    """Gradients of output_norm_gate() for dL/dy = dy: returns (do, dg [B,T,H,d_v], dgamma [d_v]), float32."""
    lib = _load()
    o = np.ascontiguousarray(o, np.float32)
    g = _in(g, d)
    gamma = np.ascontiguousarray(gamma, np.float32)
    dy = np.ascontiguousarray(dy, np.float32)
    shp = (d.B, d.T, d.H, d.d_v)
    out = (np.empty(shp, np.float32), np.empty(shp, np.float32), np.empty(d.d_v, np.float32))
    dm = _dims(d)
    _check(lib.orc_output_norm_gate_backward(_p(o), _p(g), _p(gamma), float(eps), _p(dy), ctypes.byref(dm),
                                             *(_p(x) for x in out)), "orc_output_norm_gate_backward")
    return out
