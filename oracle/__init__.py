"""Plain fp64 CPU oracle for exact grouped-query attention (decode and causal prefill).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path (the HIP
library under ``attention_gqa_decode_amd/``) never loads it and shares no code with it.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, built with gcc); this module
only marshals numpy arrays into it.  Inputs are bf16 bit patterns (``numpy.uint16``),
the exact bytes the GPU reads.  What each function computes, and which page passage it
follows, is stated in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile ``attn_oracle.c`` into ``liboracle.so`` with gcc (IEEE fp64, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_bf16_decode.argtypes = [_P, _P, _I64]
    lib.oracle_bf16_decode.restype = None
    lib.oracle_decode_f64.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, _I64, ctypes.c_double, _P, _I64, _P]
    lib.oracle_decode_f64.restype = ctypes.c_int
    lib.oracle_partial_state_f64.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, _I64, ctypes.c_double, ctypes.c_int,
                                             ctypes.c_int, _I64, _I64, _P, _P, _P]
    lib.oracle_partial_state_f64.restype = ctypes.c_int
    lib.oracle_merge_states_f64.argtypes = [ctypes.c_int, _P, _P, _P, ctypes.c_int, _P]
    lib.oracle_merge_states_f64.restype = ctypes.c_int
    lib.oracle_prefill_causal_f64.argtypes = [_P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_double, _P, _I64, _P]
    lib.oracle_prefill_causal_f64.restype = ctypes.c_int
    lib.oracle_fp8_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    lib.oracle_fp8_e4m3_to_f64.restype = ctypes.c_double
    lib.oracle_decode_fp8_f64.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          _I64, ctypes.c_double, ctypes.c_double, ctypes.c_double, _P, _I64, _P]
    lib.oracle_decode_fp8_f64.restype = ctypes.c_int
    lib.oracle_decode_multi_f64.argtypes = [_P, _P, _P, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            _I64, ctypes.c_int, ctypes.c_double, _P, _I64, _P]
    lib.oracle_decode_multi_f64.restype = ctypes.c_int
    _lib = lib
    return lib


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"expected bf16 bit patterns as uint16, got {a.dtype}")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """Threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())


def bf16_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    bits = _u16(bits)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_bf16_decode(_ptr(bits), _ptr(out), bits.size)
    return out


def decode(q, k, v, seqlens, Hq: int, KH: int, scale: float, rows=None) -> np.ndarray:
    """Decode attention.

    q: uint16 [B][Hq][Hsz]; k, v: uint16 [B][KH][S][Hsz]; seqlens: int [B].
    Returns float64 [B][Hq][Hsz].  ``rows`` optionally lists flat ``b*Hq + h`` indices
    to compute; unlisted rows are NaN.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq_, Hsz = q.shape
    assert Hq_ == Hq and k.shape[0] == B and k.shape[1] == KH and k.shape[3] == Hsz
    assert v.shape == k.shape
    S = k.shape[2]
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    out = np.full((B, Hq, Hsz), np.nan)
    if rows is None:
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nr = _ptr(rows), rows.size
    rc = _load().oracle_decode_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), B, Hq, KH, Hsz, S,
                                   float(scale), rp, nr, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode_f64 rejected its arguments")
    return out


def partial_state(q, k, v, Hq: int, KH: int, scale: float, b: int, h: int, j0: int, j1: int):
    """(m, l, o) of one (b, h) over keys [j0, j1), natural-exponent domain, o unnormalised."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, _, Hsz = q.shape
    S = k.shape[2]
    m = np.zeros(1)
    l = np.zeros(1)
    o = np.zeros(Hsz)
    rc = _load().oracle_partial_state_f64(_ptr(q), _ptr(k), _ptr(v), B, Hq, KH, Hsz, S, float(scale),
                                          b, h, j0, j1, _ptr(m), _ptr(l), _ptr(o))
    if rc != 0:
        raise ValueError("oracle_partial_state_f64 rejected its arguments")
    return float(m[0]), float(l[0]), o


def merge_states(m, l, o) -> np.ndarray:
    """Merge partial states: m, l float64 [n]; o float64 [n][Hsz]."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    o = np.ascontiguousarray(o, dtype=np.float64)
    n, Hsz = o.shape
    out = np.zeros(Hsz)
    rc = _load().oracle_merge_states_f64(n, _ptr(m), _ptr(l), _ptr(o), Hsz, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_merge_states_f64 rejected its arguments")
    return out


def prefill_causal(q, k, v, KH: int, scale: float, rows=None) -> np.ndarray:
    """Causal prefill.  q: uint16 [B][Hq][ISL][Hsz]; k, v: uint16 [B][KH][ISL][Hsz].

    Returns float64 [B][Hq][ISL][Hsz]; ``rows`` optionally lists flat
    ``(b*Hq + h)*ISL + i`` indices (unlisted rows are NaN).
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, ISL, Hsz = q.shape
    assert k.shape == (B, KH, ISL, Hsz) and v.shape == k.shape
    out = np.full(q.shape, np.nan)
    if rows is None:
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nr = _ptr(rows), rows.size
    rc = _load().oracle_prefill_causal_f64(_ptr(q), _ptr(k), _ptr(v), B, ISL, Hq, KH, Hsz,
                                           float(scale), rp, nr, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_prefill_causal_f64 rejected its arguments")
    return out


def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """Exact OCP E4M3 (e4m3fn) decode of uint8 codes to float64."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    f = _load().oracle_fp8_e4m3_to_f64
    return np.array([f(int(c)) for c in codes.ravel()], dtype=np.float64).reshape(codes.shape)


def decode_fp8(q, k, v, seqlens, Hq: int, KH: int, scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
               rows=None) -> np.ndarray:
    """Decode attention over an E4M3 KV cache.

    q: uint16 bf16 bits [B][Hq][Hsz]; k, v: uint8 E4M3 codes [B][KH][S][Hsz]; the attended
    key is k_scale * K and the value v_scale * V.  Returns float64 [B][Hq][Hsz] (NaN rows
    when ``rows`` leaves them out).
    """
    q = _u16(q)
    k = np.ascontiguousarray(k, dtype=np.uint8)
    v = np.ascontiguousarray(v, dtype=np.uint8)
    B, Hq_, Hsz = q.shape
    assert Hq_ == Hq and k.shape[0] == B and k.shape[1] == KH and k.shape[3] == Hsz and v.shape == k.shape
    S = k.shape[2]
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    out = np.full((B, Hq, Hsz), np.nan)
    if rows is None:
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nr = _ptr(rows), rows.size
    rc = _load().oracle_decode_fp8_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), B, Hq, KH, Hsz, S, float(scale),
                                       float(k_scale), float(v_scale), rp, nr, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode_fp8_f64 rejected its arguments")
    return out


def decode_multi(q, k, v, seqlens, KH: int, scale: float, rows=None) -> np.ndarray:
    """Multi-token decode: q uint16 [B][Hq][gamma][Hsz]; k, v uint16 [B][KH][S][Hsz].

    Query t of request b attends keys 0 .. L_b - gamma + t.  Returns float64
    [B][Hq][gamma][Hsz]; ``rows`` optionally lists flat ((b*Hq + h)*gamma + t) indices.
    """
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Hq, gamma, Hsz = q.shape
    assert k.shape[0] == B and k.shape[1] == KH and k.shape[3] == Hsz and v.shape == k.shape
    S = k.shape[2]
    sl = np.ascontiguousarray(seqlens, dtype=np.int32)
    out = np.full(q.shape, np.nan)
    if rows is None:
        rp, nr = None, 0
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        rp, nr = _ptr(rows), rows.size
    rc = _load().oracle_decode_multi_f64(_ptr(q), _ptr(k), _ptr(v), _ptr(sl), B, Hq, KH, Hsz, S, gamma,
                                         float(scale), rp, nr, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_decode_multi_f64 rejected its arguments")
    return out

