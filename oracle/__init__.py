"""ctypes binding of the CPU oracle (oracle/oracle.cpp).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the
benchmark's CPU-baseline leg use this; the product path never imports it.

The oracle is plain C++17 built with g++ -O2 (no fast-math) and OpenMP over
token rows.  ``build()`` compiles it into oracle/liboracle.so.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["g++", "-std=c++17", "-O2", "-fopenmp", "-fPIC", "-shared",
                        _SRC, "-o", tmp], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_dequant_int4.argtypes = [P, P, i64, i64, P]
        L.oracle_dequant_mxfp4.argtypes = [P, P, i64, i64, P]
        L.oracle_e2m1_to_double.argtypes = [ctypes.c_int]
        L.oracle_e2m1_to_double.restype = ctypes.c_double
        L.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
        L.oracle_e8m0_to_double.restype = ctypes.c_double
        L.oracle_router_logits.argtypes = [P, P, P, i64, i64, i64, P]
        L.oracle_router_topk.argtypes = [P, i64, i64, i64, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_int, P, i64, i64, P, P, P]
        L.oracle_permute.argtypes = [P, i64, i64, i64, P, P, P]
        L.oracle_expert_forward.argtypes = [P] * 6 + [i64, i64, P, P, P, ctypes.c_int]
        L.oracle_layer.argtypes = [P] * 13 + [i64, P, P, P]
        L.oracle_add_rmsnorm.argtypes = [P, P, P, i64, i64, ctypes.c_double, P, P]
        L.oracle_add_rmsnorm_router.argtypes = [P, P, P, i64, i64, ctypes.c_double, P, i64, P,
                                                P, P]
        L.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        _lib = L
    return _lib


class _Shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int64), ("E", ctypes.c_int64),
                ("k", ctypes.c_int64), ("I", ctypes.c_int64), ("SI", ctypes.c_int64),
                ("route_scale", ctypes.c_double), ("fmt", ctypes.c_int64),
                ("top_p", ctypes.c_double), ("gate", ctypes.c_int64),
                ("bias", ctypes.c_void_p), ("n_group", ctypes.c_int64),
                ("topk_group", ctypes.c_int64)]


# Weight formats: int4 nibble-8 with fp16 scale bits (uint16), MXFP4 e2m1 with
# ue8m0 scale bytes (uint8); both one scale per 32 inputs.
FORMATS = {"int4": (0, np.uint16), "mxfp4": (1, np.uint8)}


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> int:
    return lib().oracle_set_threads(int(n))


def half_to_double(h: int) -> float:
    return lib().oracle_half_to_double(int(h))


def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(int(b))


def e2m1_to_double(nib: int) -> float:
    return lib().oracle_e2m1_to_double(int(nib))


def e8m0_to_double(e: int) -> float:
    return lib().oracle_e8m0_to_double(int(e))


def dequant(q: np.ndarray, s: np.ndarray, fmt: str = "int4") -> np.ndarray:
    """Dense fp64 W[N][K] of one plane: q [N][K/2] u8 and s [N][K/32], fp16 bits
    (int4) or ue8m0 bytes (mxfp4)."""
    q = _c(q, np.uint8)
    s = _c(s, FORMATS[fmt][1])
    N, K = q.shape[0], q.shape[1] * 2
    out = np.empty((N, K), dtype=np.float64)
    f = lib().oracle_dequant_mxfp4 if fmt == "mxfp4" else lib().oracle_dequant_int4
    f(_p(q), _p(s), N, K, _p(out))
    return out


def router_logits(x: np.ndarray, w_router: np.ndarray, gate_row: Optional[np.ndarray] = None):
    """fp32 logits [T][E] (or [T][E+1] with the shared gate logit as column E)."""
    x = _c(x, np.uint16)
    w_router = _c(w_router, np.float32)
    gate_row = _c(gate_row, np.float32)
    T, H = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E + (gate_row is not None)), dtype=np.float32)
    lib().oracle_router_logits(_p(x), _p(w_router), _p(gate_row), T, H, E, _p(out))
    return out


GATES = {"softmax": 0, "sigmoid": 1}


def router_topk(logits: np.ndarray, k: int, route_scale: float = 1.0, top_p: float = 1.0,
                gate: str = "softmax", bias: Optional[np.ndarray] = None, n_group: int = 0,
                topk_group: int = 0):
    """(idx int32 [T][k], w fp32 [T][k], w fp64 [T][k]); with 0 < top_p < 1
    the picks past the top-p prefix are -1 with weight 0.  gate/bias select a
    router variant (sigmoid scores, a selection bias [E]); n_group > 1 the
    grouped routing (topk_group groups kept)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    w64 = np.empty((T, k), dtype=np.float64)
    bias = _c(bias, np.float32)
    lib().oracle_router_topk(_p(logits), T, E, k, float(route_scale), float(top_p), GATES[gate],
                             _p(bias), int(n_group), int(topk_group), _p(idx), _p(w), _p(w64))
    return idx, w, w64


def permute(idx: np.ndarray, E: int):
    """(off int32 [E+1], sorted int32 [T*k], row_of int32 [T*k]).  Picks
    outside [0, E) belong to no bucket: row_of -1, and only the first off[E]
    entries of sorted are written."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    off = np.empty(E + 1, dtype=np.int32)
    srt = np.full(T * k, -1, dtype=np.int32)
    row_of = np.empty(T * k, dtype=np.int32)
    lib().oracle_permute(_p(idx), T, k, E, _p(off), _p(srt), _p(row_of))
    return off, srt, row_of


def expert_forward(gate, up, down, x64: np.ndarray, fmt: str = "int4"):
    """One expert on one fp64 row: returns (h fp64 [I], o fp64 [H]).

    gate/up/down are (q, s) pairs of single planes."""
    fid, st = FORMATS[fmt]
    (qg, sg), (qu, su), (qd, sd) = [(_c(q, np.uint8), _c(s, st)) for q, s in (gate, up, down)]
    I, H = qg.shape[0], qg.shape[1] * 2
    x64 = _c(x64, np.float64)
    h = np.empty(I, dtype=np.float64)
    o = np.empty(H, dtype=np.float64)
    lib().oracle_expert_forward(_p(qg), _p(sg), _p(qu), _p(su), _p(qd), _p(sd), H, I,
                                _p(x64), _p(h), _p(o), fid)
    return h, o


def layer(x: np.ndarray, logits: np.ndarray, k: int, planes: Dict[str, tuple],
          shared: Optional[Dict[str, tuple]] = None, shared_gate: Optional[np.ndarray] = None,
          rows: Optional[Sequence[int]] = None, route_scale: float = 1.0, fmt: str = "int4",
          top_p: float = 1.0, gate: str = "softmax", bias: Optional[np.ndarray] = None,
          n_group: int = 0, topk_group: int = 0):
    """The whole layer on the token rows ``rows`` (default: all).

    planes: {"gate": (q [E][I][H/2], s [E][I][H/32]), "up": ..., "down": (q [E][H][I/2], s)}
    shared: same keys with single planes, or None.
    fmt: "int4" (s = fp16 bits) or "mxfp4" (s = ue8m0 bytes) for every plane.
    Returns (y fp32 [n][H], idx int32 [n][k], w fp32 [n][k])."""
    x = _c(x, np.uint16)
    logits = _c(logits, np.float32)
    T, H = x.shape
    E = logits.shape[1]
    fid, st = FORMATS[fmt]
    gq, gs = [_c(a, t) for a, t in zip(planes["gate"], (np.uint8, st))]
    uq, us = [_c(a, t) for a, t in zip(planes["up"], (np.uint8, st))]
    dq, ds = [_c(a, t) for a, t in zip(planes["down"], (np.uint8, st))]
    I = gq.shape[1]
    SI = 0
    keep = []
    sq_arr = ss_arr = None
    if shared is not None:
        sq = [_c(shared[p][0], np.uint8) for p in ("gate", "up", "down")]
        ss = [_c(shared[p][1], st) for p in ("gate", "up", "down")]
        keep += sq + ss
        SI = sq[0].shape[0]
        sq_arr = (ctypes.c_void_p * 3)(*[a.ctypes.data for a in sq])
        ss_arr = (ctypes.c_void_p * 3)(*[a.ctypes.data for a in ss])
        keep += [sq_arr, ss_arr]
        sq_arr = ctypes.cast(sq_arr, ctypes.c_void_p)
        ss_arr = ctypes.cast(ss_arr, ctypes.c_void_p)
    shared_gate = _c(shared_gate, np.float32)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    n = T if rows_a is None else len(rows_a)
    bias = _c(bias, np.float32)
    sh = _Shape(T, H, E, k, I, SI, float(route_scale), fid, float(top_p), GATES[gate],
                None if bias is None else bias.ctypes.data, int(n_group), int(topk_group))
    y = np.empty((n, H), dtype=np.float32)
    idx = np.empty((n, k), dtype=np.int32)
    w = np.empty((n, k), dtype=np.float32)
    lib().oracle_layer(ctypes.byref(sh), _p(x), _p(logits), _p(gq), _p(gs), _p(uq), _p(us),
                       _p(dq), _p(ds), sq_arr, ss_arr, _p(shared_gate), _p(rows_a), n,
                       _p(y), _p(idx), _p(w))
    return y, idx, w


def double_to_bf16(v: float) -> int:
    return lib().oracle_double_to_bf16(float(v))


def add_rmsnorm(r: np.ndarray, y: np.ndarray, g: np.ndarray, eps: float):
    """The combine folded into the residual step: (r + y as fp32 [T][H],
    bf16 bits [T][H] of the RMS-normed row times g)."""
    r = _c(r, np.float32)
    y = _c(y, np.float32)
    g = _c(g, np.float32)
    T, H = r.shape
    r_out = np.empty((T, H), dtype=np.float32)
    n_out = np.empty((T, H), dtype=np.uint16)
    lib().oracle_add_rmsnorm(_p(r), _p(y), _p(g), T, H, float(eps), _p(r_out), _p(n_out))
    return r_out, n_out


def add_rmsnorm_router(r: np.ndarray, y: np.ndarray, g: np.ndarray, eps: float,
                       w_router: np.ndarray):
    """add_rmsnorm followed by the next layer's router logits of the bf16
    normed row: (r + y fp32 [T][H], bf16 bits [T][H], logits fp32 [T][E])."""
    r = _c(r, np.float32)
    y = _c(y, np.float32)
    g = _c(g, np.float32)
    w_router = _c(w_router, np.float32)
    T, H = r.shape
    E = w_router.shape[0]
    r_out = np.empty((T, H), dtype=np.float32)
    n_out = np.empty((T, H), dtype=np.uint16)
    logits = np.empty((T, E), dtype=np.float32)
    lib().oracle_add_rmsnorm_router(_p(r), _p(y), _p(g), T, H, float(eps), _p(w_router), E,
                                    _p(r_out), _p(n_out), _p(logits))
    return r_out, n_out, logits
