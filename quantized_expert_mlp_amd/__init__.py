"""Python binding of libmoe (fused int4 MoE layer for MI355X / gfx950).

A thin ctypes layer over the C ABI in include/moe.h: the functions carry the
C entry points' names and only marshal arguments (torch tensors -> device
pointers, the current HIP stream).  Every step of the layer runs in the HIP
kernels of libmoe.so; there is no fallback: if the library is missing, or no
GPU is present, calls raise.

Build the library with ``python -m quantized_expert_mlp_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

(MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP,
 MOE_ERR_SCRATCH_LIMIT) = range(6)
MOE_STATIC_SCRATCH_BYTES = 16 << 20
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_GEMM = range(3)
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILED = range(2)
MOE_FORMAT_INT4, MOE_FORMAT_MXFP4 = range(2)
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = range(2)

# Every symbol include/moe.h declares.
EXPORTS = ("moe_router_topk", "moe_permute", "moe_permute_workspace_bytes", "moe_expert_mlp",
           "moe_layer",
           "moe_layer_profiled", "moe_pack_weights", "moe_workspace_bytes",
           "moe_status_string", "moe_debug_dequant_int4", "moe_debug_dequant_mxfp4",
           "moe_layer_residual_rmsnorm", "moe_layer_static", "moe_debug_read_probe")
STAGES = ("start", "logits", "topk", "permute", "activations", "gate_up", "shared_gate_up",
          "down", "shared_down")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))
        self.status = status


class moe_q4(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("s", ctypes.c_void_p)]


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("I", ctypes.c_int32), ("SI", ctypes.c_int32),
                ("group", ctypes.c_int32), ("route_scale", ctypes.c_float),
                ("path", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("format", ctypes.c_int32), ("top_p", ctypes.c_float),
                ("score", ctypes.c_int32), ("select_bias", ctypes.c_void_p),
                ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe.so is not built: run python -m quantized_expert_mlp_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        L.moe_router_topk.argtypes = [P, i32, i32, i32, f32, f32, i32, P, i32, i32, P, P, P]
        L.moe_permute.argtypes = [P, i32, i32, i32, P, P, P, P, ctypes.c_size_t, P]
        L.moe_permute_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_permute_workspace_bytes.restype = ctypes.c_size_t
        L.moe_expert_mlp.argtypes = [ctypes.POINTER(moe_shape), P, P, P, P, moe_q4, moe_q4,
                                     moe_q4, P, P, ctypes.c_size_t, P]
        L.moe_layer.argtypes = [ctypes.POINTER(moe_shape), P, P, P, moe_q4, moe_q4, moe_q4,
                                ctypes.POINTER(moe_q4), P, P, P, P, P, P, ctypes.c_size_t, P]
        L.moe_layer_profiled.argtypes = L.moe_layer.argtypes + [ctypes.POINTER(ctypes.c_void_p),
                                                                i32, P]
        L.moe_layer_static.argtypes = L.moe_layer.argtypes[:13] + [P]
        L.moe_layer_residual_rmsnorm.argtypes = [
            ctypes.POINTER(moe_shape), P, P, P, moe_q4, moe_q4, moe_q4, ctypes.POINTER(moe_q4), P,
            P, P, ctypes.c_float, P, P, i32, P, P, P, P, ctypes.c_size_t, P]
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(moe_shape)]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_debug_dequant_int4.argtypes = [moe_q4, i32, i32, i32, P, P]
        L.moe_debug_dequant_mxfp4.argtypes = [moe_q4, i32, i32, i32, P, P]
        L.moe_pack_weights.argtypes = [moe_q4, i32, i32, i32, i32, moe_q4, P]
        L.moe_debug_read_probe.argtypes = [P, ctypes.c_size_t, i32, P, P]
        for name in ("moe_router_topk", "moe_permute", "moe_expert_mlp", "moe_layer",
                     "moe_layer_profiled", "moe_pack_weights", "moe_debug_dequant_int4",
                     "moe_debug_dequant_mxfp4", "moe_layer_residual_rmsnorm",
                     "moe_layer_static", "moe_debug_read_probe"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(fn, rc)


def make_shape(T, H, E, k, I, SI=0, route_scale=1.0, path=MOE_PATH_AUTO, group=32,
               layout=MOE_LAYOUT_ROWS, format=MOE_FORMAT_INT4, top_p=0.0,
               score=MOE_SCORE_SOFTMAX, select_bias=None, n_group=0,
               topk_group=0) -> moe_shape:
    """select_bias: a device tensor fp32 [E] (or a raw pointer); the caller
    keeps it alive for as long as the shape is used."""
    return moe_shape(int(T), int(H), int(E), int(k), int(I), int(SI), int(group),
                     float(route_scale), int(path), int(layout), int(format), float(top_p),
                     int(score), _ptr(select_bias), int(n_group), int(topk_group))


def q4(plane: Tuple) -> moe_q4:
    """(q tensor, s tensor) -> moe_q4."""
    return moe_q4(_ptr(plane[0]), _ptr(plane[1]))


# ----------------------------------------------------------- entry points --

def moe_workspace_bytes(shape: moe_shape) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(shape))


def moe_router_topk(logits, T, E, k, route_scale, idx, w, stream=None, top_p=0.0,
                    score=MOE_SCORE_SOFTMAX, select_bias=None, n_group=0, topk_group=0) -> None:
    _check("moe_router_topk", lib().moe_router_topk(_ptr(logits), T, E, k, route_scale, top_p,
                                                    int(score), _ptr(select_bias), int(n_group),
                                                    int(topk_group), _ptr(idx), _ptr(w),
                                                    _stream(stream)))


def moe_permute_workspace_bytes(T, k, E) -> int:
    return lib().moe_permute_workspace_bytes(int(T), int(k), int(E))


def moe_permute(idx, T, k, E, off, sorted_, row_of, ws=None, ws_bytes=0, stream=None) -> None:
    _check("moe_permute", lib().moe_permute(_ptr(idx), T, k, E, _ptr(off), _ptr(sorted_),
                                            _ptr(row_of), _ptr(ws), int(ws_bytes),
                                            _stream(stream)))


def moe_expert_mlp(shape: moe_shape, x, off, sorted_, w, gate, up, down, y, ws, ws_bytes,
                   stream=None) -> None:
    _check("moe_expert_mlp", lib().moe_expert_mlp(
        ctypes.byref(shape), _ptr(x), _ptr(off), _ptr(sorted_), _ptr(w), q4(gate), q4(up),
        q4(down), _ptr(y), _ptr(ws), int(ws_bytes), _stream(stream)))


def moe_layer(shape: moe_shape, x, logits, w_router, gate, up, down,
              shared: Optional[Sequence[Tuple]], shared_gate, y, idx_out, w_out, logits_out,
              ws, ws_bytes, stream=None) -> None:
    sh_arr = None
    if shared is not None:
        sh_arr = (moe_q4 * 3)(*[q4(p) for p in shared])
    _check("moe_layer", lib().moe_layer(
        ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w_router), q4(gate), q4(up), q4(down),
        sh_arr, _ptr(shared_gate), _ptr(y), _ptr(idx_out), _ptr(w_out), _ptr(logits_out),
        _ptr(ws), int(ws_bytes), _stream(stream)))


def moe_layer_static(shape: moe_shape, x, logits, w_router, gate, up, down,
                     shared: Optional[Sequence[Tuple]], shared_gate, y, idx_out, w_out,
                     logits_out, stream=None) -> None:
    """moe_layer on the library's static per-GPU scratch (no workspace argument,
    no allocation); shapes needing more than MOE_STATIC_SCRATCH_BYTES raise
    MoeError with status MOE_ERR_SCRATCH_LIMIT."""
    sh_arr = None
    if shared is not None:
        sh_arr = (moe_q4 * 3)(*[q4(p) for p in shared])
    _check("moe_layer_static", lib().moe_layer_static(
        ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w_router), q4(gate), q4(up), q4(down),
        sh_arr, _ptr(shared_gate), _ptr(y), _ptr(idx_out), _ptr(w_out), _ptr(logits_out),
        _stream(stream)))


def moe_layer_residual_rmsnorm(shape: moe_shape, x, logits, w_router, gate, up, down,
                               shared: Optional[Sequence[Tuple]], shared_gate, residual, norm_w,
                               eps, x_next, idx_out, w_out, ws, ws_bytes, stream=None,
                               next_w_router=None, next_E=0, next_logits=None) -> None:
    """moe_layer whose combine adds into `residual` (fp32, in/out), followed by
    x_next = bf16(RMSnorm(residual) * norm_w), and with next_w_router
    ([next_E][H] fp32) the next layer's logits of x_next into next_logits."""
    sh_arr = None
    if shared is not None:
        sh_arr = (moe_q4 * 3)(*[q4(p) for p in shared])
    _check("moe_layer_residual_rmsnorm", lib().moe_layer_residual_rmsnorm(
        ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w_router), q4(gate), q4(up), q4(down),
        sh_arr, _ptr(shared_gate), _ptr(residual), _ptr(norm_w), float(eps), _ptr(x_next),
        _ptr(next_w_router), int(next_E), _ptr(next_logits), _ptr(idx_out), _ptr(w_out),
        _ptr(ws), int(ws_bytes), _stream(stream)))


def moe_layer_profiled(shape: moe_shape, x, logits, w_router, gate, up, down,
                       shared: Optional[Sequence[Tuple]], shared_gate, y, idx_out, w_out,
                       logits_out, ws, ws_bytes, events: Sequence[int], stream=None):
    """moe_layer with stage i's kernel bracketed by hipEvent_t handles
    events[2i] (start) and events[2i+1] (end); len(events) >= 2 * len(STAGES).
    Returns the names of the stages whose kernels the call launched."""
    sh_arr = None
    if shared is not None:
        sh_arr = (moe_q4 * 3)(*[q4(p) for p in shared])
    ev = (ctypes.c_void_p * len(events))(*events)
    ran = (ctypes.c_int32 * len(STAGES))()
    _check("moe_layer_profiled", lib().moe_layer_profiled(
        ctypes.byref(shape), _ptr(x), _ptr(logits), _ptr(w_router), q4(gate), q4(up), q4(down),
        sh_arr, _ptr(shared_gate), _ptr(y), _ptr(idx_out), _ptr(w_out), _ptr(logits_out),
        _ptr(ws), int(ws_bytes), _stream(stream), ev, len(events),
        ctypes.cast(ran, ctypes.c_void_p)))
    return [name for name, r in zip(STAGES, ran) if r]


def moe_pack_weights(src, E, N, K, dst, stream=None, format=MOE_FORMAT_INT4) -> None:
    """Row-layout plane set (q, s) -> tiled layout into dst (q, s) of the same sizes."""
    _check("moe_pack_weights", lib().moe_pack_weights(q4(src), E, N, K, int(format), q4(dst),
                                                      _stream(stream)))


def moe_debug_dequant_int4(plane, N, K, mode, out, stream=None) -> None:
    _check("moe_debug_dequant_int4", lib().moe_debug_dequant_int4(
        q4(plane), N, K, mode, _ptr(out), _stream(stream)))


def moe_debug_dequant_mxfp4(plane, N, K, out, stream=None, mode=1) -> None:
    _check("moe_debug_dequant_mxfp4", lib().moe_debug_dequant_mxfp4(
        q4(plane), N, K, int(mode), _ptr(out), _stream(stream)))


def moe_debug_read_probe(src, nbytes, workgroups, sink, stream=None) -> None:
    _check("moe_debug_read_probe", lib().moe_debug_read_probe(
        _ptr(src), int(nbytes), int(workgroups), _ptr(sink), _stream(stream)))
