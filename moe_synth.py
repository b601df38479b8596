"""Seeded synthetic inputs for the fused int4 / MXFP4 MoE layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It only draws random numbers and encodes them into the storage
formats the layer consumes (bf16 activations, packed int4 nibbles, fp16 group
scales, fp32 router inputs).  It holds none of the layer's arithmetic.

Workload shapes follow the MoE layers the source pages measure:
  * the 6144 -> 2048 -> 6144 int4 expert with 256 experts of the colibri
    Vulkan backend PR ("Measured performance", the expert-group table);
  * the Qwen3-30B-A3B-class 128-expert layer (expert K 768, 2048-wide router)
    and the Qwen1.5-MoE-class layer with a 5632-wide shared expert, both from
    the dasLLAMA vulkan PR's commit notes on the routed block, the router tile
    and the GEMV lane split;
  * a skewed-routing prefill whose expert popularity follows a Zipf law, the
    stand-in for the real-router skew the dasLLAMA PR reports (a few experts
    with hundreds of rows, many with none).
No model weights are used.

Storage conventions (the boundary's):
  x        uint16 [T][H]          bf16 bits, round-to-nearest-even from N(0,1)
  logits   float32 [T][E]         N(0,1) (given-logits workloads)
  w_router float32 [E][H]         N(0, 0.02)      (router-logits workloads)
  residual float32 [T][H]         N(0, 1)         (folded residual step)
  norm_w   float32 [H]            1 + N(0, 0.1)   (its next-layer RMSnorm weight)
  g        float32 [H]            N(0, 0.02)      (shared-expert gate vector)
  q        uint8 [E][N][K/2]      element kk in byte kk/2, low nibble = even kk
  s        uint16 [E][N][K/32]    fp16 bits, uniform[0.005, 0.02] rounded RNE
MXFP4 planes (fmt "mxfp4") keep q's layout (uniform bytes: every e2m1 code)
and replace s by
  s        uint8 [E][N][K/32]     ue8m0 exponents, uniform on 119..122
                                  (group scales 2^-8 .. 2^-5, so weights have
                                  the int4 planes' magnitude)
Gate/up planes have N = I, K = H; down planes have N = H, K = I.

Every array is drawn from its own counter-style stream
``numpy.random.default_rng([seed, workload_id, tag, ...])`` so that a single
expert's planes can be regenerated alone (the oracle's sampled checks need only
the experts a token touches).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Iterable, Optional

import numpy as np

GROUP = 32


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    T: int
    H: int
    E: int
    k: int
    I: int
    SI: int
    logits: str  # "given", "router" or "zipf"
    description: str

    @property
    def slots(self) -> int:
        return self.T * self.k


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 0, 4, 256, 8, 2, 128, 0, "given",
                 "tiny layer: T=4, H=256, E=8, top-2, I=128"),
        Workload("decode", 1, 1, 6144, 256, 8, 2048, 0, "given",
                 "single-token decode: T=1, H=6144, E=256, top-8, I=2048"),
        Workload("decode_batch", 2, 32, 2048, 128, 8, 768, 0, "router",
                 "decode batch: T=32, H=2048, E=128, top-8, I=768, logits = x.W_router"),
        Workload("prefill_shared", 3, 512, 2048, 60, 4, 1408, 5632, "router",
                 "prefill with shared expert: T=512, H=2048, E=60, top-4, I=1408, SI=5632"),
        Workload("prefill_skewed", 4, 2048, 6144, 256, 8, 2048, 0, "zipf",
                 "skewed prefill: T=2048, H=6144, E=256, top-8, I=2048, Zipf(1.1) expert bias"),
    ]
}

ZIPF_S = 1.1


def _rng(seed: int, *tags: int) -> np.random.Generator:
    return np.random.default_rng([int(seed)] + [int(t) for t in tags])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); return the uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def fp16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def draw_x(wl: Workload, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    T = wl.T if T is None else T
    a = _rng(seed, wl.wid, 0).standard_normal((T, wl.H), dtype=np.float32)
    return f32_to_bf16_bits(a)


def draw_logits(wl: Workload, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    """Router logits for the given-logits workloads (fp32 [T][E])."""
    T = wl.T if T is None else T
    z = _rng(seed, wl.wid, 1).standard_normal((T, wl.E), dtype=np.float32)
    if wl.logits == "zipf":
        z = (z.astype(np.float64) + zipf_bias(wl, seed)[None, :]).astype(np.float32)
    return z


def zipf_bias(wl: Workload, seed: int = 0) -> np.ndarray:
    """Per-expert logit bias -s*ln(rank): ln of a Zipf(s) pmf up to a constant.

    Ranks 1..E are assigned to experts by a seeded permutation, so popularity
    is not correlated with the expert index.
    """
    rank = _rng(seed, wl.wid, 2).permutation(wl.E) + 1
    return -ZIPF_S * np.log(rank.astype(np.float64))


def draw_router(wl: Workload, seed: int = 0) -> np.ndarray:
    return _rng(seed, wl.wid, 3).normal(0.0, 0.02, (wl.E, wl.H)).astype(np.float32)


def draw_shared_gate(wl: Workload, seed: int = 0) -> np.ndarray:
    return _rng(seed, wl.wid, 4).normal(0.0, 0.02, (wl.H,)).astype(np.float32)


def draw_residual(wl: Workload, seed: int = 0, T: Optional[int] = None) -> np.ndarray:
    """fp32 residual stream [T][H] for the folded residual step, N(0, 1)."""
    T = wl.T if T is None else T
    return _rng(seed, wl.wid, 5).standard_normal((T, wl.H), dtype=np.float32)


def draw_norm_weight(wl: Workload, seed: int = 0) -> np.ndarray:
    """fp32 RMSnorm weight [H] of the next layer, 1 + N(0, 0.1)."""
    return (1.0 + 0.1 * _rng(seed, wl.wid, 6).standard_normal(wl.H)).astype(np.float32)


def draw_plane(N: int, K: int, rng: np.random.Generator):
    """One int4 plane: packed nibbles [N][K/2] (uniform 0..15) + fp16 scales [N][K/32]."""
    q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = (rng.random((N, K // GROUP), dtype=np.float32) * np.float32(0.015)
         + np.float32(0.005)).astype(np.float16).view(np.uint16)
    return q, s


MX_EXP_LO, MX_EXP_HI = 119, 122


def draw_plane_mxfp4(N: int, K: int, rng: np.random.Generator):
    """One MXFP4 plane: packed e2m1 nibbles [N][K/2] (uniform bytes) + ue8m0 bytes [N][K/32]."""
    q = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.integers(MX_EXP_LO, MX_EXP_HI + 1, size=(N, K // GROUP), dtype=np.uint8)
    return q, s


DRAW = {"int4": draw_plane, "mxfp4": draw_plane_mxfp4}
SCALE_DTYPE = {"int4": np.uint16, "mxfp4": np.uint8}

PLANES = ("gate", "up", "down")


def plane_shape(wl: Workload, plane: str, shared: bool = False):
    inter = wl.SI if shared else wl.I
    return (inter, wl.H) if plane in ("gate", "up") else (wl.H, inter)


def draw_expert(wl: Workload, e: int, plane: str, seed: int = 0, fmt: str = "int4"):
    N, K = plane_shape(wl, plane)
    return DRAW[fmt](N, K, _rng(seed, wl.wid, 10, e, PLANES.index(plane)))


def draw_shared(wl: Workload, plane: str, seed: int = 0, fmt: str = "int4"):
    N, K = plane_shape(wl, plane, shared=True)
    return DRAW[fmt](N, K, _rng(seed, wl.wid, 11, PLANES.index(plane)))


def draw_all_experts(wl: Workload, plane: str, seed: int = 0,
                     experts: Optional[Iterable[int]] = None, fmt: str = "int4"):
    """Stacked planes [E][N][K/2] and [E][N][K/32].

    Experts not listed in ``experts`` (when given) are left as zero bytes /
    zero scales; callers that only need some experts save the draw time.
    """
    N, K = plane_shape(wl, plane)
    q = np.zeros((wl.E, N, K // 2), dtype=np.uint8)
    s = np.zeros((wl.E, N, K // GROUP), dtype=SCALE_DTYPE[fmt])
    for e in (range(wl.E) if experts is None else experts):
        q[e], s[e] = draw_expert(wl, e, plane, seed, fmt)
    return q, s


@dataclasses.dataclass
class LayerInputs:
    wl: Workload
    x: np.ndarray
    logits: Optional[np.ndarray]
    w_router: Optional[np.ndarray]
    shared_gate: Optional[np.ndarray]
    planes: Dict[str, tuple]          # name -> (q [E][N][K/2], s [E][N][K/32])
    shared: Optional[Dict[str, tuple]]  # name -> (q [N][K/2], s [N][K/32])
    fmt: str = "int4"                   # weight format of every plane


def make_layer_inputs(wl: Workload, seed: int = 0, T: Optional[int] = None,
                      experts: Optional[Iterable[int]] = None, fmt: str = "int4") -> LayerInputs:
    x = draw_x(wl, seed, T)
    logits = draw_logits(wl, seed, T) if wl.logits in ("given", "zipf") else None
    w_router = draw_router(wl, seed) if wl.logits == "router" else None
    experts = None if experts is None else sorted(set(int(e) for e in experts))
    planes = {p: draw_all_experts(wl, p, seed, experts, fmt) for p in PLANES}
    shared = shared_gate = None
    if wl.SI > 0:
        shared = {p: draw_shared(wl, p, seed, fmt) for p in PLANES}
        shared_gate = draw_shared_gate(wl, seed)
    return LayerInputs(wl, x, logits, w_router, shared_gate, planes, shared, fmt)
