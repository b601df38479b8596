"""Helpers for the GPU parity tests: device copies of seeded inputs, calls
through the C ABI (via the package binding), and the comparison bars.

Bars (fixed by the layer's accuracy requirements):
  * router indices, permutation and int4 decode: bit-exact;
  * router weights: within 1e-6 relative;
  * layer output y: per token row, max_h |y - y_ref| <= 2e-3 * max_h |y_ref|.
"""
import sys

import numpy as np
import torch

import moe_synth as S
import quantized_expert_mlp_amd as moe

Y_TOL = 2e-3
W_RTOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    return a.view(dtype) if dtype is not None else a


class DeviceLayer:
    """Device copies of one LayerInputs."""

    def __init__(self, inp: S.LayerInputs):
        self.inp = inp
        self.x = dev(inp.x)
        self.logits = None if inp.logits is None else dev(inp.logits)
        self.w_router = None if inp.w_router is None else dev(inp.w_router)
        self.shared_gate = None if inp.shared_gate is None else dev(inp.shared_gate)
        self.planes = {p: (dev(q), dev(s)) for p, (q, s) in inp.planes.items()}
        self.shared = None
        if inp.shared is not None:
            self.shared = [(dev(inp.shared[p][0]), dev(inp.shared[p][1])) for p in S.PLANES]
        self.layout = moe.MOE_LAYOUT_ROWS
        self.format = moe.MOE_FORMAT_MXFP4 if inp.fmt == "mxfp4" else moe.MOE_FORMAT_INT4

    def tiled(self) -> "DeviceLayer":
        """A copy whose planes are packed into the tiled layout on the device."""
        t = DeviceLayer.__new__(DeviceLayer)
        t.__dict__.update(self.__dict__)
        t.layout = moe.MOE_LAYOUT_TILED
        wl = self.inp.wl
        dims = {"gate": (wl.I, wl.H), "up": (wl.I, wl.H), "down": (wl.H, wl.I)}
        t.planes = {p: pack_plane(self.planes[p], *dims[p], self.format) for p in self.planes}
        if self.shared is not None:
            sd = [(wl.SI, wl.H), (wl.SI, wl.H), (wl.H, wl.SI)]
            t.shared = [pack_plane(pl, *nk, self.format) for pl, nk in zip(self.shared, sd)]
        torch.cuda.synchronize()
        return t


def pack_plane(plane, N, K, fmt=moe.MOE_FORMAT_INT4):
    """moe_pack_weights of one device plane set (E inferred from the sizes)."""
    q, s = plane
    E = q.numel() // (N * K // 2)
    dq, ds = torch.empty_like(q), torch.empty_like(s)
    moe.moe_pack_weights((q, s), E, N, K, (dq, ds), format=fmt)
    return dq, ds


def tiled_reference(q: np.ndarray, s: np.ndarray):
    """The tiled layout written out with numpy index arithmetic: per expert,
    block (b, c) of rows 32b..32b+31 and inputs 64c..64c+63 is 1 KB; within it
    row 32b+j's 16 bytes of scale group 2c+h sit at (32h + j) * 16; its scales
    at (b*(K/64) + c) * 64 + 32h + j."""
    E, N, Kh = q.shape
    K = 2 * Kh
    qt = q.reshape(E, N // 32, 32, K // 64, 2, 16).transpose(0, 1, 3, 4, 2, 5)
    st = s.reshape(E, N // 32, 32, K // 64, 2).transpose(0, 1, 3, 4, 2)
    return np.ascontiguousarray(qt).reshape(E, N, Kh), np.ascontiguousarray(st).reshape(E, N, K // 32)


# Canary words written past the end of every output and the workspace: a
# kernel that stores past its buffer changes them.
CANARY_WORDS = 64
CANARY_U32 = np.uint32(0x7FA5C3E1)  # a NaN payload no kernel writes


class Canaried:
    """A device buffer of `shape` (a view) followed by CANARY_WORDS canary
    words; check() asserts the canary is intact."""

    def __init__(self, shape, dtype, fill, what):
        n = int(np.prod(shape))
        itemsize = torch.empty((), dtype=dtype).element_size()
        extra = CANARY_WORDS * 4 // itemsize
        assert n * itemsize % 4 == 0
        self.full = torch.empty(n + extra, dtype=dtype, device="cuda")
        self.full.view(torch.int32)[n * itemsize // 4:].fill_(int(CANARY_U32.view(np.int32)))
        self.view = self.full[:n].view(*shape)
        self.view.fill_(fill)
        self.n, self.itemsize, self.what = n, itemsize, what

    def check(self):
        tail = host(self.full.view(torch.int32)[self.n * self.itemsize // 4:]).view(np.uint32)
        assert np.all(tail == CANARY_U32), "%s: write past the end of the buffer" % self.what


def run_layer(d: DeviceLayer, logits=None, use_router=False, path=moe.MOE_PATH_AUTO,
              route_scale=1.0, ws_extra=0):
    """moe_layer through the C ABI.  logits: host array to feed (given logits),
    else the inputs' own; use_router: compute logits from w_router.  The
    planes' layout and format are the DeviceLayer's."""
    wl = d.inp.wl
    T = d.inp.x.shape[0]
    sh = moe.make_shape(T, wl.H, wl.E, wl.k, wl.I, wl.SI if d.shared else 0,
                        route_scale=route_scale, path=path, layout=d.layout, format=d.format)
    nbytes = moe.moe_workspace_bytes(sh)
    assert nbytes > 0
    # poison: nothing may depend on the workspace's prior contents
    ws = Canaried((nbytes + ws_extra,), torch.uint8, 0xFF, "workspace")
    y = Canaried((T, wl.H), torch.float32, float("nan"), "y")
    idx = Canaried((T, wl.k), torch.int32, -7, "idx")
    w = Canaried((T, wl.k), torch.float32, float("nan"), "w")
    lo = Canaried((T, wl.E), torch.float32, float("nan"), "logits_out")
    if use_router:
        lg, wr = None, d.w_router
    else:
        lg = dev(logits.astype(np.float32)) if logits is not None else d.logits
        wr = None
    moe.moe_layer(sh, d.x, lg, wr, d.planes["gate"], d.planes["up"], d.planes["down"], d.shared,
                  d.shared_gate, y.view, idx.view, w.view, lo.view, ws.view, nbytes)
    torch.cuda.synchronize()
    for c in (ws, y, idx, w, lo):
        c.check()
    return host(y.view), host(idx.view), host(w.view), host(lo.view)


def y_errors(y: np.ndarray, y_ref: np.ndarray) -> np.ndarray:
    """Per-row max|y - y_ref| / max|y_ref|."""
    num = np.max(np.abs(y.astype(np.float64) - y_ref.astype(np.float64)), axis=1)
    den = np.maximum(np.max(np.abs(y_ref.astype(np.float64)), axis=1), 1e-30)
    return num / den


def assert_y_close(y, y_ref, what=""):
    assert np.all(np.isfinite(y)), "%s: non-finite outputs" % what
    err = y_errors(y, y_ref)
    worst = float(err.max()) if err.size else 0.0
    say("  %s: worst row error %.3e of max|y| (bar %.0e)" % (what, worst, Y_TOL))
    assert worst <= Y_TOL, "%s: row %d error %.3e > %.0e" % (what, int(err.argmax()), worst, Y_TOL)
    return worst


def assert_w_close(w, w_ref, what=""):
    rel = np.abs(w.astype(np.float64) - w_ref.astype(np.float64)) / np.abs(w_ref.astype(np.float64))
    worst = float(rel.max())
    say("  %s: worst router weight rel error %.3e (bar %.0e)" % (what, worst, W_RTOL))
    assert worst <= W_RTOL, what


def logits_bound(x_bits: np.ndarray, w_router: np.ndarray, gate=None) -> np.ndarray:
    """Forward-error bound of an fp32 dot of length H vs the exact value,
    (H + 2) * 2^-24 * sum_h |x_h W_eh|, plus the oracle's own rounding."""
    xa = np.abs(S.bf16_bits_to_f32(x_bits).astype(np.float64))
    wa = np.abs(w_router.astype(np.float64))
    H = x_bits.shape[1]
    return (H + 2) * 2.0 ** -24 * (xa @ wa.T)


def valid_topk(idx_row, L_ref_row, bound_row, k):
    """Is idx_row a top-k of L_ref_row under perturbations within bound_row?"""
    order = sorted(range(len(L_ref_row)), key=lambda e: (-L_ref_row[e], e))
    kth = L_ref_row[order[k - 1]]
    slack = 2 * float(np.max(bound_row)) + 1e-30
    if len(set(idx_row.tolist())) != k:
        return False
    for j, e in enumerate(idx_row):
        if L_ref_row[e] < kth - slack:
            return False
        if j > 0 and L_ref_row[e] > L_ref_row[idx_row[j - 1]] + slack:
            return False
    return True
