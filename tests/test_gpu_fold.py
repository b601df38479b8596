"""GPU tests of the layer with its combine folded into the residual step
(moe_layer_residual_rmsnorm): the residual's increment against the oracle's
FFN row, and the normed bf16 row against the oracle's add+rms applied to the
kernel's own residual (at most one bf16 unit in the last place apart: the
kernel sums squares and scales in fp32, the oracle in fp64, and both round
once to bf16)."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import (Canaried, DeviceLayer, Y_TOL, assert_w_close, assert_y_close, dev, host,
                         logits_bound, run_layer, say)
from test_gpu_parity import MID, _mid, _oracle_logits, _rows

pytestmark = pytest.mark.gpu

EPS = 1e-6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _run_fold(d, L, r, g, path=moe.MOE_PATH_AUTO, alias_x=False, next_w=None):
    """The oracle's logits L go in as given logits (the router itself is
    checked elsewhere), so both sides pick the same experts.  With next_w
    (fp32 [E'][H]) the call also returns the next layer's logits."""
    wl = d.inp.wl
    T = d.inp.x.shape[0]
    sh = moe.make_shape(T, wl.H, wl.E, wl.k, wl.I, wl.SI if d.shared else 0, path=path,
                        layout=d.layout, format=d.format)
    nbytes = moe.moe_workspace_bytes(sh)
    assert nbytes > 0
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    res = dev(r)
    gd = dev(g)
    x = d.x.clone() if alias_x else d.x
    xn = x if alias_x else torch.full((T, wl.H), 0x7FC0, dtype=torch.int16, device="cuda")
    nw = nl = None
    nE = 0
    if next_w is not None:
        nE = next_w.shape[0]
        nw = dev(next_w)
        nl = Canaried((T, nE), torch.float32, float("nan"), "next_logits")
    moe.moe_layer_residual_rmsnorm(sh, x, dev(L), None, d.planes["gate"], d.planes["up"],
                                   d.planes["down"], d.shared, d.shared_gate, res, gd, EPS, xn,
                                   None, None, ws, nbytes, next_w_router=nw, next_E=nE,
                                   next_logits=None if nl is None else nl.view)
    torch.cuda.synchronize()
    if nl is None:
        return host(res), host(xn, np.uint16)
    nl.check()
    return host(res), host(xn, np.uint16), host(nl.view)


def _check(r, r_out, n_out, y_ref, g, what):
    """Increment within the layer's bar (plus fp32 rounding at the residual's
    magnitude); normed row within one bf16 ulp of the oracle's norm of r_out."""
    inc = r_out.astype(np.float64) - r.astype(np.float64)
    err = np.max(np.abs(inc - y_ref), axis=1)
    bar = Y_TOL * np.max(np.abs(y_ref), axis=1) + 16 * 2.0 ** -24 * np.max(np.abs(r_out), axis=1)
    say("  %s: worst increment error %.3e of its bar" % (what, float(np.max(err / bar))))
    assert np.all(err <= bar), "%s: row %d" % (what, int(np.argmax(err / bar)))
    _, n_ref = oracle.add_rmsnorm(r_out, np.zeros_like(r_out), g, EPS)
    mag = lambda b: (b & 0x7FFF).astype(np.int32)
    sign_ok = ((n_out ^ n_ref) & 0x8000) == 0
    ulps = np.abs(mag(n_out) - mag(n_ref))
    assert np.all(sign_ok | ((mag(n_out) == 0) & (mag(n_ref) == 0))), what + ": sign"
    say("  %s: normed row max %d ulp, %.4f%% not bit-equal" % (what, int(ulps.max()),
                                                               100.0 * np.mean(ulps > 0)))
    assert ulps.max() <= 1, what


# (path, layout): both paths on row planes, the GEMV on tiled planes
PATH_LAYOUTS = [(moe.MOE_PATH_GEMV, "rows"), (moe.MOE_PATH_GEMM, "rows"), (moe.MOE_PATH_GEMV, "tiled")]


@pytest.mark.parametrize("path,layout", PATH_LAYOUTS, ids=["gemv", "gemm", "tiled_gemv"])
@pytest.mark.parametrize("wl", MID, ids=[w.name for w in MID])
def test_fold_mid(wl, path, layout):
    say("fold %s path=%d %s" % (wl.name, path, layout))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    r = S.draw_residual(wl, T=inp.x.shape[0])
    g = S.draw_norm_weight(wl)
    r_out, n_out = _run_fold(d, L, r, g, path=path)
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate)
    _check(r, r_out, n_out, y_ref, g, wl.name)


@pytest.mark.parametrize("name,fmt,layout", [("decode", "int4", "rows"), ("decode", "int4", "tiled"),
                                             ("decode", "mxfp4", "rows"), ("decode", "mxfp4", "tiled"),
                                             ("prefill_shared", "int4", "rows")])
def test_fold_full_size(name, fmt, layout):
    wl = S.WORKLOADS[name]
    say("fold full-size %s %s %s" % (name, fmt, layout))
    inp = S.make_layer_inputs(wl, seed=0, fmt=fmt)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    r = S.draw_residual(wl)
    g = S.draw_norm_weight(wl)
    r_out, n_out = _run_fold(d, L, r, g)
    rows = _rows(wl)
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                               rows=rows, fmt=fmt)
    sel = slice(None) if rows is None else rows
    _check(r[sel], r_out[sel], n_out[sel], y_ref, g, name)


def test_fold_x_next_in_place():
    """x_next may be x itself: the normed row overwrites the layer's input."""
    wl = MID[1]  # a gated shared expert: x is read by the gate logit and the MLPs
    inp = S.make_layer_inputs(wl, seed=3)
    d = DeviceLayer(inp)
    L = _oracle_logits(inp)
    r = S.draw_residual(wl, seed=3, T=inp.x.shape[0])
    g = S.draw_norm_weight(wl, seed=3)
    r_out, n_out = _run_fold(d, L, r, g, alias_x=True)
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate)
    _check(r, r_out, n_out, y_ref, g, wl.name + " in place")


# --------------------------------- the next layer's router folded into the norm --

def _next_router(wl, E_next, seed):
    return np.random.default_rng([seed, wl.wid, E_next, 91]).normal(
        0.0, 0.02, (E_next, wl.H)).astype(np.float32)


def _check_next_logits(n_out, lo, W, what):
    """The folded logits against the oracle's fp64 logits of the device's own
    bf16 normed rows, within the fp32 forward-error bound."""
    ref = oracle.router_logits(n_out, W)
    bound = logits_bound(n_out, W)
    err = np.abs(lo.astype(np.float64) - ref.astype(np.float64))
    say("  %s: worst next-logit error %.3e of its bound" % (what, float(np.max(err / bound))))
    assert np.all(np.isfinite(lo)) and np.all(err <= bound + 1e-30), what


# (shape, next layer's experts): shapes of up to 32 tokens and H <= 6144 take
# the one-launch fold (30 tokens: a ragged 4-row block and a ragged block of
# router rows); the 40-, 70- and 200-token ones and H = 8192 take the norm
# launch and the router-logits kernel
FOLD_ROUTER = [(MID[4], 64), (MID[7], 256), (_mid("fold_router_30", 36, 30, 256, 8, 2, 128), 101),
               (MID[3], 6), (MID[8], 16), (MID[1], 12), (MID[2], 40)]


@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
@pytest.mark.parametrize("case", FOLD_ROUTER, ids=["%s-E%d" % (c[0].name, c[1]) for c in FOLD_ROUTER])
def test_fold_next_router(case, path):
    wl, E_next = case
    say("fold with next router %s E'=%d path=%d" % (wl.name, E_next, path))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    L = _oracle_logits(inp)
    r = S.draw_residual(wl, T=inp.x.shape[0])
    g = S.draw_norm_weight(wl)
    W = _next_router(wl, E_next, 1)
    r_out, n_out, lo = _run_fold(d, L, r, g, path=path, next_w=W)
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate)
    _check(r, r_out, n_out, y_ref, g, wl.name)
    _check_next_logits(n_out, lo, W, wl.name)


def test_fold_next_router_chains_two_layers():
    """Two decode layers chained the folded way: layer 1's residual step
    writes x_next and layer 2's logits; layer 2 takes both as its input and
    given logits.  Layer 2's picks are bit-exact against the oracle's top-k
    of those logits, its weights within 1e-6 and its y within the bar."""
    wl = S.Workload("chain", 35, 3, 2048, 64, 8, 512, 0, "given", "chain")
    inp1 = S.make_layer_inputs(wl, seed=0)
    inp2 = S.make_layer_inputs(wl, seed=1)
    d1 = DeviceLayer(inp1)
    r = S.draw_residual(wl, T=wl.T)
    g = S.draw_norm_weight(wl)
    W = _next_router(wl, wl.E, 2)
    r_out, n_out, lo = _run_fold(d1, inp1.logits, r, g, next_w=W)
    _check_next_logits(n_out, lo, W, "chain layer 1")
    inp2.x = n_out
    inp2.logits = lo
    d2 = DeviceLayer(inp2)
    y, idx, w, _ = run_layer(d2)
    y_ref, idx_ref, w_ref = oracle.layer(n_out, lo, wl.k, inp2.planes)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, "chain layer 2")
    assert_y_close(y, y_ref, "chain layer 2")


def test_fold_next_router_full_size_decode():
    wl = S.WORKLOADS["decode"]
    say("fold with next router, full-size decode")
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    r = S.draw_residual(wl)
    g = S.draw_norm_weight(wl)
    W = _next_router(wl, wl.E, 3)
    r_out, n_out, lo = _run_fold(d, inp.logits, r, g, next_w=W)
    y_ref, _, _ = oracle.layer(inp.x, inp.logits, wl.k, inp.planes)
    _check(r, r_out, n_out, y_ref, g, "decode")
    _check_next_logits(n_out, lo, W, "decode")
