"""GPU tests of expert top-p (after the top-k): the router's indices (-1 for
a dropped pick) bit-exact and weights within 1e-6 of the oracle on rows whose
top-p decision has a margin, and the whole layer with top-p on both expert
paths (the GEMV path's fused small-batch routing included) against the CPU
oracle."""
import numpy as np
import pytest
import scipy.special
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import DeviceLayer, W_RTOL, assert_y_close, dev, host, run_layer, say
from test_gpu_parity import MID, _oracle_logits, _rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _decided_rows(L, k, p, margin=1e-9):
    """Rows where no prefix probability of the top-k lies within `margin` of
    p (there fp64 rounding order could flip the keep decision)."""
    P = scipy.special.softmax(L.astype(np.float64), axis=1)
    idx, _, _ = oracle.router_topk(L, k)
    cum = np.cumsum(np.take_along_axis(P, idx.astype(np.int64), axis=1), axis=1)
    return np.all(np.abs(cum - p) > margin, axis=1)


@pytest.mark.parametrize("p", [0.3, 0.7, 0.95])
@pytest.mark.parametrize("T,E,k", [(4, 8, 2), (1, 256, 8), (32, 128, 8), (512, 60, 4),
                                   (2048, 256, 8), (5, 64, 64), (33, 200, 17)])
def test_router_topk_top_p(T, E, k, p):
    say("top-p T=%d E=%d k=%d p=%.2f" % (T, E, k, p))
    rng = np.random.default_rng([T, E, k, int(p * 100)])
    L = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    idx_ref, w_ref, _ = oracle.router_topk(L, k, 1.25, p)
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(dev(L), T, E, k, 1.25, idx, w, top_p=p)
    torch.cuda.synchronize()
    idx, w = host(idx), host(w)
    ok = _decided_rows(L, k, p)
    assert ok.mean() > 0.99
    assert np.array_equal(idx[ok], idx_ref[ok])
    kept = idx_ref[ok] >= 0
    rel = np.abs(w[ok][kept].astype(np.float64) - w_ref[ok][kept]) / np.abs(w_ref[ok][kept])
    assert rel.max() <= W_RTOL
    assert np.all(w[ok][~kept] == 0.0)
    n_kept = kept.sum(axis=1)
    say("  kept picks per token: mean %.2f of %d, min %d" % (n_kept.mean(), k, n_kept.min()))


def _run_top_p(d, L, p, path):
    wl = d.inp.wl
    T = d.inp.x.shape[0]
    sh = moe.make_shape(T, wl.H, wl.E, wl.k, wl.I, wl.SI if d.shared else 0, path=path,
                        layout=d.layout, format=d.format, top_p=p)
    nbytes = moe.moe_workspace_bytes(sh)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)
    y = torch.full((T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((T, wl.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, wl.k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_layer(sh, d.x, dev(L), None, d.planes["gate"], d.planes["up"], d.planes["down"],
                  d.shared, d.shared_gate, y, idx, w, None, ws, nbytes)
    torch.cuda.synchronize()
    return host(y), host(idx), host(w)


# (path, layout): both paths on row planes, the GEMV on tiled planes
PATH_LAYOUTS = [(moe.MOE_PATH_GEMV, "rows"), (moe.MOE_PATH_GEMM, "rows"), (moe.MOE_PATH_GEMV, "tiled")]


@pytest.mark.parametrize("path,layout", PATH_LAYOUTS, ids=["gemv", "gemm", "tiled_gemv"])
@pytest.mark.parametrize("wl", MID, ids=[w.name for w in MID])
def test_layer_mid_top_p(wl, path, layout):
    p = 0.6
    say("top-p layer %s path=%d %s" % (wl.name, path, layout))
    inp = S.make_layer_inputs(wl, seed=5)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    assert np.all(_decided_rows(L, wl.k, p))
    y_ref, idx_ref, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                     top_p=p)
    y, idx, _ = _run_top_p(d, L, p, path)
    assert np.array_equal(idx, idx_ref)
    assert_y_close(y, y_ref, "%s top-p" % wl.name)


@pytest.mark.parametrize("name,layout", [("decode", "rows"), ("decode", "tiled"),
                                         ("decode_batch", "rows"), ("prefill_skewed", "rows")])
def test_layer_full_size_top_p(name, layout):
    p = 0.7
    wl = S.WORKLOADS[name]
    say("full-size top-p layer %s %s" % (name, layout))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    ok = _decided_rows(L, wl.k, p)
    y, idx, _ = _run_top_p(d, L, p, moe.MOE_PATH_AUTO)
    idx_ref, _, _ = oracle.router_topk(L, wl.k, 1.0, p)
    assert np.array_equal(idx[ok], idx_ref[ok])
    rows = [r for r in (_rows(wl) or range(wl.T)) if ok[r]]
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate, rows=rows,
                               top_p=p)
    assert_y_close(y[rows], y_ref, name + " top-p")
