"""GPU tests of the router variants (sigmoid scores, a selection bias): the
router's indices bit-exact and weights within 1e-6 of the oracle on rows
whose selection has a margin, forced ties resolved to the lower index, and
the whole layer with a variant router on both expert paths and every routing
path (the GEMV's fused small-batch routing, the one-workgroup route kernel,
the separate top-k launch) against the CPU oracle.

Selection bias draws (seeded, test-side): N(0, 0.05) beside sigmoid scores in
(0, 1); N(0, 1/E) beside softmax probabilities, whose mean is 1/E."""
import numpy as np
import pytest
import scipy.special
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import DeviceLayer, W_RTOL, assert_y_close, dev, host, say
from test_gpu_parity import MID, _oracle_logits, _rows

pytestmark = pytest.mark.gpu

VARIANTS = [("sigmoid", False), ("sigmoid", True), ("softmax", True)]
SCORE = {"softmax": moe.MOE_SCORE_SOFTMAX, "sigmoid": moe.MOE_SCORE_SIGMOID}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _bias(gate, E, seed):
    rng = np.random.default_rng([seed, E, 77])
    sd = 0.05 if gate == "sigmoid" else 1.0 / E
    return (rng.standard_normal(E) * sd).astype(np.float32)


def _keys(L, gate, bias):
    z = L.astype(np.float64)
    s = scipy.special.expit(z) if gate == "sigmoid" else scipy.special.softmax(z, axis=1)
    return s + (0.0 if bias is None else bias.astype(np.float64))


def _decided_rows(L, k, gate, bias, margin=1e-12):
    """Rows where the k+1 largest selection keys are pairwise equal or more
    than `margin` apart (closer keys could order differently under the two
    sides' fp64 rounding of exp)."""
    key = -np.sort(-_keys(L, gate, bias), axis=1)[:, :k + 1]
    gap = np.abs(np.diff(key, axis=1))
    return np.all((gap == 0.0) | (gap > margin), axis=1)


def _router(L, k, scale, gate, bias):
    T, E = L.shape
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(dev(L), T, E, k, scale, idx, w, score=SCORE[gate],
                        select_bias=None if bias is None else dev(bias))
    torch.cuda.synchronize()
    return host(idx), host(w)


@pytest.mark.parametrize("gate,with_bias", VARIANTS)
@pytest.mark.parametrize("T,E,k", [(4, 8, 2), (1, 256, 8), (32, 128, 8), (512, 60, 4),
                                   (2048, 256, 8), (5, 64, 64), (33, 200, 17), (9, 1, 1)])
def test_router_topk_variant(T, E, k, gate, with_bias):
    say("variant router %s bias=%s T=%d E=%d k=%d" % (gate, with_bias, T, E, k))
    rng = np.random.default_rng([T, E, k, 31])
    L = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    b = _bias(gate, E, T) if with_bias else None
    idx_ref, w_ref, _ = oracle.router_topk(L, k, 1.25, gate=gate, bias=b)
    idx, w = _router(L, k, 1.25, gate, b)
    ok = _decided_rows(L, k, gate, b)
    assert ok.mean() > 0.99
    assert np.array_equal(idx[ok], idx_ref[ok])
    rel = np.abs(w[ok].astype(np.float64) - w_ref[ok]) / np.abs(w_ref[ok].astype(np.float64))
    assert rel.max() <= W_RTOL
    # every row: k distinct valid experts
    srt = np.sort(idx, axis=1)
    assert np.all((idx >= 0) & (idx < E)) and np.all(np.diff(srt, axis=1) > 0)


@pytest.mark.parametrize("gate", ["sigmoid", "softmax"])
def test_router_variant_forced_ties(gate):
    """Exact key ties (repeated logits, biases from a few values) go to the
    lower expert index on both sides."""
    rng = np.random.default_rng(5)
    for E, k in [(8, 3), (64, 8), (256, 8), (100, 50)]:
        T = 16
        L = rng.integers(0, 3, size=(T, E)).astype(np.float32)
        L[0] = 1.0  # an all-equal row
        for b in (None, rng.choice(np.array([0.0, 0.25, -0.5], np.float32), E)):
            idx_ref, w_ref, _ = oracle.router_topk(L, k, 1.0, gate=gate, bias=b)
            idx, w = _router(L, k, 1.0, gate, b)
            assert np.array_equal(idx, idx_ref), (gate, E, k, b is None)
            rel = np.abs(w.astype(np.float64) - w_ref) / w_ref
            assert rel.max() <= W_RTOL
        if b is None:
            assert np.array_equal(idx[0], np.arange(k))


def test_router_variant_rejections():
    L = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    idx = torch.empty((2, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((2, 2), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_router_topk(L, 2, 8, 2, 1.0, idx, w, score=2)
    assert e.value.status == moe.MOE_ERR_INVALID_ARG
    with pytest.raises(moe.MoeError) as e:
        moe.moe_router_topk(L, 2, 8, 2, 1.0, idx, w, top_p=0.5, score=moe.MOE_SCORE_SIGMOID)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    b = torch.zeros(9, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_router_topk(L, 2, 8, 2, 1.0, idx, w, select_bias=b.data_ptr() + 2)
    assert e.value.status == moe.MOE_ERR_INVALID_ARG


def _run_variant(d, L, gate, bias, path, scale=1.0):
    wl = d.inp.wl
    T = d.inp.x.shape[0]
    bd = None if bias is None else dev(bias)
    sh = moe.make_shape(T, wl.H, wl.E, wl.k, wl.I, wl.SI if d.shared else 0, path=path,
                        route_scale=scale, layout=d.layout, format=d.format,
                        score=SCORE[gate], select_bias=bd)
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
def test_layer_mid_variant(wl, path, layout):
    gate = "sigmoid"
    say("variant layer %s path=%d %s" % (wl.name, path, layout))
    inp = S.make_layer_inputs(wl, seed=6)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    b = _bias(gate, wl.E, 1)
    assert np.all(_decided_rows(L, wl.k, gate, b))
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                         route_scale=2.5, gate=gate, bias=b)
    y, idx, w = _run_variant(d, L, gate, b, path, scale=2.5)
    assert np.array_equal(idx, idx_ref)
    rel = np.abs(w.astype(np.float64) - w_ref) / np.abs(w_ref.astype(np.float64))
    assert rel.max() <= W_RTOL
    assert_y_close(y, y_ref, "%s variant" % wl.name)


@pytest.mark.parametrize("name,gate,layout", [("decode", "sigmoid", "rows"),
                                              ("decode", "sigmoid", "tiled"),
                                              ("decode_batch", "softmax", "rows"),
                                              ("prefill_skewed", "sigmoid", "rows")])
def test_layer_full_size_variant(name, gate, layout):
    """One workload per routing path: the GEMV's fused routing (decode), the
    one-workgroup route kernel (decode_batch, 256 slots) and the separate
    top-k launch (the 16384-slot skewed prefill)."""
    wl = S.WORKLOADS[name]
    say("full-size variant layer %s %s %s" % (name, gate, layout))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    b = _bias(gate, wl.E, 2)
    ok = _decided_rows(L, wl.k, gate, b)
    y, idx, _ = _run_variant(d, L, gate, b, moe.MOE_PATH_AUTO)
    idx_ref, _, _ = oracle.router_topk(L, wl.k, 1.0, gate=gate, bias=b)
    assert np.array_equal(idx[ok], idx_ref[ok])
    rows = [r for r in (_rows(wl) or range(wl.T)) if ok[r]]
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate, rows=rows,
                               gate=gate, bias=b)
    assert_y_close(y[rows], y_ref, name + " variant")
