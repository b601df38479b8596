"""GPU tests of the grouped (noaux_tc) router: E experts in n_group groups of
consecutive experts, a group scored by the sum of its two largest selection
keys, the topk_group best groups kept, the top-k keys among their experts.

The router's indices bit-exact and weights within 1e-6 of the oracle on rows
whose group and expert selections have a margin, forced ties resolved to the
lower index, and the whole layer with a grouped router on both expert paths
and on all three routing paths (the GEMV's fused small-batch routing, the
one-workgroup route kernel, the separate top-k launch) at E = 256,
n_group = 8, topk_group = 4, k = 8, against the CPU oracle."""
import numpy as np
import pytest
import scipy.special
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import DeviceLayer, W_RTOL, assert_y_close, dev, host, say
from test_gpu_parity import MID, _mid, _oracle_logits, _rows

pytestmark = pytest.mark.gpu

SCORE = {"softmax": moe.MOE_SCORE_SOFTMAX, "sigmoid": moe.MOE_SCORE_SIGMOID}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _bias(gate, E, seed):
    rng = np.random.default_rng([seed, E, 78])
    sd = 0.05 if gate == "sigmoid" else 1.0 / E
    return (rng.standard_normal(E) * sd).astype(np.float32)


def _decided_rows(L, k, gate, bias, ng, tg, margin=1e-12):
    """Rows whose kept groups and picks cannot change under the two sides'
    fp64 rounding of exp: the topk_group + 1 largest group scores, and the
    k + 1 largest keys inside the kept groups, pairwise equal or more than
    `margin` apart."""
    z = L.astype(np.float64)
    s = scipy.special.expit(z) if gate == "sigmoid" else scipy.special.softmax(z, axis=1)
    key = s + (0.0 if bias is None else bias.astype(np.float64))
    T, E = key.shape
    gsz = E // ng
    kg = -np.sort(-key.reshape(T, ng, gsz), axis=2)
    gs = kg[:, :, 0] + (kg[:, :, 1] if gsz >= 2 else 0.0)
    ok = np.ones(T, bool)
    for t in range(T):
        order = sorted(range(ng), key=lambda g: (-gs[t, g], g))
        top = gs[t, order[:min(tg + 1, ng)]]
        gap = np.abs(np.diff(top))
        kept = [e for e in range(E) if e // gsz in order[:tg]]
        kk = -np.sort(-key[t, kept])[:k + 1]
        gap2 = np.abs(np.diff(kk))
        ok[t] = np.all((gap == 0) | (gap > margin)) and np.all((gap2 == 0) | (gap2 > margin))
    return ok


def _router(L, k, gate, bias, ng, tg, scale=1.0):
    T, E = L.shape
    idx = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(dev(L), T, E, k, scale, idx, w, score=SCORE[gate],
                        select_bias=None if bias is None else dev(bias), n_group=ng,
                        topk_group=tg)
    torch.cuda.synchronize()
    return host(idx), host(w)


ROUTER_CASES = [(1, 256, 8, 8, 4), (32, 256, 8, 8, 4), (2048, 256, 8, 8, 4), (32, 128, 8, 8, 3),
                (512, 60, 4, 4, 2), (4, 8, 2, 4, 2), (9, 64, 8, 16, 2), (5, 160, 64, 16, 16),
                (7, 12, 5, 12, 5)]


@pytest.mark.parametrize("gate,with_bias", [("sigmoid", True), ("sigmoid", False),
                                            ("softmax", True)])
@pytest.mark.parametrize("T,E,k,ng,tg", ROUTER_CASES)
def test_router_topk_grouped(T, E, k, ng, tg, gate, with_bias):
    say("grouped router %s bias=%s T=%d E=%d k=%d n_group=%d topk_group=%d"
        % (gate, with_bias, T, E, k, ng, tg))
    rng = np.random.default_rng([T, E, k, ng, 32])
    L = (rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    b = _bias(gate, E, T) if with_bias else None
    idx_ref, w_ref, _ = oracle.router_topk(L, k, 1.25, gate=gate, bias=b, n_group=ng,
                                           topk_group=tg)
    idx, w = _router(L, k, gate, b, ng, tg, 1.25)
    ok = _decided_rows(L, k, gate, b, ng, tg)
    assert ok.mean() > 0.99
    assert np.array_equal(idx[ok], idx_ref[ok])
    rel = np.abs(w[ok].astype(np.float64) - w_ref[ok]) / np.abs(w_ref[ok].astype(np.float64))
    assert rel.max() <= W_RTOL
    # every row: k distinct experts, all from at most topk_group groups
    gsz = E // ng
    for t in range(T):
        assert len(set(idx[t].tolist())) == k and np.all((idx[t] >= 0) & (idx[t] < E))
        assert len(set((idx[t] // gsz).tolist())) <= tg


@pytest.mark.parametrize("gate", ["sigmoid", "softmax"])
def test_router_grouped_forced_ties(gate):
    """Exact ties among keys and among group scores go to the lower index on
    both sides, every row.  Without a bias: integer logits from {0, 1, 2}
    (equal top-two multisets give equal group sums on each side; different
    ones are far apart).  With a bias from {0, 0.25, -0.5}: zero logits, so
    every key 1/2 + b (sigmoid) or 1/E + b (softmax) is computed the same on
    both sides and sums of different bias pairs never meet."""
    rng = np.random.default_rng(6)
    for E, k, ng, tg in [(8, 3, 4, 2), (64, 8, 8, 4), (256, 8, 8, 4), (96, 20, 12, 6)]:
        T = 24
        cases = [(rng.integers(0, 3, size=(T, E)).astype(np.float32), None),
                 (np.zeros((T, E), np.float32),
                  rng.choice(np.array([0.0, 0.25, -0.5], np.float32), E))]
        cases[0][0][0] = 1.0  # an all-equal row: groups 0..tg-1, experts in index order
        for L, b in cases:
            idx_ref, w_ref, _ = oracle.router_topk(L, k, 1.0, gate=gate, bias=b, n_group=ng,
                                                   topk_group=tg)
            idx, w = _router(L, k, gate, b, ng, tg)
            assert np.array_equal(idx, idx_ref), (gate, E, k, b is None)
            assert (np.abs(w.astype(np.float64) - w_ref) / w_ref).max() <= W_RTOL
            if b is None:
                assert np.array_equal(idx[0], np.arange(k))


def test_router_grouped_rejections():
    L = torch.zeros((2, 8), dtype=torch.float32, device="cuda")
    idx = torch.empty((2, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((2, 2), dtype=torch.float32, device="cuda")
    for kw, status in [(dict(n_group=3, topk_group=1), moe.MOE_ERR_INVALID_ARG),
                       (dict(n_group=4, topk_group=5), moe.MOE_ERR_INVALID_ARG),
                       (dict(n_group=4, topk_group=2, top_p=0.5), moe.MOE_ERR_UNSUPPORTED)]:
        with pytest.raises(moe.MoeError) as e:
            moe.moe_router_topk(L, 2, 8, 2, 1.0, idx, w, score=moe.MOE_SCORE_SIGMOID, **kw)
        assert e.value.status == status


def _run_grouped(d, L, gate, bias, ng, tg, path, scale=1.0):
    wl = d.inp.wl
    T = d.inp.x.shape[0]
    bd = None if bias is None else dev(bias)
    sh = moe.make_shape(T, wl.H, wl.E, wl.k, wl.I, wl.SI if d.shared else 0, path=path,
                        route_scale=scale, layout=d.layout, format=d.format,
                        score=SCORE[gate], select_bias=bd, n_group=ng, topk_group=tg)
    nbytes = moe.moe_workspace_bytes(sh)
    assert nbytes > 0
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    y = torch.full((T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((T, wl.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((T, wl.k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_layer(sh, d.x, dev(L), None, d.planes["gate"], d.planes["up"], d.planes["down"],
                  d.shared, d.shared_gate, y, idx, w, None, ws, nbytes)
    torch.cuda.synchronize()
    return host(y), host(idx), host(w)


# (shape, n_group, topk_group): the mid shapes whose E the grouping divides,
# and 40 tokens x E = 256, which takes the one-workgroup route kernel
GROUPED_MID = [(MID[0], 4, 2), (MID[4], 8, 4), (MID[5], 4, 2), (MID[6], 8, 4), (MID[7], 8, 4),
               (_mid("grouped_route", 34, 40, 256, 256, 8, 128), 8, 4)]


# (path, layout): both paths on row planes, the GEMV on tiled planes
PATH_LAYOUTS = [(moe.MOE_PATH_GEMV, "rows"), (moe.MOE_PATH_GEMM, "rows"), (moe.MOE_PATH_GEMV, "tiled")]


@pytest.mark.parametrize("path,layout", PATH_LAYOUTS, ids=["gemv", "gemm", "tiled_gemv"])
@pytest.mark.parametrize("case", GROUPED_MID, ids=[c[0].name for c in GROUPED_MID])
def test_layer_mid_grouped(case, path, layout):
    wl, ng, tg = case
    gate = "sigmoid"
    say("grouped layer %s n_group=%d topk_group=%d path=%d %s" % (wl.name, ng, tg, path, layout))
    inp = S.make_layer_inputs(wl, seed=7)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    b = _bias(gate, wl.E, 3)
    ok = _decided_rows(L, wl.k, gate, b, ng, tg)
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                         route_scale=2.5, gate=gate, bias=b, n_group=ng,
                                         topk_group=tg)
    y, idx, w = _run_grouped(d, L, gate, b, ng, tg, path, scale=2.5)
    assert ok.all()
    assert np.array_equal(idx, idx_ref)
    rel = np.abs(w.astype(np.float64) - w_ref) / np.abs(w_ref.astype(np.float64))
    assert rel.max() <= W_RTOL
    assert_y_close(y, y_ref, "%s grouped" % wl.name)


@pytest.mark.parametrize("name,layout", [("decode", "rows"), ("decode", "tiled"),
                                         ("prefill_skewed", "rows")])
def test_layer_full_size_grouped(name, layout):
    """E = 256, n_group = 8, topk_group = 4, k = 8 at full size: the GEMV's
    fused routing (decode) and the separate top-k launch (the 16384-slot
    skewed prefill); the route kernel's case is grouped_route above."""
    wl = S.WORKLOADS[name]
    gate = "sigmoid"
    say("full-size grouped layer %s %s" % (name, layout))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    L = _oracle_logits(inp)
    b = _bias(gate, wl.E, 4)
    ok = _decided_rows(L, wl.k, gate, b, 8, 4)
    y, idx, _ = _run_grouped(d, L, gate, b, 8, 4, moe.MOE_PATH_AUTO)
    idx_ref, _, _ = oracle.router_topk(L, wl.k, 1.0, gate=gate, bias=b, n_group=8, topk_group=4)
    assert ok.mean() > 0.99
    assert np.array_equal(idx[ok], idx_ref[ok])
    rows = [r for r in (_rows(wl) or range(wl.T)) if ok[r]]
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate, rows=rows,
                               gate=gate, bias=b, n_group=8, topk_group=4)
    assert_y_close(y[rows], y_ref, name + " grouped")
