"""GPU tests of the tiled weight layout: moe_pack_weights against the layout's
definition (bit-exact, both scale sizes), and the whole layer on tiled int4
and MXFP4 planes against the CPU oracle on both expert paths (the streaming
GEMV over tiled blocks and the MFMA GEMM), at mid sizes and at the full
decode, decode-batch and prefill sizes."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import (DeviceLayer, assert_w_close, assert_y_close, dev, host, run_layer, say,
                         tiled_reference)
from test_gpu_parity import MID, SAMPLE_ROWS, _mid, _oracle_logits, _rows
from test_gpu_router_grouped import _decided_rows as grouped_decided
from test_gpu_top_p import _decided_rows as top_p_decided

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
@pytest.mark.parametrize("E,N,K", [(1, 32, 64), (3, 96, 192), (2, 64, 6144), (4, 1408, 128)])
def test_pack_matches_layout_definition(E, N, K, fmt):
    say("pack E=%d N=%d K=%d %s" % (E, N, K, fmt))
    rng = np.random.default_rng([7, E, N, K])
    q = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    mx = fmt == "mxfp4"
    st = np.uint8 if mx else np.uint16
    s = rng.integers(0, 256 if mx else 65536, (E, N, K // 32), dtype=st)
    dq = torch.full((E, N, K // 2), 0x5A, dtype=torch.uint8, device="cuda")
    ds = (torch.full((E, N, K // 32), 0x77, dtype=torch.uint8, device="cuda") if mx else
          torch.full((E, N, K // 32), 0x1234, dtype=torch.int16, device="cuda"))
    moe.moe_pack_weights((dev(q), dev(s)), E, N, K, (dq, ds),
                         format=moe.MOE_FORMAT_MXFP4 if mx else moe.MOE_FORMAT_INT4)
    torch.cuda.synchronize()
    q_ref, s_ref = tiled_reference(q, s)
    assert np.array_equal(host(dq), q_ref)
    assert np.array_equal(host(ds, st), s_ref)


PATHS = {"auto": moe.MOE_PATH_AUTO, "gemv": moe.MOE_PATH_GEMV, "gemm": moe.MOE_PATH_GEMM}


# AUTO takes the tiled GEMV for up to four tokens (its fused routing) and
# the MFMA GEMM beyond; both paths are also forced on every shape
@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("wl", MID, ids=[w.name for w in MID])
def test_layer_mid_tiled(wl, path):
    say("tiled layer %s path %s" % (wl.name, path))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp).tiled()
    L = _oracle_logits(inp)
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                         route_scale=0.75)
    y, idx, w, lo = run_layer(d, logits=L, route_scale=0.75, path=PATHS[path])
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, wl.name)
    assert_y_close(y, y_ref, "%s tiled" % wl.name)


@pytest.mark.parametrize("path", ["auto", "gemv"])
@pytest.mark.parametrize("wl", MID, ids=[w.name for w in MID])
def test_layer_mid_tiled_mxfp4(wl, path):
    say("tiled mxfp4 layer %s path %s" % (wl.name, path))
    inp = S.make_layer_inputs(wl, seed=0, fmt="mxfp4")
    d = DeviceLayer(inp).tiled()
    L = _oracle_logits(inp)
    y_ref, idx_ref, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                     fmt="mxfp4")
    y, idx, _, _ = run_layer(d, logits=L, path=PATHS[path])
    assert np.array_equal(idx, idx_ref)
    assert_y_close(y, y_ref, "%s tiled mxfp4" % wl.name)


# AUTO's tiled GEMV at both limits of its fused routing (4 tokens, 64 slots),
# with a bucket of up to 4 rows and a grouped and a top-p router on top
FUSED_LIMIT = _mid("tiled_fused_limit", 42, 4, 512, 64, 16, 256)


@pytest.mark.parametrize("router", ["softmax", "top_p", "grouped"])
def test_layer_tiled_gemv_fused_route_limits(router):
    wl = FUSED_LIMIT
    say("tiled GEMV at the fused routing's limits (%s)" % router)
    inp = S.make_layer_inputs(wl, seed=2)
    d = DeviceLayer(inp).tiled()
    L = _oracle_logits(inp)
    # make every expert's bucket hold up to 4 rows: the tokens share most picks
    L = (L + 3.0 * L[:1]).astype(np.float32)
    kw, okw = {}, {}
    if router == "top_p":
        kw, okw = dict(top_p=0.8), dict(top_p=0.8)
        assert np.all(top_p_decided(L, wl.k, 0.8))
    elif router == "grouped":
        kw = dict(score=moe.MOE_SCORE_SIGMOID, n_group=8, topk_group=4)
        okw = dict(gate="sigmoid", n_group=8, topk_group=4)
        assert np.all(grouped_decided(L, wl.k, "sigmoid", None, 8, 4))
    sh = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I, 0, layout=d.layout, **kw)
    nbytes = moe.moe_workspace_bytes(sh)
    sh_gemv = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I, 0, layout=d.layout,
                             path=moe.MOE_PATH_GEMV, **kw)
    assert nbytes == moe.moe_workspace_bytes(sh_gemv)  # AUTO takes the GEMV here
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    y = torch.full((wl.T, wl.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((wl.T, wl.k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((wl.T, wl.k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_layer(sh, d.x, dev(L), None, d.planes["gate"], d.planes["up"], d.planes["down"],
                  None, None, y, idx, w, None, ws, nbytes)
    torch.cuda.synchronize()
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes, **okw)
    got = host(idx)
    assert np.array_equal(got, idx_ref)
    counts = np.bincount(got[got >= 0].ravel(), minlength=wl.E)
    assert counts.max() >= 2
    # dropped picks (top-p) carry weight 0; the kept ones within the bar
    got_w, kept = host(w), idx_ref >= 0
    assert np.all(got_w[~kept] == 0.0)
    assert_w_close(got_w[kept], w_ref[kept], wl.name)
    assert_y_close(host(y), y_ref, "%s %s" % (wl.name, router))


# the widest K the tiled GEMV serves (its prepared row fills 48 KB of LDS:
# 614 groups of 80 bytes), on gate/up (K = H) and on down (K = I)
WIDEST = [_mid("tiled_widest_h", 40, 2, 19648, 4, 2, 128), _mid("tiled_widest_i", 41, 3, 128, 4, 2, 19648)]


@pytest.mark.parametrize("fmt", ["int4", "mxfp4"])
@pytest.mark.parametrize("wl", WIDEST, ids=[w.name for w in WIDEST])
def test_layer_tiled_gemv_widest(wl, fmt):
    say("tiled GEMV at its widest K: %s %s" % (wl.name, fmt))
    inp = S.make_layer_inputs(wl, seed=0, fmt=fmt)
    d = DeviceLayer(inp).tiled()
    L = _oracle_logits(inp)
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes, fmt=fmt)
    y, idx, w, _ = run_layer(d, logits=L, path=moe.MOE_PATH_GEMV)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, wl.name)
    assert_y_close(y, y_ref, "%s %s" % (wl.name, fmt))


@pytest.mark.parametrize("name,fmt,path", [("prefill_shared", "int4", "auto"),
                                           ("prefill_skewed", "int4", "auto"),
                                           ("prefill_skewed", "mxfp4", "auto"),
                                           ("decode", "int4", "auto"), ("decode", "mxfp4", "auto"),
                                           ("decode_batch", "int4", "gemv")])
def test_layer_full_size_tiled(name, fmt, path):
    wl = S.WORKLOADS[name]
    say("full-size tiled layer %s %s path %s (%s)" % (name, fmt, path, wl.description))
    inp = S.make_layer_inputs(wl, seed=0, fmt=fmt)
    d = DeviceLayer(inp).tiled()
    L = _oracle_logits(inp)
    rows = _rows(wl)
    y, idx, w, _ = run_layer(d, logits=L, path=PATHS[path])
    idx_ref, w_ref, _ = oracle.router_topk(L, wl.k)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, name)
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate, rows=rows,
                               fmt=fmt)
    sel = slice(None) if rows is None else rows
    assert_y_close(y[sel], y_ref, name + " tiled " + fmt)
