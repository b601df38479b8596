"""GPU tests of MXFP4 expert weights (e2m1 nibbles, one ue8m0 exponent per 32
inputs): the MFMA decoders at the ends of the exponent range (their bit-exact
pins over every exponent are in test_gpu_decoders.py), and the whole layer on
MXFP4 planes against the CPU oracle at mid sizes on both expert paths and at
every full workload size."""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import DeviceLayer, assert_w_close, assert_y_close, dev, host, run_layer, say
from test_gpu_parity import MID, _oracle_logits, _rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _decode(q, s, mode):
    N, K = q.shape[0], q.shape[1] * 2
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_debug_dequant_mxfp4((dev(q), dev(s)), N, K, out, mode=mode)
    torch.cuda.synchronize()
    return host(out)


def test_debug_dequant_mxfp4_scale_range_ends():
    """For e <= 99 every weight, |e2m1| * 2^(e - 127) <= 6 * 2^-28, rounds to a
    signed zero in fp16 (the MFMA decoders' scale is zero there); e = 255 is
    NaN (the MX format's NaN scale) for every element of its group."""
    rng = np.random.default_rng(5)
    N, K = 4, 128
    q = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = np.array([[0, 1, 50, 99]] * N, dtype=np.uint8)
    s[3, 2] = 255
    ref = oracle.dequant(q, s, "mxfp4")
    nan = np.isnan(ref)
    assert nan[3, 64:96].all() and nan.sum() == 32
    want = ref.astype(np.float16).astype(np.float32)
    for mode in (1, 2):
        got = _decode(q, s, mode)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
        assert np.all(got[~nan] == 0.0)


@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
@pytest.mark.parametrize("wl", MID, ids=[w.name for w in MID])
def test_layer_mid_mxfp4(wl, path):
    say("mxfp4 layer %s path=%d" % (wl.name, path))
    inp = S.make_layer_inputs(wl, seed=0, fmt="mxfp4")
    d = DeviceLayer(inp)
    L = _oracle_logits(inp)
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                         route_scale=0.75, fmt="mxfp4")
    y, idx, w, _ = run_layer(d, logits=L, path=path, route_scale=0.75)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, wl.name)
    assert_y_close(y, y_ref, "%s mxfp4" % wl.name)


@pytest.mark.parametrize("name", list(S.WORKLOADS))
def test_layer_full_size_mxfp4(name):
    wl = S.WORKLOADS[name]
    say("full-size mxfp4 layer %s (%s)" % (name, wl.description))
    inp = S.make_layer_inputs(wl, seed=0, fmt="mxfp4")
    d = DeviceLayer(inp)
    L = _oracle_logits(inp)
    rows = _rows(wl)
    y, idx, w, _ = run_layer(d, logits=L)
    idx_ref, w_ref, _ = oracle.router_topk(L, wl.k)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, name)
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate, rows=rows,
                               fmt="mxfp4")
    sel = slice(None) if rows is None else rows
    assert_y_close(y[sel], y_ref, name + " mxfp4")


@pytest.mark.parametrize("name", ["decode", "decode_batch"])
def test_layer_full_size_mxfp4_mfma_path(name):
    """The decode sizes through the MFMA path as well (AUTO takes the GEMV)."""
    wl = S.WORKLOADS[name]
    say("full-size mxfp4 layer %s on the MFMA path" % name)
    inp = S.make_layer_inputs(wl, seed=1, fmt="mxfp4")
    d = DeviceLayer(inp)
    L = _oracle_logits(inp)
    y, idx, w, _ = run_layer(d, logits=L, path=moe.MOE_PATH_GEMM)
    y_ref, idx_ref, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                     fmt="mxfp4")
    assert np.array_equal(idx, idx_ref)
    assert_y_close(y, y_ref, name + " mxfp4 mfma")
