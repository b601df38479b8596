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
from test_gpu_parity import MID, _mid, _oracle_logits, _rows

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
    """Rows mixing exponents 0, 1, 50 and 99 with a NaN group (e = 255): the
    row's shift follows its largest finite exponent (99), so that group is
    exact, the groups 38 or more below it are zeros, and the NaN group is NaN
    for every element."""
    from test_gpu_decoders import _mx_mfma_expected
    rng = np.random.default_rng(5)
    N, K = 4, 128
    q = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    s = np.array([[0, 1, 50, 99]] * N, dtype=np.uint8)
    s[3, 2] = 255
    ref = oracle.dequant(q, s, "mxfp4")
    nan = np.isnan(ref)
    assert nan[3, 64:96].all() and nan.sum() == 32
    want = _mx_mfma_expected(q, s)
    assert np.array_equal(want[:, 96:], ref[:, 96:].astype(np.float32))
    for mode in (1, 2):
        got = _decode(q, s, mode)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], want[~nan])


MX_RANGE = _mid("mx_range", 37, 96, 512, 8, 2, 256)


def _shifted_exponent_inputs(case):
    """The layer with exponents outside fp16's window 103..142 where its
    values stay finite: "small_down" - every down plane at e = 88..92 (its
    weights below 2^-32; the layer output near 1e-9); "large_gate_up" - the
    first group of every gate/up row at e = 141 (codes +-6 reach 98304, past
    fp16) with the inputs it reads scaled by 2^-13, the other groups at
    119..122."""
    inp = S.make_layer_inputs(MX_RANGE, seed=0, fmt="mxfp4")
    rng = np.random.default_rng([37, len(case)])
    if case == "small_down":
        q, sc = inp.planes["down"]
        inp.planes["down"] = (q, rng.integers(88, 93, sc.shape).astype(np.uint8))
    else:
        for p in ("gate", "up"):
            q, sc = inp.planes[p]
            sc = sc.copy()
            sc[:, :, 0] = 141
            inp.planes[p] = (q, sc)
        x = S.bf16_bits_to_f32(inp.x).copy()
        x[:, :32] *= 2.0 ** -13
        inp.x = S.f32_to_bf16_bits(x)
    return inp


@pytest.mark.parametrize("layout", ["rows", "tiled"])
@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
@pytest.mark.parametrize("case", ["small_down", "large_gate_up"])
def test_layer_mxfp4_exponents_outside_fp16_window(case, path, layout):
    say("mxfp4 exponents outside the fp16 window: %s path=%d %s" % (case, path, layout))
    inp = _shifted_exponent_inputs(case)
    d = DeviceLayer(inp)
    if layout == "tiled":
        d = d.tiled()
    y_ref, idx_ref, _ = oracle.layer(inp.x, inp.logits, MX_RANGE.k, inp.planes, fmt="mxfp4")
    assert np.all(np.isfinite(y_ref))
    y, idx, _, _ = run_layer(d, path=path)
    assert np.array_equal(idx, idx_ref)
    assert_y_close(y, y_ref, "mxfp4 %s path %d %s" % (case, path, layout))


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
