"""moe_layer_static (the layer on the library's static per-GPU scratch, for
callers that cannot allocate) against moe_layer through the C ABI: the same
picks and weights bit for bit and y within the layer's bar, on two calls in a
row, the second with a smaller input; a shape past the scratch is rejected
before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import moe_synth as S
import quantized_expert_mlp_amd as moe
from gpu_harness import Canaried, DeviceLayer, assert_y_close, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()


def _wl(name, wid, T, H, E, k, I, SI=0, logits="given"):
    return S.Workload(name, wid, T, H, E, k, I, SI, logits, name)


def _both(wl, path=moe.MOE_PATH_AUTO):
    """(moe_layer outputs, moe_layer_static outputs) for one seeded input."""
    inp = S.make_layer_inputs(wl, seed=1)
    d = DeviceLayer(inp)
    sh = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I, wl.SI, path=path)
    nb = moe.moe_workspace_bytes(sh)
    assert 0 < nb <= moe.MOE_STATIC_SCRATCH_BYTES
    outs = []
    for static in (False, True):
        y = Canaried((wl.T, wl.H), torch.float32, float("nan"), "y")
        idx = Canaried((wl.T, wl.k), torch.int32, -7, "idx")
        w = Canaried((wl.T, wl.k), torch.float32, float("nan"), "w")
        lg = d.logits
        wr = d.w_router if lg is None else None
        args = (sh, d.x, lg, wr, d.planes["gate"], d.planes["up"], d.planes["down"], d.shared,
                d.shared_gate, y.view, idx.view, w.view, None)
        if static:
            moe.moe_layer_static(*args)
        else:
            ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
            moe.moe_layer(*args, ws, nb)
        torch.cuda.synchronize()
        for c in (y, idx, w):
            c.check()
        outs.append((host(y.view), host(idx.view), host(w.view)))
    return outs


def _compare(wl, path=moe.MOE_PATH_AUTO):
    say("static scratch vs workspace: %s path=%d" % (wl.name, path))
    (y0, i0, w0), (y1, i1, w1) = _both(wl, path)
    assert np.array_equal(i0, i1)
    assert np.array_equal(w0.view(np.uint32), w1.view(np.uint32))
    # same kernels; the atomics add a token's terms in no fixed order
    assert_y_close(y1, y0, "%s static vs workspace" % wl.name)


def test_static_scratch_two_calls_second_smaller():
    # a prefill with a gated shared expert and router logits (MFMA path),
    # then a smaller decode batch on the same scratch (GEMV path)
    _compare(_wl("static_prefill", 40, 300, 512, 16, 4, 192, 256, "router"))
    _compare(_wl("static_small", 41, 5, 512, 16, 2, 128))


def test_static_scratch_full_prefill_shared_then_decode():
    # the largest benchmark workload the scratch serves, then the decode layer
    _compare(S.WORKLOADS["prefill_shared"])
    _compare(S.WORKLOADS["decode"])


def test_static_scratch_rejects_past_its_size():
    wl = S.WORKLOADS["prefill_skewed"]
    sh = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I)
    assert moe.moe_workspace_bytes(sh) > moe.MOE_STATIC_SCRATCH_BYTES
    L = moe.lib()
    z = ctypes.c_void_p(1 << 20)  # never dereferenced: the check comes first
    q = moe.moe_q4(z.value, z.value)
    rc = L.moe_layer_static(ctypes.byref(sh), z, z, None, q, q, q, None, None, z, None, None,
                            None, None)
    assert rc == moe.MOE_ERR_SCRATCH_LIMIT
    assert moe.status_string(rc) == "shape needs more than the static scratch"
