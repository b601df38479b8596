"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Every input is seeded and synthetic (moe_synth); every expected value comes
from the oracle.  Small and mid-size cases are checked in full, spanning
several tiles with ragged tails; the five full-size workloads run in the
launch configuration the benchmark times, with y checked on sampled token rows
(rows are independent) and the router/permutation outputs on every row.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import (Canaried, DeviceLayer, assert_w_close, assert_y_close, dev, host,
                         logits_bound, run_layer, say, valid_topk)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    oracle.lib()
    oracle.set_threads(16)


# ---------------------------------------------------------------- router --

TOPK_CASES = [(4, 8, 2), (1, 256, 8), (32, 128, 8), (512, 60, 4), (2048, 256, 8), (7, 1, 1),
              (5, 64, 64), (9, 256, 64), (33, 200, 17), (300, 65, 3)]


@pytest.mark.parametrize("T,E,k", TOPK_CASES)
def test_router_topk(T, E, k):
    say("topk T=%d E=%d k=%d" % (T, E, k))
    rng = np.random.default_rng(T * 1000 + E * 10 + k)
    L = rng.standard_normal((T, E)).astype(np.float32) * 2
    L[::3] = rng.integers(0, 3, size=L[::3].shape).astype(np.float32)  # forced ties
    if T > 1:
        L[1] = 0.0
        L[1, ::2] = -0.0
    idx_ref, w_ref, _ = oracle.router_topk(L, k, 1.25)
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(dev(L), T, E, k, 1.25, idx, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(idx), idx_ref)
    assert_w_close(host(w), w_ref, "topk T=%d E=%d k=%d" % (T, E, k))


# ----------------------------------------------------------- permutation --

def _permute_dev(idx, E):
    """moe_permute through the C ABI with canaried outputs and, above 4096
    slots, its scratch (the multi-workgroup path)."""
    T, k = idx.shape
    off = Canaried((E + 1,), torch.int32, -5, "off")
    srt = Canaried((T * k,), torch.int32, -5, "sorted")
    row = Canaried((T * k,), torch.int32, -5, "row_of")
    nb = moe.moe_permute_workspace_bytes(T, k, E)
    ws = Canaried((max(nb, 4),), torch.uint8, 0xEE, "permute scratch")
    moe.moe_permute(dev(idx), T, k, E, off.view, srt.view, row.view, ws.view if nb else None, nb)
    torch.cuda.synchronize()
    for c in (off, srt, row, ws):
        c.check()
    return host(off.view), host(srt.view), host(row.view), nb


@pytest.mark.parametrize("T,k,E", [(4, 2, 8), (1, 8, 256), (32, 8, 128), (512, 4, 60),
                                   (2048, 8, 256), (1500, 3, 7), (37, 1, 256), (700, 8, 32)])
def test_permute(T, k, E):
    """Bit-exact against the oracle; 2048 x 8 (16384 slots), 1500 x 3 and
    700 x 8 run the multi-workgroup path with the caller's scratch."""
    say("permute T=%d k=%d E=%d" % (T, k, E))
    rng = np.random.default_rng(T + 31 * k + E)
    if E >= k:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    else:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
    off_r, srt_r, row_r = oracle.permute(idx, E)
    off, srt, row, nb = _permute_dev(idx, E)
    assert (nb > 0) == (T * k > 4096)
    assert np.array_equal(off, off_r)
    assert np.array_equal(srt, srt_r)
    assert np.array_equal(row, row_r)


@pytest.mark.parametrize("T,k,E", [(300, 4, 16), (2048, 8, 256)])
def test_permute_drops_out_of_range_picks(T, k, E):
    """Picks outside [0, E) (top-p's -1, or past the experts) against the
    oracle's dropped-pick rule, on the one-workgroup and the multi-workgroup
    permutation: off bit-exact, the valid slots' rows bit-exact, row_of -1 for
    the dropped ones."""
    rng = np.random.default_rng(5)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.1
    idx[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    off_r, srt_r, row_r = oracle.permute(idx, E)
    off, srt, row, _ = _permute_dev(idx, E)
    nval = int(off_r[E])
    assert nval < T * k
    assert np.array_equal(off, off_r)
    assert np.array_equal(srt[:nval], srt_r[:nval])
    assert np.all(srt[nval:] == -5)  # nothing written past the valid slots
    assert np.array_equal(row, row_r)


# ------------------------------------------------------------ whole layer --

def _mid(name, wid, T, H, E, k, I, SI=0, logits="given"):
    return S.Workload(name, wid, T, H, E, k, I, SI, logits, name)


MID = [
    # several GEMM row tiles with ragged tails, ragged column blocks (I = 192)
    _mid("mid_ragged", 20, 300, 512, 16, 4, 192),
    # shared expert with a gate vector, router-computed logits
    _mid("mid_shared", 21, 200, 256, 12, 2, 128, 320, "router"),
    # k = 1, E = 1 degenerate (every token to expert 0)
    _mid("mid_one_expert", 22, 70, 256, 1, 1, 64),
    # k = E: dense mixture over every expert
    _mid("mid_dense", 23, 40, 128, 6, 6, 64),
    # single token through the decode GEMV with long rows and short down rows
    _mid("mid_decode", 24, 3, 4096, 64, 8, 320),
    # 5600 slots: the permutation over many workgroups, a ragged last block
    _mid("mid_many_slots", 26, 700, 256, 32, 8, 128),
    # the largest router served: E = 256, k = 64 (1280 slots, most experts touched)
    _mid("mid_max_k", 27, 20, 256, 256, 64, 128),
    # one token with k = 64: the GEMV's fused routing at its 64-slot limit
    _mid("mid_one_token_max_k", 28, 1, 512, 256, 64, 192),
    # the widest rows the GEMV serves (256 scale groups, four per lane) on
    # both gate/up (K = H) and down (K = I)
    _mid("mid_widest_rows", 29, 2, 8192, 2, 1, 8192),
]


def _oracle_logits(inp):
    if inp.logits is not None:
        return inp.logits
    return oracle.router_logits(inp.x, inp.w_router)


@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
@pytest.mark.parametrize("wl", MID, ids=[w.name for w in MID])
def test_layer_mid(wl, path):
    say("layer %s path=%d" % (wl.name, path))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    L = _oracle_logits(inp)
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate,
                                         route_scale=0.75)
    y, idx, w, lo = run_layer(d, logits=L, path=path, route_scale=0.75)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, wl.name)
    assert np.array_equal(lo, L)
    assert_y_close(y, y_ref, "%s path %d" % (wl.name, path))


@pytest.mark.parametrize("k", [8, 64])
@pytest.mark.parametrize("kind", ["integers", "signed_zeros"])
def test_layer_one_token_ties(kind, k):
    """One token through the GEMV's fused routing (each workgroup runs only
    the arg-max rounds its pick needs, every wave on its own) with logits
    full of exact ties: picks bit-exact (the lower index wins), weights and
    y against the oracle."""
    wl = _mid("one_token_ties_k%d" % k, 45, 1, 2048, 256, k, 1536)
    say("one-token ties %s k=%d" % (kind, k))
    inp = S.make_layer_inputs(wl, seed=11)
    d = DeviceLayer(inp)
    rng = np.random.default_rng([k, 45])
    if kind == "integers":
        L = rng.integers(0, 3, size=(1, wl.E)).astype(np.float32)
    else:  # zeros of both signs, a few larger logits spread among them
        L = np.where(rng.random((1, wl.E)) < 0.5, np.float32(-0.0), np.float32(0.0))
        L[0, rng.choice(wl.E, k // 2, replace=False)] = 1.0
    y_ref, idx_ref, w_ref = oracle.layer(inp.x, L, wl.k, inp.planes)
    y, idx, w, _ = run_layer(d, logits=L, path=moe.MOE_PATH_GEMV)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, wl.name)
    assert_y_close(y, y_ref, wl.name)


def test_expert_mlp_direct():
    wl = _mid("mlp_direct", 25, 150, 256, 10, 3, 192)
    say("expert_mlp %s" % wl.name)
    inp = S.make_layer_inputs(wl)
    idx, w, _ = oracle.router_topk(inp.logits, wl.k)
    off, srt, _ = oracle.permute(idx, wl.E)
    y_ref, _, _ = oracle.layer(inp.x, inp.logits, wl.k, inp.planes)
    d = DeviceLayer(inp)
    for path in (moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM):
        sh = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I, path=path)
        nb = moe.moe_workspace_bytes(sh)
        ws = torch.full((nb,), 0xEE, dtype=torch.uint8, device="cuda")
        y = torch.full((wl.T, wl.H), float("nan"), device="cuda")
        moe.moe_expert_mlp(sh, d.x, dev(off), dev(srt), dev(w), d.planes["gate"], d.planes["up"],
                           d.planes["down"], y, ws, nb)
        torch.cuda.synchronize()
        assert_y_close(host(y), y_ref, "expert_mlp path %d" % path)


def test_expert_mlp_repeated_picks():
    """moe_expert_mlp on buckets a router never makes: every token picks
    expert 0 three times, so its bucket holds 60 rows at T = 20, more rows
    than tokens (two MFMA subtiles; the GEMV takes a token per row).  y
    against the oracle's expert rows weighted and summed per pick."""
    wl = _mid("mlp_repeats", 39, 20, 256, 4, 4, 192)
    say("expert_mlp with repeated picks")
    inp = S.make_layer_inputs(wl)
    rng = np.random.default_rng(39)
    idx = np.tile(np.array([0, 2, 0, 0], np.int32), (wl.T, 1))
    idx[:, 1] = rng.integers(1, wl.E, wl.T)
    w = rng.uniform(0.1, 1.0, idx.shape).astype(np.float32)
    off, srt, _ = oracle.permute(idx, wl.E)
    assert off[1] - off[0] == 3 * wl.T
    x64 = S.bf16_bits_to_f32(inp.x).astype(np.float64)
    pl = inp.planes
    y_ref = np.zeros((wl.T, wl.H))
    for t in range(wl.T):
        for j in range(wl.k):
            e = idx[t, j]
            _, o = oracle.expert_forward((pl["gate"][0][e], pl["gate"][1][e]),
                                         (pl["up"][0][e], pl["up"][1][e]),
                                         (pl["down"][0][e], pl["down"][1][e]), x64[t])
            y_ref[t] += float(w[t, j]) * o
    d = DeviceLayer(inp)
    for path in (moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM):
        sh = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I, path=path)
        nb = moe.moe_workspace_bytes(sh)
        ws = torch.full((nb,), 0xEE, dtype=torch.uint8, device="cuda")
        y = torch.full((wl.T, wl.H), float("nan"), device="cuda")
        moe.moe_expert_mlp(sh, d.x, dev(off), dev(srt), dev(w), d.planes["gate"], d.planes["up"],
                           d.planes["down"], y, ws, nb)
        torch.cuda.synchronize()
        assert_y_close(host(y), y_ref, "expert_mlp repeated picks path %d" % path)


@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
def test_layer_large_activations(path):
    """Activations over fp16's range (x ~ N(0, 1500^2), one entry in a
    hundred at +-4e4..65280, the largest bf16 below fp16's overflow), with
    scales of 6.2e-5..9e-5 so that the hidden row stays an fp16 number (at
    most 2.7e4 here, over every expert and token): the
    MFMA path's fp16 copy of x is exact there and both paths stay within the
    bar of the oracle."""
    wl = _mid("mid_large_x", 33, 96, 512, 8, 2, 192)
    say("large activations path=%d" % path)
    inp = S.make_layer_inputs(wl, seed=0)
    rng = np.random.default_rng(33)
    x = rng.standard_normal((wl.T, wl.H)).astype(np.float32) * 1500
    big = rng.random((wl.T, wl.H)) < 0.01
    x[big] = (rng.choice([-1.0, 1.0], int(big.sum())) *
              rng.uniform(4e4, 65280.0, int(big.sum()))).astype(np.float32)
    inp.x = S.f32_to_bf16_bits(np.clip(x, -65280.0, 65280.0))
    assert np.abs(S.bf16_bits_to_f32(inp.x)).max() <= 65280.0
    for p in S.PLANES:
        q, s_ = inp.planes[p]
        s_ = (rng.uniform(6.2e-5, 9e-5, s_.shape)).astype(np.float16).view(np.uint16)
        inp.planes[p] = (q, s_)
    d = DeviceLayer(inp)
    y_ref, idx_ref, _ = oracle.layer(inp.x, inp.logits, wl.k, inp.planes)
    assert np.all(np.isfinite(y_ref))
    y, idx, _, _ = run_layer(d, path=path)
    assert np.array_equal(idx, idx_ref)
    assert_y_close(y, y_ref, "large activations path %d" % path)


# ------------------------------------------------- full-size workloads --

SAMPLE_ROWS = {"prefill_shared": 128, "prefill_skewed": 128}


def _rows(wl):
    n = SAMPLE_ROWS.get(wl.name)
    if n is None:
        return None
    rng = np.random.default_rng(99)
    pick = set(rng.choice(wl.T, n - 2, replace=False).tolist()) | {0, wl.T - 1}
    return sorted(pick)


@pytest.mark.parametrize("name", list(S.WORKLOADS))
def test_layer_full_size(name):
    wl = S.WORKLOADS[name]
    say("full-size layer %s (%s)" % (name, wl.description))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    L = _oracle_logits(inp)
    rows = _rows(wl)
    # given logits: indices bit-exact, weights 1e-6, y on (sampled) rows
    y, idx, w, _ = run_layer(d, logits=L)
    idx_ref, w_ref, _ = oracle.router_topk(L, wl.k)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, name)
    y_ref, _, _ = oracle.layer(inp.x, L, wl.k, inp.planes, inp.shared, inp.shared_gate, rows=rows)
    sel = slice(None) if rows is None else rows
    assert_y_close(y[sel], y_ref, name)

    if wl.logits == "router":
        # logits computed on the device: within the fp32 forward-error bound
        y2, idx2, w2, lo2 = run_layer(d, use_router=True)
        bound = logits_bound(inp.x, inp.w_router)
        assert np.all(np.abs(lo2.astype(np.float64) - L.astype(np.float64)) <= bound + 1e-30)
        ok = np.array([np.array_equal(idx2[t], idx_ref[t]) for t in range(wl.T)])
        for t in np.nonzero(~ok)[0]:
            assert valid_topk(idx2[t], L[t].astype(np.float64), bound[t], wl.k), t
        say("  router path: %d of %d rows pick a near-tie differently" % (int((~ok).sum()), wl.T))
        check = [r for r in (range(wl.T) if rows is None else rows) if ok[r]]
        pos = [i for i, r in enumerate(range(wl.T) if rows is None else rows) if ok[r]]
        assert_y_close(y2[check], y_ref[pos], name + " (router logits)")


# ------------------------------------------------ router-computed logits --

ROUTER_SHAPES = [
    # ragged 16-token tiles and the gate row of a shared expert as column E
    _mid("router_small_gated", 30, 37, 256, 12, 2, 128, 192, "router"),
    # three tokens: the GEMV's fused routing reading the computed logits
    _mid("router_tiny", 31, 3, 512, 16, 4, 128, 0, "router"),
    # several token tiles, a ragged last one
    _mid("router_tiles", 32, 70, 256, 12, 2, 128, 192, "router"),
]


@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
@pytest.mark.parametrize("wl", ROUTER_SHAPES, ids=[w.name for w in ROUTER_SHAPES])
def test_layer_router_logits(wl, path):
    """Logits computed on the device: within the fp32 forward-error bound of
    the fp64 oracle; the device's own fp32 logits then feed the oracle's
    top-k (indices bit-exact, weights 1e-6) and layer (y on every row), which
    also covers the fp16 activation copy the logits launch writes for the
    MFMA path and the shared gate's logit column."""
    say("router logits %s path=%d" % (wl.name, path))
    inp = S.make_layer_inputs(wl, seed=3)
    d = DeviceLayer(inp)
    y, idx, w, lo = run_layer(d, use_router=True, path=path)
    L = oracle.router_logits(inp.x, inp.w_router)
    bound = logits_bound(inp.x, inp.w_router)
    assert np.all(np.abs(lo.astype(np.float64) - L.astype(np.float64)) <= bound + 1e-30)
    idx_ref, w_ref, _ = oracle.router_topk(lo, wl.k)
    assert np.array_equal(idx, idx_ref)
    assert_w_close(w, w_ref, wl.name)
    y_ref, _, _ = oracle.layer(inp.x, lo, wl.k, inp.planes, inp.shared, inp.shared_gate)
    assert_y_close(y, y_ref, "%s path %d (router logits)" % (wl.name, path))


# ------------------------------------------------- profiled entry point --

@pytest.mark.parametrize("path", [moe.MOE_PATH_GEMV, moe.MOE_PATH_GEMM])
def test_layer_profiled_matches_layer(path):
    """moe_layer_profiled does the same work as moe_layer (same y, picks and
    weights) and leaves every stage with a finished, non-negative interval."""
    import ctypes
    wl = MID[1]  # shared expert with a gate vector, router-computed logits
    say("profiled layer %s path=%d" % (wl.name, path))
    inp = S.make_layer_inputs(wl, seed=0)
    d = DeviceLayer(inp)
    sh = moe.make_shape(wl.T, wl.H, wl.E, wl.k, wl.I, wl.SI, path=path)
    nb = moe.moe_workspace_bytes(sh)
    outs = []
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    events = []
    for _ in range(2 * len(moe.STAGES)):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        events.append(e.value)
    for profiled in (False, True):
        ws = torch.full((nb,), 0xAB, dtype=torch.uint8, device="cuda")
        y = torch.full((wl.T, wl.H), float("nan"), device="cuda")
        idx = torch.full((wl.T, wl.k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((wl.T, wl.k), float("nan"), device="cuda")
        args = (sh, d.x, None, d.w_router, d.planes["gate"], d.planes["up"], d.planes["down"],
                d.shared, d.shared_gate, y, idx, w, None, ws, nb)
        if profiled:
            ran = moe.moe_layer_profiled(*args, events=events)
            # 200 tokens: separate top-k and permutation launches; the MFMA
            # path's logits launch writes the fp16 activations and its
            # routed launches carry the shared expert's tiles
            want = ["logits", "topk", "permute", "gate_up", "down"]
            if path == moe.MOE_PATH_GEMV:
                want += ["shared_gate_up", "shared_down"]
            assert sorted(ran) == sorted(want), ran
        else:
            moe.moe_layer(*args)
        torch.cuda.synchronize()
        outs.append((host(y), host(idx), host(w)))
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][2].view(np.uint32), outs[1][2].view(np.uint32))
    # y: same kernels, but atomics add in no fixed order
    assert_y_close(outs[1][0], outs[0][0], "profiled vs plain")
    for i in range(len(moe.STAGES)):
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), events[2 * i], events[2 * i + 1]) == 0
        assert ms.value >= 0.0, moe.STAGES[i]
    for e in events:
        hip.hipEventDestroy(e)
