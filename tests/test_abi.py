"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before enqueuing
anything (no HIP call is reached by these cases)."""
import ctypes
import os
import re

import pytest

import quantized_expert_mlp_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return moe.lib()


def test_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert set(declared) == set(moe.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    assert moe.status_string(moe.MOE_OK) == "ok"
    assert moe.status_string(moe.MOE_ERR_WORKSPACE) == "workspace too small"
    assert moe.status_string(99) == "unknown status"


def _shape(**kw):
    base = dict(T=4, H=256, E=8, k=2, I=128, SI=0)
    base.update(kw)
    return moe.make_shape(**base)


def test_workspace_bytes_valid_and_invalid(L):
    assert moe.moe_workspace_bytes(_shape()) > 0
    big = moe.moe_workspace_bytes(_shape(T=2048, H=6144, E=256, k=8, I=2048))
    # fp16 hidden rows for 16384 slots x 2048 plus the fp16 activation copy
    assert big >= 16384 * 2048 * 2 + 2048 * 6144 * 2
    for bad in [dict(T=0), dict(k=9), dict(E=300, k=2), dict(k=65, E=128), dict(H=100),
                dict(I=96), dict(SI=32), dict(group=64)]:
        assert moe.moe_workspace_bytes(_shape(**bad)) == 0, bad
    assert moe.moe_workspace_bytes(_shape(path=3)) == 0
    # router variants in the shape: unknown score, misaligned bias, top-p with a variant
    assert moe.moe_workspace_bytes(_shape(score=moe.MOE_SCORE_SIGMOID)) > 0
    assert moe.moe_workspace_bytes(_shape(select_bias=FAKE)) > 0
    for bad in [dict(score=2), dict(select_bias=FAKE + 2), dict(score=1, top_p=0.5),
                dict(select_bias=FAKE, top_p=0.9)]:
        assert moe.moe_workspace_bytes(_shape(**bad)) == 0, bad


FAKE = 1 << 20  # a non-null, 256-aligned address; never dereferenced by these cases


def test_router_topk_rejects(L):
    f = L.moe_router_topk
    assert f(None, 4, 8, 2, 1.0, 0.0, 0, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 0, 8, 2, 1.0, 0.0, 0, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 8, 9, 1.0, 0.0, 0, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 8, 0, 1.0, 0.0, 0, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE + 2, 4, 8, 2, 1.0, 0.0, 0, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 257, 2, 1.0, 0.0, 0, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(FAKE, 4, 256, 65, 1.0, 0.7, 0, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    # router variants: unknown score, misaligned bias, top-p with a variant
    assert f(FAKE, 4, 8, 2, 1.0, 0.0, 2, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 8, 2, 1.0, 0.0, -1, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 8, 2, 1.0, 0.0, 0, FAKE + 2, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 8, 2, 1.0, 0.5, 1, None, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert f(FAKE, 4, 8, 2, 1.0, 0.5, 0, FAKE, 0, 0, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    # grouped routing: E % n_group, topk_group range, enough kept experts,
    # at most 16 groups, no top-p
    G = lambda ng, tg, k=2, E=8, p=0.0: f(FAKE, 4, E, k, 1.0, p, 1, None, ng, tg, FAKE, FAKE, None)
    assert G(3, 1) == moe.MOE_ERR_INVALID_ARG                       # 8 % 3
    assert G(4, 0) == moe.MOE_ERR_INVALID_ARG
    assert G(4, 5) == moe.MOE_ERR_INVALID_ARG
    assert G(4, 1, k=3) == moe.MOE_ERR_INVALID_ARG                  # one group of 2 < k
    assert G(-1, 0) == moe.MOE_ERR_INVALID_ARG
    assert G(32, 4, E=64) == moe.MOE_ERR_UNSUPPORTED
    assert G(4, 2, p=0.5) == moe.MOE_ERR_UNSUPPORTED
    assert moe.moe_workspace_bytes(_shape(n_group=4, topk_group=2)) > 0
    assert moe.moe_workspace_bytes(_shape(n_group=3, topk_group=1)) == 0
    assert moe.moe_workspace_bytes(_shape(n_group=4, topk_group=1, k=4)) == 0


def test_permute_rejects(L):
    f = L.moe_permute
    assert f(None, 4, 2, 8, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 2, 8, None, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 0, 2, 8, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 4, 2, 257, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_UNSUPPORTED
    # above 4096 slots the multi-workgroup permutation needs its scratch
    need = moe.moe_permute_workspace_bytes(2048, 8, 256)
    assert need == 4 * 16 * 256
    assert f(FAKE, 2048, 8, 256, FAKE, FAKE, FAKE, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert f(FAKE, 2048, 8, 256, FAKE, FAKE, FAKE, FAKE, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert f(FAKE, 2048, 8, 256, FAKE, FAKE, FAKE, FAKE + 64, need, None) == \
        moe.MOE_ERR_INVALID_ARG                                          # misaligned scratch


def test_permute_workspace_bytes(L):
    assert moe.moe_permute_workspace_bytes(512, 8, 256) == 0            # 4096 slots: one workgroup
    assert moe.moe_permute_workspace_bytes(513, 8, 256) == 4 * 5 * 256
    assert moe.moe_permute_workspace_bytes(700, 8, 32) == 4 * 6 * 32
    for bad in [(0, 8, 256), (4, 0, 8), (4, 2, 0), (4, 2, 257)]:
        assert moe.moe_permute_workspace_bytes(*bad) == 0, bad


def _q(ok=True):
    return moe.moe_q4(FAKE if ok else FAKE + 8, FAKE)


def test_layer_rejects(L):
    sh = _shape()
    ws_need = moe.moe_workspace_bytes(sh)

    def call(shape=sh, x=FAKE, logits=FAKE, w_router=None, gate=None, shared=None, sg=None,
             y=FAKE, ws=FAKE, ws_bytes=ws_need):
        gate = gate or _q()
        return L.moe_layer(ctypes.byref(shape), x, logits, w_router, gate, _q(), _q(), shared, sg,
                           y, None, None, None, ws, ws_bytes, None)

    assert call(logits=None) == moe.MOE_ERR_INVALID_ARG            # neither logits nor router
    assert call(w_router=FAKE) == moe.MOE_ERR_INVALID_ARG          # both
    assert call(x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(x=FAKE + 2) == moe.MOE_ERR_INVALID_ARG             # misaligned activations
    assert call(gate=_q(False)) == moe.MOE_ERR_INVALID_ARG          # misaligned plane
    assert call(ws=FAKE + 64) == moe.MOE_ERR_INVALID_ARG            # misaligned workspace
    assert call(y=FAKE + 4) == moe.MOE_ERR_INVALID_ARG              # y cleared with 16-byte stores
    assert call(y=FAKE + 8, shape=_shape(path=moe.MOE_PATH_GEMV)) == moe.MOE_ERR_INVALID_ARG
    assert call(ws_bytes=ws_need - 1) == moe.MOE_ERR_WORKSPACE
    assert call(shape=_shape(SI=64)) == moe.MOE_ERR_INVALID_ARG     # SI without shared planes
    assert call(shape=_shape(E=512, k=2)) == moe.MOE_ERR_UNSUPPORTED
    assert call(shape=_shape(H=96)) == moe.MOE_ERR_UNSUPPORTED
    assert call(shape=_shape(k=0)) == moe.MOE_ERR_INVALID_ARG


def test_residual_rmsnorm_rejects(L):
    sh = _shape()
    need = moe.moe_workspace_bytes(sh)
    f = L.moe_layer_residual_rmsnorm

    def call(residual=FAKE, norm_w=FAKE, eps=1e-6, x_next=FAKE, shape=sh, nwr=None, nE=0,
             nlog=None):
        return f(ctypes.byref(shape), FAKE, FAKE, None, _q(), _q(), _q(), None, None, residual,
                 norm_w, eps, x_next, nwr, nE, nlog, None, None, FAKE, need, None)

    assert call(residual=None) == moe.MOE_ERR_INVALID_ARG
    assert call(norm_w=None) == moe.MOE_ERR_INVALID_ARG
    assert call(x_next=None) == moe.MOE_ERR_INVALID_ARG
    assert call(residual=FAKE + 4) == moe.MOE_ERR_INVALID_ARG       # misaligned
    assert call(x_next=FAKE + 2) == moe.MOE_ERR_INVALID_ARG
    assert call(eps=-1.0) == moe.MOE_ERR_INVALID_ARG
    assert call(eps=float("nan")) == moe.MOE_ERR_INVALID_ARG
    assert call(shape=_shape(H=96)) == moe.MOE_ERR_UNSUPPORTED
    # the next layer's router: both buffers or neither, next_E >= 1, aligned
    assert call(nwr=FAKE, nE=8) == moe.MOE_ERR_INVALID_ARG          # no logits buffer
    assert call(nlog=FAKE, nE=8) == moe.MOE_ERR_INVALID_ARG         # no router plane
    assert call(nwr=FAKE, nE=0, nlog=FAKE) == moe.MOE_ERR_INVALID_ARG
    assert call(nwr=FAKE + 4, nE=8, nlog=FAKE) == moe.MOE_ERR_INVALID_ARG
    assert call(nwr=FAKE, nE=8, nlog=FAKE + 2) == moe.MOE_ERR_INVALID_ARG


def test_expert_mlp_rejects(L):
    sh = _shape()
    need = moe.moe_workspace_bytes(sh)
    f = L.moe_expert_mlp
    args = lambda **kw: [ctypes.byref(kw.get("shape", sh)), kw.get("x", FAKE), FAKE, FAKE, FAKE,
                         _q(), _q(), _q(), kw.get("y", FAKE), FAKE, kw.get("ws_bytes", need), None]
    assert f(*args(x=None)) == moe.MOE_ERR_INVALID_ARG
    assert f(*args(y=None)) == moe.MOE_ERR_INVALID_ARG
    assert f(*args(y=FAKE + 4)) == moe.MOE_ERR_INVALID_ARG
    assert f(*args(ws_bytes=0)) == moe.MOE_ERR_WORKSPACE
    assert f(*args(shape=_shape(path=moe.MOE_PATH_GEMV, H=16384))) == moe.MOE_ERR_UNSUPPORTED


def test_tiled_layout_shape_rules(L):
    tiled = dict(layout=moe.MOE_LAYOUT_TILED)
    assert moe.moe_workspace_bytes(_shape(**tiled)) > 0
    assert moe.moe_workspace_bytes(_shape(path=moe.MOE_PATH_GEMM, **tiled)) > 0
    assert moe.moe_workspace_bytes(_shape(path=moe.MOE_PATH_GEMV, **tiled)) > 0
    assert moe.moe_workspace_bytes(_shape(layout=2)) == 0
    # AUTO on tiled planes: the GEMV for up to four tokens (no fp16 activation
    # copy in its workspace), the MFMA GEMM beyond
    for T, path in ((1, moe.MOE_PATH_GEMV), (4, moe.MOE_PATH_GEMV), (5, moe.MOE_PATH_GEMM),
                    (2048, moe.MOE_PATH_GEMM)):
        dims = dict(T=T, H=6144, E=256, k=8, I=2048, **tiled)
        assert moe.moe_workspace_bytes(_shape(**dims)) == \
            moe.moe_workspace_bytes(_shape(path=path, **dims)), T
    # the tiled GEMV holds the token's prepared row in 48 KB of LDS (80 bytes
    # per 32 inputs): K <= 19648; beyond it AUTO takes the MFMA GEMM and an
    # explicit GEMV is refused
    for H, gemv in ((19648, True), (19712, False)):
        dims = dict(T=1, H=H, E=16, k=2, I=128, **tiled)
        ws_gemv = moe.moe_workspace_bytes(_shape(path=moe.MOE_PATH_GEMV, **dims))
        assert (ws_gemv > 0) == gemv, H
        want = ws_gemv if gemv else moe.moe_workspace_bytes(_shape(path=moe.MOE_PATH_GEMM, **dims))
        assert moe.moe_workspace_bytes(_shape(**dims)) == want, H


def test_mxfp4_format_shape_rules(L):
    mx = dict(format=moe.MOE_FORMAT_MXFP4)
    assert moe.moe_workspace_bytes(_shape(**mx)) > 0                        # AUTO -> MFMA path
    assert moe.moe_workspace_bytes(_shape(path=moe.MOE_PATH_GEMM, **mx)) > 0
    assert moe.moe_workspace_bytes(_shape(path=moe.MOE_PATH_GEMV, **mx)) > 0
    assert moe.moe_workspace_bytes(_shape(layout=moe.MOE_LAYOUT_TILED, **mx)) > 0
    assert moe.moe_workspace_bytes(_shape(layout=moe.MOE_LAYOUT_TILED, path=moe.MOE_PATH_GEMV,
                                          **mx)) > 0
    assert moe.moe_workspace_bytes(_shape(format=2)) == 0
    assert moe.moe_workspace_bytes(_shape(format=-1)) == 0
    # the AUTO rule does not depend on the format: decode takes the GEMV path
    # (no fp16 activation copy in its workspace), prefill the MFMA path
    for dims in (dict(T=1, H=6144, E=256, k=8, I=2048), dict(T=2048, H=6144, E=256, k=8, I=2048)):
        assert moe.moe_workspace_bytes(_shape(**dims, **mx)) == moe.moe_workspace_bytes(_shape(**dims))
    dec = dict(T=1, H=6144, E=256, k=8, I=2048)
    assert moe.moe_workspace_bytes(_shape(path=moe.MOE_PATH_GEMM, **dec, **mx)) > \
        moe.moe_workspace_bytes(_shape(**dec, **mx))


def test_pack_weights_rejects(L):
    f = L.moe_pack_weights
    src = moe.moe_q4(FAKE, FAKE + (1 << 24))
    dst = moe.moe_q4(FAKE + (2 << 24), FAKE + (3 << 24))
    I4, MX = moe.MOE_FORMAT_INT4, moe.MOE_FORMAT_MXFP4
    assert f(moe.moe_q4(None, FAKE), 2, 64, 128, I4, dst, None) == moe.MOE_ERR_INVALID_ARG
    assert f(src, 2, 64, 128, I4, moe.moe_q4(FAKE + 8, FAKE), None) == moe.MOE_ERR_INVALID_ARG
    assert f(src, 0, 64, 128, I4, dst, None) == moe.MOE_ERR_INVALID_ARG    # E
    assert f(src, 2, 48, 128, I4, dst, None) == moe.MOE_ERR_INVALID_ARG    # N % 32
    assert f(src, 2, 64, 96, I4, dst, None) == moe.MOE_ERR_INVALID_ARG     # K % 64
    assert f(src, 2, 64, 128, 2, dst, None) == moe.MOE_ERR_INVALID_ARG     # format
    assert f(src, 2, 64, 128, MX, src, None) == moe.MOE_ERR_INVALID_ARG    # in place
    assert f(src, 2, 64, 128, I4, moe.moe_q4(FAKE + 64, FAKE + (3 << 24)), None) == \
        moe.MOE_ERR_INVALID_ARG                                        # overlapping q
    # scales overlap by their byte size: 2*64*4 fp16 scales = 1 KiB, ue8m0 = 512 B
    near = moe.moe_q4(FAKE + (2 << 24), FAKE + (1 << 24) + 768)
    assert f(src, 2, 64, 128, I4, near, None) == moe.MOE_ERR_INVALID_ARG


def test_debug_dequant_rejects(L):
    f = L.moe_debug_dequant_int4
    assert f(_q(), 4, 48, 0, FAKE, None) == moe.MOE_ERR_INVALID_ARG   # K % 32
    assert f(_q(), 4, 64, 4, FAKE, None) == moe.MOE_ERR_INVALID_ARG   # mode
    assert f(_q(), 4, 64, -1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(_q(), 0, 64, 0, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(_q(False), 4, 64, 0, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    g = L.moe_debug_dequant_mxfp4
    assert g(_q(), 4, 48, 0, FAKE, None) == moe.MOE_ERR_INVALID_ARG   # K % 32
    assert g(_q(), 4, 64, 3, FAKE, None) == moe.MOE_ERR_INVALID_ARG   # mode
    assert g(_q(), 0, 64, 1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert g(_q(False), 4, 64, 1, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert g(_q(), 4, 64, 1, None, None) == moe.MOE_ERR_INVALID_ARG


def test_read_probe_rejects(L):
    f = L.moe_debug_read_probe
    assert f(None, 1024, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 1000, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG     # bytes % 16
    assert f(FAKE + 8, 1024, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG  # misaligned
    assert f(FAKE, 1024, 0, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert f(FAKE, 1024, 64, None, None) == moe.MOE_ERR_INVALID_ARG


def test_product_path_has_no_oracle_dependency():
    """The product package neither imports nor links the oracle."""
    pkg = os.path.join(ROOT, "quantized_expert_mlp_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.replace("oracle-free", ""), fn
