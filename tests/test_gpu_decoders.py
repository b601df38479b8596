"""Bit-exact pins of every 4-bit decoder the kernels run, through the C ABI's
debug hooks (which call the same __device__ routines as the kernels' main
loops), against the oracle's exact weights.

int4 (offset-binary nibble - 8, one fp16 scale per 32 inputs):
  mode 0  gate/up GEMV decoder (bf16 128 + n)   -> the exact weight
  mode 1  MFMA decoder, tiles of 2-4 subtiles    -> exact weight rounded to fp16
  mode 2  MFMA decoder, one-subtile tiles        -> the same, for |s| <= 8188
  mode 3  down GEMV decoder (fp16 1024 + n)      -> the exact weight
MXFP4 (e2m1 nibble, one ue8m0 exponent per 32 inputs):
  mode 0  GEMV decoder (packed fp4 conversion x fp32 2^(e-127)) -> exact weight
  mode 1  MFMA decoder, tiles of 2-4 subtiles    -> fp16 operand at the row's
          shift, undone: exact for groups within 36 of the row's largest
          exponent, then once-rounded, then zero
  mode 2  MFMA decoder, one-subtile tiles        -> the same

Coverage is exhaustive where it is cheap: every finite fp16 scale with every
nibble value in every element position class, every ue8m0 exponent with every
e2m1 code, plus random planes for the element order.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
import quantized_expert_mlp_amd as moe
from gpu_harness import dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    oracle.lib()


def _structured_nibbles(groups: int) -> np.ndarray:
    """Packed nibbles [groups][16] in which group g holds n_i = (7 i + g) % 16
    at element i: every nibble value twice per group, at positions that move
    with g (7 is prime to 16)."""
    i = np.arange(32)
    g = np.arange(groups)[:, None]
    n = ((7 * i[None, :] + g) % 16).astype(np.uint8)
    return (n[:, 0::2] | (n[:, 1::2] << 4)).astype(np.uint8)


def _finite_fp16_scales(limit=None) -> np.ndarray:
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    ok = np.isfinite(v)
    if limit is not None:
        ok &= np.abs(v.astype(np.float64)) <= limit
    return bits[ok]


def _int4(q, s, mode):
    N, K = q.shape[0], q.shape[1] * 2
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_debug_dequant_int4((dev(q), dev(s)), N, K, mode, out)
    torch.cuda.synchronize()
    return host(out)


def _mx(q, s, mode):
    N, K = q.shape[0], q.shape[1] * 2
    out = torch.full((N, K), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_debug_dequant_mxfp4((dev(q), dev(s)), N, K, out, mode=mode)
    torch.cuda.synchronize()
    return host(out)


def _bits_equal(got, want, what, signed_zero=True):
    """Bit-exact; with signed_zero=False a zero may carry either sign."""
    g, w = np.asarray(got, np.float32), np.asarray(want, np.float32)
    nan_g, nan_w = np.isnan(g), np.isnan(w)
    assert np.array_equal(nan_g, nan_w), "%s: NaN positions differ" % what
    g, w = g[~nan_w], w[~nan_w]
    same = g.view(np.uint32) == w.view(np.uint32)
    if not signed_zero:
        same |= (g == 0) & (w == 0)
    bad = np.nonzero(~same)[0]
    assert bad.size == 0, "%s: %d mismatches, first %r vs %r" % (what, bad.size, g[bad[0]], w[bad[0]])


# ------------------------------------------------------------------ int4 --

def _all_scales_plane():
    """One group per finite fp16 scale (63488 groups), two groups per row."""
    s = _finite_fp16_scales()
    if s.size % 2:
        s = np.concatenate([s, s[:1]])
    q = _structured_nibbles(s.size).reshape(s.size // 2, 32)
    return q, s.reshape(s.size // 2, 2)


def test_int4_gemv_decoders_exact_every_scale():
    """Modes 0 and 3: the GEMVs' offset forms, undone exactly, give the exact
    weight (n - 8) * s for every finite fp16 scale and every nibble."""
    q, s = _all_scales_plane()
    say("int4 GEMV decoders: %d scales x 16 nibbles" % s.size)
    want = oracle.dequant(q, s).astype(np.float32)  # exact: <= 15 significant bits
    for mode in (0, 3):
        _bits_equal(_int4(q, s, mode), want, "int4 mode %d" % mode)


def test_int4_mfma_decoders_every_scale():
    """Mode 1 rounds the exact weight once to fp16 for every finite scale
    (overflow to +-inf included); mode 2 gives the same value for every scale
    with |s| <= 8188 (where -8 s is an fp16 number)."""
    q, s = _all_scales_plane()
    with np.errstate(over="ignore"):
        want = oracle.dequant(q, s).astype(np.float16).astype(np.float32)
    _bits_equal(_int4(q, s, 1), want, "int4 mode 1")
    lim = _finite_fp16_scales(8188.0)
    q2 = _structured_nibbles(lim.size + lim.size % 2).reshape(-1, 32)
    s2 = np.concatenate([lim, lim[:lim.size % 2]]).reshape(-1, 2)
    want2 = oracle.dequant(q2, s2).astype(np.float16).astype(np.float32)
    say("int4 mode 2: %d scales with |s| <= 8188" % lim.size)
    # n * s + (-8 s) is an exact zero for n = 8, which IEEE addition gives as
    # +0 where (n - 8) * s is -0 for a negative scale
    _bits_equal(_int4(q2, s2, 2), want2, "int4 mode 2", signed_zero=False)


def test_int4_mfma_cvt_decoder_large_scale_edge():
    """The documented edge of mode 2: at s = 8192, -8 s overflows fp16, so the
    group's weights for n >= 1 are -inf (or NaN), where mode 1 stays finite
    for 1 <= n <= 15 with |n - 8| * 8192 <= 65504."""
    s = np.array([[np.float16(8192).view(np.uint16)] * 2], dtype=np.uint16)
    q = _structured_nibbles(2).reshape(1, 32)
    m1, m2 = _int4(q, s, 1), _int4(q, s, 2)
    n = np.concatenate([np.stack([b & 15, b >> 4], 1).ravel() for b in q[0].reshape(2, 16)])
    finite1 = np.isfinite(m1[0])
    assert np.all(finite1[(n >= 1)])
    assert np.all(~np.isfinite(m2[0][n >= 1]))


def test_int4_decoders_random_planes():
    """Element order on random planes of the workloads' scale distribution."""
    for N, K in [(8, 64), (64, 256), (3, 6144), (96, 1408)]:
        q, s = S.draw_plane(N, K, np.random.default_rng(N * 7 + K))
        ref = oracle.dequant(q, s)
        for mode in range(4):
            want = ref.astype(np.float32) if mode in (0, 3) else \
                ref.astype(np.float16).astype(np.float32)
            _bits_equal(_int4(q, s, mode), want, "random N=%d K=%d mode %d" % (N, K, mode),
                        signed_zero=mode != 2)


# ----------------------------------------------------------------- MXFP4 --

def _all_exponents_plane(lo=0, hi=255):
    """Rows of K = 64 with exponents e and e (every code twice per group)."""
    e = np.arange(lo, hi + 1).astype(np.uint8)
    q = _structured_nibbles(2 * e.size).reshape(e.size, 32)
    s = np.stack([e, e], axis=1)
    return q, s


def test_mxfp4_gemv_decoder_exact_every_exponent():
    """Mode 0: the exact weight e2m1 * 2^(e - 127) in fp32 for every exponent
    (NaN for e = 255; the largest codes overflow fp32 at e >= 254 on both
    sides)."""
    q, s = _all_exponents_plane()
    with np.errstate(over="ignore", invalid="ignore"):
        want = oracle.dequant(q, s, "mxfp4").astype(np.float32)
    _bits_equal(_mx(q, s, 0), want, "mxfp4 mode 0")


def _mx_mfma_expected(q, s):
    """What the MFMA decoders feed, undone: per row, shift = (largest finite
    exponent) - 140; a group with e - shift >= 103 is the exact weight scaled
    by 2^-shift rounded once to fp16, a group below that is a signed zero;
    times 2^shift in fp64 (exact), then fp32."""
    w = oracle.dequant(q, s, "mxfp4")
    emax = np.where(s != 255, s.astype(np.int64), -1).max(axis=1)
    shift = np.where(emax < 0, 0, emax - 140)
    eb = np.repeat(s.astype(np.int64) - shift[:, None], 32, axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        op = np.ldexp(w, -shift[:, None]).astype(np.float16).astype(np.float64)
        op = np.where((eb <= 102) & ~np.isnan(op), 0.0 * np.sign(w), op)
        return np.ldexp(op, shift[:, None]).astype(np.float32)


def test_mxfp4_mfma_decoders_every_exponent():
    """Modes 1 and 2 on rows of one exponent: the exact weight for every e
    (the row's shift puts its scale at the top of fp16's exact window), NaN
    for e = 255, and the largest codes overflowing fp32 at e >= 254 as the
    exact weights do."""
    q, s = _all_exponents_plane()
    with np.errstate(over="ignore", invalid="ignore"):
        want = oracle.dequant(q, s, "mxfp4").astype(np.float32)
    assert np.array_equal(_mx_mfma_expected(q, s).view(np.uint32), want.view(np.uint32))
    for mode in (1, 2):
        _bits_equal(_mx(q, s, mode), want, "mxfp4 mode %d" % mode)


def test_mxfp4_mfma_decoders_exponent_spans():
    """Rows whose groups span 0..60 binades below their largest exponent, at
    every position of that largest exponent: groups within 36 exact, 37
    below rounded once to the subnormal grid, further below zero."""
    rng = np.random.default_rng(44)
    N, K = 512, 256
    top = rng.integers(0, 255, N)
    s = np.clip(top[:, None] - rng.integers(0, 61, (N, K // 32)), 0, 254).astype(np.uint8)
    s[np.arange(N), rng.integers(0, K // 32, N)] = top  # the row's largest, somewhere
    s[::17, 3] = 255                                    # NaN groups beside finite ones
    q = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    want = _mx_mfma_expected(q, s)
    for mode in (1, 2):
        _bits_equal(_mx(q, s, mode), want, "mxfp4 spans mode %d" % mode, signed_zero=False)


def test_mxfp4_decoders_random_planes():
    for N, K in [(8, 64), (64, 256), (3, 6144), (96, 1408)]:
        rng = np.random.default_rng([N, K, 4])
        q = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
        s = rng.integers(103, 107, (N, K // 32), dtype=np.uint8)
        ref = oracle.dequant(q, s, "mxfp4")
        _bits_equal(_mx(q, s, 0), ref.astype(np.float32), "mx random mode 0")
        for mode in (1, 2):  # spans of at most 3 binades: exact
            _bits_equal(_mx(q, s, mode), ref.astype(np.float32),
                        "mx random N=%d K=%d mode %d" % (N, K, mode))
