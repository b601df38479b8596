"""Pins of the CPU oracle against things other than itself.

Each check ties an oracle function to something the source pages or the
mathematics fix: hand-derived golden fixtures (tests/golden/), brute force on
tiny inputs, closed forms, library routines on special cases, and invariants
(the sparse layer equals a dense masked mixture over all experts; k = E is the
dense softmax mixture; identical experts make routing irrelevant).  The checks
are chosen so that a plausible slip in the oracle - swapped nibbles, a scale
indexed along the wrong axis, a dropped offset, a transposed plane, a wrong
tie-break, a missing term in the combine - fails at least one of them.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

import moe_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- formats --

def test_fp16_golden(orc):
    for line in open(os.path.join(GOLDEN, "fp16_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        hx, val = line.split()
        got = orc.half_to_double(int(hx, 16))
        assert got == float(val), (hx, got, val)
        assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_fp16_all_patterns_match_numpy(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decode(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 65536, 4096).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = np.array([orc.bf16_to_double(int(b)) for b in bits])
    assert np.array_equal(got, ref)
    assert orc.bf16_to_double(0x3F80) == 1.0
    assert orc.bf16_to_double(0xC040) == -3.0


# ----------------------------------------------------------------- dequant --

def _read_dequant_golden(name="dequant_k64.txt", sdtype=np.uint16):
    rows = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        tok = line.split()
        r = int(tok[1])
        if tok[2] == "bytes":
            si = tok.index("scales")
            byts = []
            for b in tok[3:si]:
                if "*" in b:
                    v, n = b.split("*")
                    byts += [int(v, 16)] * int(n)
                else:
                    byts.append(int(b, 16))
            rows.setdefault(r, {})["q"] = np.array(byts, dtype=np.uint8)
            rows[r]["s"] = np.array([int(v, 16) for v in tok[si + 1:]], dtype=sdtype)
        else:
            rows.setdefault(r, {})["expect"] = np.array([float(v) for v in tok[3:]])
    n = len(rows)
    q = np.stack([rows[r]["q"] for r in range(n)])
    s = np.stack([rows[r]["s"] for r in range(n)])
    e = np.stack([rows[r]["expect"] for r in range(n)])
    return q, s, e


def test_dequant_golden(orc):
    q, s, expect = _read_dequant_golden()
    assert q.shape == (3, 32) and expect.shape == (3, 64)
    assert np.array_equal(orc.dequant(q, s), expect)


def test_dequant_special_cases(orc):
    rng = np.random.default_rng(2)
    N, K = 5, 96
    s = S.draw_plane(N, K, rng)[1]
    sv = s.view(np.float16).astype(np.float64)
    # nibble 8 everywhere -> exactly zero
    assert np.all(orc.dequant(np.full((N, K // 2), 0x88, np.uint8), s) == 0.0)
    # nibble 9 everywhere -> the group's scale, broadcast along K
    assert np.array_equal(orc.dequant(np.full((N, K // 2), 0x99, np.uint8), s),
                          np.repeat(sv, 32, axis=1))
    # nibble 0 -> -8 * scale (the extreme of the offset-binary range)
    assert np.array_equal(orc.dequant(np.zeros((N, K // 2), np.uint8), s),
                          -8.0 * np.repeat(sv, 32, axis=1))


def test_dequant_values_fit_fp32(orc):
    # (nibble - 8) * fp16 scale needs at most 15 significant bits: exact in fp32.
    q, s = S.draw_plane(64, 256, np.random.default_rng(3))
    w = orc.dequant(q, s)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)


# ------------------------------------------------------------------ MXFP4 --

def _read_e2m1_golden():
    tab = {}
    for line in open(os.path.join(GOLDEN, "e2m1_values.txt")):
        if line.startswith("#") or not line.strip():
            continue
        c, v = line.split()
        tab[int(c, 16)] = float(v)
    assert sorted(tab) == list(range(16))
    return np.array([tab[c] for c in range(16)])


def _e8m0_library(e):
    """ue8m0 bytes -> fp64 through torch's float8_e8m0fnu conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(e, dtype=np.uint8)).view(torch.float8_e8m0fnu)
    return t.to(torch.float64).numpy()


def _dequant_mxfp4_ref(q, s):
    """Test-side MXFP4 dequant: the golden e2m1 table and the library's ue8m0."""
    tab = _read_e2m1_golden()
    q = np.asarray(q, np.uint8)
    nib = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[:-1] + (q.shape[-1] * 2,))
    return tab[nib] * np.repeat(_e8m0_library(s), 32, axis=-1)


def test_e2m1_golden(orc):
    tab = _read_e2m1_golden()
    for c in range(16):
        got = orc.e2m1_to_double(c)
        assert got == tab[c], (c, got, tab[c])
        assert math.copysign(1.0, got) == math.copysign(1.0, tab[c]), c


def test_e2m1_properties(orc):
    v = [orc.e2m1_to_double(c) for c in range(16)]
    assert all(v[c | 8] == -v[c] for c in range(8))          # bit 3 is the sign
    assert all(v[c] < v[c + 1] for c in range(7))            # codes 0..7 ascend
    assert all((2 * x).is_integer() for x in v) and max(v) == 6.0 and min(v) == -6.0


def test_e8m0_matches_library(orc):
    codes = np.arange(256, dtype=np.uint8)
    ref = _e8m0_library(codes)
    got = np.array([orc.e8m0_to_double(int(c)) for c in codes])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert orc.e8m0_to_double(127) == 1.0


def test_dequant_mxfp4_golden(orc):
    q, s, expect = _read_dequant_golden("dequant_mxfp4_k64.txt", np.uint8)
    assert q.shape == (3, 32) and s.shape == (3, 2) and expect.shape == (3, 64)
    assert np.array_equal(orc.dequant(q, s, "mxfp4"), expect)


def test_dequant_mxfp4_matches_table_and_library(orc):
    q, s = S.draw_plane_mxfp4(48, 256, np.random.default_rng(4))
    s[0, :] = [0, 1, 126, 127, 128, 200, 253, 254]  # the exponent range's ends
    assert np.array_equal(orc.dequant(q, s, "mxfp4"), _dequant_mxfp4_ref(q, s))


def test_expert_mxfp4_matches_library_matmul(orc):
    rng = np.random.default_rng(24)
    H, I = 256, 96
    gate, up, down = [S.draw_plane_mxfp4(*shape, rng) for shape in ((I, H), (I, H), (H, I))]
    x = rng.standard_normal(H)
    h, o = orc.expert_forward(gate, up, down, x, "mxfp4")
    Wg, Wu, Wd = [_dequant_mxfp4_ref(*pl) for pl in (gate, up, down)]
    g, u = Wg @ x, Wu @ x
    href = g * scipy.special.expit(g) * u
    assert np.allclose(h, href, rtol=1e-10, atol=1e-12)
    assert np.allclose(o, Wd @ href, rtol=1e-9, atol=1e-10)


def test_layer_mxfp4_equals_dense_library_mixture(orc):
    """MXFP4 layer with a gated shared expert against numpy: test-side dequant,
    brute-force top-k, scipy softmax weights, dense matmuls."""
    rng = np.random.default_rng(25)
    T, H, E, k, I, SI = 5, 64, 6, 2, 32, 64
    x = S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    planes = {}
    for p, (N, K) in zip(S.PLANES, ((I, H), (I, H), (H, I))):
        qs = [S.draw_plane_mxfp4(N, K, rng) for _ in range(E)]
        planes[p] = (np.stack([a for a, _ in qs]), np.stack([b for _, b in qs]))
    shared = {p: S.draw_plane_mxfp4(N, K, rng)
              for p, (N, K) in zip(S.PLANES, ((SI, H), (SI, H), (H, SI)))}
    gvec = rng.normal(0, 0.1, H).astype(np.float32)
    y, idx, _ = orc.layer(x, logits, k, planes, shared, gvec, fmt="mxfp4")
    xd = S.bf16_bits_to_f32(x).astype(np.float64)

    def mlp(Wg, Wu, Wd, v):
        g, u = Wg @ v, Wu @ v
        return Wd @ (g * scipy.special.expit(g) * u)

    Ws = [_dequant_mxfp4_ref(*shared[p]) for p in S.PLANES]
    p_soft = scipy.special.softmax(logits.astype(np.float64), axis=1)
    for t in range(T):
        sel = _brute_topk(list(logits[t]), k)
        assert sorted(idx[t]) == sorted(sel)
        wsel = p_soft[t, sel] / p_soft[t, sel].sum()
        ref = scipy.special.expit(xd[t] @ gvec.astype(np.float64)) * mlp(*Ws, xd[t])
        for wj, e in zip(wsel, sel):
            ref = ref + wj * mlp(*[_dequant_mxfp4_ref(planes[p][0][e], planes[p][1][e])
                                   for p in S.PLANES], xd[t])
        assert np.allclose(y[t], ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


# ---------------------------------------------------------- router: top-k --

def _brute_topk(L, k):
    return sorted(range(len(L)), key=lambda e: (-L[e], e))[:k]


def test_topk_brute_force_with_ties(orc):
    rng = np.random.default_rng(4)
    for E in range(1, 13):
        for k in range(1, E + 1):
            L = rng.integers(0, 3, size=(16, E)).astype(np.float32)  # many exact ties
            idx, _, _ = orc.router_topk(L, k)
            for t in range(L.shape[0]):
                assert list(idx[t]) == _brute_topk(list(L[t]), k), (E, k, L[t])


def test_topk_brute_force_random(orc):
    rng = np.random.default_rng(5)
    for E, k in [(8, 2), (60, 4), (128, 8), (256, 8), (256, 64), (7, 7)]:
        L = rng.standard_normal((20, E)).astype(np.float32)
        idx, _, _ = orc.router_topk(L, k)
        for t in range(20):
            assert list(idx[t]) == _brute_topk(list(L[t]), k)


def test_topk_all_equal_and_signed_zero(orc):
    L = np.zeros((2, 10), np.float32)
    L[1, ::2] = -0.0  # -0.0 == +0.0 under IEEE comparison: still a tie
    idx, w, _ = orc.router_topk(L, 4)
    assert idx.tolist() == [[0, 1, 2, 3], [0, 1, 2, 3]]
    assert np.all(w == np.float32(0.25))


# -------------------------------------------------------- router: weights --

def test_weights_k1_is_one(orc):
    L = np.random.default_rng(6).standard_normal((50, 32)).astype(np.float32) * 5
    _, w, _ = orc.router_topk(L, 1)
    assert np.all(w == 1.0)


def test_weights_sum_and_ratio(orc):
    rng = np.random.default_rng(7)
    for E, k in [(8, 2), (128, 8), (256, 8), (60, 4)]:
        L = (rng.standard_normal((40, E)) * 3).astype(np.float32)
        idx, w, w64 = orc.router_topk(L, k)
        assert np.all(np.abs(w64.sum(1) - 1.0) < 1e-15)
        assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= k * 2.0 ** -24)
        # w_i / w_j = exp(L_i - L_j): the softmax ratio identity
        Ls = np.take_along_axis(L.astype(np.float64), idx, 1)
        ratio = w64[:, 1:] / w64[:, :1]
        assert np.allclose(ratio, np.exp(Ls[:, 1:] - Ls[:, :1]), rtol=1e-13, atol=0)
        # weights are non-increasing in rank order
        assert np.all(np.diff(w64, axis=1) <= 0)


def test_weights_k_equals_E_is_softmax(orc):
    rng = np.random.default_rng(8)
    for E in [2, 8, 60, 256]:
        L = (rng.standard_normal((10, E)) * 2).astype(np.float32)
        idx, w, w64 = orc.router_topk(L, E)
        ref = scipy.special.softmax(L.astype(np.float64), axis=1)
        ref_sel = np.take_along_axis(ref, idx, 1)
        assert np.allclose(w64, ref_sel, rtol=1e-13, atol=1e-300)


def test_route_scale(orc):
    L = np.random.default_rng(9).standard_normal((5, 16)).astype(np.float32)
    _, _, w1 = orc.router_topk(L, 4, 1.0)
    _, _, w2 = orc.router_topk(L, 4, 2.5)
    assert np.allclose(w2, 2.5 * w1, rtol=1e-15)


# ------------------------------------------------------------ router logits --

def test_router_logits_exact_integers(orc):
    rng = np.random.default_rng(10)
    T, H, E = 6, 256, 9
    xv = rng.integers(-3, 4, (T, H)).astype(np.float32)
    wv = rng.integers(-5, 6, (E, H)).astype(np.float32)
    g = rng.integers(-2, 3, (H,)).astype(np.float32)
    x = S.f32_to_bf16_bits(xv)  # small integers are exact in bf16
    out = orc.router_logits(x, wv, g)
    exact = np.concatenate([xv.astype(np.int64) @ wv.astype(np.int64).T,
                            (xv.astype(np.int64) @ g.astype(np.int64))[:, None]], 1)
    assert np.array_equal(out, exact.astype(np.float32))


def test_router_logits_vs_matmul(orc):
    wl = S.WORKLOADS["decode_batch"]
    x = S.draw_x(wl)[:8]
    wr = S.draw_router(wl)
    out = orc.router_logits(x, wr)
    ref = S.bf16_bits_to_f32(x).astype(np.float64) @ wr.astype(np.float64).T
    # both are fp64 sums of the same exact products, then one rounding to fp32
    assert np.max(np.abs(out - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2.0 ** -24 * 1.0001


# ------------------------------------------------------------- permutation --

def test_permute_matches_stable_sort(orc):
    rng = np.random.default_rng(11)
    for T, k, E in [(4, 2, 8), (32, 8, 128), (512, 4, 60), (3, 3, 256), (100, 1, 5)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        off, srt, row_of = orc.permute(idx, E)
        flat = idx.ravel()
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
        assert np.array_equal(srt, np.argsort(flat, kind="stable"))
        assert np.array_equal(srt[row_of], np.arange(T * k))
        for e in range(E):
            assert np.all(flat[srt[off[e]:off[e + 1]]] == e)


def test_permute_drops_out_of_range_picks(orc):
    """A pick outside [0, E) (top-p's -1, or any index past the experts) is in
    no bucket: the buckets are those of the valid picks alone, in slot order,
    row_of is -1 for the dropped slots and off[E] counts the valid ones.
    Checked against brute force: the valid slots' stable sort by expert."""
    rng = np.random.default_rng(12)
    for T, k, E, frac in [(300, 4, 16, 0.1), (9, 8, 256, 0.5), (50, 3, 5, 1.0), (64, 2, 7, 0.0)]:
        idx = rng.integers(0, E, (T, k)).astype(np.int32)
        bad = rng.random((T, k)) < frac
        idx[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, E + rng.integers(0, 9))
        off, srt, row_of = orc.permute(idx, E)
        flat = idx.ravel()
        valid = (flat >= 0) & (flat < E)
        slots = np.nonzero(valid)[0]
        want_sorted = slots[np.argsort(flat[valid], kind="stable")]
        assert off[0] == 0 and off[E] == valid.sum()
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(np.bincount(flat[valid],
                                                                              minlength=E))]))
        assert np.array_equal(srt[: off[E]], want_sorted)
        assert np.all(row_of[~valid] == -1)
        assert np.array_equal(srt[row_of[valid]], slots)
        for e in range(E):
            assert set(srt[off[e]:off[e + 1]].tolist()) == set(np.nonzero(flat == e)[0].tolist())


# -------------------------------------------------------------- expert MLP --

def _tiny_planes(rng, H, I):
    return [S.draw_plane(*shape, rng) for shape in ((I, H), (I, H), (H, I))]


def test_expert_onehot_picks_one_column(orc):
    """x = one-hot at position c -> g = Wg[:, c], u = Wu[:, c] (pins the K axis)."""
    rng = np.random.default_rng(12)
    H, I = 64, 32
    gate, up, down = _tiny_planes(rng, H, I)
    Wg, Wu, Wd = orc.dequant(*gate), orc.dequant(*up), orc.dequant(*down)
    for c in [0, 1, 31, 32, 63]:
        x = np.zeros(H)
        x[c] = 1.0
        h, o = orc.expert_forward(gate, up, down, x)
        g, u = Wg[:, c], Wu[:, c]
        # silu(g) * u written as the closed form g / (1 + e^-g) * u
        assert np.allclose(h, [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(g, u)],
                           rtol=1e-14, atol=0)


def test_expert_down_plane_orientation(orc):
    """Only gate row r0 is non-zero -> h is one-hot at r0 -> o = Wd[:, r0] * h[r0]."""
    rng = np.random.default_rng(13)
    H, I = 64, 64
    gate, up, down = _tiny_planes(rng, H, I)
    gq = np.full_like(gate[0], 0x88)  # all zero weights
    r0 = 37
    gq[r0] = gate[0][r0]
    gate = (gq, gate[1])
    x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_normal(H).astype(np.float32))).astype(np.float64)
    h, o = orc.expert_forward(gate, up, down, x)
    assert np.count_nonzero(h) == 1 and h[r0] != 0.0
    Wd = orc.dequant(*down)
    assert np.allclose(o, Wd[:, r0] * h[r0], rtol=1e-14, atol=0)


def test_expert_closed_form_uniform_planes(orc):
    """Uniform planes give a hand-computable MLP.

    gate nibble 9, scale 0.125 -> Wg = 0.125; up nibble 10, scale 0.25 -> Wu = 0.5;
    down nibble 7, scale 0.5 -> Wd = -0.5.  With x = 0.5 everywhere (H = 32):
    g = 0.125*16 = 2, u = 0.5*16 = 8, h = silu(2)*8, o = -0.5 * I * h."""
    H, I = 32, 64
    f16 = lambda v: np.full(1, v, np.float16).view(np.uint16)[0]
    gate = (np.full((I, H // 2), 0x99, np.uint8), np.full((I, 1), f16(0.125), np.uint16))
    up = (np.full((I, H // 2), 0xAA, np.uint8), np.full((I, 1), f16(0.25), np.uint16))
    down = (np.full((H, I // 2), 0x77, np.uint8), np.full((H, 2), f16(0.5), np.uint16))
    h, o = orc.expert_forward(gate, up, down, np.full(H, 0.5))
    hv = 2.0 / (1.0 + math.exp(-2.0)) * 8.0
    assert np.allclose(h, hv, rtol=1e-15)
    assert np.allclose(o, -0.5 * I * hv, rtol=1e-14)


def test_expert_matches_library_matmul(orc):
    rng = np.random.default_rng(14)
    H, I = 256, 96
    gate, up, down = _tiny_planes(rng, H, I)
    x = rng.standard_normal(H)
    h, o = orc.expert_forward(gate, up, down, x)
    Wg, Wu, Wd = orc.dequant(*gate), orc.dequant(*up), orc.dequant(*down)
    g, u = Wg @ x, Wu @ x
    href = g * scipy.special.expit(g) * u
    assert np.allclose(h, href, rtol=1e-10, atol=1e-12)
    assert np.allclose(o, Wd @ href, rtol=1e-9, atol=1e-10)


# ------------------------------------------------------------------- layer --

def _tiny_layer_inputs(seed=15, T=6, H=64, E=6, k=2, I=32, SI=0):
    rng = np.random.default_rng(seed)
    x = S.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    planes = {}
    for p, (N, K) in zip(S.PLANES, ((I, H), (I, H), (H, I))):
        qs = [S.draw_plane(N, K, rng) for _ in range(E)]
        planes[p] = (np.stack([a for a, _ in qs]), np.stack([b for _, b in qs]))
    shared = None
    if SI:
        shared = {p: S.draw_plane(N, K, rng)
                  for p, (N, K) in zip(S.PLANES, ((SI, H), (SI, H), (H, SI)))}
    return x, logits, planes, shared


def _expert_outputs(orc, x, planes, E):
    """o[t][e] for every token and every expert (dense evaluation)."""
    T, H = x.shape
    xd = S.bf16_bits_to_f32(x).astype(np.float64)
    out = np.zeros((T, E, H))
    for e in range(E):
        pl = [(planes[p][0][e], planes[p][1][e]) for p in S.PLANES]
        for t in range(T):
            out[t, e] = orc.expert_forward(*pl, xd[t])[1]
    return out


def test_layer_equals_dense_masked_mixture(orc):
    x, logits, planes, _ = _tiny_layer_inputs()
    T, E, k = x.shape[0], logits.shape[1], 2
    y, idx, w = orc.layer(x, logits, k, planes)
    dense = _expert_outputs(orc, x, planes, E)
    # mask m_e and renormalised softmax weights over the selected experts
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    for t in range(T):
        m = np.zeros(E)
        m[_brute_topk(list(logits[t]), k)] = 1.0
        wt = m * p[t] / np.sum(m * p[t])
        ref = (wt[:, None] * dense[t]).sum(0)
        assert np.allclose(y[t], ref, rtol=1e-6, atol=1e-6 * np.max(np.abs(ref)))
        assert sorted(idx[t]) == sorted(np.nonzero(m)[0])


def test_layer_k_equals_E_is_dense_softmax_mixture(orc):
    x, logits, planes, _ = _tiny_layer_inputs(seed=16, E=5)
    E = 5
    y, _, _ = orc.layer(x, logits, E, planes)
    dense = _expert_outputs(orc, x, planes, E)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    ref = np.einsum("te,teh->th", p, dense)
    assert np.allclose(y, ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


def test_layer_identical_experts_ignore_routing(orc):
    x, logits, planes, _ = _tiny_layer_inputs(seed=17)
    E = logits.shape[1]
    same = {p: (np.repeat(planes[p][0][:1], E, 0), np.repeat(planes[p][1][:1], E, 0))
            for p in S.PLANES}
    y, _, _ = orc.layer(x, logits, 3, same)
    one = _expert_outputs(orc, x, {p: (same[p][0][:1], same[p][1][:1]) for p in S.PLANES}, 1)[:, 0]
    assert np.allclose(y, one, rtol=1e-6, atol=1e-6 * np.abs(one).max())


def test_layer_rows_subset_matches_full(orc):
    x, logits, planes, shared = _tiny_layer_inputs(seed=18, SI=48)
    g = np.random.default_rng(1).normal(0, 0.1, x.shape[1]).astype(np.float32)
    yf, idf, wf = orc.layer(x, logits, 2, planes, shared, g)
    rows = [4, 0, 2]
    ys, ids, ws = orc.layer(x, logits, 2, planes, shared, g, rows=rows)
    assert np.array_equal(ys, yf[rows]) and np.array_equal(ids, idf[rows]) and np.array_equal(ws, wf[rows])


def test_layer_shared_expert_gate(orc):
    """g = 0 -> sigma = 1/2 exactly; zero routed experts isolate the shared term,
    which must equal the same planes run as a routed expert at weight one."""
    T, H, E, I, SI = 4, 64, 4, 32, 96
    x, logits, planes, shared = _tiny_layer_inputs(seed=19, T=T, H=H, E=E, I=I, SI=SI)
    zero = {p: (np.full_like(planes[p][0], 0x88), planes[p][1]) for p in S.PLANES}
    y_half, _, _ = orc.layer(x, logits, 2, zero, shared, np.zeros(H, np.float32))
    y_one, _, _ = orc.layer(x, logits, 2, zero, shared, None)  # ungated: weight one
    as_routed = {p: (shared[p][0][None], shared[p][1][None]) for p in S.PLANES}
    y_ref, _, _ = orc.layer(x, np.zeros((T, 1), np.float32), 1, as_routed)
    assert np.array_equal(y_one, y_ref)
    assert np.allclose(y_half, 0.5 * y_ref.astype(np.float64), rtol=1e-6, atol=0)
    # with a real gate vector the shared term scales by sigma(x . g)
    gvec = np.random.default_rng(2).normal(0, 0.05, H).astype(np.float32)
    y_g, _, _ = orc.layer(x, logits, 2, zero, shared, gvec)
    a = S.bf16_bits_to_f32(x).astype(np.float64) @ gvec.astype(np.float64)
    assert np.allclose(y_g, scipy.special.expit(a)[:, None] * y_ref, rtol=1e-6, atol=1e-7)
    # and the shared term adds to the routed mixture (no term dropped)
    y_full, _, _ = orc.layer(x, logits, 2, planes, shared, gvec)
    y_routed, _, _ = orc.layer(x, logits, 2, planes)
    assert np.allclose(y_full, y_routed.astype(np.float64) + y_g, rtol=1e-5,
                       atol=1e-5 * np.abs(y_full).max())


# ------------------------------------------------- combine folded: add+rms --

def test_bf16_rounding_golden(orc):
    n = 0
    for line in open(os.path.join(GOLDEN, "bf16_rounding.txt")):
        if line.startswith("#") or not line.strip():
            continue
        m, e, bits = line.split()[:3]
        v = math.ldexp(int(m), int(e))
        assert orc.double_to_bf16(v) == int(bits, 16), line
        n += 1
    assert n == 11


def test_bf16_rounding_matches_library_on_fp32_values(orc):
    """For values already in fp32 one rounding is the library's fp32 -> bf16."""
    import torch
    rng = np.random.default_rng(30)
    f = np.concatenate([rng.standard_normal(3000).astype(np.float32),
                        (rng.standard_normal(500) * 1e-38).astype(np.float32),
                        np.float32([3.3e38, -3.39e38, 1.0, 0.0])])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.double_to_bf16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_add_rmsnorm_matches_library_rms_norm(orc):
    import torch
    rng = np.random.default_rng(31)
    T, H, eps = 5, 384, 1e-6
    r = rng.standard_normal((T, H)).astype(np.float32)
    y = (0.1 * rng.standard_normal((T, H))).astype(np.float32)
    g = (1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32)
    r_out, n_out = orc.add_rmsnorm(r, y, g, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(r_out.astype(np.float64)), (H,),
                                       torch.from_numpy(g.astype(np.float64)), eps).numpy()
    want = np.array([orc.double_to_bf16(v) for v in ref.ravel()], dtype=np.uint16).reshape(T, H)
    assert np.array_equal(n_out, want)


def test_add_rmsnorm_special_cases(orc):
    H = 64
    g = np.ones(H, np.float32)
    c = np.full((2, H), 3.0, np.float32)
    c[1] = -0.25
    z = np.zeros_like(c)
    # y = 0 leaves the residual; a constant row normalises to its sign (eps = 0)
    r_out, n_out = orc.add_rmsnorm(c, z, g, 0.0)
    assert np.array_equal(r_out, c)
    assert np.all(n_out[0] == 0x3F80) and np.all(n_out[1] == 0xBF80)
    # eps = c^2 halves the mean square's weight: 1/sqrt(2)
    _, n_eps = orc.add_rmsnorm(c[:1], z[:1], g, 9.0)
    assert np.all(n_eps == orc.double_to_bf16(1.0 / math.sqrt(2.0)))
    # r = 0 passes y through; the weight scales the normed row elementwise
    g2 = np.arange(1, H + 1, dtype=np.float32)
    r_out, n_out = orc.add_rmsnorm(z[:1], c[:1], g2, 0.0)
    assert np.array_equal(r_out, c[:1])
    assert np.array_equal(n_out[0], [orc.double_to_bf16(float(v)) for v in g2])
    # the add is one rounding of the exact sum: 1 + 2^-24 + 2^-40 rounds up
    r1 = np.ones((1, H), np.float32)
    y1 = np.full((1, H), np.float32(2.0 ** -24 + 2.0 ** -40), np.float32)
    r_out, _ = orc.add_rmsnorm(r1, y1, g, 0.0)
    assert np.all(r_out == np.float32(1.0 + 2.0 ** -23))


# --------------------------------------------------------- expert top-p --

def _log_row(probs):
    return np.log(np.asarray([probs], dtype=np.float64)).astype(np.float32)


def test_top_p_closed_form(orc):
    """Probabilities 1/2, 1/4, 1/8, 1/8: p = 0.7 keeps two picks (1/2 < 0.7,
    3/4 >= 0.7), p = 0.76 three, p = 0.1 one; weights renormalise over them."""
    L = _log_row([4, 2, 1, 1])
    idx, w, _ = orc.router_topk(L, 4, 1.0, 0.7)
    assert list(idx[0]) == [0, 1, -1, -1]
    assert np.allclose(w[0], [2 / 3, 1 / 3, 0, 0], rtol=1e-6, atol=0)
    idx, w, _ = orc.router_topk(L, 4, 2.0, 0.76)
    assert list(idx[0]) == [0, 1, 2, -1]
    assert np.allclose(w[0], [8 / 7, 4 / 7, 2 / 7, 0], rtol=1e-6, atol=0)
    idx, w, _ = orc.router_topk(L, 4, 1.5, 0.1)
    assert list(idx[0]) == [0, -1, -1, -1] and list(w[0]) == [1.5, 0, 0, 0]
    # the mass of unpicked experts counts: probabilities 8, 4, 2, 2, 1, 1, 1, 1
    # over 20; p = 0.45 keeps two picks (0.4 < 0.45 <= 0.6), where a mass over
    # the four picks alone (0.5 >= 0.45) would keep one
    L2 = _log_row([8, 4, 2, 2, 1, 1, 1, 1])
    idx, w, _ = orc.router_topk(L2, 4, 1.0, 0.45)
    assert list(idx[0]) == [0, 1, -1, -1]


def test_top_p_off_values_keep_all(orc):
    rng = np.random.default_rng(40)
    L = rng.standard_normal((20, 32)).astype(np.float32)
    ref = orc.router_topk(L, 6, 1.25)
    for p in (0.0, 1.0, 1.5, -0.3):
        got = orc.router_topk(L, 6, 1.25, p)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_top_p_prefix_property(orc):
    """Against the library softmax: the kept picks are the shortest rank-order
    prefix of the top-k whose probability reaches p (or all k), and their
    weights are the renormalised softmax times the scale."""
    rng = np.random.default_rng(41)
    T, E, k, p, scale = 200, 64, 8, 0.6, 1.5
    L = (2.0 * rng.standard_normal((T, E))).astype(np.float32)
    idx_all, _, _ = orc.router_topk(L, k, scale)
    idx, w, w64 = orc.router_topk(L, k, scale, p)
    P = scipy.special.softmax(L.astype(np.float64), axis=1)
    for t in range(T):
        pr = P[t, idx_all[t]]
        cum = np.concatenate([[0.0], np.cumsum(pr)])
        kept = int(np.sum(idx[t] >= 0))
        assert np.array_equal(idx[t][:kept], idx_all[t][:kept]) and np.all(idx[t][kept:] == -1)
        assert cum[kept - 1] < p and (kept == k or cum[kept] >= p)
        assert np.allclose(w64[t][:kept], scale * pr[:kept] / pr[:kept].sum(), rtol=1e-12)
        assert np.all(w[t][kept:] == 0.0)


def test_layer_top_p_is_mixture_over_kept_picks(orc):
    x, logits, planes, _ = _tiny_layer_inputs(seed=42, E=6)
    T, E, k, p = x.shape[0], 6, 4, 0.55
    y, idx, w = orc.layer(x, logits, k, planes, top_p=p)
    dense = _expert_outputs(orc, x, planes, E)
    P = scipy.special.softmax(logits.astype(np.float64), axis=1)
    for t in range(T):
        order = _brute_topk(list(logits[t]), k)
        cum = np.concatenate([[0.0], np.cumsum(P[t, order])])
        kept = next((j for j in range(1, k + 1) if j == k or cum[j] >= p), k)
        sel = order[:kept]
        ref = (P[t, sel][:, None] * dense[t, sel]).sum(0) / P[t, sel].sum()
        assert np.allclose(y[t], ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
        assert list(idx[t][:kept]) == list(sel) and np.all(idx[t][kept:] == -1)


# ------------------------------------------- router variants (gate, bias) --

def test_sigmoid_gate_and_bias_closed_form(orc):
    """sigma(0) = 1/2, sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4."""
    L = np.array([[0.0, math.log(3.0), -math.log(3.0), -5.0]], dtype=np.float32)
    idx, w, _ = orc.router_topk(L, 2, 1.0, gate="sigmoid")
    assert list(idx[0]) == [1, 0] and np.allclose(w[0], [0.6, 0.4], rtol=1e-6)
    # a selection bias of 0.6 lifts expert 2's key to 0.85: it is picked first,
    # but its weight comes from its unbiased score 1/4
    b = np.array([0.0, 0.0, 0.6, 0.0], np.float32)
    idx, w, _ = orc.router_topk(L, 2, 2.0, gate="sigmoid", bias=b)
    assert list(idx[0]) == [2, 1] and np.allclose(w[0], [0.5, 1.5], rtol=1e-6)
    # softmax gate with a bias: probabilities of [0, ln 3] alone are 1/4, 3/4
    L2 = np.array([[0.0, math.log(3.0)]], dtype=np.float32)
    idx, w, _ = orc.router_topk(L2, 1, 1.0, bias=np.array([0.6, 0.0], np.float32))
    assert list(idx[0]) == [0] and w[0][0] == 1.0


def test_variant_reductions(orc):
    rng = np.random.default_rng(50)
    T, E, k = 30, 40, 6
    L = (1.5 * rng.standard_normal((T, E))).astype(np.float32)
    plain = orc.router_topk(L, k, 1.25)
    zero_bias = orc.router_topk(L, k, 1.25, bias=np.zeros(E, np.float32))
    assert np.array_equal(plain[0], zero_bias[0])
    assert np.allclose(plain[2], zero_bias[2], rtol=1e-12)
    # sigmoid gate, k = E: weights are sigma(L) renormalised (library expit)
    idx, _, w64 = orc.router_topk(L, E, 1.0, gate="sigmoid")
    s = scipy.special.expit(L.astype(np.float64))
    for t in range(T):
        assert np.allclose(w64[t], s[t, idx[t]] / s[t].sum(), rtol=1e-12)
        assert list(idx[t]) == sorted(range(E), key=lambda e: (-s[t, e], e))
    # a dominant bias picks its experts first, in bias order
    b = np.zeros(E, np.float32)
    b[[7, 3, 21]] = [30.0, 20.0, 10.0]
    idx, _, _ = orc.router_topk(L, 3, 1.0, gate="sigmoid", bias=b)
    assert np.all(idx == [7, 3, 21])


def test_variant_ties_lower_index(orc):
    L = np.zeros((1, 8), np.float32)
    b = np.array([0, 1, 0, 1, 0, 1, 0, 1], np.float32)
    idx, w, _ = orc.router_topk(L, 5, 1.0, gate="sigmoid", bias=b)
    assert list(idx[0]) == [1, 3, 5, 7, 0] and np.allclose(w[0], 0.2, rtol=1e-12)


def test_layer_variant_is_mixture_over_picks(orc):
    x, logits, planes, _ = _tiny_layer_inputs(seed=51, E=6)
    T, E, k = x.shape[0], 6, 3
    b = np.random.default_rng(52).normal(0, 0.3, E).astype(np.float32)
    y, idx, w = orc.layer(x, logits, k, planes, gate="sigmoid", bias=b)
    dense = _expert_outputs(orc, x, planes, E)
    s = scipy.special.expit(logits.astype(np.float64))
    for t in range(T):
        sel = sorted(range(E), key=lambda e: (-(s[t, e] + float(b[e])), e))[:k]
        ref = (s[t, sel][:, None] * dense[t, sel]).sum(0) / s[t, sel].sum()
        assert list(idx[t]) == sel
        assert np.allclose(y[t], ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())


# ------------------------------------------- grouped routing (noaux_tc) --

def test_grouped_closed_form(orc):
    """E = 8 in four groups of two, keep two groups, k = 2, sigmoid scores.
    Expert 0 has the largest key, but its group's score (sigma(5) + sigma(-5)
    = 1) ranks below groups 1 (2 sigma(2) = 1.76) and 2 (2 sigma(1) = 1.46),
    so the picks are experts 2 and 3 (equal keys: the lower index first) at
    weight 1/2 each; the plain top-2 would take expert 0.  A uniform negative
    bias (every key below zero) changes nothing: experts outside the kept
    groups are out of the selection, not given a key of zero."""
    L = np.array([[5.0, -5.0, 2.0, 2.0, 1.0, 1.0, 0.0, 0.0]], np.float32)
    idx, w, _ = orc.router_topk(L, 2, 1.0, gate="sigmoid", n_group=4, topk_group=2)
    assert list(idx[0]) == [2, 3] and np.allclose(w[0], [0.5, 0.5], rtol=1e-12)
    plain, _, _ = orc.router_topk(L, 2, 1.0, gate="sigmoid")
    assert list(plain[0]) == [0, 2]
    b = np.full(8, -1.0, np.float32)
    idx, w, _ = orc.router_topk(L, 2, 3.0, gate="sigmoid", bias=b, n_group=4, topk_group=2)
    assert list(idx[0]) == [2, 3] and np.allclose(w[0], [1.5, 1.5], rtol=1e-12)
    # keep three groups, k = 3: group 3 (score 1.0) ties group 0 (1.0 up to
    # rounding, sigma(5) + sigma(-5) in fp64), so the third kept group is one
    # of them: with group 0, expert 0's key ranks first; with group 3, expert
    # 4 (sigma(1)) is the third pick
    idx, _, _ = orc.router_topk(L, 3, 1.0, gate="sigmoid", n_group=4, topk_group=3)
    assert list(idx[0]) in ([0, 2, 3], [2, 3, 4])


def _brute_grouped(key, s, k, n_group, topk_group):
    """Picks and weights by exhaustion: the kept groups are the subset of
    topk_group groups with the largest total score (the lexicographically
    smallest such subset on ties), a group's score the sum of its two
    largest keys; the picks a full stable sort of the kept experts.  Subsets
    are compared by their scores sorted in descending order: the largest such
    tuple is that of a largest-total subset (the top scores), and equal
    tuples are equal totals, with no fp rounding of sums in the way."""
    E = len(key)
    gsz = E // n_group
    gs = []
    for g in range(n_group):
        top = sorted(key[g * gsz:(g + 1) * gsz], reverse=True)
        gs.append(top[0] + top[1] if gsz >= 2 else top[0])
    best = None
    for sub in itertools.combinations(range(n_group), topk_group):  # ascending tuples
        tot = sorted((gs[g] for g in sub), reverse=True)
        if best is None or tot > best[0]:
            best = (tot, sub)
    allowed = [e for e in range(E) if e // gsz in best[1]]
    sel = sorted(allowed, key=lambda e: (-key[e], e))[:k]
    w = np.array([s[e] for e in sel]) / sum(s[e] for e in sel)
    return sel, w


def test_grouped_brute_force(orc):
    """Small rows with many exact ties (integer logits from {0, 1, 2}, biases
    from three values): the oracle's grouped picks and weights against
    exhaustion over the group subsets, for both score functions."""
    for E, n_group, topk_group, k in [(8, 4, 2, 3), (12, 3, 2, 5), (12, 6, 3, 4), (16, 8, 4, 8),
                                      (6, 6, 2, 2), (10, 2, 1, 5)]:
        _grouped_brute_force_case(orc, E, n_group, topk_group, k)


def _grouped_brute_force_case(orc, E, n_group, topk_group, k):
    rng = np.random.default_rng(E * 100 + n_group * 10 + k)
    T = 60
    L = rng.integers(0, 3, (T, E)).astype(np.float32)
    b = rng.choice(np.array([0.0, 0.125, -0.25], np.float32), E)
    for gate in ("sigmoid", "softmax"):
        idx, _, w64 = orc.router_topk(L, k, 1.0, gate=gate, bias=b, n_group=n_group,
                                      topk_group=topk_group)
        Ld = L.astype(np.float64)
        s = scipy.special.expit(Ld) if gate == "sigmoid" else scipy.special.softmax(Ld, axis=1)
        for t in range(T):
            key = [float(s[t, e]) + float(b[e]) for e in range(E)]
            sel, w = _brute_grouped(key, s[t], k, n_group, topk_group)
            assert list(idx[t]) == sel, (gate, t)
            assert np.allclose(w64[t], w, rtol=1e-12)


def test_grouped_reductions(orc):
    """Keeping every group, or groups of one expert with as many kept as
    picks, is the ungrouped variant."""
    rng = np.random.default_rng(53)
    T, E, k = 40, 32, 6
    L = (1.5 * rng.standard_normal((T, E))).astype(np.float32)
    b = rng.normal(0, 0.05, E).astype(np.float32)
    plain = orc.router_topk(L, k, 1.0, gate="sigmoid", bias=b)
    for ng, tg in [(4, 4), (8, 8), (32, k)]:
        g = orc.router_topk(L, k, 1.0, gate="sigmoid", bias=b, n_group=ng, topk_group=tg)
        assert np.array_equal(plain[0], g[0]), (ng, tg)
        assert np.array_equal(plain[2], g[2])


def test_layer_grouped_is_mixture_over_picks(orc):
    x, logits, planes, _ = _tiny_layer_inputs(seed=54, E=6)
    T, E, k = x.shape[0], 6, 2
    b = np.random.default_rng(55).normal(0, 0.3, E).astype(np.float32)
    y, idx, w = orc.layer(x, logits, k, planes, gate="sigmoid", bias=b, n_group=3, topk_group=1)
    dense = _expert_outputs(orc, x, planes, E)
    s = scipy.special.expit(logits.astype(np.float64))
    for t in range(T):
        key = [float(s[t, e]) + float(b[e]) for e in range(E)]
        sel, wt = _brute_grouped(key, s[t], k, 3, 1)
        assert sel[0] // 2 == sel[1] // 2  # one kept group of two experts: both picked
        ref = (wt[:, None] * dense[t, sel]).sum(0)
        assert np.allclose(y[t], ref, rtol=1e-6, atol=1e-6 * np.abs(ref).max())
        assert list(idx[t]) == sel


# ------------------------------- residual step with the next router folded --

def test_add_rmsnorm_router_one_hot_rows(orc):
    """One-hot router rows read single features of the bf16 normed row
    exactly (a product by one, no sum), and a row of twos doubles it; the
    first outputs equal add_rmsnorm's."""
    rng = np.random.default_rng(57)
    T, H = 4, 256
    r = rng.standard_normal((T, H)).astype(np.float32)
    y = (0.1 * rng.standard_normal((T, H))).astype(np.float32)
    g = (1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32)
    cols = [0, 17, 255, 128]
    W = np.zeros((len(cols) + 1, H), np.float32)
    for e, c in enumerate(cols):
        W[e, c] = 1.0
    W[-1, 3] = 2.0
    r_out, n_out, L = orc.add_rmsnorm_router(r, y, g, 1e-6, W)
    r2, n2 = orc.add_rmsnorm(r, y, g, 1e-6)
    assert np.array_equal(r_out, r2) and np.array_equal(n_out, n2)
    nf = S.bf16_bits_to_f32(n_out)
    assert np.array_equal(L[:, :len(cols)], nf[:, cols])
    assert np.array_equal(L[:, -1], 2.0 * nf[:, 3])


def test_add_rmsnorm_router_matches_library(orc):
    """The logits are the fp64 matrix product of the bf16 normed row (as
    bf16, not the unrounded norm) with the router plane, rounded to fp32;
    checked against torch's rms_norm, bf16 rounding and float64 matmul."""
    import torch
    rng = np.random.default_rng(58)
    T, H, E, eps = 6, 512, 24, 1e-5
    r = rng.standard_normal((T, H)).astype(np.float32)
    y = (0.1 * rng.standard_normal((T, H))).astype(np.float32)
    g = (1.0 + 0.2 * rng.standard_normal(H)).astype(np.float32)
    W = rng.normal(0, 0.02, (E, H)).astype(np.float32)
    _, n_out, L = orc.add_rmsnorm_router(r, y, g, eps, W)
    r64 = torch.from_numpy((r.astype(np.float64) + y.astype(np.float64)).astype(np.float32)
                           .astype(np.float64))
    nrm = torch.nn.functional.rms_norm(r64, (H,), torch.from_numpy(g.astype(np.float64)), eps)
    xb = nrm.to(torch.bfloat16).to(torch.float64)
    assert np.array_equal(S.f32_to_bf16_bits(xb.numpy().astype(np.float32)), n_out)
    ref = (xb @ torch.from_numpy(W.astype(np.float64)).T).numpy().astype(np.float32)
    assert np.max(np.abs(L - ref) / np.maximum(np.abs(ref), 1e-30)) <= 2.0 ** -24 * 1.0001
    # the unrounded norm would give different logits
    unrounded = (nrm @ torch.from_numpy(W.astype(np.float64)).T).numpy().astype(np.float32)
    assert not np.array_equal(L, unrounded)
