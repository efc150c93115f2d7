"""Pins of the oracle's number formats (E2M1, E8M0 block exponents, UE4M3)
against brute-force nearest-value searches and the values the APA post prints
('Pass 1: FP4 everywhere, with a hot test', format paragraph)."""
import ctypes as C
import json
import os

import numpy as np

from brute_apa import quantise_blocks
from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
FACTS = json.load(open(os.path.join(HERE, "golden", "page_facts.json")))
MAGS = np.array(FACTS["e2m1_values"]["value"], np.float64)


def nearest_even(a):
    """Nearest E2M1 magnitude code by search; ties to the even code."""
    a = min(abs(a), 6.0)
    d = np.abs(MAGS - a)
    best = np.flatnonzero(d == d.min())
    ev = [i for i in best if i % 2 == 0]
    return int(ev[0] if ev else best[0])


def test_e2m1_value_table_matches_page():
    for c in range(16):
        v = O.e2m1_value(c)
        assert abs(v) == MAGS[c & 7]
        assert (v < 0 or (v == 0 and np.signbit(v))) == bool(c & 8) or (c & 7) == 0


def test_e2m1_rne_exhaustive_fp16_times_scales():
    # every positive finite fp16 value, scaled by 2^k for k in -3..3: covers all
    # rounding neighbourhoods with 11-bit mantissas, including every tie
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    L = O.lib()
    for k in (-3, -1, 0, 1, 3):
        xs = h * 2.0 ** k
        xs = xs[xs <= 8.0]
        got = np.array([L.orc_e2m1_mag(float(x)) for x in xs])
        want = np.array([nearest_even(x) for x in xs])
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (k, xs[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_ties_and_sign():
    # ties to the even code (0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4)
    for x, v in [(0.25, 0), (0.75, 1), (1.25, 1), (1.75, 2), (2.5, 2), (3.5, 4), (5.0, 4),
                 (6.0, 6), (7.0, 6), (100.0, 6)]:
        assert MAGS[O.e2m1_mag(x)] == v
    assert O.e2m1_code(-0.1) == 0x8          # IEEE sign of a value rounding to zero
    assert O.e2m1_code(-0.0) == 0x8
    assert O.e2m1_code(0.0) == 0x0
    assert O.e2m1_code(-6.0) == 0xF


def test_e8m0_block_exponent_lands_max_in_upper_octave():
    rng = np.random.default_rng(0)
    for a in np.concatenate([rng.uniform(1e-30, 1e30, 2000) ** rng.uniform(0, 1, 2000),
                             [6.0, 3.0, 3.0000001, 12.0, 6 * 2.0 ** -120, 1e-3]]):
        e = O.e8m0_exp(float(a))
        if -127 < e < 127:
            assert a <= 6.0 * 2.0 ** e and a > 6.0 * 2.0 ** (e - 1)
            r = a / 2.0 ** e
            assert 3.0 < r <= 6.0                # "anywhere in (3, 6]" for power-of-two scales
    assert O.e8m0_exp(0.0) == -127
    assert O.e8m0_exp(1e-300) == -127


def test_ue4m3_nearest_and_max():
    vals = sorted({O.ue4m3_rn(v) for v in np.linspace(0, 500, 20001)})
    assert max(vals) == FACTS["ue4m3_max"]["value"]
    # every representable value: e in 1..15 normal, e=0 subnormal (step 2^-9)
    rep = [m * 2.0 ** -9 for m in range(8)] + [(1 + m / 8) * 2.0 ** (e - 7)
                                               for e in range(1, 16) for m in range(8)][:-1]
    rep = np.array(sorted(rep))
    rng = np.random.default_rng(1)
    for a in np.concatenate([rng.uniform(0, 450, 3000), rep, (rep[1:] + rep[:-1]) / 2]):
        got = O.ue4m3_rn(float(a))
        d = np.abs(rep - a)
        best = np.flatnonzero(d == d.min())
        if len(best) == 1:
            assert got == rep[best[0]], a
        else:  # tie: even mantissa (index parity within the encoding)
            assert got in rep[best]
            enc = [i for i in range(127) if O.scale_value(i, O.NV) == got][0]
            assert enc % 2 == 0, (a, got)


def test_nv_blob_and_footprint_match_page():
    # K (64 keys x 128 ch) and V^T (128 ch x 64 keys) in 4-bit codes, one
    # one-byte UE4M3 scale per 16 values: the page's 9216-byte tile blob
    D, T, bs = 128, 64, FACTS["nv_block"]["value"]
    blob = 2 * (T * D // 2) + 2 * (T * D // bs)
    assert blob == FACTS["nv_tile_blob_bytes_d128"]["value"]
    tiles = 122880 // FACTS["tile_keys"]["value"]
    mib = tiles * 8 * blob / 2 ** 20
    assert round(mib, 1) == FACTS["nv_fp4_kv_mib_8heads_122880keys"]["value"]
    win = (1 + 2 * 96) * 8 * blob / 2 ** 20
    assert round(win, 1) == FACTS["nv_kv_window_mib"]["value"]
    assert 6 * FACTS["ue4m3_max"]["value"] == FACTS["nv_head_max"]["value"]
    assert 2048 * 24 == FACTS["row_head_pairs_2048_rows"]["value"]


def test_quant_rows_roundtrip_and_bound():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((50, 128)).astype(np.float32) * 3
    inv = np.float32(6.0 / np.abs(X).max())
    codes, scales = O.quant_rows(X, inv)
    xn = np.clip((X * inv).astype(np.float32), -6, 6).astype(np.float64)
    for r in range(50):
        for b in range(4):
            e = int(scales[r, b]) - 127
            blk = xn[r, 32 * b:32 * b + 32]
            assert e == O.e8m0_exp(float(np.abs(blk).max()))
            for i in range(32):
                byte = codes[r, (32 * b + i) // 2]
                c = (byte >> 4) if (i & 1) else (byte & 15)
                want = nearest_even(blk[i] / 2.0 ** e)
                assert (c & 7) == want
                assert bool(c & 8) == bool(np.signbit(blk[i]))
    # representable values round-trip exactly
    Y = np.array([[v * s for v in [0, .5, 1, 1.5, 2, 3, 4, 6] * 4 for s in (1,)]], np.float32)
    c2, s2 = O.quant_rows(Y, 1.0)
    assert s2[0, 0] == 127
    vals = [O.e2m1_value((c2[0, i // 2] >> (4 * (i & 1))) & 15) for i in range(32)]
    assert np.array_equal(vals, Y[0])


def test_quant_rows2_first_term_and_residual_by_nearest_search():
    # two-term quantisation ("Second hunt"): the first term is the one-term
    # quantisation; the second is the nearest-value quantisation of the FP32
    # residual x' - Q1 with its own block exponent; the residual error never
    # grows and stays within half the coarsest E2M1 step of the second scale
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((40, 128)) * np.exp(rng.standard_normal((40, 1)))).astype(np.float32)
    X[3, :32] = 0.0                       # an all-zero block
    inv = np.float32(6.0 / np.abs(X).max())
    L = O.lib()
    c1 = np.zeros((40, 64), np.uint8)
    s1 = np.zeros((40, 4), np.uint8)
    c2, s2 = np.zeros_like(c1), np.zeros_like(s1)
    L.orc_quant_rows2(O._ptr(X), 40, 128, C.c_float(inv), O.MX, O._ptr(c1), O._ptr(s1),
                      O._ptr(c2), O._ptr(s2))
    r1c, r1s = O.quant_rows(X, inv)
    assert np.array_equal(c1, r1c) and np.array_equal(s1, r1s)

    def deq(c, sb):
        lo, hi = c & 15, c >> 4
        codes = np.stack([lo, hi], -1).reshape(c.shape[0], -1)
        sign = np.where(codes & 8, -1.0, 1.0)
        scale = np.ldexp(1.0, sb.astype(np.int64) - 127).repeat(32, axis=1)
        return sign * MAGS[codes & 7] * scale

    xn = np.clip((X * inv).astype(np.float32), -6, 6)
    d1 = deq(c1, s1)
    res = (xn.astype(np.float64) - d1).astype(np.float32)
    assert np.array_equal(deq(c2, s2), quantise_blocks(res))
    err1 = np.abs(xn - d1)
    err2 = np.abs(xn - d1 - deq(c2, s2))
    assert np.all(err2 <= err1)
    step2 = np.ldexp(1.0, s2.astype(np.int64) - 127).repeat(32, axis=1)
    assert np.all(err2 <= step2 + 0.0)
    assert np.all(c2[3, :16] == 0) and np.all(s2[3, 0] == 0)   # E8M0 floor 2^-127
    assert np.all(deq(c2, s2)[res == 0] == 0)
    assert err2.mean() < 0.2 * err1.mean()


def test_k_least_squares_block_exponents():
    # "Second hunt": each K block scale is the candidate with the smallest
    # squared error.  Candidates e (no clipping), e-1, e+1; the oracle's pick
    # has the smallest FP64 error up to FP32 rounding of the error sums, its
    # codes are the nearest-value codes at that exponent, and the search
    # lowers the total error against the nearest rule
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((64, 128)) ** 3).astype(np.float32)  # heavy tails
    inv = np.float32(6.0 / np.abs(X).max())
    L = O.lib()
    c = np.zeros((64, 64), np.uint8)
    s = np.zeros((64, 4), np.uint8)
    L.orc_quant_rows_lsq(O._ptr(X), 64, 128, None, C.c_float(inv), O._ptr(c), O._ptr(s))
    cn, sn = O.quant_rows(X, inv)
    xn = np.clip((X * inv).astype(np.float32), -6, 6).astype(np.float64).reshape(64, 4, 32)

    def sse(e):
        sc = np.ldexp(1.0, e)[..., None]
        codes = np.array([[[nearest_even(v) for v in blk] for blk in row] for row in xn / sc])
        q = np.sign(xn) * MAGS[codes] * sc
        return ((xn - q) ** 2).sum(-1), q

    e0 = sn.astype(np.int64) - 127
    errs = {d: sse(e0 + d)[0] for d in (-1, 0, 1)}
    best = np.minimum(np.minimum(errs[-1], errs[0]), errs[1])
    el = s.astype(np.int64) - 127
    assert set(np.unique(el - e0)) <= {-1, 0, 1}
    got = np.choose(el - e0 + 1, [errs[-1], errs[0], errs[1]])
    assert np.all(got <= best * (1 + 1e-5) + 1e-30)
    assert (el != e0).any() and (el == e0).any()
    _, q = sse(el)
    lo, hi = c & 15, c >> 4
    codes = np.stack([lo, hi], -1).reshape(64, 4, 32)
    dq = np.where(codes & 8, -1.0, 1.0) * MAGS[codes & 7] * np.ldexp(1.0, el)[..., None]
    assert np.array_equal(dq, q)
    assert got.sum() < errs[0].sum()
