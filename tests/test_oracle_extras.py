"""Pins of the oracle's remaining parts, each against something other than the
oracle itself:

* the per-cell margin max_r (l_r - eps lambda_r) / lambda_r against the
  frame-free brute force's own l and lambda (bitwise: the ratio does not
  depend on the frame);
* the key mean against an exactly rounded sum (math.fsum) of the keys in a
  shuffled order, for fp16 and bf16 inputs ("What else is in the box": fixed
  reduction order -- for these inputs every order gives the same value);
* the FP64 reports (true share of each cold tile, hot/cold split of the
  reference output, "Pass 1" on safe cold verdicts and "The bug") against an
  independent numpy softmax, closed forms (shares sum to 1, parts sum to the
  reference) and the eps limits;
* the per-operand emulation ("Second hunt: which operand is to blame"):
  every switch on is the oracle itself, each single operand against the brute
  force with only that operand quantised, all off against FP64 attention;
* the sliding window ("What else is in the box") against the brute force and
  a masked numpy softmax;
* the value-norm weighted hot test ("Honest limits", mass versus output)
  against the brute force (norms by numpy's norm routine), the closed forms
  of equal norms (every weight 1: the mass test itself) and of one planted
  tile, the output-norm bound it promises, and its effect on the error;
* NVFP4 pass 1 against the brute force's own NV quantisation.
"""
import math

import numpy as np
import pytest

from brute_apa import MAGS, brute_apa, nearest_mag_code
from mixed_precision_long_amd.inputs import outlier_value_tiles, make_inputs, small_workload
from oracle import oracle as O


def _frame_scale(m):
    return np.where(np.isfinite(m), np.exp2(np.where(np.isfinite(m), m, 0.0)), 0.0)


# ---------------------------------------------------------------------------
# margin
# ---------------------------------------------------------------------------

MARGIN_CASES = [  # Hq, Hkv, Nq, Nkv, D, eps, causal, seed, window
    (2, 1, 256, 1024, 64, 0.005, 1, 1, 0),
    (2, 1, 100, 700, 64, 0.05, 1, 2, 0),
    (4, 2, 37, 300, 32, 0.02, 1, 3, 0),
    (2, 2, 64, 200, 64, 0.1, 0, 4, 0),
    (2, 1, 64, 1024, 64, 1.0, 1, 6, 0),
    (2, 1, 96, 2048, 64, 0.02, 1, 41, 300),
]


@pytest.mark.parametrize("case", MARGIN_CASES)
def test_margin_matches_brute_force(case):
    """The oracle's margin of every visited cell is the brute force's, bit for
    bit; a slip such as judging against lambda before the current tile, or
    against another row's sum, changes it."""
    Hq, Hkv, Nq, Nkv, D, eps, causal, seed, window = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed, causal=causal)
    Q, K, V = make_inputs(w)
    p = O.Params(1, Hq, Hkv, Nq, Nkv, D, causal=causal, scale=w.scale, eps=eps, window=window)
    r = O.run(p, Q, K, V, pass2=False)
    b = brute_apa(Q, K, V, eps, w.scale, bool(causal), window=window)
    om, bm = r["margin"][0], b["margin"]
    assert np.array_equal(np.isnan(om), np.isnan(bm))
    vis = ~np.isnan(om)
    assert vis.any()
    assert np.array_equal(om[vis], bm[vis])
    # the margin decides the verdict: hot exactly where it is positive
    # (eps = 0 aside, which marks every visited cell hot)
    assert np.array_equal(om[vis] > 0, r["hot"][0][vis].astype(bool))


def test_margin_is_not_the_previous_lambda():
    """A plausible slip -- the margin against lambda before the current tile
    -- gives different values on these inputs, so the pin above can see it."""
    w = small_workload(1, 2, 1, 64, 1024, 64, seed=1)
    Q, K, V = make_inputs(w)
    b = brute_apa(Q, K, V, 0.02, w.scale)
    r = O.run(O.Params(1, 2, 1, 64, 1024, 64, scale=w.scale, eps=0.02), Q, K, V, pass2=False)
    vis = ~np.isnan(r["margin"][0])
    # on the first visited tile the margin is 1 - eps exactly (l = lambda)
    first = r["margin"][0][..., 0]
    assert np.all(first == (1.0 - np.float64(np.float32(0.02))))
    assert vis.sum() > 10 and np.array_equal(r["margin"][0][vis], b["margin"][vis])


# ---------------------------------------------------------------------------
# key mean
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,mode", [("fp16", "path"), ("bf16", "gauss"), ("fp16", "gauss")])
def test_key_mean_is_order_free(dtype, mode):
    """k-bar equals fl32(S / Nkv) with S the exactly rounded sum of the keys
    (math.fsum over a shuffled order), for every channel: for these inputs
    every partial sum is exact in FP64, so the oracle's fixed order (keys in a
    tile, tiles in a chunk, chunks) and any other give the same value."""
    w = small_workload(1, 2, 2, 64, 5000, 64, dtype=dtype, mode=mode, seed=17)
    _, K, _ = make_inputs(w)
    rng = np.random.default_rng(0)
    for hk in range(2):
        Kh = np.ascontiguousarray(K[0, hk])
        kb = np.zeros(64, np.float32)
        am = np.zeros(1, np.float32)
        O.lib().orc_key_stats(O._ptr(Kh), Kh.shape[0], 64, 64, O._ptr(kb), O._ptr(am))
        perm = rng.permutation(Kh.shape[0])
        for d in range(64):
            s = math.fsum(float(x) for x in Kh[perm, d])
            assert kb[d] == np.float32(s / Kh.shape[0]), (hk, d)
            # exactness of the FP64 running sum in the survey's plain ascending order
            acc = 0.0
            for x in Kh[:, d]:
                acc += float(x)
            assert acc == s
        # amax: the largest |K - kbar| over the head, from the FP32 differences
        assert am[0] == np.abs((Kh - kb[None, :]).astype(np.float32)).max()


# ---------------------------------------------------------------------------
# FP64 reports
# ---------------------------------------------------------------------------

def _numpy_reports(p, Q, K, V, hot, rows):
    """Softmax shares and output parts from a numpy FP64 matrix product."""
    G = p.Hq // p.Hkv
    scale = p.scale if p.scale > 0 else 1.0 / np.sqrt(p.D)
    out = []
    for b, h, r in rows:
        q = Q[b, h, r].astype(np.float64)
        Kh = K[b, h // G].astype(np.float64)
        Vh = V[b, h // G].astype(np.float64)
        keys = np.arange(p.Nkv)
        vis = keys <= r + p.Nkv - p.Nq if p.causal else np.ones(p.Nkv, bool)
        if p.window > 0:
            vis &= keys > r + p.Nkv - p.Nq - p.window
        s = np.where(vis, scale * (Kh @ q), -np.inf)
        wgt = np.exp(s - s.max())
        wgt /= wgt.sum()
        tiles = np.zeros(p.n_tiles)
        np.add.at(tiles, keys // 64, wgt)
        hk = hot[b, h, r // 16].astype(bool)
        keyhot = hk[keys // 64]
        cold_tiles = np.where(hk, -1.0, tiles)
        out.append(dict(hot_share=tiles[hk].sum(), cold_share=tiles[~hk].sum(),
                        cold_tile_max=max(0.0, cold_tiles.max()),
                        O_hot=(wgt[keyhot, None] * Vh[keyhot]).sum(0),
                        O_cold=(wgt[~keyhot, None] * Vh[~keyhot]).sum(0)))
    return out


@pytest.mark.parametrize("eps,window", [(0.02, 0), (0.005, 0), (0.05, 200)])
def test_reports_against_numpy_softmax(eps, window):
    w = small_workload(1, 4, 2, 96, 1500, 64, seed=23)
    Q, K, V = make_inputs(w)
    p = O.Params(1, 4, 2, 96, 1500, 64, scale=w.scale, eps=eps, window=window)
    r = O.run(p, Q, K, V, pass2=True)
    rows = np.array([(0, h, rr) for h in range(4) for rr in (0, 17, 50, 95)], np.int32)
    rep = O.reports(p, Q, K, V, r["hot"], rows)
    ref = _numpy_reports(p, Q, K, V, r["hot"], rows)
    Oe, lse = O.exact(p, Q, K, V, rows=rows)
    for i, x in enumerate(ref):
        for k in ("hot_share", "cold_share", "cold_tile_max"):
            assert abs(rep[k][i] - x[k]) <= 1e-12, (k, rep[k][i], x[k])
        assert np.abs(rep["O_hot"][i] - x["O_hot"]).max() <= 1e-12
        assert np.abs(rep["O_cold"][i] - x["O_cold"]).max() <= 1e-12
    # closed forms: the shares cover the row's mass, the parts its output
    assert np.abs(rep["hot_share"] + rep["cold_share"] - 1.0).max() <= 1e-12
    assert np.abs(rep["O_hot"] + rep["O_cold"] - rep["O_ref"]).max() <= 1e-12
    assert np.abs(rep["O_ref"] - Oe).max() <= 1e-12 and np.abs(rep["lse"] - lse).max() <= 1e-12
    # the largest cold tile is one of the cold tiles, and holds cold_tile_max
    for i, (b, h, rr) in enumerate(rows):
        t = rep["cold_tile_arg"][i]
        if t >= 0:
            assert not r["hot"][b, h, rr // 16, t]


def test_reports_eps_limits():
    w = small_workload(1, 2, 1, 64, 800, 64, seed=24)
    Q, K, V = make_inputs(w)
    rows = np.array([(0, h, rr) for h in range(2) for rr in range(0, 64, 7)], np.int32)
    p0 = O.Params(1, 2, 1, 64, 800, 64, scale=w.scale, eps=0.0)
    r0 = O.run(p0, Q, K, V, pass2=False)
    rep0 = O.reports(p0, Q, K, V, r0["hot"], rows)
    # eps = 0: every visited tile hot, nothing of the mass or output is cold
    assert np.all(rep0["cold_share"] == 0.0) and np.all(rep0["cold_tile_arg"] == -1)
    assert np.array_equal(rep0["O_hot"], rep0["O_ref"])
    p1 = O.Params(1, 2, 1, 64, 800, 64, scale=w.scale, eps=1.0)
    r1 = O.run(p1, Q, K, V, pass2=False)
    rep1 = O.reports(p1, Q, K, V, r1["hot"], rows)
    # eps = 1: nothing hot, the whole output is cold
    assert np.all(rep1["hot_share"] == 0.0)
    assert np.array_equal(rep1["O_cold"], rep1["O_ref"])


def test_cold_tiles_true_share_near_eps():
    """The page's observation in numbers: the bound on a cold tile is on its
    FP4 mass, so its true FP64 share can exceed eps somewhat (0.0118 at
    eps = 0.005 on the page's dumps), but stays of the order of eps."""
    w = small_workload(1, 4, 1, 128, 8192, 64, seed=25)
    Q, K, V = make_inputs(w)
    p = O.Params(1, 4, 1, 128, 8192, 64, scale=w.scale, eps=0.005)
    r = O.run(p, Q, K, V, pass2=False)
    rep = O.reports(p, Q, K, V, r["hot"])
    assert rep["cold_tile_max"].max() < 10 * 0.005
    assert rep["cold_share"].max() > 0.0


def test_compare_rows():
    a = np.array([[1.0, 0.0], [0.0, 0.0], [0.0, 0.0], [3.0, 4.0]])
    b = np.array([[2.0, 0.0], [0.0, 0.0], [1.0, 0.0], [3.0, 4.0]])
    c = O.compare_rows(a, b)
    assert list(c["cos"]) == [1.0, 1.0, -1.0, 1.0]
    assert c["max_abs"] == 1.0 and abs(c["mse"] - 2.0 / 8) < 1e-15


# ---------------------------------------------------------------------------
# per-operand emulation
# ---------------------------------------------------------------------------

QUANT_LETTERS = {"Q": O.QUANT_Q, "K": O.QUANT_K, "V": O.QUANT_V, "P": O.QUANT_P}


def test_all_switches_on_is_the_oracle():
    w = small_workload(1, 2, 1, 100, 700, 64, seed=2)
    Q, K, V = make_inputs(w)
    a = O.run(O.Params(1, 2, 1, 100, 700, 64, scale=w.scale, eps=0.05), Q, K, V)
    b = O.run(O.Params(1, 2, 1, 100, 700, 64, scale=w.scale, eps=0.05, qmask=O.QUANT_ALL), Q, K,
              V)
    for k in ("hot", "m1", "l1", "lam", "o1", "O", "lse"):
        assert np.array_equal(np.nan_to_num(a[k]), np.nan_to_num(b[k])), k


@pytest.mark.parametrize("only", ["Q", "K", "V", "P", "QKVP", ""])
@pytest.mark.parametrize("case", [(2, 1, 100, 700, 64, 0.05, 2), (4, 2, 64, 1024, 64, 0.01, 5)])
def test_single_operand_emulation_matches_brute_force(only, case):
    """Pass 1 with only the named operands quantised, against the frame-free
    brute force with the same operands quantised (exact operands there are
    the same normalised values): the same verdicts wherever the margin is not
    within rounding of the threshold, and the same state to FP32 rounding
    (the brute force takes its FP64 sums and exp2 in another order)."""
    Hq, Hkv, Nq, Nkv, D, eps, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed)
    Q, K, V = make_inputs(w)
    mask = sum(QUANT_LETTERS[c] for c in only)
    p = O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, qmask=mask)
    r = O.run(p, Q, K, V, pass2=False)
    b = brute_apa(Q, K, V, eps, w.scale, quant=only)
    sc = _frame_scale(r["m1"][0])
    near = np.abs(r["margin"][0]) <= 1e-6
    assert np.array_equal(r["hot"][0].astype(bool)[~near], b["hot"][~near])
    exact_bits = only == "QKVP"
    for key, got in (("l", r["l1"][0] * sc), ("lam", r["lam"][0] * sc),
                     ("o", r["o1"][0] * sc[..., None])):
        want = b[key]
        if exact_bits:
            assert np.array_equal(got.astype(np.float32), want), key
        else:
            tol = 4e-7 * np.abs(want).max()
            assert np.abs(got - want).max() <= tol, (key, np.abs(got - want).max(), tol)


@pytest.mark.parametrize("eps", [0.0, 0.005, 0.05, 1.0])
def test_all_operands_exact_is_fp64_attention(eps):
    """With no FP4 rounding at all, pass 1's cold state plus pass 2 and the
    merge give exact attention for any eps, up to the FP32 scores and state
    (about 1e-7 relative per operation): within 1e-6 on unit-scale outputs."""
    w = small_workload(1, 4, 2, 96, 1500, 64, seed=26)
    Q, K, V = make_inputs(w)
    p = O.Params(1, 4, 2, 96, 1500, 64, scale=w.scale, eps=eps, qmask=0)
    r = O.run(p, Q, K, V)
    Oe, lse = O.exact(p, Q, K, V)
    err = np.abs(r["O"].reshape(-1, 64) - Oe).max()
    assert err <= 1e-6, err
    assert np.abs(r["lse"].reshape(-1) - lse).max() <= 1e-6


def test_emulation_finds_the_operand():
    """The page's use of the emulation: quantising one operand at a time
    shows which rounding moves the output most.  On these inputs each single
    operand's error is below that of all four together, and the sum of the
    four single errors is of the order of the full error."""
    w = small_workload(1, 2, 1, 128, 4096, 64, seed=27)
    Q, K, V = make_inputs(w)
    Oe, _ = O.exact(O.Params(1, 2, 1, 128, 4096, 64, scale=w.scale), Q, K, V)
    err = {}
    for only in ("", "Q", "K", "V", "P", "QKVP"):
        mask = sum(QUANT_LETTERS[c] for c in only)
        p = O.Params(1, 2, 1, 128, 4096, 64, scale=w.scale, eps=1.0, qmask=mask)
        r = O.run(p, Q, K, V)
        err[only] = np.sqrt(((r["O"].reshape(-1, 64) - Oe) ** 2).mean())
    assert err[""] < 1e-6
    for c in "QKVP":
        assert err[""] < err[c] < err["QKVP"] * 1.5, err
    singles = sum(err[c] for c in "QKVP")
    assert 0.5 * err["QKVP"] < singles < 4 * err["QKVP"], err


# ---------------------------------------------------------------------------
# sliding window
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", [
    (2, 1, 96, 2048, 64, 0.02, 300, 41),   # window inside the keys: no sink
    (2, 1, 128, 128, 64, 0.05, 64, 42),    # self-attention
    (4, 2, 64, 1000, 64, 0.01, 700, 43),   # window reaching tile 0 for early rows
])
def test_window_pass1_bitwise_vs_brute_force(case):
    Hq, Hkv, Nq, Nkv, D, eps, window, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed)
    Q, K, V = make_inputs(w)
    p = O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, window=window)
    r = O.run(p, Q, K, V, pass2=False)
    b = brute_apa(Q, K, V, eps, w.scale, window=window)
    sc = _frame_scale(r["m1"][0])
    assert np.array_equal(r["hot"][0].astype(bool), b["hot"])
    assert np.array_equal((r["l1"][0] * sc).astype(np.float32), b["l"])
    assert np.array_equal((r["lam"][0] * sc).astype(np.float32), b["lam"])
    assert np.array_equal((r["o1"][0] * sc[..., None]).astype(np.float32), b["o"])


def test_window_exact_and_eps0():
    """The window's exact attention against a masked numpy softmax, and at
    eps = 0 the windowed APA output equals it (every visited tile exact)."""
    w = small_workload(1, 2, 1, 96, 2048, 64, seed=44)
    Q, K, V = make_inputs(w)
    p = O.Params(1, 2, 1, 96, 2048, 64, scale=w.scale, eps=0.0, window=500)
    Oe, _ = O.exact(p, Q, K, V)
    rows = [(0, h, r) for h in range(2) for r in range(96)]
    hot = np.ones((1, 2, 6, 32), np.uint8)
    ref = _numpy_reports(p, Q, K, V, hot, rows)
    for i, x in enumerate(ref):
        assert np.abs(x["O_hot"] - Oe[i]).max() <= 1e-12
    r = O.run(p, Q, K, V)
    # pass 2 scores in log2 units with sl = fl32(scale * fl32(log2 e)): about
    # 1e-8 relative on the scores, below 1e-7 on these outputs
    assert np.abs(r["O"].reshape(-1, 64) - Oe).max() <= 1e-7
    # keys outside every row's window are never hot
    assert not r["hot"][..., :(2048 - 96 - 500) // 64].any()


# ---------------------------------------------------------------------------
# value-norm weighted hot test
# ---------------------------------------------------------------------------

def _same_norm_values(V, seed):
    """Every key's value a signed permutation of one vector with entries in
    [0.5, 2): all key norms are equal, and their FP64 squares and sums are
    exact."""
    rng = np.random.default_rng(seed)
    B, Hkv, Nkv, D = V.shape
    u = np.float16(rng.uniform(0.5, 2.0, D)).astype(np.float32)
    out = np.empty_like(V)
    for b in range(B):
        for j in range(Hkv):
            for k in range(Nkv):
                out[b, j, k] = rng.permutation(u) * rng.choice([-1.0, 1.0], D)
    return out


@pytest.mark.parametrize("case", [
    (2, 1, 128, 2048, 64, 0.02, 0, 3, 4.0, 61),
    (4, 2, 100, 1300, 64, 0.05, 0, 2, 8.0, 62),
    (2, 1, 96, 2048, 64, 0.05, 300, 3, 16.0, 71),  # with a sliding window
])
def test_hot_weight_pass1_bitwise_vs_brute_force(case):
    """The weighted hot test against the brute force, which takes its norms
    with numpy's own norm routine: weights, verdicts, margins and the cold
    state agree bit for bit."""
    Hq, Hkv, Nq, Nkv, D, eps, window, nb, factor, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed)
    Q, K, V = make_inputs(w)
    p = O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, window=window, hot_weight=1)
    outlier_value_tiles(V, nb, factor, seed=seed, first_tile=p.first_tile)
    prep = O.quantize(p, Q, K, V)
    r = O.run(p, Q, K, V, prep, pass2=False)
    b = brute_apa(Q, K, V, eps, w.scale, window=window, hot_weight=True)
    for j in range(Hkv):
        assert np.array_equal(prep["vw"][0, j], b["ops"][j]["vw"])
    assert (prep["vw"] > 1.0).any()
    sc = _frame_scale(r["m1"][0])
    assert np.array_equal(r["hot"][0].astype(bool), b["hot"])
    om, bm = r["margin"][0], b["margin"]
    vis = ~np.isnan(om)
    assert np.array_equal(vis, ~np.isnan(bm)) and np.array_equal(om[vis], bm[vis])
    assert np.array_equal((r["l1"][0] * sc).astype(np.float32), b["l"])
    assert np.array_equal((r["o1"][0] * sc[..., None]).astype(np.float32), b["o"])
    # and the weights change verdicts on these inputs
    r0 = O.run(O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, window=window),
               Q, K, V, pass2=False)
    assert r["hot"].sum() > r0["hot"].sum()


def test_hot_weight_equal_norms_is_the_mass_test():
    """With every key's value norm equal, every weight is exactly 1 and the
    weighted run is the unweighted one, bit for bit."""
    w = small_workload(1, 2, 1, 128, 2048, 64, seed=64)
    Q, K, V = make_inputs(w)
    V = _same_norm_values(V, 64)
    p0 = O.Params(1, 2, 1, 128, 2048, 64, scale=w.scale, eps=0.01)
    p1 = O.Params(1, 2, 1, 128, 2048, 64, scale=w.scale, eps=0.01, hot_weight=1)
    prep = O.quantize(p1, Q, K, V)
    assert np.all(prep["vw"] == 1.0)
    r0 = O.run(p0, Q, K, V)
    r1 = O.run(p1, Q, K, V, prep)
    for k in ("hot", "margin", "l1", "o1", "m1", "O"):
        assert np.array_equal(r0[k], r1[k], equal_nan=True), k


def test_hot_weight_planted_tile_closed_form():
    """Equal norms nu everywhere except one tile whose values are 2^j times
    larger: nu_bar = nu (n - 64 + 64 2^j) / n, so that tile's weight is
    fl32(2^j n / (n - 64 + 64 2^j)) and every other weight is 1."""
    Nkv, t_big, j = 2048, 9, 3
    w = small_workload(1, 2, 1, 64, Nkv, 64, seed=65)
    Q, K, V = make_inputs(w)
    V = _same_norm_values(V, 65)
    V[0, 0, 64 * t_big:64 * t_big + 64] *= np.float32(2.0 ** j)
    p = O.Params(1, 2, 1, 64, Nkv, 64, scale=w.scale, hot_weight=1)
    prep = O.quantize(p, Q, K, V)
    want = np.ones(Nkv // 64, np.float32)
    want[t_big] = np.float32(2.0 ** j * Nkv / (Nkv - 64 + 64 * 2.0 ** j))
    assert np.array_equal(prep["vw"][0, 0], want)


@pytest.mark.parametrize("eps", [0.005, 0.02])
def test_hot_weight_bounds_cold_output_norm(eps):
    """The bound the weighted test gives: for every cold cell, the FP4 mass of
    each row times the tile's largest value norm stays under eps * lambda *
    nu_bar (lambda final, so at least what the vote saw); the norms here are
    recomputed independently."""
    Nq, Nkv = 128, 8192
    w = small_workload(1, 2, 1, Nq, Nkv, 64, seed=66)
    Q, K, V = make_inputs(w)
    outlier_value_tiles(V, 4, 8.0, seed=66)
    b = brute_apa(Q, K, V, eps, w.scale, hot_weight=True)
    nu = np.linalg.norm(V[0, 0].astype(np.float64), axis=1)
    nbar = nu.mean()
    ops = b["ops"][0]
    off = Nkv - Nq
    checked = 0
    for h in range(2):
        hd = ops["heads"][h]
        s = (hd["alpha"] * (hd["qd"] @ ops["kd"].T)).astype(np.float32).astype(np.float64)
        for g in range(Nq // 16):
            rows = np.arange(16 * g, 16 * g + 16)
            lam = b["lam"][h, rows].astype(np.float64)
            for t in np.flatnonzero(~b["hot"][h, g]):
                if 64 * t > rows[-1] + off:
                    continue
                st = s[rows, 64 * t:64 * t + 64].copy()
                st[np.arange(64 * t, 64 * t + 64)[None, :] > rows[:, None] + off] = -np.inf
                mass = np.zeros(16)
                for q0 in (0, 32):
                    gg = st[:, q0:q0 + 32]
                    cg = gg.max(1)
                    live = np.isfinite(cg)
                    cg = np.where(live, cg, 0.0)
                    E = np.ceil(cg - np.log2(6.0))
                    E = np.where(np.exp2(cg - E) > 6, E + 1, E)
                    E = np.where(np.exp2(cg - E + 1) <= 6, E - 1, E)
                    with np.errstate(invalid="ignore"):
                        pq = MAGS[nearest_mag_code(np.exp2(gg - E[:, None]))]
                    pq = np.where(np.isfinite(gg), pq, 0.0)
                    mass += np.where(live, (pq * np.exp2(E)[:, None]).sum(1), 0.0)
                numax = nu[64 * t:64 * t + 64].max()
                assert np.all(mass * numax <= eps * lam * nbar * (1 + 1e-6)), (h, g, t)
                assert np.all(mass <= eps * lam * (1 + 1e-6))
                checked += 1
    assert checked > 100


def test_hot_weight_lowers_the_error_of_large_value_tiles():
    """On inputs with tiles of outsized values the weighted test makes more
    tiles exact and brings the output closer to FP64 attention (an inverted
    weight, or one applied to lambda instead of the tile, would not)."""
    Nq, Nkv = 128, 4096
    w = small_workload(1, 4, 1, Nq, Nkv, 64, seed=67)
    Q, K, V = make_inputs(w)
    outlier_value_tiles(V, 6, 16.0, seed=67)
    Oe, _ = O.exact(O.Params(1, 4, 1, Nq, Nkv, 64, scale=w.scale), Q, K, V)
    err, nhot = {}, {}
    for hw in (0, 1):
        p = O.Params(1, 4, 1, Nq, Nkv, 64, scale=w.scale, eps=0.02, hot_weight=hw)
        r = O.run(p, Q, K, V)
        err[hw] = np.abs(r["O"].reshape(-1, 64) - Oe.reshape(-1, 64)).max()
        nhot[hw] = int(r["hot"].sum())
    assert nhot[1] > nhot[0]
    assert err[1] < 0.7 * err[0], err


# ---------------------------------------------------------------------------
# NVFP4 pass 1 (the page's own format; an oracle option)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("eps,seed", [(0.03, 81), (0.1, 82)])
def test_nv_pass1_bitwise_vs_brute_force_on_flat_scores(eps, seed):
    """NVFP4 mode ("Pass 1: FP4 everywhere, with a hot test": UE4M3 scales per
    16 elements, per-head scales to 6 x 448, P in 16-key groups) against the
    brute force's own NV quantisation (UE4M3 values built from the format's
    bit layout, nearest search; P scales rounded to 4 significant bits with
    no exponent limit).  Frame-free agreement needs every P group scale
    inside UE4M3's normal range in the oracle's frame: with scores spanning
    less than 2.4 log2 units no group maximum falls more than 3.4 below the
    frame, so the 2^-6 floor never binds (checked below); the floor itself is
    pinned by the sink-bug test."""
    Nkv = 3000
    w = small_workload(1, 2, 1, 96, Nkv, 64, mode="gauss", delta=0.0, seed=seed)
    Q, K, V = make_inputs(w)
    scale = 0.03
    p = O.Params(1, 2, 1, 96, Nkv, 64, scale=scale, eps=eps, fmt=O.NV)
    r = O.run(p, Q, K, V, pass2=False)
    b = brute_apa(Q, K, V, eps, scale, fmt="NV")
    ops = b["ops"][0]
    off = Nkv - 96
    for h in range(2):
        hd = ops["heads"][h]
        s = (hd["alpha"] * (hd["qd"] @ ops["kd"].T)).astype(np.float32).astype(np.float64)
        vis = np.arange(Nkv)[None, :] <= np.arange(96)[:, None] + off
        sv = np.where(vis, s, -np.inf)
        smax = sv.max()
        # the smallest maximum of any 16-key group of any row that sees one
        pad = -(-Nkv // 16) * 16 - Nkv
        gmax = np.pad(sv, ((0, 0), (0, pad)), constant_values=-np.inf).reshape(96, -1, 16).max(2)
        gm = gmax[np.isfinite(gmax)].min()
        assert smax + 1.0 - gm < 3.4, (smax, gm)
    sc = _frame_scale(r["m1"][0])
    assert np.array_equal(r["hot"][0].astype(bool), b["hot"])
    assert 0 < b["hot"].sum() < (~np.isnan(r["margin"][0])).sum()
    assert np.array_equal((r["l1"][0] * sc).astype(np.float32), b["l"])
    assert np.array_equal((r["lam"][0] * sc).astype(np.float32), b["lam"])
    assert np.array_equal((r["o1"][0] * sc[..., None]).astype(np.float32), b["o"])


@pytest.mark.parametrize("case", [
    (8, 2, 128, 32768, 128, "path", 11, 0.005),
    (8, 2, 128, 32768, 128, "gauss", 12, 0.005),
    (4, 1, 64, 16384, 256, "path", 14, 0.02),
], ids=["path_D128", "gauss_D128", "path_D256_eps0.02"])
def test_tied_q_scale_costs_no_accuracy(case):
    """Ablation of the tied Q scale (Q normalised so that the score factor is
    a power of two) against Q at a head scale of its own (6 / max|Q|, like
    K's): at long contexts, where most tiles are cold, the APA output's
    distance from FP64 attention and the hot share are the same within the
    spread of the inputs.  (A mis-scaled Q in either form shows as a many-fold
    larger error.)"""
    Hq, Hkv, Nq, Nkv, D, mode, seed, eps = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, mode=mode, seed=seed)
    Q, K, V = make_inputs(w)
    Oe, _ = O.exact(O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale), Q, K, V)
    e = Oe.reshape(-1, D)
    res = {}
    for qs in ("tied", "own"):
        p = O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, q_scale=qs)
        r = O.run(p, Q, K, V, O.quantize(p, Q, K, V))
        o = r["O"].reshape(-1, D)
        cos = (o * e).sum(1) / (np.linalg.norm(o, axis=1) * np.linalg.norm(e, axis=1))
        vis = ~np.isnan(r["margin"])
        res[qs] = dict(cos_min=cos.min(), cos_med=np.median(cos), mse=((o - e) ** 2).mean(),
                       hot=r["hot"][vis].mean())
    t, o = res["tied"], res["own"]
    print("[tied Q scale]", {k: {kk: float("%.6g" % vv) for kk, vv in v.items()} for k, v in res.items()})
    assert 0.05 < t["hot"] < 0.9  # most tiles are decided, some cold
    assert abs(t["hot"] - o["hot"]) <= 0.02
    assert t["mse"] <= 1.15 * o["mse"] and o["mse"] <= 1.15 * t["mse"]
    assert abs(t["cos_min"] - o["cos_min"]) <= 0.01
    assert abs(t["cos_med"] - o["cos_med"]) <= 2e-4
