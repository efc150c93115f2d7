"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bars (floating point): quantised codes, scales and per-head scales bitwise;
hot masks agree on >= 99.9 % of visited (group, tile) cells with every
mismatch within 1e-3 of the threshold (|l_t - eps*lambda| <= 1e-3 lambda);
APA output cosine >= 0.9999 per (row, head) and max abs <= 2e-3 against the
oracle; apa_exact within 1e-3 max abs of FP64 attention."""
import numpy as np
import pytest

from gpu_util import cosine_rows, problem_for, run_exact_gpu, run_gpu
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import WORKLOADS, make_inputs, small_workload
from oracle import oracle as O

pytestmark = pytest.mark.gpu

MASK_AGREE = 0.999
MASK_MARGIN = 1e-3
COS_MIN = 0.9999
ABS_MAX = 2e-3
EXACT_ABS = 1e-3

# Hq, Hkv, Nq, Nkv, D, eps, causal, seed
CASES = [
    (2, 1, 256, 1024, 64, 0.005, 1, 1),     # the tiny workload (every tile hot)
    (2, 1, 256, 1024, 64, 0.05, 1, 1),      # same inputs, mixed hot/cold
    (6, 2, 200, 1500, 128, 0.02, 1, 2),     # GQA 3, ragged Nq and Nkv
    (8, 2, 64, 4096, 128, 0.01, 1, 3),      # GQA 4, many cold tiles
    (2, 2, 96, 640, 64, 0.05, 0, 4),        # non-causal
    (2, 1, 1, 1000, 64, 0.01, 1, 5),        # a single query row
    (2, 2, 512, 512, 128, 0.02, 1, 6),      # self-attention
    (2, 1, 64, 2048, 256, 0.02, 1, 7),      # D = 256
    (2, 1, 100, 700, 64, 0.0, 1, 8),        # eps = 0: every visited tile hot
    (2, 1, 100, 700, 64, 1.0, 1, 9),        # eps = 1: nothing hot
]


def oracle_for(w, eps, causal, groups=None, q_terms=1, k_lsq=0):
    p = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, causal=causal, scale=w.scale, eps=eps,
                 q_terms=q_terms, k_lsq=k_lsq)
    return p


def check_quant(g, prep, first_tile=0):
    """Codes, scale bytes and per-head scales bitwise.  With a sliding window
    the K/V codes are compared from the first tile some row sees on (the
    library does not write the others; they are never read)."""
    f = g["fp4"]
    assert f["status"] == 0
    cut = {"kc": (2, 64), "ks": (2, 64), "vc": (3, 32), "vs": (3, 2)}
    for k in ("qc", "qs", "kc", "ks", "vc", "vs", "qc2", "qs2"):
        assert (k in f) == (k in prep), k
        if k in f:
            a, b = f[k], prep[k]
            if first_tile and k in cut:
                ax, per = cut[k]
                sl = [slice(None)] * a.ndim
                sl[ax] = slice(first_tile * per, None)
                a, b = a[tuple(sl)], b[tuple(sl)]
            assert np.array_equal(a, b), k
    assert np.array_equal(f["kbar"], prep["kbar"])
    kv = f["kv_head"]
    assert np.array_equal(kv[..., 0], prep["amax_k"])
    assert np.array_equal(kv[..., 2], prep["inv_k"])
    assert np.array_equal(kv[..., 4], prep["g_v"])
    assert np.array_equal(f["q_head"][..., 1], prep["inv_q"])
    assert np.array_equal(f["q_head"][..., 2].astype(np.int32), prep["jq"])


def check_mask(ghot, r, groups=None):
    vis = ~np.isnan(r["margin"])
    if groups is not None:
        sel = np.zeros_like(vis)
        for b, h, gg in groups:
            sel[b, h, gg] = True
        vis &= sel
    ohot = r["hot"].astype(bool)
    mism = vis & (ghot != ohot)
    agree = 1.0 - mism.sum() / max(vis.sum(), 1)
    assert agree >= MASK_AGREE, agree
    if mism.any():
        assert np.all(np.abs(r["margin"][mism]) <= MASK_MARGIN), r["margin"][mism]
    # never hot where the oracle did not visit
    assert not (ghot & ~vis).any() if groups is None else True
    return mism


def check_cold_state(g, r, mism, groups=None):
    """Pass 1's cold state in frame-free units (l 2^m, o / l) on the row groups
    whose verdicts all agree with the oracle's (only the listed groups when
    `groups` is given).  A row that is empty on one side and not on the other
    fails, and so does a wrong total mass (l 2^m is scale-sensitive where the
    per-row cosine of the output is not)."""
    B, Hq, Nq = g["l"].shape
    NG = -(-Nq // 16)
    gm = np.where(g["m"] == np.iinfo(np.int32).min, np.nan, g["m"].astype(np.float64))
    ok_rows = np.zeros((B, Hq, Nq), bool)
    todo = ([(b, h, gg) for b in range(B) for h in range(Hq) for gg in range(NG)]
            if groups is None else [tuple(x) for x in groups])
    for b, h, gg in todo:
        if not mism[b, h, gg].any():
            ok_rows[b, h, 16 * gg:16 * gg + 16] = True
    assert ok_rows.any()
    gl_pos = g["l"] > 0
    ol_pos = np.nan_to_num(r["l1"], nan=0.0) > 0
    assert np.array_equal(gl_pos[ok_rows], ol_pos[ok_rows]), "a cold state is missing or extra"
    both = ok_rows & gl_pos & ol_pos
    if both.any():
        gl = g["l"] * np.exp2(np.nan_to_num(gm))
        ol = r["l1"] * np.exp2(np.nan_to_num(r["m1"]))
        assert np.allclose(gl[both], ol[both], rtol=1e-3), np.abs(gl[both] / ol[both] - 1).max()
        gco = g["o"] / g["l"][..., None]
        oco = r["o1"] / r["l1"][..., None]
        assert np.abs(gco[both] - oco[both]).max() <= 1e-3


def out_tol(base, O, dtype):
    """The bar on the method's arithmetic, plus, for bf16 outputs, the output
    format's own rounding, since the oracle's O is not rounded: RNE to 8
    significant bits moves a value by at most half a unit in the last place,
    which is at most 2^-8 of the value."""
    return base + (2.0 ** -8) * np.abs(O) if dtype == "bf16" else base


def check_output(gout, oO, rows=None, dtype="fp16"):
    if rows is not None:
        gout = gout[rows[:, 0], rows[:, 1], rows[:, 2]]
        oO = oO[rows[:, 0], rows[:, 1], rows[:, 2]]
    cos = cosine_rows(gout, oO)
    assert cos.min() >= COS_MIN, cos.min()
    excess = np.abs(gout - oO) - out_tol(ABS_MAX, oO, dtype)
    assert excess.max() <= 0.0, (np.abs(gout - oO).max(), excess.max())


@pytest.mark.parametrize("case", CASES, ids=lambda c: "Hq%d_Hkv%d_Nq%d_Nkv%d_D%d_eps%g_c%d" % c[:7])
def test_apa_matches_oracle(case):
    Hq, Hkv, Nq, Nkv, D, eps, causal, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed, causal=causal)
    Q, K, V = make_inputs(w)
    po = oracle_for(w, eps, causal)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w), Q, K, V, eps)
    check_quant(g, prep)
    mism = check_mask(g["hot"], r)
    if eps == 0.0:
        assert np.all(g["l"] == 0)
    if eps >= 1.0:
        assert not g["hot"].any()
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"])
    fin = np.isfinite(r["lse"])
    assert np.abs(g["lse"][fin] - r["lse"][fin]).max() <= 2e-3


# the pages' second-hunt fix for Q: a second FP4 term for what the first leaves
# over, sharing its scale; with and without the split pass-1 schedules
@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[3], CASES[4], CASES[7], CASES[8]],
                         ids=["mixed", "gqa3", "gqa4", "noncausal", "d256", "eps0"])
@pytest.mark.parametrize("split", [True, False], ids=["split", "whole"])
def test_two_term_q_matches_oracle(case, split):
    Hq, Hkv, Nq, Nkv, D, eps, causal, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed, causal=causal)
    Q, K, V = make_inputs(w)
    po = oracle_for(w, eps, causal, q_terms=2)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w, q_terms=2), Q, K, V, eps, split=split)
    check_quant(g, prep)
    mism = check_mask(g["hot"], r)
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"])


# the pages' other second-hunt fix: K block exponents by least squared error,
# alone and with two Q terms (the pages' full accuracy configuration)
@pytest.mark.parametrize("case", [CASES[1], CASES[2], CASES[4], CASES[7]],
                         ids=["mixed", "gqa3", "noncausal", "d256"])
@pytest.mark.parametrize("q_terms", [1, 2])
def test_k_lsq_matches_oracle(case, q_terms):
    Hq, Hkv, Nq, Nkv, D, eps, causal, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed, causal=causal)
    Q, K, V = make_inputs(w)
    po = oracle_for(w, eps, causal, q_terms=q_terms, k_lsq=1)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w, q_terms=q_terms, k_lsq=1), Q, K, V, eps)
    check_quant(g, prep)
    mism = check_mask(g["hot"], r)
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"])


def test_two_term_q_long3b_sampled_groups():
    w = WORKLOADS["long3b"]
    Q, K, V = make_inputs(w, threads=16)
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps, q_terms=2)
    g = run_gpu(problem_for(w, q_terms=2), Q, K, V, w.eps, lam=False)
    sel = O.all_groups(po)[np.random.default_rng(5).choice(3072, 6, replace=False)]
    prep = O.quantize(po, Q, K, V)
    check_quant(g, prep)
    r = O.run(po, Q, K, V, prep, groups=sel)
    check_mask(g["hot"], r, groups=sel)
    rows = np.array([(b, h, gg * 16 + i) for b, h, gg in sel for i in range(16)], np.int32)
    check_output(g["out"], r["O"], rows)


@pytest.mark.parametrize("case", [CASES[2], CASES[4], CASES[6]], ids=["gqa3", "noncausal", "self"])
def test_exact_matches_fp64(case):
    Hq, Hkv, Nq, Nkv, D, eps, causal, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed, causal=causal)
    Q, K, V = make_inputs(w)
    po = oracle_for(w, eps, causal)
    Oe, lse = O.exact(po, Q, K, V)
    go, gl = run_exact_gpu(problem_for(w), Q, K, V)
    assert np.abs(go.reshape(-1, D) - Oe).max() <= EXACT_ABS
    assert np.abs(gl.reshape(-1) - lse).max() <= 1e-3


@pytest.mark.parametrize("shape", [(6, 2, 200, 1500, 128), (4, 1, 128, 4096, 128),
                                   (4, 1, 96, 4096, 256)],
                         ids=["one_split", "four_splits", "d256_splits"])
def test_standalone_merge_equals_fused(shape):
    """The fused merge in the pass-2 epilogue (one key split) or in the split
    combine (several) equals pass 2's hot state merged by apa_merge, bit for
    bit."""
    w = small_workload(1, *shape, seed=2)
    Q, K, V = make_inputs(w)
    p = problem_for(w)
    a = run_gpu(p, Q, K, V, 0.02, fused=True)
    b = run_gpu(p, Q, K, V, 0.02, fused=False)
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["lse"], b["lse"])


def test_deterministic_reruns():
    w = small_workload(1, 6, 2, 200, 1500, 128, seed=2)
    Q, K, V = make_inputs(w)
    p = problem_for(w)
    runs = [run_gpu(p, Q, K, V, 0.02) for _ in range(3)]
    for r in runs[1:]:
        for k in ("out", "lse", "m", "l", "o", "hot"):
            assert np.array_equal(np.nan_to_num(r[k]), np.nan_to_num(runs[0][k])), k


_INPUTS = {}


def _workload_inputs(name, delta=None):
    """Full-size inputs of a named workload, generated once per process (the
    parity tests at one shape share them)."""
    key = (name, delta)
    if key not in _INPUTS:
        _INPUTS.clear()
        w = WORKLOADS[name]
        print("[%s] generating inputs (delta %s)" % (name, delta), flush=True)
        Q, K, V = make_inputs(w, delta=delta, threads=16)
        po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps)
        _INPUTS[key] = (Q, K, V, O.quantize(po, Q, K, V))
    return _INPUTS[key]


def _check_groups(name, sel, eps=None, delta=None):
    """The whole path on the GPU at the workload's full size; the oracle on the
    row groups `sel` [n, 3]: codes, masks, cold state, output and LSE."""
    w = WORKLOADS[name]
    eps = w.eps if eps is None else eps
    Q, K, V, prep = _workload_inputs(name, delta)
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=eps)
    g = run_gpu(problem_for(w), Q, K, V, eps, dtype=w.dtype, lam=False)
    check_quant(g, prep)
    r = O.run(po, Q, K, V, prep, groups=sel, nthreads=16)
    mism = check_mask(g["hot"], r, groups=sel)
    check_cold_state(g, r, mism, groups=sel)
    rows = np.array([(b, h, gg * 16 + i) for b, h, gg in sel for i in range(16)
                     if gg * 16 + i < w.Nq], np.int32)
    check_output(g["out"], r["O"], rows, dtype=w.dtype)
    lg = g["lse"][rows[:, 0], rows[:, 1], rows[:, 2]]
    lo = r["lse"][rows[:, 0], rows[:, 1], rows[:, 2]]
    assert np.abs(lg - lo).max() <= 2e-3
    cells = sum(1 for b, h, gg in sel for t in range(r["hot"].shape[-1])
                if not np.isnan(r["margin"][b, h, gg, t]))
    print("[%s eps %g] %d groups, %d cells, %d mask mismatches, hot %.4f" % (
        name, eps, len(sel), cells, int(mism.sum()),
        float(np.mean([r["hot"][b, h, gg].sum() for b, h, gg in sel]))), flush=True)
    return g, r


def _sampled(name, ngroups, seed=0, delta=None):
    w = WORKLOADS[name]
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps)
    allg = O.all_groups(po)
    sel = allg[np.random.default_rng(seed).choice(len(allg), ngroups, replace=False)]
    _check_groups(name, sel, delta=delta)


def test_short3b_sampled_groups():
    _sampled("short3b", 12)


@pytest.mark.parametrize("eps", [0.002, 0.005, 0.02])
def test_long3b_every_group_of_one_kv_head(eps):
    """The headline shape (2048 rows at the tail of 122880 keys, 24 query
    heads over 8) at each of its three eps: every row group of the three
    query heads that share KV head 0 (384 groups, about 0.74 M visited cells)
    -- not a sample ("The bug": a 1 % sample overstates the worst case)."""
    w = WORKLOADS["long3b"]
    G = w.Hq // w.Hkv
    sel = np.array([(0, h, gg) for h in range(G) for gg in range(w.Nq // 16)], np.int32)
    _check_groups("long3b", sel, eps=eps)


@pytest.mark.parametrize("delta", [0.0, 4.0, 8.0, 12.0])
def test_full32k_sampled_groups(delta):
    """Full causal prefill 32768 x 32768 (32 query heads over 8) at each sink
    strength of its sweep, at full size on sampled row groups (the longest
    groups included)."""
    w = WORKLOADS["full32k"]
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps)
    allg = O.all_groups(po)
    rng = np.random.default_rng(int(delta))
    sel = allg[rng.choice(len(allg), 8, replace=False)]
    last = np.array([(0, int(rng.integers(w.Hq)), w.Nq // 16 - 1)], np.int32)
    _check_groups("full32k", np.concatenate([sel, last]), delta=delta)


@pytest.mark.parametrize("delta", [0.0, 4.0, 8.0, 12.0])
def test_full_causal_sink_sweep(delta):
    """The sink-strength sweep of the full causal workload, at 1024 x 1024
    with the same head layout, every row group checked."""
    w = small_workload(1, 32, 8, 1024, 1024, 128, delta=delta, seed=4)
    Q, K, V = make_inputs(w)
    po = oracle_for(w, w.eps, 1)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w), Q, K, V, w.eps)
    check_quant(g, prep)
    check_mask(g["hot"], r)
    check_output(g["out"], r["O"])


# bf16 inputs and the large head dimension: Hq, Hkv, Nq, Nkv, D, eps, seed, dtype, mode
DTYPE_CASES = [
    (8, 2, 100, 700, 128, 0.02, 11, "bf16", "path"),
    (4, 1, 96, 512, 512, 0.005, 12, "bf16", "gauss"),
    (4, 1, 64, 640, 512, 0.02, 13, "fp16", "path"),
    (2, 1, 40, 300, 256, 0.01, 14, "bf16", "gauss"),
]


@pytest.mark.parametrize("case", DTYPE_CASES, ids=lambda c: "%s_%s_D%d_Nq%d_Nkv%d" % (c[7], c[8], c[4], c[2], c[3]))
def test_apa_dtypes_and_large_head_dim(case):
    Hq, Hkv, Nq, Nkv, D, eps, seed, dtype, mode = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, dtype=dtype, mode=mode, seed=seed)
    Q, K, V = make_inputs(w)
    po = oracle_for(w, eps, 1)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w), Q, K, V, eps, dtype=dtype)
    check_quant(g, prep)
    check_mask(g["hot"], r)
    check_output(g["out"], r["O"], dtype=dtype)
    fin = np.isfinite(r["lse"])
    assert np.abs(g["lse"][fin] - r["lse"][fin]).max() <= 2e-3


@pytest.mark.parametrize("case", DTYPE_CASES, ids=lambda c: "%s_%s_D%d" % (c[7], c[8], c[4]))
def test_exact_dtypes_and_large_head_dim(case):
    Hq, Hkv, Nq, Nkv, D, eps, seed, dtype, mode = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, dtype=dtype, mode=mode, seed=seed)
    Q, K, V = make_inputs(w)
    po = oracle_for(w, eps, 1)
    Oe, lse = O.exact(po, Q, K, V)
    go, gl = run_exact_gpu(problem_for(w), Q, K, V, dtype=dtype)
    excess = np.abs(go.reshape(-1, D) - Oe) - out_tol(EXACT_ABS, Oe, dtype)
    assert excess.max() <= 0.0, excess.max()
    assert np.abs(gl.reshape(-1) - lse).max() <= 1e-3


def test_bigd_sampled_groups():
    """Large head dimension, bf16: 32 query heads over 8, D = 512, 1024 rows
    at the tail of 4096 keys, at full size on sampled row groups."""
    _sampled("bigd", 32)


def test_long3b_exact_sampled_rows():
    """The all-exact path at the headline shape (its key range runs as
    several splits), on sampled rows against FP64 attention."""
    w = WORKLOADS["long3b"]
    Q, K, V = make_inputs(w, threads=16)
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps)
    go, gl = run_exact_gpu(problem_for(w), Q, K, V)
    rng = np.random.default_rng(5)
    rows = np.stack([np.zeros(24, np.int32), rng.integers(0, w.Hq, 24), rng.integers(0, w.Nq, 24)],
                    axis=1).astype(np.int32)
    Oe, lse = O.exact(po, Q, K, V, rows=rows)
    assert np.abs(go[rows[:, 0], rows[:, 1], rows[:, 2]] - Oe).max() <= EXACT_ABS
    assert np.abs(gl[rows[:, 0], rows[:, 1], rows[:, 2]] - lse).max() <= 1e-3


def test_quantize_group_above_eight():
    """apa_quantize with 12 query heads per KV head (pass 2 does not take such
    groups; quantise and pass 1 do): codes, scales and the tied Q scales of
    all twelve heads bitwise, and pass 1's mask against the oracle."""
    w = small_workload(1, 12, 1, 96, 1024, 64, seed=71)
    Q, K, V = make_inputs(w)
    po = O.Params(1, 12, 1, 96, 1024, 64, scale=w.scale, eps=0.02)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep, pass2=False)
    import torch
    from gpu_util import fp4_sections, torch_inputs, unpack_bits
    p = problem_for(w)
    q, k, v = torch_inputs(Q, K, V)
    bufs = apa.alloc(p)
    apa.quantize(p, q, k, v, bufs.fp4, bufs.ws_q)
    apa.pass1(p, bufs.fp4, 0.02, bufs.cold_m, bufs.cold_l, bufs.cold_o, bufs.bits, None,
              ws=bufs.ws_p1)
    torch.cuda.synchronize()
    check_quant({"fp4": fp4_sections(p, bufs.fp4.cpu().numpy())}, prep)
    check_mask(unpack_bits(p, bufs.bits.cpu().numpy()), r)
