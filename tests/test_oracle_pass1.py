"""Pins of the oracle's pass 1: bitwise agreement with the independent
frame-free brute force, frame invariance, cold-verdict safety, tile order,
and the NV-mode sink bug ("APA: sloppy attention, exact where it counts",
'Pass 1' steps 1-5, 'Tile order', 'The bug: a sink that drowned the tail')."""
import json
import os

import numpy as np
import pytest

from brute_apa import MAGS, brute_apa, nearest_mag_code, prepare
from mixed_precision_long_amd.inputs import make_inputs, small_workload
from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))

CASES = [  # Hq, Hkv, Nq, Nkv, D, eps, causal, seed
    (2, 1, 256, 1024, 64, 0.005, 1, 1),
    (2, 1, 100, 700, 64, 0.05, 1, 2),      # ragged Nq and Nkv
    (4, 2, 37, 300, 32, 0.02, 1, 3),       # GQA, tiny D, ragged
    (2, 2, 64, 200, 64, 0.1, 0, 4),        # non-causal
    (3, 1, 48, 512, 64, 0.0, 1, 5),        # eps = 0
    (2, 1, 64, 1024, 64, 1.0, 1, 6),       # eps = 1: nothing hot
    (2, 1, 1, 640, 64, 0.01, 1, 7),        # a single query row
    (2, 1, 128, 128, 64, 0.02, 1, 8),      # self-attention
]


def _frame_scale(m):
    return np.where(np.isfinite(m), np.exp2(np.where(np.isfinite(m), m, 0.0)), 0.0)


@pytest.mark.parametrize("case", CASES)
def test_pass1_bitwise_vs_framefree_brute_force(case):
    Hq, Hkv, Nq, Nkv, D, eps, causal, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed)
    Q, K, V = make_inputs(w)
    p = O.Params(1, Hq, Hkv, Nq, Nkv, D, causal=causal, scale=w.scale, eps=eps)
    r = O.run(p, Q, K, V, pass2=False)
    b = brute_apa(Q, K, V, eps, w.scale, bool(causal))
    sc = _frame_scale(r["m1"][0])
    assert np.array_equal(r["hot"][0].astype(bool), b["hot"])
    assert np.array_equal((r["l1"][0] * sc).astype(np.float32), b["l"])
    assert np.array_equal((r["lam"][0] * sc).astype(np.float32), b["lam"])
    assert np.array_equal((r["o1"][0] * sc[..., None]).astype(np.float32), b["o"])


@pytest.mark.parametrize("case", [CASES[0], CASES[2], CASES[3], CASES[4]])
def test_two_term_q_pass1_bitwise_vs_framefree_brute_force(case):
    # "Second hunt: which operand is to blame": a second FP4 term of Q for what
    # the first leaves over, sharing its scale, on the same K codes
    Hq, Hkv, Nq, Nkv, D, eps, causal, seed = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed)
    Q, K, V = make_inputs(w)
    p = O.Params(1, Hq, Hkv, Nq, Nkv, D, causal=causal, scale=w.scale, eps=eps, q_terms=2)
    r = O.run(p, Q, K, V, pass2=False)
    b = brute_apa(Q, K, V, eps, w.scale, bool(causal), q_terms=2)
    sc = _frame_scale(r["m1"][0])
    assert np.array_equal(r["hot"][0].astype(bool), b["hot"])
    assert np.array_equal((r["l1"][0] * sc).astype(np.float32), b["l"])
    assert np.array_equal((r["lam"][0] * sc).astype(np.float32), b["lam"])
    assert np.array_equal((r["o1"][0] * sc[..., None]).astype(np.float32), b["o"])
    # the second term changes the scores: a one-term brute force disagrees
    b1 = brute_apa(Q, K, V, eps, w.scale, bool(causal), q_terms=1)
    assert not np.array_equal(b1["lam"], b["lam"])


def test_two_term_q_brings_scores_closer_to_exact():
    # the residual term removes most of Q's quantisation error: FP4 scores
    # against the exact scores of the centred keys (same K codes)
    w = small_workload(1, 2, 1, 64, 512, 64, seed=21)
    Q, K, V = make_inputs(w)
    err = {}
    for qt in (1, 2):
        ops = prepare(Q[0], K[0], V[0], w.scale, qt)
        kv = ops[0]
        kd = kv["kd"].astype(np.float64)
        for hd in kv["heads"]:
            Qh = hd["Qh"].astype(np.float64)
            # exact Q against the quantised K, in the same normalised units
            qn = Qh / np.abs(Qh).max()
            qdn = hd["qd"] / np.abs(hd["qd"]).max()
            e = np.abs(qdn @ kd.T - qn @ kd.T).mean() / np.abs(qn @ kd.T).mean()
            err.setdefault(qt, []).append(e)
    e1, e2 = np.mean(err[1]), np.mean(err[2])
    assert e2 < 0.25 * e1, (e1, e2)


def test_frame_invariance_over_tau_and_H():
    w = small_workload(1, 2, 1, 96, 1024, 64, seed=11)
    Q, K, V = make_inputs(w)
    ref = None
    for tau in (0.0, 4.0, 8.0):
        for H in (0.0, 32.0, 64.0):
            p = O.Params(1, 2, 1, 96, 1024, 64, scale=w.scale, eps=0.02, tau=tau, hoff=H)
            r = O.run(p, Q, K, V, pass2=False)
            sc = _frame_scale(r["m1"][0])
            cur = (r["hot"].copy(), r["l1"][0] * sc, r["o1"][0] * sc[..., None], r["lam"][0] * sc)
            if ref is None:
                ref = cur
            else:
                for a, b in zip(ref, cur):
                    assert np.array_equal(a, b), (tau, H)


def test_cold_verdicts_are_safe():
    # every cold cell: its FP4 tile mass stays below eps of the final lambda
    w = small_workload(1, 2, 1, 128, 2048, 64, seed=12)
    Q, K, V = make_inputs(w)
    for eps in (0.005, 0.02, 0.1):
        p = O.Params(1, 2, 1, 128, 2048, 64, scale=w.scale, eps=eps)
        b = brute_apa(Q, K, V, eps, w.scale)
        ops = b["ops"][0]
        for h in range(2):
            hd = ops["heads"][h]
            s = (hd["alpha"] * (hd["qd"] @ ops["kd"].T)).astype(np.float32).astype(np.float64)
            for g in range(8):
                rows = np.arange(16 * g, 16 * g + 16)
                lam = b["lam"][h, rows].astype(np.float64)
                for t in np.flatnonzero(~b["hot"][h, g]):
                    if t > (rows[-1] + 2048 - 128) // 64:
                        continue
                    # frame-free FP4 mass of the cold tile, recomputed
                    st = s[rows, 64 * t:64 * t + 64].copy()
                    st[np.arange(64 * t, 64 * t + 64)[None, :] > rows[:, None] + 1920] = -np.inf
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
                    assert np.all(mass <= eps * lam * (1 + 1e-6)), (eps, h, g, t)


def test_visit_orders_match_hand_derivation():
    cases = json.load(open(os.path.join(HERE, "golden", "visit_orders.json")))["cases"]
    for c in cases:
        p = O.Params(1, 1, 1, c["Nq"], c["Nkv"], 64, causal=c["causal"], window=c.get("window", 0))
        assert O.visit_order(p, c["group"]) == c["order"], c


def test_ascending_order_makes_more_tiles_hot():
    # sink-and-diagonal-first vs a left-to-right walk: the latter judges early
    # tiles against a small running sum ('Tile order')
    w = small_workload(1, 2, 1, 64, 4096, 64, seed=13)
    Q, K, V = make_inputs(w)
    p = O.Params(1, 2, 1, 64, 4096, 64, scale=w.scale, eps=0.01)
    r = O.run(p, Q, K, V, pass2=False)
    b = brute_apa(Q, K, V, 0.01, w.scale)
    assert np.array_equal(r["hot"][0].astype(bool), b["hot"])
    import brute_apa as BA
    saved = BA.visit_order
    try:
        BA.visit_order = lambda last, off, Nkv, causal, tile=64, **kw: list(
            range(0, (min(Nkv - 1, last + off) // tile) + 1))
        asc = BA.brute_apa(Q, K, V, 0.01, w.scale)
    finally:
        BA.visit_order = saved
    assert asc["hot"].sum() > b["hot"].sum()


def test_nv_mode_sink_bug_and_decoupled_frame():
    # NV P scales clamp at 2^-6, so with the frame set by a strong sink (H = 0)
    # thin cold groups round to zero and the cold mass vanishes; H = 32
    # keeps it ('The bug: a sink that drowned the tail')
    w = small_workload(1, 2, 1, 64, 8192, 64, seed=14, delta=14.0, a=1.0)
    Q, K, V = make_inputs(w)
    lost = {}
    for H in (0.0, 32.0):
        p = O.Params(1, 2, 1, 64, 8192, 64, scale=w.scale, eps=0.01, fmt=O.NV, hoff=H)
        r = O.run(p, Q, K, V, pass2=False)
        lost[H] = np.mean(r["l1"][0] == 0)
    pm = O.Params(1, 2, 1, 64, 8192, 64, scale=w.scale, eps=0.01, fmt=O.MX, hoff=0.0)
    rm = O.run(pm, Q, K, V, pass2=False)
    assert lost[0.0] > 0.5          # most rows lose their whole cold state
    assert lost[32.0] < lost[0.0]   # the decoupled frame recovers it
    assert np.mean(rm["l1"][0] == 0) == 0.0  # MX scales have no such floor
