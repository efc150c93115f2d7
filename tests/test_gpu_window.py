"""The sliding-window variant ("What else is in the box": sliding window) on
the GPU against the oracle: row r sees only its `window` most recent keys;
a row group whose first row no longer sees tile 0 visits its tiles from the
causal diagonal backwards.  Same bars as the other parity tests, for the
whole APA path (codes, masks, cold state, output, LSE) and the all-exact
path, with pass 1 whole and split; at the headline shape with a 4096-key
window every row group of one KV head is checked."""
import numpy as np
import pytest

from gpu_util import problem_for, run_exact_gpu, run_gpu
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import WORKLOADS, make_inputs, small_workload
from oracle import oracle as O
from test_gpu_parity import (EXACT_ABS, check_cold_state, check_mask, check_output, check_quant,
                             out_tol)

pytestmark = pytest.mark.gpu

# Hq, Hkv, Nq, Nkv, D, eps, window, seed, dtype, mode
CASES = [
    (2, 1, 256, 4096, 64, 0.02, 700, 71, "fp16", "path"),     # window inside the keys
    (6, 2, 200, 3000, 128, 0.01, 1000, 72, "fp16", "path"),   # GQA 3, ragged rows and keys
    (2, 1, 512, 512, 128, 0.02, 300, 73, "fp16", "path"),     # self-attention
    (4, 1, 96, 2048, 256, 0.02, 1500, 74, "fp16", "path"),    # D = 256
    (4, 1, 96, 2048, 512, 0.02, 900, 75, "bf16", "gauss"),    # D = 512, bf16
    (2, 1, 128, 6000, 64, 0.0, 2000, 76, "fp16", "path"),     # eps = 0: exact on the window
    (2, 1, 64, 2000, 64, 0.01, 5000, 77, "fp16", "path"),     # window longer than the keys
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "D%d_W%d_eps%g_%s" % (c[4], c[6], c[5], c[8]))
def test_window_matches_oracle(case):
    Hq, Hkv, Nq, Nkv, D, eps, window, seed, dtype, mode = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, dtype=dtype, mode=mode, seed=seed)
    Q, K, V = make_inputs(w)
    po = O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, window=window)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w, window=window), Q, K, V, eps, dtype=dtype)
    check_quant(g, prep, po.first_tile)
    mism = check_mask(g["hot"], r)
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"], dtype=dtype)
    fin = np.isfinite(r["lse"])
    assert np.abs(g["lse"][fin] - r["lse"][fin]).max() <= 2e-3
    # nothing is hot outside the windows of a group's rows
    off = Nkv - Nq
    for gg in range(g["hot"].shape[2]):
        first = max(0, 16 * gg + off - window + 1) // 64
        assert not g["hot"][:, :, gg, :first].any()
    Oe, lse = O.exact(po, Q, K, V)
    go, gl = run_exact_gpu(problem_for(w, window=window), Q, K, V, dtype=dtype)
    excess = np.abs(go.reshape(-1, D) - Oe) - out_tol(EXACT_ABS, Oe, dtype)
    assert excess.max() <= 0.0, excess.max()
    assert np.abs(gl.reshape(-1) - lse).max() <= 1e-3


@pytest.mark.parametrize("sched", [apa.SCHED_PAIRS, apa.SCHED_TRIPLES])
def test_window_split_schedules(sched):
    """Windows of about 190 tiles at 16384 keys: pass 1 cut into head and tail
    walks over orders that do not start with tile 0."""
    w = small_workload(1, 2, 1, 128, 16384, 64, mode="gauss", seed=78)
    Q, K, V = make_inputs(w)
    window = 12000
    p = problem_for(w, window=window, sched=sched)
    assert apa.pass1_split(p, 188)[1] < 188
    po = O.Params(1, 2, 1, 128, 16384, 64, scale=w.scale, eps=0.02, window=window)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(p, Q, K, V, 0.02)
    assert len(g["tail"]) > 0
    check_quant(g, prep, po.first_tile)
    mism = check_mask(g["hot"], r)
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"])


def test_long3b_window_4096_every_group_of_one_kv_head():
    """The page's sliding-window case: 2048 rows at 122880 keys with a
    4096-key window, eps 0.005, every row group of the three query heads of
    KV head 0."""
    w = WORKLOADS["long3b"]
    window = 4096
    Q, K, V = make_inputs(w, threads=16)
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps, window=window)
    g = run_gpu(problem_for(w, window=window), Q, K, V, w.eps, lam=False)
    prep = O.quantize(po, Q, K, V)
    check_quant(g, prep, po.first_tile)
    assert po.first_tile == (122880 - 2048 - 4096 + 1) // 64
    G = w.Hq // w.Hkv
    sel = np.array([(0, h, gg) for h in range(G) for gg in range(w.Nq // 16)], np.int32)
    r = O.run(po, Q, K, V, prep, groups=sel, nthreads=16)
    mism = check_mask(g["hot"], r, groups=sel)
    check_cold_state(g, r, mism, groups=sel)
    rows = np.array([(0, h, gg * 16 + i) for _, h, gg in sel for i in range(16)], np.int32)
    check_output(g["out"], r["O"], rows)
    ix = (rows[:, 0], rows[:, 1], rows[:, 2])
    assert np.abs(g["lse"][ix] - r["lse"][ix]).max() <= 2e-3
