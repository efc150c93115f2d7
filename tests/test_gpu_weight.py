"""The value-norm weighted hot test ("APA: sloppy attention, exact where it
counts", section "Honest limits", on mass versus output) on the GPU against
the oracle: a tile's mass counts w_t = max(1, nu_t / nu_bar) times in the
vote, nu_t the largest value norm among its keys and nu_bar the head's mean
value norm.  The inputs carry a few key tiles with outsized values (the
hazard the weights target).  Same bars as the other parity tests -- codes,
masks, cold state, output, LSE -- plus the weights themselves; pass 1 whole
and split (the split's undecided tail tiles are re-judged with the same
weights), and every row group of one KV head at the 122880-key shape."""
import numpy as np
import pytest

from gpu_util import problem_for, run_gpu
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import (WORKLOADS, outlier_value_tiles, make_inputs,
                                             small_workload)
from oracle import oracle as O
from test_gpu_parity import check_cold_state, check_mask, check_output, check_quant

pytestmark = pytest.mark.gpu

# The GPU sums each key's squares in FP32 (8 channels per lane, then a
# butterfly over the lanes) and the head's mean norm in FP64 of FP32 norms,
# where the oracle works in FP64 throughout: about D/8 + log2(D/8) + 3 FP32
# roundings, well under 1e-5 relative for D <= 512.
W_RTOL = 1e-5


def check_weights(g, prep, first_tile=0):
    """The GPU's tile weights and mean value norm against the oracle's (from
    the first tile some row sees; the others are not written)."""
    gw = g["fp4"]["tile_w"][..., first_tile:]
    ow = prep["vw"][..., first_tile:]
    assert np.all(gw >= 1.0)
    assert np.allclose(gw, ow, rtol=W_RTOL, atol=0.0), np.abs(gw / ow - 1).max()
    nb = g["fp4"]["kv_head"][..., 6]
    assert np.allclose(nb, prep["nu_bar"], rtol=W_RTOL, atol=0.0)


# Hq, Hkv, Nq, Nkv, D, eps, boosted tiles, factor, seed, dtype, mode, window
CASES = [
    (2, 1, 256, 4096, 64, 0.02, 4, 8.0, 91, "fp16", "path", 0),
    (6, 2, 200, 3000, 128, 0.02, 6, 16.0, 92, "fp16", "path", 0),   # GQA 3, ragged
    (4, 1, 96, 2048, 256, 0.02, 6, 16.0, 93, "fp16", "path", 0),    # D = 256
    (4, 1, 96, 2048, 512, 0.05, 3, 8.0, 94, "bf16", "gauss", 0),    # D = 512, bf16
    (2, 1, 256, 4096, 64, 0.02, 3, 16.0, 95, "fp16", "path", 1500), # sliding window
    (2, 1, 128, 3000, 64, 0.0, 3, 8.0, 96, "fp16", "path", 0),      # eps = 0
    (2, 1, 128, 3000, 64, 1.0, 3, 8.0, 97, "fp16", "path", 0),      # eps = 1
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: "D%d_eps%g_W%d_%s" % (c[4], c[5], c[11], c[9]))
def test_weighted_matches_oracle(case):
    Hq, Hkv, Nq, Nkv, D, eps, nb, factor, seed, dtype, mode, window = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, dtype=dtype, mode=mode, seed=seed)
    Q, K, V = make_inputs(w)
    po = O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, window=window, hot_weight=1)
    outlier_value_tiles(V, nb, factor, seed=seed, first_tile=po.first_tile, dtype=dtype)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w, window=window, hot_weight=1), Q, K, V, eps, dtype=dtype)
    check_quant(g, prep, po.first_tile)
    check_weights(g, prep, po.first_tile)
    mism = check_mask(g["hot"], r)
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"], dtype=dtype)
    fin = np.isfinite(r["lse"])
    assert np.abs(g["lse"][fin] - r["lse"][fin]).max() <= 2e-3
    if 0.0 < eps < 1.0:
        # the weights are live: the unweighted oracle marks fewer cells hot
        r0 = O.run(O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, window=window),
                   Q, K, V, pass2=False)
        assert r["hot"].sum() > r0["hot"].sum()


@pytest.mark.parametrize("sched", [apa.SCHED_PAIRS, apa.SCHED_TRIPLES])
def test_weighted_split_schedules(sched):
    """Visit orders of 192 tiles cut into head and tail walks: the tail's
    undecided tiles are recorded and settled against the head's lambda with
    the same weights."""
    w = small_workload(1, 2, 1, 128, 12288, 64, mode="gauss", seed=98)
    Q, K, V = make_inputs(w)
    outlier_value_tiles(V, 12, 8.0, seed=98)
    p = problem_for(w, sched=sched, hot_weight=1)
    assert apa.pass1_split(p, 192)[1] < 192
    po = O.Params(1, 2, 1, 128, 12288, 64, scale=w.scale, eps=0.02, hot_weight=1)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(p, Q, K, V, 0.02)
    assert len(g["tail"]) > 0
    print("[split %d] tail outcomes %s" % (sched, np.bincount(g["tail"] + 1)), flush=True)
    check_quant(g, prep)
    check_weights(g, prep)
    mism = check_mask(g["hot"], r)
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"])


def test_weighted_long3b_every_group_of_one_kv_head():
    """2048 rows at 122880 keys (eps 0.005) with 64 tiles of 4x values per KV
    head: every row group of the three query heads of KV head 0."""
    w = WORKLOADS["long3b"]
    Q, K, V = make_inputs(w, threads=16)
    outlier_value_tiles(V, 64, 4.0, seed=99)
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=w.eps, hot_weight=1)
    g = run_gpu(problem_for(w, hot_weight=1), Q, K, V, w.eps, lam=False)
    prep = O.quantize(po, Q, K, V)
    check_quant(g, prep)
    check_weights(g, prep)
    G = w.Hq // w.Hkv
    sel = np.array([(0, h, gg) for h in range(G) for gg in range(w.Nq // 16)], np.int32)
    r = O.run(po, Q, K, V, prep, groups=sel, nthreads=16)
    mism = check_mask(g["hot"], r, groups=sel)
    check_cold_state(g, r, mism, groups=sel)
    rows = np.array([(0, h, gg * 16 + i) for _, h, gg in sel for i in range(16)], np.int32)
    check_output(g["out"], r["O"], rows)
    ix = (rows[:, 0], rows[:, 1], rows[:, 2])
    assert np.abs(g["lse"][ix] - r["lse"][ix]).max() <= 2e-3
    print("[long3b weighted] %d mask mismatches, hot cells %d" % (
        int(mism.sum()), int(g["hot"][0, :G].sum())), flush=True)
