"""Pass 1 with its workspace: each long visit order runs as a head and a tail
walk in one work group, the tail finishing the unit; with the pair schedule
every 32-row block has its own tail wave, with the triple schedule one wave
walks the tails of three blocks one after the other.  Checked against the oracle (same bars as the other
parity tests) and against the one-wave walk of the same inputs, with the
tail's outcome per 32-row block read back from the workspace to show which
way the tail finished: records decided (the lower bound of lambda left some
tail tiles undecided), or a second walk of the whole tail from the head's
state (record full, or a score jump that needs a re-base of the state
frame)."""
import numpy as np
import pytest

from gpu_util import pass1_schedule, problem_for, run_gpu
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import make_inputs, small_workload
from oracle import oracle as O
from test_gpu_parity import check_cold_state, check_mask, check_output, check_quant

pytestmark = pytest.mark.gpu


def lift_key(w, Q, K, key, nats):
    """Raise the logit of one key by about `nats` for the rows of every head
    (the sink construction of the input generator, applied to one key)."""
    G = w.Hq // w.Hkv
    for b in range(w.B):
        for j in range(w.Hkv):
            u = Q[b, j * G:(j + 1) * G].reshape(-1, w.D).astype(np.float64).mean(axis=0)
            K[b, j, key] = np.float16(K[b, j, key] + nats * u / (w.scale * float(u @ u)))
    return K


SCHEDS = [apa.SCHED_PAIRS, apa.SCHED_TRIPLES]


def run_case(w, eps, Q, K, V, sched):
    p = problem_for(w, sched=sched)
    assert apa.workspace_bytes(p, apa.CALL_PASS1) > 0, "this shape should run split"
    assert pass1_schedule(p) == sched
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, causal=w.causal, scale=w.scale, eps=eps)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(p, Q, K, V, eps)
    print("tail outcomes", np.unique(g["tail"], return_counts=True), flush=True)
    check_quant(g, prep)
    mism = check_mask(g["hot"], r)
    check_cold_state(g, r, mism)
    check_output(g["out"], r["O"], dtype=w.dtype)
    fin = np.isfinite(r["lse"])
    assert np.abs(g["lse"][fin] - r["lse"][fin]).max() <= 2e-3
    # the one-wave walk: the same verdicts away from the threshold, the same
    # outputs within the method's bar
    one = run_gpu(p, Q, K, V, eps, split=False)
    diff = one["hot"] != g["hot"]
    if diff.any():
        assert np.all(np.abs(r["margin"][diff]) <= 1e-3), r["margin"][diff]
    check_output(g["out"], one["out"], dtype=w.dtype)
    return g


# gauss inputs: every tile carries about the same mass, so lambda grows
# linearly and the tail's bounded test passes for its first tiles
@pytest.mark.parametrize("sched", SCHEDS)
def test_split_decides_undecided_tail_tiles(sched):
    w = small_workload(1, 2, 1, 64, 16384, 64, mode="gauss", seed=31)
    Q, K, V = make_inputs(w)
    g = run_case(w, 0.02, Q, K, V, sched)
    assert (g["tail"] > 0).any(), g["tail"]
    assert (g["tail"] >= 0).all(), g["tail"]


@pytest.mark.parametrize("sched,nkv", [(apa.SCHED_PAIRS, 73728), (apa.SCHED_TRIPLES, 163840)])
def test_split_full_record_walks_the_tail(sched, nkv):
    # about 541 (pairs) or 536 (triples) tail positions per block, nearly all
    # undecided: more than the 512 records
    w = small_workload(1, 2, 1, 64, nkv, 64, mode="gauss", seed=32)
    Q, K, V = make_inputs(w)
    g = run_case(w, 1e-4, Q, K, V, sched)
    assert (g["tail"] == -1).all(), g["tail"]


@pytest.mark.parametrize("sched", SCHEDS)
def test_split_rebase_in_tail_walks_the_tail(sched):
    w = small_workload(1, 2, 1, 64, 16384, 64, seed=33)
    Q, K, V = make_inputs(w)
    K = lift_key(w, Q, K, 20 * 64 + 7, 70.0)  # tile 20: in every block's tail segment
    g = run_case(w, 0.005, Q, K, V, sched)
    assert (g["tail"] == -1).all(), g["tail"]


@pytest.mark.parametrize("sched", SCHEDS)
def test_split_hot_tail_tile_leaves_the_state(sched):
    """A key lifted by 8 nats in the tail segment makes its tile hot for every
    row group: the tail records it undecided, accumulates it as cold, and at
    its end finds it hot and takes its P V back out."""
    w = small_workload(1, 2, 1, 64, 16384, 64, seed=37)
    Q, K, V = make_inputs(w)
    K = lift_key(w, Q, K, 20 * 64 + 7, 8.0)
    g = run_case(w, 0.005, Q, K, V, sched)
    assert (g["tail"] > 0).all(), g["tail"]
    assert g["hot"][..., 20].all()


@pytest.mark.parametrize("sched", SCHEDS)
@pytest.mark.parametrize("case", [
    (2, 1, 32, 266240, 64, 0.005, 38, 1),   # 4160 key tiles: hot words kept in the tile loop
    (6, 2, 200, 9000, 128, 0.005, 34, 1),   # GQA 3, ragged rows and keys
    (4, 1, 96, 12000, 64, 0.01, 35, 0),     # non-causal
    (2, 1, 64, 12288, 256, 0.005, 36, 1),   # D = 256
    (2, 1, 64, 12288, 64, 0.0, 39, 1),      # eps = 0: every visited tile hot, no records
])
def test_split_path_inputs(case, sched):
    Hq, Hkv, Nq, Nkv, D, eps, seed, causal = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, seed=seed, causal=causal)
    Q, K, V = make_inputs(w)
    run_case(w, eps, Q, K, V, sched)


@pytest.mark.parametrize("sched", SCHEDS)
def test_split_orders_near_the_cut(sched):
    """Visit orders of 61 to 180 positions, diffuse gauss rows without a sink:
    orders the cut rule leaves without a tail of 8 positions run whole, the
    rest are cut inside the order.  Regression: an earlier rule cut orders of
    64 to 108 positions at or past their end under the triple schedule; the
    tail then visited tile 0 a second time and tiles before it, which the
    strict cold-state check (no missing or extra mass) sees."""
    w = small_workload(1, 2, 1, 7680, 11520, 64, mode="gauss", delta=0.0, seed=40)
    p = problem_for(w, sched=sched)
    cuts = [apa.pass1_split(p, n)[1] for n in range(61, 181)]
    assert all(c == n or 32 <= c <= n - 8 for c, n in zip(cuts, range(61, 181)))
    assert any(c < n for c, n in zip(cuts, range(61, 181)))
    Q, K, V = make_inputs(w)
    g = run_case(w, 0.02, Q, K, V, sched)
    assert len(g["tail"]) > 0
