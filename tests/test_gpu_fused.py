"""f1: pass 1 and pass 2 in one persistent launch (APA page, "Pass 2: exact
FP16 on the hot tiles": one work group per compute unit takes ordered
tickets, pass-1 work first, then pass-2 work).

apa_fused must give exactly what apa_pass1 (with its workspace) and then
apa_pass2 with the fused merge give: the same cold state, lambda, hot mask,
output and LSE, bit for bit, with bit 1 of the status word (a wait that gave
up) clear.  The shapes cover the three pass-1 schedules, tails that give up
and are walked again inside the launch, one key split (the split merges
itself), an odd number of splits (the last ticket of a work group runs one
split), GQA groups 1 and 3, batches, no causal mask, a sliding window, bf16
inputs, two Q terms, the value-norm weighted test, paged K/V, two calls in a
row on one workspace, and the headline shape.  Checked against the
oracle once."""
import numpy as np
import pytest
import torch

from gpu_util import pass1_schedule, problem_for, torch_inputs, unpack_bits
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import (WORKLOADS, make_inputs, outlier_value_tiles,
                                             small_workload)
from oracle import oracle as O
from test_gpu_parity import check_mask, check_output
from test_gpu_split import lift_key

pytestmark = pytest.mark.gpu


def _host(p, b, fp4_status=False):
    r = dict(m=b.cold_m.cpu().numpy(), l=b.cold_l.cpu().numpy(), o=b.cold_o.cpu().numpy(),
             lam=b.lam.cpu().numpy(), hot=unpack_bits(p, b.bits.cpu().numpy()),
             out=b.out.float().cpu().numpy(), lse=b.lse.cpu().numpy())
    L = apa.fp4_layout(p)
    r["status"] = int(b.fp4[L.status:L.status + 4].cpu().numpy().view(np.uint32)[0])
    return r


def run_pair(p, q, k, v, eps, repeat=1):
    """(separate launches, single launch) outputs on the same inputs."""
    ref = apa.alloc(p, with_lambda=True)
    apa.quantize(p, q, k, v, ref.fp4, ref.ws_q)
    apa.pass1(p, ref.fp4, eps, ref.cold_m, ref.cold_l, ref.cold_o, ref.bits, ref.lam,
              ws=ref.ws_p1)
    apa.pass2(p, q, k, v, ref.fp4, ref.bits, ref.cold_m, ref.cold_l, ref.cold_o, True,
              out=ref.out, lse=ref.lse, ws=ref.ws_p2)
    fz = apa.alloc(p, with_lambda=True, with_fused=True)
    assert fz.ws_fused is not None, "the single launch should cover this problem"
    apa.quantize(p, q, k, v, fz.fp4, fz.ws_q)
    runs = []
    for _ in range(repeat):
        for x in (fz.cold_m, fz.cold_l, fz.cold_o, fz.bits, fz.lam, fz.lse):
            x.fill_(7)
        fz.out.fill_(7)
        apa.fused(p, q, k, v, fz.fp4, eps, fz.cold_m, fz.cold_l, fz.cold_o, fz.bits, fz.out,
                  lse=fz.lse, lam=fz.lam, ws=fz.ws_fused)
        torch.cuda.synchronize()
        runs.append(_host(p, fz))
    torch.cuda.synchronize()
    return _host(p, ref), runs


def assert_same(a, b):
    for key in ("m", "l", "o", "lam", "hot", "out", "lse"):
        x, y = a[key], b[key]
        assert x.shape == y.shape, key
        assert np.array_equal(np.nan_to_num(x), np.nan_to_num(y)), (key, np.argwhere(x != y)[:5])
    assert b["status"] & 2 == 0, "a wait of the single launch gave up"


CASES = [
    # B, Hq, Hkv, Nq, Nkv, eps, causal, window, mode, sched
    (1, 6, 2, 200, 9000, 0.01, 1, 0, "path", apa.SCHED_AUTO),      # GQA 3, ragged, 8 splits
    (1, 6, 2, 200, 5120, 0.02, 1, 0, "path", apa.SCHED_AUTO),      # 5 splits: an idle half
    (1, 4, 2, 64, 1000, 0.02, 1, 0, "path", apa.SCHED_AUTO),       # one split, whole schedule
    (2, 8, 2, 96, 4000, 0.01, 0, 0, "gauss", apa.SCHED_AUTO),      # batches, no causal mask
    (1, 4, 4, 160, 7000, 0.005, 1, 0, "path", apa.SCHED_AUTO),     # GQA 1
    (1, 6, 2, 300, 6000, 0.01, 1, 1500, "path", apa.SCHED_AUTO),   # sliding window
    (1, 6, 2, 256, 12000, 0.005, 1, 0, "path", apa.SCHED_PAIRS),   # pair schedule
    (1, 6, 2, 256, 12000, 0.005, 1, 0, "path", apa.SCHED_TRIPLES), # triple schedule
]


@pytest.mark.parametrize("case", CASES, ids=["gqa3", "odd_splits", "one_split", "batch_noncausal",
                                             "gqa1", "window", "pairs", "triples"])
def test_fused_equals_separate_launches(case):
    B, Hq, Hkv, Nq, Nkv, eps, causal, window, mode, sched = case
    w = small_workload(B, Hq, Hkv, Nq, Nkv, 128, causal=causal, mode=mode, seed=95)
    Q, K, V = make_inputs(w)
    p = problem_for(w, sched=sched, window=window)
    print("[fused] case", case, "schedule", pass1_schedule(p), flush=True)
    q, k, v = torch_inputs(Q, K, V, "fp16")
    ref, runs = run_pair(p, q, k, v, eps)
    assert_same(ref, runs[0])


@pytest.mark.parametrize("case", ["bf16", "two_term_q", "hot_weight", "bf16_two_term_weight"])
def test_fused_variants(case):
    """bf16 inputs (pass 2 converts V to fp16 in LDS), two Q terms in pass 1,
    the value-norm weighted hot test, and all three together."""
    bf = "bf16" in case
    qt = 2 if "two_term" in case else 1
    hw = 1 if "weight" in case else 0
    w = small_workload(1, 6, 2, 200, 9000, 128, dtype="bf16" if bf else "fp16",
                       mode="gauss" if bf else "path", seed=98)
    Q, K, V = make_inputs(w)
    if hw:
        outlier_value_tiles(V, 4, 8.0, seed=98)
    p = problem_for(w, q_terms=qt, hot_weight=hw)
    q, k, v = torch_inputs(Q, K, V, "bf16" if bf else "fp16")
    ref, runs = run_pair(p, q, k, v, 0.01)
    assert_same(ref, runs[0])


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fused_d64(dtype):
    """D = 64 (the merge takes four rows per wave pass): GQA 4, ragged."""
    w = small_workload(1, 8, 2, 96, 12000, 64, dtype=dtype, mode="gauss" if dtype == "bf16" else "path",
                       seed=100)
    Q, K, V = make_inputs(w)
    p = problem_for(w)
    q, k, v = torch_inputs(Q, K, V, dtype)
    ref, runs = run_pair(p, q, k, v, 0.005)
    assert_same(ref, runs[0])


def test_fused_over_paged_kv():
    """16-bit K/V through a block table (unused page slots NaN): the same
    results as the separate launches over the same pages, clean status."""
    from test_gpu_chunked import _pages
    B, Hq, Hkv, Nq, Nkv, D = 2, 6, 2, 160, 7000, 128
    w = small_workload(B, Hq, Hkv, Nq, Nkv, D, seed=99)
    Q, K, V = make_inputs(w)
    NT = -(-Nkv // 64)
    npages = B * NT + 3
    perm = np.random.default_rng(5).permutation(npages)[:B * NT].reshape(B, NT).astype(np.int32)
    bt = torch.from_numpy(np.ascontiguousarray(perm)).cuda()
    kp, vp = (_pages(x, B, Hkv, Nkv, D, perm, npages, torch.float16) for x in (K, V))
    q = torch.from_numpy(Q).half().cuda()
    p = problem_for(w, block_table=bt)
    ref, runs = run_pair(p, q, kp, vp, 0.01)
    assert_same(ref, runs[0])
    assert runs[0]["status"] == 0


@pytest.mark.parametrize("sched", [apa.SCHED_PAIRS, apa.SCHED_TRIPLES])
def test_fused_walks_given_up_tails_again(sched):
    """A key 70 nats up in every block's tail segment: each tail needs a
    re-base of its frame, gives up, and the single launch walks the tail again
    from the head's state before the block's units count as done."""
    w = small_workload(1, 2, 1, 64, 16384, 128, seed=33)
    Q, K, V = make_inputs(w)
    K = lift_key(w, Q, K, 20 * 64 + 7, 70.0)
    p = problem_for(w, sched=sched)
    assert pass1_schedule(p) == sched
    q, k, v = torch_inputs(Q, K, V, "fp16")
    ref, runs = run_pair(p, q, k, v, 0.005)
    assert_same(ref, runs[0])


def test_fused_twice_on_one_workspace_and_oracle():
    """Two calls in a row on one workspace (its control words cleared by each
    call) give the same results; and the oracle's bars hold."""
    w = small_workload(1, 6, 2, 200, 9000, 128, seed=96)
    Q, K, V = make_inputs(w)
    eps = 0.01
    p = problem_for(w)
    q, k, v = torch_inputs(Q, K, V, "fp16")
    ref, runs = run_pair(p, q, k, v, eps, repeat=2)
    assert_same(ref, runs[0])
    assert_same(ref, runs[1])
    po = O.Params(1, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=eps)
    r = O.run(po, Q, K, V, O.quantize(po, Q, K, V))
    check_mask(runs[1]["hot"], r)
    check_output(runs[1]["out"], r["O"], dtype="fp16")


def test_fused_uncovered_problems_are_refused():
    w = small_workload(1, 4, 2, 64, 2000, 256, seed=97)
    p = problem_for(w)
    assert apa.workspace_bytes(p, apa.CALL_FUSED) == 0
    b = apa.alloc(p, with_lambda=True)
    Q, K, V = make_inputs(w)
    q, k, v = torch_inputs(Q, K, V, "fp16")
    with pytest.raises(RuntimeError, match="UNSUPPORTED|unsupported"):
        apa.fused(p, q, k, v, b.fp4, 0.01, b.cold_m, b.cold_l, b.cold_o, b.bits, b.out,
                  lse=b.lse, ws=b.ws_p2)


def test_fused_long3b():
    """The headline shape, 2048 x 122880 at eps = 0.005 (triple schedule, four
    key splits): the single launch equals the separate launches bit for bit."""
    w = WORKLOADS["long3b"]
    Q, K, V = make_inputs(w, threads=16)
    p = problem_for(w)
    q, k, v = torch_inputs(Q, K, V, "fp16")
    ref, runs = run_pair(p, q, k, v, w.eps)
    assert_same(ref, runs[0])
