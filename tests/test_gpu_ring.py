"""KV window ring ("What else is in the box": the FP4 copy of K and V held to
a sink tile plus two ring halves of R tiles per KV head, the next key segment
quantised while pass 1 walks the current one).

apa_ring_pass1 walks every 32-row block's visit order in segments of R key
tiles, top down, carrying each block's state between launches; it must give
exactly what quantise + pass 1 with one wave per block (the unbroken walk)
give: the same cold state, lambda and hot mask bit for bit, the same
statistics, scales, Q codes and frames in the FP4 buffer, and then the same
pass-2 output.  Also checked against the oracle once per shape."""
import numpy as np
import pytest
import torch

from gpu_util import problem_for, torch_inputs, unpack_bits
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import WORKLOADS, make_inputs, small_workload
from oracle import oracle as O
from test_gpu_parity import check_mask, check_output

pytestmark = pytest.mark.gpu


def _sections(p, fp4):
    """The FP4 buffer's sections outside the K/V blobs (the ring keeps only
    1 + 2R of those)."""
    L = apa.fp4_layout(p)
    h = fp4.cpu().numpy()
    return {"kbar": h[L.kbar:L.kv_head], "kv_head": h[L.kv_head:L.tile_w],
            "status": h[L.status:L.status + 4], "q": h[L.q_codes:L.q_head],
            "q_head": h[L.q_head:L.q_frame], "q_frame": h[L.q_frame:L.q2_codes],
            "q2": h[L.q2_codes:L.total]}


def run_both(w, R, eps, q_terms=1, tensors=None):
    dt = apa.APA_F16 if w.dtype == "fp16" else apa.APA_BF16
    Q, K, V = make_inputs(w) if tensors is None else tensors
    q, k, v = torch_inputs(Q, K, V, w.dtype)
    kw = dict(dtype=dt, causal=w.causal, scale=w.scale, q_terms=q_terms)
    pr = apa.problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, sched=apa.SCHED_WHOLE, **kw)
    pg = apa.problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, ring_tiles=R, **kw)
    res = {}
    for name, p in (("ref", pr), ("ring", pg)):
        b = apa.alloc(p, with_lambda=True)
        b.fp4.zero_()
        if name == "ref":
            apa.quantize(p, q, k, v, b.fp4, b.ws_q)
            apa.pass1(p, b.fp4, eps, b.cold_m, b.cold_l, b.cold_o, b.bits, b.lam, ws=None)
        else:
            apa.ring_pass1(p, q, k, v, b.fp4, eps, b.cold_m, b.cold_l, b.cold_o, b.bits, b.lam,
                           ws=b.ws_ring)
        apa.pass2(p, q, k, v, b.fp4, b.bits, b.cold_m, b.cold_l, b.cold_o, True, out=b.out,
                  lse=b.lse, ws=b.ws_p2)
        torch.cuda.synchronize()
        res[name] = dict(m=b.cold_m.cpu().numpy(), l=b.cold_l.cpu().numpy(),
                         o=b.cold_o.cpu().numpy(), lam=b.lam.cpu().numpy(),
                         hot=unpack_bits(p, b.bits.cpu().numpy()), out=b.out.float().cpu().numpy(),
                         lse=b.lse.cpu().numpy(), sec=_sections(p, b.fp4),
                         fp4_bytes=apa.fp4_bytes(p))
    return res, (Q, K, V)


def assert_same(res):
    a, b = res["ref"], res["ring"]
    for key in ("m", "l", "o", "lam", "hot", "out", "lse"):
        assert np.array_equal(np.nan_to_num(a[key]), np.nan_to_num(b[key])), key
    for key in a["sec"]:
        assert np.array_equal(a["sec"][key], b["sec"][key]), key
    assert int(b["sec"]["status"].view(np.uint32)[0]) == 0


@pytest.mark.parametrize("case", [
    # Hq, Hkv, Nq, Nkv, D, dtype, R, eps, q_terms, causal
    (6, 2, 200, 9000, 128, "fp16", 32, 0.01, 1, 1),   # GQA 3, ragged, 5 segments
    (8, 2, 96, 12288, 64, "bf16", 64, 0.005, 1, 1),   # GQA 4, three segments of 64
    (4, 1, 64, 6144, 256, "fp16", 32, 0.02, 1, 1),    # D = 256, segments of 32
    (6, 2, 128, 8192, 128, "fp16", 96, 0.01, 2, 1),   # two Q terms, R = 96
    (4, 2, 64, 4000, 128, "fp16", 32, 0.02, 1, 0),    # non-causal
    (4, 2, 64, 1000, 128, "fp16", 96, 0.02, 1, 1),    # one segment: first and last launch
], ids=["gqa3_D128", "bf16_D64", "D256", "two_term_q", "noncausal", "one_segment"])
def test_ring_equals_the_unbroken_walk(case):
    Hq, Hkv, Nq, Nkv, D, dtype, R, eps, qt, causal = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, dtype=dtype, causal=causal, seed=91,
                       mode="gauss" if dtype == "bf16" else "path")
    res, (Q, K, V) = run_both(w, R, eps, q_terms=qt)
    assert_same(res)
    assert res["ring"]["fp4_bytes"] < res["ref"]["fp4_bytes"] or Nkv <= 64 * (1 + 2 * R)
    # and the oracle, as for the unbroken walk
    po = O.Params(1, Hq, Hkv, Nq, Nkv, D, scale=w.scale, eps=eps, causal=causal, q_terms=qt)
    r = O.run(po, Q, K, V, O.quantize(po, Q, K, V))
    check_mask(res["ring"]["hot"], r)
    check_output(res["ring"]["out"], r["O"], dtype=dtype)


def test_ring_long3b():
    """The headline shape, 2048 x 122880, with the page's R = 96: 20
    segments; the FP4 K/V copy is 193 tiles per KV head instead of 1920."""
    w = WORKLOADS["long3b"]
    res, _ = run_both(w, 96, w.eps, tensors=make_inputs(w, threads=16))
    assert_same(res)
    print("[ring long3b] FP4 buffer %d MB against %d MB" % (res["ring"]["fp4_bytes"] >> 20,
                                                           res["ref"]["fp4_bytes"] >> 20),
          flush=True)


def test_ring_over_paged_kv():
    """The ring reads its 16-bit K/V through a block table like every other
    call: paged pools (unused slots NaN) give the flat ring's results bit for
    bit, with a clean status word."""
    from test_gpu_chunked import _pages
    B, Hq, Hkv, Nq, Nkv, D, R = 2, 6, 2, 160, 7000, 128, 32
    w = small_workload(B, Hq, Hkv, Nq, Nkv, D, seed=93)
    Q, K, V = make_inputs(w)
    NT = -(-Nkv // 64)
    npages = B * NT + 3
    perm = np.random.default_rng(4).permutation(npages)[:B * NT].reshape(B, NT).astype(np.int32)
    bt = torch.from_numpy(np.ascontiguousarray(perm)).cuda()
    kp, vp = (_pages(x, B, Hkv, Nkv, D, perm, npages, torch.float16) for x in (K, V))
    q = torch.from_numpy(Q).half().cuda()
    kf, vf = (torch.from_numpy(x).half().cuda() for x in (K, V))
    eps = 0.01
    outs = []
    for kk, vv, table in ((kf, vf, None), (kp, vp, bt)):
        p = apa.problem(B, Hq, Hkv, Nq, Nkv, D, scale=w.scale, ring_tiles=R, block_table=table)
        b = apa.alloc(p, with_lambda=True)
        b.fp4.zero_()  # the sections' alignment padding is never written
        apa.ring_pass1(p, q, kk, vv, b.fp4, eps, b.cold_m, b.cold_l, b.cold_o, b.bits, b.lam,
                       ws=b.ws_ring)
        apa.pass2(p, q, kk, vv, b.fp4, b.bits, b.cold_m, b.cold_l, b.cold_o, True, out=b.out,
                  lse=b.lse, ws=b.ws_p2)
        torch.cuda.synchronize()
        outs.append(dict(m=b.cold_m.cpu().numpy(), o=b.cold_o.cpu().numpy(),
                         bits=b.bits.cpu().numpy(), out=b.out.float().cpu().numpy(),
                         sec=_sections(p, b.fp4)))
    a, c = outs
    for key in ("m", "o", "bits", "out"):
        assert np.array_equal(np.nan_to_num(a[key]), np.nan_to_num(c[key])), key
    for key in a["sec"]:
        assert np.array_equal(a["sec"][key], c["sec"][key]), key
    assert int(c["sec"]["status"].view(np.uint32)[0]) == 0
