"""Pass 2's hot-tile compaction (the union list each 16-bit attention work
group walks) checked element by element against its definition, on the
GPU's own hot mask: for work group (b, kv-head, four row blocks), every tile
hot for any of its eight 16-row groups, ascending, with a mask whose bit
2w + k says the tile is hot for wave w's k-th group.  Row blocks are
numbered position-major, head-minor inside a kv-head (block j: query head
hk * G + j % G, rows 32 * (j // G) ..).  Also the order pass 2 takes a
head's work groups in: by descending tile count, ties in ascending order.
Index work, so bit-exact; also at the 2048 x 122880 shape."""
import numpy as np
import pytest
import torch

from gpu_util import problem_for, torch_inputs, unpack_bits
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import WORKLOADS, make_inputs, small_workload

pytestmark = pytest.mark.gpu

ORDER_MAX = 2048  # work groups per kv-head up to which pass 2 orders them by list length


def expected_lists(p, hot):
    """hot [B, Hq, NG, NT] bool -> (tiles, masks) per work group."""
    B, Hq, Hkv, Nq = p.B, p.Hq, p.Hkv, p.Nq
    G, NG, NT = Hq // Hkv, hot.shape[2], hot.shape[3]
    nrb = G * -(-Nq // 32)
    nwg = -(-nrb // 4)
    out = []
    for b in range(B):
        for hk in range(Hkv):
            for wg in range(nwg):
                mask = np.zeros(NT, np.uint32)
                for w in range(4):
                    j = wg * 4 + w
                    if j >= nrb:
                        continue
                    h = hk * G + j % G
                    for k in range(2):
                        grp = (j // G) * 2 + k
                        if grp < NG:
                            mask |= hot[b, h, grp].astype(np.uint32) << np.uint32(2 * w + k)
                tiles = np.flatnonzero(mask)
                out.append((tiles.astype(np.int32), mask[tiles]))
    return out


def check(p, q, k, v, eps):
    bufs = apa.alloc(p)
    apa.quantize(p, q, k, v, bufs.fp4, bufs.ws_q)
    apa.pass1(p, bufs.fp4, eps, bufs.cold_m, bufs.cold_l, bufs.cold_o, bufs.bits, None,
              ws=bufs.ws_p1)
    apa.pass2(p, q, k, v, bufs.fp4, bufs.bits, bufs.cold_m, bufs.cold_l, bufs.cold_o, True,
              out=bufs.out, lse=bufs.lse, ws=bufs.ws_p2)
    torch.cuda.synchronize()
    hot = unpack_bits(p, bufs.bits.cpu().numpy())
    want = expected_lists(p, hot)
    units, NT = len(want), hot.shape[3]
    # the pass-2 workspace starts with the lists: tiles [units][NT] int32,
    # masks [units][NT] uint32, counts [units] int32, then the order
    # [units] int32, each 256-byte aligned
    ws = bufs.ws_p2.cpu().numpy()
    a = lambda n: (n + 255) // 256 * 256
    t_off, m_off = 0, a(units * NT * 4)
    c_off = m_off + a(units * NT * 4)
    tiles = ws[t_off:t_off + units * NT * 4].view(np.int32).reshape(units, NT)
    masks = ws[m_off:m_off + units * NT * 4].view(np.uint32).reshape(units, NT)
    count = ws[c_off:c_off + units * 4].view(np.int32)
    for u, (tl, ml) in enumerate(want):
        n = int(count[u])
        assert n == len(tl), (u, n, len(tl))
        assert np.array_equal(tiles[u, :n], tl), u
        assert np.array_equal(masks[u, :n], ml), u
    o_off = c_off + a(units * 4)
    order = ws[o_off:o_off + units * 4].view(np.int32).reshape(p.B * p.Hkv, -1)
    for bk, ordk in enumerate(order):
        cnt = count[bk * len(ordk):(bk + 1) * len(ordk)]
        if len(ordk) > ORDER_MAX:
            want_o = list(range(len(ordk)))  # above the cap: the identity
        else:
            want_o = sorted(range(len(ordk)), key=lambda w: (-int(cnt[w]), w))
        assert np.array_equal(ordk, want_o), bk
    return sum(len(t) for t, _ in want), units


@pytest.mark.parametrize("case", [
    (6, 2, 200, 3000, 128, 0.01, "fp16"),   # GQA 3, ragged rows and keys
    (8, 2, 96, 4096, 64, 0.02, "fp16"),     # GQA 4, a partial last work group
    (4, 1, 96, 2048, 512, 0.02, "bf16"),    # D = 512
])
def test_compaction_matches_its_definition(case):
    Hq, Hkv, Nq, Nkv, D, eps, dtype = case
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, dtype=dtype,
                       mode="gauss" if D == 512 else "path", seed=61)
    Q, K, V = make_inputs(w)
    q, k, v = torch_inputs(Q, K, V, dtype)
    n, units = check(problem_for(w), q, k, v, eps)
    assert n > units


@pytest.mark.parametrize("eps", [0.002, 0.005])
def test_compaction_long3b(eps):
    w = WORKLOADS["long3b"]
    Q, K, V = make_inputs(w, threads=16)
    q, k, v = torch_inputs(Q, K, V)
    n, units = check(problem_for(w), q, k, v, eps)
    print("[long3b eps %g] %d work groups, %d listed tiles" % (eps, units, n), flush=True)


def test_order_is_the_identity_above_the_cap():
    """2049 work groups per kv-head (65568 query rows, GQA 4, non-causal over
    two key tiles): the order is the identity, the lists still match their
    definition, and the output matches the oracle on sampled row groups."""
    from gpu_util import run_gpu
    from oracle import oracle as O
    from test_gpu_parity import check_output
    Hq, Hkv, Nq, Nkv, D = 4, 1, 65568, 128, 64
    w = small_workload(1, Hq, Hkv, Nq, Nkv, D, causal=0, mode="gauss", seed=63)
    Q, K, V = make_inputs(w)
    q, k, v = torch_inputs(Q, K, V)
    p = problem_for(w, causal=0)
    assert -(-(Hq // Hkv) * -(-Nq // 32) // 4) > ORDER_MAX
    eps = 0.7  # the first visited tile is always hot, the second often cold
    check(p, q, k, v, eps)
    g = run_gpu(p, Q, K, V, eps)
    rng = np.random.default_rng(5)
    sel = np.array([(0, h, gg) for h in range(Hq) for gg in rng.choice(-(-Nq // 16), 8, replace=False)],
                   np.int32)
    po = O.Params(1, Hq, Hkv, Nq, Nkv, D, causal=0, scale=w.scale, eps=eps)
    r = O.run(po, Q, K, V, O.quantize(po, Q, K, V), groups=sel)
    rows = np.array([(0, h, gg * 16 + i) for _, h, gg in sel for i in range(16) if gg * 16 + i < Nq])
    check_output(g["out"], r["O"], rows=rows)
