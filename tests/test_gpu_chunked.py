"""Chunked prefill over a persistent FP4 K/V cache, and paged K/V ("What else
is in the box": paged KV and chunked prefill -- pass 2 reads through a block
table; chunked prefill keeps the quantised tiles, quantises only new keys,
and restats once the context has grown by 1.125x).

Chunked prefill: one FP4 buffer with a key capacity serves every chunk; the
first chunk quantises with statistics over its keys, a later chunk within
1.125x of them quantises only its new tiles with those statistics
(apa_quantize_tiles), and a chunk past 1.125x restats.  Each chunk is checked
against the oracle with the same statistics range, and against a one-shot
quantisation of the same problem.

Paged K/V: the K and V tiles of every (batch, kv-head) are scattered over a
page pool through a block table (padding rows and unused pages hold NaN, so
any read of them would show); every output, the cold state, the hot mask and
the all-exact output must equal the flat run's bit for bit."""
import numpy as np
import pytest
import torch

from gpu_util import fp4_sections, problem_for, run_exact_gpu, run_gpu, torch_inputs
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import outlier_value_tiles, make_inputs, small_workload
from oracle import oracle as O
from test_gpu_parity import check_cold_state, check_mask, check_output, check_quant
from test_gpu_weight import check_weights

pytestmark = pytest.mark.gpu

RESTAT = 1.125


@pytest.mark.parametrize("D,dtype,hw", [(128, "fp16", 0), (64, "bf16", 0), (128, "fp16", 1)])
def test_chunked_prefill_over_a_persistent_fp4_cache(D, dtype, hw):
    """hw = 1: the value-norm weighted hot test, whose new tiles take their
    weights against the cache's mean value norm."""
    Hq, Hkv, N = 4, 2, 2400
    chunks = [2048, 2200, 2400]  # 2200 < 1.125 x 2048: tiles only; 2400 > 2304: restat
    w = small_workload(1, Hq, Hkv, N, N, D, dtype=dtype, seed=81)
    Qall, Kall, Vall = make_inputs(w)
    if hw:
        outlier_value_tiles(Vall, 4, 8.0, seed=81)
    eps = 0.02
    cap = N
    # one device copy of K/V at full length; each chunk's problem uses its prefix
    _, kd, vd = torch_inputs(Qall[:, :, :1], Kall, Vall, dtype)
    probs = []
    n0, stat = 0, 0
    for n in chunks:
        restat = stat == 0 or n >= RESTAT * stat
        if restat:
            stat = n
        probs.append((n0, n, stat, restat))
        n0 = n
    fp4_size = max(apa.fp4_bytes(apa.problem(1, Hq, Hkv, n - a, n, D, kv_capacity=cap,
                                             scale=w.scale)) for a, n, _, _ in probs)
    fp4 = torch.zeros(fp4_size, dtype=torch.uint8, device="cuda")
    assert [r for *_, r in probs] == [True, False, True]
    for a, n, stat, restat in probs:
        nq = n - a
        # this chunk's queries (positions a .. n-1), tail-aligned to keys 0 .. n-1
        Q, K, V = Qall[:, :, a:n], Kall[:, :, :n], Vall[:, :, :n]
        qd = torch_inputs(Q, Q[:, :1, :1], Q[:, :1, :1], dtype)[0]
        kk = kd[:, :, :n].contiguous()
        vv = vd[:, :, :n].contiguous()
        p = apa.problem(1, Hq, Hkv, nq, n, D, dtype=apa.APA_F16 if dtype == "fp16" else apa.APA_BF16,
                        scale=w.scale, kv_capacity=cap, stat_keys=0 if stat == n else stat,
                        hot_weight=hw)
        bufs = apa.alloc(p, with_lambda=True)
        bufs.fp4 = fp4
        if restat:
            apa.quantize(p, qd, kk, vv, fp4, bufs.ws_q)
        else:
            apa.quantize_tiles(p, qd, kk, vv, fp4, a // 64, -(-n // 64), bufs.ws_q)
        apa.pass1(p, fp4, eps, bufs.cold_m, bufs.cold_l, bufs.cold_o, bufs.bits, bufs.lam,
                  ws=bufs.ws_p1)
        apa.pass2(p, qd, kk, vv, fp4, bufs.bits, bufs.cold_m, bufs.cold_l, bufs.cold_o, True,
                  out=bufs.out, lse=bufs.lse, ws=bufs.ws_p2)
        torch.cuda.synchronize()
        from gpu_util import unpack_bits
        g = dict(fp4=fp4_sections(p, fp4.cpu().numpy()), m=bufs.cold_m.cpu().numpy(),
                 l=bufs.cold_l.cpu().numpy(), o=bufs.cold_o.cpu().numpy(),
                 hot=unpack_bits(p, bufs.bits.cpu().numpy()), out=bufs.out.float().cpu().numpy(),
                 lse=bufs.lse.cpu().numpy())
        po = O.Params(1, Hq, Hkv, nq, n, D, scale=w.scale, eps=eps,
                      stat_keys=0 if stat == n else stat, hot_weight=hw)
        prep = O.quantize(po, Q, K, V)
        r = O.run(po, Q, K, V, prep)
        check_quant(g, prep)
        if hw:
            check_weights(g, prep)
        mism = check_mask(g["hot"], r)
        check_cold_state(g, r, mism)
        check_output(g["out"], r["O"], dtype=dtype)
        fin = np.isfinite(r["lse"])
        assert np.abs(g["lse"][fin] - r["lse"][fin]).max() <= 2e-3
        # the same problem quantised in one shot with the same statistics
        one = run_gpu(apa.problem(1, Hq, Hkv, nq, n, D,
                                  dtype=apa.APA_F16 if dtype == "fp16" else apa.APA_BF16,
                                  scale=w.scale, stat_keys=0 if stat == n else stat,
                                  hot_weight=hw),
                      Q, K, V, eps, dtype=dtype)
        for key in ("out", "lse", "hot"):
            assert np.array_equal(np.nan_to_num(one[key]), np.nan_to_num(g[key])), key


def _pages(arr, B, Hkv, Nkv, D, perm, npages, dt):
    """[B, Hkv, Nkv, D] -> a page pool [npages, Hkv, 64, D] (tile t of batch b
    at page perm[b, t]); padding rows and unused pages hold NaN."""
    NT = -(-Nkv // 64)
    pool = np.full((npages, Hkv, 64, D), np.nan, np.float32)
    for b in range(B):
        for t in range(NT):
            k0, k1 = 64 * t, min(Nkv, 64 * t + 64)
            pool[perm[b, t], :, :k1 - k0] = arr[b, :, k0:k1]
    return torch.from_numpy(pool).to(dt).cuda()


@pytest.mark.parametrize("case", [
    (2, 6, 2, 200, 3000, 128, "fp16", "path", 0, 0),
    (2, 4, 1, 96, 2048, 512, "bf16", "gauss", 0, 0),
    (1, 4, 2, 128, 5000, 64, "fp16", "path", 1500, 0),   # with a sliding window
    (2, 6, 2, 200, 3000, 128, "fp16", "path", 0, 1),     # value-norm weighted test
], ids=["gqa3_D128", "bf16_D512", "window", "weighted"])
def test_paged_kv_equals_flat(case):
    B, Hq, Hkv, Nq, Nkv, D, dtype, mode, window, hw = case
    w = small_workload(B, Hq, Hkv, Nq, Nkv, D, dtype=dtype, mode=mode, seed=82)
    Q, K, V = make_inputs(w)
    if hw:
        outlier_value_tiles(V, 4, 8.0, seed=82)
    eps = 0.02
    NT = -(-Nkv // 64)
    npages = B * NT + 5
    perm = np.random.default_rng(3).permutation(npages)[:B * NT].reshape(B, NT).astype(np.int32)
    dt = torch.float16 if dtype == "fp16" else torch.bfloat16
    bt = torch.from_numpy(np.ascontiguousarray(perm)).cuda()
    kp, vp = (_pages(x, B, Hkv, Nkv, D, perm, npages, dt) for x in (K, V))
    q = torch.from_numpy(Q).to(dt).cuda()
    kw = dict(dtype=apa.APA_F16 if dtype == "fp16" else apa.APA_BF16, scale=w.scale,
              window=window, hot_weight=hw)
    flat = run_gpu(apa.problem(B, Hq, Hkv, Nq, Nkv, D, **kw), Q, K, V, eps, dtype=dtype)
    paged = run_gpu(apa.problem(B, Hq, Hkv, Nq, Nkv, D, block_table=bt, **kw), Q, K, V, eps,
                    dtype=dtype, tensors=(q, kp, vp))
    assert paged["fp4"]["status"] == 0  # no NaN padding row or page was read
    for key in ("m", "l", "o", "hot", "out", "lse"):
        assert np.array_equal(np.nan_to_num(flat[key]), np.nan_to_num(paged[key])), key
    # the codes the library writes (with a window: from the first visible tile)
    t0 = max(0, Nkv - Nq - window + 1) // 64 if window else 0
    cut = {"kc": (2, 64), "ks": (2, 64), "vc": (3, 32), "vs": (3, 2)}
    cut["tile_w"] = (2, 1)
    for key in ("kc", "ks", "vc", "vs", "qc", "qs", "kbar", "kv_head", "q_head", "q_frame") + (
            ("tile_w",) if hw else ()):
        a, b = flat["fp4"][key], paged["fp4"][key]
        if key in cut:
            ax, per = cut[key]
            a, b = np.take(a, range(t0 * per, a.shape[ax]), ax), np.take(b, range(t0 * per, b.shape[ax]), ax)
        assert np.array_equal(a, b), key
    fo, fl = run_exact_gpu(apa.problem(B, Hq, Hkv, Nq, Nkv, D, **kw), Q, K, V, dtype=dtype)
    po_, pl = run_exact_gpu(apa.problem(B, Hq, Hkv, Nq, Nkv, D, block_table=bt, **kw), Q, K, V,
                            dtype=dtype, tensors=(q, kp, vp))
    assert np.array_equal(fo, po_) and np.array_equal(fl, pl)
