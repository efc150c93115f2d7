"""Boundary behaviour of the C ABI on the GPU: bf16 V beyond the fp16 range
(pass 2 and the exact path scale each head's V into that range by a power of
two and back, so nothing is clamped), and the status word's bit for
non-finite inputs."""
import numpy as np
import pytest

from gpu_util import problem_for, run_exact_gpu, run_gpu
from mixed_precision_long_amd.inputs import make_inputs, small_workload
from oracle import oracle as O
from test_gpu_parity import EXACT_ABS, check_mask, check_output, out_tol

pytestmark = pytest.mark.gpu

BIG = 2.0 ** 20  # |V| up to about 4.7e6, 72 times the fp16 maximum


@pytest.mark.parametrize("D", [128, 512])
def test_bf16_v_beyond_fp16_range_exact(D):
    """apa_exact with bf16 V scaled by 2^20 gives 2^20 times the output for
    the unscaled V (to the bar of the FP64 reference): no clamp at 65504."""
    w = small_workload(1, 4, 1, 96, 640, D, dtype="bf16", mode="gauss", seed=51)
    Q, K, V = make_inputs(w)
    p = problem_for(w)
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale)
    Oe, _ = O.exact(po, Q, K, V)
    assert np.abs(V * BIG).max() > 65504.0 * 64
    go, _ = run_exact_gpu(p, Q, K, V * BIG, dtype="bf16")
    got = go.reshape(-1, D) / BIG
    excess = np.abs(got - Oe) - out_tol(EXACT_ABS, Oe, "bf16")
    assert excess.max() <= 0.0, excess.max()


@pytest.mark.parametrize("D", [128, 512])
def test_bf16_v_beyond_fp16_range_apa(D):
    """The whole APA path with the same scaled V: V's FP4 codes are those of
    the unscaled V and its block exponents 20 larger (V is coded at its own
    scale), the cold state is 2^20 times larger, pass 2 scales its V into the
    fp16 range, and the output over 2^20 meets the usual bars against the
    oracle on the unscaled V."""
    w = small_workload(1, 4, 1, 96, 4096, D, dtype="bf16", mode="gauss", seed=52)
    Q, K, V = make_inputs(w)
    eps = 0.05
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=eps)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w), Q, K, V * BIG, eps, dtype="bf16")
    assert g["fp4"]["status"] == 0
    assert np.array_equal(g["fp4"]["vc"], prep["vc"])
    vs = prep["vs"].astype(np.int32)
    assert np.array_equal(g["fp4"]["vs"], np.where(vs == 0, 0, vs + 20))
    check_mask(g["hot"], r)
    check_output(g["out"] / BIG, r["O"], dtype="bf16")
    # the hot part ran in pass 2 (some tiles hot, some cold)
    assert g["hot"].any() and (g["l"] > 0).any()


def test_bf16_v_beyond_fp16_range_past_the_statistics_keys():
    """Statistics over the first 2048 of 4096 keys, and bf16 V of the later
    keys 2^16 times larger (beyond the fp16 range, unlike any statistics
    key's): the per-head max |V| that pass 2 shifts V by covers every key
    coded, so the output is finite and meets the usual bars against the
    oracle, each row measured against its own largest magnitude.  With
    eps = 0 every tile with any mass is hot, so pass 2 computes all of them
    (a cold tile of the large values would carry FP4 differences 2^16 times
    larger than the rest, whatever the range shift does)."""
    w = small_workload(1, 4, 1, 96, 4096, 128, dtype="bf16", mode="gauss", seed=53)
    Q, K, V = make_inputs(w)
    V[:, :, 2048:] *= 2.0 ** 16
    assert np.abs(V[:, :, :2048]).max() < 65504.0 < np.abs(V[:, :, 2048:]).max()
    eps = 0.0
    po = O.Params(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D, scale=w.scale, eps=eps, stat_keys=2048)
    prep = O.quantize(po, Q, K, V)
    r = O.run(po, Q, K, V, prep)
    g = run_gpu(problem_for(w, stat_keys=2048), Q, K, V, eps, dtype="bf16")
    assert g["fp4"]["status"] == 0
    assert g["fp4"]["kv_head"][0, 0, 3] == np.float32(np.abs(V).max())
    check_mask(g["hot"], r)
    assert np.isfinite(g["out"]).all()
    # the hot part ran in pass 2 on tiles of both ranges
    hot_t = np.flatnonzero(g["hot"].any(axis=(0, 1, 2)))
    assert (hot_t < 32).any() and (hot_t >= 32).any()
    mag = np.abs(r["O"]).max(axis=-1, keepdims=True)
    mag = np.where(mag > 0, mag, 1.0)
    check_output(g["out"] / mag, r["O"] / mag, dtype="bf16")


@pytest.mark.parametrize("where", ["q", "k", "v"])
def test_nonfinite_input_sets_the_status_bit(where):
    """One NaN (or infinity) anywhere in Q, K or V sets bit 0 of the FP4
    buffer's status word; finite inputs leave it clear (checked by every
    parity test)."""
    w = small_workload(1, 2, 1, 64, 512, 64, seed=53)
    Q, K, V = make_inputs(w)
    X = {"q": Q, "k": K, "v": V}[where]
    X[0, 0, 37, 5] = np.nan if where != "v" else np.inf
    g = run_gpu(problem_for(w), Q, K, V, 0.02)
    assert g["fp4"]["status"] & 1 == 1
