"""apa_quantize_static, the quantisation entry point for callers that cannot
allocate (its scratch is the library's fixed device array), against
apa_quantize with a caller workspace: the whole FP4 buffer bit for bit, on
two calls in a row, the second with a smaller problem (so the array holds
the first call's larger contents when the second starts)."""
import numpy as np
import pytest
import torch

from gpu_util import fp4_sections, problem_for, torch_inputs
from mixed_precision_long_amd import apa
from mixed_precision_long_amd.inputs import make_inputs, small_workload

pytestmark = pytest.mark.gpu


def _both(w):
    Q, K, V = make_inputs(w)
    p = problem_for(w)
    q, k, v = torch_inputs(Q, K, V, w.dtype)
    n = apa.fp4_bytes(p)
    a = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    b = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = torch.empty(apa.workspace_bytes(p, apa.CALL_QUANTIZE), dtype=torch.uint8, device="cuda")
    apa.quantize(p, q, k, v, a, ws)
    apa.quantize_static(p, q, k, v, b)
    torch.cuda.synchronize()
    return p, a.cpu().numpy(), b.cpu().numpy()


def test_quantize_static_matches_quantize_twice():
    shapes = [
        small_workload(1, 24, 8, 2048, 8192, 128, seed=2),            # 3B-shaped, larger first
        small_workload(1, 4, 1, 100, 700, 64, dtype="bf16", mode="gauss", seed=61),
    ]
    for w in shapes:
        p, a, b = _both(w)
        assert np.array_equal(a, b)
        sa, sb = fp4_sections(p, a), fp4_sections(p, b)
        assert sa["status"] == 0 and np.array_equal(sa["kc"], sb["kc"])
        assert (sa["kv_head"] != 0).any()


def test_quantize_static_rejects_problems_beyond_its_scratch():
    # about 21 MB of statistics scratch: more than the fixed 16 MiB
    p = apa.problem(1, 10, 10, 64, 1 << 20, 128)
    assert apa.workspace_bytes(p, apa.CALL_QUANTIZE) > 16 << 20
    x = torch.empty(1, dtype=torch.uint8, device="cuda")
    with pytest.raises(apa.ApaError) as e:
        apa.quantize_static(p, x, x, x, x)
    assert e.value.code == apa.APA_ERR_WORKSPACE
