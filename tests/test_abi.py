"""The C ABI without a GPU: the library loads, exports every function
include/apa.h declares, and validates its arguments (status codes, size
queries) before anything would be enqueued."""
import ctypes as C
import math
import os
import re

import pytest

from mixed_precision_long_amd import apa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = C.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "apa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(apa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 11
    L = apa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(apa.EXPORTS)


def test_status_strings():
    for code in range(5):
        s = apa.status_string(code)
        assert s.startswith("APA_")
    assert "unknown" in apa.status_string(99)


def prob(**kw):
    p = apa.problem(1, 24, 8, 2048, 122880, 128)
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def test_sizes_and_layout():
    p = prob()
    L = apa.fp4_layout(p)
    # the K/V sections first (a persistent cache keeps them), then the queries'
    offs = [L.kv_blobs, L.kbar, L.kv_head, L.status, L.q_codes, L.q_scales, L.q_head, L.q_frame,
            L.q2_codes, L.q2_scales, L.total]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs) and L.kv_blobs == 0
    # one Q term: the residual sections are empty; two: each as large as Q's
    assert L.q2_scales == L.q2_codes == L.total
    L2 = apa.fp4_layout(prob(q_terms=2))
    assert L2.q2_scales - L2.q2_codes == L.q_scales - L.q_codes
    assert L2.total - L2.q2_scales >= 24 * 2048 * 4
    assert [L2.q_codes, L2.kv_blobs, L2.status] == [L.q_codes, L.kv_blobs, L.status]
    assert L.q_frame - L.q_head >= 24 * 4 * 4
    # one 68*D-byte blob per 64-key tile and kv-head: 8704 B at D = 128
    assert L.kbar - L.kv_blobs == 8 * 1920 * 8704
    assert apa.fp4_bytes(p) == L.total
    assert apa.hotmask_bytes(p) == 24 * 128 * 60 * 4
    assert apa.workspace_bytes(p, apa.CALL_PASS1) > 0
    # a capacity sizes the K/V sections and keeps them where they are for any
    # Nq and any Nkv up to it (a persistent FP4 cache across chunks)
    cap = [apa.fp4_layout(prob(Nq=nq, Nkv=nkv, kv_capacity=131072))
           for nq, nkv in ((2048, 122880), (512, 65536), (64, 100000))]
    for c in cap:
        assert (c.kv_blobs, c.kbar, c.kv_head, c.status) == (cap[0].kv_blobs, cap[0].kbar,
                                                             cap[0].kv_head, cap[0].status)
        assert c.kbar - c.kv_blobs == 8 * 2048 * 8704
    # enough row blocks to fill the GPU, or visit orders too short to cut:
    # pass 1 runs one wave per block and needs no workspace
    assert apa.workspace_bytes(prob(Nq=32768, Nkv=32768, Hq=32), apa.CALL_PASS1) == 0
    assert apa.workspace_bytes(prob(Nkv=4000), apa.CALL_PASS1) == 0
    assert apa.workspace_bytes(p, apa.CALL_QUANTIZE) > 0
    assert apa.workspace_bytes(p, apa.CALL_PASS2) > 0
    # ragged shapes round up
    q = prob(Nq=100, Nkv=700)
    assert apa.hotmask_bytes(q) == 24 * 7 * 1 * 4


@pytest.mark.parametrize("field,value", [
    ("Hkv", 5), ("D", 96), ("tile", 32), ("row_group", 8), ("Nkv", 1000), ("dtype", 7),
    ("is_causal", 2), ("tau", -1.0), ("tau", 40.0), ("hot_frame_offset", 2.5),
    ("hot_frame_offset", 65.0),
    ("scale", float("nan")), ("fmt", 9), ("pass1_schedule", -1), ("pass1_schedule", 4),
    ("q_terms", 0), ("q_terms", 3), ("k_scale_lsq", 2), ("window", -1),
    ("window+noncausal", 4096), ("kv_capacity", 1000), ("kv_capacity", -1),
    ("stat_keys", -1), ("stat_keys", 200000), ("block_table_stride", 1000),
    ("ring_tiles", -32), ("ring_tiles", 96 + 16)])
def test_invalid_problems_are_rejected(field, value):
    if field == "window+noncausal":
        p = prob(window=value, is_causal=0)  # a sliding window needs the causal mask
    elif field == "block_table_stride":
        # a block table needs an entry for every tile of a batch row
        p = prob(block_table=FAKE.value, block_table_stride=value)
    else:
        p = prob(**{field: value})
    assert apa.lib().apa_quantize(C.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == \
        apa.APA_ERR_INVALID_ARG
    assert apa.fp4_bytes(p) == 0


def test_null_pointers_and_bad_arguments():
    L = apa.lib()
    p = prob()
    assert L.apa_quantize(None, FAKE, FAKE, FAKE, FAKE, FAKE, 1, None) == apa.APA_ERR_INVALID_ARG
    assert L.apa_quantize(C.byref(p), None, FAKE, FAKE, FAKE, FAKE, 1, None) == apa.APA_ERR_INVALID_ARG
    assert L.apa_pass1(C.byref(p), FAKE, 0.01, None, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                       None) == apa.APA_ERR_INVALID_ARG
    for eps in (float("nan"), -0.1):
        assert L.apa_pass1(C.byref(p), FAKE, eps, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40,
                           None) == apa.APA_ERR_INVALID_ARG
    # pass 2: fuse flag, and the pointers each mode needs
    args = [FAKE] * 8
    assert L.apa_pass2(C.byref(p), *args, 2, FAKE, None, None, None, None, FAKE, 1 << 40, None) == \
        apa.APA_ERR_INVALID_ARG
    assert L.apa_pass2(C.byref(p), *args, 1, None, None, None, None, None, FAKE, 1 << 40, None) == \
        apa.APA_ERR_INVALID_ARG
    assert L.apa_pass2(C.byref(p), *args, 0, None, None, None, None, None, FAKE, 1 << 40, None) == \
        apa.APA_ERR_INVALID_ARG
    assert L.apa_merge(C.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None) == \
        apa.APA_ERR_INVALID_ARG
    assert L.apa_exact(C.byref(p), FAKE, FAKE, None, FAKE, None, None, 0, None) == \
        apa.APA_ERR_INVALID_ARG


def test_workspace_too_small():
    L = apa.lib()
    p = prob()
    need = apa.workspace_bytes(p, apa.CALL_QUANTIZE)
    assert L.apa_quantize(C.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        apa.APA_ERR_WORKSPACE
    assert L.apa_quantize(C.byref(p), FAKE, FAKE, FAKE, FAKE, None, need, None) == \
        apa.APA_ERR_WORKSPACE
    few = prob(Nq=256)  # few row blocks: the key range runs as several splits
    need_ex = apa.workspace_bytes(few, apa.CALL_EXACT)
    assert need_ex > 0
    assert L.apa_exact(C.byref(few), FAKE, FAKE, FAKE, FAKE, None, FAKE, need_ex - 1, None) == \
        apa.APA_ERR_WORKSPACE
    # pass 1 runs split (two waves per 32-row block) while the blocks do not
    # fill the GPU: 1536 of them at 2048 x 122880 with 24 over 8 heads
    need1 = apa.workspace_bytes(p, apa.CALL_PASS1)
    assert need1 > 0
    assert L.apa_pass1(C.byref(p), FAKE, 0.01, FAKE, FAKE, FAKE, FAKE, None, FAKE, need1 - 1,
                       None) == apa.APA_ERR_WORKSPACE
    need2 = apa.workspace_bytes(p, apa.CALL_PASS2)
    assert L.apa_pass2(C.byref(p), *([FAKE] * 8), 1, FAKE, None, None, None, None, FAKE, need2 - 1,
                       None) == apa.APA_ERR_WORKSPACE


def test_unsupported_variants_say_so():
    L = apa.lib()
    nv = prob(fmt=apa.APA_NVFP4)
    assert L.apa_quantize(C.byref(nv), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == \
        apa.APA_ERR_UNSUPPORTED
    big2 = prob(D=512, q_terms=2)  # the second Q term stops at D = 256
    assert L.apa_quantize(C.byref(big2), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == \
        apa.APA_ERR_UNSUPPORTED
    assert L.apa_pass1(C.byref(big2), FAKE, 0.01, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                       None) == apa.APA_ERR_UNSUPPORTED
    g5 = prob(Hq=40)  # group of 5 query heads
    assert L.apa_exact(C.byref(g5), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == \
        apa.APA_ERR_UNSUPPORTED


def test_empty_problems_do_nothing():
    L = apa.lib()
    for kw in ({"Nq": 0}, {"B": 0}):
        p = prob(**kw)
        assert L.apa_pass1(C.byref(p), FAKE, 0.01, FAKE, FAKE, FAKE, FAKE, None, None, 0,
                           None) == apa.APA_OK
        assert L.apa_exact(C.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, 0, None) == apa.APA_OK
        assert L.apa_merge(C.byref(p), *([FAKE] * 8), None, None) == apa.APA_OK
        assert L.apa_pass2(C.byref(p), *([FAKE] * 8), 1, FAKE, None, None, None, None, FAKE, 1 << 40,
                           None) == apa.APA_OK


def test_problem_defaults():
    p = apa.problem(2, 8, 2, 16, 64, 64)
    assert (p.tile, p.row_group, p.tau, p.hot_frame_offset, p.is_causal) == (64, 16, 4.0, 32.0, 1)
    assert p.scale == 0.0 and p.fmt == apa.APA_MXFP4 and p.dtype == apa.APA_F16
    assert p.pass1_schedule == apa.SCHED_AUTO and p.q_terms == 1 and p.k_scale_lsq == 0
    assert math.isfinite(p.tau)


def test_pass1_schedule_sizes_the_workspace():
    """The pass-1 workspace follows the schedule a launch would run: none for
    one wave per block; per block the outcome word, the records of a tail (at
    most 512, up to the longest tail of the schedule's cut) and the hand-off
    area.  The 2048 x 122880 shape (1536 blocks) runs the triple schedule by
    default, with shorter tails than the pair schedule."""
    def ws(sched, **kw):
        return apa.workspace_bytes(prob(pass1_schedule=sched, **kw), apa.CALL_PASS1)
    units = 24 * 2048 // 32
    auto, pairs, triples = ws(apa.SCHED_AUTO), ws(apa.SCHED_PAIRS), ws(apa.SCHED_TRIPLES)
    assert ws(apa.SCHED_WHOLE) == 0
    assert auto == triples and 0 < triples < pairs
    hand = (128 * 128 + 1040 + 255) // 256 * 256
    for total, sched in ((pairs, apa.SCHED_PAIRS), (triples, apa.SCHED_TRIPLES)):
        p = prob(pass1_schedule=sched)
        # records: the longest tail of any visit order up to 1920 positions
        cap = min(512, max(n - apa.pass1_split(p, n)[1] for n in range(1921)))
        assert cap == apa.pass1_split(p, 1920)[2] and cap > 300
        assert total == units * ((cap * 292 + 16 + 255) // 256 * 256 + hand)
    # few blocks: pairs by default; at D = 512 every unit runs as two waves
    # (one per half of the output channels) and is never cut
    assert ws(apa.SCHED_AUTO, Nq=64) == ws(apa.SCHED_PAIRS, Nq=64)
    for sched in (apa.SCHED_AUTO, apa.SCHED_PAIRS, apa.SCHED_TRIPLES):
        assert ws(sched, D=512, Nq=64) == 0


@pytest.mark.parametrize("sched", [apa.SCHED_PAIRS, apa.SCHED_TRIPLES])
def test_pass1_split_points(sched):
    """Every visit order is either walked whole or cut so that the head walks
    at least the 32 positions the tail replays and the tail walks at least 8
    of its own: never past the end of the order (a cut at or beyond it would
    visit tiles that do not exist)."""
    p = prob(pass1_schedule=sched)
    NT = -(-p.Nkv // 64)
    s, _, rec = apa.pass1_split(p, 0)
    assert s == sched and 0 < rec <= 512
    longest = 0
    cut_any = False
    for npos in range(0, NT + 1):
        s2, cut, rec2 = apa.pass1_split(p, npos)
        assert (s2, rec2) == (s, rec)
        if cut == npos:
            assert npos < 64 or sched == apa.SCHED_TRIPLES, npos
            continue
        cut_any = True
        assert 32 <= cut <= npos - 8, (npos, cut)
        longest = max(longest, npos - cut)
    assert cut_any and rec == min(512, longest)
    # under the triple rule short orders (64 .. 108 positions among them) run whole
    if sched == apa.SCHED_TRIPLES:
        assert all(apa.pass1_split(p, n)[1] == n for n in range(64, 109))


def test_pass1_split_whole_without_tails():
    # a problem whose every order is too short to cut runs one wave per block
    p = prob(Nkv=4000)
    assert apa.pass1_split(p, 60) == (apa.SCHED_WHOLE, 60, 0)
    assert apa.pass1_split(prob(D=512), 1000) == (apa.SCHED_WHOLE, 1000, 0)
    with pytest.raises(apa.ApaError):
        apa.pass1_split(prob(D=96), 10)


def test_quantize_tiles_validates_its_range():
    L = apa.lib()
    p = prob()
    need = apa.workspace_bytes(p, apa.CALL_QUANTIZE)
    for tb, te in ((-1, 10), (5, 4), (0, 1921)):
        assert L.apa_quantize_tiles(C.byref(p), FAKE, FAKE, FAKE, FAKE, tb, te, FAKE, need,
                                    None) == apa.APA_ERR_INVALID_ARG
    assert L.apa_quantize_tiles(C.byref(p), FAKE, FAKE, FAKE, FAKE, 0, 10, FAKE, need - 1,
                                None) == apa.APA_ERR_WORKSPACE
    # with a window the range starts at the window's first tile
    pw = prob(window=4096)
    first = (122880 - 2048 - 4096 + 1) // 64
    assert L.apa_quantize_tiles(C.byref(pw), FAKE, FAKE, FAKE, FAKE, first - 1, 1920, FAKE,
                                need, None) == apa.APA_ERR_INVALID_ARG


def test_ring_problems():
    """A KV window ring: the FP4 buffer holds 1 + 2R tile blobs per kv-head
    whatever Nkv is; only apa_ring_pass1 fills and walks them; it needs
    D <= 256, no window and the mass test; its workspace is the quantise
    scratch and a hand-off state per 32-row block and query head."""
    L = apa.lib()
    p = prob()  # 2048 x 122880, 24 over 8 heads, D = 128
    r = prob(ring_tiles=96)
    lay, lr = apa.fp4_layout(p), apa.fp4_layout(r)
    blob = 68 * 128
    assert lr.kbar - lr.kv_blobs >= 8 * 193 * blob > lr.kbar - lr.kv_blobs - 256
    assert apa.fp4_bytes(p) - apa.fp4_bytes(r) >= 8 * (1920 - 193) * blob - 4096
    for call in (lambda x: L.apa_quantize(C.byref(x), FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None),
                 lambda x: L.apa_quantize_tiles(C.byref(x), FAKE, FAKE, FAKE, FAKE, 0, 1, FAKE,
                                                1 << 40, None),
                 lambda x: L.apa_pass1(C.byref(x), FAKE, 0.01, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                       1 << 40, None)):
        assert call(r) == apa.APA_ERR_UNSUPPORTED
    ring = lambda x, nbytes: L.apa_ring_pass1(C.byref(x), FAKE, FAKE, FAKE, FAKE, 0.01, FAKE, FAKE,
                                              FAKE, FAKE, None, FAKE, nbytes, None)
    assert ring(p, 1 << 40) == apa.APA_ERR_UNSUPPORTED  # no ring in the problem
    for kw in ({"D": 512}, {"window": 4096}, {"hot_weight": 1}):
        assert ring(prob(ring_tiles=96, **kw), 1 << 40) == apa.APA_ERR_UNSUPPORTED, kw
    need = apa.workspace_bytes(r, apa.CALL_RING_PASS1)
    units = 8 * 64 * 3
    state = units * ((128 * 128 + 1040 + 255) // 256 * 256)
    qneed = (apa.workspace_bytes(r, apa.CALL_QUANTIZE) + 255) // 256 * 256
    assert need == qneed + state
    assert apa.workspace_bytes(p, apa.CALL_RING_PASS1) == 0
    assert ring(r, need - 1) == apa.APA_ERR_WORKSPACE
    assert L.apa_ring_pass1(C.byref(r), FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, FAKE, FAKE,
                            FAKE, None, FAKE, need, None) == apa.APA_ERR_INVALID_ARG


def test_fused_problems():
    """The single launch: covered problems (D 64 or 128, at most 4096 key
    tiles, no ring, the GQA groups of pass 2) have a workspace of control
    words, the pass-1 workspace and the split states; others report 0 bytes
    and get APA_ERR_UNSUPPORTED before any device work; NULL required
    pointers, a NaN eps and a short workspace are refused."""
    L = apa.lib()
    p = prob()  # 2048 x 122880, 24 over 8 heads, D = 128: 1920 tiles
    need = apa.workspace_bytes(p, apa.CALL_FUSED)
    nitems = 8 * ((3 * 64 + 3) // 4)
    ctl = ((64 + 2 * nitems) * 4 + 255) // 256 * 256
    S = 4
    rows = 24 * 2048
    split_states = sum((x + 255) // 256 * 256 for x in (S * rows * 4, S * rows * 4, S * rows * 128 * 4))
    assert need == ctl + apa.workspace_bytes(p, apa.CALL_PASS1) + split_states
    fused = lambda x, ws, nbytes, eps=0.01, out=FAKE: L.apa_fused(
        C.byref(x), FAKE, FAKE, FAKE, FAKE, eps, FAKE, FAKE, FAKE, FAKE, None, out, None, ws,
        nbytes, None)
    for kw in ({"D": 256}, {"D": 512}, {"ring_tiles": 96}, {"Nkv": 4097 * 64}, {"Hq": 40}):
        x = prob(**kw)
        assert apa.workspace_bytes(x, apa.CALL_FUSED) == 0, kw
        assert fused(x, FAKE, 1 << 40) == apa.APA_ERR_UNSUPPORTED, kw
    assert apa.workspace_bytes(prob(D=64), apa.CALL_FUSED) > 0
    assert fused(p, FAKE, need - 1) == apa.APA_ERR_WORKSPACE
    assert fused(p, None, 1 << 40) == apa.APA_ERR_WORKSPACE
    assert fused(p, FAKE, 1 << 40, out=None) == apa.APA_ERR_INVALID_ARG
    assert fused(p, FAKE, 1 << 40, eps=float("nan")) == apa.APA_ERR_INVALID_ARG
