"""Thin ctypes binding of libapa.so (declared in include/apa.h).

Argument marshalling only: every step of the method runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  Loading
fails loudly if the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libapa.so")

APA_OK, APA_ERR_INVALID_ARG, APA_ERR_UNSUPPORTED, APA_ERR_WORKSPACE, APA_ERR_HIP = range(5)
APA_F16, APA_BF16 = 0, 1
APA_MXFP4, APA_NVFP4 = 0, 1
SCHED_AUTO, SCHED_WHOLE, SCHED_PAIRS, SCHED_TRIPLES = range(4)
CALL_QUANTIZE, CALL_PASS1, CALL_PASS2, CALL_MERGE, CALL_EXACT, CALL_RING_PASS1, CALL_FUSED = range(7)

EXPORTS = ["apa_problem_init", "apa_fp4_layout_of", "apa_fp4_bytes", "apa_hotmask_bytes",
           "apa_workspace_bytes", "apa_status_string", "apa_last_hip_error", "apa_quantize",
           "apa_quantize_static", "apa_quantize_tiles", "apa_pass1",
           "apa_pass1_split", "apa_pass2", "apa_merge", "apa_exact", "apa_ring_pass1",
           "apa_fused"]


class ApaError(RuntimeError):
    def __init__(self, code: int, what: str):
        msg = "%s failed: %s" % (what, status_string(code))
        if code == APA_ERR_HIP:
            msg += " (%s)" % lib().apa_last_hip_error().decode()
        super().__init__(msg)
        self.code = code


class Problem(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("Nq", C.c_int32),
                ("Nkv", C.c_int32), ("D", C.c_int32), ("dtype", C.c_int32),
                ("is_causal", C.c_int32), ("scale", C.c_float), ("tile", C.c_int32),
                ("row_group", C.c_int32), ("fmt", C.c_int32), ("tau", C.c_float),
                ("hot_frame_offset", C.c_float), ("pass1_schedule", C.c_int32),
                ("q_terms", C.c_int32), ("k_scale_lsq", C.c_int32), ("window", C.c_int32),
                ("kv_capacity", C.c_int32), ("stat_keys", C.c_int32),
                ("block_table", C.c_void_p), ("block_table_stride", C.c_int32),
                ("hot_weight", C.c_int32), ("ring_tiles", C.c_int32)]


class Fp4Layout(C.Structure):
    _fields_ = [(k, C.c_size_t) for k in ("q_codes", "q_scales", "kv_blobs", "kbar", "kv_head",
                                          "tile_w", "q_head", "q_frame", "status", "q2_codes",
                                          "q2_scales", "total")]


_lib = None


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libapa.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        # PyTorch ships its own HIP runtime (same soname).  Load it first so the
        # library binds to that one runtime instead of pulling in a second.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        P, VP, S = C.POINTER(Problem), C.c_void_p, C.c_size_t
        L.apa_problem_init.argtypes = [P] + [C.c_int32] * 6
        L.apa_problem_init.restype = None
        L.apa_fp4_layout_of.argtypes = [P, C.POINTER(Fp4Layout)]
        L.apa_fp4_bytes.argtypes = [P]
        L.apa_fp4_bytes.restype = S
        L.apa_hotmask_bytes.argtypes = [P]
        L.apa_hotmask_bytes.restype = S
        L.apa_workspace_bytes.argtypes = [P, C.c_int32]
        L.apa_workspace_bytes.restype = S
        L.apa_status_string.argtypes = [C.c_int]
        L.apa_status_string.restype = C.c_char_p
        L.apa_last_hip_error.argtypes = []
        L.apa_last_hip_error.restype = C.c_char_p
        L.apa_pass1_split.argtypes = [P, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
        L.apa_pass1_split.restype = C.c_int32
        L.apa_quantize.argtypes = [P, VP, VP, VP, VP, VP, S, VP]
        L.apa_quantize_static.argtypes = [P, VP, VP, VP, VP, VP]
        L.apa_quantize_tiles.argtypes = [P, VP, VP, VP, VP, C.c_int32, C.c_int32, VP, S, VP]
        L.apa_pass1.argtypes = [P, VP, C.c_float, VP, VP, VP, VP, VP, VP, S, VP]
        L.apa_ring_pass1.argtypes = [P, VP, VP, VP, VP, C.c_float, VP, VP, VP, VP, VP, VP, S, VP]
        L.apa_pass2.argtypes = [P, VP, VP, VP, VP, VP, VP, VP, VP, C.c_int32, VP, VP, VP, VP, VP,
                                VP, S, VP]
        L.apa_fused.argtypes = [P, VP, VP, VP, VP, C.c_float, VP, VP, VP, VP, VP, VP, VP, VP, S,
                                VP]
        L.apa_merge.argtypes = [P, VP, VP, VP, VP, VP, VP, VP, VP, VP, VP]
        L.apa_exact.argtypes = [P, VP, VP, VP, VP, VP, VP, S, VP]
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().apa_status_string(int(code)).decode()


def problem(B, Hq, Hkv, Nq, Nkv, D, *, dtype=APA_F16, causal=1, scale=0.0, tau=4.0, hoff=32.0,
            fmt=APA_MXFP4, sched=SCHED_AUTO, q_terms=1, k_lsq=0, window=0, kv_capacity=0,
            stat_keys=0, block_table=None, hot_weight=0, ring_tiles=0) -> Problem:
    """block_table: a device int32 tensor [B, stride] of page indices (paged
    K/V), or None; hot_weight: 1 for the value-norm weighted hot test;
    ring_tiles: tiles per half of a KV window ring (0: none)."""
    p = Problem()
    lib().apa_problem_init(C.byref(p), B, Hq, Hkv, Nq, Nkv, D)
    p.dtype, p.is_causal, p.scale, p.tau, p.hot_frame_offset, p.fmt, p.pass1_schedule = (
        dtype, causal, scale, tau, hoff, fmt, sched)
    p.q_terms = q_terms
    p.k_scale_lsq = k_lsq
    p.window = window
    p.kv_capacity = kv_capacity
    p.stat_keys = stat_keys
    p.hot_weight = hot_weight
    p.ring_tiles = ring_tiles
    if block_table is not None:
        p.block_table = block_table.data_ptr()
        p.block_table_stride = block_table.shape[-1]
    return p


def fp4_layout(p: Problem) -> Fp4Layout:
    L = Fp4Layout()
    _check(lib().apa_fp4_layout_of(C.byref(p), C.byref(L)), "apa_fp4_layout_of")
    return L


def fp4_bytes(p: Problem) -> int:
    return lib().apa_fp4_bytes(C.byref(p))


def hotmask_bytes(p: Problem) -> int:
    return lib().apa_hotmask_bytes(C.byref(p))


def workspace_bytes(p: Problem, call: int) -> int:
    return lib().apa_workspace_bytes(C.byref(p), call)


def pass1_split(p: Problem, npos: int):
    """(schedule, first tail position, records per block) of apa_pass1 with a
    workspace for a visit order of npos positions (host-only query)."""
    cut, rec = C.c_int32(0), C.c_int32(0)
    s = lib().apa_pass1_split(C.byref(p), int(npos), C.byref(cut), C.byref(rec))
    if s < 0:
        raise ApaError(APA_ERR_INVALID_ARG, "apa_pass1_split")
    return int(s), int(cut.value), int(rec.value)


def _check(code: int, what: str):
    if code != APA_OK:
        raise ApaError(code, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------
# calls on torch tensors (device memory); all asynchronous on the stream
# ---------------------------------------------------------------------------

def quantize(p: Problem, q, k, v, fp4, ws, stream=None):
    _check(lib().apa_quantize(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fp4), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream)), "apa_quantize")


def quantize_tiles(p: Problem, q, k, v, fp4, tile_begin: int, tile_end: int, ws,
                   stream=None):
    """Q and the K/V tiles [tile_begin, tile_end) with the cache's statistics."""
    _check(lib().apa_quantize_tiles(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fp4),
                                    int(tile_begin), int(tile_end), _ptr(ws),
                                    0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)), "apa_quantize_tiles")


def quantize_static(p: Problem, q, k, v, fp4, stream=None):
    """apa_quantize with the library's fixed scratch (allocates nothing)."""
    _check(lib().apa_quantize_static(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fp4),
                                     _stream(stream)), "apa_quantize_static")


def pass1(p: Problem, fp4, eps: float, cold_m, cold_l, cold_o, hot_bits, lam=None, ws=None,
          stream=None):
    """Pass 1.  ws: workspace of workspace_bytes(p, CALL_PASS1) bytes (may be
    None when that is 0)."""
    _check(lib().apa_pass1(C.byref(p), _ptr(fp4), float(eps), _ptr(cold_m), _ptr(cold_l),
                           _ptr(cold_o), _ptr(hot_bits), _ptr(lam), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "apa_pass1")


def ring_pass1(p: Problem, q, k, v, fp4, eps: float, cold_m, cold_l, cold_o, hot_bits, lam=None,
               ws=None, stream=None):
    """Quantise and pass 1 over a KV window ring.  ws: workspace of
    workspace_bytes(p, CALL_RING_PASS1) bytes."""
    _check(lib().apa_ring_pass1(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fp4), float(eps),
                                _ptr(cold_m), _ptr(cold_l), _ptr(cold_o), _ptr(hot_bits),
                                _ptr(lam), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(),
                                _stream(stream)),
           "apa_ring_pass1")


def pass2(p: Problem, q, k, v, fp4, hot_bits, cold_m, cold_l, cold_o, fuse_merge: bool, out=None,
          lse=None, hot_m=None, hot_l=None, hot_o=None, ws=None, stream=None):
    _check(lib().apa_pass2(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fp4), _ptr(hot_bits),
                           _ptr(cold_m), _ptr(cold_l), _ptr(cold_o), 1 if fuse_merge else 0,
                           _ptr(out), _ptr(lse), _ptr(hot_m), _ptr(hot_l), _ptr(hot_o), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "apa_pass2")


def fused(p: Problem, q, k, v, fp4, eps: float, cold_m, cold_l, cold_o, hot_bits, out, lse=None,
          lam=None, ws=None, stream=None):
    """Pass 1 and pass 2 (fused merge) in one persistent launch.  ws: workspace
    of workspace_bytes(p, CALL_FUSED) bytes."""
    _check(lib().apa_fused(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(fp4), float(eps),
                           _ptr(cold_m), _ptr(cold_l), _ptr(cold_o), _ptr(hot_bits), _ptr(lam),
                           _ptr(out), _ptr(lse), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "apa_fused")


def merge(p: Problem, fp4, cold_m, cold_l, cold_o, hot_m, hot_l, hot_o, out, lse=None,
          stream=None):
    _check(lib().apa_merge(C.byref(p), _ptr(fp4), _ptr(cold_m), _ptr(cold_l), _ptr(cold_o),
                           _ptr(hot_m), _ptr(hot_l), _ptr(hot_o), _ptr(out), _ptr(lse),
                           _stream(stream)), "apa_merge")


def exact(p: Problem, q, k, v, out, lse=None, ws=None, stream=None):
    """All-exact 16-bit attention.  ws: workspace of workspace_bytes(p,
    CALL_EXACT) bytes (allocated here as a torch tensor when not given)."""
    if ws is None:
        need = workspace_bytes(p, CALL_EXACT)
        if need > 0:
            import torch
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib().apa_exact(C.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws),
                           0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "apa_exact")


@dataclass
class Buffers:
    """Device buffers of one APA problem (allocated once, reused per call)."""
    fp4: object
    ws_q: object
    ws_p1: object
    ws_p2: object
    ws_ex: object
    cold_m: object
    cold_l: object
    cold_o: object
    bits: object
    lam: object
    out: object
    lse: object
    ws_ring: object = None  # KV window ring problems: the ring pass's workspace
    ws_fused: object = None  # problems the single launch covers: its workspace


def alloc(p: Problem, device="cuda", with_lambda: bool = False,
          with_fused: bool = False) -> Buffers:
    import torch
    B, Hq, Nq, D = p.B, p.Hq, p.Nq, p.D

    def u8(n):
        return torch.empty(max(int(n), 1), dtype=torch.uint8, device=device)

    odt = torch.float16 if p.dtype == APA_F16 else torch.bfloat16
    return Buffers(
        fp4=u8(fp4_bytes(p)), ws_q=u8(workspace_bytes(p, CALL_QUANTIZE)),
        ws_p1=u8(workspace_bytes(p, CALL_PASS1)) if workspace_bytes(p, CALL_PASS1) > 0 else None,
        ws_p2=u8(workspace_bytes(p, CALL_PASS2)), ws_ex=u8(workspace_bytes(p, CALL_EXACT)),
        cold_m=torch.empty((B, Hq, Nq), dtype=torch.int32, device=device),
        cold_l=torch.empty((B, Hq, Nq), dtype=torch.float32, device=device),
        cold_o=torch.empty((B, Hq, Nq, D), dtype=torch.float32, device=device),
        bits=torch.empty(max(hotmask_bytes(p) // 4, 1), dtype=torch.int32, device=device),
        lam=torch.empty((B, Hq, Nq), dtype=torch.float32, device=device) if with_lambda else None,
        out=torch.empty((B, Hq, Nq, D), dtype=odt, device=device),
        lse=torch.empty((B, Hq, Nq), dtype=torch.float32, device=device),
        ws_ring=u8(workspace_bytes(p, CALL_RING_PASS1)) if p.ring_tiles > 0 else None,
        ws_fused=(u8(workspace_bytes(p, CALL_FUSED))
                  if with_fused and workspace_bytes(p, CALL_FUSED) > 0 else None))


def apa_forward(p: Problem, q, k, v, eps: float, bufs: Buffers, stream=None):
    """The whole hot path: quantize -> pass 1 -> pass 2 with the fused merge."""
    quantize(p, q, k, v, bufs.fp4, bufs.ws_q, stream)
    pass1(p, bufs.fp4, eps, bufs.cold_m, bufs.cold_l, bufs.cold_o, bufs.bits, bufs.lam,
          ws=bufs.ws_p1, stream=stream)
    pass2(p, q, k, v, bufs.fp4, bufs.bits, bufs.cold_m, bufs.cold_l, bufs.cold_o, True,
          out=bufs.out, lse=bufs.lse, ws=bufs.ws_p2, stream=stream)
    return bufs.out, bufs.lse
