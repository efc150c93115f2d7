"""Python front end of the CPU oracle (``apa_oracle.c``) for adaptive-precision
attention prefill.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module; the product path
(``mixed_precision_long_amd``) never does, and shares no code with it.

The arithmetic lives in ``apa_oracle.c`` (plain scalar C, FP64 where the
method is exact, every FP32 rounding of the method simulated).  This module
only builds that library with gcc, marshals numpy arrays, and strings the
steps together in the order "APA: sloppy attention, exact where it counts"
(rfriedmann.de) gives them: statistics and quantisation ("Mean-centred K",
"Pass 1" format paragraph), pass 1 (numbered steps 1-5), pass 2 ("Pass 2:
exact FP16 on the hot tiles") and the merge ("The merge that makes it exact").
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "apa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MX, NV = 0, 1
# per-operand switches of pass 1's FP4 roundings (see apa_oracle.c, ORC_QUANT_*)
QUANT_Q, QUANT_K, QUANT_V, QUANT_P = 1, 2, 4, 8
QUANT_ALL = 15


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


class _Params(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("Nq", C.c_int32),
                ("Nkv", C.c_int32), ("D", C.c_int32), ("causal", C.c_int32), ("scale", C.c_float),
                ("fmt", C.c_int32), ("int_frame", C.c_int32), ("tau", C.c_float),
                ("hoff", C.c_float), ("eps", C.c_float), ("tile", C.c_int32), ("rg", C.c_int32),
                ("q_terms", C.c_int32), ("k_lsq", C.c_int32), ("qmask", C.c_int32),
                ("window", C.c_int32), ("vweight", C.c_int32)]


_P = C.c_void_p


class _Job(C.Structure):
    _fields_ = [("p", _P), ("Q", _P), ("K", _P), ("V", _P),
                ("qc", _P), ("qs", _P), ("kc", _P), ("ks", _P), ("vc", _P), ("vs", _P),
                ("qc2", _P), ("qs2", _P), ("kbar", _P), ("g_v", _P), ("jq", _P),
                ("inv_q", _P), ("inv_k", _P), ("inv_v", _P), ("vw", _P), ("alpha_q", _P),
                ("groups", _P), ("ngroups", C.c_int),
                ("hot", _P), ("margin", _P), ("m1", _P), ("l1", _P), ("lam", _P), ("o1", _P),
                ("shift", _P), ("m2", _P), ("l2", _P), ("o2", _P), ("cr", _P), ("O", _P),
                ("lse", _P), ("do_pass2", C.c_int), ("next", C.c_int),
                ("mu", C.c_int64 * 8)]


class _ReportJob(C.Structure):
    _fields_ = [("p", _P), ("Q", _P), ("K", _P), ("V", _P), ("hot", _P), ("rows", _P),
                ("nrows", C.c_int), ("O_ref", _P), ("O_hot", _P), ("O_cold", _P), ("lse", _P),
                ("hot_share", _P), ("cold_share", _P), ("cold_tile_max", _P),
                ("cold_tile_arg", _P), ("next", C.c_int), ("mu", C.c_int64 * 8)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = C.CDLL(build())
        L = _lib
        L.orc_e2m1_mag.argtypes = [C.c_double]
        L.orc_e2m1_code.argtypes = [C.c_double]
        L.orc_e2m1_value.argtypes = [C.c_int]
        L.orc_e2m1_value.restype = C.c_double
        L.orc_ue4m3_rn.argtypes = [C.c_double]
        L.orc_ue4m3_rn.restype = C.c_double
        L.orc_e8m0_exp.argtypes = [C.c_double]
        L.orc_scale_value.argtypes = [C.c_uint8, C.c_int]
        L.orc_scale_value.restype = C.c_double
        L.orc_key_stats.argtypes = [_P, C.c_int, C.c_int, C.c_int, _P, _P]
        L.orc_absmax.argtypes = [_P, C.c_size_t]
        L.orc_absmax.restype = C.c_float
        L.orc_head_scale.argtypes = [C.c_float, C.c_int, _P, _P]
        L.orc_q_scale.argtypes = [C.c_float, C.c_float, C.c_float, C.c_int, _P, _P]
        L.orc_quant_rows.argtypes = [_P, C.c_int, C.c_int, _P, C.c_float, C.c_int, _P, _P]
        L.orc_quant_rows_lsq.argtypes = [_P, C.c_int, C.c_int, _P, C.c_float, _P, _P]
        L.orc_quant_rows2.argtypes = [_P, C.c_int, C.c_int, C.c_float, C.c_int, _P, _P, _P, _P]
        L.orc_quant_vt.argtypes = [_P, C.c_int, C.c_int, C.c_int, C.c_float, C.c_int, C.c_int,
                                   _P, _P]
        L.orc_sl.argtypes = [_P]
        L.orc_sl.restype = C.c_float
        L.orc_visit_order.argtypes = [_P, C.c_int, _P]
        L.orc_run_groups.argtypes = [_P, C.c_int]
        L.orc_exact_rows.argtypes = [_P, _P, _P, _P, _P, C.c_int, _P, _P, C.c_int]
        L.orc_merge_row.argtypes = [C.c_int, C.c_double, C.c_double, _P, C.c_double, C.c_double,
                                    _P, C.c_double, _P, _P]
        L.orc_report_rows.argtypes = [_P, C.c_int]
        L.orc_report_job_size.restype = C.c_size_t
        assert L.orc_report_job_size() <= C.sizeof(_ReportJob)
        L.orc_job_size.restype = C.c_size_t
        L.orc_params_size.restype = C.c_size_t
        assert L.orc_params_size() == C.sizeof(_Params)
        assert L.orc_job_size() <= C.sizeof(_Job), (L.orc_job_size(), C.sizeof(_Job))
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


@dataclass
class Params:
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    causal: int = 1
    scale: float = 0.0      # <= 0: 1/sqrt(D)
    fmt: int = MX
    int_frame: int = 1
    tau: float = 4.0
    hoff: float = 32.0
    eps: float = 0.005
    tile: int = 64
    rg: int = 16
    q_terms: int = 1        # 2: Q plus its FP4 residual term
    k_lsq: int = 0          # 1: K block exponents by least squared error (MX)
    qmask: int = QUANT_ALL  # pass 1's FP4 roundings that apply (per-operand emulation)
    window: int = 0         # > 0: causal sliding window of this many keys
    stat_keys: int = 0      # > 0: K/V statistics over the keys before this one (chunked
                            # prefill: frozen at the last restat); 0: over all keys
    hot_weight: int = 0     # 1: the hot test weighs a tile's mass by its value-norm
                            # weight (see tile_weights); 0: mass only
    q_scale: str = "tied"   # "own": an ablation of the tied Q scale -- Q normalised by
                            # 6 / max|Q| of its head, the score factor sl * g_k * g_q

    def c(self) -> _Params:
        assert self.rg == 16, "the oracle keeps 16-row verdict groups"
        assert self.Hq % self.Hkv == 0
        assert self.q_terms in (1, 2)
        assert self.k_lsq in (0, 1) and not (self.k_lsq and self.fmt != MX)
        assert 0 <= self.qmask <= QUANT_ALL
        assert self.window >= 0 and (self.window == 0 or self.causal)
        assert self.stat_keys == 0 or self.first_tile * self.tile < self.stat_keys <= self.Nkv
        assert self.hot_weight in (0, 1)
        assert self.q_scale in ("tied", "own") and (self.q_scale == "tied" or self.fmt == MX)
        bs = 16 if self.fmt == NV else 32
        assert self.D % bs == 0
        return _Params(self.B, self.Hq, self.Hkv, self.Nq, self.Nkv, self.D, self.causal,
                       self.scale, self.fmt, self.int_frame, self.tau, self.hoff, self.eps,
                       self.tile, self.rg, self.q_terms, self.k_lsq, self.qmask, self.window,
                       self.hot_weight)

    @property
    def n_tiles(self) -> int:
        return (self.Nkv + self.tile - 1) // self.tile

    @property
    def n_groups(self) -> int:
        return (self.Nq + self.rg - 1) // self.rg

    @property
    def block(self) -> int:
        return 16 if self.fmt == NV else 32

    @property
    def first_tile(self) -> int:
        """The first key tile any query row sees: 0, or with a sliding window
        the tile of the first key of row 0 (key Nkv - Nq - window + 1)."""
        if self.window > 0 and self.causal:
            return max(0, self.Nkv - self.Nq - self.window + 1) // self.tile
        return 0


# --------------------------------------------------------------------------
# format helpers (thin wrappers, used by the pins)
# --------------------------------------------------------------------------

def e2m1_mag(a: float) -> int:
    return lib().orc_e2m1_mag(float(a))


def e2m1_code(x: float) -> int:
    return lib().orc_e2m1_code(float(x))


def e2m1_value(code: int) -> float:
    return lib().orc_e2m1_value(int(code))


def ue4m3_rn(a: float) -> float:
    return lib().orc_ue4m3_rn(float(a))


def e8m0_exp(a: float) -> int:
    return lib().orc_e8m0_exp(float(a))


def scale_value(b: int, fmt: int = MX) -> float:
    return lib().orc_scale_value(int(b), fmt)


def sl(p: Params) -> float:
    cp = p.c()
    return lib().orc_sl(C.byref(cp))


def visit_order(p: Params, g: int) -> list:
    cp = p.c()
    buf = np.zeros(p.n_tiles + 1, np.int32)
    n = lib().orc_visit_order(C.byref(cp), int(g), _ptr(buf))
    return buf[:n].tolist()


def quant_rows(X: np.ndarray, inv: float, fmt: int = MX, centre=None):
    """Quantise rows of X [n, D] along D.  Returns (codes [n, D/2], scales [n, D/Bs])."""
    X = np.ascontiguousarray(X, np.float32)
    n, D = X.shape
    bs = 16 if fmt == NV else 32
    codes = np.zeros((n, D // 2), np.uint8)
    scales = np.zeros((n, D // bs), np.uint8)
    c = None if centre is None else np.ascontiguousarray(centre, np.float32)
    lib().orc_quant_rows(_ptr(X), n, D, _ptr(c), float(inv), fmt, _ptr(codes), _ptr(scales))
    return codes, scales


# --------------------------------------------------------------------------
# a1 + a2: statistics, per-head scales, quantisation
# --------------------------------------------------------------------------

def tile_weights(p: Params, Vh: np.ndarray):
    """Value-norm weights of the hot test for one (b, kv-head), V [Nkv, D].

    "APA: sloppy attention, exact where it counts", section "Honest limits",
    its point on mass versus output: the hot test bounds a cold tile's share
    of the softmax mass, while what the tile adds to the output also scales
    with the size of its values; the page proposes weighing the test by value
    norm.
    Reading taken here: nu_k = ||v_k||_2 of every key (FP64); nu_bar = their
    mean over the keys the K/V statistics cover; a tile's weight is
    w_t = max(1, fl32(max_{k in t} nu_k / nu_bar)) (1 when nu_bar is 0).  The
    weighted test marks a tile hot when fl32(l_t * w_t) > fl32(eps * lambda).
    A cold tile t then adds at most l_t * max nu_k <= eps * lambda * nu_bar to
    the output's norm, and, since w_t >= 1, its share of the mass stays under
    eps as before.  Returns (w [NT] float32, nu_bar); tiles before first_tile
    (never visited) get weight 1."""
    Nkv, NT, T = p.Nkv, p.n_tiles, p.tile
    k0 = p.first_tile * T
    ks_hi = p.stat_keys if p.stat_keys > 0 else Nkv
    v = np.asarray(Vh, np.float64)
    nu = np.sqrt((v * v).sum(axis=1))          # squares exact, FP64 sum
    nbar = float(nu[k0:ks_hi].sum() / (ks_hi - k0)) if ks_hi > k0 else 0.0
    w = np.ones(NT, np.float32)
    if nbar > 0.0:
        for t in range(p.first_tile, NT):
            r = np.float32(nu[t * T:min(Nkv, t * T + T)].max() / nbar)
            w[t] = max(np.float32(1.0), r)
    return w, nbar


def quantize(p: Params, Q: np.ndarray, K: np.ndarray, V: np.ndarray) -> dict:
    """Stats and block-scaled FP4 quantisation of Q, K (centred), V (along keys).

    Q [B,Hq,Nq,D], K/V [B,Hkv,Nkv,D] float32 arrays holding the fp16/bf16
    input values.  Returns codes, scale bytes, per-head scales and the hot
    test's value-norm weights (vw [B,Hkv,NT], nu_bar [B,Hkv]).  With a
    sliding window the K/V statistics (key mean, per-head scales) and codes
    cover the key tiles from first_tile on, the ones some row sees.  With
    stat_keys the statistics cover only the keys before it (values of later
    keys beyond the frozen range clamp at the format's largest value).  In MX
    mode V enters at its own scale (g_v = inv_v = 1; amax_v is still
    recorded): its E8M0 block exponents carry the range that NVFP4's narrow
    UE4M3 block scales leave to the per-head scale (the section "Pass 1: FP4
    everywhere, with a hot test" of "APA: sloppy attention, exact where it
    counts" gives one FP32 scale per head for that format).
    """
    L = lib()
    cp = p.c()
    Q = np.ascontiguousarray(Q, np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    B, Hq, Hkv, Nq, Nkv, D = p.B, p.Hq, p.Hkv, p.Nq, p.Nkv, p.D
    G = Hq // Hkv
    bs = p.block
    NkvP = p.n_tiles * p.tile
    s_l = L.orc_sl(C.byref(cp))
    out = dict(
        kbar=np.zeros((B, Hkv, D), np.float32), amax_k=np.zeros((B, Hkv), np.float32),
        g_k=np.zeros((B, Hkv), np.float32), inv_k=np.zeros((B, Hkv), np.float32),
        amax_v=np.zeros((B, Hkv), np.float32), g_v=np.zeros((B, Hkv), np.float32),
        inv_v=np.zeros((B, Hkv), np.float32), amax_q=np.zeros((B, Hq), np.float32),
        inv_q=np.zeros((B, Hq), np.float32), jq=np.zeros((B, Hq), np.int32),
        qc=np.zeros((B, Hq, Nq, D // 2), np.uint8), qs=np.zeros((B, Hq, Nq, D // bs), np.uint8),
        kc=np.zeros((B, Hkv, Nkv, D // 2), np.uint8),
        ks=np.zeros((B, Hkv, Nkv, D // bs), np.uint8),
        vc=np.zeros((B, Hkv, D, NkvP // 2), np.uint8),
        vs=np.zeros((B, Hkv, D, NkvP // bs), np.uint8), sl=np.float32(s_l),
        vw=np.ones((B, Hkv, p.n_tiles), np.float32), nu_bar=np.zeros((B, Hkv)))
    f = np.zeros(2, np.float32)
    ji = np.zeros(1, np.int32)
    for b in range(B):
        for hk in range(Hkv):
            # statistics and codes over the key tiles some query row sees:
            # all, or with a sliding window from first_tile on (the others
            # are never read; their codes stay zero here); with stat_keys the
            # statistics stop before that key (chunked prefill keeps them
            # from the last restat) while the codes cover every key
            k0 = p.first_tile * p.tile
            nk = Nkv - k0
            ks_hi = p.stat_keys if p.stat_keys > 0 else Nkv
            Kh = np.ascontiguousarray(K[b, hk, k0:])
            Vh = np.ascontiguousarray(V[b, hk, k0:])
            Ks = np.ascontiguousarray(K[b, hk, k0:ks_hi])
            kb = np.zeros(D, np.float32)
            am = np.zeros(1, np.float32)
            L.orc_key_stats(_ptr(Ks), ks_hi - k0, D, p.tile, _ptr(kb), _ptr(am))
            out["kbar"][b, hk] = kb
            out["amax_k"][b, hk] = am[0]
            L.orc_head_scale(C.c_float(am[0]), p.fmt, _ptr(f[0:1]), _ptr(f[1:2]))
            out["g_k"][b, hk], out["inv_k"][b, hk] = f[0], f[1]
            Vs = np.ascontiguousarray(V[b, hk, k0:ks_hi])
            av = L.orc_absmax(_ptr(Vs), Vs.size)
            out["amax_v"][b, hk] = av
            if p.fmt == MX:
                # V at its own scale: per-head scale 1 (see orc_quant_vt)
                out["g_v"][b, hk], out["inv_v"][b, hk] = 1.0, 1.0
            else:
                L.orc_head_scale(C.c_float(av), p.fmt, _ptr(f[0:1]), _ptr(f[1:2]))
                out["g_v"][b, hk], out["inv_v"][b, hk] = f[0], f[1]
            kc = np.zeros((nk, D // 2), np.uint8)
            ks = np.zeros((nk, D // bs), np.uint8)
            if p.k_lsq:
                L.orc_quant_rows_lsq(_ptr(Kh), nk, D, _ptr(kb), C.c_float(out["inv_k"][b, hk]),
                                     _ptr(kc), _ptr(ks))
            else:
                L.orc_quant_rows(_ptr(Kh), nk, D, _ptr(kb), C.c_float(out["inv_k"][b, hk]),
                                 p.fmt, _ptr(kc), _ptr(ks))
            out["kc"][b, hk, k0:], out["ks"][b, hk, k0:] = kc, ks
            vc = np.zeros((D, (NkvP - k0) // 2), np.uint8)
            vs = np.zeros((D, (NkvP - k0) // bs), np.uint8)
            L.orc_quant_vt(_ptr(Vh), nk, NkvP - k0, D, C.c_float(out["inv_v"][b, hk]), p.fmt,
                           1 if p.fmt == MX else 0,
                           _ptr(vc), _ptr(vs))
            out["vc"][b, hk, :, k0 // 2:], out["vs"][b, hk, :, k0 // bs:] = vc, vs
            out["vw"][b, hk], out["nu_bar"][b, hk] = tile_weights(p, V[b, hk])
        for h in range(Hq):
            Qh = np.ascontiguousarray(Q[b, h])
            aq = L.orc_absmax(_ptr(Qh), Qh.size)
            out["amax_q"][b, h] = aq
            L.orc_q_scale(C.c_float(aq), C.c_float(s_l), C.c_float(out["g_k"][b, h // G]), p.fmt,
                          _ptr(f[0:1]), _ptr(ji))
            out["inv_q"][b, h], out["jq"][b, h] = f[0], ji[0]
            if p.q_scale == "own":
                # Q at its own head scale, amax/6 like K's; the score factor
                # then carries both head scales and sl (no longer a power of two)
                L.orc_head_scale(C.c_float(aq), p.fmt, _ptr(f[0:1]), _ptr(f[1:2]))
                out["inv_q"][b, h] = f[1]
                out.setdefault("alpha_q", np.zeros((B, Hq), np.float64))[b, h] = (
                    float(np.float32(s_l)) * float(out["g_k"][b, h // G]) * float(f[0]))
            qc = np.zeros((Nq, D // 2), np.uint8)
            qs = np.zeros((Nq, D // bs), np.uint8)
            if p.q_terms == 2:
                qc2 = np.zeros((Nq, D // 2), np.uint8)
                qs2 = np.zeros((Nq, D // bs), np.uint8)
                L.orc_quant_rows2(_ptr(Qh), Nq, D, C.c_float(out["inv_q"][b, h]), p.fmt, _ptr(qc), _ptr(qs),
                                  _ptr(qc2), _ptr(qs2))
                out.setdefault("qc2", np.zeros((B, Hq, Nq, D // 2), np.uint8))[b, h] = qc2
                out.setdefault("qs2", np.zeros((B, Hq, Nq, D // bs), np.uint8))[b, h] = qs2
            else:
                L.orc_quant_rows(_ptr(Qh), Nq, D, None, C.c_float(out["inv_q"][b, h]), p.fmt,
                                 _ptr(qc), _ptr(qs))
            out["qc"][b, h], out["qs"][b, h] = qc, qs
    return out


def all_groups(p: Params) -> np.ndarray:
    g = [(b, h, i) for b in range(p.B) for h in range(p.Hq) for i in range(p.n_groups)]
    return np.array(g, np.int32).reshape(-1, 3)


# --------------------------------------------------------------------------
# a3..a10: pass 1, pass 2, merge for a list of row groups
# --------------------------------------------------------------------------

def run(p: Params, Q, K, V, prep: dict | None = None, groups=None, nthreads: int | None = None,
        pass2: bool = True) -> dict:
    """APA on the CPU.  groups: array [n, 3] of (b, q-head, row group); all if None.

    Returns the pass-1 state (m1 frame, l1, o1 = o * g_v, lambda), the hot
    cells (one byte per (b, h, group, tile)) with their margins, and, if
    pass2, the exact pass-2 state, the frame constants c_r and the merged
    output O (FP64) with LSE (natural log).  Only rows of listed groups are
    written; others stay NaN.
    """
    L = lib()
    cp = p.c()
    Q = np.ascontiguousarray(Q, np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    if prep is None:
        prep = quantize(p, Q, K, V)
    if groups is None:
        groups = all_groups(p)
    groups = np.ascontiguousarray(groups, np.int32).reshape(-1, 3)
    B, Hq, Nq, D = p.B, p.Hq, p.Nq, p.D
    NG, NT = p.n_groups, p.n_tiles
    nan = np.nan
    res = dict(
        hot=np.zeros((B, Hq, NG, NT), np.uint8), margin=np.full((B, Hq, NG, NT), nan),
        m1=np.full((B, Hq, Nq), nan), l1=np.full((B, Hq, Nq), nan, np.float32),
        lam=np.full((B, Hq, Nq), nan, np.float32), o1=np.full((B, Hq, Nq, D), nan, np.float32),
        shift=np.full((B, Hq, Nq), nan), m2=np.full((B, Hq, Nq), nan),
        l2=np.full((B, Hq, Nq), nan), o2=np.full((B, Hq, Nq, D), nan),
        cr=np.full((B, Hq, Nq), nan), O=np.full((B, Hq, Nq, D), nan),
        lse=np.full((B, Hq, Nq), nan))
    keep = [Q, K, V, prep, groups]
    job = _Job()
    job.p = C.cast(C.pointer(cp), C.c_void_p)
    job.Q, job.K, job.V = _ptr(Q), _ptr(K), _ptr(V)
    for k in ("qc", "qs", "kc", "ks", "vc", "vs", "kbar", "g_v"):
        setattr(job, k, _ptr(prep[k]))
    job.jq = _ptr(prep["jq"])
    job.inv_q, job.inv_k, job.inv_v = (_ptr(prep[k]) for k in ("inv_q", "inv_k", "inv_v"))
    job.vw = _ptr(prep["vw"]) if p.hot_weight else None
    job.alpha_q = _ptr(prep["alpha_q"]) if p.q_scale == "own" else None
    job.qc2 = _ptr(prep.get("qc2")) if p.q_terms == 2 else None
    job.qs2 = _ptr(prep.get("qs2")) if p.q_terms == 2 else None
    job.groups, job.ngroups = _ptr(groups), len(groups)
    for k in ("hot", "margin", "m1", "l1", "lam", "o1", "shift", "m2", "l2", "o2", "cr", "O",
              "lse"):
        setattr(job, k, _ptr(res[k]))
    job.do_pass2 = 1 if pass2 else 0
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    L.orc_run_groups(C.byref(job), int(nthreads))
    del keep
    res["prep"] = prep
    res["groups"] = groups
    res["threads"] = int(nthreads)
    return res


def exact(p: Params, Q, K, V, rows=None, nthreads: int | None = None):
    """Reference attention in FP64 for rows [n, 3] of (b, q-head, r); all if None.

    Returns (O [n, D] float64, lse [n] float64)."""
    L = lib()
    cp = p.c()
    Q = np.ascontiguousarray(Q, np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    if rows is None:
        rows = np.array([(b, h, r) for b in range(p.B) for h in range(p.Hq) for r in range(p.Nq)],
                        np.int32).reshape(-1, 3)
    rows = np.ascontiguousarray(rows, np.int32).reshape(-1, 3)
    O = np.zeros((len(rows), p.D))
    lse = np.zeros(len(rows))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    L.orc_exact_rows(C.byref(cp), _ptr(Q), _ptr(K), _ptr(V), _ptr(rows), len(rows), _ptr(O),
                     _ptr(lse), int(nthreads))
    return O, lse


def merge_row(D, m1, l1, o1, m2, l2, o2, c):
    """Merge two states of one row (FP64).  Returns (O [D], lse)."""
    o1 = np.ascontiguousarray(o1, np.float64)
    o2 = np.ascontiguousarray(o2, np.float64)
    O = np.zeros(D)
    lse = np.zeros(1)
    lib().orc_merge_row(int(D), float(m1), float(l1), _ptr(o1), float(m2), float(l2), _ptr(o2),
                        float(c), _ptr(O), _ptr(lse))
    return O, float(lse[0])


# --------------------------------------------------------------------------
# reports against exact FP64 attention
# --------------------------------------------------------------------------

def reports(p: Params, Q, K, V, hot, rows=None, nthreads: int | None = None) -> dict:
    """Where the exact FP64 softmax mass and output of each listed row sit
    relative to a hot mask hot [B, Hq, NG, NT] (the method's, or a GPU's):
    O_ref (exact attention), its parts O_hot and O_cold over the keys of hot
    and of other tiles, lse, the mass on hot and on other tiles, and the
    largest mass of one tile not marked hot (its index in cold_tile_arg, -1 if
    none).  rows [n, 3] of (b, q-head, r); all rows if None."""
    L = lib()
    cp = p.c()
    Q = np.ascontiguousarray(Q, np.float32)
    K = np.ascontiguousarray(K, np.float32)
    V = np.ascontiguousarray(V, np.float32)
    hot = np.ascontiguousarray(hot, np.uint8)
    assert hot.shape == (p.B, p.Hq, p.n_groups, p.n_tiles), hot.shape
    if rows is None:
        rows = np.array([(b, h, r) for b in range(p.B) for h in range(p.Hq) for r in range(p.Nq)],
                        np.int32).reshape(-1, 3)
    rows = np.ascontiguousarray(rows, np.int32).reshape(-1, 3)
    n = len(rows)
    out = dict(O_ref=np.zeros((n, p.D)), O_hot=np.zeros((n, p.D)), O_cold=np.zeros((n, p.D)),
               lse=np.zeros(n), hot_share=np.zeros(n), cold_share=np.zeros(n),
               cold_tile_max=np.zeros(n), cold_tile_arg=np.zeros(n, np.int32))
    job = _ReportJob()
    job.p = C.cast(C.pointer(cp), C.c_void_p)
    job.Q, job.K, job.V, job.hot, job.rows, job.nrows = (_ptr(Q), _ptr(K), _ptr(V), _ptr(hot),
                                                         _ptr(rows), n)
    for k in out:
        setattr(job, k, _ptr(out[k]))
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    L.orc_report_rows(C.byref(job), int(nthreads))
    out["rows"] = rows
    return out


def compare_rows(O_test, O_ref) -> dict:
    """Per-row agreement of an output with the reference: cosine (a row that
    is zero on exactly one side scores -1, zero on both 1), mean squared
    error and largest absolute difference, over every element."""
    a = np.asarray(O_test, np.float64).reshape(-1, np.shape(O_ref)[-1])
    b = np.asarray(O_ref, np.float64).reshape(a.shape)
    na, nb = np.linalg.norm(a, axis=1), np.linalg.norm(b, axis=1)
    cos = np.where((na > 0) != (nb > 0), -1.0, 1.0)
    ok = (na > 0) & (nb > 0)
    cos[ok] = (a[ok] * b[ok]).sum(1) / (na[ok] * nb[ok])
    d = a - b
    return dict(cos=cos, mse=float((d * d).mean()), max_abs=float(np.abs(d).max()),
                row_mse=(d * d).mean(axis=1))
