"""An independent, frame-free numpy brute force of APA's pass 1 for tiny inputs.

It re-derives everything from the raw inputs with different arithmetic than
the oracle: quantisation by nearest-value search (not threshold counting),
scores as an FP64 matrix product of dequantised operands, and pass 1 without
any logit frame.  In MX mode with an integer frame the per-group exponent
E = ceil(c_g - m - log2 6) shifts by exactly the frame, so every quantity of
pass 1 (P, the tile row sums, lambda, the cold l and o) is the frame-free
value times an exact power of two -- the tau/H frame logic only relabels it.
Agreement with the oracle, bit for bit, therefore pins the lazy maximum, the
decoupled cold frame and every rescale, as well as the visit order and the
hot test ("APA: sloppy attention, exact where it counts", "Pass 1" steps 1-5,
"Tile order", "The bug: a sink that drowned the tail").

Valid while no block exponent reaches the E8M0 floor (2^-127) and nothing
underflows FP32; the tiny workloads used by the tests stay far from both.

Options mirror the oracle's: `quant` switches each operand's FP4 rounding
(Q, K, V, P; an operand switched off enters at its exact value in the same
normalised units, "Second hunt: which operand is to blame"), and `window`
restricts every row to its `window` most recent keys ("What else is in the
box": sliding window).  With `hot_weight` the hot test weighs each tile's
mass by max(1, max key value norm in the tile / mean key value norm of the
head) ("Honest limits", mass versus output), the norms taken here with
numpy's own norm routine.  The per-cell margin max_r (l_r w - eps lambda_r) /
lambda_r is recomputed from this brute force's own l and lambda.
"""
from __future__ import annotations

import numpy as np

MAGS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
LOG2E32 = np.float32(np.log2(np.e))


def f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


def nearest_mag_code(a: np.ndarray) -> np.ndarray:
    """3-bit E2M1 magnitude code of |a| by nearest-value search; ties go to the
    even code; values above 6 saturate."""
    a = np.minimum(np.abs(np.asarray(a, np.float64)), 6.0)
    dist = np.abs(a[..., None] - MAGS)
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    # among tied candidates prefer the even code index
    idx = np.arange(8)
    score = np.where(cand, (idx % 2) * 16 + idx, 1000)
    return score.argmin(axis=-1)


def block_exp(a: np.ndarray) -> np.ndarray:
    """Smallest integer e with a <= 6 * 2^e (a > 0), clamped to [-127, 127]."""
    a = np.asarray(a, np.float64)
    e = np.full(a.shape, -127, np.int64)
    pos = a > 0
    with np.errstate(divide="ignore"):
        guess = np.floor(np.log2(np.where(pos, a, 1.0) / 6.0)).astype(np.int64) - 1
    for _ in range(4):  # walk up to the smallest passing exponent
        ok = 6.0 * np.ldexp(1.0, guess) >= a
        guess = np.where(ok, guess, guess + 1)
    e = np.where(pos, guess, -127)
    return np.clip(e, -127, 127)


def quantise_blocks(x: np.ndarray, bs: int = 32):
    """x [..., n] normalised values -> dequantised values (same shape)."""
    sh = x.shape
    xb = np.asarray(x, np.float64).reshape(sh[:-1] + (sh[-1] // bs, bs))
    e = block_exp(np.abs(xb).max(axis=-1))
    sc = np.ldexp(1.0, e)[..., None]
    code = nearest_mag_code(xb / sc)
    val = np.sign(xb) * MAGS[code] * sc
    return val.reshape(sh)


QUANT_ALL = "QKVP"


def _ue4m3_values() -> np.ndarray:
    """Every finite unsigned E4M3 value, ascending (encoding order): exponent
    bias 7, 3 mantissa bits, subnormals below 2^-6, the top encoding NaN."""
    vals = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            vals.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


UE4M3 = _ue4m3_values()


def ue4m3_nearest(a) -> np.ndarray:
    """Nearest UE4M3 value (ties to the even encoding), saturating at 448."""
    a = np.minimum(np.asarray(a, np.float64), UE4M3[-1])
    dist = np.abs(a[..., None] - UE4M3)
    cand = dist == dist.min(axis=-1, keepdims=True)
    idx = np.arange(len(UE4M3))
    return UE4M3[np.where(cand, (idx % 2) * 1000 + idx, 10 ** 6).argmin(axis=-1)]


def rn_4bits(x) -> np.ndarray:
    """x > 0 rounded to 4 significant bits, ties to even, with no exponent
    limit: UE4M3 rounding wherever its normal range holds, and scale
    invariant (rn(x 2^k) = rn(x) 2^k)."""
    m, e = np.frexp(np.asarray(x, np.float64))
    return np.ldexp(np.round(m * 16.0) / 16.0, e)


def quantise_blocks_nv(x: np.ndarray, bs: int = 16):
    """NVFP4 blocks of 16: scale = nearest UE4M3 of the block max / 6, codes
    by nearest-value search of x / scale (a zero scale gives zero values)."""
    sh = x.shape
    xb = np.asarray(x, np.float64).reshape(sh[:-1] + (sh[-1] // bs, bs))
    sc = ue4m3_nearest(np.abs(xb).max(axis=-1) / 6.0)[..., None]
    with np.errstate(invalid="ignore", divide="ignore"):
        code = nearest_mag_code(np.where(sc > 0, xb / np.where(sc > 0, sc, 1.0), 0.0))
    return (np.sign(xb) * MAGS[code] * sc).reshape(sh)


def prepare(Q, K, V, scale: float, q_terms: int = 1, quant: str = QUANT_ALL, k0: int = 0,
            fmt: str = "MX"):
    """Per-head scales and dequantised operands (without the per-head factors
    that fold into alpha and g_v).  Q [Hq,Nq,D] etc. for one batch entry.
    q_terms=2 adds the quantised residual of Q (section "Second hunt": a second
    FP4 term for what the first leaves over, sharing its scale) to the
    dequantised Q.  An operand missing from `quant` is kept at its exact value
    in normalised units (FP64, no clamp).  The K/V statistics (key mean,
    per-head scales) are taken over keys k0.. (a sliding window's first visible
    tile; 0 otherwise).  fmt "NV": blocks of 16 with UE4M3 scales and per-head
    scales mapping the head maximum to 6 x 448 (V included)."""
    Hq, Nq, D = Q.shape
    nv = fmt == "NV"
    X = 2688.0 if nv else 6.0
    qblocks = quantise_blocks_nv if nv else quantise_blocks
    Hkv = K.shape[0]
    G = Hq // Hkv
    sl = np.float32(np.float32(scale) * LOG2E32)
    out = []
    for hk in range(Hkv):
        Kh = K[hk].astype(np.float32)
        kbar = f32(Kh[k0:].astype(np.float64).sum(axis=0) / (Kh.shape[0] - k0))
        kc = (Kh - kbar).astype(np.float32)              # fl32 subtraction
        amax_k = np.abs(kc[k0:]).max() if kc[k0:].size else np.float32(0)
        g_k = f32(amax_k / X) if amax_k > 0 else np.float32(1)
        inv_k = f32(X / amax_k) if amax_k > 0 else np.float32(1)
        kn = np.clip((kc * inv_k).astype(np.float32), -X, X)
        kd = (qblocks(kn) if "K" in quant else
              (Kh.astype(np.float64) - kbar.astype(np.float64)) * np.float64(inv_k))
        Vh = V[hk].astype(np.float32)
        if nv:
            amax_v = np.abs(Vh[k0:]).max()
            g_v = f32(amax_v / X) if amax_v > 0 else np.float32(1)
            inv_v = f32(X / amax_v) if amax_v > 0 else np.float32(1)
            vn = np.clip((Vh * inv_v).astype(np.float32), -X, X)
        else:
            # MX: V at its own scale (per-head scale 1, no clamp); the block
            # exponents take the range
            g_v = np.float32(1)
            inv_v = np.float32(1)
            vn = Vh
        Nkv = Vh.shape[0]
        NkvP = -(-Nkv // 64) * 64
        vpad = np.zeros((NkvP, D), np.float32)
        vpad[:Nkv] = vn
        vd = qblocks(vpad.T).T[:Nkv]                      # blocks of keys per channel
        if "V" not in quant:
            vd = Vh.astype(np.float64) * np.float64(inv_v)
        # value-norm weights of the hot test, per 64-key tile
        nu = np.linalg.norm(Vh.astype(np.float64), axis=1)
        nbar = nu[k0:].mean() if Nkv > k0 else 0.0
        vw = np.ones(NkvP // 64, np.float32)
        if nbar > 0:
            for t in range(k0 // 64, NkvP // 64):
                vw[t] = max(1.0, f32(nu[64 * t:64 * t + 64].max() / nbar))
        w = np.float32(sl * g_k)
        heads = []
        for i in range(G):
            Qh = Q[hk * G + i].astype(np.float32)
            amax_q = np.abs(Qh).max()
            j = 0
            if amax_q > 0:
                prod = float(amax_q) * float(w)
                j = int(np.ceil(np.log2(prod / X))) - 1
                while X * 2.0 ** j < prod:
                    j += 1
            inv_q = np.float32(np.ldexp(np.float64(w), -j))
            qn = np.clip((Qh * inv_q).astype(np.float32), -X, X)
            qd = qblocks(qn)
            if "Q" not in quant:
                qd = Qh.astype(np.float64) * np.float64(inv_q)
            elif q_terms == 2:
                # the residual in FP32, quantised as blocks of its own; the sum
                # of the two dequantised terms is exact in FP64
                qd = qd + quantise_blocks((qn.astype(np.float64) - qd).astype(np.float32))
            heads.append(dict(qd=qd, alpha=2.0 ** j, Qh=Qh))
        out.append(dict(kd=kd, vd=vd, g_v=g_v, heads=heads, kbar=kbar, sl=sl, vw=vw))
    return out


def visit_order(last_row: int, off: int, Nkv: int, causal: bool, tile: int = 64,
                first_row: int = 0, window: int = 0):
    nt = -(-Nkv // tile)
    d = min(Nkv - 1, last_row + off) // tile if causal else nt - 1
    lo = max(0, first_row + off - window + 1) // tile if (causal and window > 0) else 0
    if lo > 0:
        return list(range(d, lo - 1, -1))
    return [0] + list(range(d, 0, -1))


def pass1_group(scores: np.ndarray, vd: np.ndarray, eps: float, rows: np.ndarray, off: int,
                Nkv: int, causal: bool, quant_p: bool = True, window: int = 0, tw=None,
                fmt: str = "MX"):
    """Frame-free pass 1 of one row group.

    scores: [R, Nkv] FP4 scores in log2 units (fl32), vd: [Nkv, D] dequantised
    V', tw: per-tile weights of the hot test or None.  Returns (hot [NT] bool, l [R], o [R, D], lam [R], margin [NT]) in
    frame-free units; margin is NaN for tiles not visited.
    """
    R = scores.shape[0]
    D = vd.shape[1]
    nt = -(-Nkv // 64)
    hot = np.zeros(nt, bool)
    margin = np.full(nt, np.nan)
    lam = np.zeros(R, np.float32)
    lsum = np.zeros(R, np.float32)
    o = np.zeros((R, D), np.float32)
    keys = np.arange(Nkv)
    vis = (keys[None, :] <= rows[:, None] + off) if causal else np.ones((R, Nkv), bool)
    if causal and window > 0:
        vis &= keys[None, :] > rows[:, None] + off - window
    s = np.where(vis, scores.astype(np.float64), -np.inf)
    eps32 = np.float32(eps)
    for t in visit_order(int(rows[-1]), off, Nkv, causal, first_row=int(rows[0]), window=window):
        k0, k1 = 64 * t, min(Nkv, 64 * t + 64)
        st = np.full((R, 64), -np.inf)
        st[:, :k1 - k0] = s[:, k0:k1]
        if not np.isfinite(st).any():
            continue  # no row of the group sees a key of this tile: not visited
        ph = np.zeros((R, 64))
        if fmt == "NV":
            # P in groups of 16 keys, scale = the group maximum / 6 rounded
            # to 4 significant bits (UE4M3 inside its normal range, which
            # inputs flat enough for the frame never to leave keep)
            for q0 in range(0, 64, 16):
                g = st[:, q0:q0 + 16]
                cg = g.max(axis=1)
                live = np.isfinite(cg)
                sg = rn_4bits(np.exp2(np.where(live, cg, 0.0)) / 6.0)[:, None]
                with np.errstate(invalid="ignore", over="ignore"):
                    code = nearest_mag_code(np.exp2(g) / sg)
                ph[:, q0:q0 + 16] = np.where(np.isfinite(g), MAGS[code] * sg, 0.0)
        for q0 in ((0, 32) if fmt == "MX" else ()):
            if not quant_p:
                g = st[:, q0:q0 + 32]
                with np.errstate(invalid="ignore", over="ignore"):
                    ph[:, q0:q0 + 32] = np.where(np.isfinite(g), np.exp2(g), 0.0)
                continue
            g = st[:, q0:q0 + 32]
            cg = g.max(axis=1)
            E = np.where(np.isfinite(cg), np.ceil(cg - np.log2(6.0)), 0).astype(np.int64)
            # exact adjustment of the ceiling
            E = np.where(np.exp2(cg - E) > 6.0, E + 1, E)
            E = np.where(np.exp2(cg - (E - 1)) <= 6.0, E - 1, E)
            with np.errstate(invalid="ignore", over="ignore"):
                code = nearest_mag_code(np.exp2(g - E[:, None]))
            ph[:, q0:q0 + 32] = np.where(np.isfinite(g), MAGS[code] * np.ldexp(1.0, E)[:, None], 0)
        ell = f32(ph.sum(axis=1))
        lam = (lam + ell).astype(np.float32)
        thr = (eps32 * lam).astype(np.float32)
        lw = ell if tw is None else (ell * np.float32(tw[t])).astype(np.float32)
        h = (eps == 0.0) or bool(np.any(lw > thr))
        hot[t] = h
        pos = lam > 0
        lam64 = lam.astype(np.float64)
        mg = (lw.astype(np.float64) - np.float64(eps32) * lam64) / np.where(pos, lam64, 1.0)
        margin[t] = mg[pos].max() if pos.any() else -np.inf
        if not h:
            vt = np.zeros((64, D))
            vt[:k1 - k0] = vd[k0:k1]
            pv = f32(ph @ vt)
            o = (o + pv).astype(np.float32)
            lsum = (lsum + ell).astype(np.float32)
    return hot, lsum, o, lam, margin


def brute_apa(Q, K, V, eps: float, scale: float, causal: bool = True, q_terms: int = 1,
              quant: str = QUANT_ALL, window: int = 0, hot_weight: bool = False,
              fmt: str = "MX"):
    """Frame-free pass 1 for every row group of a batch-1 problem.

    Returns dict with hot [Hq, NG, NT], l [Hq, Nq], o [Hq, Nq, D] (o already
    times g_v), lam [Hq, Nq], all frame-free, and margin [Hq, NG, NT]."""
    Q, K, V = Q[0], K[0], V[0]
    Hq, Nq, D = Q.shape
    Nkv = K.shape[1]
    G = Hq // K.shape[0]
    off = Nkv - Nq
    nt = -(-Nkv // 64)
    ng = -(-Nq // 16)
    k0 = max(0, off - window + 1) // 64 * 64 if (causal and window > 0) else 0
    ops = prepare(Q, K, V, scale, q_terms, quant, k0, fmt)
    hot = np.zeros((Hq, ng, nt), bool)
    margin = np.full((Hq, ng, nt), np.nan)
    lo = np.zeros((Hq, Nq), np.float32)
    oo = np.zeros((Hq, Nq, D), np.float32)
    la = np.zeros((Hq, Nq), np.float32)
    for h in range(Hq):
        kv = ops[h // G]
        hd = kv["heads"][h % G]
        dot = f32(hd["qd"].astype(np.float64) @ kv["kd"].astype(np.float64).T)
        scores = f32(hd["alpha"] * dot.astype(np.float64))
        for g in range(ng):
            rows = np.arange(16 * g, min(Nq, 16 * g + 16))
            hh, l, o, lam, mg = pass1_group(scores[rows], kv["vd"], eps, rows, off, Nkv, causal,
                                            quant_p="P" in quant, window=window,
                                            tw=kv["vw"] if hot_weight else None, fmt=fmt)
            hot[h, g] = hh
            margin[h, g] = mg
            lo[h, rows] = l
            oo[h, rows] = (o * kv["g_v"]).astype(np.float32)
            la[h, rows] = lam
    return dict(hot=hot, l=lo, o=oo, lam=la, margin=margin, ops=ops)
