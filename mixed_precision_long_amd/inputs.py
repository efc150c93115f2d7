"""Seeded synthetic inputs for causal GQA attention prefill.

This module only synthesises tensors; it holds none of the attention method's
arithmetic, and both the HIP path's tests/benchmark and the CPU oracle draw
their inputs from it.

The workloads stand in for Llama-3.2-3B query/key/value activations, which the
method's description ("APA: sloppy attention, exact where it counts",
rfriedmann.de, introduction and "Why this can work at all") measures on but
which are not available here.  They reproduce the structure that section
describes: an attention sink in the first keys, dominant tiles on the causal
diagonal, and a thin long middle.

* path mode: a smooth unit-vector path c(t) per (batch, kv-head), each channel
  a sum of 8 random sinusoids with log-uniform periods in [64, 131072]
  positions; K[k] = N(0, I)/sqrt(D) + a c(k), Q[h, r] = N(0, I)/sqrt(D)
  + a c(r + Nkv - Nq) (queries sit at the KV tail), V ~ N(0, 1); softmax
  scale 1.
* gauss mode: Q, K, V ~ N(0, 1); softmax scale 1/sqrt(D).
* sink: keys 0..3 get + delta * u / (scale |u|^2), u the mean rounded query of
  the kv-head's group, so the mean logit lift over the group's rows is delta
  nats (the "sink logit lift" parameterisation of the P-Cast abstract on
  thelatestinai.com).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

N_SINES = 8
PERIOD_MIN, PERIOD_MAX = 64.0, 131072.0
SINK_KEYS = 4


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest even); returns float32."""
    x = np.ascontiguousarray(x, np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return np.asarray(x, np.float64).astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        return round_bf16(np.asarray(x, np.float64).astype(np.float32))
    raise ValueError(dtype)


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nkv: int
    D: int
    dtype: str = "fp16"
    mode: str = "path"          # "path" or "gauss"
    a: float = 2.0
    delta: float = 6.0
    eps: float = 0.005
    seed: int = 1
    causal: int = 1
    eps_sweep: tuple = field(default_factory=tuple)
    delta_sweep: tuple = field(default_factory=tuple)

    @property
    def scale(self) -> float:
        return 1.0 if self.mode == "path" else float(1.0 / np.sqrt(self.D))

    def shape(self) -> dict:
        return dict(B=self.B, Hq=self.Hq, Hkv=self.Hkv, Nq=self.Nq, Nkv=self.Nkv, D=self.D)


# The five workloads: tiny check, the 3B-shaped short case, the headline long
# prefill (2048 query rows at 122880 keys), full causal prefill at 32768 with a
# sink-strength sweep, and large head dim in bf16.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 1, 256, 1024, 64, seed=1),
    "short3b": Workload("short3b", 1, 24, 8, 2048, 8192, 128, seed=2),
    "long3b": Workload("long3b", 1, 24, 8, 2048, 122880, 128, seed=3,
                       eps_sweep=(0.002, 0.005, 0.02)),
    "full32k": Workload("full32k", 1, 32, 8, 32768, 32768, 128, seed=4,
                        delta_sweep=(0.0, 4.0, 8.0, 12.0)),
    "bigd": Workload("bigd", 1, 32, 8, 1024, 4096, 512, dtype="bf16", mode="gauss", seed=5),
}


def _path(rng, n_pos: int, pos0: int, D: int, amp, per, ph) -> np.ndarray:
    """Unit path vectors c(t) for t = pos0 .. pos0 + n_pos - 1, shape [n_pos, D].
    (rng is unused; the path is a deterministic function of its parameters.)"""
    out = np.empty((n_pos, D), np.float64)
    step = 4096
    w = 2.0 * np.pi / per  # [8, D]
    for s in range(0, n_pos, step):
        t = np.arange(pos0 + s, pos0 + min(n_pos, s + step), dtype=np.float64)
        v = np.zeros((len(t), D))
        for i in range(N_SINES):
            v += amp[i] * np.sin(t[:, None] * w[i] + ph[i])
        out[s:s + len(t)] = v / np.linalg.norm(v, axis=1, keepdims=True)
    return out


def _kv_group(w: Workload, b: int, j: int, delta: float):
    """Q rows of the group's query heads, K and V of kv-head j (float32 values
    of w.dtype).  Own random stream per (seed, b, j): draw order path
    parameters, K noise, V, then the Q noise of each query head ascending."""
    rng = np.random.default_rng([w.seed, b, j])
    Nq, Nkv, D, G = w.Nq, w.Nkv, w.D, w.Hq // w.Hkv
    off = Nkv - Nq
    Qg = np.empty((G, Nq, D), np.float32)
    if w.mode == "path":
        amp = rng.standard_normal((N_SINES, D))
        per = np.exp(rng.uniform(np.log(PERIOD_MIN), np.log(PERIOD_MAX), (N_SINES, D)))
        ph = rng.uniform(0.0, 2.0 * np.pi, (N_SINES, D))
        kk = rng.standard_normal((Nkv, D)) / np.sqrt(D)
        ck = _path(rng, Nkv, 0, D, amp, per, ph)
        kk += w.a * ck
        Vj = round_to(rng.standard_normal((Nkv, D)), w.dtype)
        # query positions off .. Nkv-1 are key positions: same path values
        cq = w.a * ck[off:off + Nq]
        del ck
        for i in range(G):
            Qg[i] = round_to(rng.standard_normal((Nq, D)) / np.sqrt(D) + cq, w.dtype)
    else:
        kk = rng.standard_normal((Nkv, D))
        Vj = round_to(rng.standard_normal((Nkv, D)), w.dtype)
        for i in range(G):
            Qg[i] = round_to(rng.standard_normal((Nq, D)), w.dtype)
    if delta != 0.0 and Nkv > 0 and Nq > 0:
        u = Qg.astype(np.float64).reshape(-1, D).mean(axis=0)
        nu = float(u @ u)
        if nu > 0:
            kk[:SINK_KEYS] += delta * u / (w.scale * nu)
    return Qg, round_to(kk, w.dtype), Vj


def make_inputs(w: Workload, delta: float | None = None, kv_heads=None, threads: int = 8):
    """Returns (Q, K, V) as float32 arrays holding values of w.dtype.

    Q [B, Hq, Nq, D], K and V [B, Hkv, Nkv, D].  Deterministic in w.seed; each
    (batch, kv-head) has its own random stream, so kv_heads (a list of
    (b, j)) may restrict generation to some groups (the rest stay zero).
    """
    from concurrent.futures import ThreadPoolExecutor
    delta = w.delta if delta is None else delta
    B, Hq, Hkv, Nq, Nkv, D = w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D
    G = Hq // Hkv
    Q = np.zeros((B, Hq, Nq, D), np.float32)
    K = np.zeros((B, Hkv, Nkv, D), np.float32)
    V = np.zeros((B, Hkv, Nkv, D), np.float32)
    todo = [(b, j) for b in range(B) for j in range(Hkv)] if kv_heads is None else list(kv_heads)

    def one(bj):
        b, j = bj
        Q[b, j * G:(j + 1) * G], K[b, j], V[b, j] = _kv_group(w, b, j, delta)

    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(todo)))) as ex:
        list(ex.map(one, todo))
    return Q, K, V


def small_workload(B=1, Hq=2, Hkv=1, Nq=64, Nkv=256, D=64, dtype="fp16", mode="path", a=2.0,
                   delta=6.0, eps=0.005, seed=0, causal=1) -> Workload:
    return Workload("custom", B, Hq, Hkv, Nq, Nkv, D, dtype=dtype, mode=mode, a=a, delta=delta,
                    eps=eps, seed=seed, causal=causal)


def digest(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def outlier_value_tiles(V: np.ndarray, n_tiles: int, factor: float = 4.0, seed: int = 0,
                        tile: int = 64, first_tile: int = 0, dtype: str = "fp16") -> np.ndarray:
    """A few key tiles whose values are `factor` times larger than the rest's,
    in place: the chosen tiles keep their values and every other key's value
    is divided by factor, so the largest values stay at the input's own scale.

    Stands in for the tokens with outsized value vectors behind the hazard
    of a cold tile whose small mass carries a large output component ("APA:
    sloppy attention, exact where it counts", section "Honest limits"): per
    (batch, kv-head), n_tiles distinct tiles drawn from [first_tile,
    ceil(Nkv / tile)) by a seeded generator.  The shrunken values are
    rounded to `dtype` again (a power-of-two factor changes only their
    exponent, except where fp16 values fall below its normal range).  Returns
    the chosen tiles [B][Hkv][n]."""
    B, Hkv, Nkv, _ = V.shape
    nt = -(-Nkv // tile)
    rng = np.random.default_rng(seed)
    picks = np.zeros((B, Hkv, n_tiles), np.int64)
    keep = np.zeros(Nkv, bool)
    for b in range(B):
        for j in range(Hkv):
            ts = rng.choice(np.arange(first_tile, nt), size=n_tiles, replace=False)
            picks[b, j] = ts
            keep[:] = False
            for t in ts:
                keep[t * tile:min(Nkv, t * tile + tile)] = True
            V[b, j, ~keep] = round_to(V[b, j, ~keep] / np.float64(factor), dtype)
    return picks
