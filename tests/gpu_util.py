"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
unpack its buffers into the oracle's canonical layouts."""
from __future__ import annotations

import numpy as np

from mixed_precision_long_amd import apa

# position run -> key run inside a 32-key block of the V^T codes
V_RUN_ORDER = [0, 2, 4, 6, 1, 3, 5, 7]


def torch_inputs(Q, K, V, dtype="fp16"):
    import torch
    dt = torch.float16 if dtype == "fp16" else torch.bfloat16
    return tuple(torch.from_numpy(np.ascontiguousarray(x)).to(dt).cuda() for x in (Q, K, V))


def problem_for(w, causal=None, **kw):
    return apa.problem(w.B, w.Hq, w.Hkv, w.Nq, w.Nkv, w.D,
                       dtype=apa.APA_F16 if w.dtype == "fp16" else apa.APA_BF16,
                       causal=w.causal if causal is None else causal, scale=w.scale, **kw)


def nibbles(b: np.ndarray) -> np.ndarray:
    """uint8 [..., n] -> codes [..., 2n], element 2i from the low nibble."""
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.uint8)
    out[..., 0::2] = b & 15
    out[..., 1::2] = b >> 4
    return out


def pack(c: np.ndarray) -> np.ndarray:
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpermute_v(vcodes_gpu: np.ndarray) -> np.ndarray:
    """GPU V^T codes (runs permuted inside 32-key blocks) -> canonical bytes."""
    c = nibbles(vcodes_gpu)
    sh = c.shape
    c = c.reshape(sh[:-1] + (sh[-1] // 32, 8, 4))
    canon = np.empty_like(c)
    for pos, run in enumerate(V_RUN_ORDER):
        canon[..., run, :] = c[..., pos, :]
    return pack(canon.reshape(sh))


def unblob(blobs: np.ndarray, D: int, Nkv: int) -> dict:
    """Per-tile blobs [B, Hkv, NTc, 68 D] (NTc >= NT: a capacity) -> canonical K
    codes/scales [B, Hkv, Nkv, .] and V^T codes/scales [B, Hkv, D, NkvP/.]."""
    blobs = blobs[:, :, :-(-Nkv // 64)]
    B, Hkv, NT, _ = blobs.shape
    kc = blobs[..., :32 * D].reshape(B, Hkv, NT * 64, D // 2)[:, :, :Nkv]
    ks = blobs[..., 32 * D:34 * D].reshape(B, Hkv, NT * 64, D // 32)[:, :, :Nkv]
    vcb = blobs[..., 34 * D:66 * D].reshape(B, Hkv, NT, D, 32)          # [.., t, ch, 32 B]
    vc = unpermute_v(np.ascontiguousarray(vcb.transpose(0, 1, 3, 2, 4)).reshape(B, Hkv, D, NT * 32))
    vsb = blobs[..., 66 * D:68 * D].reshape(B, Hkv, NT, 32, 2, D // 32)  # [.., t, n, hh, db]
    vs = np.ascontiguousarray(vsb.transpose(0, 1, 5, 3, 2, 4)).reshape(B, Hkv, D, NT * 2)
    return dict(kc=kc, ks=ks, vc=vc, vs=vs)


def fp4_sections(p, fp4_host: np.ndarray) -> dict:
    L = apa.fp4_layout(p)
    B, Hq, Hkv, Nq, Nkv, D = p.B, p.Hq, p.Hkv, p.Nq, p.Nkv, p.D
    NqP = -(-Nq // 32) * 32
    NkvP = -(-max(Nkv, p.kv_capacity) // 64) * 64

    def sec(off, count, dtype, shape):
        return np.frombuffer(fp4_host[off:off + count * np.dtype(dtype).itemsize].tobytes(),
                             dtype).reshape(shape)

    extra = {}
    if p.q_terms == 2:
        extra = dict(
            qc2=sec(L.q2_codes, B * Hq * NqP * D // 2, np.uint8, (B, Hq, NqP, D // 2))[:, :, :Nq],
            qs2=sec(L.q2_scales, B * Hq * NqP * D // 32, np.uint8,
                    (B, Hq, NqP, D // 32))[:, :, :Nq])
    return dict(
        **extra,
        qc=sec(L.q_codes, B * Hq * NqP * D // 2, np.uint8, (B, Hq, NqP, D // 2))[:, :, :Nq],
        qs=sec(L.q_scales, B * Hq * NqP * D // 32, np.uint8, (B, Hq, NqP, D // 32))[:, :, :Nq],
        **unblob(sec(L.kv_blobs, B * Hkv * (NkvP // 64) * 68 * D, np.uint8,
                     (B, Hkv, NkvP // 64, 68 * D)), D, Nkv),
        kbar=sec(L.kbar, B * Hkv * D, np.float32, (B, Hkv, D)),
        kv_head=sec(L.kv_head, B * Hkv * 8, np.float32, (B, Hkv, 8)),
        tile_w=sec(L.tile_w, B * Hkv * (NkvP // 64), np.float32,
                   (B, Hkv, NkvP // 64))[..., :-(-Nkv // 64)],
        q_head=sec(L.q_head, B * Hq * 4, np.float32, (B, Hq, 4)),
        q_frame=sec(L.q_frame, B * Hq * NqP, np.float32, (B, Hq, NqP))[:, :, :Nq],
        status=int(sec(L.status, 1, np.uint32, (1,))[0]))


def unpack_bits(p, words: np.ndarray) -> np.ndarray:
    """hot words [B*Hq*NG*W] int32 -> bool [B, Hq, NG, NT]."""
    NT = -(-p.Nkv // 64)
    NG = -(-p.Nq // 16)
    W = -(-NT // 32)
    w = words.view(np.uint32).reshape(p.B, p.Hq, NG, W)
    bits = (w[..., None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(p.B, p.Hq, NG, W * 32)[..., :NT].astype(bool)


def pass1_schedule(p) -> int:
    """The pass-1 schedule a launch with a workspace runs (the library's own
    host-side query)."""
    return apa.pass1_split(p, 0)[0]


# Pass-1 workspace of a split problem (the layout of pass1.hip's Cand): per
# 32-row block the tail's outcome (records kept, or -1: it gave up and the
# head's state walks the tail again) in the first 4 bytes, then `cap` records
# of 292 bytes, rounded up to 256 bytes, then the hand-off state (128 D + 1040
# bytes, rounded up to 256).  The cut of each visit order and cap come from
# the library's query.
def tail_outcomes(p, ws) -> np.ndarray:
    """Outcome of every block whose visit order was cut: number of undecided
    tail tiles decided at the end, or -1 where the tail positions were walked
    again from the head's state."""
    G, NT, nq32 = p.Hq // p.Hkv, -(-p.Nkv // 64), -(-p.Nq // 32)
    cap = apa.pass1_split(p, NT)[2]
    stride = (cap * 292 + 16 + 255) // 256 * 256 + (128 * p.D + 1040 + 255) // 256 * 256
    raw = ws.cpu().numpy()
    out = []
    for b in range(p.B):
        for hk in range(p.Hkv):
            for qb in range(nq32):
                last = min(qb * 32 + 31, p.Nq - 1)
                dW = min(p.Nkv - 1, last + p.Nkv - p.Nq) // 64 if p.is_causal else NT - 1
                if apa.pass1_split(p, dW + 1)[1] >= dW + 1:
                    continue  # walked whole by its head wave
                for gi in range(G):
                    u = ((b * p.Hkv + hk) * nq32 + qb) * G + gi
                    out.append(int(raw[u * stride:u * stride + 4].view(np.int32)[0]))
    return np.array(out, np.int64)


def run_gpu(p, Q, K, V, eps, dtype="fp16", fused=True, lam=True, split=True, tensors=None):
    """Whole APA forward on the GPU; returns numpy copies of every output.
    split=False runs pass 1 without its workspace (one wave per 32-row block).
    tensors: device (q, k, v) to pass instead of Q, K, V (e.g. paged pools)."""
    import torch
    q, k, v = torch_inputs(Q, K, V, dtype) if tensors is None else tensors
    bufs = apa.alloc(p, with_lambda=lam)
    apa.quantize(p, q, k, v, bufs.fp4, bufs.ws_q)
    ws1 = bufs.ws_p1 if split else None
    apa.pass1(p, bufs.fp4, eps, bufs.cold_m, bufs.cold_l, bufs.cold_o, bufs.bits, bufs.lam,
              ws=ws1)
    res = {"tail": tail_outcomes(p, ws1) if ws1 is not None else None}
    if fused:
        apa.pass2(p, q, k, v, bufs.fp4, bufs.bits, bufs.cold_m, bufs.cold_l, bufs.cold_o, True,
                  out=bufs.out, lse=bufs.lse, ws=bufs.ws_p2)
    else:
        B, Hq, Nq, D = p.B, p.Hq, p.Nq, p.D
        hm = torch.empty((B, Hq, Nq), dtype=torch.float32, device="cuda")
        hl = torch.empty_like(hm)
        ho = torch.empty((B, Hq, Nq, D), dtype=torch.float32, device="cuda")
        apa.pass2(p, q, k, v, bufs.fp4, bufs.bits, bufs.cold_m, bufs.cold_l, bufs.cold_o, False,
                  hot_m=hm, hot_l=hl, hot_o=ho, ws=bufs.ws_p2)
        apa.merge(p, bufs.fp4, bufs.cold_m, bufs.cold_l, bufs.cold_o, hm, hl, ho, bufs.out,
                  bufs.lse)
        res.update(hot_m=hm.cpu().numpy(), hot_l=hl.cpu().numpy(), hot_o=ho.cpu().numpy())
    torch.cuda.synchronize()
    res.update(
        fp4=fp4_sections(p, bufs.fp4.cpu().numpy()),
        m=bufs.cold_m.cpu().numpy(), l=bufs.cold_l.cpu().numpy(), o=bufs.cold_o.cpu().numpy(),
        lam=bufs.lam.cpu().numpy() if lam else None,
        hot=unpack_bits(p, bufs.bits.cpu().numpy()),
        out=bufs.out.float().cpu().numpy(), lse=bufs.lse.cpu().numpy())
    return res


def run_exact_gpu(p, Q, K, V, dtype="fp16", tensors=None):
    import torch
    q, k, v = torch_inputs(Q, K, V, dtype) if tensors is None else tensors
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device="cuda")
    apa.exact(p, q, k, v, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def cosine_rows(a, b):
    """Per-row cosine; 1 where both rows are zero, -1 (a failure) where exactly
    one of them is."""
    a = a.reshape(-1, a.shape[-1]).astype(np.float64)
    b = b.reshape(-1, b.shape[-1]).astype(np.float64)
    na, nb = np.linalg.norm(a, axis=1), np.linalg.norm(b, axis=1)
    ok = (na > 0) & (nb > 0)
    c = np.where((na > 0) != (nb > 0), -1.0, 1.0)
    c[ok] = (a[ok] * b[ok]).sum(1) / (na[ok] * nb[ok])
    return c
