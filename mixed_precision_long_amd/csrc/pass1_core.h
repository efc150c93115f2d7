// a3..a7: pass 1 of APA -- every visited key tile in block-scaled FP4 with the
// hot test ("APA: sloppy attention, exact where it counts", rfriedmann.de,
// section "Pass 1: FP4 everywhere, with a hot test", steps 1-5, "Tile order",
// the lazy maximum, and the decoupled cold frame of "The bug: a sink that
// drowned the tail").
//
// One wavefront owns 32 query rows of one query head (two 16-row verdict
// groups) and walks its tiles in the order 0, d, d-1, ..., 1 on its own: no
// cross-wave synchronisation.  Waves are numbered (batch, kv-head, 32-row
// block, head) so the waves of a work group, and the work groups of an XCD,
// stream the same per-tile FP4 blobs through L1/L2 (GQA row packing).  Per
// tile, with the wave's rows as MFMA columns (S^T = K Q^T, so a row's scores
// stay in one lane pair):
//   S^T     : 2x(D/64) scaled FP4 MFMAs 32x32x64 of absolute log2 scores (the
//             power of two that maps FP4 dot products to log2 units is folded
//             into Q's E8M0 bytes).  They do not depend on the frame, so the
//             next tile's are issued as soon as this tile's P is formed and run
//             on the matrix cores during its vote and P V product; K operands
//             are prefetched two tiles ahead, V operands at the tile's start;
//   frame   : integer lazy maximum m, moved to ceil(c) only when the tile max
//             exceeds it by more than tau; a hot tile lifts it to at most
//             max(m, c - H);
//   P       : per 32-key group exponent E = max(-127, ceil(c_g - m - log2 6));
//             code E2M1(2^s / 2^(E + m)) from exp2 of the absolute score and
//             the scaled FP4 conversion, whose power-of-two divisor carries
//             E + m = max(ceil(c_g - log2 6), m - 127); one V_PERMLANE32_SWAP
//             per dword turns the accumulator layout into the MFMA operand
//             layout (V^T is stored in the matching key order);
//   l_t     : one FP4 MFMA of P against a ones selector (numerator and
//             denominator carry the same quantisation);
//   vote    : row hot iff l_t > eps * lambda (lambda includes this tile),
//             with value-norm weights l_t * w_t > eps * lambda; ballot over
//             16 rows;
//   cold PV : O^T += V^T P^T for the rows of cold groups, FP4 MFMA.
// The accumulated state (o, l, lambda) is held in a second integer frame m_o
// per row that trails the method's frame: P's E8M0 byte is E + m - m_o + 127,
// so l_t, lambda, l and o arrive already scaled by the exact power of two
// 2^(m - m_o), and a moving frame costs no rescale of o.  m_o is re-based
// (o, l, lambda scaled down by an exact power of two) on the first tile and
// whenever m runs more than kFrameGuard ahead, which keeps every scale byte
// and the state inside FP32 range; the outputs are returned in the method's
// frame.  Powers of two commute with rounding, so the verdicts and the state
// equal those of the method's own frame bookkeeping (up to FP32 underflow of
// values 2^-100 below the row maximum).
// Hot bits are written as whole 32-tile words, so every word of the mask is
// defined without a clearing pass.  Up to 4096 key tiles the loop only logs
// each tile's two verdicts as an LDS byte, and the words are built after the
// walk (lane j builds one word); beyond that they are kept in the loop.
//
// Balance.  With fewer units than the chip's wave slots, a wave per unit
// leaves SIMDs idle while others run two waves, so each long visit order is
// cut in two and walked by two waves of one work group at once: the head wave
// takes positions [0, h) (tile 0, the diagonal and the recent part), a tail
// wave positions [h, n).  While two waves per unit fit the slots, every unit
// has its own tail wave (cut near the middle); while four waves per three
// units fit, a work group holds three units, their three head waves and one
// wave that walks the three tails (cut near three quarters) one after the
// other, parking each tail's state in the workspace until the heads are done,
// so that every SIMD keeps two waves to the end.  A tail walk does not know
// lambda at position h.  It first replays positions [0, 32) without P V (a
// prefix of the head's walk, so its lambda is a lower bound of the head's),
// then walks its own tiles with the vote taken against a lower bound plus its
// own running lambda: the larger of the replayed lambda and the head's
// current lambda, which the head keeps publishing in LDS (lambda only grows,
// so any value read is a bound).  A group that fails the bounded test fails
// the true one, so it is cold for sure; a group that passes it is undecided:
// it is treated as cold for now (its P V is accumulated) and its per-row l_t,
// running tail lambda and frame are recorded in the workspace.  At its end the
// head leaves its state in LDS; the tail waits for it, decides every recorded
// group against the head's final lambda, takes the P V of the ones that turn
// out hot back out of its state (the same FP4 codes with the sign bit set, so
// the subtraction is of exactly what was added), sets their bits, and merges
// the two states (their frames only scale them).  If the record fills up, or
// the tail's frame would need a re-base, the tail walks positions [h, n) again
// from the head's state instead.
#pragma once

#include <type_traits>

#include "apa_device.h"
#include "apa_kernels.h"

namespace apa {

namespace {

constexpr float kFrameGuard = 80.0f; // largest lead of m over m_o before re-basing
constexpr int kMinSplit = 64;        // shortest visit order that runs as two waves
constexpr int kMinTail = 8;          // fewest positions a tail wave walks past its replay
constexpr int kReplay = 32;          // leading positions the tail wave replays
constexpr int kCandCap = 512;        // most undecided tail tiles recorded per unit

enum Role { kWhole = 0, kHead = 1, kTail = 2 };

// a float in LDS (an address-space-3 pointer keeps the accesses DS
// instructions, which wait on their own counter, not on vector memory)
typedef __attribute__((address_space(3))) float lds_float;
// a read-only global float read through the scalar cache (uniform index)
typedef __attribute__((address_space(4))) const float cfloat;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Problems with at most this many key tiles log each visited tile's verdict
// as one LDS byte per wave and build the hot words after the walk (no word
// bookkeeping in the tile loop); longer ones keep the words in the loop.
constexpr int kLogTiles = 4096;

// Two waves per SIMD up to D = 128; one above, where the output accumulators
// (D/2 per lane) need the accumulation registers.
template <int D>
constexpr int kWavesPerSimd = D >= 256 ? 1 : 2;

// Wavefronts per work group: with two waves per SIMD (D <= 128) a group of
// eight, so the two waves that share a SIMD (w and w + 4) belong to one
// group and pace each other through LDS (a wave behind its partner takes the
// higher issue priority; by default the older wave wins every tie and the
// younger one finishes alone, at the lower one-wave rate); four above.
template <int D>
constexpr int kP1Waves = D >= 256 ? 4 : 8;

// Head states a work group holds in LDS: three per four waves (triple
// schedule) up to D = 256; none used at D = 512 (one wave pair per unit, no
// head/tail split).
template <int D>
constexpr int kSlots = D >= 512 ? 1 : 3 * kP1Waves<D> / 4;

typedef __attribute__((address_space(3))) int lds_int;

// Output channels per wave.  At D = 512 a unit runs as two waves, each with
// the accumulators of half of the output channels (32 x 256 FP32: 128
// registers per lane instead of 256, which with the operands of a tile would
// not fit): both walk the same tiles with the same scores, frames and
// verdicts (the same arithmetic on the same operands), each adds the P V of
// its own channels, and only the first writes the row scalars and hot words.
template <int D>
constexpr int kOutSplit = D >= 512 ? 2 : 1;

template <int D>
struct Tile {
  static constexpr int NH = D / 64;       // 64-channel halves of the QK contraction
  static constexpr int ND = D / 32;       // 32-channel blocks of the output
  static constexpr int NDO = ND / kOutSplit<D>;  // of them, held by one wave
  static constexpr int NW = (D / 32 + 3) / 4;  // 32-bit words of one key's scale bytes
  static constexpr int NWO = (NDO + 3) / 4;    // of one V lane's scale bytes (a wave's)
  static constexpr int BLOB = 68 * D;
};

// Scaled FP4 MFMA 32x32x64; the E8M0 scales are byte `opa` of sa (A rows)
// and byte `opb` of sb (B columns).  The selectors fold to constants after
// unrolling.
template <int OPA, int OPB>
__device__ __forceinline__ v16f mfma4_sel(v4i a, v4i b, v16f c, int sa, int sb) {
  v8i A = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i B = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, OPA, sa, OPB, sb);
}
__device__ __forceinline__ v16f mfma4(v4i a, v4i b, v16f c, int sa, int opa, int sb) {
  switch (opa) {
    case 0: return mfma4_sel<0, 0>(a, b, c, sa, sb);
    case 1: return mfma4_sel<1, 0>(a, b, c, sa, sb);
    case 2: return mfma4_sel<2, 0>(a, b, c, sa, sb);
    default: return mfma4_sel<3, 0>(a, b, c, sa, sb);
  }
}

// Row sums of the quantised P by one scaled FP4 MFMA 16x16x128 (half the
// matrix cycles of a 32x32x64 product against ones).  It reads the P operand,
// laid out for the 32x32x64 products (lane l: row l%32, keys 32*(l/32)..+31),
// as column l%16 with K block l/16, so column c holds row c in blocks 0 and 2
// and row c+16 in blocks 1 and 3.  The selector operand holds E2M1 ones in
// blocks 0 and 2 of rows 0 and 8 and in blocks 1 and 3 of rows 4 and 12 (zeros
// elsewhere); row c's sum then lands in C[0][c] and C[8][c], row c+16's in
// C[4][c] and C[12][c], and the result register 0 of lane l (element
// C[4*(l/16)][l%16]) is the sum of the lane's own row.
__device__ __forceinline__ v4i rowsum_selector(int lane) {
  const int r = lane & 7;          // row l%16 of A, modulo 8
  const int odd = (lane >> 4) & 1;  // K block l/16 is 1 or 3
  const int w = (r == 0 && !odd) || (r == 4 && odd) ? kE2M1Ones : 0;
  return v4i{w, w, w, w};
}

__device__ __forceinline__ float rowsum4(v4i sel, v4i p, int sp) {
  v8i A = {sel[0], sel[1], sel[2], sel[3], 0, 0, 0, 0};
  v8i B = {p[0], p[1], p[2], p[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, v4f{}, 4, 4, 0, kE8M0One, 0,
                                                          sp)[0];
}

// A unit's tile blobs are read through a buffer resource: the lane's offset
// inside a blob is a fixed 32-bit VGPR, the tile's offset a scalar, so no
// per-tile 64-bit address arithmetic and no address registers per load.
typedef __amdgpu_buffer_rsrc_t Rsrc;

__device__ __forceinline__ Rsrc blob_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ v4i bload128(Rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// NB scale bytes (of one key, or one V lane's blocks) as little-endian words.
template <int NB>
__device__ __forceinline__ void load_scales(uint32_t (&w)[(NB + 3) / 4], Rsrc r, uint32_t voff,
                                            uint32_t soff) {
  if constexpr (NB == 2) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  } else if constexpr (NB == 4) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  } else if constexpr (NB == 8) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    w[0] = x[0];
    w[1] = x[1];
  } else {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    w[0] = x[0];
    w[1] = x[1];
    w[2] = x[2];
    w[3] = x[3];
  }
}

template <int D>
struct KOps {
  v4i a[2][Tile<D>::NH];
  uint32_t s[2][Tile<D>::NW];  // shifted so byte 2*(h%2) of word h/2 is block 2h + hh
};

template <int D>
__device__ __forceinline__ void load_k(KOps<D>& k, Rsrc r, uint32_t soff, uint32_t koff,
                                       uint32_t ksoff, int hh) {
  constexpr int NH = Tile<D>::NH;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int h = 0; h < NH; ++h) k.a[kb][h] = bload128(r, koff + kb * 32 * (D / 2) + 32 * h, soff);
    load_scales<D / 32>(k.s[kb], r, ksoff + kb * 32 * (D / 32), soff);
#pragma unroll
    for (int w = 0; w < Tile<D>::NW; ++w) k.s[kb][w] >>= 8 * hh;
  }
}

// S^T for one tile: two 32-key blocks, absolute log2 scores.
template <int D>
__device__ __forceinline__ void qk(v16f (&acc)[2], const KOps<D>& k, const v4i* qa, const int* qs) {
  constexpr int NH = Tile<D>::NH;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    acc[kb] = mfma4(k.a[kb][0], qa[0], v16f{}, (int)k.s[kb][0], 0, qs[0]);
#pragma unroll
    for (int h = 1; h < NH; ++h)
      acc[kb] = mfma4(k.a[kb][h], qa[h], acc[kb], (int)k.s[kb][h >> 1], 2 * (h & 1), qs[h]);
  }
}


// One unit: 32 query rows of one query head.
struct UnitId {
  int b, hk, qb, gi;
};

// Units are numbered (batch, kv-head, 32-row block, head in group), heads
// innermost.
__device__ __forceinline__ UnitId unit_id(const Geom& g, int u) {
  const int nq32 = g.NqP / 32;
  UnitId id;
  id.gi = u % g.G; u /= g.G;
  id.qb = u % nq32; u /= nq32;
  id.hk = u % g.Hkv;
  id.b = u / g.Hkv;
  return id;
}

__device__ __forceinline__ int unit_index(const Geom& g, const UnitId& id) {
  return ((id.b * g.Hkv + id.hk) * (g.NqP / 32) + id.qb) * g.G + id.gi;
}

// What a wave needs to walk one unit's tiles.
template <int D>
struct CtxBase {
  size_t bhq, bhk;
  int r0, row, d0, d1, dW;
  // sliding window: the first tile each verdict group sees (0 without one);
  // sh = 1 when the walk starts with tile 0 (the first row sees it), so
  // position p is tile 0 for p = 0 and dW + 1 - p after; sh = 0: dW - p
  int lo0, lo1, sh;
  int tmask;     // tiles t >= tmask need the mask (diagonal, padding keys, rows past Nq)
  int tmask_lo;  // tiles t < tmask_lo need the window's lower mask
  bool row_ok, has_g1;
  v4i qa[Tile<D>::NH];  // Q^T operand, 16 bytes per 64-channel half
  int qs[Tile<D>::NH];  // its E8M0 bytes (block scale + head exponent)
  Rsrc blobs;  // the unit's kv-head: NT tile blobs
  uint32_t koff, ksoff, voff, vsoff;  // this lane's byte offsets inside a blob
  int dh;     // which share of the output channels the wave holds
  bool lead;  // the wave that writes the row scalars and hot words (dh = 0)
  float g_v;
  const cfloat* tw;  // value-norm weights of the kv-head's tiles (nullptr: mass test)
  uint32_t *bits0, *bits1;  // hot words of the two verdict groups
  int ring_delta;  // window ring: blob slot of tile t >= 1 is t + ring_delta
  // the visit order: positions [0, npos()), position p at tile tile_of(p)
  __device__ __forceinline__ int npos() const { return dW + 1 - lo0; }
  __device__ __forceinline__ int tile_of(int p) const { return sh && p == 0 ? 0 : dW + sh - p; }
};

// The context with one Q term, and with two (the FP4 residual of Q as a
// second B operand of the score MFMAs, beside the first, on the K operands
// already loaded: "Second
// hunt: which operand is to blame").
template <int D, int QT>
struct Ctx : CtxBase<D> {};
template <int D>
struct Ctx<D, 2> : CtxBase<D> {
  v4i qa2[Tile<D>::NH];
  int qs2[Tile<D>::NH];
};

template <int D>
__device__ __forceinline__ void make_ctx(CtxBase<D>& c, const Geom& g, const Fp4Ptrs& f,
                                         const Pass1Out& out, const UnitId& id, int lane,
                                         int dh = 0) {
  constexpr int NH = Tile<D>::NH;
  constexpr int ND = Tile<D>::ND;
  const int n = lane & 31, hh = lane >> 5;
  const int hq = id.hk * g.G + id.gi;
  c.bhq = (size_t)id.b * g.Hq + hq;
  c.bhk = (size_t)id.b * g.Hkv + id.hk;
  c.r0 = id.qb * 32;
  c.row = c.r0 + n;
  c.row_ok = c.row < g.Nq;
  auto diag = [&](int lr) { return g.causal ? min(g.Nkv - 1, lr + g.off) / kTile : g.NT - 1; };
  c.has_g1 = c.r0 + 16 < g.Nq;
  c.d0 = diag(min(c.r0 + 15, g.Nq - 1));
  c.d1 = c.has_g1 ? diag(min(c.r0 + 31, g.Nq - 1)) : -1;
  c.dW = max(c.d0, c.d1);
  // with a window, the first key of row r is r + off - window + 1
  const bool win = g.causal && g.window > 0;
  auto first_tile = [&](int fr) { return win ? max(0, fr + g.off - g.window + 1) / kTile : 0; };
  c.lo0 = first_tile(c.r0);
  c.lo1 = c.has_g1 ? first_tile(c.r0 + 16) : 0x7fffffff;
  c.sh = c.lo0 == 0 ? 1 : 0;
  {
    const int e = c.r0 + 31 + g.off - g.window;  // keys <= e are outside some row's window
    c.tmask_lo = win && e >= 0 ? e / kTile + 1 : 0;
  }
  // a tile needs the mask when it holds keys past Nkv (t >= Nkv / 64), keys
  // past a row's diagonal (64 t + 63 > r0 + off) or rows past Nq
  c.tmask = c.r0 + 31 >= g.Nq ? 0 : min(g.Nkv / kTile, g.causal ? (c.r0 + g.off + 1) / kTile : g.NT);
  const int jq = (int)f.q_head[c.bhq * 4 + 2];
  const uint8_t* qc = f.q_codes + (c.bhq * g.NqP + c.row) * (D / 2);
  const uint8_t* qsc = f.q_scales + (c.bhq * g.NqP + c.row) * (D / 32);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    c.qa[h] = *reinterpret_cast<const v4i*>(qc + 32 * h + 16 * hh);
    const int sb = (int)qsc[2 * h + hh] + jq;
    c.qs[h] = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
  }
  c.g_v = f.kv_head[c.bhk * 8 + 4];
  c.tw = g.vweight ? (const cfloat*)(f.tile_w + c.bhk * (size_t)g.NTc) : nullptr;
  c.blobs = blob_rsrc(f.kv_blob + c.bhk * (size_t)g.NTc * Tile<D>::BLOB,
                      (uint32_t)(g.ring ? g.NTc : g.NT) * Tile<D>::BLOB);
  c.ring_delta = g.ring_delta;
  c.koff = n * (D / 2) + 16 * hh;
  c.ksoff = 32 * D + n * (D / 32);
  constexpr int NDO = Tile<D>::NDO;
  c.dh = dh;
  c.lead = dh == 0;
  c.voff = 34 * D + n * 32 + 16 * hh + dh * NDO * 32 * 32;
  c.vsoff = 66 * D + (2 * n + hh) * ND + dh * NDO;
  c.bits0 = out.bits + (c.bhq * g.NG + (c.r0 >> 4)) * g.W;
  c.bits1 = c.bits0 + g.W;
}

// S^T with every Q term of the context: the residual term accumulates into
// the same scores, on the K operands already loaded.
template <int D>
__device__ __forceinline__ void qk_all(v16f (&acc)[2], const KOps<D>& k, const Ctx<D, 1>& c) {
  qk<D>(acc, k, c.qa, c.qs);
}
template <int D>
__device__ __forceinline__ void qk_all(v16f (&acc)[2], const KOps<D>& k, const Ctx<D, 2>& c) {
  constexpr int NH = Tile<D>::NH;
  qk<D>(acc, k, c.qa, c.qs);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < NH; ++h)
      acc[kb] = mfma4(k.a[kb][h], c.qa2[h], acc[kb], (int)k.s[kb][h >> 1], 2 * (h & 1), c.qs2[h]);
}

// The residual Q term's operand and E8M0 bytes (with the same head exponent
// as the first term); nothing with one term.
template <int D>
__device__ __forceinline__ void load_q2(Ctx<D, 1>&, const Geom&, const Fp4Ptrs&, int) {}
template <int D>
__device__ __forceinline__ void load_q2(Ctx<D, 2>& c, const Geom& g, const Fp4Ptrs& f, int lane) {
  const int hh = lane >> 5;
  const int jq = (int)f.q_head[c.bhq * 4 + 2];
  const uint8_t* qc = f.q2_codes + (c.bhq * g.NqP + c.row) * (D / 2);
  const uint8_t* qsc = f.q2_scales + (c.bhq * g.NqP + c.row) * (D / 32);
#pragma unroll
  for (int h = 0; h < Tile<D>::NH; ++h) {
    c.qa2[h] = *reinterpret_cast<const v4i*>(qc + 32 * h + 16 * hh);
    const int sb = (int)qsc[2 * h + hh] + jq;
    c.qs2[h] = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
  }
}

// The accumulated cold state of one row (both lane halves hold the row's
// scalars; o is in the MFMA result layout).
template <int D>
struct St {
  float mf;  // the method's frame: an integer, -inf before the first key
  int mo;    // the state's frame
  float lam, lsum;
  v16f o[Tile<D>::NDO];
};

// Rows past Nq never see a key and sit at frame 64 so every derived quantity
// stays finite (and their P divisors inside the conversion's fast range); mo
// starts far below any frame so that the first tile re-bases.
template <int D>
__device__ __forceinline__ void init_state(St<D>& st, bool row_ok) {
  st.mf = row_ok ? -__builtin_inff() : 64.0f;
  st.mo = -(1 << 20);
  st.lam = 0.0f;
  st.lsum = 0.0f;
#pragma unroll
  for (int i = 0; i < Tile<D>::NDO; ++i) st.o[i] = v16f{};
}

// Hot words a walk could not complete by itself: word 0 (tile 0 belongs to the
// head segment of a split unit) and the word holding both sides of the split
// point (wb; -1 when the split point is a word boundary or the unit is whole).
struct Words {
  int wb;
  uint32_t p00, p01, p10, p11;  // word 0 / word wb, verdict group 0 / 1
};

__device__ __forceinline__ int shared_word(int tb) { return ((tb + 1) & 31) ? (tb >> 5) : -1; }

// Schedules of the 32-row units over wavefronts (the values of the problem's
// pass-1 schedule): one wave per unit; a head and a tail wave per unit; three
// head waves and one wave that walks the three tails, per three units.
enum Sched { kSchedWhole = 1, kSchedPairs = 2, kSchedTriples = 3 };

// Where a visit order of npos positions is cut: the head walks [0, cut), the
// tail replays kReplay positions and walks [cut, npos), and its tiles cost a
// little more (the record keeping).  With a tail per unit the head takes half
// of npos + kReplay plus about 1.5 %; with one tail wave for three units,
// three quarters of it (the tail wave then walks three quarter tails and
// settles three units) plus about 3 %, the share that measured fastest at
// 2048 x 122880.  A unit is cut only when that leaves the tail at least
// kMinTail positions (under the triple rule from about 150 positions on);
// otherwise the result is npos and its head wave walks it whole.  Either way
// kReplay <= cut <= npos, and cut < npos means a tail of >= kMinTail positions.
__host__ __device__ inline int split_cut(int npos, int sched) {
  if (npos < kMinSplit) return npos;
  const int cut = sched == kSchedTriples ? 3 * (npos + kReplay) / 4 + npos / 32
                                         : (npos + kReplay) / 2 + npos / 64;
  return npos - cut >= kMinTail ? cut : npos;
}

template <int D>
__device__ __forceinline__ void put_word(const CtxBase<D>& c, Words& wd, int w, uint32_t b0,
                                         uint32_t b1, int lane) {
  if (w == 0) {
    wd.p00 |= b0;
    wd.p01 |= b1;
  } else if (w == wd.wb) {
    wd.p10 |= b0;
    wd.p11 |= b1;
  } else if (lane == 0 && c.lead) {
    c.bits0[w] = b0;
    if (c.has_g1) c.bits1[w] = b1;
  }
}

// Undecided tail tiles of one unit, in the workspace: the tail's outcome
// (records kept, or -1 when it gave up and walked again from the head's
// state), then `cap` records of the tile (with a flag per verdict group) and,
// per row, l_t, the tail's running lambda and the lazy frame as an offset from
// the state frame (0 .. 80).  Accessed through a buffer resource over the
// unit's block (scalar base and offsets, so the rarely taken record branch
// holds no 64-bit address registers).
struct Cand {
  Rsrc r;
  uint32_t tile, ell, lamb, dm;  // byte offsets of the arrays in the block
};

__host__ __device__ inline size_t cand_bytes(int cap) {
  return ((size_t)cap * 292 + 16 + 255) & ~(size_t)255;
}

// After the records: room for the head's final state, which a tail that gave
// up leaves there for the re-walk (k_pass1_rewalk, or the single launch's
// re-walk step): o in lane order, then the per-lane scalars mf, mo, lambda,
// l, then the head's partial words.
__host__ __device__ inline size_t handoff_bytes(int D) {
  return ((size_t)128 * D + 1024 + 16 + 255) & ~(size_t)255;
}

__host__ __device__ inline size_t cand_stride(int cap, int D) {
  return cand_bytes(cap) + handoff_bytes(D);
}

__device__ __forceinline__ Cand cand_of(uint8_t* ws, int unit, int cap, int D) {
  const size_t stride = cand_stride(cap, D);
  return Cand{blob_rsrc(ws + (size_t)unit * stride, (uint32_t)stride), 16u, 16u + 4u * cap,
              16u + 132u * cap, 16u + 260u * cap};
}

// The head wave's final state, handed to the tail wave in LDS.
template <int D>
struct HeadState {
  v4f o[Tile<D>::NDO * 4][64];  // o in lane order: float4 chunk q of block db at [4 db + q]
  float sc[4][64];             // mf, mo (its bits), lambda, l per lane
  uint32_t words[4];           // partial words: word 0 and word wb, groups 0 and 1
  int done;
};

// masking: causal diagonal, padding keys, rows past Nq (wave-uniform test)
template <int D>
__device__ __forceinline__ void mask_scores(v16f (&acc)[2], const Geom& g, const CtxBase<D>& c, int t,
                                            int hh) {
  const int k0 = t * kTile;
  if (t >= c.tmask || t < c.tmask_lo) {
    const int lim = g.causal ? c.row + g.off : 0x7fffffff;
    const int lim_lo = g.causal && g.window > 0 ? c.row + g.off - g.window : -1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
        if (!(c.row_ok && key < g.Nkv && key <= lim && key > lim_lo))
          acc[kb][j] = -__builtin_inff();
      }
  }
}

// Maxima of the tile's two 32-key groups (keys 0-31: b0, 32-63: b1) of this
// lane's row, in every lane: each lane's partial maxima, one exchange that
// gives lanes < 32 both halves of group 0 and lanes >= 32 both halves of
// group 1, and one that hands each lane the other group's maximum.
__device__ __forceinline__ void group_maxima(const v16f (&acc)[2], float& b0, float& b1) {
  float gl0 = vmax(acc[0][0], acc[0][1]), gl1 = vmax(acc[1][0], acc[1][1]);
#pragma unroll
  for (int j = 2; j < 16; j += 2) {
    gl0 = vmax3(gl0, acc[0][j], acc[0][j + 1]);
    gl1 = vmax3(gl1, acc[1][j], acc[1][j + 1]);
  }
  int x0, x1;
  swap_halves(__float_as_int(gl0), __float_as_int(gl1), x0, x1);
  const int own = __float_as_int(vmax(__int_as_float(x0), __int_as_float(x1)));
  swap_halves(own, own, x0, x1);
  b0 = __int_as_float(x0);
  b1 = __int_as_float(x1);
}

// Whether both P divisors 2^x0, 2^x1 of every lane are normal with room below
// for the codes that matter: the fast form of the conversion.
__device__ __forceinline__ bool divisors_fast(int x0, int x1) {
  return __ballot((unsigned)(x0 + 124) > 244u || (unsigned)(x1 + 124) > 244u) == 0ull;
}

// Step 2: the FP4 codes of P for divisors 2^x0 (keys 0-31) and 2^x1 (keys
// 32-63), rearranged into the MFMA operand layout (lanes < 32 carry keys 0-31,
// lanes >= 32 keys 32-63).  fast: see divisors_fast.
__device__ __forceinline__ v4i p_operand(const v16f (&acc)[2], int x0, int x1, float x0f,
                                         float x1f, bool fast) {
  unsigned pk[2][2];
  if (fast) {
    const float sc0 = __int_as_float((x0 + 127) << 23), sc1 = __int_as_float((x1 + 127) << 23);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float sc = kb ? sc1 : sc0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // every byte is written below: the starting value does not matter (a
        // distinct non-volatile placeholder per word: no move, no barrier)
        unsigned w;
        asm("" : "=v"(w) : "n"(2 * kb + j));
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int i = 8 * j + 2 * p;
          w = cvt_fp4x2(w, fast_exp2(acc[kb][i]), fast_exp2(acc[kb][i + 1]), sc, p);
        }
        pk[kb][j] = w;
      }
    }
  } else {
    // frame-relative form 2^(s - X) with a unit divisor
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float sub = kb ? x1f : x0f;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        unsigned w;
        asm("" : "=v"(w) : "n"(4 + 2 * kb + j));
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int i = 8 * j + 2 * p;
          w = cvt_fp4x2(w, fast_exp2(acc[kb][i] - sub), fast_exp2(acc[kb][i + 1] - sub), 1.0f, p);
        }
        pk[kb][j] = w;
      }
    }
  }
  v4i r = {(int)pk[0][0], (int)pk[0][1], (int)pk[1][0], (int)pk[1][1]};
  int a, b;
  swap_halves(r[0], r[2], a, b);
  r[0] = a;
  r[2] = b;
  swap_halves(r[1], r[3], a, b);
  r[1] = a;
  r[3] = b;
  return r;
}

// The hot words of a walk's positions [P0, P0 + np) from its verdict log
// (tile t at vlog[t]): the tiles of positions max(P0, sh) .. P0 + np - 1 (a
// descending run) and, when the order starts with tile 0 and P0 = 0, tile 0.
// Lane j builds word w_lo + j; words 0 and wb go to the partial words, the
// others are stored.
template <int D>
__device__ __forceinline__ void assemble_words(const CtxBase<D>& c, Words& wd, const lds_u8* vlog,
                                               int P0, int np, int lane) {
  const int t_hi = c.dW + c.sh - max(P0, c.sh);  // tile of the first position past tile 0
  const int t_lo = c.dW + c.sh - (P0 + np - 1);  // tile of the last position
  if (c.sh && P0 == 0 && np > 0) {
    const uint32_t v = vlog[0];
    wd.p00 |= v & 1u;
    wd.p01 |= v >> 1;
  }
  if (t_lo > t_hi) return;
  for (int w0 = t_lo >> 5; w0 <= (t_hi >> 5); w0 += 64) {
    const int w = w0 + lane;
    uint32_t b0 = 0u, b1 = 0u;
    if (w <= (t_hi >> 5)) {
      const int a = max(32 * w, t_lo), e = min(32 * w + 31, t_hi);
      for (int tt = a; tt <= e; ++tt) {
        const uint32_t v = vlog[tt];
        b0 |= (v & 1u) << (tt & 31);
        b1 |= (v >> 1) << (tt & 31);
      }
      if (w != 0 && w != wd.wb && c.lead) {
        c.bits0[w] = b0;
        if (c.has_g1) c.bits1[w] = b1;
      }
    }
    // the partial words, from the lane that built them
    if (w0 == 0) {
      wd.p00 |= (uint32_t)__builtin_amdgcn_readlane((int)b0, 0);
      wd.p01 |= (uint32_t)__builtin_amdgcn_readlane((int)b1, 0);
    }
    if (wd.wb > 0 && wd.wb >= w0 && wd.wb < w0 + 64) {
      wd.p10 |= (uint32_t)__builtin_amdgcn_readlane((int)b0, wd.wb - w0);
      wd.p11 |= (uint32_t)__builtin_amdgcn_readlane((int)b1, wd.wb - w0);
    }
  }
}

// Walks cnt positions of a unit's visit order 0, d, d-1, ..., 1: first the
// positions 0 .. nrep-1 as a replay (state and vote only: no P V, no hot
// bits), then positions p0, p0+1, ...  A walk with a replay is a tail walk:
// after the replay its vote is taken against a lower bound of the head's
// lambda (the replayed lambda, or what the head has published in `pub_in`,
// whichever is larger) plus its own lambda; groups that pass are recorded in
// cr and treated as cold, and it returns the number of records, or -1 when it
// has to give up (record full, or a re-base of the state frame).  Other walks
// return 0.  A head walk publishes its lambda from position nrep_tail on in
// `pub_out`, in the state frame it had there (the frame the tail's replay ends
// in).
template <int D, bool LOG, bool TAIL, bool VW, int QT, bool RING = false>
__device__ __forceinline__ int walk(const Geom& g, const Ctx<D, QT>& c, St<D>& st, Words& wd, int nrep,
                                    int p0, int cnt, float eps, float tau, float Hf, const Cand& cr,
                                    int cap, const volatile lds_float* pub_in,
                                    volatile lds_float* pub_out, lds_u8* vlog, int lane,
                                    volatile lds_int* pace_me = nullptr,
                                    const volatile lds_int* pace_mate = nullptr,
                                    int pace_base = 0) {
  constexpr int ND = Tile<D>::NDO;  // output blocks of this wave
  constexpr int NW = Tile<D>::NWO;
  constexpr int BLOB = Tile<D>::BLOB;
  const int n = lane & 31;  // the wave's row handled by this lane
  const int hh = lane >> 5; // which half of the K dimension this lane feeds
  // lanes of verdict group 0 (rows r0 .. r0+15) in both lane halves
  constexpr unsigned long long kGroup0 = 0x0000FFFF0000FFFFull;
  const bool tail = TAIL;  // a tail walk (nrep > 0); its own copy of the loop
  auto tile_at = [&](int i) { return c.tile_of(i < nrep ? i : p0 + (i - nrep)); };
  float lam_lo = 0.0f;
  int mo_ref = 0;
  int ncand = 0;
  bool gave_up = false;  // leaves the loop at its latch (one exit keeps the state in place)
  int cur_w = -1;
  uint32_t cur_b0 = 0, cur_b1 = 0;

  // pipeline: when position i starts, its scores are in acc, the K operand
  // of position i+1 in kn and its own V^T operand in va; once this tile's P
  // is formed, QK(i+1) is issued into acc and K of position i+2 is fetched
  // into kn; once its P V product is issued, V^T of position i+1 is fetched
  // into va (prefetches past the last position re-read the last tile: in
  // bounds, unused)
  auto next_blob = [&](int i) {
    const int t = tile_at(min(i, cnt - 1));
    return (uint32_t)((RING && t ? t + c.ring_delta : t) * BLOB);
  };
  KOps<D> kn;
  v16f acc[2];
  v4i va[ND];
  uint32_t vsw[NW];
  auto load_v = [&](uint32_t blob) {
#pragma unroll
    for (int db = 0; db < ND; ++db) va[db] = bload128(c.blobs, c.voff + db * 32 * 32, blob);
    load_scales<ND>(vsw, c.blobs, c.vsoff, blob);
  };
  // (issued in the loop's own order, K(i+1) before V(i), so the waits the
  // compiler places at the loop head count only the loads they need)
  // the selector operand of the row-sum MFMA, kept in registers (made opaque
  // before any load is in flight)
  v4i ones = rowsum_selector(lane);
  asm volatile("" : "+v"(ones));
  load_k<D>(kn, c.blobs, next_blob(0), c.koff, c.ksoff, hh);
  // blob offset of the K operand fetched last (position i + 1 when position
  // i starts): the V operand of position i + 1 is fetched from it at the end
  // of position i
  qk_all<D>(acc, kn, c);
  uint32_t kblob = next_blob(1);
  load_k<D>(kn, c.blobs, kblob, c.koff, c.ksoff, hh);
  load_v(next_blob(0));
  // eps = 0 marks every visited tile hot: with -1 as the factor, every row
  // with mass so far passes (l_t > -lambda), and every visible group has one
  const float epsv = eps == 0.0f ? -1.0f : eps;

  for (int i = 0; i < cnt && !gave_up; ++i) {
    const int t = tile_at(i);
    // the tile's weight in the vote (a scalar load, consumed after the MFMAs;
    // the mass test compiles without it)
    const float wt = VW ? c.tw[t] : 1.0f;
    const bool replay = i < nrep;
    // pacing: publish this wave's position count; the SIMD partner's is read
    // now and compared once the tile's maxima are done
    int mate = 0;
    if (pace_me) {
      *pace_me = pace_base + i;
      mate = *pace_mate;
    }
    if (tail && i == nrep) {
      lam_lo = st.lam;
      st.lam = 0.0f;
    }
    if (!TAIL && i == kReplay) mo_ref = st.mo;

    const bool vis0 = t <= c.d0 && t >= c.lo0, vis1 = t <= c.d1 && t >= c.lo1;
    mask_scores<D>(acc, g, c, t, hh);
    float b0, b1;
    group_maxima(acc, b0, b1);
    const float cmax = vmax(b0, b1);
    if (pace_me) {
      if (pace_base + i > __builtin_amdgcn_readfirstlane(mate))
        __builtin_amdgcn_s_setprio(0);
      else
        __builtin_amdgcn_s_setprio(1);
    }

    // ---- lazy maximum (integer frame): the frame moves only where the tile
    // maximum exceeds it by more than tau (never for a row without a visible
    // key here), which after the first tiles is rare
    float mcf = st.mf;
    if (__ballot(cmax > st.mf + tau) != 0ull) {
      if (cmax > st.mf + tau) mcf = ceilf(cmax);
      // re-base the state to m_o = max(m, mc - H), a lower bound of every
      // later frame, when the frame has run too far ahead (all lanes; exact
      // powers of two).  Only a moving frame can need it: after every tile
      // m <= mc <= m_o + kFrameGuard.
      if (__ballot(mcf - (float)st.mo > kFrameGuard) != 0ull) {
        if (tail && !replay) gave_up = true;
        const int mo_new = (int)vmax(st.mf, mcf - Hf);
        const int sh = st.mo - mo_new;
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) st.o[db][j] = ldexpf(st.o[db][j], sh);
        st.lsum = ldexpf(st.lsum, sh);
        st.lam = ldexpf(st.lam, sh);
        st.mo = mo_new;
      }
    }

    // ---- step 2: the conversion divisor 2^X of each 32-key group,
    // X = E + m = max(ceil(c_g - log2 6), m - 127)
    const float lo = mcf - 127.0f;
    const float x0 = vmax(ceilf(b0 - kLog2_6), lo);
    const float x1 = vmax(ceilf(b1 - kLog2_6), lo);
    const int x0i = (int)x0, x1i = (int)x1;
    const v4i pb = p_operand(acc, x0i, x1i, x0, x1, divisors_fast(x0i, x1i));
    // E8M0 byte of this lane's 32-key group (the B operand's K block) in the
    // state's frame
    const int pscale = (hh ? x1i : x0i) - st.mo + 127;

    // ---- step 3: l_t as an MFMA of the quantised P itself (state's frame)
    const float ell = rowsum4(ones, pb, pscale);
    // this tile's scores are consumed: the next tile's go to the matrix cores
    // behind the row sum and run during the vote and the P V product
    __builtin_amdgcn_sched_barrier(0);
    qk_all<D>(acc, kn, c);
    const uint32_t vblob = kblob;
    kblob = next_blob(i + 2);
    load_k<D>(kn, c.blobs, kblob, c.koff, c.ksoff, hh);

    // ---- step 4: the hot test (lambda includes this tile); a row's scalars
    // are the same in both lane halves, so the low 32 ballot bits are the rows
    st.lam += ell;
    if (!TAIL && pub_out && i >= kReplay) pub_out[n] = ldexpf(st.lam, st.mo - mo_ref);
    float lam_t = st.lam;  // the running mass the vote compares against
    if (TAIL) lam_t = (pub_in && !replay ? vmax(lam_lo, pub_in[n]) : lam_lo) + st.lam;
    const unsigned long long hb = __ballot(ell * wt > epsv * lam_t);
    bool hot0 = vis0 && (hb & 0xFFFFull) != 0ull;
    bool hot1 = vis1 && (hb & 0xFFFF0000ull) != 0ull;
    if (tail && !replay && eps != 0.0f && (hot0 || hot1)) {
      // undecided under the lower bound: record it and treat it as cold for
      // now
      if (ncand == cap) {
        gave_up = true;
      } else {
        if (lane == 0)
          __builtin_amdgcn_raw_buffer_store_b32(
              (uint32_t)t | (hot0 ? 1u << 30 : 0u) | (hot1 ? 1u << 31 : 0u), cr.r, 0u,
              cr.tile + 4u * ncand, 0);
        if (hh == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ell), cr.r, 4u * n,
                                                cr.ell + 128u * ncand, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(st.lam), cr.r, 4u * n,
                                                cr.lamb + 128u * ncand, 0);
          __builtin_amdgcn_raw_buffer_store_b8((uint8_t)((int)mcf - st.mo), cr.r, (uint32_t)n,
                                               cr.dm + 32u * ncand, 0);
        }
        ++ncand;
      }
      hot0 = hot1 = false;
    }
    // ---- frame update: cold -> mc; hot -> max(m, mc - H), which is m unless
    // the lazy test fired
    if (hot0 || hot1) {
      const unsigned long long hot_lanes = (hot0 ? kGroup0 : 0ull) | (hot1 ? ~kGroup0 : 0ull);
      const bool my_hot = __builtin_amdgcn_inverse_ballot_w64(hot_lanes);
      st.mf = my_hot ? vmax(st.mf, mcf - Hf) : mcf;
    } else {
      st.mf = mcf;
    }

    // ---- step 5: cold tiles accumulate P V in FP4 (not while replaying).  A
    // group that does not see this tile has all scores masked, so its P and
    // l_t are exact zeros: only a hot group's rows need taking out.
    if (!replay && !(hot0 && hot1)) {
      v4i pz = pb;
      float ez = ell;
      if (hot0 || hot1) {
        const bool keep = __builtin_amdgcn_inverse_ballot_w64(hot0 ? ~kGroup0 : kGroup0);
        pz = keep ? pb : v4i{0, 0, 0, 0};
        ez = keep ? ell : 0.0f;
      }
#pragma unroll
      for (int db = 0; db < ND; ++db)
        st.o[db] = mfma4(va[db], pz, st.o[db], (int)vsw[db >> 2], db & 3, pscale);
      st.lsum += ez;
    }
    load_v(vblob);

    // ---- hot bits: one log byte per tile, or whole words (visited in
    // descending order after tile 0)
    if (LOG) {
      if (!replay && lane == 0) vlog[t] = (uint8_t)((hot0 ? 1 : 0) | (hot1 ? 2 : 0));
    } else if (!replay) {
      const int w = t >> 5;
      if (w != cur_w) {
        if (cur_w >= 0) put_word(c, wd, cur_w, cur_b0, cur_b1, lane);
        cur_w = w;
        cur_b0 = cur_b1 = 0u;
      }
      if (hot0) cur_b0 |= 1u << (t & 31);
      if (hot1) cur_b1 |= 1u << (t & 31);
    }
  }
  if (LOG) {
    assemble_words<D>(c, wd, vlog, p0, cnt - nrep, lane);
  } else if (cur_w >= 0) {
    put_word(c, wd, cur_w, cur_b0, cur_b1, lane);
  }
  return gave_up ? -1 : ncand;
}

// The cold state's outputs in the method's frame m = mf (o * 2^(mo - m) * g_v,
// with the power of two folded into g_v: exact).
template <int D>
__device__ __forceinline__ void store_state(const Geom& g, const CtxBase<D>& c, const Pass1Out& out,
                                            const St<D>& st, int lane) {
  if (!c.row_ok) return;
  const int hh = lane >> 5;
  const size_t r = c.bhq * g.Nq + c.row;
  const int m = (int)st.mf;
  const int sh = st.mo - m;
  if (hh == 0 && c.lead) {
    out.m[r] = m;
    out.l[r] = ldexpf(st.lsum, sh);
    if (out.lam) out.lam[r] = ldexpf(st.lam, sh);
  }
  const float gs = ldexpf(c.g_v, sh);
  float* orow = out.o + r * D + c.dh * Tile<D>::NDO * 32;
#pragma unroll
  for (int db = 0; db < Tile<D>::NDO; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v4f x = {st.o[db][4 * q] * gs, st.o[db][4 * q + 1] * gs, st.o[db][4 * q + 2] * gs,
               st.o[db][4 * q + 3] * gs};
      *reinterpret_cast<v4f*>(orow + db * 32 + 8 * q + 4 * hh) = x;
    }
}

// zero the hot words the walk does not write: those above each group's
// diagonal word, and, with a window, those between word 0 (always written as
// a partial word) and the word of the walk's first tile
template <int D>
__device__ __forceinline__ void zero_outside(const Geom& g, const CtxBase<D>& c, int lane) {
  if (!c.lead) return;
  for (int w = c.d0 / 32 + 1 + lane; w < g.W; w += 64) c.bits0[w] = 0u;
  if (c.has_g1)
    for (int w = c.d1 / 32 + 1 + lane; w < g.W; w += 64) c.bits1[w] = 0u;
  for (int w = 1 + lane; w < c.lo0 / 32; w += 64) {
    c.bits0[w] = 0u;
    if (c.has_g1) c.bits1[w] = 0u;
  }
}

// The tail's end of a split unit, once the head's final state is in LDS:
// decide the recorded groups against the head's lambda, take the P V of those
// that are hot after all back out of the tail's state (the same FP4 codes with
// their sign bits set, so exactly what was added), and set their bits.
template <int D, bool VW, int QT>
__device__ __forceinline__ void settle(const Geom& g, const Ctx<D, QT>& c, St<D>& st, Words& tw,
                                       const Cand& cr, int ncand, float lam_a, float eps,
                                       int lane) {
  constexpr int ND = Tile<D>::NDO;
  constexpr int NW = Tile<D>::NWO;
  constexpr int BLOB = Tile<D>::BLOB;
  constexpr unsigned long long kGroup0 = 0x0000FFFF0000FFFFull;
  const int n = lane & 31, hh = lane >> 5;
  constexpr int kBatch = 4;  // records decided per round of loads
  for (int j0 = 0; j0 < ncand; j0 += kBatch) {
    float e[kBatch], lbv[kBatch];
    uint32_t hd[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const uint32_t j = (uint32_t)min(j0 + k, ncand - 1);
      hd[k] = __builtin_amdgcn_raw_buffer_load_b32(cr.r, 0u, cr.tile + 4u * j, 0);
      e[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(cr.r, 4u * n, cr.ell + 128u * j, 0));
      lbv[k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(cr.r, 4u * n, cr.lamb + 128u * j, 0));
    }
    uint32_t found = 0;  // 2 bits per record: groups hot after all
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const uint32_t hdr = (uint32_t)__builtin_amdgcn_readfirstlane((int)hd[k]);
      const float wk = VW ? c.tw[hdr & 0x3FFFFFFFu] : 1.0f;
      const unsigned long long hb = __ballot(e[k] * wk > eps * (lam_a + lbv[k]) && hh == 0);
      const uint32_t gr = ((hdr >> 30 & 1u) && (hb & 0xFFFFull) != 0ull ? 1u : 0u) |
                          ((hdr >> 31) && (hb & 0xFFFF0000ull) != 0ull ? 2u : 0u);
      if (j0 + k < ncand) found |= gr << (2 * k);
    }
    found = (uint32_t)__builtin_amdgcn_readfirstlane((int)found);
    while (found) {
      const int kr = __builtin_ctz(found) >> 1;
      const uint32_t gr = (found >> (2 * kr)) & 3u;
      found &= ~(3u << (2 * kr));
      const uint32_t j = (uint32_t)(j0 + kr);
      const uint32_t hdr = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)__builtin_amdgcn_raw_buffer_load_b32(cr.r, 0u, cr.tile + 4u * j, 0));
      const int t = (int)(hdr & 0x3FFFFFFFu);
      const float ell =
          __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(cr.r, 4u * n, cr.ell + 128u * j, 0));
      const float mcf = (float)(st.mo + (int)__builtin_amdgcn_raw_buffer_load_b8(
                                            cr.r, (uint32_t)n, cr.dm + 32u * j, 0));
      const bool f0 = gr & 1u, f1 = gr & 2u;
      KOps<D> k;
      v16f acc[2];
      const uint32_t blob = (uint32_t)(t * BLOB);
      load_k<D>(k, c.blobs, blob, c.koff, c.ksoff, hh);
      qk_all<D>(acc, k, c);
      mask_scores<D>(acc, g, c, t, hh);
      float b0, b1;
      group_maxima(acc, b0, b1);
      const float lo = mcf - 127.0f;
      const float x0 = vmax(ceilf(b0 - kLog2_6), lo);
      const float x1 = vmax(ceilf(b1 - kLog2_6), lo);
      const int x0i = (int)x0, x1i = (int)x1;
      const v4i pb = p_operand(acc, x0i, x1i, x0, x1, divisors_fast(x0i, x1i));
      const int pscale = (hh ? x1i : x0i) - st.mo + 127;
      const unsigned long long hot_lanes = (f0 ? kGroup0 : 0ull) | (f1 ? ~kGroup0 : 0ull);
      const bool keep = __builtin_amdgcn_inverse_ballot_w64(hot_lanes);
      const int neg = (int)0x88888888u;
      const v4i pz = keep ? (pb ^ v4i{neg, neg, neg, neg}) : v4i{0, 0, 0, 0};
      v4i va[ND];
      uint32_t vsw[NW];
#pragma unroll
      for (int db = 0; db < ND; ++db) va[db] = bload128(c.blobs, c.voff + db * 32 * 32, blob);
      load_scales<ND>(vsw, c.blobs, c.vsoff, blob);
#pragma unroll
      for (int db = 0; db < ND; ++db)
        st.o[db] = mfma4(va[db], pz, st.o[db], (int)vsw[db >> 2], db & 3, pscale);
      st.lsum = keep ? st.lsum - ell : st.lsum;
      const int w = t >> 5;
      const uint32_t bit = 1u << (t & 31);
      if (w == 0) {
        if (f0) tw.p00 |= bit;
        if (f1) tw.p01 |= bit;
      } else if (w == tw.wb) {
        if (f0) tw.p10 |= bit;
        if (f1) tw.p11 |= bit;
      } else if (lane == 0) {
        if (f0) c.bits0[w] |= bit;
        if (f1) c.bits1[w] |= bit;
      }
    }
  }
}

// A wave's state in the hand-off area of a unit's workspace block (after its
// records): o in lane order (float4 chunk q of block db at [4 db + q]), then
// mf, mo (its bits), lambda and l per lane, then the four partial hot words
// (word k from lane k).  The tail of the triple schedule parks its state
// there while it walks the next unit's tail; a tail that gave up leaves its
// head's state there for the re-walk.  Each lane reads back only
// what it wrote.
template <int D>
__device__ __forceinline__ float* handoff_of(uint8_t* split, int unit, int cap) {
  return reinterpret_cast<float*>(split + (size_t)unit * cand_stride(cap, D) + cand_bytes(cap));
}

template <int D>
__device__ __forceinline__ void save_state(float* dst, const St<D>& st, const Words& wd, int lane) {
#pragma unroll
  for (int db = 0; db < Tile<D>::NDO; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      reinterpret_cast<v4f*>(dst)[(4 * db + q) * 64 + lane] =
          v4f{st.o[db][4 * q], st.o[db][4 * q + 1], st.o[db][4 * q + 2], st.o[db][4 * q + 3]};
  dst[32 * D + lane] = st.mf;
  dst[32 * D + 64 + lane] = __int_as_float(st.mo);
  dst[32 * D + 128 + lane] = st.lam;
  dst[32 * D + 192 + lane] = st.lsum;
  const uint32_t w = lane == 0 ? wd.p00 : lane == 1 ? wd.p01 : lane == 2 ? wd.p10 : wd.p11;
  if (lane < 4) reinterpret_cast<uint32_t*>(dst)[32 * D + 256 + lane] = w;
}

template <int D>
__device__ __forceinline__ void load_state(const float* src, St<D>& st, Words& wd, int lane) {
#pragma unroll
  for (int db = 0; db < Tile<D>::NDO; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f x = reinterpret_cast<const v4f*>(src)[(4 * db + q) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) st.o[db][4 * q + e] = x[e];
    }
  st.mf = src[32 * D + lane];
  st.mo = __float_as_int(src[32 * D + 64 + lane]);
  st.lam = src[32 * D + 128 + lane];
  st.lsum = src[32 * D + 192 + lane];
  const int w = lane < 4 ? (int)reinterpret_cast<const uint32_t*>(src)[32 * D + 256 + lane] : 0;
  wd.p00 = (uint32_t)__builtin_amdgcn_readlane(w, 0);
  wd.p01 = (uint32_t)__builtin_amdgcn_readlane(w, 1);
  wd.p10 = (uint32_t)__builtin_amdgcn_readlane(w, 2);
  wd.p11 = (uint32_t)__builtin_amdgcn_readlane(w, 3);
}

// A work group's LDS in pass 1: per head slot its running lambda and final
// state, the waves' verdict logs and their position counts (for the SIMD
// partner).
template <int D, bool LOG>
struct P1Lds {
  float pub[kSlots<D>][32];
  HeadState<D> hs[kSlots<D>];
  uint8_t vlog[LOG ? kP1Waves<D> : 1][LOG ? kLogTiles : 1];
  int pace[kP1Waves<D>];
};

// Units run one wave each, or, with a split workspace, as a head and a tail
// walk (see split_cut).  With the pair schedule a work group holds two units,
// its waves numbered (unit, role); with the triple schedule it holds three,
// waves 0-2 their heads and wave 3 the tail of each, one after the other.  A
// head hands its running lambda to its tail through LDS while both walk, and
// its final state at its end; the tail finishes the unit.  Units are numbered
// (batch, kv-head, 32-row block, head), so the waves of a work group, and the
// groups of an XCD, stream the same tiles.
// (block blk of the launch: its units start at blk times the units per group)
template <int D, bool LOG, int QT, bool VW>
__device__ __forceinline__ void pass1_block(const Geom& g, const Fp4Ptrs& f, float eps, float tau,
                                            int hoff, const Pass1Out& out, uint8_t* split,
                                            int cap, int sched, int nunits, int blk,
                                            P1Lds<D, LOG>& L) {
  constexpr int ND = Tile<D>::NDO;
  constexpr int NS = kSlots<D>;
  constexpr int W = kP1Waves<D>;
  auto& pub = L.pub;
  auto& hs = L.hs;
  auto& vlog_sh = L.vlog;
  auto& pace = L.pace;
  const int lane = threadIdx.x & 63;
  const int hh = lane >> 5;
  // the wave index is wave-uniform: keep everything derived from it in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (wave == 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (lane < 32) pub[s][lane] = 0.0f;
      if (lane == 0) hs[s].done = 0;
    }
    if (lane < W) pace[lane] = 0;
  }
  __syncthreads();
  if (sched == kSchedTriples && NS < 3) return;  // never launched so (too little LDS)
  if (kOutSplit<D> > 1 && sched != kSchedWhole) return;  // never launched so
  // the wave's role, its (first) unit, the number of units it walks and the
  // LDS slot of the first
  int role, u0, nu = 1, slot, dh = 0;
  if (sched == kSchedTriples) {
    // per four waves: three heads and the wave that walks their tails
    const int grp = wave >> 2, wq = wave & 3;
    role = wq < 3 ? kHead : kTail;
    slot = grp * 3 + (wq < 3 ? wq : 0);
    u0 = blk * (3 * W / 4) + slot;
    if (wq == 3) nu = min(3, nunits - u0);
  } else if (sched == kSchedPairs) {
    role = (wave & 1) ? kTail : kHead;
    slot = wave >> 1;
    u0 = blk * (W / 2) + slot;
  } else {
    // (at D = 512 two consecutive waves per unit, one per half of the output)
    role = kWhole;
    slot = 0;
    u0 = (blk * W + wave) / kOutSplit<D>;
    dh = (blk * W + wave) % kOutSplit<D>;
  }
  if (u0 >= nunits) return;
  lds_u8* vlog = (lds_u8*)vlog_sh[LOG ? wave : 0];
  const float Hf = (float)hoff;
  // the partner on this wave's SIMD (waves w and w + 4 of a group of eight)
  volatile lds_int* pace_me = W == 8 ? (volatile lds_int*)&pace[wave] : nullptr;
  const volatile lds_int* pace_mate = W == 8 ? (const volatile lds_int*)&pace[wave ^ 4] : nullptr;

  if (role != kTail) {
    Ctx<D, QT> c;
    make_ctx<D>(c, g, f, out, unit_id(g, u0), lane, dh);
    load_q2<D>(c, g, f, lane);
    const int npos = c.npos();
    const int h = split_cut(npos, sched);  // head positions [0, h), tail [h, npos)
    if (h >= npos) role = kWhole;  // nothing to cut: its tail wave skips it
    St<D> st;
    init_state<D>(st, c.row_ok);
    Words wd = {role == kWhole ? -1 : shared_word(c.tile_of(h)), 0u, 0u, 0u, 0u};
    zero_outside<D>(g, c, lane);
    walk<D, LOG, false, VW>(g, c, st, wd, 0, 0, role == kWhole ? npos : h, eps, tau, Hf,
                        cand_of(f.kv_blob, 0, 0, D), 0, nullptr,
                        role == kHead ? (volatile lds_float*)pub[slot] : nullptr, vlog, lane,
                        pace_me, pace_mate, 0);
    if (kOutSplit<D> == 1 && role == kHead) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          hs[slot].o[4 * db + q][lane] = v4f{st.o[db][4 * q], st.o[db][4 * q + 1],
                                             st.o[db][4 * q + 2], st.o[db][4 * q + 3]};
      hs[slot].sc[0][lane] = st.mf;
      hs[slot].sc[1][lane] = __int_as_float(st.mo);
      hs[slot].sc[2][lane] = st.lam;
      hs[slot].sc[3][lane] = st.lsum;
      if (lane == 0) {
        hs[slot].words[0] = wd.p00;
        hs[slot].words[1] = wd.p01;
        hs[slot].words[2] = wd.p10;
        hs[slot].words[3] = wd.p11;
        __hip_atomic_store(&hs[slot].done, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      return;
    }
    // a whole unit: word 0 (which also holds tile 0) and the state
    if (lane == 0 && c.lead) {
      c.bits0[0] = wd.p00;
      if (c.has_g1) c.bits1[0] = wd.p01;
    }
    store_state<D>(g, c, out, st, lane);
    return;
  }

  // A tail wave: walk the tails of units u0 .. u0 + nu - 1 (one loop, so one
  // inlined copy of the walk), keeping each outcome (records kept; -1 gave
  // up; -2 no tail: a short visit order its head wave walked whole).  Each
  // walked state waits in its unit's hand-off area until the heads are done,
  // so no state lives across the loops.
  if constexpr (kOutSplit<D> == 1) {
  uint32_t outcomes = 0u;  // outcome + 2 in 10 bits per unit
  int walked = 0;          // positions walked so far (pacing)
#pragma nounroll
  for (int k = 0; k < nu; ++k) {
    const int u = u0 + k;
    Ctx<D, QT> c;
    make_ctx<D>(c, g, f, out, unit_id(g, u), lane);
    load_q2<D>(c, g, f, lane);
    const int npos = c.npos();
    const int h = split_cut(npos, sched);
    int oc = -2;
    if (h < npos) {
      St<D> st;
      init_state<D>(st, c.row_ok);
      Words wd = {shared_word(c.tile_of(h)), 0u, 0u, 0u, 0u};
      oc = walk<D, LOG, true, VW>(g, c, st, wd, kReplay, h, kReplay + npos - h, eps, tau, Hf,
                              cand_of(split, u, cap, D), cap,
                              (volatile lds_float*)pub[slot + k], nullptr, vlog, lane, pace_me,
                              pace_mate, walked);
      walked += kReplay + npos - h;
      if (oc >= 0) save_state<D>(handoff_of<D>(split, u, cap), st, wd, lane);
    }
    outcomes |= (uint32_t)(oc + 2) << (10 * k);
  }
  // Finish each unit once its head is done, the last walked first.
  __builtin_amdgcn_s_setprio(0);
#pragma nounroll
  for (int k = nu - 1; k >= 0; --k) {
    const int oc = (int)((outcomes >> (10 * k)) & 1023u) - 2;
    if (oc == -2) continue;
    const int u = u0 + k;
    Ctx<D, QT> c;
    make_ctx<D>(c, g, f, out, unit_id(g, u), lane);
    load_q2<D>(c, g, f, lane);
    const int wb = shared_word(c.tile_of(split_cut(c.npos(), sched)));
    float* ho = handoff_of<D>(split, u, cap);
    HeadState<D>& H = hs[slot + k];
    while (__hip_atomic_load(&H.done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) == 0)
      __builtin_amdgcn_s_sleep(2);
    const Cand cr = cand_of(split, u, cap, D);
    if (lane == 0) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)oc, cr.r, 0u, 0u, 0);
    if (oc < 0) {
      // gave up: leave the head's state for the re-walk
#pragma unroll 2
      for (int q = 0; q < ND * 4; ++q) reinterpret_cast<v4f*>(ho)[q * 64 + lane] = H.o[q][lane];
#pragma unroll
      for (int q = 0; q < 4; ++q) ho[32 * D + 64 * q + lane] = H.sc[q][lane];
      if (lane < 4) reinterpret_cast<uint32_t*>(ho)[32 * D + 256 + lane] = H.words[lane];
      continue;
    }
    St<D> st;
    Words wd;
    load_state<D>(ho, st, wd, lane);
    wd.wb = wb;
    const float a_mf = H.sc[0][lane];
    const int a_mo = __float_as_int(H.sc[1][lane]);
    const float a_lam = H.sc[2][lane];
    const float a_lsum = H.sc[3][lane];
    // the head's lambda in the tail's state frame (the tail never re-based)
    settle<D, VW>(g, c, st, wd, cr, oc, ldexpf(a_lam, a_mo - st.mo), eps, lane);
    // the shared words: the head's part and the tail's
    if (lane == 0) {
      c.bits0[0] = H.words[0] | wd.p00;
      if (c.has_g1) c.bits1[0] = H.words[1] | wd.p01;
      if (wb > 0) {
        c.bits0[wb] = H.words[2] | wd.p10;
        if (c.has_g1) c.bits1[wb] = H.words[3] | wd.p11;
      }
    }
    // merge: the larger frame, each state scaled into it by an exact power of two
    if (!c.row_ok) continue;
    const size_t r = c.bhq * g.Nq + c.row;
    const int m = (int)vmax(a_mf, st.mf);
    const int sa = a_mo - m, sb = st.mo - m;
    if (hh == 0) {
      out.m[r] = m;
      out.l[r] = ldexpf(a_lsum, sa) + ldexpf(st.lsum, sb);
      if (out.lam) out.lam[r] = ldexpf(a_lam, sa) + ldexpf(st.lam, sb);
    }
    float* orow = out.o + r * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f xa = H.o[4 * db + q][lane];
        v4f x;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = (ldexpf(xa[e], sa) + ldexpf(st.o[db][4 * q + e], sb)) * c.g_v;
        *reinterpret_cast<v4f*>(orow + db * 32 + 8 * q + 4 * hh) = x;
      }
  }
  }
}

// The re-walk of units whose tail gave up (record full, or a re-base of its
// frame): the head's state, left in the workspace, walks the tail positions.
// One wave per unit: nothing to do unless its tail gave up.
template <int D, bool LOG, int QT, bool VW>
__device__ __forceinline__ void rewalk_unit(const Geom& g, const Fp4Ptrs& f, float eps, float tau,
                                            int hoff, const Pass1Out& out, uint8_t* split,
                                            int cap, int sched, int unit, lds_u8* vlog) {
  constexpr int ND = Tile<D>::ND;
  const int lane = threadIdx.x & 63;
  const UnitId id = unit_id(g, unit);
  const uint8_t* base = split + (size_t)unit * cand_stride(cap, D);
  Ctx<D, QT> c;
  make_ctx<D>(c, g, f, out, id, lane);
  load_q2<D>(c, g, f, lane);
  const int npos = c.npos();
  const int h = split_cut(npos, sched);
  if (h >= npos) return;
  if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(base)) >= 0) return;
  const int wb = shared_word(c.tile_of(h));
  const float* src = reinterpret_cast<const float*>(base + cand_bytes(cap));
  St<D> st;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const v4f x = reinterpret_cast<const v4f*>(src)[(4 * db + q) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) st.o[db][4 * q + e] = x[e];
    }
  st.mf = src[32 * D + lane];
  st.mo = __float_as_int(src[32 * D + 64 + lane]);
  st.lam = src[32 * D + 128 + lane];
  st.lsum = src[32 * D + 192 + lane];
  const uint32_t* hw = reinterpret_cast<const uint32_t*>(src + 32 * D + 256);
  Words wd = {wb, 0u, 0u, 0u, 0u};
  const Cand none = cand_of(f.kv_blob, 0, 0, D);
  walk<D, LOG, false, VW>(g, c, st, wd, 0, h, npos - h, eps, tau, (float)hoff, none, 0, nullptr,
                      nullptr, vlog, lane);
  if (lane == 0) {
    c.bits0[0] = hw[0] | wd.p00;
    if (c.has_g1) c.bits1[0] = hw[1] | wd.p01;
    if (wb > 0) {
      c.bits0[wb] = hw[2] | wd.p10;
      if (c.has_g1) c.bits1[wb] = hw[3] | wd.p11;
    }
  }
  store_state<D>(g, c, out, st, lane);
}


// The schedule a launch with a workspace runs: the caller's, else two waves
// per unit while those fit the GPU's wave slots at once, four waves per three
// units while those do, else one wave per unit (then there is no workspace).
// Visit orders shorter than kMinSplit positions leave nothing to cut, the
// triple schedule needs three head states in LDS (D <= 256), and at D = 512
// every unit already runs as two waves (one per half of the output channels).
// Longest tail any visit order of at most NT positions gets under a schedule
// (0: no order is cut).
inline int longest_tail(int NT, int sched) {
  int m = 0;
  for (int n = kMinSplit; n <= NT; ++n) m = max(m, n - split_cut(n, sched));
  return m;
}

inline int pass1_sched(const Geom& g) {
  const long units = (long)g.B * g.Hkv * (g.NqP / 32) * g.G;
  const long slots = 1024L * (g.D >= 256 ? 1 : 2);
  if (units == 0 || g.NT < kMinSplit || g.D >= 512) return kSchedWhole;
  int s = g.sched;
  if (s != kSchedWhole && s != kSchedPairs && s != kSchedTriples)
    s = 2 * units <= slots ? kSchedPairs : (4 * units <= 3 * slots ? kSchedTriples : kSchedWhole);
  // a schedule under which no visit order of this problem is cut is the whole one
  if (s != kSchedWhole && longest_tail(g.NT, s) == 0) s = kSchedWhole;
  return s;
}

// Records per unit: every position of the longest tail, at most kCandCap (a
// tail with more undecided tiles gives up and is walked again).
inline int cand_cap(const Geom& g, int sched) { return min(kCandCap, longest_tail(g.NT, sched)); }

}  // namespace
}  // namespace apa
