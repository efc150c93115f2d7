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
//   l_t     : one FP4 MFMA of P against an all-ones operand (numerator and
//             denominator carry the same quantisation);
//   vote    : row hot iff l_t > eps * lambda (lambda includes this tile),
//             ballot over 16 rows;
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
// defined without a clearing pass.
#include "apa_device.h"
#include "apa_kernels.h"

namespace apa {

namespace {

constexpr int kWaves = 4;            // wavefronts per work group
constexpr float kFrameGuard = 80.0f; // largest lead of m over m_o before re-basing

// Two waves per SIMD up to D = 128; one above, where the output accumulators
// (D/2 per lane) need the accumulation registers.
template <int D>
constexpr int kWavesPerSimd = D >= 256 ? 1 : 2;

template <int D>
struct Tile {
  static constexpr int NH = D / 64;       // 64-channel halves of the QK contraction
  static constexpr int ND = D / 32;       // 32-channel blocks of the output
  static constexpr int NW = (D / 32 + 3) / 4;  // 32-bit words of one key's scale bytes
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

// The scale bytes of one key (or one V lane) as little-endian words.
template <int D>
__device__ __forceinline__ void load_scales(uint32_t (&w)[Tile<D>::NW], const uint8_t* p) {
  if constexpr (D == 64) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (D == 128) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (D == 256) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x;
    w[1] = x.y;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    w[0] = x.x;
    w[1] = x.y;
    w[2] = x.z;
    w[3] = x.w;
  }
}

template <int D>
struct KOps {
  v4i a[2][Tile<D>::NH];
  uint32_t s[2][Tile<D>::NW];  // shifted so byte 2*(h%2) of word h/2 is block 2h + hh
};

template <int D>
__device__ __forceinline__ void load_k(KOps<D>& k, const uint8_t* blob, uint32_t koff,
                                       uint32_t ksoff, int hh) {
  constexpr int NH = Tile<D>::NH;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
      k.a[kb][h] = *reinterpret_cast<const v4i*>(blob + koff + kb * 32 * (D / 2) + 32 * h);
    load_scales<D>(k.s[kb], blob + ksoff + kb * 32 * (D / 32));
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

template <int D>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>))) void k_pass1(
    Geom g, Fp4Ptrs f, float eps, float tau, int hoff, Pass1Out out, int nunits) {
  constexpr int NH = Tile<D>::NH;
  constexpr int ND = Tile<D>::ND;
  constexpr int NW = Tile<D>::NW;
  constexpr int BLOB = Tile<D>::BLOB;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;       // the wave's row handled by this lane
  const int hh = lane >> 5;      // which half of the K dimension this lane feeds
  // the wave index is wave-uniform: keep everything derived from it in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int unit = xcd_remap(blockIdx.x, gridDim.x) * kWaves + wave;
  if (unit >= nunits) return;

  // unit -> (b, kv-head, 32-row block, head in group), heads innermost
  const int nq32 = g.NqP / 32;
  int u = unit;
  const int gi = u % g.G; u /= g.G;
  const int qb = u % nq32; u /= nq32;
  const int hk = u % g.Hkv; u /= g.Hkv;
  const int b = u;
  const int hq = hk * g.G + gi;
  const size_t bhq = (size_t)b * g.Hq + hq, bhk = (size_t)b * g.Hkv + hk;
  const int r0 = qb * 32;
  const int row = r0 + n;
  const bool row_ok = row < g.Nq;
  auto diag = [&](int lr) { return g.causal ? min(g.Nkv - 1, lr + g.off) / kTile : g.NT - 1; };
  const bool has_g1 = r0 + 16 < g.Nq;
  const int d0 = diag(min(r0 + 15, g.Nq - 1));
  const int d1 = has_g1 ? diag(min(r0 + 31, g.Nq - 1)) : -1;
  const int dW = max(d0, d1);
  // lanes of verdict group 0 (rows r0 .. r0+15) in both lane halves
  constexpr unsigned long long kGroup0 = 0x0000FFFF0000FFFFull;

  // Q^T operand (resident): 16 bytes per 64-channel half, E8M0 byte + j
  v4i qa[NH];
  int qs[NH];
  {
    const int jq = (int)f.q_head[bhq * 4 + 2];
    const uint8_t* qc = f.q_codes + (bhq * g.NqP + row) * (D / 2);
    const uint8_t* qsc = f.q_scales + (bhq * g.NqP + row) * (D / 32);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      qa[h] = *reinterpret_cast<const v4i*>(qc + 32 * h + 16 * hh);
      const int sb = (int)qsc[2 * h + hh] + jq;
      qs[h] = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
    }
  }
  const float g_v = f.kv_head[bhk * 8 + 4];
  const uint8_t* blobs = f.kv_blob + bhk * (size_t)g.NT * BLOB;
  // this lane's byte offsets inside a blob
  const uint32_t koff = n * (D / 2) + 16 * hh;
  const uint32_t ksoff = 32 * D + n * (D / 32);
  const uint32_t voff = 34 * D + n * 32 + 16 * hh;
  const uint32_t vsoff = 66 * D + (2 * n + hh) * ND;

  // frames: mf is the method's (an integer; -inf before the first key), mo the
  // state's.  Rows past Nq never see a key and sit at frame 127 so every
  // derived quantity stays finite; mo starts far below any frame so that the
  // first tile re-bases.
  float mf = row_ok ? -__builtin_inff() : 127.0f;
  int mo = -(1 << 20);
  float lam = 0.0f, lsum = 0.0f;
  v16f o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = v16f{};
  const float Hf = (float)hoff;

  // hot-bit words: zero the words above each group's diagonal word first
  uint32_t* bits0 = out.bits + (bhq * g.NG + (r0 >> 4)) * g.W;
  uint32_t* bits1 = bits0 + g.W;
  for (int w = d0 / 32 + 1 + lane; w < g.W; w += 64) bits0[w] = 0u;
  if (has_g1)
    for (int w = d1 / 32 + 1 + lane; w < g.W; w += 64) bits1[w] = 0u;
  uint32_t tile0_b0 = 0, tile0_b1 = 0, cur_b0 = 0, cur_b1 = 0;
  int cur_w = -1;

  const int ntiles = dW + 1;
  auto tile_of = [&](int it) { return it == 0 ? 0 : dW - it + 1; };

  // pipeline: when tile it starts, its scores are in acc and the K operand of
  // tile it+1 in kn; once this tile's P is formed, QK(it+1) is issued into acc
  // and K of tile it+2 is fetched into kn (prefetches past the last tile
  // re-read the last tile: in bounds, unused)
  auto next_blob = [&](int it) { return blobs + (size_t)tile_of(min(it, ntiles - 1)) * BLOB; };
  KOps<D> kn;
  v16f acc[2];
  load_k<D>(kn, blobs, koff, ksoff, hh);
  qk<D>(acc, kn, qa, qs);
  load_k<D>(kn, next_blob(1), koff, ksoff, hh);

  for (int it = 0; it < ntiles; ++it) {
    const int t = tile_of(it);
    const uint8_t* blob = blobs + (size_t)t * BLOB;
    // V^T operand and scales of this tile (used at its end)
    v4i va[ND];
    uint32_t vsw[NW];
#pragma unroll
    for (int db = 0; db < ND; ++db)
      va[db] = *reinterpret_cast<const v4i*>(blob + voff + db * 32 * 32);
    load_scales<D>(vsw, blob + vsoff);

    const int k0 = t * kTile;
    const bool vis0 = t <= d0, vis1 = t <= d1;
    // masking: causal diagonal, padding keys, rows past Nq (wave-uniform test)
    if ((k0 + kTile > g.Nkv) || (g.causal && k0 + kTile - 1 > r0 + g.off) || (r0 + 31 >= g.Nq)) {
      const int lim = g.causal ? row + g.off : 0x7fffffff;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (!(row_ok && key < g.Nkv && key <= lim)) acc[kb][j] = -__builtin_inff();
        }
    }
    // group maxima: gown of this lane's block hh, goth of the other block
    float gl0 = vmax(acc[0][0], acc[0][1]), gl1 = vmax(acc[1][0], acc[1][1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) {
      gl0 = vmax3(gl0, acc[0][j], acc[0][j + 1]);
      gl1 = vmax3(gl1, acc[1][j], acc[1][j + 1]);
    }
    int x0, x1;
    swap_halves(__float_as_int(gl0), __float_as_int(gl1), x0, x1);
    const float gown = vmax(__int_as_float(x0), __int_as_float(x1));
    const float goth = xor32(gown);
    const float c = vmax(gown, goth);

    // ---- lazy maximum (integer frame)
    const bool fire = c > mf + tau;     // never for a row without a visible key here
    const float mcf = fire ? ceilf(c) : mf;

    // re-base the state to m_o = max(m, mc - H), a lower bound of every later
    // frame, when the frame has run too far ahead (all lanes; exact powers of two)
    if (__ballot(mcf - (float)mo > kFrameGuard) != 0ull) {
      const int mo_new = (int)vmax(mf, mcf - Hf);
      const int sh = mo - mo_new;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] = ldexpf(o[db][j], sh);
      lsum = ldexpf(lsum, sh);
      lam = ldexpf(lam, sh);
      mo = mo_new;
    }

    // ---- step 2: the conversion divisor 2^X of each 32-key group,
    // X = E + m = max(ceil(c_g - log2 6), m - 127)
    const float lo = mcf - 127.0f;
    const float xof = vmax(ceilf(gown - kLog2_6), lo);
    const float xtf = vmax(ceilf(goth - kLog2_6), lo);
    const int xo = (int)xof, xt = (int)xtf;
    // fast path: both divisors normal with room below for the codes that matter
    const bool odd = (unsigned)(xo + 124) > 244u || (unsigned)(xt + 124) > 244u;
    unsigned pk[2][2];
    if (__ballot(odd) == 0ull) {
      const float so = __int_as_float((xo + 127) << 23), st = __int_as_float((xt + 127) << 23);
      const float sc0 = hh ? st : so, sc1 = hh ? so : st;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float sc = kb ? sc1 : sc0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          unsigned w = 0;
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
        const float sub = (kb == hh) ? xof : xtf;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          unsigned w = 0;
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int i = 8 * j + 2 * p;
            w = cvt_fp4x2(w, fast_exp2(acc[kb][i] - sub), fast_exp2(acc[kb][i + 1] - sub), 1.0f, p);
          }
          pk[kb][j] = w;
        }
      }
    }
    // operand layout: lanes < 32 carry keys 0-31, lanes >= 32 keys 32-63
    v4i pb;
    {
      int a0, b0, a1, b1;
      swap_halves((int)pk[0][0], (int)pk[1][0], a0, b0);
      swap_halves((int)pk[0][1], (int)pk[1][1], a1, b1);
      pb = v4i{a0, a1, b0, b1};
    }
    // E8M0 byte of this lane's 32-key group in the state's frame
    const int pscale = xo - mo + 127;

    // ---- step 3: l_t as an MFMA of the quantised P itself (state's frame)
    const v4i ones = {kE2M1Ones, kE2M1Ones, kE2M1Ones, kE2M1Ones};
    const v16f ones_acc = mfma4(ones, pb, v16f{}, kE8M0One, 0, pscale);
    // this tile's scores are consumed: the next tile's go to the matrix cores
    // behind the row sum and run during the vote and the P V product
    __builtin_amdgcn_sched_barrier(0);
    qk<D>(acc, kn, qa, qs);
    load_k<D>(kn, next_blob(it + 2), koff, ksoff, hh);
    const float ell = ones_acc[0];

    // ---- step 4: the hot test (lambda includes this tile)
    lam += ell;
    const unsigned long long hb = __ballot(ell > eps * lam && hh == 0);
    const bool hot0 = vis0 && (eps == 0.0f || (hb & 0xFFFFull) != 0ull);
    const bool hot1 = vis1 && (eps == 0.0f || (hb & 0xFFFF0000ull) != 0ull);
    const unsigned long long hot_lanes = (hot0 ? kGroup0 : 0ull) | (hot1 ? ~kGroup0 : 0ull);
    const bool my_hot = __builtin_amdgcn_inverse_ballot_w64(hot_lanes);

    // ---- frame update: cold -> mc; hot -> max(m, mc - H), which is m unless
    // the lazy test fired
    mf = my_hot ? vmax(mf, mcf - Hf) : mcf;

    // ---- step 5: cold tiles accumulate P V in FP4
    const bool cold0 = vis0 && !hot0, cold1 = vis1 && !hot1;
    if (cold0 || cold1) {
      const unsigned long long cold_lanes = (cold0 ? kGroup0 : 0ull) | (cold1 ? ~kGroup0 : 0ull);
      const bool keep = __builtin_amdgcn_inverse_ballot_w64(cold_lanes);
      const v4i pz = keep ? pb : v4i{0, 0, 0, 0};
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] = mfma4(va[db], pz, o[db], (int)vsw[db >> 2], db & 3, pscale);
      lsum = keep ? lsum + ell : lsum;
    }

    // ---- hot bits, whole words
    if (it == 0) {
      tile0_b0 = hot0 ? 1u : 0u;
      tile0_b1 = hot1 ? 1u : 0u;
    } else {
      const int w = t >> 5;
      if (w != cur_w) {
        if (cur_w > 0 && lane == 0) {
          bits0[cur_w] = cur_b0;
          if (has_g1) bits1[cur_w] = cur_b1;
        }
        cur_w = w;
        cur_b0 = cur_b1 = 0u;
      }
      if (hot0) cur_b0 |= 1u << (t & 31);
      if (hot1) cur_b1 |= 1u << (t & 31);
    }
  }
  // flush the last word (word 0, which also holds tile 0)
  if (lane == 0) {
    if (cur_w > 0) {
      bits0[cur_w] = cur_b0;
      if (has_g1) bits1[cur_w] = cur_b1;
    }
    bits0[0] = tile0_b0 | (cur_w == 0 ? cur_b0 : 0u);
    if (has_g1) bits1[0] = tile0_b1 | (cur_w == 0 ? cur_b1 : 0u);
  }

  // ---- outputs of the cold state, in the method's frame m
  if (row_ok) {
    const size_t r = bhq * g.Nq + row;
    const int m = (int)mf;
    const int sh = mo - m;
    if (hh == 0) {
      out.m[r] = m;
      out.l[r] = ldexpf(lsum, sh);
      if (out.lam) out.lam[r] = ldexpf(lam, sh);
    }
    // o * 2^sh * g_v, with 2^sh folded into g_v (exact)
    const float gs = ldexpf(g_v, sh);
    float* orow = out.o + r * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4f x = {o[db][4 * q] * gs, o[db][4 * q + 1] * gs, o[db][4 * q + 2] * gs,
                 o[db][4 * q + 3] * gs};
        *reinterpret_cast<v4f*>(orow + db * 32 + 8 * q + 4 * hh) = x;
      }
  }
}

template <int D>
hipError_t run(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
               const Pass1Out& o, hipStream_t s) {
  const int nunits = g.B * g.Hkv * (g.NqP / 32) * g.G;
  if (nunits == 0) return hipSuccess;
  const int nblocks = (nunits + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(k_pass1<D>, dim3(nblocks), dim3(kWaves * 64), 0, s, g, f, eps, tau, hoff, o,
                     nunits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pass1(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                        const Pass1Out& o, hipStream_t s) {
  switch (g.D) {
    case 64: return run<64>(g, f, eps, tau, hoff, o, s);
    case 128: return run<128>(g, f, eps, tau, hoff, o, s);
    case 256: return run<256>(g, f, eps, tau, hoff, o, s);
    case 512: return run<512>(g, f, eps, tau, hoff, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace apa
