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
//   frame   : integer lazy maximum, moved to ceil(c) only when the tile max
//             exceeds the frame by more than tau;
//   P       : per 32-key group exponent E = ceil(c_g - m - log2 6); code
//             E2M1(2^s / 2^(E + m)) from exp2 and the scaled FP4 conversion
//             (the frame rides in the conversion's power-of-two divisor); one
//             V_PERMLANE32_SWAP per dword turns the accumulator layout into the
//             MFMA operand layout (V^T is stored in the matching key order);
//   l_t     : one FP4 MFMA of P against an all-ones operand (numerator and
//             denominator carry the same quantisation);
//   vote    : row hot iff l_t > eps * lambda (lambda includes this tile),
//             ballot over 16 rows;
//   cold PV : O^T += V^T P^T for the rows of cold groups, FP4 MFMA.
// Hot bits are written as whole 32-tile words, so every word of the mask is
// defined without a clearing pass.
#include "apa_device.h"
#include "apa_kernels.h"

namespace apa {

namespace {

constexpr int kWaves = 4;                 // wavefronts per work group
constexpr int kNoFrame = -(1 << 30);      // frame of a row that has seen no key

template <int D>
struct Tile {
  static constexpr int NH = D / 64;       // 64-channel halves of the QK contraction
  static constexpr int ND = D / 32;       // 32-channel blocks of the output
  static constexpr int BLOB = 68 * D;
};

// The D/32 scale bytes of one key (or of one V lane), as little-endian words.
template <int D>
__device__ __forceinline__ void load_scales(uint32_t (&w)[2], const uint8_t* p) {
  if constexpr (D == 64) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
    w[1] = 0u;
  } else if constexpr (D == 128) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
    w[1] = 0u;
  } else {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x;
    w[1] = x.y;
  }
}

__device__ __forceinline__ int scale_byte(const uint32_t (&w)[2], int byte) {
  return (w[byte >> 2] >> (8 * (byte & 3))) & 255;
}

template <int D>
struct KOps {
  v4i a[2][Tile<D>::NH];
  uint32_t s[2][2];
};

template <int D>
__device__ __forceinline__ void load_k(KOps<D>& k, const uint8_t* blob, int n, int hh) {
  constexpr int NH = Tile<D>::NH;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const uint8_t* kr = blob + (kb * 32 + n) * (D / 2) + 16 * hh;
#pragma unroll
    for (int h = 0; h < NH; ++h) k.a[kb][h] = *reinterpret_cast<const v4i*>(kr + 32 * h);
    load_scales<D>(k.s[kb], blob + 32 * D + (kb * 32 + n) * (D / 32));
  }
}

// S^T for one tile: two 32-key blocks, absolute log2 scores.
template <int D>
__device__ __forceinline__ void qk(v16f (&acc)[2], const KOps<D>& k, const v4i* qa, const int* qs,
                                   int hh) {
  constexpr int NH = Tile<D>::NH;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    acc[kb] = mfma_fp4(k.a[kb][0], qa[0], v16f{}, scale_byte(k.s[kb], hh), qs[0]);
#pragma unroll
    for (int h = 1; h < NH; ++h)
      acc[kb] = mfma_fp4(k.a[kb][h], qa[h], acc[kb], scale_byte(k.s[kb], 2 * h + hh), qs[h]);
  }
}

template <int D>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_pass1(Geom g, Fp4Ptrs f, float eps, float tau,
                                                       int hoff, Pass1Out out, int nunits) {
  constexpr int NH = Tile<D>::NH;
  constexpr int ND = Tile<D>::ND;
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
  const int grp = n >> 4;

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

  // running state of this lane's row (m = kNoFrame: no key seen yet)
  int m = kNoFrame;
  float lam = 0.0f, lsum = 0.0f;
  v16f o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = v16f{};

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
  // and K of tile it+2 is fetched into kn
  KOps<D> kn;
  v16f acc[2];
  // (prefetches past the last tile re-read the last tile: in bounds, unused)
  auto next_blob = [&](int it) { return blobs + (size_t)tile_of(min(it, ntiles - 1)) * BLOB; };
  load_k<D>(kn, blobs, n, hh);
  qk<D>(acc, kn, qa, qs, hh);
  load_k<D>(kn, next_blob(1), n, hh);

  for (int it = 0; it < ntiles; ++it) {
    const int t = tile_of(it);
    const uint8_t* blob = blobs + (size_t)t * BLOB;
    // V^T operand and scales of this tile (used at its end)
    v4i va[ND];
    uint32_t vsw[2];
#pragma unroll
    for (int db = 0; db < ND; ++db)
      va[db] = *reinterpret_cast<const v4i*>(blob + 34 * D + (db * 32 + n) * 32 + 16 * hh);
    load_scales<D>(vsw, blob + 66 * D + (2 * n + hh) * ND);

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
    // group maxima: lanes < 32 end with block 0's, lanes >= 32 with block 1's
    float gl0 = vmax(acc[0][0], acc[0][1]), gl1 = vmax(acc[1][0], acc[1][1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) {
      gl0 = vmax3(gl0, acc[0][j], acc[0][j + 1]);
      gl1 = vmax3(gl1, acc[1][j], acc[1][j + 1]);
    }
    int x0, x1;
    swap_halves(__float_as_int(gl0), __float_as_int(gl1), x0, x1);
    const float gown = vmax(__int_as_float(x0), __int_as_float(x1));  // block hh
    const float gother = xor32(gown);                                // block 1-hh
    const float G0 = hh ? gother : gown;                             // absolute
    const float G1 = hh ? gown : gother;
    const float c = vmax(G0, G1);

    // ---- lazy maximum (integer frame)
    const bool fire = c > (float)m + tau;          // never for an all-masked row
    const int mc = fire ? (int)ceilf(c) : m;

    // ---- step 2: P per 32-key group, E = ceil(c_g - mc - log2 6) >= -127;
    // code = E2M1(2^s / 2^(E + mc)), exact while 2^s stays a normal float over
    // the group's range, else the frame-relative form 2^(s - mc - E)
    const bool live0 = G0 != -__builtin_inff(), live1 = G1 != -__builtin_inff();
    const int E0 = live0 ? max(-127, (int)ceilf(G0 - (float)mc - kLog2_6)) : -127;
    const int E1 = live1 ? max(-127, (int)ceilf(G1 - (float)mc - kLog2_6)) : -127;
    const bool odd = (live0 && (G0 > 120.0f || G0 < -110.0f || E0 <= -124)) ||
                     (live1 && (G1 > 120.0f || G1 < -110.0f || E1 <= -124));
    unsigned pk[2][2];
    if (__ballot(odd) == 0ull) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool live = kb ? live1 : live0;
        const float sc = pow2_scale(live ? (kb ? E1 : E0) + mc : 0);
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
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool live = kb ? live1 : live0;
        const float sub = live ? (float)(mc + (kb ? E1 : E0)) : 0.0f;
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
    const int pscale = (hh ? E1 : E0) + 127;

    // ---- step 3: row sums from the same quantised P
    const v4i ones = {kE2M1Ones, kE2M1Ones, kE2M1Ones, kE2M1Ones};
    const v16f ones_acc = mfma_fp4(ones, pb, v16f{}, kE8M0One, pscale);
    // this tile's scores are consumed: the next tile's go to the matrix cores
    // behind the row sum and run during the vote and the P V product
    __builtin_amdgcn_sched_barrier(0);
    qk<D>(acc, kn, qa, qs, hh);
    load_k<D>(kn, next_blob(it + 2), n, hh);
    const float ell = ones_acc[0];

    // ---- step 4: the hot test (lambda includes this tile)
    const float lam_c = ldexpf(lam, m - mc) + ell;   // lam = 0 while m = kNoFrame
    const unsigned long long hb = __ballot(ell > eps * lam_c && hh == 0);
    const bool hot0 = vis0 && (eps == 0.0f || (hb & 0xFFFFull) != 0ull);
    const bool hot1 = vis1 && (eps == 0.0f || (hb & 0xFFFF0000ull) != 0ull);
    const bool my_hot = grp ? hot1 : hot0;

    // ---- frame update: cold -> mc; hot -> decoupled lift max(m, mc - H)
    const int mn = !my_hot ? mc : (fire ? max(m, mc - hoff) : m);
    const int oshift = m == kNoFrame ? 0 : mn - m;   // o, l scale by 2^-oshift
    if (__ballot(oshift != 0) != 0ull) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] = ldexpf(o[db][j], -oshift);
      lsum = ldexpf(lsum, -oshift);
    }
    lam = ldexpf(lam_c, mc - mn);
    m = mn;

    // ---- step 5: cold tiles accumulate P V in FP4
    const bool cold0 = vis0 && !hot0, cold1 = vis1 && !hot1;
    if (cold0 || cold1) {
      const bool keep = grp ? cold1 : cold0;
      const v4i pz = keep ? pb : v4i{0, 0, 0, 0};
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] = mfma_fp4(va[db], pz, o[db], scale_byte(vsw, db), pscale);
      if (keep) lsum += ell;
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

  // ---- outputs of the cold state
  if (row_ok) {
    const size_t r = bhq * g.Nq + row;
    if (hh == 0) {
      out.m[r] = m == kNoFrame ? (int32_t)0x80000000 : m;
      out.l[r] = lsum;
      if (out.lam) out.lam[r] = lam;
    }
    float* orow = out.o + r * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4f x = {o[db][4 * q] * g_v, o[db][4 * q + 1] * g_v, o[db][4 * q + 2] * g_v,
                 o[db][4 * q + 3] * g_v};
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace apa
