// a3..a7: pass 1 of APA -- every visited key tile in block-scaled FP4 with the
// hot test ("APA: sloppy attention, exact where it counts", rfriedmann.de,
// section "Pass 1: FP4 everywhere, with a hot test", steps 1-5, "Tile order",
// the lazy maximum, and the decoupled cold frame of "The bug: a sink that
// drowned the tail").
//
// One wavefront owns 32 query rows of one query head = two 16-row verdict
// groups.  Per tile, with the wave's rows as MFMA columns (S^T = K Q^T, so a
// row's scores stay in its own lane pair):
//   S^T     : 2x(D/64) scaled FP4 MFMAs 32x32x64; the accumulator starts at
//             -m, so the MFMA returns scores already in the row's log2 frame
//             (Q's per-head scale is tied to K's so the score factor is the
//             power of two folded into Q's E8M0 bytes);
//   frame   : integer lazy maximum, moved to ceil(c) only when a score exceeds
//             the frame by more than tau;
//   P       : per 32-key group exponent E = ceil(c_g - log2 6); codes
//             E2M1(2^y / 2^E) from exp2 and the scaled FP4 conversion; one
//             V_PERMLANE32_SWAP per dword turns the accumulator layout into the
//             MFMA operand layout (V^T is stored in the matching key order);
//   l_t     : one FP4 MFMA of P against an all-ones operand (numerator and
//             denominator carry the same quantisation);
//   vote    : row hot iff l_t > eps * lambda (lambda includes this tile),
//             ballot over 16 rows;
//   cold PV : O^T += V^T P^T for the rows of cold groups, FP4 MFMA.
// Hot bits are written as whole 32-tile words, so every word of the mask is
// defined without a clearing pass.  No cross-wave synchronisation.
#include "apa_device.h"
#include "apa_kernels.h"

namespace apa {

namespace {

constexpr int kWaves = 4;  // wavefronts per block

template <int D>
__global__ __launch_bounds__(kWaves * 64) void k_pass1(Geom g, Fp4Ptrs f, float eps, float tau,
                                                       int hoff, Pass1Out out, int nunits) {
  constexpr int NH = D / 64;  // 64-channel halves of the QK contraction
  constexpr int ND = D / 32;  // 32-channel blocks of the output
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;       // the wave's row handled by this lane
  const int hh = lane >> 5;      // which half of the K dimension this lane feeds
  const int nblocks = gridDim.x;
  const int lb = xcd_remap(blockIdx.x, nblocks);
  const int unit = lb * kWaves + (threadIdx.x >> 6);
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
  const int last = min(r0 + 31, g.Nq - 1);
  auto diag = [&](int lr) { return g.causal ? min(g.Nkv - 1, lr + g.off) / kTile : g.NT - 1; };
  const int dW = diag(last);
  const bool has_g1 = r0 + 16 < g.Nq;
  const int d0 = diag(min(r0 + 15, g.Nq - 1));
  const int d1 = has_g1 ? diag(last) : -1;
  const int grp = n >> 4;

  // Q^T operand (resident): 16 bytes per 64-channel half, E8M0 byte + j
  const int jq = (int)f.q_head[bhq * 4 + 2];
  v4i qa[NH];
  int qs[NH];
  {
    const uint8_t* qc = f.q_codes + (bhq * g.NqP + row) * (D / 2);
    const uint8_t* qsc = f.q_scales + (bhq * g.NqP + row) * (D / 32);
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      qa[h] = *reinterpret_cast<const v4i*>(qc + 32 * h + 16 * hh);
      int sb = (int)qsc[2 * h + hh] + jq;
      qs[h] = sb < 0 ? 0 : (sb > 254 ? 254 : sb);
    }
  }
  const float g_v = f.kv_head[bhk * 8 + 4];

  const uint8_t* kc_base = f.k_codes + bhk * g.NkvP * (D / 2);
  const uint8_t* ks_base = f.k_scales + bhk * g.NkvP * (D / 32);
  const uint8_t* vc_base = f.v_codes + bhk * D * (g.NkvP / 2);
  const uint8_t* vs_base = f.v_scales + bhk * D * (g.NkvP / 32);

  // running state of this lane's row
  int m = 0;
  bool mvalid = false;
  float lam = 0.0f, lsum = 0.0f;
  v16f o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
    for (int j = 0; j < 16; ++j) o[i][j] = 0.0f;

  // hot-bit words: zero the words above the diagonal word first
  uint32_t* bits0 = out.bits + (bhq * g.NG + (r0 >> 4)) * g.W;
  uint32_t* bits1 = bits0 + g.W;
  for (int w = dW / 32 + 1 + lane; w < g.W; w += 64) {
    bits0[w] = 0u;
    if (has_g1) bits1[w] = 0u;
  }
  uint32_t tile0_b0 = 0, tile0_b1 = 0, cur_b0 = 0, cur_b1 = 0;
  int cur_w = -1;

  const int ntiles = dW + 1;
  for (int it = 0; it < ntiles; ++it) {
    const int t = it == 0 ? 0 : dW - it + 1;
    const int k0 = t * kTile;
    const bool vis0 = t <= d0, vis1 = has_g1 && t <= d1;

    // ---- loads: K operand (keys k0 + 32 kb + n), V^T operand, scales
    v4i ka[2][NH];
    int ks[2][NH];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const size_t key = (size_t)k0 + kb * 32 + n;
      const uint8_t* kc = kc_base + key * (D / 2);
      const uint8_t* kss = ks_base + key * (D / 32);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        ka[kb][h] = *reinterpret_cast<const v4i*>(kc + 32 * h + 16 * hh);
        ks[kb][h] = kss[2 * h + hh];
      }
    }
    v4i va[ND];
    int vsc[ND];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const size_t ch = (size_t)db * 32 + n;
      va[db] = *reinterpret_cast<const v4i*>(vc_base + ch * (g.NkvP / 2) + t * 32 + hh * 16);
      vsc[db] = vs_base[ch * (g.NkvP / 32) + t * 2 + hh];
    }

    // ---- step 1: scores in the current frame
    const float cinit = mvalid ? -(float)m : 0.0f;
    v16f acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[kb][j] = cinit;
#pragma unroll
      for (int h = 0; h < NH; ++h) acc[kb] = mfma_fp4(ka[kb][h], qa[h], acc[kb], ks[kb][h], qs[h]);
    }
    // wave-uniform: does any (row, key) of this tile need masking?
    const bool need_mask = (k0 + kTile > g.Nkv) || (g.causal && k0 + kTile - 1 > r0 + g.off) ||
                           (r0 + 31 >= g.Nq);
    if (need_mask) {
      const int lim = g.causal ? row + g.off : 0x7fffffff;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          const bool vis = row_ok && key < g.Nkv && key <= lim;
          if (!vis) acc[kb][j] = -__builtin_inff();
        }
    }
    // group maxima: lanes < 32 end with block 0's, lanes >= 32 with block 1's
    float gl0 = acc[0][0], gl1 = acc[1][0];
#pragma unroll
    for (int j = 1; j < 16; ++j) {
      gl0 = fmaxf(gl0, acc[0][j]);
      gl1 = fmaxf(gl1, acc[1][j]);
    }
    int x0, x1;
    swap_halves(__float_as_int(gl0), __float_as_int(gl1), x0, x1);
    const float gown = fmaxf(__int_as_float(x0), __int_as_float(x1));  // max of block hh
    const float gother = xor32(gown);                                 // max of block 1-hh
    float G0 = hh ? gother : gown;
    float G1 = hh ? gown : gother;
    const float c = fmaxf(G0, G1);

    // ---- lazy maximum (integer frame)
    const bool fire = mvalid ? (c > tau) : (c > -__builtin_inff());
    const int delta = fire ? (int)ceilf(c) : 0;
    if (__ballot(fire && delta != 0) != 0ull) {
      const float fd = (float)delta;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[kb][j] -= fd;
      G0 -= fd;
      G1 -= fd;
    }
    const int mc = fire ? (mvalid ? m + delta : delta) : m;
    const bool mc_valid = mvalid || fire;

    // ---- step 2: P per 32-key group
    const int E0 = G0 == -__builtin_inff() ? -127 : max(-127, (int)ceilf(G0 - kLog2_6));
    const int E1 = G1 == -__builtin_inff() ? -127 : max(-127, (int)ceilf(G1 - kLog2_6));
    unsigned pk[2][2];
    // exp2 flushes results below 2^-126: a group that far below the frame is
    // converted from 2^(y - E) instead (rare; wave-uniform branch)
    const bool deep = (G0 != -__builtin_inff() && E0 <= -124) || (G1 != -__builtin_inff() && E1 <= -124);
    const bool slow = __ballot(deep) != 0ull;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int E = kb ? E1 : E0;
      float sc;
      float sub;
      if (!slow) { sc = pow2_scale(E); sub = 0.0f; }
      else { sc = 1.0f; sub = (float)E; }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        unsigned w = 0;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int i = 8 * j + 2 * p;
          w = cvt_fp4x2(w, fast_exp2(acc[kb][i] - sub), fast_exp2(acc[kb][i + 1] - sub), sc, p);
        }
        pk[kb][j] = w;
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
    const int Eown = hh ? E1 : E0;
    const int pscale = Eown + 127;

    // ---- step 3: row sums from the same quantised P
    v16f ones_acc;
#pragma unroll
    for (int j = 0; j < 16; ++j) ones_acc[j] = 0.0f;
    const v4i ones = {kE2M1Ones, kE2M1Ones, kE2M1Ones, kE2M1Ones};
    ones_acc = mfma_fp4(ones, pb, ones_acc, kE8M0One, pscale);
    const float ell = ones_acc[0];

    // ---- step 4: the hot test
    const float lam_c = (mvalid ? ldexpf(lam, m - mc) : 0.0f) + ell;
    const bool row_hot = ell > eps * lam_c;
    const unsigned long long hb = __ballot(row_hot && hh == 0);
    const bool any0 = (hb & 0xFFFFull) != 0ull, any1 = (hb & 0xFFFF0000ull) != 0ull;
    const bool hot0 = vis0 && (eps == 0.0f || any0);
    const bool hot1 = vis1 && (eps == 0.0f || any1);
    const bool my_hot = grp ? hot1 : hot0;

    // ---- frame update: cold -> mc; hot -> decoupled lift max(m, mc - H)
    int mn;
    bool mn_valid;
    if (!my_hot) {
      mn = mc;
      mn_valid = mc_valid;
    } else if (fire) {
      mn = mvalid ? max(m, mc - hoff) : mc - hoff;
      mn_valid = true;
    } else {
      mn = m;
      mn_valid = mvalid;
    }
    const int oshift = (mvalid && mn_valid) ? mn - m : 0;  // o, l scale by 2^-oshift
    if (__ballot(oshift != 0) != 0ull) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] = ldexpf(o[db][j], -oshift);
      lsum = ldexpf(lsum, -oshift);
    }
    lam = mc_valid && mn_valid ? ldexpf(lam_c, mc - mn) : lam_c;
    m = mn;
    mvalid = mn_valid;

    // ---- step 5: cold tiles accumulate P V in FP4
    const bool cold0 = vis0 && !hot0, cold1 = vis1 && !hot1;
    if (cold0 || cold1) {
      const bool keep = grp ? cold1 : cold0;
      const v4i pz = keep ? pb : v4i{0, 0, 0, 0};
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] = mfma_fp4(va[db], pz, o[db], vsc[db], pscale);
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
      bits0[0] = tile0_b0;
      if (has_g1) bits1[0] = tile0_b1;
    } else {
      bits0[0] = tile0_b0 | (cur_w == 0 ? cur_b0 : 0u);
      if (has_g1) bits1[0] = tile0_b1 | (cur_w == 0 ? cur_b1 : 0u);
    }
  }

  // ---- outputs of the cold state
  if (row_ok) {
    const size_t r = bhq * g.Nq + row;
    if (hh == 0) {
      out.m[r] = mvalid ? m : (int32_t)0x80000000;
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
