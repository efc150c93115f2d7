// a1 statistics and a2 block-scaled FP4 quantisation.
//
// "APA: sloppy attention, exact where it counts" (rfriedmann.de), section
// "Pass 1: FP4 everywhere, with a hot test": before pass 1, K and V^T are
// stored as E2M1 codes with their scales, K centred on its per-channel mean
// ("Mean-centred K"), with one FP32 scale per head.  Here the block format is
// MXFP4: one E8M0 exponent per 32 elements (Q and K along channels, V along
// keys), the smallest that fits the block maximum under 6, and E2M1 codes
// rounded to nearest even by the hardware's scaled conversion.  The page's
// per-head scale serves NVFP4's narrow UE4M3 block scales; with E8M0 block
// exponents it only moves the mantissas of the normalised values, so V, whose
// codes need no statistics, enters at its own scale (per-head scale 1) and is
// coded in the statistics pass.  K needs its mean first and Q its tie to K's
// scale, so they are coded in a second pass.
//
// HBM-bound work: K is read twice (statistics, then quantisation), V and Q
// once each (Q twice: its maximum, then its codes); every reduction has a
// fixed order, so results are deterministic.  The quantisation pass takes Q
// and the KV heads in the reverse of the order the statistics pass read
// them, so the data read last, still in the last-level (Infinity) cache, is
// read again first.
#include "apa_device.h"
#include "apa_kernels.h"
#include <type_traits>

namespace apa {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

namespace {

// Block-wide max over blockDim.x threads (<= 512) through LDS.
__device__ float block_max(float v, float* red) {
  const int t = threadIdx.x;
  // wave-level reduction first
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  __syncthreads();
  if ((t & 63) == 0) red[t >> 6] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < (int)((blockDim.x + 63) >> 6); ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// Per (b, kv-head, chunk of 16 tiles of 64 keys): per-channel FP64 sums of K
// in a fixed order (keys ascending inside a tile, the chunk's tile sums
// ascending), min and max of K over the statistics keys, and a non-finite
// check over every key read.  Thread (tile tt, channel group cg) owns 8
// consecutive channels of one tile (16-byte loads); a block of
// min(2*D, 512) threads takes the chunk's 16 tiles at once (in two passes of
// 8 at D = 512).
template <typename T>
__device__ void k_chunk_stats(const T* __restrict__ K, const Geom& g, const QuantWs& ws, int ch,
                              int bh, double* sh) {
  const int D = g.D, ncg = D / 8;
  const int tpp = blockDim.x / ncg;  // tiles per pass
  const int cg = threadIdx.x % ncg;
  double* ssum = sh;
  float* smn = reinterpret_cast<float*>(sh + 16 * D);
  float* smx = smn + 16 * D;
  bool bad = false;
  for (int tt = threadIdx.x / ncg; tt < 16; tt += tpp) {
    const int t = ch * 16 + tt;
    double s[8];
    float mn[8], mx[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) { s[i] = 0.0; mn[i] = __builtin_inff(); mx[i] = -__builtin_inff(); }
    if (t < g.NT && t >= g.qt0 && t < g.qt1) {
      // keys [k0, k1) feed the statistics, [k1, kend) only the check
      const int k0 = t * kTile, kend = min(g.Nkv, k0 + kTile);
      const int k1 = max(k0, min(stat_khi(g), kend));
      // the tile's keys are contiguous (flat or paged input)
      const size_t base = kv_elem(g, bh / g.Hkv, bh % g.Hkv, k0) + cg * 8;
      auto row = [&](int k) {
        return *reinterpret_cast<const uint4*>(K + base + (size_t)(k - k0) * D);
      };
      // rows in batches of eight: every load of a batch is issued before the
      // first is used
      constexpr int kB = 8;
      int k = k0;
      if constexpr (std::is_same<T, _Float16>::value) {
        // fp16: minima and maxima two channels at a time in fp16 (exact)
        h2 hmn[4], hmx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hmn[j] = h2{(_Float16)__builtin_inff(), (_Float16)__builtin_inff()};
          hmx[j] = -hmn[j];
        }
        auto add = [&](const uint4& rk) {
          const h2* e2 = reinterpret_cast<const h2*>(&rk);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            hmn[j] = __builtin_elementwise_min(hmn[j], e2[j]);
            hmx[j] = __builtin_elementwise_max(hmx[j], e2[j]);
            s[2 * j] += (double)(float)e2[j][0];
            s[2 * j + 1] += (double)(float)e2[j][1];
          }
        };
        for (; k + kB <= k1; k += kB) {
          uint4 r[kB];
#pragma unroll
          for (int u = 0; u < kB; ++u) r[u] = row(k + u);
#pragma unroll
          for (int u = 0; u < kB; ++u) add(r[u]);
        }
        for (; k < k1; ++k) add(row(k));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          mn[i] = (float)hmn[i >> 1][i & 1];
          mx[i] = (float)hmx[i >> 1][i & 1];
        }
      } else {
        auto add = [&](const uint4& rk) {
          const T* ek = reinterpret_cast<const T*>(&rk);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = to_f32<T>(ek[i]);
            s[i] += (double)x;
            mn[i] = fminf(mn[i], x);
            mx[i] = fmaxf(mx[i], x);
          }
        };
        for (; k + kB <= k1; k += kB) {
          uint4 r[kB];
#pragma unroll
          for (int u = 0; u < kB; ++u) r[u] = row(k + u);
#pragma unroll
          for (int u = 0; u < kB; ++u) add(r[u]);
        }
        for (; k < k1; ++k) add(row(k));
      }
      // a NaN or an infinity among the statistics keys leaves its channel's
      // FP64 sum non-finite (the sum of finite 16-bit values over one tile is
      // far inside the FP64 range)
#pragma unroll
      for (int i = 0; i < 8; ++i) bad |= !__builtin_isfinite(s[i]);
      for (int k = k1; k < kend; ++k) {
        const uint4 rk = *reinterpret_cast<const uint4*>(K + base + (size_t)(k - k0) * D);
        const T* ek = reinterpret_cast<const T*>(&rk);
#pragma unroll
        for (int i = 0; i < 8; ++i) bad |= !__builtin_isfinite(to_f32<T>(ek[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ssum[tt * D + cg * 8 + i] = s[i];
      smn[tt * D + cg * 8 + i] = mn[i];
      smx[tt * D + cg * 8 + i] = mx[i];
    }
  }
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) ws.flags[(size_t)bh * ws.nch + ch] = bad ? 1u : 0u;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    double c = 0.0;
    float a = __builtin_inff(), b = -__builtin_inff();
    for (int i = 0; i < 16; ++i) {  // the chunk's tile sums, ascending
      c += ssum[i * D + d];
      a = fminf(a, smn[i * D + d]);
      b = fmaxf(b, smx[i * D + d]);
    }
    const size_t o = ((size_t)bh * ws.nch + ch) * D + d;
    ws.ksum[o] = c;
    ws.kmin[o] = a;
    ws.kmax[o] = b;
  }
}

// V^T codes of the V items (b, kv-head, 64-key tile, 128-channel slice cz)
// of tiles t0 .. t0 + nt - 1.  V enters at its own scale: its E8M0 block
// exponents carry the range, so its codes need no statistics.  Each tile's
// slice is staged in LDS (16-byte loads, zeros for keys past Nkv), then
// thread (channel c, key half) takes one 32-key block: the smallest exponent
// that fits its maximum under 6, E2M1 codes stored with the eight 4-key runs
// in the order 0,2,4,6,1,3,5,7.  Also: max |V| over the keys and the
// non-finite flag (per block); with the weighted test and cz = 0, every key's
// value norm (squares in FP32 in channel order inside a thread, over the
// threads of the key by an xor butterfly; from the staged slice when it holds
// the whole row, D <= 128), each tile's largest norm and the FP64 sum of its
// statistics keys' norms, keys ascending.
template <typename T>
__device__ void v_items(const T* __restrict__ V, const Geom& g, const QuantWs& ws,
                        const Fp4Ptrs& f, int bh, int t0, int nt, int cz, T* tile, float* red,
                        float* knu) {
  // a staged row is ld elements apart whatever nch is, so that every column
  // read below has a constant offset from one base
  constexpr int CH = 128, PADH = 8, ld = CH + PADH;
  const int D = g.D, c0 = cz * CH, nch = min(CH, D - c0);
  const int b = bh / g.Hkv, hk = bh % g.Hkv;
  const int per_row = nch / 8;
  // 64 rows x nch channels in 16-byte pieces, kStage per thread (the block has
  // 2 * nch threads); a tile's rows are contiguous (flat or paged), rows past
  // Nkv re-read the last key and are stored as zeros.  The next tile's loads
  // are in flight while this tile is coded.
  constexpr int kStage = 4;
  uint4 r[kStage];
  auto load = [&](int t) {
    const int k0 = t * kTile, last = min(g.Nkv, k0 + kTile) - 1 - k0;
    const T* src = V + kv_elem(g, b, hk, k0) + c0;
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      const int kk = i / per_row, c = (i % per_row) * 8;
      r[j] = *reinterpret_cast<const uint4*>(src + (size_t)min(kk, last) * D + c);
    }
  };
  const int c = threadIdx.x % nch, half = threadIdx.x / nch;
  bool bad = false;
  float as = 0.0f;
  load(t0);
  for (int it = 0; it < nt; ++it) {
    const int t = t0 + it;
    const int k0 = t * kTile, kend = min(g.Nkv, k0 + kTile);
    const int k1 = max(k0, min(stat_khi(g), kend));
    const int last = kend - 1 - k0;
    if (it > 0) __syncthreads();  // every read of the previous tile is done
#pragma unroll
    for (int j = 0; j < kStage; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      const int kk = i / per_row, cc = (i % per_row) * 8;
      *reinterpret_cast<uint4*>(&tile[kk * ld + cc]) = kk <= last ? r[j] : uint4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    if (it + 1 < nt) load(t + 1);
    {
      // two passes over the staged column (the block maximum, then the
      // codes), so that the 32 values need not stay in registers
      const T* col = tile + half * 32 * ld + c;
      auto xv = [&](int i) { return to_f32<T>(col[i * ld]); };
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float x = xv(i);
        bad |= !__builtin_isfinite(x);
        a = fmaxf(a, fabsf(x));
      }
      as = fmaxf(as, a);  // rows past Nkv are zeros
      const int e = e8m0_exponent(a);
      const float sc = pow2_scale(e);
      constexpr int perm[8] = {0, 2, 4, 6, 1, 3, 5, 7};
      unsigned out[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        unsigned w = 0;
        const int ra = perm[2 * j] * 4, rb = perm[2 * j + 1] * 4;
        w = cvt_fp4x2(w, xv(ra + 0), xv(ra + 1), sc, 0);
        w = cvt_fp4x2(w, xv(ra + 2), xv(ra + 3), sc, 1);
        w = cvt_fp4x2(w, xv(rb + 0), xv(rb + 1), sc, 2);
        w = cvt_fp4x2(w, xv(rb + 2), xv(rb + 3), sc, 3);
        out[j] = w;
      }
      const int ch = c0 + c;
      uint8_t* blob = f.kv_blob + ((size_t)bh * g.NTc + blob_slot(g, t)) * blob_bytes(D);
      *reinterpret_cast<uint4*>(blob + 34 * D + ch * 32 + half * 16) =
          uint4{out[0], out[1], out[2], out[3]};
      blob[66 * D + ((ch % 32) * 2 + half) * (D / 32) + ch / 32] = (uint8_t)(e + 127);
    }
    if (g.vweight && cz == 0) {
      // parts threads per key, each D / parts consecutive channels
      const int parts = blockDim.x / kTile, cpp = D / parts;
      const int kk = threadIdx.x / parts, part = threadIdx.x % parts;
      float q = 0.0f;
      if (nch == D) {
        // the whole row is in the staged slice (zeros past Nkv)
        const T* row = tile + kk * ld + part * cpp;
        for (int c8 = 0; c8 < cpp; c8 += 8) {
          const uint4 rr = *reinterpret_cast<const uint4*>(row + c8);
          const T* e = reinterpret_cast<const T*>(&rr);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float y = to_f32<T>(e[i]);
            q = fmaf(y, y, q);
          }
        }
      } else if (k0 + kk < kend) {
        const T* row = V + kv_elem(g, b, hk, k0 + kk) + part * cpp;
        for (int c8 = 0; c8 < cpp; c8 += 8) {
          const uint4 rr = *reinterpret_cast<const uint4*>(row + c8);
          const T* e = reinterpret_cast<const T*>(&rr);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float y = to_f32<T>(e[i]);
            q = fmaf(y, y, q);
          }
        }
      }
      for (int o = 1; o < parts; o <<= 1) q += __shfl_xor(q, o);
      if (part == 0) knu[kk] = sqrtf(q);
      __syncthreads();
      if (threadIdx.x == 0) {
        float mx = 0.0f;
        double sn = 0.0;
        for (int i = 0; i < kTile; ++i) {
          mx = fmaxf(mx, knu[i]);
          if (k0 + i < k1) sn += (double)knu[i];
        }
        ws.vnt[(size_t)bh * g.NT + t] = mx;
        ws.vnst[(size_t)bh * g.NT + t] = sn;
      }
    }
  }
  // the block's max |V| and flag go to its first item, 0 to the others (the
  // finalize step folds them per head)
  bad = __syncthreads_or(bad);
  const float m = block_max(as, red);
  if (threadIdx.x < nt) {
    const size_t item = ((size_t)bh * g.NT + t0 + threadIdx.x) * ws.nvz + cz;
    ws.vamax[item] = threadIdx.x == 0 ? m : 0.0f;
    ws.flags[vflag0(g, ws) + item] = (threadIdx.x == 0 && bad) ? 1u : 0u;
  }
}

// max |Q| and the non-finite check per (b, q-head, 64-row tile), any block
// size.
template <typename T>
__device__ void q_stats(const T* __restrict__ Q, const Geom& g, const QuantWs& ws, int t, int bh,
                        float* red) {
  // the tile's rows are contiguous: 16-byte pieces, kQB per thread per round,
  // every load of a round issued before the first is used
  constexpr int kQB = 4;
  const int r0 = t * 64, n = (min(g.Nq, r0 + 64) - r0) * (g.D / 8);
  const T* src = Q + ((size_t)bh * g.Nq + r0) * g.D;
  float a = 0.0f;
  bool bad = false;
  for (int i0 = threadIdx.x; i0 < n; i0 += kQB * (int)blockDim.x) {
    uint4 r[kQB];
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      const int i = i0 + j * (int)blockDim.x;
      r[j] = i < n ? *reinterpret_cast<const uint4*>(src + (size_t)i * 8) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kQB; ++j) {
      const T* e = reinterpret_cast<const T*>(&r[j]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float x = to_f32<T>(e[k]);
        bad |= !__builtin_isfinite(x);
        a = fmaxf(a, fabsf(x));
      }
    }
  }
  bad = __syncthreads_or(bad);
  float m = block_max(a, red);
  if (threadIdx.x == 0) {
    ws.qamax[(size_t)bh * ws.nqt + t] = m;
    ws.flags[qflag0(g, ws) + (size_t)bh * ws.nqt + t] = bad ? 1u : 0u;
  }
}

// Head scale mapping amax to 6: g = fl32(amax/6), inv = fl32(6/amax); the FP64
// quotient rounded once is the correctly rounded binary32 quotient.
__device__ void head_scale(float amax, float* gs, float* inv) {
  if (!(amax > 0.0f)) { *gs = 1.0f; *inv = 1.0f; return; }
  *gs = (float)((double)amax / 6.0);
  *inv = (float)(6.0 / (double)amax);
}

// Chunk statistics are read in batches of kFinBatch chunks with every load of
// a batch in flight (the block is latency-bound: few blocks, short chains).
constexpr int kFinBatch = 16;

// Per (b, kv-head), in two parts.  The key part (after the statistics pass):
// key mean, |K - kbar| max, the K head scale (V's is 1) and the tied Q scales
// of the group's query heads, folding the non-finite flags of its K chunks
// and Q tiles.  The value part (after the V coding): max |V|; with the
// weighted hot test the mean value norm nu_bar (FP64: each thread sums a
// contiguous run of tiles ascending, then the runs are added in thread order;
// a frozen cache keeps its own) and the weight w_t = max(1, nu_t / nu_bar) of
// every tile read (1 when nu_bar is 0), folding the flags of its V items.
// Each ORs its flags into the status word (cleared before either runs).
// Key part: block 2D threads; value part: any block size.
__device__ void finalize_kq(const Geom& g, const QuantWs& ws, const Fp4Ptrs& f, int bh,
                            float* xch, float* red) {
  const int d = threadIdx.x, nthr = blockDim.x, D = g.D;
  const bool own = d < D;  // threads D .. 2D-1 fold min and max, and join the block reductions
  const size_t base = (size_t)bh * ws.nch * D + (own ? d : d - D);
  const int b = bh / g.Hkv, hk = bh % g.Hkv;
  // first the loads that do not wait on the key statistics, so that they are
  // in flight with them: this head's non-finite flags (its K chunks [ch0,
  // ch1), the Q tiles of its query heads) and each query head's max |Q|
  unsigned badf = 0u;
  float qa[8];
  {
    for (int c = ws.ch0 + d; c < ws.ch1; c += nthr) badf |= ws.flags[(size_t)bh * ws.nch + c];
    const size_t q0 = ((size_t)b * g.Hq + (size_t)hk * g.G) * ws.nqt;
    const int nq = g.code_q ? g.G * ws.nqt : 0;  // Q's flags and maxima, when Q was read
    for (int i = d; i < nq; i += nthr) badf |= ws.flags[qflag0(g, ws) + q0 + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[i] = 0.0f;
      if (i < g.G && g.code_q)
        for (int t = d; t < ws.nqt; t += nthr) qa[i] = fmaxf(qa[i], ws.qamax[q0 + (size_t)i * ws.nqt + t]);
    }
  }
  double s = 0.0;
  float mn = __builtin_inff(), mx = -__builtin_inff();
  for (int c0 = ws.ch0; c0 < ws.ch1 && !g.frozen; c0 += kFinBatch) {
    if (own) {
      // channel d's chunk sums, added in ascending order
      double v[kFinBatch];
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
        v[i] = c0 + i < ws.ch1 ? ws.ksum[base + (size_t)(c0 + i) * D] : 0.0;
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i)
        if (c0 + i < ws.ch1) s += v[i];
    } else {
      float a[kFinBatch], b[kFinBatch];
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i) {
        const bool in = c0 + i < ws.ch1;
        a[i] = in ? ws.kmin[base + (size_t)(c0 + i) * D] : __builtin_inff();
        b[i] = in ? ws.kmax[base + (size_t)(c0 + i) * D] : -__builtin_inff();
      }
#pragma unroll
      for (int i = 0; i < kFinBatch; ++i) {
        mn = fminf(mn, a[i]);
        mx = fmaxf(mx, b[i]);
      }
    }
  }
  if (!own) {
    xch[d - D] = mn;
    xch[d] = mx;  // = xch[D + (d - D)]
  }
  __syncthreads();
  float dev = 0.0f;
  if (own) {
    mn = xch[d];
    mx = xch[D + d];
    const int nk = stat_khi(g) - stat_t0(g) * kTile;  // the keys the statistics cover
    const float kb = nk > 0 ? (float)(s / (double)nk) : 0.0f;
    if (!g.frozen) f.kbar[(size_t)bh * D + d] = kb;
    if (nk > 0) dev = fmaxf(mx - kb, kb - mn);
  }
  badf = __syncthreads_or(badf != 0u);
  if (d == 0 && badf) atomicOr(f.status, 1u);
  const float amax_k = block_max(dev, red);
  float gk, ik;
  head_scale(amax_k, &gk, &ik);
  // frozen statistics: the K/V scales stay the cache's; Q's tie to its g_K
  if (g.frozen) gk = f.kv_head[(size_t)bh * 8 + 1];
  if (d == 0 && !g.frozen) {
    // V is coded at its own scale (per-head scale 1); entries 3 and 6 are the
    // value part's
    float* kh = f.kv_head + (size_t)bh * 8;
    kh[0] = amax_k; kh[1] = gk; kh[2] = ik; kh[4] = 1.0f; kh[5] = 1.0f; kh[7] = 0.0f;
  }
  // Q heads of this group: inv_q = w * 2^-j, w = fl32(sl * g_k), j the
  // smallest integer with amax_q * w <= 6 * 2^j.  The first eight heads' max
  // |Q| were loaded above; further heads (groups above 8) load theirs here.
  // A call that leaves Q as it is (the ring's later segments) keeps them.
  if (!g.code_q) return;
  const float w = g.sl * gk;
  auto q_scale = [&](int i, float qv) {
    const size_t bq = (size_t)b * g.Hq + hk * g.G + i;
    const float amax_q = block_max(qv, red);
    if (d == 0) {
      int j = 0;
      if (amax_q > 0.0f && w > 0.0f) {
        const double prod = (double)amax_q * (double)w;  // exact
        int x;
        frexp(prod / 6.0, &x);
        j = x - 2;
        while (6.0 * ldexp(1.0, j) < prod) ++j;
        while (6.0 * ldexp(1.0, j - 1) >= prod) --j;
      }
      float* qh = f.q_head + bq * 4;
      qh[0] = amax_q;
      qh[1] = (float)ldexp((double)w, -j);
      qh[2] = (float)j;
      qh[3] = 0.0f;
    }
  };
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if (i < g.G) q_scale(i, qa[i]);
  for (int i = 8; i < g.G; ++i) {
    const size_t q0 = ((size_t)b * g.Hq + (size_t)hk * g.G + i) * ws.nqt;
    float qv = 0.0f;
    for (int t = d; t < ws.nqt; t += nthr) qv = fmaxf(qv, ws.qamax[q0 + t]);
    q_scale(i, qv);
  }
}

__device__ void finalize_v(const Geom& g, const QuantWs& ws, const Fp4Ptrs& f, int bh,
                           float* red, float* nbs, double* part) {
  const int d = threadIdx.x, nthr = blockDim.x;
  unsigned badf = 0u;
  float va = 0.0f;
  {
    const size_t i0 = ((size_t)bh * g.NT + g.ct0) * ws.nvz;
    const int n = (g.ct1 - g.ct0) * ws.nvz;
#pragma unroll 4
    for (int i = d; i < n; i += nthr) {
      va = fmaxf(va, ws.vamax[i0 + i]);
      badf |= ws.flags[vflag0(g, ws) + i0 + i];
    }
  }
  badf = __syncthreads_or(badf != 0u);
  if (d == 0 && badf) atomicOr(f.status, 1u);
  const float amax_v = block_max(va, red);
  if (g.vweight) {
    if (!g.frozen) {
      // thread d sums tiles [qt0 + d * run, qt0 + (d + 1) * run), ascending
      const int n = g.ct1 - g.ct0, run = (n + nthr - 1) / nthr;
      double sv = 0.0;
      for (int i = d * run; i < min(n, (d + 1) * run); ++i)
        sv += ws.vnst[(size_t)bh * g.NT + g.ct0 + i];
      part[d] = sv;
    }
    __syncthreads();
    if (d == 0) {
      float nb = f.kv_head[(size_t)bh * 8 + 6];
      if (!g.frozen) {
        double sv = 0.0;
        for (int i = 0; i < nthr; ++i) sv += part[i];
        const int nk = stat_khi(g) - stat_t0(g) * kTile;
        nb = nk > 0 ? (float)(sv / (double)nk) : 0.0f;
      }
      *nbs = nb;
    }
    __syncthreads();
    const float nb = *nbs;
    for (int t = g.ct0 + d; t < g.ct1; t += nthr) {
      const float nt = ws.vnt[(size_t)bh * g.NT + t];
      f.tile_w[(size_t)bh * g.NTc + t] = nb > 0.0f ? fmaxf(1.0f, nt / nb) : 1.0f;
    }
  }
  if (d == 0) {
    // max |V| over every key coded, for the 16-bit pass's range shift of
    // bf16 V: with frozen statistics the cache's value grows to cover the
    // new tiles too
    float* kh = f.kv_head + (size_t)bh * 8;
    kh[3] = g.frozen ? fmaxf(kh[3], amax_v) : amax_v;
    if (!g.frozen) kh[6] = g.vweight ? *nbs : 0.0f;
  }
}

// Block exponent of K by squared error ("Second hunt: which operand is to
// blame"), for a 32-element block held 8 per thread by 4 consecutive lanes:
// each candidate exponent quantises the block, and the one whose dequantised
// values lie closest to the inputs wins.  Candidates: e0 (no clipping), then
// e0 - 1 and e0 + 1, clamped to [-127, 127]; a later one wins only with a
// strictly smaller error.  The error is summed in FP32: d*d added in element
// order inside a lane, then the lanes' sums as (r0 + r1) + (r2 + r3).
__device__ __forceinline__ int lsq_exponent(const float (&x)[8], int e0) {
  constexpr float kMag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  int best = e0;
  float best_err = 0.0f;
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    int e = e0 + (c == 0 ? 0 : (c == 1 ? -1 : 1));
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    const float s = pow2_scale(e);
    unsigned w = 0;
    w = cvt_fp4x2(w, x[0], x[1], s, 0);
    w = cvt_fp4x2(w, x[2], x[3], s, 1);
    w = cvt_fp4x2(w, x[4], x[5], s, 2);
    w = cvt_fp4x2(w, x[6], x[7], s, 3);
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned code = (w >> (4 * i)) & 15u;
      const float q = kMag[code & 7u] * s;
      const float d = x[i] - ((code & 8u) ? -q : q);
      acc = acc + d * d;
    }
    acc = acc + __shfl_xor(acc, 1);
    acc = acc + __shfl_xor(acc, 2);
    if (c == 0 || acc < best_err) {
      best_err = acc;
      best = e;
    }
  }
  return best;
}

// Rows of one sub-block of 256 threads (thread: 8 consecutive channels of a
// row): the row of this thread, and its 16 input bytes (zeros for padding
// rows [Nrows, NP) and past the sub-blocks of the head).
template <typename T, bool IS_Q>
__device__ __forceinline__ uint4 load_row(const T* __restrict__ X, const Geom& g, int sub,
                                          int bh, int* row_out) {
  const int H = IS_Q ? g.Hq : g.Hkv;
  const int Nrows = IS_Q ? g.Nq : g.Nkv;
  const int lt = __builtin_ctz(g.D / 8);  // threads per row: D / 8, a power of two
  const int gid = sub * 256 + threadIdx.x;
  const int row = gid >> lt, c8 = (gid & ((1 << lt) - 1)) * 8;
  *row_out = row;
  if (row >= Nrows) return uint4{0u, 0u, 0u, 0u};
  const int b = bh / H, h = bh % H;
  const int hk = IS_Q ? h / g.G : h;
  const T* src = X + (IS_Q ? ((size_t)bh * Nrows + row) * g.D : kv_elem(g, b, hk, row)) + c8;
  return *reinterpret_cast<const uint4*>(src);
}

// The maximum over the four lanes of a quad (the threads of one 32-channel
// block), by two DPP quad permutations; every lane of the quad is active.
__device__ __forceinline__ float quad_max(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, false)));
  return fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, false)));
}

// What every row of a block's sub-blocks shares for one thread: its 8
// channels' kbar, the head's scale and the channel offset (loaded once per
// block: the code stores go through byte pointers, which the compiler must
// assume alias any global load after them).
struct RowConst {
  float kb[8];
  float inv;
  int c8;
};

template <bool IS_Q>
__device__ __forceinline__ RowConst row_const(const Geom& g, const Fp4Ptrs& f, int bh) {
  RowConst rc;
  rc.c8 = (threadIdx.x & (g.D / 8 - 1)) * 8;  // the same in every sub-block (256 % (D/8) == 0)
  const int H = IS_Q ? g.Hq : g.Hkv;
  const int b = bh / H, h = bh % H;
  const int hk = IS_Q ? h / g.G : h;
  const size_t bk = (size_t)b * g.Hkv + hk;
  rc.inv = IS_Q ? f.q_head[(size_t)bh * 4 + 1] : f.kv_head[bk * 8 + 2];
  const float4* kp = reinterpret_cast<const float4*>(f.kbar + bk * g.D + rc.c8);
  const float4 k0 = kp[0], k1 = kp[1];
  rc.kb[0] = k0.x; rc.kb[1] = k0.y; rc.kb[2] = k0.z; rc.kb[3] = k0.w;
  rc.kb[4] = k1.x; rc.kb[5] = k1.y; rc.kb[6] = k1.z; rc.kb[7] = k1.w;
  return rc;
}

// Quantise rows along channels (Q, or K - kbar).  Each thread owns 8
// consecutive channels of row `row` (its input in raw); 4 threads form one
// 32-channel block.  Rows in [Nrows, NP) are padding and get zero codes.  For
// Q it also writes the frame constant c_r = sl * q.kbar (FP32).
template <typename T, bool IS_Q>
__device__ void quant_rows(const uint4 raw, const Geom& g, const Fp4Ptrs& f, int row, int bh,
                           const RowConst& rc) {
  const int Nrows = IS_Q ? g.Nq : g.Nkv;
  const int NP = IS_Q ? g.NqP : g.NkvP;
  const int tpr = g.D / 8;                     // threads per row
  const int c8 = rc.c8;
  if (row >= NP) return;                       // whole rows exit together
  float x[8];
  float cdot = 0.0f;
  if (row < Nrows) {
    const T* e = reinterpret_cast<const T*>(&raw);
    for (int i = 0; i < 8; ++i) {
      float v = to_f32<T>(e[i]);
      if (IS_Q) {
        cdot = fmaf(v, rc.kb[i], cdot);
      } else {
        v = v - rc.kb[i];
      }
      float n = v * rc.inv;
      x[i] = fminf(fmaxf(n, -6.0f), 6.0f);
    }
  } else {
    for (int i = 0; i < 8; ++i) x[i] = 0.0f;
  }
  float a = 0.0f;
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(x[i]));
  a = quad_max(a);
  int e = e8m0_exponent(a);
  if (!IS_Q && g.klsq) e = lsq_exponent(x, e);
  const float s = pow2_scale(e);
  unsigned w = 0;
  w = cvt_fp4x2(w, x[0], x[1], s, 0);
  w = cvt_fp4x2(w, x[2], x[3], s, 1);
  w = cvt_fp4x2(w, x[4], x[5], s, 2);
  w = cvt_fp4x2(w, x[6], x[7], s, 3);
  const size_t r = (size_t)bh * NP + row;
  uint8_t *crow, *srow;
  if (IS_Q) {
    crow = f.q_codes + r * (g.D / 2);
    srow = f.q_scales + r * (g.D / 32);
  } else {
    uint8_t* blob = f.kv_blob + ((size_t)bh * g.NTc + blob_slot(g, row / kTile)) * blob_bytes(g.D);
    crow = blob + (row % kTile) * (g.D / 2);
    srow = blob + 32 * g.D + (row % kTile) * (g.D / 32);
  }
  *reinterpret_cast<unsigned*>(crow + c8 / 2) = w;
  if ((c8 & 31) == 0) srow[c8 / 32] = (uint8_t)(e + 127);
  if (IS_Q && g.qterms == 2) {
    // the second term: the FP32 residual of each normalised value after the
    // first term's dequantised value, quantised as a block of its own
    constexpr float kMag[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
    float a2 = 0.0f;
    for (int i = 0; i < 8; ++i) {
      const unsigned c = (w >> (4 * i)) & 15u;
      const float d = kMag[c & 7u] * s;  // exact: a power of two times a short value
      x[i] = x[i] - ((c & 8u) ? -d : d);
      a2 = fmaxf(a2, fabsf(x[i]));
    }
    a2 = quad_max(a2);
    const int e2 = e8m0_exponent(a2);
    const float s2 = pow2_scale(e2);
    unsigned w2 = 0;
    w2 = cvt_fp4x2(w2, x[0], x[1], s2, 0);
    w2 = cvt_fp4x2(w2, x[2], x[3], s2, 1);
    w2 = cvt_fp4x2(w2, x[4], x[5], s2, 2);
    w2 = cvt_fp4x2(w2, x[6], x[7], s2, 3);
    *reinterpret_cast<unsigned*>(f.q2_codes + r * (g.D / 2) + c8 / 2) = w2;
    if ((c8 & 31) == 0) f.q2_scales[r * (g.D / 32) + c8 / 32] = (uint8_t)(e2 + 127);
  }
  if (IS_Q) {
    // row reduction of the frame constant over the D/8 threads of the row
    for (int o = 1; o < tpr; o <<= 1) cdot += __shfl_xor(cdot, o);
    if (c8 == 0) f.q_frame[r] = row < Nrows ? g.sl * cdot : 0.0f;
  }
}

// K and Q statistics in one launch: blocks [0, NKB) take (kv-head, 16-tile
// chunk) of K, the rest (q-head, 64-row tile).  Block 0 clears the status word
// first (the finalize blocks OR into it).  block min(2*D, 512) threads,
// dynamic LDS 16*D*(8+4+4) bytes (the K chunk sums).
template <typename T>
__global__ __launch_bounds__(512) void k_stats(const T* __restrict__ Q, const T* __restrict__ K,
                                               Geom g, QuantWs ws, Fp4Ptrs f, int nkb) {
  extern __shared__ double sh[];
  __shared__ float red[16];
  if (!g.keep_status && blockIdx.x == 0 && threadIdx.x == 0) *f.status = 0u;
  const int bx = blockIdx.x;
  if (bx < nkb) {
    const int nc = ws.ch1 - ws.ch0;  // the chunks of the tiles read
    k_chunk_stats<T>(K, g, ws, ws.ch0 + bx % nc, bx / nc, sh);
  } else {
    const int qb = bx - nkb;
    q_stats<T>(Q, g, ws, qb % ws.nqt, qb / ws.nqt, red);
  }
}

// Tiles of V per V-coding block.
constexpr int kVTiles = 4;

// The V items of the tiles read (per kv-head, tile, 128-channel slice),
// kVTiles consecutive tiles of one slice per block, 2 * min(D, 128) threads.  Runs after k_stats, whose
// block 0 cleared the status word.  Up to D = 128 (block = 2D threads) the
// first nfin blocks are the key part of the finalize step, one per (b,
// kv-head): it needs only the statistics pass, so it runs beside the V coding
// rather than as a launch of its own; clear: the statistics pass did not run,
// so block 0 clears the status word (there are then no flags to fold).
template <typename T>
__global__ __launch_bounds__(256) void k_vcode(const T* __restrict__ V, Geom g, QuantWs ws,
                                               Fp4Ptrs f, int nfin, int clear) {
  __shared__ __attribute__((aligned(16))) T tile[kTile * (128 + 8)];
  __shared__ float red[16];
  __shared__ float knu[kTile];  // a tile's key norms
  if ((int)blockIdx.x < nfin) {
    float* xch = reinterpret_cast<float*>(tile);  // [2][D] (D <= 128)
    if (clear && !g.keep_status && blockIdx.x == 0 && threadIdx.x == 0) *f.status = 0u;
    finalize_kq(g, ws, f, blockIdx.x, xch, red);
    return;
  }
  const int blk = blockIdx.x - nfin;
  const int ngrp = (g.ct1 - g.ct0 + kVTiles - 1) / kVTiles;
  const int per_head = ngrp * ws.nvz;
  const int r = blk % per_head;
  const int t0 = g.ct0 + (r / ws.nvz) * kVTiles;
  v_items<T>(V, g, ws, f, blk / per_head, t0, min(kVTiles, g.ct1 - t0), r % ws.nvz, tile, red,
             knu);
}

// Both finalize parts as a launch of their own (D > 128, where the V coding's
// blocks are not 2D threads): one block of 2D threads per (b, kv-head).
__global__ void k_finalize(Geom g, QuantWs ws, Fp4Ptrs f, int clear) {
  extern __shared__ float xch[];  // [2][D]: min and max of each channel
  __shared__ float red[16];
  __shared__ float nbs;           // nu_bar
  __shared__ double part[1024];   // the threads' runs of tile norm sums
  if (clear && !g.keep_status && blockIdx.x == 0 && threadIdx.x == 0) *f.status = 0u;
  finalize_kq(g, ws, f, blockIdx.x, xch, red);
  __syncthreads();
  finalize_v(g, ws, f, blockIdx.x, red, &nbs, part);
}

// Quantisation in one launch: blocks for Q rows first, then per (b, kv-head),
// last first, its K rows -- the reverse of the order the statistics pass read
// them.  A block takes up to kSubs consecutive sub-blocks of 256 threads (2048
// elements each: 16 rows of 128 channels, or the same at other D), their
// loads issued together before any is used.
constexpr int kSubs = 4;
// The first nfin blocks (D <= 128) are the value part of the finalize step,
// one per (b, kv-head): it needs only the V coding before it.
template <typename T>
__global__ __launch_bounds__(256) void k_quant(const T* __restrict__ Q, const T* __restrict__ K,
                                               Geom g, Fp4Ptrs f, QuantWs ws, int kpt, int qpb,
                                               int nq, int nfin) {
  int b = blockIdx.x;
  if (b < nfin) {
    __shared__ float red[16];
    __shared__ float nbs;
    __shared__ double part[256];
    finalize_v(g, ws, f, b, red, &nbs, part);
    return;
  }
  b -= nfin;
  uint4 raw[kSubs];
  int row[kSubs];
  if (b < nq) {
    const int bpq = (qpb + kSubs - 1) / kSubs;  // blocks per q-head
    const int bh = b / bpq, s0 = (b % bpq) * kSubs, ns = min(kSubs, qpb - s0);
#pragma unroll
    for (int i = 0; i < kSubs; ++i)
      raw[i] = i < ns ? load_row<T, true>(Q, g, s0 + i, bh, &row[i]) : uint4{0u, 0u, 0u, 0u};
    const RowConst rc = row_const<true>(g, f, bh);
#pragma unroll
    for (int i = 0; i < kSubs; ++i)
      if (i < ns) quant_rows<T, true>(raw[i], g, f, row[i], bh, rc);
    return;
  }
  b -= nq;
  // the head's sub-blocks [qt0 * kpt, qt1 * kpt) (16-row groups at D = 128),
  // kSubs consecutive ones per block, across tile boundaries
  const int s_lo = g.ct0 * kpt, s_hi = g.ct1 * kpt;
  const int per_head = (s_hi - s_lo + kSubs - 1) / kSubs;
  const int bh = g.B * g.Hkv - 1 - b / per_head;
  const int s0 = s_lo + (b % per_head) * kSubs;
  const int ns = min(kSubs, s_hi - s0);
#pragma unroll
  for (int i = 0; i < kSubs; ++i)
    raw[i] = i < ns ? load_row<T, false>(K, g, s0 + i, bh, &row[i]) : uint4{0u, 0u, 0u, 0u};
  const RowConst rc = row_const<false>(g, f, bh);
#pragma unroll
  for (int i = 0; i < kSubs; ++i)
    if (i < ns) quant_rows<T, false>(raw[i], g, f, row[i], bh, rc);
}

template <typename T>
hipError_t run_quantize(const Geom& g, const T* q, const T* k, const T* v, const Fp4Ptrs& f,
                        const QuantWs& ws, hipStream_t s) {
  const int nkvh = g.B * g.Hkv;
  const size_t stats_lds = 16 * (size_t)g.D * (sizeof(double) + 2 * sizeof(float));
  static bool stats_attr = false;  // above 64 KB (D = 512) the launch must opt in
  if (!stats_attr) {
    hipError_t e = hipFuncSetAttribute((const void*)k_stats<T>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 512 * 256);
    if (e != hipSuccess) return e;
    stats_attr = true;
  }
  const int nkb = g.Nkv > 0 ? (ws.ch1 - ws.ch0) * nkvh : 0;
  const int nvb = g.Nkv > 0 ? (g.ct1 - g.ct0 + kVTiles - 1) / kVTiles * ws.nvz * nkvh : 0;
  const int nqb = g.Nq > 0 && g.code_q ? ws.nqt * g.B * g.Hq : 0;
  if (nkb + nqb > 0)
    hipLaunchKernelGGL(k_stats<T>, dim3(nkb + nqb), dim3(min(2 * g.D, 512)), stats_lds, s, q, k,
                       g, ws, f, nkb);
  const int clear = nkb + nqb > 0 ? 0 : 1;
  // up to D = 128 the finalize parts ride in the V coding and K/Q coding launches
  const bool fuse = g.D <= 128;
  const int nfin = fuse ? nkvh : 0;
  if (nvb + nfin > 0)
    hipLaunchKernelGGL(k_vcode<T>, dim3(nvb + nfin), dim3(2 * min(g.D, 128)), 0, s, v, g, ws, f,
                       nfin, clear);
  if (!fuse)
    hipLaunchKernelGGL(k_finalize, dim3(nkvh), dim3(2 * g.D), 2 * g.D * sizeof(float), s, g, ws,
                       f, clear);
  // K rows: a 64-key tile of D channels is kTile * D / 8 threads, D / 32
  // sub-blocks of 256; Q: qpb sub-blocks per head
  const int kpt = g.D / 32;
  const int qpb = (int)(((long)g.NqP * (g.D / 8) + 255) / 256);
  const long nq = g.code_q ? (long)((qpb + kSubs - 1) / kSubs) * g.B * g.Hq : 0;
  const long nblk = nfin + nq + (long)nkvh * (((g.ct1 - g.ct0) * kpt + kSubs - 1) / kSubs);
  if (nblk > 0)
    hipLaunchKernelGGL(k_quant<T>, dim3((unsigned)nblk), dim3(256), 0, s, q, k, g, f, ws, kpt,
                       qpb, (int)nq, nfin);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const Geom& g, const void* q, const void* k, const void* v,
                           const Fp4Ptrs& f, const QuantWs& ws, hipStream_t s) {
  if (g.bf16)
    return run_quantize<uint16_t>(g, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                  f, ws, s);
  return run_quantize<_Float16>(g, (const _Float16*)q, (const _Float16*)k, (const _Float16*)v, f,
                                ws, s);
}

}  // namespace apa
