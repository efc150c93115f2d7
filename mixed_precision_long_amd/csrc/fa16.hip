// a8..a11: FP16 MFMA flash attention -- the exact pass 2 over compacted hot
// tiles with the fused log-sum-exp merge, the standalone merge, and the
// all-exact baseline.
//
// "APA: sloppy attention, exact where it counts" (rfriedmann.de): section
// "Pass 2: exact FP16 on the hot tiles" (a work group takes the rows of one
// pass-1 block, collects the union of their hot tiles, streams them from the
// original FP16 K and V, each wavefront computes only its own hot tiles with
// an FP32 online softmax and merges with its pass-1 state) and "The merge that
// makes it exact".  The introduction's all-exact baseline is the same core over
// every visible tile.
//
// Work group = (batch, kv-head, 64 query positions) x all G query heads of the
// group: 2G wavefronts of 32 rows each, so every K/V tile staged in LDS feeds
// all heads that share it.  Per wave and tile (D = 128):
//   S^T = K Q^T   16 MFMA 32x32x16 f16, K from LDS (row pad 16 B), Q resident;
//   softmax       scores sl*q.k - c_r in log2 units, FP32 running max/sum;
//   O^T += V^T P^T 16 MFMA 32x32x16 f16; P stays in the accumulator's lanes
//                 (its key order is matched by the V^T operand), V^T comes
//                 from LDS by DS_READ_B64_TR_B16 (row pad 64 B).
#include "apa_device.h"
#include "apa_kernels.h"

namespace apa {

namespace {

enum Mode { kExact = 0, kPass2 = 1 };

template <int D>
struct Lds {
  static constexpr int KS = D + 8;   // halves per K row (16-byte pad)
  static constexpr int VS = D + 32;  // halves per V row (64-byte pad)
  static constexpr int K_HALVES = kTile * KS;
  static constexpr int V_HALVES = kTile * VS;
  static constexpr int STAGE = K_HALVES + V_HALVES;
  static constexpr size_t BYTES = 2 * STAGE * sizeof(_Float16);
};

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void k_fa16(Geom g, const _Float16* __restrict__ Q,
                                                  const _Float16* __restrict__ K,
                                                  const _Float16* __restrict__ V, Fp4Ptrs f,
                                                  Pass2Args a, int nunits) {
  extern __shared__ _Float16 smem[];
  using L = Lds<D>;
  constexpr int NC = D / 16;          // 16-channel chunks of the QK contraction
  constexpr int ND = D / 32;          // 32-channel blocks of the output
  constexpr int CHUNKS = 2 * kTile * D / 8;           // 16-byte chunks per K+V tile
  constexpr int PER = (CHUNKS + NW * 64 - 1) / (NW * 64);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, hh = lane >> 5;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  if (unit >= nunits) return;  // uniform over the block
  const int nqb = (g.Nq + 63) / 64;
  const int qblk = unit % nqb;
  const int hk = (unit / nqb) % g.Hkv;
  const int b = unit / (nqb * g.Hkv);
  const int gi = wave >> 1, half = wave & 1;
  const int hq = hk * g.G + gi;
  const size_t bhq = (size_t)b * g.Hq + hq, bhk = (size_t)b * g.Hkv + hk;
  const int r0 = qblk * 64 + half * 32;
  const int row = r0 + n;
  const bool row_ok = row < g.Nq;
  const bool wave_live = r0 < g.Nq;
  auto diag = [&](int lr) { return g.causal ? min(g.Nkv - 1, lr + g.off) / kTile : g.NT - 1; };
  const int d_wave = wave_live ? diag(min(r0 + 31, g.Nq - 1)) : -1;

  // tile list
  int ntiles;
  const int32_t* tiles = nullptr;
  const uint32_t* masks = nullptr;
  if (MODE == kExact) {
    ntiles = diag(min(qblk * 64 + 63, g.Nq - 1)) + 1;
  } else {
    ntiles = a.list_count[unit];
    tiles = a.list_tiles + (size_t)unit * g.NT;
    masks = a.list_masks + (size_t)unit * g.NT;
  }

  // resident Q^T operand: 8 halves per 16-channel chunk
  v8h qf[NC];
  {
    const int rl = row_ok ? row : (g.Nq > 0 ? g.Nq - 1 : 0);
    const _Float16* qp = Q + ((bhq * g.Nq) + rl) * D + 8 * hh;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const v8h*>(qp + 16 * c);
  }
  const float c_r = (MODE == kPass2) ? f.q_frame[bhq * g.NqP + (row_ok ? row : 0)] : 0.0f;
  const float sl = g.sl;

  float m = -__builtin_inff(), l = 0.0f;
  v16f o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i)
    for (int j = 0; j < 16; ++j) o[i][j] = 0.0f;

  const _Float16* Kh = K + bhk * (size_t)g.Nkv * D;
  const _Float16* Vh = V + bhk * (size_t)g.Nkv * D;

  // cooperative staging: chunk c < CHUNKS/2 is K (row c / (D/8)), else V
  uint4 pre[PER];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NW * 64;
      uint4 z = {0u, 0u, 0u, 0u};
      if (c < CHUNKS) {
        const int isv = c >= CHUNKS / 2;
        const int cc = isv ? c - CHUNKS / 2 : c;
        const int r = cc / (D / 8), col = (cc % (D / 8)) * 8;
        const int key = t * kTile + r;
        if (key < g.Nkv) z = *reinterpret_cast<const uint4*>((isv ? Vh : Kh) + (size_t)key * D + col);
      }
      pre[i] = z;
    }
  };
  auto stash = [&](int buf) {
    _Float16* st = smem + buf * L::STAGE;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * NW * 64;
      if (c < CHUNKS) {
        const int isv = c >= CHUNKS / 2;
        const int cc = isv ? c - CHUNKS / 2 : c;
        const int r = cc / (D / 8), col = (cc % (D / 8)) * 8;
        _Float16* dst = isv ? st + L::K_HALVES + r * L::VS + col : st + r * L::KS + col;
        *reinterpret_cast<uint4*>(dst) = pre[i];
      }
    }
  };

  if (ntiles > 0) {
    fetch(MODE == kExact ? 0 : tiles[0]);
    stash(0);
  }
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int t = MODE == kExact ? it : tiles[it];
    const int buf = it & 1;
    if (it + 1 < ntiles) fetch(MODE == kExact ? it + 1 : tiles[it + 1]);

    // does this wave compute tile t, and for which of its two groups?
    bool on0, on1;
    if (MODE == kExact) {
      on0 = on1 = t <= d_wave;
    } else {
      const uint32_t mk = masks[it];
      const int bit = gi * 4 + half * 2;
      on0 = (mk >> bit) & 1u;
      on1 = (mk >> (bit + 1)) & 1u;
    }
    if (wave_live && (on0 || on1)) {
      const _Float16* Ks = smem + buf * L::STAGE;
      const _Float16* Vs = Ks + L::K_HALVES;
      const int k0 = t * kTile;
      // ---- S^T = K Q^T
      v16f acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[kb][j] = 0.0f;
        const _Float16* kr = Ks + (kb * 32 + n) * L::KS + 8 * hh;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const v8h kf = *reinterpret_cast<const v8h*>(kr + 16 * c);
          acc[kb] = mfma_f16(kf, qf[c], acc[kb]);
        }
      }
      // ---- scores in log2 units, masking
      const bool grp_on = (n >> 4) ? on1 : on0;
      const bool need_mask = (k0 + kTile > g.Nkv) || (g.causal && k0 + kTile - 1 > r0 + g.off) ||
                             (r0 + 31 >= g.Nq) || (on0 != on1);
      const int lim = g.causal ? row + g.off : 0x7fffffff;
      float tmax = -__builtin_inff();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float s = fmaf(acc[kb][j], sl, -c_r);
          if (need_mask) {
            const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            if (!(grp_on && row_ok && key < g.Nkv && key <= lim)) s = -__builtin_inff();
          }
          acc[kb][j] = s;
          tmax = vmax(tmax, s);
        }
      tmax = vmax(tmax, xor32(tmax));
      const float mnew = vmax(m, tmax);
      if (__ballot(mnew > m) != 0ull) {
        const float alpha = (mnew > m) ? fast_exp2(m - mnew) : 1.0f;  // m=-inf -> 0
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
          for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
        l *= alpha;
        m = mnew;
      }
      const float ms = m == -__builtin_inff() ? 0.0f : m;
      // ---- P (fp16) and its row sum
      v8h pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = fast_exp2(acc[kb][8 * c + j] - ms);
            l += p;
            pf[kb][c][j] = (_Float16)p;
          }
      // ---- O^T += V^T P^T
      const int G16 = lane >> 4, i16 = lane & 15;
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const int ch0 = db * 32 + 16 * (G16 & 1) + 4 * (i16 & 3);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int keyb = kb * 32 + 16 * c + 4 * (G16 >> 1) + (i16 >> 2);
            const _Float16* p0 = Vs + keyb * L::VS + ch0;
            const _Float16* p1 = p0 + 8 * L::VS;
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(p0));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(p1));
            const v8h vf = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = mfma_f16(vf, pf[kb][c], o[db]);
          }
      }
    }
    if (it + 1 < ntiles) stash(buf ^ 1);
    __syncthreads();
  }

  if (!wave_live) return;
  l += xor32(l);
  if (!row_ok) return;
  const size_t r = bhq * g.Nq + row;
  // ---- epilogue
  if (MODE == kPass2 && !a.fuse) {
    if (hh == 0) {
      a.hot_m[r] = l > 0.0f ? m : -__builtin_inff();
      a.hot_l[r] = l;
    }
    float* orow = a.hot_o + r * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4f x = {o[db][4 * q], o[db][4 * q + 1], o[db][4 * q + 2], o[db][4 * q + 3]};
        *reinterpret_cast<v4f*>(orow + db * 32 + 8 * q + 4 * hh) = x;
      }
    return;
  }
  float w1 = 0.0f, w2 = 0.0f, M = 0.0f, Lsum = 0.0f;
  const float* o1 = nullptr;
  if (MODE == kPass2) {
    const int m1i = a.cold_m[r];
    const float l1 = a.cold_l[r];
    const bool e1 = l1 > 0.0f && m1i != (int32_t)0x80000000, e2 = l > 0.0f;
    const float m1 = (float)m1i;
    M = -__builtin_inff();
    if (e1) M = m1;
    if (e2) M = fmaxf(M, m);
    w1 = e1 ? fast_exp2(m1 - M) : 0.0f;
    w2 = e2 ? fast_exp2(m - M) : 0.0f;
    Lsum = w1 * l1 + w2 * l;
    o1 = a.cold_o + r * D;
  } else {
    M = m;
    w2 = 1.0f;
    Lsum = l;
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  _Float16* orow = reinterpret_cast<_Float16*>(a.out) + r * D;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = db * 32 + 8 * q + 4 * hh;
      v4f c1 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (MODE == kPass2 && w1 != 0.0f) c1 = *reinterpret_cast<const v4f*>(o1 + ch);
      v4h y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (_Float16)((w1 * c1[e] + w2 * o[db][4 * q + e]) * inv);
      *reinterpret_cast<v4h*>(orow + ch) = y;
    }
  if (a.lse && hh == 0) {
    const float c0 = MODE == kPass2 ? c_r : 0.0f;
    a.lse[r] = Lsum > 0.0f ? 0.69314718055994531f * (c0 + M + __log2f(Lsum)) : -__builtin_inff();
  }
}

// Hot mask -> per work group list of the tiles hot for any of its 4G row
// groups, ascending, with a bit mask of the groups each tile is hot for
// (bit gi*4 + local group).  One wavefront per work group.
__global__ __launch_bounds__(64) void k_compact(Geom g, const uint32_t* __restrict__ bits,
                                                int32_t* tiles, uint32_t* masks, int32_t* count,
                                                int nunits) {
  const int unit = blockIdx.x;
  if (unit >= nunits) return;
  const int lane = threadIdx.x;
  const int nqb = (g.Nq + 63) / 64;
  const int qblk = unit % nqb;
  const int hk = (unit / nqb) % g.Hkv;
  const int b = unit / (nqb * g.Hkv);
  int base = 0;
  for (int w0 = 0; w0 < g.W; w0 += 64) {
    const int w = w0 + lane;
    uint32_t u = 0u;
    if (w < g.W) {
      for (int gi = 0; gi < g.G; ++gi) {
        const size_t bhq = (size_t)b * g.Hq + hk * g.G + gi;
        for (int lg = 0; lg < 4; ++lg) {
          const int grp = qblk * 4 + lg;
          if (grp < g.NG) u |= bits[(bhq * g.NG + grp) * g.W + w];
        }
      }
    }
    const int cnt = __popc(u);
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int pos = base + incl - cnt;
    uint32_t rem = u;
    while (rem) {
      const int bit = __ffs(rem) - 1;
      rem &= rem - 1u;
      const int t = w * 32 + bit;
      uint32_t mk = 0u;
      for (int gi = 0; gi < g.G; ++gi) {
        const size_t bhq = (size_t)b * g.Hq + hk * g.G + gi;
        for (int lg = 0; lg < 4; ++lg) {
          const int grp = qblk * 4 + lg;
          if (grp < g.NG && ((bits[(bhq * g.NG + grp) * g.W + w] >> bit) & 1u))
            mk |= 1u << (gi * 4 + lg);
        }
      }
      tiles[(size_t)unit * g.NT + pos] = t;
      masks[(size_t)unit * g.NT + pos] = mk;
      ++pos;
    }
    base += __shfl(incl, 63);
  }
  if (lane == 0) count[unit] = base;
}

// Standalone merge of the cold (pass-1) and hot (pass-2) states; one thread
// per (row, 4 channels).
template <int D>
__global__ void k_merge(Geom g, Fp4Ptrs f, const int32_t* __restrict__ cm,
                        const float* __restrict__ cl, const float* __restrict__ co,
                        const float* __restrict__ hm, const float* __restrict__ hl,
                        const float* __restrict__ ho, _Float16* out, float* lse, long nrows) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long r = gid / (D / 4);
  const int ch = (int)(gid % (D / 4)) * 4;
  if (r >= nrows) return;
  const int m1i = cm[r];
  const float l1 = cl[r], l2 = hl[r], m2 = hm[r];
  const bool e1 = l1 > 0.0f && m1i != (int32_t)0x80000000, e2 = l2 > 0.0f;
  float M = -__builtin_inff();
  if (e1) M = (float)m1i;
  if (e2) M = fmaxf(M, m2);
  const float w1 = e1 ? fast_exp2((float)m1i - M) : 0.0f;
  const float w2 = e2 ? fast_exp2(m2 - M) : 0.0f;
  const float Ls = w1 * l1 + w2 * l2;
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  v4f a = e1 ? *reinterpret_cast<const v4f*>(co + r * D + ch) : v4f{0, 0, 0, 0};
  v4f c = e2 ? *reinterpret_cast<const v4f*>(ho + r * D + ch) : v4f{0, 0, 0, 0};
  v4h y;
  for (int e = 0; e < 4; ++e) y[e] = (_Float16)((w1 * a[e] + w2 * c[e]) * inv);
  *reinterpret_cast<v4h*>(out + r * D + ch) = y;
  if (lse && ch == 0) {
    const long bh = r / g.Nq, rr = r % g.Nq;
    const float c0 = f.q_frame[bh * g.NqP + rr];
    lse[r] = Ls > 0.0f ? 0.69314718055994531f * (c0 + M + __log2f(Ls)) : -__builtin_inff();
  }
}

template <int D, int NW, int MODE>
hipError_t run_fa(const Geom& g, const void* q, const void* k, const void* v, const Fp4Ptrs& f,
                  const Pass2Args& a, hipStream_t s) {
  const int nunits = g.B * g.Hkv * ((g.Nq + 63) / 64);
  if (nunits == 0) return hipSuccess;
  auto kern = k_fa16<D, NW, MODE>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)Lds<D>::BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kern, dim3(nunits), dim3(NW * 64), Lds<D>::BYTES, s, g, (const _Float16*)q,
                     (const _Float16*)k, (const _Float16*)v, f, a, nunits);
  return hipGetLastError();
}

template <int MODE>
hipError_t dispatch(const Geom& g, const void* q, const void* k, const void* v, const Fp4Ptrs& f,
                    const Pass2Args& a, hipStream_t s) {
#define APA_FA_CASE(DD, GG)                                                   \
  if (g.D == DD && g.G == GG) return run_fa<DD, 2 * GG, MODE>(g, q, k, v, f, a, s);
#define APA_FA_D(DD) APA_FA_CASE(DD, 1) APA_FA_CASE(DD, 2) APA_FA_CASE(DD, 3) \
  APA_FA_CASE(DD, 4) APA_FA_CASE(DD, 6) APA_FA_CASE(DD, 8)
  APA_FA_D(64)
  APA_FA_D(128)
  APA_FA_D(256)
#undef APA_FA_D
#undef APA_FA_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_pass2(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a, hipStream_t s) {
  const int nunits = g.B * g.Hkv * ((g.Nq + 63) / 64);
  if (nunits == 0) return hipSuccess;
  hipLaunchKernelGGL(k_compact, dim3(nunits), dim3(64), 0, s, g, a.bits, a.list_tiles,
                     a.list_masks, a.list_count, nunits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dispatch<kPass2>(g, a.q, a.k, a.v, f, a, s);
}

hipError_t launch_exact(const Geom& g, const void* q, const void* k, const void* v, void* out,
                        float* lse, hipStream_t s) {
  Pass2Args a = {};
  a.out = out;
  a.lse = lse;
  Fp4Ptrs f = {};
  return dispatch<kExact>(g, q, k, v, f, a, s);
}

hipError_t launch_merge(const Geom& g, const Fp4Ptrs& f, const int32_t* cold_m,
                        const float* cold_l, const float* cold_o, const float* hot_m,
                        const float* hot_l, const float* hot_o, void* out, float* lse,
                        hipStream_t s) {
  const long nrows = (long)g.B * g.Hq * g.Nq;
  if (nrows == 0) return hipSuccess;
  const long thr = nrows * (g.D / 4);
  const unsigned nb = (unsigned)((thr + 255) / 256);
  switch (g.D) {
    case 64: hipLaunchKernelGGL(k_merge<64>, dim3(nb), dim3(256), 0, s, g, f, cold_m, cold_l, cold_o, hot_m, hot_l, hot_o, (_Float16*)out, lse, nrows); break;
    case 128: hipLaunchKernelGGL(k_merge<128>, dim3(nb), dim3(256), 0, s, g, f, cold_m, cold_l, cold_o, hot_m, hot_l, hot_o, (_Float16*)out, lse, nrows); break;
    case 256: hipLaunchKernelGGL(k_merge<256>, dim3(nb), dim3(256), 0, s, g, f, cold_m, cold_l, cold_o, hot_m, hot_l, hot_o, (_Float16*)out, lse, nrows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace apa
