// a8..a11: 16-bit MFMA flash attention -- the exact pass 2 over compacted hot
// tiles with the fused log-sum-exp merge, the standalone merge, and the
// all-exact baseline; fp16 or bf16 inputs.
//
// "APA: sloppy attention, exact where it counts" (rfriedmann.de): section
// "Pass 2: exact FP16 on the hot tiles" (a work group takes the rows of one
// pass-1 block, gathers the tiles hot for any of them, streams those from the
// original 16-bit K and V; a wavefront works only on tiles hot for its rows,
// with an FP32 online softmax, and combines the result with the cold state of
// pass 1) and "The merge that
// makes it exact".  The introduction's all-exact baseline is the same core over
// every visible tile.  Large head dimensions follow the FFPA documentation's
// interface (same layout and semantics at D = 512).
//
// Work group = (batch, kv-head, POS query positions) x all G query heads of the
// group: G*POS/32 wavefronts of 32 rows each, so every K/V tile staged in LDS
// feeds all heads that share it.  POS is 64 for D <= 256 (LDS double
// buffered, the next tile prefetched into registers) and 32 for D = 512 (one
// LDS stage; the output accumulators live in the accumulation registers).
// A unit's key range is cut into S splits that run as separate work groups
// when there are too few units to fill the chip; each split writes a partial
// online-softmax state and a combine kernel merges them in split order
// (deterministic).  Per wave and tile (D = 128):
//   S^T = K Q^T   16 MFMA 32x32x16, K from LDS (row pad 16 B), Q resident;
//   softmax       scores sl*q.k - c_r in log2 units, FP32 running max/sum;
//   O^T += V^T P^T 16 MFMA 32x32x16 f16; P stays in the accumulator's lanes
//                 (its key order is matched by the V^T operand), V^T comes
//                 from LDS by DS_READ_B64_TR_B16 (row pad 64 B).  With bf16
//                 inputs the scores use the bf16 MFMA and V is staged as fp16,
//                 so P keeps 11 significant bits.
#include <type_traits>

#include "apa_device.h"
#include "apa_kernels.h"

namespace apa {

namespace {

enum Mode { kExact = 0, kPass2 = 1 };

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));

// 16-bit element types: the MFMA and the conversions.
template <typename T>
struct E16;
template <>
struct E16<_Float16> {
  typedef v8h V8;
  typedef v4h V4;
  static __device__ __forceinline__ v16f mma(V8 a, V8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ _Float16 from(float x) { return (_Float16)x; }
};
template <>
struct E16<__bf16> {
  typedef v8bf V8;
  typedef v4bf V4;
  static __device__ __forceinline__ v16f mma(V8 a, V8 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ __bf16 from(float x) { return (__bf16)x; }
};

template <int D>
struct Cfg {
  static constexpr int POS = D >= 512 ? 32 : 64;  // query positions per work group
  static constexpr int STAGES = D >= 512 ? 1 : 2;
  static constexpr int KS = D + 8;    // halves per K row (16-byte pad)
  static constexpr int VS = D + 32;   // halves per V row (64-byte pad)
  static constexpr int K_HALVES = kTile * KS;
  static constexpr int V_HALVES = kTile * VS;
  static constexpr int STAGE = K_HALVES + V_HALVES;
  static constexpr size_t BYTES = (size_t)STAGES * STAGE * 2;
  static constexpr int CHUNKS = 2 * kTile * D / 8;  // 16-byte chunks per K+V tile
};

__device__ __forceinline__ float merge_weight(bool live, float m, float M) {
  return live ? fast_exp2(m - M) : 0.0f;
}

// bf16 values of V as fp16 for the P V product: exact inside the fp16 range
// (8 significant bits fit in 11); magnitudes beyond it are clamped to 65504.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 z) {
  const uint32_t w[4] = {z.x, z.y, z.z, z.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = fminf(fmaxf(__uint_as_float(w[i] << 16), -65504.0f), 65504.0f);
    const float hi = fminf(fmaxf(__uint_as_float(w[i] & 0xFFFF0000u), -65504.0f), 65504.0f);
    const _Float16 a = (_Float16)lo, b = (_Float16)hi;
    r[i] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
  return uint4{r[0], r[1], r[2], r[3]};
}

// Split s of n items out of `total` (balanced, contiguous).
__device__ __forceinline__ int split_lo(int total, int s, int S) {
  return (int)(((long long)total * s) / S);
}

template <int D, typename T, int MODE, int NW>
__device__ __forceinline__ void attn_body(const Geom& g, const T* __restrict__ Q,
                                          const T* __restrict__ K, const T* __restrict__ V,
                                          const Fp4Ptrs& f, const Pass2Args& a, int nunits,
                                          int S) {
  using C = Cfg<D>;
  using E = E16<T>;
  typedef typename E::V8 V8;
  typedef typename E::V4 V4;
  extern __shared__ uint16_t smem[];
  constexpr int POS = C::POS;
  constexpr int WPH = POS / 32;       // waves per head
  constexpr int GPU = POS / 16;       // 16-row groups per head and work group
  constexpr int NC = D / 16;          // 16-channel chunks of the QK contraction
  constexpr int ND = D / 32;          // 32-channel blocks of the output
  constexpr int PER = (C::CHUNKS + NW * 64 - 1) / (NW * 64);
  constexpr int RND = C::STAGES == 2 ? PER : (PER < 8 ? PER : 8);  // chunks per staging round

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int unit = xcd_remap(blockIdx.x, gridDim.x);
  if (unit >= nunits) return;  // uniform over the block
  const int nqb = (g.Nq + POS - 1) / POS;
  const int qblk = unit % nqb;
  int u = unit / nqb;
  const int sp = u % S; u /= S;
  const int hk = u % g.Hkv;
  const int b = u / g.Hkv;
  const int base_unit = (b * g.Hkv + hk) * nqb + qblk;
  const int gi = wave / WPH, half = wave % WPH;
  const int hq = hk * g.G + gi;
  const size_t bhq = (size_t)b * g.Hq + hq, bhk = (size_t)b * g.Hkv + hk;
  const int r0 = qblk * POS + half * 32;
  const int row = r0 + n;
  const bool row_ok = row < g.Nq;
  const bool wave_live = r0 < g.Nq;
  auto diag = [&](int lr) { return g.causal ? min(g.Nkv - 1, lr + g.off) / kTile : g.NT - 1; };
  const int d_wave = wave_live ? diag(min(r0 + 31, g.Nq - 1)) : -1;

  // this split's part of the unit's tile list
  int lo, hi;
  const int32_t* tiles = nullptr;
  const uint32_t* masks = nullptr;
  if (MODE == kExact) {
    const int ntot = diag(min(qblk * POS + POS - 1, g.Nq - 1)) + 1;
    lo = split_lo(ntot, sp, S);
    hi = split_lo(ntot, sp + 1, S);
  } else {
    const int ntot = a.list_count[base_unit];
    lo = split_lo(ntot, sp, S);
    hi = split_lo(ntot, sp + 1, S);
    tiles = a.list_tiles + (size_t)base_unit * g.NT;
    masks = a.list_masks + (size_t)base_unit * g.NT;
  }
  auto tile_at = [&](int it) { return MODE == kExact ? it : tiles[it]; };

  // resident Q^T operand: 8 elements per 16-channel chunk
  V8 qf[NC];
  {
    const int rl = row_ok ? row : (g.Nq > 0 ? g.Nq - 1 : 0);
    const T* qp = Q + ((bhq * g.Nq) + rl) * D + 8 * hh;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const V8*>(qp + 16 * c);
  }
  const float c_r = (MODE == kPass2) ? f.q_frame[bhq * g.NqP + (row_ok ? row : 0)] : 0.0f;
  const float sl = g.sl;

  float m = -__builtin_inff(), l = 0.0f;
  v16f o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = v16f{};

  const uint16_t* Kh = reinterpret_cast<const uint16_t*>(K) + bhk * (size_t)g.Nkv * D;
  const uint16_t* Vh = reinterpret_cast<const uint16_t*>(V) + bhk * (size_t)g.Nkv * D;

  // cooperative staging: chunk c < CHUNKS/2 is K (row c / (D/8)), else V
  auto fetch1 = [&](int t, int c) {
    uint4 z = {0u, 0u, 0u, 0u};
    if (c < C::CHUNKS) {
      const int isv = c >= C::CHUNKS / 2;
      const int cc = isv ? c - C::CHUNKS / 2 : c;
      const int r = cc / (D / 8), col = (cc % (D / 8)) * 8;
      const int key = t * kTile + r;
      if (key < g.Nkv) z = *reinterpret_cast<const uint4*>((isv ? Vh : Kh) + (size_t)key * D + col);
    }
    return z;
  };
  auto stash1 = [&](int buf, int c, uint4 z) {
    if (c < C::CHUNKS) {
      uint16_t* st = smem + buf * C::STAGE;
      const int isv = c >= C::CHUNKS / 2;
      if (std::is_same<T, __bf16>::value && isv) z = bf16x8_to_f16x8(z);
      const int cc = isv ? c - C::CHUNKS / 2 : c;
      const int r = cc / (D / 8), col = (cc % (D / 8)) * 8;
      uint16_t* dst = isv ? st + C::K_HALVES + r * C::VS + col : st + r * C::KS + col;
      *reinterpret_cast<uint4*>(dst) = z;
    }
  };
  uint4 pre[RND];
  auto fetch = [&](int t) {
#pragma unroll
    for (int i = 0; i < RND; ++i) pre[i] = fetch1(t, tid + i * NW * 64);
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RND; ++i) stash1(buf, tid + i * NW * 64, pre[i]);
  };
  // single-stage staging of a whole tile in rounds (large D)
  auto stage_all = [&](int t) {
    for (int r0c = 0; r0c < PER; r0c += RND) {
#pragma unroll
      for (int i = 0; i < RND; ++i) pre[i] = fetch1(t, tid + (r0c + i) * NW * 64);
#pragma unroll
      for (int i = 0; i < RND; ++i) stash1(0, tid + (r0c + i) * NW * 64, pre[i]);
    }
  };

  if (C::STAGES == 2 && lo < hi) {
    fetch(tile_at(lo));
    stash(0);
  }
  if (C::STAGES == 2) __syncthreads();

  for (int it = lo; it < hi; ++it) {
    const int t = tile_at(it);
    const int buf = C::STAGES == 2 ? ((it - lo) & 1) : 0;
    if (C::STAGES == 2) {
      if (it + 1 < hi) fetch(tile_at(it + 1));
    } else {
      __syncthreads();
      stage_all(t);
      __syncthreads();
    }

    // does this wave compute tile t, and for which of its two groups?
    bool on0, on1;
    if (MODE == kExact) {
      on0 = on1 = t <= d_wave;
    } else {
      const uint32_t mk = masks[it];
      const int bit = gi * GPU + half * 2;
      on0 = (mk >> bit) & 1u;
      on1 = (mk >> (bit + 1)) & 1u;
    }
    if (wave_live && (on0 || on1)) {
      const uint16_t* Ks = smem + buf * C::STAGE;
      const uint16_t* Vs = Ks + C::K_HALVES;
      const int k0 = t * kTile;
      // ---- S^T = K Q^T
      v16f acc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        acc[kb] = v16f{};
        const uint16_t* kr = Ks + (kb * 32 + n) * C::KS + 8 * hh;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const V8 kf = *reinterpret_cast<const V8*>(kr + 16 * c);
          acc[kb] = E::mma(kf, qf[c], acc[kb]);
        }
      }
      // ---- scores in log2 units, masking
      const bool grp_on = (n >> 4) ? on1 : on0;
      const bool need_mask = (k0 + kTile > g.Nkv) || (g.causal && k0 + kTile - 1 > r0 + g.off) ||
                             (r0 + 31 >= g.Nq) || (on0 != on1);
      const int lim = g.causal ? row + g.off : 0x7fffffff;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[kb][j] = fmaf(acc[kb][j], sl, -c_r);
      if (need_mask) {  // wave-uniform: diagonal, padding and half-masked tiles only
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            if (!(grp_on && row_ok && key < g.Nkv && key <= lim)) acc[kb][j] = -__builtin_inff();
          }
      }
      float tmax = vmax(acc[0][0], acc[0][1]);
#pragma unroll
      for (int j = 2; j < 16; j += 2) tmax = vmax3(tmax, acc[0][j], acc[0][j + 1]);
#pragma unroll
      for (int j = 0; j < 16; j += 2) tmax = vmax3(tmax, acc[1][j], acc[1][j + 1]);
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
      // ---- P (fp16, also for bf16 inputs: 11 significant bits) and its row sum
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
            const uint16_t* p0 = Vs + keyb * C::VS + ch0;
            const uint16_t* p1 = p0 + 8 * C::VS;
            const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(p0));
            const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s*)(p1));
            const v8h vf = __builtin_bit_cast(v8h, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = mfma_f16(vf, pf[kb][c], o[db]);
          }
      }
    }
    if (C::STAGES == 2) {
      if (it + 1 < hi) stash(buf ^ 1);
      __syncthreads();
    }
  }

  if (!wave_live) return;
  l += xor32(l);
  if (!row_ok) return;
  const size_t r = bhq * g.Nq + row;
  const size_t rows = (size_t)g.B * g.Hq * g.Nq;

  // ---- partial state of one split (merged by k_combine)
  if (S > 1 || (MODE == kPass2 && !a.fuse)) {
    float* pm = S > 1 ? a.part_m + (size_t)sp * rows : a.hot_m;
    float* pl = S > 1 ? a.part_l + (size_t)sp * rows : a.hot_l;
    float* po = S > 1 ? a.part_o + (size_t)sp * rows * D : a.hot_o;
    if (hh == 0) {
      pm[r] = l > 0.0f ? m : -__builtin_inff();
      pl[r] = l;
    }
    float* orow = po + r * D;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4f x = {o[db][4 * q], o[db][4 * q + 1], o[db][4 * q + 2], o[db][4 * q + 3]};
        *reinterpret_cast<v4f*>(orow + db * 32 + 8 * q + 4 * hh) = x;
      }
    return;
  }
  // ---- one split: output directly (pass 2: merged with the cold state)
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
    w1 = merge_weight(e1, m1, M);
    w2 = merge_weight(e2, m, M);
    Lsum = w1 * l1 + w2 * l;
    o1 = a.cold_o + r * D;
  } else {
    M = m;
    w2 = 1.0f;
    Lsum = l;
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  T* orow = reinterpret_cast<T*>(a.out) + r * D;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = db * 32 + 8 * q + 4 * hh;
      v4f c1 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (MODE == kPass2 && w1 != 0.0f) c1 = *reinterpret_cast<const v4f*>(o1 + ch);
      V4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = E::from((w1 * c1[e] + w2 * o[db][4 * q + e]) * inv);
      *reinterpret_cast<V4*>(orow + ch) = y;
    }
  if (a.lse && hh == 0) {
    const float c0 = MODE == kPass2 ? c_r : 0.0f;
    a.lse[r] = Lsum > 0.0f ? 0.69314718055994531f * (c0 + M + __log2f(Lsum)) : -__builtin_inff();
  }
}

template <int D, typename T, int MODE, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn(Geom g, const T* __restrict__ Q,
                                                  const T* __restrict__ K,
                                                  const T* __restrict__ V, Fp4Ptrs f, Pass2Args a,
                                                  int nunits, int S) {
  attn_body<D, T, MODE, NW>(g, Q, K, V, f, a, nunits, S);
}

// D = 512: one wave per SIMD, so the 256 output accumulators per lane can sit
// in the accumulation registers beside the resident Q operand.
template <int D, typename T, int MODE, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attn_big(
    Geom g, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, Fp4Ptrs f,
    Pass2Args a, int nunits, int S) {
  attn_body<D, T, MODE, NW>(g, Q, K, V, f, a, nunits, S);
}

// Hot mask -> per unit (batch, kv-head, POS positions) list of the tiles hot
// for any of its G*POS/16 row groups, ascending, with a bit mask of the groups
// each tile is hot for (bit gi*POS/16 + local group).  One wavefront per unit.
__global__ __launch_bounds__(64) void k_compact(Geom g, int pos, const uint32_t* __restrict__ bits,
                                                int32_t* tiles, uint32_t* masks, int32_t* count,
                                                int nunits) {
  const int unit = blockIdx.x;
  if (unit >= nunits) return;
  const int lane = threadIdx.x;
  const int gpu = pos / 16;
  const int nqb = (g.Nq + pos - 1) / pos;
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
        for (int lg = 0; lg < gpu; ++lg) {
          const int grp = qblk * gpu + lg;
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
    int pos_out = base + incl - cnt;
    uint32_t rem = u;
    while (rem) {
      const int bit = __ffs(rem) - 1;
      rem &= rem - 1u;
      const int t = w * 32 + bit;
      uint32_t mk = 0u;
      for (int gi = 0; gi < g.G; ++gi) {
        const size_t bhq = (size_t)b * g.Hq + hk * g.G + gi;
        for (int lg = 0; lg < gpu; ++lg) {
          const int grp = qblk * gpu + lg;
          if (grp < g.NG && ((bits[(bhq * g.NG + grp) * g.W + w] >> bit) & 1u))
            mk |= 1u << (gi * gpu + lg);
        }
      }
      tiles[(size_t)unit * g.NT + pos_out] = t;
      masks[(size_t)unit * g.NT + pos_out] = mk;
      ++pos_out;
    }
    base += __shfl(incl, 63);
  }
  if (lane == 0) count[unit] = base;
}

// The merge of a cold (pass-1) state (m1 integer frame, l1, o1) and a hot
// state (m2, l2, o2) for 4 channels: shared by the standalone merge and the
// split combine so both round identically.
template <typename T>
__device__ __forceinline__ void merge4(int m1i, float l1, v4f a1, float m2, float l2, v4f a2,
                                       float c0, T* out, float* lse_out) {
  typedef typename E16<T>::V4 V4;
  const bool e1 = l1 > 0.0f && m1i != (int32_t)0x80000000, e2 = l2 > 0.0f;
  float M = -__builtin_inff();
  if (e1) M = (float)m1i;
  if (e2) M = fmaxf(M, m2);
  const float w1 = merge_weight(e1, (float)m1i, M);
  const float w2 = merge_weight(e2, m2, M);
  const float Ls = w1 * l1 + w2 * l2;
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  if (!e1) a1 = v4f{0, 0, 0, 0};
  if (!e2) a2 = v4f{0, 0, 0, 0};
  V4 y;
  for (int e = 0; e < 4; ++e) y[e] = E16<T>::from((w1 * a1[e] + w2 * a2[e]) * inv);
  *reinterpret_cast<V4*>(out) = y;
  if (lse_out)
    *lse_out = Ls > 0.0f ? 0.69314718055994531f * (c0 + M + __log2f(Ls)) : -__builtin_inff();
}

// Standalone merge of the cold and hot states; one thread per (row, 4 channels).
template <int D, typename T>
__global__ void k_merge(Geom g, Fp4Ptrs f, const int32_t* __restrict__ cm,
                        const float* __restrict__ cl, const float* __restrict__ co,
                        const float* __restrict__ hm, const float* __restrict__ hl,
                        const float* __restrict__ ho, T* out, float* lse, long nrows) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long r = gid / (D / 4);
  const int ch = (int)(gid % (D / 4)) * 4;
  if (r >= nrows) return;
  const float l1 = cl[r], l2 = hl[r];
  const v4f a1 = l1 > 0.0f ? *reinterpret_cast<const v4f*>(co + r * D + ch) : v4f{0, 0, 0, 0};
  const v4f a2 = l2 > 0.0f ? *reinterpret_cast<const v4f*>(ho + r * D + ch) : v4f{0, 0, 0, 0};
  const long bh = r / g.Nq, rr = r % g.Nq;
  const float c0 = (lse && ch == 0) ? f.q_frame[bh * g.NqP + rr] : 0.0f;
  merge4<T>(cm[r], l1, a1, hm[r], l2, a2, c0, out + r * D + ch,
            (lse && ch == 0) ? lse + r : nullptr);
}

// Combine the S split states of each row (in split order), then: exact ->
// output; pass 2 fused -> merge with the cold state; pass 2 unfused -> the hot
// state.  One thread per (row, 4 channels).
template <int D, typename T, int MODE>
__global__ void k_combine(Geom g, Fp4Ptrs f, Pass2Args a, int S, long nrows) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long r = gid / (D / 4);
  const int ch = (int)(gid % (D / 4)) * 4;
  if (r >= nrows) return;
  float Mh = -__builtin_inff();
  for (int s = 0; s < S; ++s)
    if (a.part_l[s * nrows + r] > 0.0f) Mh = fmaxf(Mh, a.part_m[s * nrows + r]);
  float Lh = 0.0f;
  v4f oh = {0, 0, 0, 0};
  for (int s = 0; s < S; ++s) {
    const float ls = a.part_l[s * nrows + r];
    if (ls > 0.0f) {
      const float w = fast_exp2(a.part_m[s * nrows + r] - Mh);
      Lh += w * ls;
      const v4f x = *reinterpret_cast<const v4f*>(a.part_o + (s * nrows + r) * D + ch);
      for (int e = 0; e < 4; ++e) oh[e] += w * x[e];
    }
  }
  const bool want_lse = a.lse && ch == 0;
  if (MODE == kExact) {
    // the state alone: same arithmetic as a merge with an empty cold state
    merge4<T>((int32_t)0x80000000, 0.0f, v4f{0, 0, 0, 0}, Mh, Lh, oh, 0.0f,
              reinterpret_cast<T*>(a.out) + r * D + ch, want_lse ? a.lse + r : nullptr);
    return;
  }
  if (!a.fuse) {
    if (ch == 0) {
      a.hot_m[r] = Lh > 0.0f ? Mh : -__builtin_inff();
      a.hot_l[r] = Lh;
    }
    *reinterpret_cast<v4f*>(a.hot_o + r * D + ch) = oh;
    return;
  }
  const float l1 = a.cold_l[r];
  const v4f a1 = l1 > 0.0f ? *reinterpret_cast<const v4f*>(a.cold_o + r * D + ch) : v4f{0, 0, 0, 0};
  const long bh = r / g.Nq, rr = r % g.Nq;
  const float c0 = want_lse ? f.q_frame[bh * g.NqP + rr] : 0.0f;
  merge4<T>(a.cold_m[r], l1, a1, Lh > 0.0f ? Mh : -__builtin_inff(), Lh, oh, c0,
            reinterpret_cast<T*>(a.out) + r * D + ch, want_lse ? a.lse + r : nullptr);
}

template <int D, typename T, int MODE, int NW>
hipError_t run_attn(const Geom& g, const void* q, const void* k, const void* v, const Fp4Ptrs& f,
                    const Pass2Args& a, int S, hipStream_t s) {
  const int nunits = g.B * g.Hkv * ((g.Nq + Cfg<D>::POS - 1) / Cfg<D>::POS) * S;
  if (nunits == 0) return hipSuccess;
  void (*kern)(Geom, const T*, const T*, const T*, Fp4Ptrs, Pass2Args, int, int);
  if constexpr (D >= 512) kern = k_attn_big<D, T, MODE, NW>;
  else kern = k_attn<D, T, MODE, NW>;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)Cfg<D>::BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL(kern, dim3(nunits), dim3(NW * 64), Cfg<D>::BYTES, s, g, (const T*)q,
                     (const T*)k, (const T*)v, f, a, nunits, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const long nrows = (long)g.B * g.Hq * g.Nq;
  const long thr = nrows * (D / 4);
  hipLaunchKernelGGL((k_combine<D, T, MODE>), dim3((unsigned)((thr + 255) / 256)), dim3(256), 0, s,
                     g, f, a, S, nrows);
  return hipGetLastError();
}

template <int MODE, typename T>
hipError_t dispatch_t(const Geom& g, const void* q, const void* k, const void* v,
                      const Fp4Ptrs& f, const Pass2Args& a, int S, hipStream_t s) {
#define APA_FA_CASE(DD, GG)                                                              \
  if (g.D == DD && g.G == GG)                                                            \
    return run_attn<DD, T, MODE, GG * Cfg<DD>::POS / 32>(g, q, k, v, f, a, S, s);
#define APA_FA_D(DD) APA_FA_CASE(DD, 1) APA_FA_CASE(DD, 2) APA_FA_CASE(DD, 3) \
  APA_FA_CASE(DD, 4) APA_FA_CASE(DD, 6) APA_FA_CASE(DD, 8)
  APA_FA_D(64)
  APA_FA_D(128)
  APA_FA_D(256)
  APA_FA_D(512)
#undef APA_FA_D
#undef APA_FA_CASE
  return hipErrorInvalidValue;
}

template <int MODE>
hipError_t dispatch(const Geom& g, const void* q, const void* k, const void* v, const Fp4Ptrs& f,
                    const Pass2Args& a, int S, hipStream_t s) {
  return g.bf16 ? dispatch_t<MODE, __bf16>(g, q, k, v, f, a, S, s)
                : dispatch_t<MODE, _Float16>(g, q, k, v, f, a, S, s);
}

}  // namespace

int attn_positions(int D) { return D >= 512 ? 32 : 64; }

int attn_splits(const Geom& g) {
  const int pos = attn_positions(g.D);
  const long units = (long)g.B * g.Hkv * ((g.Nq + pos - 1) / pos);
  if (units <= 0) return 1;
  // one work group per compute unit of the 256-CU part (the register use of
  // the D <= 256 kernels allows one resident group of G*POS/32 waves per CU)
  long S = (256 + units - 1) / units;
  if (S > 8) S = 8;
  // at least 4 tiles per split of the longest key range
  long maxs = g.NT / 4;
  if (maxs < 1) maxs = 1;
  if (S > maxs) S = maxs;
  return (int)(S < 1 ? 1 : S);
}

hipError_t launch_pass2(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a, hipStream_t s) {
  const int pos = attn_positions(g.D);
  const int nunits = g.B * g.Hkv * ((g.Nq + pos - 1) / pos);
  if (nunits == 0) return hipSuccess;
  hipLaunchKernelGGL(k_compact, dim3(nunits), dim3(64), 0, s, g, pos, a.bits, a.list_tiles,
                     a.list_masks, a.list_count, nunits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dispatch<kPass2>(g, a.q, a.k, a.v, f, a, attn_splits(g), s);
}

hipError_t launch_exact(const Geom& g, const void* q, const void* k, const void* v, void* out,
                        float* lse, const Pass2Args& parts, hipStream_t s) {
  Pass2Args a = parts;
  a.out = out;
  a.lse = lse;
  Fp4Ptrs f = {};
  return dispatch<kExact>(g, q, k, v, f, a, attn_splits(g), s);
}

hipError_t launch_merge(const Geom& g, const Fp4Ptrs& f, const int32_t* cold_m,
                        const float* cold_l, const float* cold_o, const float* hot_m,
                        const float* hot_l, const float* hot_o, void* out, float* lse,
                        hipStream_t s) {
  const long nrows = (long)g.B * g.Hq * g.Nq;
  if (nrows == 0) return hipSuccess;
  const long thr = nrows * (g.D / 4);
  const unsigned nb = (unsigned)((thr + 255) / 256);
#define APA_MERGE(DD, TT)                                                                      \
  hipLaunchKernelGGL((k_merge<DD, TT>), dim3(nb), dim3(256), 0, s, g, f, cold_m, cold_l, cold_o, \
                     hot_m, hot_l, hot_o, (TT*)out, lse, nrows);                               \
  break;
  if (g.bf16) {
    switch (g.D) {
      case 64: APA_MERGE(64, __bf16)
      case 128: APA_MERGE(128, __bf16)
      case 256: APA_MERGE(256, __bf16)
      case 512: APA_MERGE(512, __bf16)
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (g.D) {
      case 64: APA_MERGE(64, _Float16)
      case 128: APA_MERGE(128, _Float16)
      case 256: APA_MERGE(256, _Float16)
      case 512: APA_MERGE(512, _Float16)
      default: return hipErrorInvalidValue;
    }
  }
#undef APA_MERGE
  return hipGetLastError();
}

}  // namespace apa
