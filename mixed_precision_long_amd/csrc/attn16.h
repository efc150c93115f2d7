// Shared pieces of the 16-bit MFMA attention kernels (the exact pass 2 over
// hot tiles, its merge, and the all-exact baseline): element types, the row
// blocks a work group takes, the split bookkeeping and the epilogue.
//
// "APA: sloppy attention, exact where it counts" (rfriedmann.de): section
// "Pass 2: exact FP16 on the hot tiles" and "The merge that makes it exact".
#pragma once

#include <type_traits>

#include "apa_device.h"
#include "apa_kernels.h"

namespace apa {

namespace {

enum Mode { kExact = 0, kPass2 = 1 };

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

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

// Row blocks of one (batch, kv-head) and the work groups over them.
struct RowBlocks {
  int nqb;  // 32-position blocks
  int nrb;  // row blocks (G per position block)
  int nwg;  // work groups of four row blocks
};

__host__ __device__ inline RowBlocks row_blocks(const Geom& g) {
  RowBlocks r;
  r.nqb = (g.Nq + 31) / 32;
  r.nrb = g.G * r.nqb;
  r.nwg = (r.nrb + 3) / 4;
  return r;
}

constexpr int kWgWaves = 4;      // wavefronts per work group (one row block each)
constexpr float kLazy = 8.0f;    // lead (log2 units) a row maximum needs to move m

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

// The row block of wave `wave` in work group `wg`: its head in the group and
// its first query position; live = false past the last row block.
struct WaveRows {
  bool live;
  int gi, r0;
};

__device__ __forceinline__ WaveRows wave_rows(const Geom& g, const RowBlocks& rb, int wg, int wave) {
  const int j = wg * kWgWaves + wave;
  WaveRows w;
  w.live = j < rb.nrb;
  w.gi = w.live ? j % g.G : 0;
  w.r0 = w.live ? (j / g.G) * 32 : 0;
  return w;
}

// The key tiles a work group visits in exact mode: up to the diagonal of its
// last live row.
__device__ __forceinline__ int exact_tiles(const Geom& g, const RowBlocks& rb, int wg) {
  const int jl = min(wg * kWgWaves + kWgWaves - 1, rb.nrb - 1);
  const int lr = min((jl / g.G) * 32 + 31, g.Nq - 1);
  return g.causal ? min(g.Nkv - 1, lr + g.off) / kTile + 1 : g.NT;
}

// The epilogue shared by both kernels: a split's partial state (S > 1 or an
// unfused pass 2), else the output -- merged with the cold state in pass 2.
// Lane (n, hh) holds row n's output channels ch0 + 32*db + 8*q + 4*hh + 0..3
// in o[db][4q .. 4q+3] for db < ND (all D channels, or the share of a wave
// that holds part of them); l is already summed over both lane halves.  The
// row scalars (partial m and l, LSE) are written when `scalars` is set.
template <int D, typename T, int MODE, int ND = D / 32>
__device__ __forceinline__ void finish_row(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a,
                                           int S, int sp, size_t bhq, int row, int hh, float m,
                                           float l, float c_r, const v16f* o, int ch0 = 0,
                                           bool scalars = true) {
  using E = E16<T>;
  typedef typename E::V4 V4;
  const size_t r = bhq * g.Nq + row;
  const size_t rows = (size_t)g.B * g.Hq * g.Nq;
  if (S > 1 || (MODE == kPass2 && !a.fuse)) {
    float* pm = S > 1 ? a.part_m + (size_t)sp * rows : a.hot_m;
    float* pl = S > 1 ? a.part_l + (size_t)sp * rows : a.hot_l;
    float* po = S > 1 ? a.part_o + (size_t)sp * rows * D : a.hot_o;
    if (hh == 0 && scalars) {
      pm[r] = l > 0.0f ? m : -__builtin_inff();
      pl[r] = l;
    }
    float* orow = po + r * D + ch0;
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
    w1 = merge_weight(e1, m1, M);
    w2 = merge_weight(e2, m, M);
    Lsum = w1 * l1 + w2 * l;
    o1 = a.cold_o + r * D + ch0;
  } else {
    M = m;
    w2 = 1.0f;
    Lsum = l;
  }
  const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
  T* orow = reinterpret_cast<T*>(a.out) + r * D + ch0;
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
  if (a.lse && hh == 0 && scalars) {
    const float c0 = MODE == kPass2 ? c_r : 0.0f;
    a.lse[r] = Lsum > 0.0f ? 0.69314718055994531f * (c0 + M + __log2f(Lsum)) : -__builtin_inff();
  }
}


}  // namespace

// The 16-bit core at D = 512 (defined with its kernel): launches the work
// groups of S key splits per unit for the problem's element type; mode 0 the
// exact baseline, 1 pass 2 over the compacted hot tiles.  The split states, if
// S > 1, are combined by the caller.
hipError_t launch_attn_big(const Geom& g, const void* q, const void* k, const void* v,
                           const Fp4Ptrs& f, const Pass2Args& a, int S, int mode, hipStream_t s);

}  // namespace apa
