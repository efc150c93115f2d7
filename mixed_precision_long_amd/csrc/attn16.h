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
// Memory a kernel only reads and that no wave writes while it runs (the
// compacted tile lists of pass 2, written by an earlier launch): reads through
// the constant address space become scalar loads, which wait on their own
// counter instead of the vector-memory counter that also tracks the
// LDS-writing tile loads in flight.
typedef __attribute__((address_space(4))) const int32_t cint32;
typedef __attribute__((address_space(4))) const uint32_t cuint32;

// Buffer resources over one key tile's 64 rows of a 16-bit K or V input
// (flat, or the tile's page with a block table; the page index is a scalar
// load) and the byte offset of key `key` (a key of tile t) inside it.
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Geom& g, const T* X, int b,
                                                            int hk, int t) {
  size_t e;
  if (g.bt) {
    const int pg = ((const cint32*)g.bt)[(size_t)b * g.bts + t];
    e = ((size_t)pg * g.Hkv + hk) * 64 * g.D;
  } else {
    e = (((size_t)b * g.Hkv + hk) * g.Nkv + (size_t)t * 64) * g.D;
  }
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(X) + e, (short)0, 64 * g.D * 2,
                                           0x00020000);
}

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

// The power of two 2^s by which a kv-head's bf16 V is divided so that its
// largest magnitude amax fits the fp16 range: s = 0 up to 65504, else with
// amax = f 2^x (f in [0.5, 1); a bf16 value has f <= 1 - 2^-8), s = x - 16
// brings it to f 2^16 <= 65280.  Non-finite amax (flagged by the status
// word) gives 0.
__device__ __forceinline__ int v_shift(float amax) {
  if (!(amax > 65504.0f) || !(amax < __builtin_inff())) return 0;
  int x;
  (void)frexpf(amax, &x);
  return x - 16;
}

// bf16 values of V times 2^-s (down = 2^-s, s from v_shift) as fp16 for the
// P V product: exact in the fp16 normal range (8 significant bits fit in 11);
// below 2^-14 the fp16 subnormal spacing 2^-24 bounds the rounding.  The
// product is scaled back by 2^s in the epilogue.
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 z, float down) {
  const uint32_t w[4] = {z.x, z.y, z.z, z.w};
  uint32_t r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(w[i] << 16) * down;
    const float hi = __uint_as_float(w[i] & 0xFFFF0000u) * down;
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

// The first key tile a row from `first_row` on sees with a sliding window
// (row r sees keys r + off - window < k <= r + off); 0 without one.
__host__ __device__ inline int window_lo(const Geom& g, int first_row) {
  const int first_key = first_row + g.off - g.window + 1;
  return g.causal && g.window > 0 && first_key > 0 ? first_key / kTile : 0;
}

// The key tiles a work group visits in exact mode: up to the diagonal of its
// last live row (from window_lo of its first row).
__device__ __forceinline__ int exact_tiles(const Geom& g, const RowBlocks& rb, int wg) {
  const int jl = min(wg * kWgWaves + kWgWaves - 1, rb.nrb - 1);
  const int lr = min((jl / g.G) * 32 + 31, g.Nq - 1);
  return g.causal ? min(g.Nkv - 1, lr + g.off) / kTile + 1 : g.NT;
}

// The largest |V| of a kv-head for the bf16 conversion: from the FP4
// buffer's per-head statistics in pass 2, from the exact path's chunk
// maxima otherwise (nullptr for fp16 inputs, where it is not needed).
__device__ __forceinline__ float head_vamax(const Fp4Ptrs& f, const Pass2Args& a, size_t bhk,
                                            int mode_pass2) {
  if (mode_pass2) return f.kv_head[bhk * 8 + 3];
  float m = 0.0f;
  for (int c = 0; c < a.vmax_nch; ++c) m = fmaxf(m, a.vmax[bhk * a.vmax_nch + c]);
  return m;
}

// Loads and stores of split and cold states.  COH: device-coherent (relaxed
// agent-scope atomics, which bypass the per-XCD caches), for states another
// work group of the same launch writes or reads; plain accesses otherwise.
template <bool COH>
__device__ __forceinline__ float ldf(const float* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool COH>
__device__ __forceinline__ int32_t ldi(const int32_t* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}
template <bool COH>
__device__ __forceinline__ v4f ld4(const float* p) {
  if constexpr (COH) return v4f{ldf<true>(p), ldf<true>(p + 1), ldf<true>(p + 2), ldf<true>(p + 3)};
  return *reinterpret_cast<const v4f*>(p);
}
template <bool COH>
__device__ __forceinline__ void stf(float* p, float v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ void st4(float* p, v4f v) {
  if constexpr (COH) {
#pragma unroll
    for (int e = 0; e < 4; ++e) stf<true>(p + e, v[e]);
  } else {
    *reinterpret_cast<v4f*>(p) = v;
  }
}

// 16-byte device-coherent accesses (cache policy SC1: agent scope, as the
// relaxed atomics above) through a buffer resource over one 32-row block of
// a [rows][D] float array (base: the block's first row; offsets in bytes).
constexpr int kCpolSc1 = 16;
typedef unsigned v4u __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rowblock_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, 32 * D * 4,
                                           0x00020000);
}
__device__ __forceinline__ v4f coh_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCpolSc1));
}
__device__ __forceinline__ void coh_st4(__amdgpu_buffer_rsrc_t r, uint32_t off, v4f v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, v), r, off, 0, kCpolSc1);
}

// The epilogue shared by both kernels: a split's partial state (S > 1 or an
// unfused pass 2), else the output -- merged with the cold state in pass 2.
// Lane (n, hh) holds row n's output channels ch0 + 32*db + 8*q + 4*hh + 0..3
// in o[db][4q .. 4q+3] for db < ND (all D channels, or the share of a wave
// that holds part of them); l is already summed over both lane halves.  The
// row scalars (partial m and l, LSE) are written when `scalars` is set.  o is
// in units of 2^-vsh (bf16 V scaled into the fp16 range), scaled back here.
template <int D, typename T, int MODE, int ND = D / 32, bool COH = false>
__device__ __forceinline__ void finish_row(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a,
                                           int S, int sp, size_t bhq, int row, int hh, float m,
                                           float l, float c_r, const v16f* o, int vsh,
                                           int ch0 = 0, bool scalars = true) {
  const float up = __int_as_float((vsh + 127) << 23);  // 2^vsh, vsh in [0, 112]
  using E = E16<T>;
  typedef typename E::V4 V4;
  const size_t r = bhq * g.Nq + row;
  const size_t rows = (size_t)g.B * g.Hq * g.Nq;
  if (S > 1 || (MODE == kPass2 && !a.fuse)) {
    float* pm = S > 1 ? a.part_m + (size_t)sp * rows : a.hot_m;
    float* pl = S > 1 ? a.part_l + (size_t)sp * rows : a.hot_l;
    float* po = S > 1 ? a.part_o + (size_t)sp * rows * D : a.hot_o;
    if (hh == 0 && scalars) {
      stf<COH>(pm + r, l > 0.0f ? m : -__builtin_inff());
      stf<COH>(pl + r, l);
    }
    float* orow = po + r * D + ch0;
    // COH: the row block's region (the wave's rows are one 32-row block)
    const int n = threadIdx.x & 31;
    const int r0w = COH ? __builtin_amdgcn_readfirstlane(row - n) : 0;
    const auto rs = rowblock_rsrc<D>(po + (bhq * g.Nq + r0w) * D + ch0);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4f x = {o[db][4 * q] * up, o[db][4 * q + 1] * up, o[db][4 * q + 2] * up,
                 o[db][4 * q + 3] * up};
        if constexpr (COH)
          coh_st4(rs, (uint32_t)((n * D + db * 32 + 8 * q + 4 * hh) * 4), x);
        else
          *reinterpret_cast<v4f*>(orow + db * 32 + 8 * q + 4 * hh) = x;
      }
    return;
  }
  float w1 = 0.0f, w2 = 0.0f, M = 0.0f, Lsum = 0.0f;
  const float* o1 = nullptr;
  if (MODE == kPass2) {
    const int m1i = ldi<COH>(a.cold_m + r);
    const float l1 = ldf<COH>(a.cold_l + r);
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
  w2 *= up;  // exact: a power of two
  T* orow = reinterpret_cast<T*>(a.out) + r * D + ch0;
#pragma unroll
  for (int db = 0; db < ND; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = db * 32 + 8 * q + 4 * hh;
      v4f c1 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (MODE == kPass2 && w1 != 0.0f) {
        if constexpr (COH) {
          const int n = threadIdx.x & 31;
          const int r0w = __builtin_amdgcn_readfirstlane(row - n);
          c1 = coh_ld4(rowblock_rsrc<D>(a.cold_o + (bhq * g.Nq + r0w) * D + ch0),
                       (uint32_t)((n * D + ch) * 4));
        } else {
          c1 = *reinterpret_cast<const v4f*>(o1 + ch);
        }
      }
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
