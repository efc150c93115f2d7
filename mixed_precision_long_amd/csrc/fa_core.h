// The 16-bit MFMA attention core (one split of one work group over its tile
// list) and the merges of split and cold states, shared by the pass-2 and
// exact kernels and the single-launch path.
//
// "APA: sloppy attention, exact where it counts" (rfriedmann.de): sections
// "Pass 2: exact FP16 on the hot tiles" and "The merge that makes it exact".
#pragma once

#include "attn16.h"

namespace apa {

namespace {

// ---------------------------------------------------------------------------
// D <= 256: direct-to-LDS double-buffered tiles, four waves per work group.

template <int D>
struct FaCfg {
  static constexpr int TB = kTile * D * 2;  // bytes of one K or V tile
  static constexpr int STAGE = 2 * TB;      // K then V
  static constexpr size_t BYTES = 2 * (size_t)STAGE;
  static constexpr int NLD = D / 32;  // 16-byte LDS loads per lane per tile half
  static constexpr int GRP = kTile * 64;  // bytes of one 32-channel group of a tile
};

// A work group's tile list as pass 2's compaction left it in memory (scalar
// loads), or the exact path's run of consecutive tiles from base.
template <int MODE>
struct GList {
  int base;
  const cint32* tiles;
  const cuint32* masks;
  __device__ __forceinline__ int tile(int it) const { return MODE == kExact ? base + it : tiles[it]; }
  __device__ __forceinline__ uint32_t mask(int it) const { return masks[it]; }
};

// One split of one work group (four row blocks, one wave each) of the 16-bit
// core: positions [lo, hi) of its tile list, staged through the double buffer
// at smem (FaCfg<D>::BYTES of LDS); wave is the wave's index among the four
// (its share of the tile loads), rw the row block it computes (wave, or a
// permutation of the four).
// list.tile(it) and list.mask(it) give a position's key tile and the mask of
// the verdict groups it is hot for (pass 2).  TEAM: two such splits share
// the work group, one per four waves, and meet at every barrier: the loop
// runs nit >= hi - lo iterations, the extra ones only at the barrier.  COH:
// split states and the cold state go through device-coherent accesses
// (another work group of the same launch wrote or reads them).
// TAG only tells call sites apart: each kernel that calls the core directly
// names its own specialization (the host pass of hipcc rejects a second
// kernel specialization that calls the same one).
template <int D, typename T, int MODE, bool TEAM, bool COH, int TAG, class List>
__device__ __forceinline__ void fa_split(const Geom& g, const T* __restrict__ Q,
                                         const T* __restrict__ K, const T* __restrict__ V,
                                         const Fp4Ptrs& f, const Pass2Args& a, int S, int u,
                                         int wg, int sp, int wave, int rw, uint8_t* smem, int lo,
                                         int hi,
                                         int nit, const List& list) {
  using C = FaCfg<D>;
  using E = E16<T>;
  typedef typename E::V8 V8;
  constexpr int NC = D / 16;  // 16-channel chunks of the QK contraction
  constexpr int ND = D / 32;  // 32-channel blocks of the output
  constexpr bool BF = std::is_same<T, __bf16>::value;

  const int lane = threadIdx.x & 63;
  const int n = lane & 31, hh = lane >> 5;
  const RowBlocks rb = row_blocks(g);
  const int hk = u % g.Hkv;
  const int b = u / g.Hkv;
  const WaveRows wr = wave_rows(g, rb, wg, rw);
  const int hq = hk * g.G + wr.gi;
  const size_t bhq = (size_t)b * g.Hq + hq, bhk = (size_t)b * g.Hkv + hk;
  const int r0 = wr.r0;
  const int row = r0 + n;
  const bool row_ok = wr.live && row < g.Nq;
  const int d_wave =
      wr.live ? (g.causal ? min(g.Nkv - 1, min(r0 + 31, g.Nq - 1) + g.off) / kTile : g.NT - 1) : -1;
  const int lo_wave = window_lo(g, r0);  // with a sliding window, the first tile it sees

  // resident Q^T operand: 8 elements per 16-channel chunk
  V8 qf[NC];
  {
    const int rl = row_ok ? row : 0;
    const T* qp = Q + ((bhq * g.Nq) + rl) * D + 8 * hh;
#pragma unroll
    for (int c = 0; c < NC; ++c) qf[c] = *reinterpret_cast<const V8*>(qp + 16 * c);
  }
  const float c_r = (MODE == kPass2) ? f.q_frame[bhq * g.NqP + (row_ok ? row : 0)] : 0.0f;
  const float sl = g.sl;
  // bf16 V: the head's power-of-two shift into the fp16 range
  const int vsh = BF ? v_shift(head_vamax(f, a, bhk, MODE == kPass2)) : 0;
  const float vdown = __int_as_float((127 - vsh) << 23);

  // LDS-writing loads: wave w loads 16-key block w of every 32-channel group;
  // lane L carries key 16w + L/4 and the row's 16-byte slot L%4 (K: chunk
  // (L%4) ^ ((key/4)%4), so the slot holds that chunk; V: chunk L%4).
  const int ckey = wave * 16 + (lane >> 2);
  const uint32_t cK = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
  const uint32_t cV = (uint32_t)((lane & 3) * 16);
  const int b_ = (int)(bhk / g.Hkv), hk_ = (int)(bhk % g.Hkv);
  auto issue = [&](int t, int sb) {
    // one tile's rows (flat or paged); rows past the last key re-read the
    // last key (their scores are masked)
    const auto rK = tile_rsrc<T>(g, K, b_, hk_, t);
    const auto rV = tile_rsrc<T>(g, V, b_, hk_, t);
    const uint32_t rowoff =
        (uint32_t)(min(t * kTile + ckey, g.Nkv - 1) - t * kTile) * (uint32_t)(D * 2);
    uint8_t* st = smem + sb * C::STAGE + wave * 1024;
#pragma unroll
    for (int i = 0; i < C::NLD; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void*)(st + i * C::GRP), 16, rowoff + cK,
                                               i * 64, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void*)(st + C::TB + i * C::GRP), 16,
                                               rowoff + cV, i * 64, 0, 0);
    }
  };

  // per-lane LDS read offsets inside a 32-channel group
  const int kx = (n >> 2) & 3;
  const uint32_t kE = (uint32_t)(n * 64 + ((hh ^ kx) * 16));
  const uint32_t kO = (uint32_t)(n * 64 + (((2 + hh) ^ kx) * 16));
  const int G16 = lane >> 4, i16 = lane & 15;
  const uint32_t vl = (uint32_t)((4 * (G16 >> 1) + (i16 >> 2)) * 64 +
                                 (2 * (G16 & 1) + ((i16 & 3) >> 1)) * 16 + (i16 & 1) * 8);

  float m = -__builtin_inff(), l = 0.0f;
  v16f o[ND];
#pragma unroll
  for (int i = 0; i < ND; ++i) o[i] = v16f{};
  const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};

  int t_next = lo < hi ? list.tile(lo) : 0;
  if (lo < hi) issue(t_next, 0);
  for (int it = lo; it < (TEAM ? lo + nit : hi); ++it) {
    const bool mine = !TEAM || it < hi;  // a team's extra iterations: the barrier only
    const int t = t_next;
    const int sb = (it - lo) & 1;
    // the next tile's index and this tile's mask, read before the wait so
    // their latency hides behind it
    t_next = it + 1 < hi ? list.tile(it + 1) : 0;
    const uint32_t mk = MODE == kPass2 && mine ? list.mask(it) : 0u;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of tile t are in LDS
    if (BF && mine) {
      // the V rows this wave loaded, to fp16 in place
      uint8_t* st = smem + sb * C::STAGE + C::TB + wave * 1024 + lane * 16;
#pragma unroll
      for (int i = 0; i < C::NLD; ++i) {
        uint4* p = reinterpret_cast<uint4*>(st + i * C::GRP);
        *p = bf16x8_to_f16x8(*p, vdown);
      }
    }
    __syncthreads();
    if (it + 1 < hi) issue(t_next, sb ^ 1);
    if (TEAM && !mine) continue;

    // does this wave compute tile t, and for which of its two groups?
    bool on0, on1;
    if (MODE == kExact) {
      on0 = on1 = t <= d_wave && t >= lo_wave;
    } else {
      on0 = (mk >> (2 * rw)) & 1u;
      on1 = (mk >> (2 * rw + 1)) & 1u;
    }
    if (!(wr.live && (on0 || on1))) continue;
    const uint8_t* Ks = smem + sb * C::STAGE;
    const uint8_t* Vs = Ks + C::TB;
    const int k0 = t * kTile;

    // ---- S^T = K Q^T (raw dot products)
    v16f acc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      acc[kb] = v16f{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const V8 kf = *reinterpret_cast<const V8*>(Ks + (c >> 1) * C::GRP + kb * 2048 +
                                                   ((c & 1) ? kO : kE));
        acc[kb] = E::mma(kf, qf[c], acc[kb]);
      }
    }
    // ---- V^T operands (DS_READ_B64_TR_B16 in P's key order); up to D = 128
    // the whole tile's are read here, so the reads overlap the softmax
    auto vread = [&](int db, int kb, int c) {
      const uint8_t* p0 = Vs + db * C::GRP + (kb * 32 + 16 * c) * 64 + vl;
      const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(p0));
      const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(p0 + 8 * 64));
      return __builtin_bit_cast(v8h, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int NV = D <= 128 ? ND : 1;
    v8h vf[NV][2][2];
    if (D <= 128) {
#pragma unroll
      for (int db = 0; db < NV; ++db)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int c = 0; c < 2; ++c) vf[db][kb][c] = vread(db, kb, c);
    }
    // ---- key masking: diagonal and padding tiles, rows past Nq (wave-uniform)
    const bool win = g.causal && g.window > 0;
    const bool need_mask = (k0 + kTile > g.Nkv) || (g.causal && k0 + kTile - 1 > r0 + g.off) ||
                           (r0 + 31 >= g.Nq) || (win && k0 <= r0 + 31 + g.off - g.window);
    if (need_mask) {
      const int lim = g.causal ? row + g.off : 0x7fffffff;
      const int lim_lo = win ? row + g.off - g.window : -1;  // keys <= lim_lo: outside the window
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          if (!(row_ok && key < g.Nkv && key <= lim && key > lim_lo))
            acc[kb][j] = -__builtin_inff();
        }
    }
    // ---- row maximum (raw), then in log2 units; lazy move of m
    float tmax = vmax(acc[0][0], acc[0][1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) tmax = vmax3(tmax, acc[0][j], acc[0][j + 1]);
#pragma unroll
    for (int j = 0; j < 16; j += 2) tmax = vmax3(tmax, acc[1][j], acc[1][j + 1]);
    tmax = vmax(tmax, xor32(tmax));
    // pass 2: a 16-row group the tile is not hot for sees no key of it
    const bool grp_on = MODE == kExact || ((n >> 4) ? on1 : on0);
    const float smax = grp_on ? fmaf(tmax, sl, -c_r) : -__builtin_inff();
    const bool up = smax > m + kLazy;  // m = -inf: any visible key
    if (__ballot(up) != 0ull) {
      const float alpha = up ? fast_exp2(m - smax) : 1.0f;  // m = -inf -> 0
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
      l *= alpha;
      m = up ? smax : m;
    }
    const float bias =
        grp_on ? -(c_r + (m == -__builtin_inff() ? 0.0f : m)) : -__builtin_inff();
    // ---- P = 2^(s - m) in fp16 (also for bf16 inputs) and its row sum
    v8h pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const v2f p2 = {fast_exp2(fmaf(acc[kb][8 * c + j], sl, bias)),
                          fast_exp2(fmaf(acc[kb][8 * c + j + 1], sl, bias))};
          const v2h h2 = __builtin_convertvector(p2, v2h);
          l = __builtin_amdgcn_fdot2(h2, ones, l, false);
          pf[kb][c][j] = h2[0];
          pf[kb][c][j + 1] = h2[1];
        }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
          o[db] = mfma_f16(D <= 128 ? vf[db % NV][kb][c] : vread(db, kb, c), pf[kb][c], o[db]);
  }

  if (TEAM && sp >= S) return;  // the idle half of a work group's last pair
  if (!wr.live) return;
  l += xor32(l);
  if (!row_ok) return;
  finish_row<D, T, MODE, D / 32, COH>(g, f, a, S, sp, bhq, row, hh, m, l, c_r, o, vsh);
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

// The S split states of row r, channels ch .. ch + 3, combined in split order,
// then: exact -> output; pass 2 fused -> merged with the cold state; pass 2
// unfused -> the hot state.  COH: the states come from other work groups of
// the same launch.
template <int D, typename T, int MODE, bool COH>
__device__ __forceinline__ void combine_row4(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a,
                                             int S, long nrows, long r, int ch) {
  float Mh = -__builtin_inff();
  for (int s = 0; s < S; ++s)
    if (ldf<COH>(a.part_l + s * nrows + r) > 0.0f) Mh = fmaxf(Mh, ldf<COH>(a.part_m + s * nrows + r));
  float Lh = 0.0f;
  v4f oh = {0, 0, 0, 0};
  for (int s = 0; s < S; ++s) {
    const float ls = ldf<COH>(a.part_l + s * nrows + r);
    if (ls > 0.0f) {
      const float w = fast_exp2(ldf<COH>(a.part_m + s * nrows + r) - Mh);
      Lh += w * ls;
      const v4f x = ld4<COH>(a.part_o + (s * nrows + r) * D + ch);
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
  const float l1 = ldf<COH>(a.cold_l + r);
  const v4f a1 = l1 > 0.0f ? ld4<COH>(a.cold_o + r * D + ch) : v4f{0, 0, 0, 0};
  const long bh = r / g.Nq, rr = r % g.Nq;
  const float c0 = want_lse ? f.q_frame[bh * g.NqP + rr] : 0.0f;
  merge4<T>(ldi<COH>(a.cold_m + r), l1, a1, Lh > 0.0f ? Mh : -__builtin_inff(), Lh, oh, c0,
            reinterpret_cast<T*>(a.out) + r * D + ch, want_lse ? a.lse + r : nullptr);
}

}  // namespace

}  // namespace apa
