// a9, a11 at D = 512: the 16-bit MFMA attention core (the exact pass 2 over
// compacted hot tiles, fused with the merge, and the all-exact baseline) for
// large head dimensions, fp16 or bf16 inputs.
//
// "APA: sloppy attention, exact where it counts" (rfriedmann.de): section
// "Pass 2: exact FP16 on the hot tiles" and the introduction's all-exact
// baseline; large head dimensions follow the FFPA documentation's interface
// (same layout and semantics at D = 512).
//
// At D = 512 the output of a wave's 32 rows (32 x 512 FP32) takes 256
// registers per lane and its resident Q operand 128 more: with the operands of
// a tile that is more than a lane holds.  So a unit's four row blocks run as
// two work groups, one per half of the output channels.  Each wave computes
// its rows' scores over all 512 channels (the Q K^T products are done once
// per half: 1.5x the matrix work of one pass) and adds P V for its 256
// channels; both groups take the same softmax decisions, the second writes
// only its channels.  Keys are staged 32 at a time: the K rows over all
// channels (32 KB, K row slots XOR-swizzled as in the D <= 256 kernel) and the
// V rows of the group's half (16 KB), double buffered (96 KB of LDS), written
// by buffer loads straight into LDS.  Per wave and stage:
//   S^T = K Q^T     32 MFMA 32x32x16 (K from LDS, Q^T resident);
//   softmax         lazy running maximum, p = exp2(sl*q.k - (c_r + m)) in fp16,
//                   row sums by V_DOT2;
//   O^T += V^T P^T  16 MFMA 32x32x16 f16 (V^T by DS_READ_B64_TR_B16).
#include "attn16.h"

namespace apa {

namespace {

struct BigCfg {
  static constexpr int D = 512;
  static constexpr int KEYS = 32;            // keys per stage
  static constexpr int GRP = KEYS * 64;      // bytes of one 32-channel group of a stage
  static constexpr int KB = (D / 32) * GRP;  // K rows, all channels
  static constexpr int VB = (D / 64) * GRP;  // V rows, the group's half of the channels
  static constexpr int STAGE = KB + VB;
  static constexpr size_t BYTES = 2 * (size_t)STAGE;
  static constexpr int NDO = D / 64;         // 32-channel output blocks per wave
};

// (the body is a device function: the target builtins it uses must not be
// instantiated for the host side of the kernel)
template <typename T, int MODE>
__device__ __forceinline__ void big_body(const Geom& g, const T* __restrict__ Q,
                                         const T* __restrict__ K, const T* __restrict__ V,
                                         const Fp4Ptrs& f, const Pass2Args& a, int nitems, int S) {
  using C = BigCfg;
  using E = E16<T>;
  typedef typename E::V8 V8;
  constexpr int D = C::D;
  constexpr int NC = D / 16;   // 16-channel chunks of the QK contraction
  constexpr int NDO = C::NDO;
  constexpr bool BF = std::is_same<T, __bf16>::value;
  extern __shared__ __attribute__((aligned(16))) uint8_t big_smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, hh = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= nitems) return;  // uniform over the block
  const RowBlocks rb = row_blocks(g);
  // items: (batch, kv-head, split, work group, half), the half innermost so
  // both halves of a unit run side by side on one XCD (they read the same K)
  const int dh = item & 1;
  int u = item >> 1;
  const int wg = MODE == kExact ? rb.nwg - 1 - u % rb.nwg : u % rb.nwg;
  u /= rb.nwg;
  const int sp = u % S;
  u /= S;
  const int hk = u % g.Hkv;
  const int b = u / g.Hkv;
  const int unit = (b * g.Hkv + hk) * rb.nwg + wg;
  const WaveRows wr = wave_rows(g, rb, wg, wave);
  const int hq = hk * g.G + wr.gi;
  const size_t bhq = (size_t)b * g.Hq + hq, bhk = (size_t)b * g.Hkv + hk;
  const int r0 = wr.r0;
  const int row = r0 + n;
  const bool row_ok = wr.live && row < g.Nq;
  const int d_wave =
      wr.live ? (g.causal ? min(g.Nkv - 1, min(r0 + 31, g.Nq - 1) + g.off) / kTile : g.NT - 1) : -1;
  const int lo_wave = window_lo(g, r0);  // with a sliding window, the first tile it sees

  // this split's part of the work group's tile list
  int lo, hi, base = 0;
  const cint32* tiles = nullptr;
  const cuint32* masks = nullptr;
  {
    // exact: the tiles from the first row's window start to the last row's diagonal
    if (MODE == kExact) base = window_lo(g, wave_rows(g, rb, wg, 0).r0);
    const int ntot = MODE == kExact ? exact_tiles(g, rb, wg) - base : a.list_count[unit];
    lo = split_lo(ntot, sp, S);
    hi = split_lo(ntot, sp + 1, S);
    if (MODE == kPass2) {
      tiles = (const cint32*)(a.list_tiles + (size_t)unit * g.NT);
      masks = (const cuint32*)(a.list_masks + (size_t)unit * g.NT);
    }
  }
  auto tile_at = [&](int it) { return MODE == kExact ? base + it : tiles[it]; };

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

  // LDS-writing loads of a stage: wave w fills keys 16 (w % 2) .. +15 of the
  // groups w / 2, w / 2 + 2, ... (eight K groups, four V groups of the half);
  // lane L carries key 16 (w % 2) + L / 4 and the row's 16-byte slot L % 4
  // (K: channel chunk (L % 4) ^ ((key / 4) % 4), so the slot holds that chunk;
  // V: chunk L % 4).
  const int kblk = wave & 1, g0 = wave >> 1;
  const int b_ = (int)(bhk / g.Hkv), hk_ = (int)(bhk % g.Hkv);
  const uint32_t cK = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) * 16);
  const uint32_t cV = (uint32_t)((lane & 3) * 16);
  auto issue = [&](int t, int half, int sb) {
    // rows past the last key re-read the last key (their scores are masked)
    // one tile's rows (flat or paged)
    const auto rK = tile_rsrc<T>(g, K, b_, hk_, t);
    const auto rV = tile_rsrc<T>(g, V, b_, hk_, t);
    const int key = t * kTile + half * C::KEYS + 16 * kblk + (lane >> 2);
    const uint32_t rowoff = (uint32_t)(min(key, g.Nkv - 1) - t * kTile) * (uint32_t)(D * 2);
    uint8_t* st = big_smem + sb * C::STAGE + kblk * 1024;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int grp = g0 + 2 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rK, (lds_void*)(st + grp * C::GRP), 16,
                                               rowoff + cK, grp * 64, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < D / 128; ++i) {
      const int grp = g0 + 2 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_void*)(st + C::KB + grp * C::GRP), 16,
                                               rowoff + cV, (dh * NDO + grp) * 64, 0, 0);
    }
  };

  // per-lane LDS read offsets inside a 32-channel group of a stage
  const int kx = (n >> 2) & 3;
  const uint32_t kE = (uint32_t)(n * 64 + ((hh ^ kx) * 16));
  const uint32_t kO = (uint32_t)(n * 64 + (((2 + hh) ^ kx) * 16));
  const int G16 = lane >> 4, i16 = lane & 15;
  const uint32_t vl = (uint32_t)((4 * (G16 >> 1) + (i16 >> 2)) * 64 +
                                 (2 * (G16 & 1) + ((i16 & 3) >> 1)) * 16 + (i16 & 1) * 8);

  float m = -__builtin_inff(), l = 0.0f;
  v16f o[NDO];
#pragma unroll
  for (int i = 0; i < NDO; ++i) o[i] = v16f{};
  const v2h ones = {(_Float16)1.0f, (_Float16)1.0f};

  // stages: the two 32-key halves of each tile of the range, in order
  const int nst = 2 * (hi - lo);
  int t_cur = nst > 0 ? tile_at(lo) : 0;
  if (nst > 0) issue(t_cur, 0, 0);
  for (int q = 0; q < nst; ++q) {
    const int it = lo + (q >> 1), half = q & 1;
    const int sb = q & 1;
    // the next tile's index and this tile's mask (scalar loads), read before
    // the wait so their latency hides behind it
    const int t = t_cur;
    const int t_next = half && it + 1 < hi ? tile_at(it + 1) : t;
    t_cur = t_next;
    const uint32_t mk = MODE == kPass2 ? masks[it] : 0u;
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of the stage are in LDS
    if (BF) {
      // the V rows this wave loaded, to fp16 in place
      uint8_t* st = big_smem + sb * C::STAGE + C::KB + kblk * 1024 + lane * 16;
#pragma unroll
      for (int i = 0; i < D / 128; ++i) {
        uint4* p = reinterpret_cast<uint4*>(st + (g0 + 2 * i) * C::GRP);
        *p = bf16x8_to_f16x8(*p, vdown);
      }
    }
    __syncthreads();
    if (q + 1 < nst) issue(t_next, half ^ 1, sb ^ 1);

    // does this wave compute tile t, and for which of its two groups?
    bool on0, on1;
    if (MODE == kExact) {
      on0 = on1 = t <= d_wave && t >= lo_wave;
    } else {
      on0 = (mk >> (2 * wave)) & 1u;
      on1 = (mk >> (2 * wave + 1)) & 1u;
    }
    if (!(wr.live && (on0 || on1))) continue;
    const uint8_t* Ks = big_smem + sb * C::STAGE;
    const uint8_t* Vs = Ks + C::KB;
    const int k0 = t * kTile + half * C::KEYS;

    // ---- S^T = K Q^T (raw dot products) for the stage's 32 keys
    v16f acc = v16f{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const V8 kf = *reinterpret_cast<const V8*>(Ks + (c >> 1) * C::GRP + ((c & 1) ? kO : kE));
      acc = E::mma(kf, qf[c], acc);
    }
    // ---- key masking: diagonal and padding keys, rows past Nq (wave-uniform)
    const bool win = g.causal && g.window > 0;
    const bool need_mask = (k0 + C::KEYS > g.Nkv) || (g.causal && k0 + C::KEYS - 1 > r0 + g.off) ||
                           (r0 + 31 >= g.Nq) || (win && k0 <= r0 + 31 + g.off - g.window);
    if (need_mask) {
      const int lim = g.causal ? row + g.off : 0x7fffffff;
      const int lim_lo = win ? row + g.off - g.window : -1;  // keys <= lim_lo: outside the window
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = k0 + 8 * (j >> 2) + 4 * hh + (j & 3);
        if (!(row_ok && key < g.Nkv && key <= lim && key > lim_lo)) acc[j] = -__builtin_inff();
      }
    }
    // ---- row maximum (raw), then in log2 units; lazy move of m
    float tmax = vmax(acc[0], acc[1]);
#pragma unroll
    for (int j = 2; j < 16; j += 2) tmax = vmax3(tmax, acc[j], acc[j + 1]);
    tmax = vmax(tmax, xor32(tmax));
    // pass 2: a 16-row group the tile is not hot for sees no key of it
    const bool grp_on = MODE == kExact || ((n >> 4) ? on1 : on0);
    const float smax = grp_on ? fmaf(tmax, sl, -c_r) : -__builtin_inff();
    const bool up = smax > m + kLazy;  // m = -inf: any visible key
    if (__ballot(up) != 0ull) {
      const float alpha = up ? fast_exp2(m - smax) : 1.0f;  // m = -inf -> 0
#pragma unroll
      for (int db = 0; db < NDO; ++db)
#pragma unroll
        for (int j = 0; j < 16; ++j) o[db][j] *= alpha;
      l *= alpha;
      m = up ? smax : m;
    }
    const float bias =
        grp_on ? -(c_r + (m == -__builtin_inff() ? 0.0f : m)) : -__builtin_inff();
    // ---- P = 2^(s - m) in fp16 (also for bf16 inputs) and its row sum
    v8h pf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const v2f p2 = {fast_exp2(fmaf(acc[8 * c + j], sl, bias)),
                        fast_exp2(fmaf(acc[8 * c + j + 1], sl, bias))};
        const v2h h2 = __builtin_convertvector(p2, v2h);
        l = __builtin_amdgcn_fdot2(h2, ones, l, false);
        pf[c][j] = h2[0];
        pf[c][j + 1] = h2[1];
      }
    // ---- O^T += V^T P^T for this half's channels (V^T in P's key order)
#pragma unroll
    for (int db = 0; db < NDO; ++db)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint8_t* p0 = Vs + db * C::GRP + (16 * c) * 64 + vl;
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(p0));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) v4s*)(p0 + 8 * 64));
        const v8h vf =
            __builtin_bit_cast(v8h, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = mfma_f16(vf, pf[c], o[db]);
      }
  }

  if (!wr.live) return;
  l += xor32(l);
  if (!row_ok) return;
  finish_row<D, T, MODE, NDO>(g, f, a, S, sp, bhq, row, hh, m, l, c_r, o, vsh, dh * NDO * 32,
                              dh == 0);
}

template <typename T, int MODE>
__global__ __launch_bounds__(kWgWaves * 64) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attn_big(
    Geom g, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, Fp4Ptrs f,
    Pass2Args a, int nitems, int S) {
  big_body<T, MODE>(g, Q, K, V, f, a, nitems, S);
}

template <typename T, int MODE>
hipError_t run_big(const Geom& g, const void* q, const void* k, const void* v, const Fp4Ptrs& f,
                   const Pass2Args& a, int S, hipStream_t s) {
  const int nitems = attn_units(g) * S * 2;
  if (nitems == 0) return hipSuccess;
  static bool attr_done = false;
  if (!attr_done) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)k_attn_big<T, MODE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)BigCfg::BYTES);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  hipLaunchKernelGGL((k_attn_big<T, MODE>), dim3(nitems), dim3(kWgWaves * 64), BigCfg::BYTES, s,
                     g, (const T*)q, (const T*)k, (const T*)v, f, a, nitems, S);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_big(const Geom& g, const void* q, const void* k, const void* v,
                           const Fp4Ptrs& f, const Pass2Args& a, int S, int mode, hipStream_t s) {
  if (g.D != BigCfg::D) return hipErrorInvalidValue;
  if (g.bf16)
    return mode ? run_big<__bf16, kPass2>(g, q, k, v, f, a, S, s)
                : run_big<__bf16, kExact>(g, q, k, v, f, a, S, s);
  return mode ? run_big<_Float16, kPass2>(g, q, k, v, f, a, S, s)
              : run_big<_Float16, kExact>(g, q, k, v, f, a, S, s);
}

}  // namespace apa
