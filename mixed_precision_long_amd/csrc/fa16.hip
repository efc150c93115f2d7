// a8..a11: 16-bit MFMA flash attention -- the exact pass 2 over compacted hot
// tiles with the fused log-sum-exp merge, the standalone merge, and the
// all-exact baseline; fp16 or bf16 inputs.
//
// "APA: sloppy attention, exact where it counts" (rfriedmann.de): section
// "Pass 2: exact FP16 on the hot tiles" (a work group takes the rows of a few
// pass-1 blocks, gathers the tiles hot for any of them, streams those from the
// original 16-bit K and V; a wavefront works only on tiles hot for its rows,
// with an FP32 online softmax, and combines the result with the cold state of
// pass 1) and "The merge that makes it exact".  The introduction's all-exact
// baseline is the same core over every visible tile.  Large head dimensions
// follow the FFPA documentation's interface (same layout and semantics at
// D = 512).
//
// Row blocks.  A row block is 32 consecutive query positions of one query
// head; the row blocks of one (batch, kv-head) are numbered position-major,
// head-minor, and a work group takes four consecutive ones, one wavefront
// each, so the K/V tiles it stages feed every head of the KV group that shares
// them.  A work group's key range can be cut into S splits that run as
// separate work groups; each split writes a partial online-softmax state and a
// combine kernel merges them in split order (deterministic).
//
// D <= 256 (k_fa): four wavefronts, one per SIMD, and two work groups per
// compute unit up to D = 128, so every SIMD runs two independent waves (their
// matrix and vector phases interleave; the waves of one group meet at one
// barrier per tile).  K/V tiles go from HBM straight into LDS with buffer
// loads that write LDS (no staging registers), double buffered.  LDS holds a
// tile as [D/32][64 keys][32 channels] (64-byte rows): the transposing V reads
// are conflict-free as laid out, and the K rows have their four 16-byte slots
// XOR-swizzled by (key / 4) % 4 so that sixteen consecutive keys of one slot
// hit distinct banks.  Per wave and tile (D = 128):
//   S^T = K Q^T   16 MFMA 32x32x16, K from LDS, Q^T resident in registers;
//   softmax       raw maxima, then p = exp2(sl*q.k - (c_r + m)) in one FMA and
//                 one exp2 per score; the running maximum m moves only when a
//                 row's maximum exceeds it by more than 8 (log2 units), so the
//                 rescale of o is rare; row sums by V_DOT2 of the fp16 P;
//   O^T += V^T P^T 16 MFMA 32x32x16 f16; P stays in the accumulator's lanes
//                 (its key order is matched by the V^T operand), V^T comes
//                 from LDS by DS_READ_B64_TR_B16.  With bf16 inputs the scores
//                 use the bf16 MFMA and each wave converts the V rows it loaded
//                 to fp16 in LDS, so P keeps 11 significant bits; V is first
//                 divided by a per-head power of two that brings its largest
//                 magnitude into the fp16 range (exact), undone in the
//                 epilogue.
// D = 512 runs in big16.hip (two work groups per unit, one per half of the
// output channels).
#include "fa_core.h"

namespace apa {

namespace {

// ---------------------------------------------------------------------------
// D <= 256: direct-to-LDS double-buffered tiles, four waves per work group.

template <int D, typename T, int MODE>
__device__ __forceinline__ void fa_body(const Geom& g, const T* __restrict__ Q,
                                        const T* __restrict__ K, const T* __restrict__ V,
                                        const Fp4Ptrs& f, const Pass2Args& a, int nitems, int S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t fa_smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= nitems) return;  // uniform over the block
  const RowBlocks rb = row_blocks(g);
  int wg, sp, u;
  if (MODE == kExact) {
    // each (batch, kv-head, split) from its last query positions (the
    // longest causal key ranges) down
    wg = rb.nwg - 1 - item % rb.nwg;
    u = item / rb.nwg;
    sp = u % S;
    u /= S;
  } else {
    // per (batch, kv-head) and split, its work groups longest list first (a
    // greedy longest-first schedule over the compute units its items land
    // on); the splits stay in turn, so the work groups running together read
    // the same part of their lists
    const int per = rb.nwg * S;
    u = item / per;
    const int j = item % per;
    wg = __builtin_amdgcn_readfirstlane(a.list_order[(size_t)u * rb.nwg + j % rb.nwg]);
    sp = j / rb.nwg;
  }
  const int hk = u % g.Hkv;
  const int b = u / g.Hkv;
  const int unit = (b * g.Hkv + hk) * rb.nwg + wg;
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
  const GList<MODE> list = {base, tiles, masks};
  fa_split<D, T, MODE, false, false, 0>(g, Q, K, V, f, a, S, u, wg, sp, wave, wave, fa_smem, lo,
                                     hi, hi - lo, list);
}

// Two work groups per compute unit up to D = 128 (registers <= 256 per
// lane, LDS 2 x 64 KB), one at D = 256.
template <int D, typename T, int MODE>
__global__ __launch_bounds__(kWgWaves * 64) __attribute__((amdgpu_waves_per_eu(D >= 256 ? 1 : 2, D >= 256 ? 1 : 2)))
void k_fa(Geom g, const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
          Fp4Ptrs f, Pass2Args a, int nitems, int S) {
  fa_body<D, T, MODE>(g, Q, K, V, f, a, nitems, S);
}

// ---------------------------------------------------------------------------

// Hot mask -> per work group (batch, kv-head, four row blocks) the list of the
// tiles hot for any of its verdict groups, ascending, with a mask of the
// groups each tile is hot for (bit 2w + k: wave w's k-th 16-row group).  One
// wavefront per work group; lane j handles hot word j (+64, ...).
__global__ __launch_bounds__(64) void k_compact(Geom g, const uint32_t* __restrict__ bits,
                                                int32_t* tiles, uint32_t* masks, int32_t* count,
                                                int nunits) {
  const int unit = blockIdx.x;
  if (unit >= nunits) return;
  const int lane = threadIdx.x;
  const RowBlocks rb = row_blocks(g);
  const int wg = unit % rb.nwg;
  const int bk = unit / rb.nwg;
  const int b = bk / g.Hkv, hk = bk % g.Hkv;
  // the hot words of the eight verdict groups (nullptr when absent)
  const uint32_t* gp[2 * kWgWaves];
#pragma unroll
  for (int w = 0; w < kWgWaves; ++w) {
    const WaveRows wr = wave_rows(g, rb, wg, w);
    const size_t bhq = (size_t)b * g.Hq + hk * g.G + wr.gi;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int grp = wr.r0 / 16 + k;
      gp[2 * w + k] = (wr.live && grp < g.NG) ? bits + (bhq * g.NG + grp) * g.W : nullptr;
    }
  }
  int32_t* tl = tiles + (size_t)unit * g.NT;
  uint32_t* ml = masks + (size_t)unit * g.NT;
  int base = 0;
  for (int w0 = 0; w0 < g.W; w0 += 64) {
    const int w = w0 + lane;
    uint32_t word[2 * kWgWaves];
    uint32_t un = 0u;
#pragma unroll
    for (int k = 0; k < 2 * kWgWaves; ++k) {
      word[k] = (w < g.W && gp[k]) ? gp[k][w] : 0u;
      un |= word[k];
    }
    const int cnt = __popc(un);
    int incl = cnt;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    int pos = base + incl - cnt;
    uint32_t rem = un;
    while (rem) {
      const int bit = __ffs(rem) - 1;
      rem &= rem - 1u;
      uint32_t mk = 0u;
#pragma unroll
      for (int k = 0; k < 2 * kWgWaves; ++k) mk |= ((word[k] >> bit) & 1u) << k;
      tl[pos] = w * 32 + bit;
      ml[pos] = mk;
      ++pos;
    }
    base += __shfl(incl, 63);
  }
  if (lane == 0) count[unit] = base;
}

// Per (b, kv-head), its pass-2 work groups ordered by descending tile count,
// ties in ascending order (the rank of each among the head's counts, staged
// in LDS: nwg^2 / 256 comparisons per thread, a few microseconds at 1024);
// above kOrderMax work groups per head the order is the identity.
// One block of 256 threads per (b, kv-head).  The order only schedules: every
// work group computes the same values whenever it runs.
constexpr int kOrderMax = 2048;
__global__ __launch_bounds__(256) void k_order(const int32_t* __restrict__ count,
                                               int32_t* __restrict__ order, int nwg) {
  __shared__ int c[kOrderMax];
  const int32_t* cnt = count + (size_t)blockIdx.x * nwg;
  int32_t* ord = order + (size_t)blockIdx.x * nwg;
  if (nwg > kOrderMax) {
    for (int w = threadIdx.x; w < nwg; w += blockDim.x) ord[w] = w;
    return;
  }
  for (int w = threadIdx.x; w < nwg; w += blockDim.x) c[w] = cnt[w];
  __syncthreads();
  for (int w = threadIdx.x; w < nwg; w += blockDim.x) {
    const int x = c[w];
    int r = 0;
    for (int j = 0; j < nwg; ++j) {
      const int y = c[j];
      r += (y > x) | ((y == x) & (j < w));
    }
    ord[r] = w;
  }
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

// Combine the S split states of each row (see combine_row4).  One thread per
// (row, 4 channels).
template <int D, typename T, int MODE>
__global__ void k_combine(Geom g, Fp4Ptrs f, Pass2Args a, int S, long nrows) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long r = gid / (D / 4);
  const int ch = (int)(gid % (D / 4)) * 4;
  if (r >= nrows) return;
  combine_row4<D, T, MODE, false>(g, f, a, S, nrows, r, ch);
}

// max |V| per (b, kv-head) and chunk of kVmaxChunk keys, for bf16 inputs of
// the exact path (the NaN-ignoring maximum: non-finite inputs give undefined
// outputs either way).  grid (nch, B*Hkv), 256 threads, 16-byte loads.
__global__ __launch_bounds__(256) void k_vmax(Geom g, const uint16_t* __restrict__ V, float* out,
                                              int nch) {
  const int c = blockIdx.x, bh = blockIdx.y;
  float m = 0.0f;
  // the chunk's key tiles (contiguous rows each, flat or paged)
  for (int t = c * (kVmaxChunk / 64); t < min(g.NT, (c + 1) * (kVmaxChunk / 64)); ++t) {
    const long n8 = (long)min(64, g.Nkv - t * 64) * g.D / 8;
    const uint4* src = reinterpret_cast<const uint4*>(V + kv_elem(g, bh / g.Hkv, bh % g.Hkv, t * 64));
    for (long i = threadIdx.x; i < n8; i += 256) {
      const uint4 z = src[i];
      const uint32_t w[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[j] << 16)),
                           fabsf(__uint_as_float(w[j] & 0xFFFF0000u))));
    }
  }
  __shared__ float red[4];
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) out[(size_t)bh * nch + c] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

template <int D, typename T, int MODE>
hipError_t run_attn(const Geom& g, const void* q, const void* k, const void* v, const Fp4Ptrs& f,
                    const Pass2Args& a, int S, hipStream_t s) {
  const int nitems = attn_units(g) * S;
  if (nitems == 0) return hipSuccess;
  hipError_t e;
  if constexpr (D >= 512) {
    e = launch_attn_big(g, q, k, v, f, a, S, MODE, s);
  } else {
    auto kern = k_fa<D, T, MODE>;
    constexpr size_t bytes = FaCfg<D>::BYTES;
    static bool attr_done = false;
    if (!attr_done) {
      e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)bytes);
      if (e != hipSuccess) return e;
      attr_done = true;
    }
    hipLaunchKernelGGL(kern, dim3(nitems), dim3(kWgWaves * 64), bytes, s, g, (const T*)q,
                       (const T*)k, (const T*)v, f, a, nitems, S);
    e = hipGetLastError();
  }
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
  switch (g.D) {
    case 64: return run_attn<64, T, MODE>(g, q, k, v, f, a, S, s);
    case 128: return run_attn<128, T, MODE>(g, q, k, v, f, a, S, s);
    case 256: return run_attn<256, T, MODE>(g, q, k, v, f, a, S, s);
    case 512: return run_attn<512, T, MODE>(g, q, k, v, f, a, S, s);
    default: return hipErrorInvalidValue;
  }
}

template <int MODE>
hipError_t dispatch(const Geom& g, const void* q, const void* k, const void* v, const Fp4Ptrs& f,
                    const Pass2Args& a, int S, hipStream_t s) {
  return g.bf16 ? dispatch_t<MODE, __bf16>(g, q, k, v, f, a, S, s)
                : dispatch_t<MODE, _Float16>(g, q, k, v, f, a, S, s);
}

}  // namespace

int attn_units(const Geom& g) { return g.B * g.Hkv * row_blocks(g).nwg; }

int attn_splits(const Geom& g) {
  const long units = attn_units(g);
  if (units <= 0) return 1;
  // about three work groups per resident slot of the 256-CU part (two per CU
  // up to D = 128, one above), so the dispatcher can even out their lengths;
  // at D = 512 each unit and split runs as two work groups (output halves)
  const long slots = 256L * (g.D <= 128 ? 2 : 1);
  const long wgs = units * (g.D >= 512 ? 2 : 1);
  long S = (3 * slots + wgs - 1) / wgs;
  if (S > 8) S = 8;
  // at least 16 tiles per split of the longest key range
  long maxs = g.NT / 16;
  if (maxs < 1) maxs = 1;
  if (S > maxs) S = maxs;
  return (int)(S < 1 ? 1 : S);
}

hipError_t launch_pass2(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a, hipStream_t s) {
  const int nunits = attn_units(g);
  if (nunits == 0) return hipSuccess;
  hipLaunchKernelGGL(k_compact, dim3(nunits), dim3(64), 0, s, g, a.bits, a.list_tiles,
                     a.list_masks, a.list_count, nunits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_order, dim3(g.B * g.Hkv), dim3(256), 0, s, a.list_count, a.list_order,
                     row_blocks(g).nwg);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return dispatch<kPass2>(g, a.q, a.k, a.v, f, a, attn_splits(g), s);
}

hipError_t launch_exact(const Geom& g, const void* q, const void* k, const void* v, void* out,
                        float* lse, const Pass2Args& parts, hipStream_t s) {
  Pass2Args a = parts;
  a.out = out;
  a.lse = lse;
  Fp4Ptrs f = {};
  if (g.bf16 && g.Nkv > 0) {
    // the largest |V| of each kv-head, for the shift of bf16 V into the fp16 range
    hipLaunchKernelGGL(k_vmax, dim3(a.vmax_nch, g.B * g.Hkv), dim3(256), 0, s, g,
                       (const uint16_t*)v, a.vmax, a.vmax_nch);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
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
