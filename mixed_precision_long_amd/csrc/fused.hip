// f1: both passes of APA in one persistent launch ("APA: sloppy attention,
// exact where it counts", rfriedmann.de, section "Pass 2: exact FP16 on the
// hot tiles": one work group per compute unit takes ordered tickets, first
// the pass-1 work, then the pass-2 work; a wait is only ever on a ticket that
// a running work group already holds, so the scheme cannot deadlock, and the
// pass-2 work fills the compute units that pass 1's last wave would leave
// idle).
//
// A work group has eight waves.  A pass-1 ticket is one pass-1 work group of
// the separate launch (its units, the same head and tail roles, pacing and
// code), followed by the re-walk of any of its units whose tail gave up, so
// its units are final when the ticket ends.  A pass-2 ticket is a pair of
// consecutive key splits of one pass-2 work group (four row blocks): the work
// group builds that group's hot-tile list in LDS from the hot words, and its
// two halves of four waves each run one split with the 16-bit core, meeting
// at every tile's barrier (the two splits' lengths differ by at most one
// tile).  Its row blocks' pass-1 units must be done first: per pass-2 work
// group a counter of finished units.  The last ticket of a pass-2 work group
// to finish merges the split states with the cold state, in split order with
// the same arithmetic as the separate combine, so the outputs equal those of
// the separate launches bit for bit.
//
// Memory between work groups of the launch.  Work groups on different XCDs do
// not share an L2.  A pass-1 ticket's waves write their outputs with plain
// stores and end with an agent-scope release fence (their L2 lines written
// back) before the ticket's units are counted; pass-2 tickets read the hot
// words and the cold state, and write and read split states, with relaxed
// agent-scope atomic accesses, which the hardware keeps coherent across XCDs;
// a counter is raised only after the writes it covers have completed.  Every
// wait is bounded: a wait that gives up sets the launch's timeout flag (and
// the FP4 buffer's status word) and goes on, so the launch always ends.
#include "pass1_core.h"
#include "fa_core.h"

namespace apa {

namespace {

constexpr int kFusedWaves = 8;
constexpr int kMaxLds = 160 * 1024;
constexpr int kMaxSpin = 1 << 21;  // a few seconds of polls (a legitimate wait is < 2 ms)

// The launch's control words (at the start of its workspace, cleared by
// k_fused_init): per XCD a pass-1 and a pass-2 ticket counter, the timeout
// flag, then per pass-2 work group the finished pass-1 units and the finished
// pass-2 tickets.
struct FusedCtl {
  int q1[8], q2[8], timeout, pad[47];
};
constexpr int kCtlWords = 64;

// The pass-2 tile list in LDS: (tile << 8) | the mask of its hot verdict groups.
struct LList {
  const uint32_t* e;
  __device__ __forceinline__ int tile(int it) const {
    return __builtin_amdgcn_readfirstlane((int)(e[it] >> 8));
  }
  __device__ __forceinline__ uint32_t mask(int it) const {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(e[it] & 0xFFu));
  }
};

// Entries the LDS list can hold beside the two halves' tile buffers.
template <int D>
constexpr int list_cap() {
  return (kMaxLds - 2 * (int)FaCfg<D>::BYTES - 256) / 4;
}

template <int D, bool LOG>
constexpr size_t fused_lds() {
  const size_t p1 = sizeof(P1Lds<D, LOG>);
  const size_t p2 = 2 * FaCfg<D>::BYTES + 4 * (size_t)list_cap<D>();
  return p1 > p2 ? p1 : p2;
}

__global__ void k_fused_init(int* ctl, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) ctl[i] = 0;
}

__device__ __forceinline__ int atomic_add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tickets come from eight queues, one per XCD, holding the positions that
// the XCD-contiguous numbering of the separate launches (xcd_remap) gives the
// work groups dispatched to that XCD, so a work group first takes work whose
// K/V its XCD's L2 already holds; an empty queue sends it to the next XCD's.
// Called by all of wave 0: the position of a ticket in [0, n), or -1 once
// every queue is empty.
__device__ __forceinline__ int take_ticket(int* q, int n, int xcc, int lane);

// Control flow around the barriers stays wave-uniform: the counters are
// raised by every lane of wave 0 (lane 0 adds v, the others 0) and the value
// lane 0 saw is taken with readfirstlane, so no branch on the lane index
// encloses a barrier or a loop edge (a region that only thread 0 runs, at
// the end and start of a loop with barriers, can be laid out so that the
// other lanes re-enter the loop without it).
__device__ __forceinline__ int wave_fetch_add(int* p, int v, int lane) {
  return __builtin_amdgcn_readfirstlane(atomic_add_agent(p, lane == 0 ? v : 0));
}

__device__ __forceinline__ int take_ticket(int* q, int n, int xcc, int lane) {
  const int full = n & ~7, per = full >> 3;
  for (int k = 0; k < 8; ++k) {
    const int x = (xcc + k) & 7;
    const int cnt = per + (x < n - full ? 1 : 0);
    if (cnt == 0) continue;
    const int i = wave_fetch_add(q + x, 1, lane);
    if (i < cnt) return i < per ? x * per + i : full + x;
  }
  return -1;
}

// The last ticket's merge of a pass-2 work group's split states with the cold
// state, for 16 rows of one row block (r0: its first query position) and one
// wave: lane (h, c) takes row rlo + R i + h (R = 64 / (D / 4) rows at a time)
// and channels 4 c .. 4 c + 3.  The
// arithmetic of combine_row4 in the same order (the same results); the loads
// of every split go out together, 16 bytes at a time, device-coherent.
template <int D, typename T>
__device__ __forceinline__ void combine_rows(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a,
                                             int S, long nrows, size_t bhq, int r0, int rlo,
                                             int lane) {
  static_assert(D == 64 || D == 128, "whole rows per wave");
  constexpr int NQ = D / 4;       // lanes per row
  constexpr int RPI = 64 / NQ;    // rows per pass of the wave
  constexpr int kMaxS = 8;
  const long rb0 = (long)bhq * g.Nq + r0;
  const int c = lane % NQ, h = lane / NQ;
  const int ch = 4 * c;
  __amdgpu_buffer_rsrc_t ro[kMaxS];
#pragma unroll
  for (int s = 0; s < kMaxS; ++s)
    ro[s] = rowblock_rsrc<D>(a.part_o + ((long)min(s, S - 1) * nrows + rb0) * D);
  const auto rc = rowblock_rsrc<D>(a.cold_o + rb0 * D);
  for (int i = rlo + h; i < rlo + 16; i += RPI) {
    if (r0 + i >= g.Nq) break;
    const long r = rb0 + i;
    const uint32_t off = (uint32_t)((i * D + ch) * 4);
    float ls[kMaxS], ms[kMaxS];
    v4f os[kMaxS];
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      if (s < S) {
        ls[s] = ldf<true>(a.part_l + s * nrows + r);
        ms[s] = ldf<true>(a.part_m + s * nrows + r);
        os[s] = coh_ld4(ro[s], off);
      }
    }
    const float l1 = ldf<true>(a.cold_l + r);
    const int m1 = ldi<true>(a.cold_m + r);
    const v4f c1 = coh_ld4(rc, off);
    float Mh = -__builtin_inff();
#pragma unroll
    for (int s = 0; s < kMaxS; ++s)
      if (s < S && ls[s] > 0.0f) Mh = fmaxf(Mh, ms[s]);
    float Lh = 0.0f;
    v4f oh = {0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < kMaxS; ++s) {
      if (s < S && ls[s] > 0.0f) {
        const float w = fast_exp2(ms[s] - Mh);
        Lh += w * ls[s];
        for (int e = 0; e < 4; ++e) oh[e] += w * os[s][e];
      }
    }
    const bool want_lse = a.lse && ch == 0;
    const long bh = r / g.Nq, rr = r % g.Nq;
    const float c0 = want_lse ? f.q_frame[bh * g.NqP + rr] : 0.0f;
    merge4<T>(m1, l1, l1 > 0.0f ? c1 : v4f{0, 0, 0, 0}, Lh > 0.0f ? Mh : -__builtin_inff(), Lh,
              oh, c0, reinterpret_cast<T*>(a.out) + r * D + ch, want_lse ? a.lse + r : nullptr);
  }
}

template <int D, typename T, bool LOG, int QT, bool VW>
__global__ __launch_bounds__(kFusedWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_fused(Geom g, Fp4Ptrs f, float eps, float tau, int hoff, Pass1Out out, uint8_t* split,
             int cap, int sched, int nunits, int n1, Pass2Args a, int S, int* ctl) {
  extern __shared__ __attribute__((aligned(16))) uint8_t fsm[];
  __shared__ int bc[4];
  FusedCtl* C = reinterpret_cast<FusedCtl*>(ctl);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const RowBlocks rb = row_blocks(g);
  const int nitems = g.B * g.Hkv * rb.nwg;
  int* ready = ctl + kCtlWords;      // [nitems] pass-1 units done
  int* done = ready + nitems;        // [nitems] pass-2 tickets done
  const int npairs = (S + 1) / 2;
  const int n2 = nitems * npairs;
  const int per1 = sched == kSchedTriples ? 3 * kFusedWaves / 4
                   : (sched == kSchedPairs ? kFusedWaves / 2 : kFusedWaves);
  const int nq32 = g.NqP / 32;
  const long nrows = (long)g.B * g.Hq * g.Nq;
  // this work group's XCD (the hardware register; it only steers which
  // queue is tried first)
  const int xcc = __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 7;
  // pass-1 tickets, until none is left
  for (;;) {
    if (wave == 0) bc[0] = take_ticket(C->q1, n1, xcc, lane);
    __syncthreads();
    const int t = __builtin_amdgcn_readfirstlane(bc[0]);
    __syncthreads();
    if (t < 0) break;
    {
      // ---- pass 1: the work group of the separate launch at position t
      const int blk = n1 - 1 - t;
      P1Lds<D, LOG>& L = *reinterpret_cast<P1Lds<D, LOG>*>(fsm);
      pass1_block<D, LOG, QT, VW>(g, f, eps, tau, hoff, out, split, cap, sched, nunits, blk, L);
      __builtin_amdgcn_s_setprio(0);
      __syncthreads();
      // tails that gave up: walked again from their head's state
      if (split) {
        for (int k = wave; k < per1; k += kFusedWaves) {
          const int u = blk * per1 + k;
          if (u < nunits)
            rewalk_unit<D, LOG, QT, VW>(g, f, eps, tau, hoff, out, split, cap, sched, u,
                                        (lds_u8*)L.vlog[LOG ? wave : 0]);
        }
      }
      // the outputs to the device-coherent level, then count the units
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __syncthreads();
      if (wave == 0) {
        // lane k counts unit k of the block (one per row block with rows)
        const int u = blk * per1 + lane;
        const int bk = u / (nq32 * g.G), j = u % (nq32 * g.G);
        const bool live = lane < per1 && u < nunits && j < rb.nrb;
        atomic_add_agent(ready + (live ? bk * rb.nwg + j / 4 : 0), live ? 1 : 0);
      }
    }
  }

  // pass-2 tickets: splits 2 pr and 2 pr + 1 of one work group
  for (;;) {
    if (wave == 0) bc[0] = take_ticket(C->q2, n2, xcc, lane);
    __syncthreads();
    const int x = __builtin_amdgcn_readfirstlane(bc[0]);
    __syncthreads();
    if (x < 0) break;
    const int per2 = rb.nwg * npairs;
    const int u = x / per2;  // (batch, kv-head)
    const int jx = x % per2;
    const int wg = rb.nwg - 1 - jx % rb.nwg;  // the last row blocks (longest lists) first
    const int pr = jx / rb.nwg;
    const int item = u * rb.nwg + wg;
    if (wave == 0) {
      // the whole wave polls (a uniform loop), bounded
      const int need = min(4, rb.nrb - 4 * wg);
      for (int spins = 0;; ++spins) {
        if (__builtin_amdgcn_readfirstlane(load_agent(ready + item)) >= need) break;
        if (spins == kMaxSpin) {
          if (lane == 0) {
            __hip_atomic_store(&C->timeout, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(f.status, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          break;
        }
        __builtin_amdgcn_s_sleep(8);
      }
    }
    __syncthreads();
    // the work group's hot-tile list (as the separate compaction builds it)
    uint32_t* lst = reinterpret_cast<uint32_t*>(fsm + 2 * FaCfg<D>::BYTES);
    if (wave == 0) {
      const int b = u / g.Hkv, hk = u % g.Hkv;
      const uint32_t* gp[2 * kWgWaves];
#pragma unroll
      for (int w = 0; w < kWgWaves; ++w) {
        const WaveRows wr = wave_rows(g, rb, wg, w);
        const size_t bhq = (size_t)b * g.Hq + hk * g.G + wr.gi;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int grp = wr.r0 / 16 + k;
          gp[2 * w + k] = (wr.live && grp < g.NG) ? out.bits + (bhq * g.NG + grp) * g.W : nullptr;
        }
      }
      int base = 0;
      for (int w0 = 0; w0 < g.W; w0 += 64) {
        const int w = w0 + lane;
        uint32_t word[2 * kWgWaves];
        uint32_t un = 0u;
#pragma unroll
        for (int k = 0; k < 2 * kWgWaves; ++k) {
          word[k] = (w < g.W && gp[k])
                        ? (uint32_t)load_agent(reinterpret_cast<const int*>(gp[k] + w))
                        : 0u;
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
          lst[pos] = ((uint32_t)(w * 32 + bit) << 8) | mk;
          ++pos;
        }
        base += __shfl(incl, 63);
      }
      bc[1] = __shfl(base, 0);
    }
    __syncthreads();
    const int ntot = __builtin_amdgcn_readfirstlane(bc[1]);
    const int team = wave >> 2;
    const int sp = 2 * pr + team;
    const int lo0 = split_lo(ntot, 2 * pr, S), mid = split_lo(ntot, 2 * pr + 1, S);
    const int hi1 = 2 * pr + 1 < S ? split_lo(ntot, 2 * pr + 2, S) : mid;
    const int nit = max(mid - lo0, hi1 - mid);
    const int lo = team ? mid : lo0, hi = team ? hi1 : mid;
    const LList list = {lst};
    // the second half computes the row blocks two SIMDs over, so that each
    // SIMD carries two different row blocks' hot tiles
    fa_split<D, T, kPass2, true, true, 2 * QT + VW>(g, (const T*)a.q, (const T*)a.k, (const T*)a.v, f, a, S,
                                       u, wg, sp, wave & 3, (wave & 3) ^ (team << 1),
                                       fsm + (size_t)team * FaCfg<D>::BYTES, lo, hi, nit, list);
    if (S == 1) continue;  // the split merged itself with the cold state
    // split states complete before the count; the last ticket merges them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (wave == 0) bc[2] = wave_fetch_add(done + item, 1, lane) == npairs - 1;
    __syncthreads();
    if (!__builtin_amdgcn_readfirstlane(bc[2])) continue;
    // wave w merges rows 16 (w % 2) .. + 15 of row block w / 2
    {
      const WaveRows wr = wave_rows(g, rb, wg, wave >> 1);
      if (wr.live) {
        const size_t bhq = (size_t)(u / g.Hkv) * g.Hq + (u % g.Hkv) * g.G + wr.gi;
        combine_rows<D, T>(g, f, a, S, nrows, bhq, wr.r0, 16 * (wave & 1), lane);
      }
    }
  }
}

template <int D, typename T, int QT, bool VW>
hipError_t run_fused(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                     const Pass1Out& o, void* split, const Pass2Args& a, int32_t* ctl,
                     hipStream_t s) {
  const int nunits = g.B * g.Hkv * (g.NqP / 32) * g.G;
  const int sched = split ? pass1_sched(g) : kSchedWhole;
  const int per = sched == kSchedTriples ? 3 * kFusedWaves / 4
                  : (sched == kSchedPairs ? kFusedWaves / 2 : kFusedWaves);
  const int n1 = (nunits + per - 1) / per;
  const int cap = sched != kSchedWhole ? cand_cap(g, sched) : 0;
  const int S = attn_splits(g);
  const RowBlocks rb = row_blocks(g);
  const int nitems = g.B * g.Hkv * rb.nwg;
  const int nctl = kCtlWords + 2 * nitems;
  hipLaunchKernelGGL(k_fused_init, dim3((nctl + 255) / 256), dim3(256), 0, s, ctl, nctl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto kern = k_fused<D, T, true, QT, VW>;
  constexpr size_t bytes = fused_lds<D, true>();
  static bool attr_done = false;
  if (!attr_done) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)bytes);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  int dev = 0, cus = 0;
  e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const int n2 = nitems * ((S + 1) / 2);
  const int grid = max(1, min(cus, n1 + n2));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kFusedWaves * 64), bytes, s, g, f, eps, tau, hoff, o,
                     (uint8_t*)split, cap, sched, nunits, n1, a, S, ctl);
  return hipGetLastError();
}

}  // namespace

bool fused_covers(const Geom& g) {
  if ((g.D != 64 && g.D != 128) || g.ring) return false;
  if (g.NT > kLogTiles) return false;
  return g.NT <= (g.D == 64 ? list_cap<64>() : list_cap<128>());
}

size_t fused_ctl_bytes(const Geom& g) {
  const int nitems = g.B * g.Hkv * row_blocks(g).nwg;
  return ((size_t)(kCtlWords + 2 * nitems) * 4 + 255) & ~(size_t)255;
}

hipError_t launch_fused(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                        const Pass1Out& o, void* split, const Pass2Args& a, int32_t* ctl,
                        hipStream_t s) {
  if (!fused_covers(g)) return hipErrorInvalidValue;
  // (head size, input type, Q terms, value-norm weights) as the separate
  // launches take them
  auto go = [&](auto d, auto t, auto qt, auto vw) {
    return run_fused<decltype(d)::value, decltype(t), decltype(qt)::value, decltype(vw)::value>(
        g, f, eps, tau, hoff, o, split, a, ctl, s);
  };
  auto by_d = [&](auto t, auto qt, auto vw) {
    if (g.D == 64) return go(std::integral_constant<int, 64>{}, t, qt, vw);
    return go(std::integral_constant<int, 128>{}, t, qt, vw);
  };
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using T = std::true_type;
  using F = std::false_type;
  if (g.bf16) {
    if (g.qterms == 2) return g.vweight ? by_d(__bf16{}, Q2{}, T{}) : by_d(__bf16{}, Q2{}, F{});
    return g.vweight ? by_d(__bf16{}, Q1{}, T{}) : by_d(__bf16{}, Q1{}, F{});
  }
  if (g.qterms == 2) return g.vweight ? by_d(_Float16{}, Q2{}, T{}) : by_d(_Float16{}, Q2{}, F{});
  return g.vweight ? by_d(_Float16{}, Q1{}, T{}) : by_d(_Float16{}, Q1{}, F{});
}

}  // namespace apa
