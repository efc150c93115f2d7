// a3..a7: pass 1 of APA, its kernels and launchers ("APA: sloppy attention,
// exact where it counts", rfriedmann.de, section "Pass 1: FP4 everywhere, with
// a hot test"); the walk itself is in pass1_core.h.
#include "pass1_core.h"

namespace apa {

namespace {

template <int D, bool LOG, int QT, bool VW>
__global__ __launch_bounds__(kP1Waves<D> * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>))) void k_pass1(
    Geom g, Fp4Ptrs f, float eps, float tau, int hoff, Pass1Out out, uint8_t* split, int cap,
    int sched, int nunits) {
  __shared__ P1Lds<D, LOG> L;
  // work groups in descending unit order: with causal masking the last row
  // blocks of a kv-head have the longest visit orders, and they start first
  // (the dispatcher then fills in with shorter ones); XCD ranges stay contiguous
  const int blk = (int)gridDim.x - 1 - xcd_remap(blockIdx.x, gridDim.x);
  pass1_block<D, LOG, QT, VW>(g, f, eps, tau, hoff, out, split, cap, sched, nunits, blk, L);
}

template <int D, bool LOG, int QT, bool VW>
__global__ __launch_bounds__(64) void k_pass1_rewalk(Geom g, Fp4Ptrs f, float eps, float tau,
                                                     int hoff, Pass1Out out, uint8_t* split,
                                                     int cap, int sched) {
  __shared__ uint8_t vlog_sh[LOG ? kLogTiles : 1];
  rewalk_unit<D, LOG, QT, VW>(g, f, eps, tau, hoff, out, split, cap, sched, blockIdx.x,
                              (lds_u8*)vlog_sh);
}

// KV window ring ("What else is in the box": the FP4 copy of K and V kept to
// a sink tile and two ring halves): the walk of every unit cut at fixed key
// tile ranges [t_lo, t_hi], one launch per range from the top down, so that
// only the range being walked needs FP4 blobs (the next one is coded into the
// other half meanwhile).  A launch walks each unit's positions whose tiles lie
// in the range (a contiguous run of its visit order: 0, d, d-1, ..., 1); the
// first launch also takes tile 0 and starts the state, the last writes the
// outputs; in between each unit's state waits in the workspace (the hand-off
// layout of the split schedules).  The same walk over the same positions in
// the same order as one unbroken walk: the same verdicts, state and outputs.
// One wave per unit (no value-norm weights, no window, D <= 256).
template <int D, bool LOG, int QT>
__global__ __launch_bounds__(64) void k_pass1_seg(Geom g, Fp4Ptrs f, float eps, float tau,
                                                  int hoff, Pass1Out out, uint8_t* state,
                                                  int t_lo, int t_hi, int first, int last) {
  const int lane = threadIdx.x;
  // units of one kv-head on one XCD, so its L2 holds that head's segment
  const int u = xcd_remap(blockIdx.x, gridDim.x);
  Ctx<D, QT> c;
  make_ctx<D>(c, g, f, out, unit_id(g, u), lane);
  load_q2<D>(c, g, f, lane);
  // the unit's positions of tiles [a, b]: dW + 1 - b .. dW + 1 - a; with
  // tile 0 first in the first launch (then b == dW whenever a <= dW, since
  // the first range holds the highest diagonal)
  const int a = max(t_lo, 1), b = min(t_hi, c.dW);
  int p0 = b >= a ? c.dW + 1 - b : 0;
  int cnt = b >= a ? b - a + 1 : 0;
  if (first) {
    p0 = 0;
    cnt += 1;
  }
  float* slot = reinterpret_cast<float*>(state + (size_t)u * handoff_bytes(D));
  St<D> st;
  Words wd = {-1, 0u, 0u, 0u, 0u};
  if (first) {
    init_state<D>(st, c.row_ok);
    zero_outside<D>(g, c, lane);
  } else {
    load_state<D>(slot, st, wd, lane);
    wd.wb = -1;
  }
  if (cnt > 0) {
    __shared__ uint8_t vlog_sh[LOG ? kLogTiles : 1];
    walk<D, LOG, false, false, QT, true>(g, c, st, wd, 0, p0, cnt, eps, tau, (float)hoff,
                                         cand_of(f.kv_blob, 0, 0, D), 0, nullptr, nullptr,
                                         (lds_u8*)vlog_sh, lane);
  }
  if (!last) {
    save_state<D>(slot, st, wd, lane);
    return;
  }
  if (lane == 0 && c.lead) {
    c.bits0[0] = wd.p00;
    if (c.has_g1) c.bits1[0] = wd.p01;
  }
  store_state<D>(g, c, out, st, lane);
}


}  // namespace

size_t pass1_ws_bytes(const Geom& g) {
  const int s = pass1_sched(g);
  if (s == kSchedWhole) return 0;
  return (size_t)g.B * g.Hkv * (g.NqP / 32) * g.G * cand_stride(cand_cap(g, s), g.D);
}

int pass1_split_info(const Geom& g, int npos, int* cut, int* cap) {
  const int s = pass1_sched(g);
  if (cut) *cut = s == kSchedWhole ? npos : split_cut(npos, s);
  if (cap) *cap = s == kSchedWhole ? 0 : cand_cap(g, s);
  return s;
}

namespace {

template <int D, int QT>
hipError_t run_qt(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                  const Pass1Out& o, void* ws, hipStream_t s) {
  const int nunits = g.B * g.Hkv * (g.NqP / 32) * g.G;
  if (nunits == 0) return hipSuccess;
  const int sched = ws ? pass1_sched(g) : kSchedWhole;
  uint8_t* split = sched != kSchedWhole ? static_cast<uint8_t*>(ws) : nullptr;
  constexpr int W = kP1Waves<D>;
  const int per = sched == kSchedTriples ? 3 * W / 4
                  : (sched == kSchedPairs ? W / 2 : W / kOutSplit<D>);
  const int nblocks = (nunits + per - 1) / per;
  const int cap = split ? cand_cap(g, sched) : 0;
  const bool log = g.NT <= kLogTiles;
  // kernels per (log, weighted): the mass test carries no weight loads
  auto main = [&](auto lg, auto vw) {
    hipLaunchKernelGGL((k_pass1<D, decltype(lg)::value, QT, decltype(vw)::value>),
                       dim3(nblocks), dim3(W * 64), 0, s, g, f, eps, tau, hoff, o, split, cap,
                       sched, nunits);
  };
  auto rewalk = [&](auto lg, auto vw) {
    hipLaunchKernelGGL((k_pass1_rewalk<D, decltype(lg)::value, QT, decltype(vw)::value>),
                       dim3(nunits), dim3(64), 0, s, g, f, eps, tau, hoff, o, split, cap, sched);
  };
  using T = std::true_type;
  using F = std::false_type;
  if (log) {
    if (g.vweight) main(T{}, T{}); else main(T{}, F{});
  } else {
    if (g.vweight) main(F{}, T{}); else main(F{}, F{});
  }
  if constexpr (kOutSplit<D> == 1) {
    if (!split) return hipGetLastError();
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (log) {
      if (g.vweight) rewalk(T{}, T{}); else rewalk(T{}, F{});
    } else {
      if (g.vweight) rewalk(F{}, T{}); else rewalk(F{}, F{});
    }
  }
  return hipGetLastError();
}

// One Q term, or two (up to D = 256: at D = 512 the second term's operands
// do not fit beside the others).
template <int D>
hipError_t run(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
               const Pass1Out& o, void* ws, hipStream_t s) {
  if (g.qterms == 2) {
    if constexpr (D <= 256) return run_qt<D, 2>(g, f, eps, tau, hoff, o, ws, s);
    return hipErrorInvalidValue;
  }
  return run_qt<D, 1>(g, f, eps, tau, hoff, o, ws, s);
}

template <int D, int QT>
hipError_t run_seg(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                   const Pass1Out& o, void* state, int t_lo, int t_hi, int first, int last,
                   hipStream_t s) {
  const int nunits = g.B * g.Hkv * (g.NqP / 32) * g.G;
  if (nunits == 0) return hipSuccess;
  uint8_t* st = static_cast<uint8_t*>(state);
  if (g.NT <= kLogTiles)
    hipLaunchKernelGGL((k_pass1_seg<D, true, QT>), dim3(nunits), dim3(64), 0, s, g, f, eps, tau,
                       hoff, o, st, t_lo, t_hi, first, last);
  else
    hipLaunchKernelGGL((k_pass1_seg<D, false, QT>), dim3(nunits), dim3(64), 0, s, g, f, eps, tau,
                       hoff, o, st, t_lo, t_hi, first, last);
  return hipGetLastError();
}

template <int D>
hipError_t run_seg_d(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                     const Pass1Out& o, void* state, int t_lo, int t_hi, int first, int last,
                     hipStream_t s) {
  if (g.qterms == 2) return run_seg<D, 2>(g, f, eps, tau, hoff, o, state, t_lo, t_hi, first, last, s);
  return run_seg<D, 1>(g, f, eps, tau, hoff, o, state, t_lo, t_hi, first, last, s);
}

}  // namespace

size_t pass1_seg_state_bytes(const Geom& g) {
  return (size_t)g.B * g.Hkv * (g.NqP / 32) * g.G * handoff_bytes(g.D);
}

hipError_t launch_pass1_segment(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                                const Pass1Out& o, void* state, int t_lo, int t_hi, int first,
                                int last, hipStream_t s) {
  switch (g.D) {
    case 64: return run_seg_d<64>(g, f, eps, tau, hoff, o, state, t_lo, t_hi, first, last, s);
    case 128: return run_seg_d<128>(g, f, eps, tau, hoff, o, state, t_lo, t_hi, first, last, s);
    case 256: return run_seg_d<256>(g, f, eps, tau, hoff, o, state, t_lo, t_hi, first, last, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pass1(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                        const Pass1Out& o, void* ws, hipStream_t s) {
  switch (g.D) {
    case 64: return run<64>(g, f, eps, tau, hoff, o, ws, s);
    case 128: return run<128>(g, f, eps, tau, hoff, o, ws, s);
    case 256: return run<256>(g, f, eps, tau, hoff, o, ws, s);
    case 512: return run<512>(g, f, eps, tau, hoff, o, ws, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace apa
