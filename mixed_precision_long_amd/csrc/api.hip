// C ABI of the APA library: validation, buffer layout, workspace sizing and
// stream-ordered launches.  No allocation, no synchronisation, no exceptions
// across the ABI.  Declarations and argument documentation: include/apa.h.
#include <math.h>
#include <string.h>

#include <mutex>

#include "../../include/apa.h"
#include "apa_kernels.h"

using namespace apa;

// Scratch of apa_quantize_static: a fixed device array of the library, one
// copy per GPU (held until the process ends).  In host code `scratch` names
// a host-side stand-in, not device memory: its device address is fetched
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is handed to kernels.  The statistics kernels write
// every word they later read (partial sums, extrema, flags), so nothing in
// it needs clearing between calls.
constexpr size_t kStaticScratch = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratch];

namespace {

constexpr float kLog2e32 = 1.44269502162933349609375f;  // fl32(log2 e)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
size_t rup(size_t x, size_t m) { return (x + m - 1) / m * m; }

bool valid_problem(const apa_problem* p) {
  if (!p) return false;
  if (p->B < 0 || p->Hq < 0 || p->Hkv < 1 || p->Nq < 0 || p->Nkv < 0) return false;
  if (p->Hq % p->Hkv != 0) return false;
  if (p->D != 64 && p->D != 128 && p->D != 256 && p->D != 512) return false;
  if (p->dtype != APA_F16 && p->dtype != APA_BF16) return false;
  if (p->is_causal != 0 && p->is_causal != 1) return false;
  if (p->is_causal && p->Nkv < p->Nq) return false;
  if (p->tile != 64 || p->row_group != 16) return false;
  if (p->fmt != APA_MXFP4 && p->fmt != APA_NVFP4) return false;
  if (!(p->tau >= 0.0f && p->tau <= 32.0f)) return false;
  const float H = p->hot_frame_offset;
  if (!(H >= 0.0f && H <= 64.0f) || floorf(H) != H) return false;
  if (isnan(p->scale)) return false;
  if (p->Nq > 0 && p->Nkv == 0) return false;
  if (p->pass1_schedule < APA_SCHED_AUTO || p->pass1_schedule > APA_SCHED_TRIPLES) return false;
  if (p->q_terms != 1 && p->q_terms != 2) return false;
  if (p->k_scale_lsq != 0 && p->k_scale_lsq != 1) return false;
  if (p->window < 0 || (p->window > 0 && !p->is_causal)) return false;
  if (p->kv_capacity < 0 || (p->kv_capacity > 0 && p->kv_capacity < p->Nkv)) return false;
  if (p->stat_keys < 0 || p->stat_keys > p->Nkv) return false;
  if (p->block_table && (p->block_table_stride < (p->Nkv + 63) / 64)) return false;
  if (p->hot_weight != 0 && p->hot_weight != 1) return false;
  if (p->ring_tiles < 0 || p->ring_tiles % 32 != 0) return false;
  return true;
}

bool empty(const apa_problem* p) { return p->B == 0 || p->Hq == 0 || p->Nq == 0; }

Geom geom(const apa_problem* p) {
  Geom g;
  g.B = p->B; g.Hq = p->Hq; g.Hkv = p->Hkv; g.G = p->Hq / p->Hkv;
  g.Nq = p->Nq; g.Nkv = p->Nkv; g.D = p->D;
  g.NqP = (int)rup(p->Nq, 32);
  g.NT = (p->Nkv + 63) / 64;
  g.NkvP = g.NT * 64;
  g.NG = (p->Nq + 15) / 16;
  g.W = (g.NT + 31) / 32;
  g.causal = p->is_causal;
  g.off = p->Nkv - p->Nq;
  g.bf16 = p->dtype == APA_BF16;
  const float scale = p->scale > 0.0f ? p->scale : (float)(1.0 / sqrt((double)p->D));
  g.sl = scale * kLog2e32;
  g.sched = p->pass1_schedule;
  g.qterms = p->q_terms;
  g.klsq = p->k_scale_lsq;
  g.window = p->window;
  g.NTc = p->kv_capacity > 0 ? (p->kv_capacity + 63) / 64 : g.NT;
  g.stat_hi = p->stat_keys > 0 ? p->stat_keys : p->Nkv;
  g.qt0 = first_key_tile(g);
  g.qt1 = g.NT;
  g.ct0 = g.qt0;
  g.ct1 = g.qt1;
  g.frozen = 0;
  g.keep_status = 0;
  g.code_q = 1;
  g.ring = p->ring_tiles;
  g.ring_delta = 0;
  if (g.ring) g.NTc = 1 + 2 * g.ring;
  g.bt = p->block_table;
  g.bts = p->block_table_stride;
  g.vweight = p->hot_weight;
  return g;
}

void layout(const apa_problem* p, apa_fp4_layout* L) {
  const Geom g = geom(p);
  const size_t B = p->B, Hq = p->Hq, Hkv = p->Hkv, D = p->D;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  // the K/V sections first (sized by the capacity), so that a persistent
  // cache keeps them in place while the query sections change
  L->kv_blobs = take(B * Hkv * g.NTc * blob_bytes(p->D));
  L->kbar = take(B * Hkv * D * 4);
  L->kv_head = take(B * Hkv * 8 * 4);
  L->tile_w = take(B * Hkv * g.NTc * 4);
  L->status = take(4);
  L->q_codes = take(B * Hq * g.NqP * D / 2);
  L->q_scales = take(B * Hq * g.NqP * D / 32);
  L->q_head = take(B * Hq * 4 * 4);
  L->q_frame = take(B * Hq * g.NqP * 4);
  const size_t q2 = p->q_terms == 2 ? 1 : 0;
  L->q2_codes = take(q2 * B * Hq * g.NqP * D / 2);
  L->q2_scales = take(q2 * B * Hq * g.NqP * D / 32);
  L->total = o;
}

Fp4Ptrs fp4_ptrs(const apa_problem* p, const void* base) {
  apa_fp4_layout L;
  layout(p, &L);
  uint8_t* b = (uint8_t*)base;
  Fp4Ptrs f;
  f.q_codes = b + L.q_codes; f.q_scales = b + L.q_scales;
  f.kv_blob = b + L.kv_blobs;
  f.kbar = (float*)(b + L.kbar); f.kv_head = (float*)(b + L.kv_head);
  f.q_head = (float*)(b + L.q_head); f.q_frame = (float*)(b + L.q_frame);
  f.status = (unsigned*)(b + L.status);
  f.tile_w = (float*)(b + L.tile_w);
  f.q2_codes = p->q_terms == 2 ? b + L.q2_codes : nullptr;
  f.q2_scales = p->q_terms == 2 ? b + L.q2_scales : nullptr;
  return f;
}

size_t quant_ws(const apa_problem* p, QuantWs* ws, void* base) {
  const Geom g = geom(p);
  const int nch = (g.NT + 15) / 16;
  const int nvz = (p->D + 127) / 128;
  const size_t nkv = (size_t)p->B * p->Hkv * nch;
  const size_t nvi = (size_t)p->B * p->Hkv * g.NT * nvz;
  const int nqt = (p->Nq + 63) / 64;
  const size_t nqf = (size_t)p->B * p->Hq * nqt;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const size_t a = take(nkv * p->D * 8), b = take(nkv * p->D * 4), c = take(nkv * p->D * 4),
               d = take((nvi > 0 ? nvi : 1) * 4), e = take((nqf > 0 ? nqf : 1) * 4),
               fl = take((nkv + nvi + nqf > 0 ? nkv + nvi + nqf : 1) * 4);
  // value norms, with the weighted hot test only
  const size_t vn = p->hot_weight ? (size_t)p->B * p->Hkv * g.NT : 0;
  const size_t t1 = take(vn * 4), s1 = take(vn * 8);
  if (ws && base) {
    uint8_t* bb = (uint8_t*)base;
    ws->ksum = (double*)(bb + a); ws->kmin = (float*)(bb + b); ws->kmax = (float*)(bb + c);
    ws->vamax = (float*)(bb + d); ws->qamax = (float*)(bb + e);
    ws->flags = (unsigned*)(bb + fl);
    ws->vnt = vn ? (float*)(bb + t1) : nullptr;
    ws->vnst = vn ? (double*)(bb + s1) : nullptr;
    ws->nqt = nqt;
    ws->nch = nch;
    ws->nvz = nvz;
    ws->ch0 = g.qt0 / 16;
    ws->ch1 = (g.qt1 + 15) / 16;
  }
  return o;
}

// Split states of the 16-bit attention kernels (none when one split suffices).
size_t split_ws(const apa_problem* p, size_t o, Pass2Args* a, void* base) {
  const Geom g = geom(p);
  const int S = attn_splits(g);
  if (S <= 1) return o;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const size_t rows = (size_t)p->B * p->Hq * p->Nq;
  const size_t m = take(S * rows * 4), l = take(S * rows * 4), po = take(S * rows * p->D * 4);
  if (a && base) {
    uint8_t* bb = (uint8_t*)base;
    a->part_m = (float*)(bb + m); a->part_l = (float*)(bb + l); a->part_o = (float*)(bb + po);
  }
  return o;
}

size_t pass2_ws(const apa_problem* p, Pass2Args* a, void* base) {
  const Geom g = geom(p);
  const size_t units = (size_t)attn_units(g);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const size_t t = take(units * g.NT * 4), m = take(units * g.NT * 4), c = take(units * 4),
               r = take(units * 4);
  if (a && base) {
    uint8_t* bb = (uint8_t*)base;
    a->list_tiles = (int32_t*)(bb + t); a->list_masks = (uint32_t*)(bb + m);
    a->list_count = (int32_t*)(bb + c); a->list_order = (int32_t*)(bb + r);
  }
  return split_ws(p, o, a, base);
}

// The single launch's workspace: its control words, the pass-1 workspace,
// then the split states.
size_t fused_ws(const apa_problem* p, int32_t** ctl, void** split, Pass2Args* a, void* base) {
  const Geom g = geom(p);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  const size_t c = take(fused_ctl_bytes(g));
  const size_t p1 = pass1_ws_bytes(g);
  const size_t s1 = take(p1);
  if (base) {
    uint8_t* bb = (uint8_t*)base;
    if (ctl) *ctl = (int32_t*)(bb + c);
    if (split) *split = p1 ? (void*)(bb + s1) : nullptr;
  }
  return split_ws(p, o, a, base);
}

// The exact path's workspace: with bf16 inputs the per-(b, kv-head, key
// chunk) maxima of |V|, then the split states.
size_t exact_ws(const apa_problem* p, Pass2Args* a, void* base) {
  size_t o = 0;
  if (p->dtype == APA_BF16 && p->Nkv > 0) {
    const int nch = (p->Nkv + kVmaxChunk - 1) / kVmaxChunk;
    if (a && base) {
      a->vmax = (float*)base;
      a->vmax_nch = nch;
    }
    o = align256((size_t)p->B * p->Hkv * nch * 4);
  }
  return split_ws(p, o, a, base);
}

// D and dtype the device kernels implement for each call
bool kernels_cover(const apa_problem* p, int call) {
  if (p->fmt != APA_MXFP4) return false;
  // the ring's blobs are written and walked by apa_ring_pass1 only
  if (p->ring_tiles > 0 && (call == APA_CALL_QUANTIZE || call == APA_CALL_PASS1)) return false;
  if (call == APA_CALL_RING_PASS1)
    return p->ring_tiles > 0 && p->D <= 256 && p->window == 0 && p->hot_weight == 0;
  if (call == APA_CALL_FUSED) {
    const int G = p->Hq / p->Hkv;
    return (G == 1 || G == 2 || G == 3 || G == 4 || G == 6 || G == 8) && fused_covers(geom(p));
  }
  if (p->q_terms == 2 && p->D > 256 && (call == APA_CALL_QUANTIZE || call == APA_CALL_PASS1))
    return false;
  if (call == APA_CALL_QUANTIZE || call == APA_CALL_PASS1 || call == APA_CALL_MERGE) return true;
  const int G = p->Hq / p->Hkv;
  if (call == APA_CALL_PASS2 || call == APA_CALL_EXACT)
    return G == 1 || G == 2 || G == 3 || G == 4 || G == 6 || G == 8;
  return true;
}

thread_local hipError_t g_last_hip = hipSuccess;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, fetched on its first use.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

apa_status hip_status(hipError_t e) {
  g_last_hip = e;
  return e == hipSuccess ? APA_OK : APA_ERR_HIP;
}

// Drop any error a previous, unrelated HIP call left behind, so a launch check
// reports only this call's kernels.
void clear_hip_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

void apa_problem_init(apa_problem* p, int32_t B, int32_t Hq, int32_t Hkv, int32_t Nq,
                      int32_t Nkv, int32_t D) {
  if (!p) return;
  memset(p, 0, sizeof(*p));
  p->B = B; p->Hq = Hq; p->Hkv = Hkv; p->Nq = Nq; p->Nkv = Nkv; p->D = D;
  p->dtype = APA_F16;
  p->is_causal = 1;
  p->scale = 0.0f;
  p->tile = 64;
  p->row_group = 16;
  p->fmt = APA_MXFP4;
  p->tau = 4.0f;
  p->hot_frame_offset = 32.0f;
  p->pass1_schedule = APA_SCHED_AUTO;
  p->q_terms = 1;
  p->k_scale_lsq = 0;
  p->window = 0;
  p->kv_capacity = 0;
  p->stat_keys = 0;
  p->block_table = nullptr;
  p->block_table_stride = 0;
  p->hot_weight = 0;
  p->ring_tiles = 0;
}

const char* apa_last_hip_error(void) { return hipGetErrorString(g_last_hip); }

const char* apa_status_string(apa_status s) {
  switch (s) {
    case APA_OK: return "APA_OK";
    case APA_ERR_INVALID_ARG: return "APA_ERR_INVALID_ARG: invalid argument";
    case APA_ERR_UNSUPPORTED: return "APA_ERR_UNSUPPORTED: not implemented for this problem";
    case APA_ERR_WORKSPACE: return "APA_ERR_WORKSPACE: workspace too small";
    case APA_ERR_HIP: return "APA_ERR_HIP: kernel launch failed";
  }
  return "APA: unknown status";
}

apa_status apa_fp4_layout_of(const apa_problem* p, apa_fp4_layout* out) {
  if (!valid_problem(p) || !out) return APA_ERR_INVALID_ARG;
  layout(p, out);
  return APA_OK;
}

size_t apa_fp4_bytes(const apa_problem* p) {
  if (!valid_problem(p)) return 0;
  apa_fp4_layout L;
  layout(p, &L);
  return L.total;
}

size_t apa_hotmask_bytes(const apa_problem* p) {
  if (!valid_problem(p)) return 0;
  const Geom g = geom(p);
  return (size_t)p->B * p->Hq * g.NG * g.W * 4;
}

size_t apa_workspace_bytes(const apa_problem* p, int32_t which) {
  if (!valid_problem(p)) return 0;
  switch (which) {
    case APA_CALL_QUANTIZE: return quant_ws(p, nullptr, nullptr);
    case APA_CALL_PASS1: return pass1_ws_bytes(geom(p));
    case APA_CALL_PASS2: return pass2_ws(p, nullptr, nullptr);
    case APA_CALL_EXACT: return exact_ws(p, nullptr, nullptr);
    case APA_CALL_RING_PASS1:
      return p->ring_tiles > 0 ? align256(quant_ws(p, nullptr, nullptr)) +
                                     pass1_seg_state_bytes(geom(p))
                               : 0;
    case APA_CALL_FUSED:
      return kernels_cover(p, APA_CALL_FUSED) ? fused_ws(p, nullptr, nullptr, nullptr, nullptr) : 0;
    default: return 0;
  }
}

apa_status apa_quantize(const apa_problem* p, const void* q, const void* k, const void* v,
                        void* fp4, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!q || !k || !v || !fp4) return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_QUANTIZE)) return APA_ERR_UNSUPPORTED;
  if (p->B == 0 || p->Hkv == 0) return APA_OK;
  const size_t need = quant_ws(p, nullptr, nullptr);
  if (!ws || ws_bytes < need) return APA_ERR_WORKSPACE;
  QuantWs w;
  quant_ws(p, &w, ws);
  clear_hip_error();
  return hip_status(launch_quantize(geom(p), q, k, v, fp4_ptrs(p, fp4), w, (hipStream_t)stream));
}

apa_status apa_quantize_tiles(const apa_problem* p, const void* q, const void* k, const void* v,
                              void* fp4, int32_t tile_begin, int32_t tile_end, void* ws,
                              size_t ws_bytes, void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!q || !k || !v || !fp4) return APA_ERR_INVALID_ARG;
  Geom g = geom(p);
  if (tile_begin < first_key_tile(g) || tile_end > g.NT || tile_begin > tile_end)
    return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_QUANTIZE)) return APA_ERR_UNSUPPORTED;
  if (p->B == 0 || p->Hkv == 0) return APA_OK;
  const size_t need = quant_ws(p, nullptr, nullptr);
  if (!ws || ws_bytes < need) return APA_ERR_WORKSPACE;
  g.frozen = 1;
  g.qt0 = g.ct0 = tile_begin;
  g.qt1 = g.ct1 = tile_end;
  QuantWs w;
  quant_ws(p, &w, ws);
  w.ch0 = tile_begin / 16;
  w.ch1 = (tile_end + 15) / 16;
  clear_hip_error();
  return hip_status(launch_quantize(g, q, k, v, fp4_ptrs(p, fp4), w, (hipStream_t)stream));
}

apa_status apa_quantize_static(const apa_problem* p, const void* q, const void* k, const void* v,
                               void* fp4, void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!q || !k || !v || !fp4) return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_QUANTIZE)) return APA_ERR_UNSUPPORTED;
  if (p->B == 0 || p->Hkv == 0) return APA_OK;
  if (quant_ws(p, nullptr, nullptr) > kStaticScratch) return APA_ERR_WORKSPACE;
  clear_hip_error();
  void* base = nullptr;
  const hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return hip_status(e);
  QuantWs w;
  quant_ws(p, &w, base);
  return hip_status(launch_quantize(geom(p), q, k, v, fp4_ptrs(p, fp4), w, (hipStream_t)stream));
}

apa_status apa_pass1(const apa_problem* p, const void* fp4, float eps, int32_t* cold_m,
                     float* cold_l, float* cold_o, uint32_t* hot_bits, float* lambda_out,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!fp4 || !cold_m || !cold_l || !cold_o || !hot_bits) return APA_ERR_INVALID_ARG;
  if (isnan(eps) || eps < 0.0f) return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_PASS1)) return APA_ERR_UNSUPPORTED;
  if (empty(p)) return APA_OK;
  // the workspace is optional: without it every unit runs as one wave
  const size_t need = pass1_ws_bytes(geom(p));
  if (need > 0 && ws && ws_bytes < need) return APA_ERR_WORKSPACE;
  Pass1Out o = {cold_m, cold_l, cold_o, hot_bits, lambda_out};
  clear_hip_error();
  return hip_status(launch_pass1(geom(p), fp4_ptrs(p, fp4), eps, p->tau,
                                 (int)p->hot_frame_offset, o, need > 0 ? ws : nullptr,
                                 (hipStream_t)stream));
}

namespace {

// The stream each device's ring quantisation runs on (created on first use,
// default priority, never blocking the null stream).
std::mutex g_ring_mu;
hipStream_t g_ring_stream[kMaxDevices] = {};

hipError_t ring_stream(hipStream_t* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_ring_mu);
  if (!g_ring_stream[dev]) {
    e = hipStreamCreateWithFlags(&g_ring_stream[dev], hipStreamNonBlocking);
    if (e != hipSuccess) return e;
  }
  *out = g_ring_stream[dev];
  return hipSuccess;
}

}  // namespace

apa_status apa_ring_pass1(const apa_problem* p, const void* q, const void* k, const void* v,
                          void* fp4, float eps, int32_t* cold_m, float* cold_l, float* cold_o,
                          uint32_t* hot_bits, float* lambda_out, void* ws, size_t ws_bytes,
                          void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!q || !k || !v || !fp4 || !cold_m || !cold_l || !cold_o || !hot_bits)
    return APA_ERR_INVALID_ARG;
  if (isnan(eps) || eps < 0.0f) return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_RING_PASS1)) return APA_ERR_UNSUPPORTED;
  if (p->B == 0 || p->Hkv == 0) return APA_OK;
  const size_t qbytes = align256(quant_ws(p, nullptr, nullptr));
  const Geom g0 = geom(p);
  if (!ws || ws_bytes < qbytes + pass1_seg_state_bytes(g0)) return APA_ERR_WORKSPACE;
  QuantWs w;
  quant_ws(p, &w, ws);
  uint8_t* state = static_cast<uint8_t*>(ws) + qbytes;
  const Fp4Ptrs f = fp4_ptrs(p, fp4);
  const hipStream_t ps = (hipStream_t)stream;
  clear_hip_error();
  hipStream_t qs;
  hipError_t e = ring_stream(&qs);
  if (e != hipSuccess) return hip_status(e);
  // 1. statistics over every key, Q's codes, the sink tile's codes
  Geom gs = g0;
  gs.ct0 = 0;
  gs.ct1 = g0.NT > 0 ? 1 : 0;
  e = launch_quantize(gs, q, k, v, f, w, ps);
  if (e != hipSuccess || empty(p)) return hip_status(e);
  // 2. the segments, top down: segment s holds tiles [s R, s R + R), tile 0
  // excepted, in ring half s % 2; the walk of s waits for its codes, the codes
  // of s wait for the walk of s + 2 (the last reader of that half)
  const int R = p->ring_tiles;
  const int top = (g0.NT - 1) / R;
  hipEvent_t ev_stats = nullptr, ev_q[2] = {}, ev_p[2] = {};
  auto make = [&](hipEvent_t* x) {
    return e == hipSuccess ? (e = hipEventCreateWithFlags(x, hipEventDisableTiming)) : e;
  };
  for (hipEvent_t* x : {&ev_stats, &ev_q[0], &ev_q[1], &ev_p[0], &ev_p[1]}) (void)make(x);
  if (e == hipSuccess) e = hipEventRecord(ev_stats, ps);
  if (e == hipSuccess) e = hipStreamWaitEvent(qs, ev_stats, 0);
  Pass1Out o = {cold_m, cold_l, cold_o, hot_bits, lambda_out};
  for (int sgm = top; sgm >= 0 && e == hipSuccess; --sgm) {
    const int h = sgm & 1;
    Geom gq = g0;
    gq.frozen = 1;
    gq.keep_status = 1;
    gq.code_q = 0;
    gq.qt0 = sgm * R;
    gq.qt1 = gq.ct1 = min(g0.NT, sgm * R + R);
    // tile 0 stays in its sink slot from step 1 (the first walk may still be
    // reading it while segment 0 is coded)
    gq.ct0 = sgm == 0 ? min(1, gq.ct1) : sgm * R;
    gq.ring_delta = 1 + h * R - sgm * R;
    QuantWs wq = w;
    wq.ch0 = gq.qt0 / 16;
    wq.ch1 = (gq.qt1 + 15) / 16;
    if ((e = hipStreamWaitEvent(qs, ev_p[h], 0)) != hipSuccess) break;
    if ((e = launch_quantize(gq, q, k, v, f, wq, qs)) != hipSuccess) break;
    if ((e = hipEventRecord(ev_q[h], qs)) != hipSuccess) break;
    if ((e = hipStreamWaitEvent(ps, ev_q[h], 0)) != hipSuccess) break;
    Geom gp = g0;
    gp.ring_delta = gq.ring_delta;
    if ((e = launch_pass1_segment(gp, f, eps, p->tau, (int)p->hot_frame_offset, o, state,
                                  sgm * R, sgm * R + R - 1, sgm == top, sgm == 0, ps)) !=
        hipSuccess)
      break;
    e = hipEventRecord(ev_p[h], ps);
  }
  for (hipEvent_t x : {ev_stats, ev_q[0], ev_q[1], ev_p[0], ev_p[1]})
    if (x) (void)hipEventDestroy(x);
  return hip_status(e);
}

int32_t apa_pass1_split(const apa_problem* p, int32_t npos, int32_t* cut, int32_t* records) {
  if (!valid_problem(p) || npos < 0) return -1;
  int c = npos, r = 0;
  const int s = pass1_split_info(geom(p), npos, &c, &r);
  if (cut) *cut = c;
  if (records) *records = r;
  return s;
}

apa_status apa_pass2(const apa_problem* p, const void* q, const void* k, const void* v,
                     const void* fp4, const uint32_t* hot_bits, const int32_t* cold_m,
                     const float* cold_l, const float* cold_o, int32_t fuse_merge, void* out,
                     float* lse, float* hot_m, float* hot_l, float* hot_o, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!q || !k || !v || !fp4 || !hot_bits) return APA_ERR_INVALID_ARG;
  if (fuse_merge != 0 && fuse_merge != 1) return APA_ERR_INVALID_ARG;
  if (fuse_merge && (!cold_m || !cold_l || !cold_o || !out)) return APA_ERR_INVALID_ARG;
  if (!fuse_merge && (!hot_m || !hot_l || !hot_o)) return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_PASS2)) return APA_ERR_UNSUPPORTED;
  if (empty(p)) return APA_OK;
  const size_t need = pass2_ws(p, nullptr, nullptr);
  if (!ws || ws_bytes < need) return APA_ERR_WORKSPACE;
  Pass2Args a = {};
  a.q = q; a.k = k; a.v = v; a.bits = hot_bits;
  a.cold_m = cold_m; a.cold_l = cold_l; a.cold_o = cold_o;
  a.fuse = fuse_merge; a.out = out; a.lse = lse;
  a.hot_m = hot_m; a.hot_l = hot_l; a.hot_o = hot_o;
  pass2_ws(p, &a, ws);
  clear_hip_error();
  return hip_status(launch_pass2(geom(p), fp4_ptrs(p, fp4), a, (hipStream_t)stream));
}

apa_status apa_fused(const apa_problem* p, const void* q, const void* k, const void* v,
                     const void* fp4, float eps, int32_t* cold_m, float* cold_l, float* cold_o,
                     uint32_t* hot_bits, float* lambda_out, void* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!q || !k || !v || !fp4 || !cold_m || !cold_l || !cold_o || !hot_bits || !out)
    return APA_ERR_INVALID_ARG;
  if (isnan(eps) || eps < 0.0f) return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_FUSED)) return APA_ERR_UNSUPPORTED;
  if (empty(p)) return APA_OK;
  const size_t need = fused_ws(p, nullptr, nullptr, nullptr, nullptr);
  if (!ws || ws_bytes < need) return APA_ERR_WORKSPACE;
  Pass1Out o = {cold_m, cold_l, cold_o, hot_bits, lambda_out};
  Pass2Args a = {};
  a.q = q; a.k = k; a.v = v; a.bits = hot_bits;
  a.cold_m = cold_m; a.cold_l = cold_l; a.cold_o = cold_o;
  a.fuse = 1; a.out = out; a.lse = lse;
  int32_t* ctl = nullptr;
  void* split = nullptr;
  fused_ws(p, &ctl, &split, &a, ws);
  clear_hip_error();
  return hip_status(launch_fused(geom(p), fp4_ptrs(p, fp4), eps, p->tau,
                                 (int)p->hot_frame_offset, o, split, a, ctl,
                                 (hipStream_t)stream));
}

apa_status apa_merge(const apa_problem* p, const void* fp4, const int32_t* cold_m,
                     const float* cold_l, const float* cold_o, const float* hot_m,
                     const float* hot_l, const float* hot_o, void* out, float* lse,
                     void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!fp4 || !cold_m || !cold_l || !cold_o || !hot_m || !hot_l || !hot_o || !out)
    return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_MERGE)) return APA_ERR_UNSUPPORTED;
  if (empty(p)) return APA_OK;
  clear_hip_error();
  return hip_status(launch_merge(geom(p), fp4_ptrs(p, fp4), cold_m, cold_l, cold_o, hot_m, hot_l,
                                 hot_o, out, lse, (hipStream_t)stream));
}

apa_status apa_exact(const apa_problem* p, const void* q, const void* k, const void* v,
                     void* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (!valid_problem(p)) return APA_ERR_INVALID_ARG;
  if (!q || !k || !v || !out) return APA_ERR_INVALID_ARG;
  if (!kernels_cover(p, APA_CALL_EXACT)) return APA_ERR_UNSUPPORTED;
  if (empty(p)) return APA_OK;
  const size_t need = exact_ws(p, nullptr, nullptr);
  if (need > 0 && (!ws || ws_bytes < need)) return APA_ERR_WORKSPACE;
  Pass2Args parts = {};
  exact_ws(p, &parts, ws);
  clear_hip_error();
  return hip_status(launch_exact(geom(p), q, k, v, out, lse, parts, (hipStream_t)stream));
}

}  // extern "C"
