// Kernel argument blocks and host-side launchers shared by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace apa {

struct Geom {
  int B, Hq, Hkv, G, Nq, Nkv, D, NqP, NkvP, NT, NG, W, causal, off, bf16;
  float sl;   // fl32(scale * fl32(log2 e))
  int sched;  // requested pass-1 schedule (APA_SCHED_*)
  int qterms; // FP4 terms of Q: 1, or 2 with the residual term
  int klsq;   // 1: K block exponents by least squared error
  int window; // > 0: causal sliding window of this many keys (row r sees
              // keys r + off - window < k <= r + off); 0: none
  int NTc;    // key tiles per (b, kv-head) in the FP4 blob section (capacity >= NT)
  int stat_hi;  // K/V statistics cover keys [first_key_tile * 64, stat_hi)
  int qt0, qt1; // K/V tiles a quantise call reads (statistics and checks)
  int ct0, ct1; // K/V tiles whose codes it writes (within [qt0, qt1), or [0, 1))
  int frozen;   // 1: keep the FP4 buffer's K/V statistics (quantise only tiles)
  int keep_status;  // 1: the call ORs into the status word without clearing it
  int code_q;       // 1: the call reads and codes Q (0: Q's codes and scales stay)
  // KV window ring: 0, or the tiles of each of its two halves; the blob
  // section then holds 1 + 2 * ring slots per (b, kv-head), tile 0 in slot 0
  // and tile t >= 1 of the segment in use at slot t + ring_delta
  int ring, ring_delta;
  // paged 16-bit K/V: logical tile t of batch b is page bt[b * bts + t] of
  // pools [pages][Hkv][64][D]; nullptr: [B][Hkv][Nkv][D]
  const int32_t* bt;
  int bts;
  int vweight;  // 1: the hot test weighs each tile's mass by its value-norm weight
};

// Element offset of key k of (b, kv-head hk) in a 16-bit K or V input.  The
// 64 keys of a tile are contiguous in both layouts.
__device__ __forceinline__ size_t kv_elem(const Geom& g, int b, int hk, int k) {
  if (g.bt) {
    const int pg = g.bt[(size_t)b * g.bts + (k >> 6)];
    return (((size_t)pg * g.Hkv + hk) * 64 + (k & 63)) * g.D;
  }
  return (((size_t)b * g.Hkv + hk) * g.Nkv + k) * g.D;
}

// Per (b, kv-head, 64-key tile) FP4 blob of 68*D bytes, laid out for the
// MFMA operands of pass 1:
//   [0, 32D)     K codes  [64 keys][D/2]
//   [32D, 34D)   K scales [64 keys][D/32]
//   [34D, 66D)   V codes  [D channels][32]: 16 bytes per 32-key half, whose
//                eight 4-key runs are stored in the order 0,2,4,6,1,3,5,7
//   [66D, 68D)   V scales [32][2][D/32]: channel 32*db + n, key half hh at
//                byte (2n + hh) * D/32 + db
struct Fp4Ptrs {
  uint8_t *q_codes, *q_scales, *kv_blob;
  uint8_t *q2_codes, *q2_scales;  // the residual term of Q (nullptr with one term)
  float *kbar, *kv_head, *q_head, *q_frame;
  float* tile_w;  // [B][Hkv][NTc] value-norm weights of the hot test
  unsigned* status;
};

__host__ __device__ inline size_t blob_bytes(int D) { return (size_t)68 * D; }

// The blob slot of key tile t (see Geom::ring).
__host__ __device__ inline int blob_slot(const Geom& g, int t) {
  return g.ring && t ? t + g.ring_delta : t;
}

// The first key tile any query row sees: 0, or with a sliding window the
// tile of row 0's first key (Nkv - Nq - window + 1).  K/V statistics and
// codes cover the tiles from there on; earlier blobs are never read.
__host__ __device__ inline int first_key_tile(const Geom& g) {
  const int k = g.off - g.window + 1;
  return g.causal && g.window > 0 && k > 0 ? k / 64 : 0;
}

// A quantise call reads the K/V tiles it codes, [qt0, qt1): for their
// non-finite check and value norms, and, up to the key stat_khi, for the
// statistics, which start at tile stat_t0.  With frozen
// statistics (quantising only tiles [qt0, qt1) of a persistent cache) none
// are taken.
__host__ __device__ inline int stat_t0(const Geom& g) { return g.frozen ? g.qt0 : first_key_tile(g); }
__host__ __device__ inline int stat_khi(const Geom& g) { return g.frozen ? g.Nkv : g.stat_hi; }

// Statistics scratch.  V items are (b, kv-head, tile, 128-channel slice); a
// V-coding block codes four consecutive items of one slice and keeps its max
// |V| and flag in the first of them (zeros in the others).  flags: one word
// per K chunk, V item and Q tile (a non-finite input seen), K chunks first,
// then V items, then Q tiles.
struct QuantWs {
  double* ksum;   // [B*Hkv][NCH][D]  per chunk of 16 tiles
  float* kmin;    // [B*Hkv][NCH][D]
  float* kmax;    // [B*Hkv][NCH][D]
  float* vamax;   // [B*Hkv][NT][NVZ] max |V| over the keys of each V item
  float* qamax;   // [B*Hq][NQT]
  unsigned* flags;  // [B*Hkv*NCH + B*Hkv*NT*NVZ + B*Hq*NQT]
  float* vnt;     // [B*Hkv][NT]  largest value norm of each tile read (weighted test)
  double* vnst;   // [B*Hkv][NT]  the sum of its statistics keys' value norms
  int nqt;        // ceil(Nq / 64)
  int nch;        // ceil(NT / 16)
  int nvz;        // 128-channel slices of V per tile: ceil(D / 128)
  int ch0, ch1;   // the chunks holding the tiles read, [qt0, qt1)
};
__host__ __device__ inline size_t vflag0(const Geom& g, const QuantWs& ws) {
  return (size_t)g.B * g.Hkv * ws.nch;
}
__host__ __device__ inline size_t qflag0(const Geom& g, const QuantWs& ws) {
  return vflag0(g, ws) + (size_t)g.B * g.Hkv * g.NT * ws.nvz;
}

struct Pass1Out {
  int32_t* m;
  float* l;
  float* o;
  uint32_t* bits;
  float* lam;
};

hipError_t launch_quantize(const Geom& g, const void* q, const void* k, const void* v,
                           const Fp4Ptrs& f, const QuantWs& ws, hipStream_t s);
// Pass-1 workspace bytes (0: the problem runs one wave per unit); with ws the
// long visit orders are cut into a head and a tail walk (two waves per unit,
// or three heads and one tail wave per three units) plus a re-walk kernel.
size_t pass1_ws_bytes(const Geom& g);
// The schedule a pass-1 launch with a workspace runs (APA_SCHED_*), the first
// tail position of a visit order of npos positions under it (npos: walked
// whole) and the undecided-tile records kept per unit.
int pass1_split_info(const Geom& g, int npos, int* cut, int* cap);
// KV window ring: bytes of the per-unit state kept between segment launches,
// and one segment launch (tiles [t_lo, t_hi]; first: also tile 0 and the
// initial state; last: writes the outputs).
size_t pass1_seg_state_bytes(const Geom& g);
hipError_t launch_pass1_segment(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                                const Pass1Out& o, void* state, int t_lo, int t_hi, int first,
                                int last, hipStream_t s);
hipError_t launch_pass1(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                        const Pass1Out& o, void* ws, hipStream_t s);

struct Pass2Args {
  const void *q, *k, *v;
  const uint32_t* bits;
  const int32_t* cold_m;
  const float *cold_l, *cold_o;
  int fuse;
  void* out;
  float* lse;
  float *hot_m, *hot_l, *hot_o;
  int32_t* list_tiles;   // [units][NT]  (units: see attn_units)
  uint32_t* list_masks;  // [units][NT]
  int32_t* list_count;   // [units]
  // per (b, kv-head): its work groups by descending tile count (ties in
  // ascending order), the order pass 2 takes them in; [units]
  int32_t* list_order;
  // split states when a unit's keys run as S work groups: [S][rows] and
  // [S][rows][D] (rows = B*Hq*Nq)
  float *part_m, *part_l, *part_o;
  // exact path with bf16 inputs: max |V| per (b, kv-head) and chunk of
  // kVmaxChunk keys, [B*Hkv][vmax_nch] (written by a pre-pass)
  float* vmax;
  int vmax_nch;
};
constexpr int kVmaxChunk = 1024;
// Work groups of the 16-bit attention kernels (per batch and kv-head, one per
// four 32-row blocks of its query heads), and the number of key splits each
// runs as for a problem.
int attn_units(const Geom& g);
int attn_splits(const Geom& g);
hipError_t launch_pass2(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a, hipStream_t s);
hipError_t launch_merge(const Geom& g, const Fp4Ptrs& f, const int32_t* cold_m,
                        const float* cold_l, const float* cold_o, const float* hot_m,
                        const float* hot_l, const float* hot_o, void* out, float* lse,
                        hipStream_t s);
// f1: pass 1 and pass 2 (fused merge) in one persistent launch.  The problems
// it takes; the bytes of its control words (zeroed by the launch); the launch
// (split: the pass-1 workspace or nullptr; a: pass 2's arguments with the
// split states; ctl: the control words).
bool fused_covers(const Geom& g);
size_t fused_ctl_bytes(const Geom& g);
hipError_t launch_fused(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                        const Pass1Out& o, void* split, const Pass2Args& a, int32_t* ctl,
                        hipStream_t s);
hipError_t launch_exact(const Geom& g, const void* q, const void* k, const void* v, void* out,
                        float* lse, const Pass2Args& parts, hipStream_t s);

}  // namespace apa
