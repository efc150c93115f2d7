// Kernel argument blocks and host-side launchers shared by the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace apa {

struct Geom {
  int B, Hq, Hkv, G, Nq, Nkv, D, NqP, NkvP, NT, NG, W, causal, off, bf16;
  float sl;  // fl32(scale * fl32(log2 e))
};

struct Fp4Ptrs {
  uint8_t *q_codes, *q_scales, *k_codes, *k_scales, *v_codes, *v_scales;
  float *kbar, *kv_head, *q_head, *q_frame;
  unsigned* status;
};

struct QuantWs {
  double* ksum;   // [B*Hkv][NT][D]
  float* kmin;    // [B*Hkv][NT][D]
  float* kmax;    // [B*Hkv][NT][D]
  float* vamax;   // [B*Hkv][NT]
  float* qamax;   // [B*Hq][NQT]
  int nqt;        // ceil(Nq / 64)
};

struct Pass1Out {
  int32_t* m;
  float* l;
  float* o;
  uint32_t* bits;
  float* lam;
};

hipError_t launch_quantize(const Geom& g, const void* q, const void* k, const void* v,
                           const Fp4Ptrs& f, const QuantWs& ws, hipStream_t s);
hipError_t launch_pass1(const Geom& g, const Fp4Ptrs& f, float eps, float tau, int hoff,
                        const Pass1Out& o, hipStream_t s);

struct Pass2Args {
  const void *q, *k, *v;
  const uint32_t* bits;
  const int32_t* cold_m;
  const float *cold_l, *cold_o;
  int fuse;
  void* out;
  float* lse;
  float *hot_m, *hot_l, *hot_o;
  int32_t* list_tiles;   // [units][NT]
  uint32_t* list_masks;  // [units][NT]
  int32_t* list_count;   // [units]
};
hipError_t launch_pass2(const Geom& g, const Fp4Ptrs& f, const Pass2Args& a, hipStream_t s);
hipError_t launch_merge(const Geom& g, const Fp4Ptrs& f, const int32_t* cold_m,
                        const float* cold_l, const float* cold_o, const float* hot_m,
                        const float* hot_l, const float* hot_o, void* out, float* lse,
                        hipStream_t s);
hipError_t launch_exact(const Geom& g, const void* q, const void* k, const void* v, void* out,
                        float* lse, hipStream_t s);

}  // namespace apa
