// Device-side primitives for gfx950 (CDNA4) shared by the APA kernels.
//
// Lane layouts below were checked on the hardware with in-bounds probes:
//  * V_MFMA_SCALE_F32_32X32X64_F8F6F4 with E2M1 operands: lane l holds row
//    (A) or column (B) l%32 and K elements 32*(l/32) .. +31 as 16 bytes, element
//    2i in the low nibble of byte i; its E8M0 scale (one per 32 K elements) is
//    byte `opsel` of the scale operand; the 32x32 fp32 result has element
//    C[8*(i/4) + 4*(l/32) + i%4][l%32] in register i of lane l.
//  * V_MFMA_F32_32X32X16_F16: lane l holds row/column l%32, K elements
//    8*(l/32) .. +7; same result layout.
//  * V_PERMLANE32_SWAP(x, y): result.first is x in lanes 0-31 and y of lane
//    l-32 in lanes 32-63; result.second is x of lane l+32 in lanes 0-31 and y in
//    lanes 32-63.
//  * V_CVT_SCALEF32_PK_FP4_F32(old, a, b, s, sel): writes byte `sel` of old
//    with E2M1(a / 2^e) in the low and E2M1(b / 2^e) in the high nibble, e the
//    unbiased exponent field of s (field 0 counts as 2^-127); round to nearest
//    even, saturating at 6, IEEE sign kept (-0.1 -> 0x8).
//  * DS_READ_B64_TR_B16: inside each 16-lane group, lane i receives element
//    (i % 4) of the 4-element reads of lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.
//  * V_EXP_F32 (exp2): <= 0.77 ulp on normal results; flushes results below
//    2^-126 to zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace apa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int kTile = 64;      // keys per tile
constexpr int kRowGroup = 16;  // rows per hot verdict
constexpr int kWaveRows = 32;  // rows per wavefront
constexpr float kLog2_6 = 2.58496250072115618f;  // log2(6)
constexpr int kE2M1Ones = 0x22222222;            // eight E2M1 codes of 1.0
constexpr int kE8M0One = 127;                    // E8M0 byte of 2^0

// Block-scaled FP4 x FP4 -> FP32, 32x32x64 (both operands E2M1).
__device__ __forceinline__ v16f mfma_fp4(v4i a, v4i b, v16f c, int scale_a, int scale_b) {
  v8i A = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i B = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, scale_a, 0, scale_b);
}

__device__ __forceinline__ v16f mfma_f16(v8h a, v8h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Value of lane l ^ 32.
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  int lo = (int)(threadIdx.x & 32);
  return __int_as_float(lo ? r[0] : r[1]);
}

// Exchange two per-lane values between the lane halves: lanes 0-31 end up with
// (own x, x of lane l+32), lanes 32-63 with (y of lane l-32, own y).
__device__ __forceinline__ void swap_halves(int x, int y, int& first, int& second) {
  auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  first = r[0];
  second = r[1];
}

// fp32 with exponent field e + 127 (e >= -126) or the subnormal 2^-127: the
// divisor the scaled FP4 conversion applies.
__device__ __forceinline__ float pow2_scale(int e) {
  return e > -127 ? __int_as_float((e + 127) << 23) : __int_as_float(0x00400000);
}

__device__ __forceinline__ unsigned cvt_fp4x2(unsigned old, float a, float b, float s, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, s, 3);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// IEEE maximum (NaN-propagating).  Unlike fmaxf it needs no canonicalising
// of MFMA results and lowers to V_MAXIMUM3_F32, two new operands per
// instruction.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Smallest integer e with a <= 6 * 2^e (a >= 0), clamped to [-127, 127]:
// with a = f * 2^x, f in [0.5, 1), 6 * 2^(x-3) = 0.75 * 2^x covers a iff f <= 0.75.
__device__ __forceinline__ int e8m0_exponent(float a) {
  if (!(a > 0.0f)) return -127;
  int x;
  float f = frexpf(a, &x);
  int e = x - 3 + (f > 0.75f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<_Float16>(_Float16 x) { return (float)x; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t x) {  // bf16 bits
  return __uint_as_float(((unsigned)x) << 16);
}

// XCD-aware block order: dispatch sends block b to XCD b % 8; renumber so each
// XCD receives a contiguous range of logical blocks (which share KV heads and
// therefore L2 lines).  Identity for the tail that does not fill all XCDs.
__device__ __forceinline__ int xcd_remap(int b, int nblocks) {
  const int full = nblocks & ~7;
  if (b >= full) return b;
  const int per = full >> 3;
  return (b & 7) * per + (b >> 3);
}

}  // namespace apa
