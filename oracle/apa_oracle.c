/*
 * apa_oracle.c -- plain, slow, scalar CPU oracle for adaptive-precision
 * attention prefill (APA).  TEST INFRASTRUCTURE ONLY: nothing in the product
 * path may link, load or call this file; only the tests, the smoke check and
 * the CPU-baseline leg of the benchmark do.
 *
 * Source: "APA: sloppy attention, exact where it counts" (rfriedmann.de blog),
 * sections "The merge that makes it exact", "Pass 1: FP4 everywhere, with a hot
 * test" (numbered steps 1-5, tile order, the three FP4 tricks), "Pass 2: exact
 * FP16 on the hot tiles" and "The bug: a sink that drowned the tail"
 * (decoupled cold frame).  Interface semantics (GQA head mapping, causal mask
 * aligned to the KV tail) follow the FFPA documentation page (the note on
 * cross-attention / GQA / causal).  The log-sum-exp merge conventions (empty
 * partial = -inf, ascending merge order) follow "Half the bytes, exactly
 * merged" (coreyjames.ai), section "The merge".
 *
 * Every rounding of the method is simulated: E2M1 round-to-nearest-even codes,
 * power-of-two (E8M0, MX) or UE4M3 (NV) block scales, FP32 accumulation of the
 * running state, the visit order and the 16-row verdict granularity.  Pass 2
 * and the reference attention are computed in FP64 (exact up to FP64
 * rounding).  Build with -O2 -ffp-contract=off: every `float` expression below
 * is one IEEE binary32 operation rounded to nearest even.
 *
 * Exactness of FP4 dot products: codes are half-integers, so each 32-element
 * block sum is an exact small integer multiple of 2^-2; blocks are combined in
 * FP64, which is exact whenever the block exponents of one dot product span
 * fewer than ~38 octaves (always the case for the workloads here) and
 * otherwise adds one FP64 rounding.
 *
 * Pins (tests/): the quantisers exhaustively against a nearest-value search;
 * the scores against an FP64 matrix product of the dequantised operands; pass 1
 * (mask, cold state) bitwise against an independent frame-free brute force;
 * eps=0 against FP64 exact attention; eps>=1 against the frame-free all-FP4
 * result; the merge against softmax over the union of arbitrary key splits;
 * the cold-verdict safety bound; frame invariance over (tau, H); the NV-mode
 * sink bug; the tile order against hand-derived orders; the two-term Q
 * quantisation against a nearest-value search of the residual, and its scores
 * against the brute force; the per-cell margin bitwise against the brute
 * force's own l and lambda; the key mean against an exactly rounded sum in
 * a shuffled order; the reports (true share of each cold tile, hot and cold
 * parts of the reference output) against a numpy softmax and their closed
 * forms; the per-operand emulation against the brute force with the same
 * operands quantised and, with none, against FP64 attention; the sliding
 * window against the brute force and a masked softmax; the value-norm
 * weighted hot test (weights computed by the Python side of the oracle)
 * against the brute force, the closed forms of equal value norms and of one
 * planted tile, and the output-norm bound it gives; NVFP4 mode (blocks of 16
 * with UE4M3 scales, P in 16-key groups) bitwise against the brute force's own
 * NV quantisation on inputs whose P scales stay in UE4M3's normal range, and
 * its 2^-6 scale floor through the sink bug; the Q head-scale ablation
 * (alpha_q: Q at a scale of its own) by its FP64 error matching the tied
 * scale's, which a mis-scaled Q would multiply.  Parity unpinned: the
 * pages' measured numbers (they come from activation dumps that are not
 * available), listed as such in the design notes.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_MX 0
#define ORC_NV 1

typedef struct {
  int32_t B, Hq, Hkv, Nq, Nkv, D;
  int32_t causal;
  float scale;      /* softmax scale; <= 0 means 1/sqrt(D) */
  int32_t fmt;      /* ORC_MX or ORC_NV */
  int32_t int_frame;/* 1: integer log2 frame (ceil of the max), 0: float frame */
  float tau;        /* lazy-max threshold, log2 units */
  float hoff;       /* hot-tile frame offset H */
  float eps;        /* hot threshold */
  int32_t tile;     /* keys per tile (64) */
  int32_t rg;       /* rows per verdict (16) */
  int32_t q_terms;  /* 1: Q quantised once; 2: plus the FP4 residual term */
  int32_t k_lsq;    /* 1: K block exponents by least squared error (MX) */
  int32_t qmask;    /* which of pass 1's FP4 roundings apply: ORC_QUANT_Q | _K | _V | _P
                       (all: the method; fewer: the per-operand emulation) */
  int32_t window;   /* > 0: causal sliding window of this many keys; 0: full causal */
  int32_t vweight;  /* 1: the hot test weighs each tile's mass by its value-norm weight
                       (orc_job.vw); 0: mass only */
} orc_params;

/* Per-operand switches of pass 1's FP4 roundings ("Second hunt: which operand
 * is to blame": the page finds the guilty operand by emulating pass 1 with one
 * quantisation at a time).  An operand whose bit is clear enters pass 1 at its
 * exact value, in the same normalised units (Q: q * inv_q, K: (k - kbar) *
 * inv_k, V: v * inv_v, each product exact in FP64, no clamp), and P at its
 * exact value 2^(s - m) (FP64 exp2).  Everything else -- the FP32 scores,
 * frames, sums and state updates -- is the method's arithmetic unchanged, so
 * with every bit set this is the oracle itself. */
#define ORC_QUANT_Q 1
#define ORC_QUANT_K 2
#define ORC_QUANT_V 4
#define ORC_QUANT_P 8
#define ORC_QUANT_ALL 15

/* ------------------------------------------------------------------------ */
/* Formats                                                                   */
/* ------------------------------------------------------------------------ */

/* E2M1 magnitudes, indexed by the 3-bit magnitude code. */
static const double E2M1_VAL[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Round |x| to the nearest E2M1 magnitude, ties to the even code, saturating
 * at 6.  The midpoints between neighbours are 0.25, 0.75, 1.25, 1.75, 2.5,
 * 3.5, 5; at a midpoint the even code wins: 0.25->0, 0.75->1.0 (code 2),
 * 1.25->1.0 (code 2), 1.75->2.0 (code 4), 2.5->2.0 (code 4), 3.5->4.0
 * (code 6), 5->4.0 (code 6). */
int orc_e2m1_mag(double a) {
  int c = 0;
  c += a > 0.25;
  c += a >= 0.75;
  c += a > 1.25;
  c += a >= 1.75;
  c += a > 2.5;
  c += a >= 3.5;
  c += a > 5.0;
  return c;
}

/* Full 4-bit code: the sign bit is the IEEE sign of x (so -0.1 -> 0x8). */
int orc_e2m1_code(double x) {
  int s = signbit(x) ? 8 : 0;
  return s | orc_e2m1_mag(fabs(x));
}

double orc_e2m1_value(int code) {
  double v = E2M1_VAL[code & 7];
  return (code & 8) ? -v : v;
}

/* UE4M3 (unsigned E4M3, bias 7, no inf, max 448, subnormal step 2^-9):
 * round a >= 0 to the nearest representable value, ties to even mantissa,
 * saturating at 448.  Brute force over the 127 finite values. */
static double ue4m3_table[127];
static int ue4m3_ready = 0;
static void ue4m3_init(void) {
  if (ue4m3_ready) return;
  for (int e = 0; e < 16; ++e)
    for (int m = 0; m < 8; ++m) {
      int idx = e * 8 + m;
      if (idx >= 127) break; /* e=15,m=7 is NaN */
      double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
      ue4m3_table[idx] = v;
    }
  ue4m3_ready = 1;
}
double orc_ue4m3_rn(double a) {
  ue4m3_init();
  if (!(a > 0)) return 0.0;
  if (a >= 448.0) return 448.0;
  int best = 0;
  for (int i = 1; i < 127; ++i) {
    double di = fabs(ue4m3_table[i] - a), db = fabs(ue4m3_table[best] - a);
    if (di < db || (di == db && (i & 1) == 0)) best = i;
  }
  return ue4m3_table[best];
}

/* Smallest integer e with a <= 6*2^e (a > 0), clamped to [-127, 127];
 * a == 0 gives -127.  The comparison 6*2^e >= a is exact in FP64. */
int orc_e8m0_exp(double a) {
  if (!(a > 0)) return -127;
  int x;
  frexp(a, &x); /* a in [2^(x-1), 2^x) */
  int e = x - 4;
  while (6.0 * ldexp(1.0, e) < a) ++e;
  while (6.0 * ldexp(1.0, e - 1) >= a) --e;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

/* Smallest integer E with 2^ymax <= 6*2^E, i.e. E = ceil(ymax - log2 6),
 * clamped below at -127.  ymax = -inf (an all-invisible group) gives -127. */
static int p_group_exp(double ymax) {
  if (ymax == -INFINITY) return -127;
  int E = (int)ceil(ymax - log2(6.0));
  while (exp2(ymax - E) > 6.0) ++E;
  while (exp2(ymax - (E - 1)) <= 6.0) --E;
  if (E < -127) E = -127;
  return E;
}

/* ------------------------------------------------------------------------ */
/* a1: statistics                                                            */
/* ------------------------------------------------------------------------ */

/* Per-channel key mean of one (b, kv-head): the FP64 sum runs in a fixed
 * three-level order -- keys ascending inside each 64-key tile, tile sums
 * ascending inside each chunk of 16 tiles, chunk sums ascending (the page
 * fixes the order of its reductions, 'What else is in the box'); for fp16 keys
 * of ordinary magnitude every partial sum is exact, so the order only matters
 * for extreme inputs.  k̄ = fl32(sum / Nkv) with the division in FP64.  Also the per-channel
 * min and max, and amax_K = max over channels of
 * max(fl32(max_k K - k̄), fl32(k̄ - min_k K)) -- the largest |K - k̄| over the
 * head, exact because rounding is monotone. (Pass 1, "Mean-centred K".) */
void orc_key_stats(const float* K, int Nkv, int D, int tile, float* kbar, float* amax_out) {
  float amax = 0.0f;
  for (int d = 0; d < D; ++d) {
    double total = 0.0;
    float mn = INFINITY, mx = -INFINITY;
    for (int c0 = 0; c0 < Nkv; c0 += 16 * tile) {
      double chunk = 0.0;
      for (int t0 = c0; t0 < Nkv && t0 < c0 + 16 * tile; t0 += tile) {
        double part = 0.0;
        for (int k = t0; k < Nkv && k < t0 + tile; ++k) {
          float x = K[(size_t)k * D + d];
          part += (double)x;
          if (x < mn) mn = x;
          if (x > mx) mx = x;
        }
        chunk += part;
      }
      total += chunk;
    }
    float kb = Nkv > 0 ? (float)(total / (double)Nkv) : 0.0f;
    kbar[d] = kb;
    if (Nkv > 0) {
      float up = mx - kb, dn = kb - mn;
      if (up > amax) amax = up;
      if (dn > amax) amax = dn;
    }
  }
  *amax_out = amax;
}

float orc_absmax(const float* X, size_t n) {
  float a = 0.0f;
  for (size_t i = 0; i < n; ++i) {
    float v = fabsf(X[i]);
    if (v > a) a = v;
  }
  return a;
}

/* ------------------------------------------------------------------------ */
/* a2: per-head scales and quantisation                                      */
/* ------------------------------------------------------------------------ */

static double fmt_xmax(int fmt) { return fmt == ORC_NV ? 2688.0 : 6.0; }

/* One FP32 scale per head that maps the head's largest magnitude to the
 * format's largest value (MX: 6; NV: 6 x 448 = 2688).  g = fl32(amax/X),
 * inv = fl32(X/amax); amax == 0 gives g = inv = 1.  Computing the quotient in
 * FP64 and rounding once is the correctly rounded binary32 quotient. */
void orc_head_scale(float amax, int fmt, float* g, float* inv) {
  double X = fmt_xmax(fmt);
  if (!(amax > 0.0f)) { *g = 1.0f; *inv = 1.0f; return; }
  *g = (float)((double)amax / X);
  *inv = (float)(X / (double)amax);
}

/* Q's per-head scale is tied to K's so that the factor turning an FP4 dot
 * product into a log2-domain score is an exact power of two, alpha = 2^j:
 * w = fl32(sl * g_k), j = the smallest integer with amax_Q * w <= X * 2^j, and
 * Q is normalised by inv_q = w * 2^-j.  The head's largest |q| then lands in
 * (X/2, X] instead of exactly on X; with per-block power-of-two scales this
 * only moves where each block maximum falls inside its octave. */
void orc_q_scale(float amax_q, float sl, float g_k, int fmt, float* inv_q, int* j_out) {
  double X = fmt_xmax(fmt);
  float w = sl * g_k;
  int j = 0;
  if (amax_q > 0.0f && w > 0.0f) {
    double prod = (double)amax_q * (double)w; /* exact: 24x24 bits */
    int x;
    frexp(prod / X, &x);
    j = x - 2;
    while (X * ldexp(1.0, j) < prod) ++j;
    while (X * ldexp(1.0, j - 1) >= prod) --j;
  }
  *j_out = j;
  *inv_q = (float)ldexp((double)w, -j);
}

/* Normalise one value: x' = clamp(fl32(xc * inv), -X, X). */
static float normalise(float xc, float inv, int fmt) {
  float X = (float)fmt_xmax(fmt);
  float v = xc * inv;
  if (v > X) v = X;
  if (v < -X) v = -X;
  return v;
}

/* Quantise one block of n normalised values (MX: n=32, E8M0 exponent byte
 * e+127 with e the smallest integer such that the block max fits 6*2^e; NV:
 * n=16, UE4M3 scale s = RN(amax/6) stored as its byte encoding).  codes[i] is
 * the 4-bit code of element i. */
static void quant_block(const float* xs, int n, int fmt, uint8_t* codes, uint8_t* scale_byte) {
  double a = 0.0;
  for (int i = 0; i < n; ++i) if (fabs((double)xs[i]) > a) a = fabs((double)xs[i]);
  if (fmt == ORC_MX) {
    int e = orc_e8m0_exp(a);
    for (int i = 0; i < n; ++i) codes[i] = (uint8_t)orc_e2m1_code(ldexp((double)xs[i], -e));
    *scale_byte = (uint8_t)(e + 127);
  } else {
    double s = orc_ue4m3_rn(a / 6.0);
    ue4m3_init();
    int idx = 0;
    for (int i = 0; i < 127; ++i) if (ue4m3_table[i] == s) { idx = i; break; }
    for (int i = 0; i < n; ++i) {
      double q = s > 0 ? (double)xs[i] / s : 0.0 * xs[i];
      if (s == 0) q = copysign(0.0, (double)xs[i]);
      codes[i] = (uint8_t)orc_e2m1_code(q);
    }
    *scale_byte = (uint8_t)idx;
  }
}

/* Value of a scale byte: MX 2^(byte-127); NV the UE4M3 value. */
double orc_scale_value(uint8_t b, int fmt) {
  if (fmt == ORC_MX) return ldexp(1.0, (int)b - 127);
  ue4m3_init();
  return b < 127 ? ue4m3_table[b] : NAN;
}

/* Quantise rows along the channel axis (Q and K).  X: [n][D] floats; centre:
 * per-channel value subtracted first (K's mean, in FP32) or NULL.  codes:
 * [n][D/2] bytes, element 2i in the low nibble of byte i; scales: [n][D/Bs]. */
void orc_quant_rows(const float* X, int n, int D, const float* centre, float inv, int fmt,
                    uint8_t* codes, uint8_t* scales) {
  int Bs = fmt == ORC_NV ? 16 : 32;
  float buf[32];
  uint8_t cb[32];
  for (int r = 0; r < n; ++r) {
    for (int b0 = 0; b0 < D; b0 += Bs) {
      for (int i = 0; i < Bs; ++i) {
        float x = X[(size_t)r * D + b0 + i];
        float xc = centre ? x - centre[b0 + i] : x;
        buf[i] = normalise(xc, inv, fmt);
      }
      quant_block(buf, Bs, fmt, cb, &scales[(size_t)r * (D / Bs) + b0 / Bs]);
      for (int i = 0; i < Bs; i += 2)
        codes[(size_t)r * (D / 2) + (b0 + i) / 2] = (uint8_t)(cb[i] | (cb[i + 1] << 4));
    }
  }
}

/* Least-squares block exponent (section "Second hunt: which operand is to
 * blame": for K, a block's scale is the candidate with the smallest squared
 * quantisation error rather than the nearest-rule one).  MX only.
 * Candidates: the no-clipping exponent e of orc_e8m0_exp, then e-1 (finer
 * steps, the largest values clipped at 6) and e+1, each clamped to [-127,
 * 127]; a later candidate wins only with a strictly smaller error, so ties
 * keep e.  The error is a float decision taken in FP32 in a fixed order: per
 * run of 8 consecutive elements d = fl32(x - q), acc = fl32(acc + fl32(d*d))
 * in element order, then the four run sums as (r0 + r1) + (r2 + r3). */
static int lsq_block_exp(const float* xs) {
  double a = 0.0;
  for (int i = 0; i < 32; ++i) if (fabs((double)xs[i]) > a) a = fabs((double)xs[i]);
  int e0 = orc_e8m0_exp(a);
  int cand[3] = {e0, e0 - 1, e0 + 1};
  int best = e0;
  float best_err = 0.0f;
  for (int c = 0; c < 3; ++c) {
    int e = cand[c] < -127 ? -127 : (cand[c] > 127 ? 127 : cand[c]);
    float run[4];
    for (int r = 0; r < 4; ++r) {
      float acc = 0.0f;
      for (int i = 8 * r; i < 8 * r + 8; ++i) {
        float q = (float)(ldexp(1.0, e) * orc_e2m1_value(orc_e2m1_code(ldexp((double)xs[i], -e))));
        float d = xs[i] - q;
        float sq = d * d;
        acc = acc + sq;
      }
      run[r] = acc;
    }
    float err = (run[0] + run[1]) + (run[2] + run[3]);
    if (c == 0 || err < best_err) {
      best_err = err;
      best = e;
    }
  }
  return best;
}

/* orc_quant_rows with least-squares block exponents (MX, 32-element blocks). */
void orc_quant_rows_lsq(const float* X, int n, int D, const float* centre, float inv,
                        uint8_t* codes, uint8_t* scales) {
  float buf[32];
  for (int r = 0; r < n; ++r) {
    for (int b0 = 0; b0 < D; b0 += 32) {
      for (int i = 0; i < 32; ++i) {
        float x = X[(size_t)r * D + b0 + i];
        float xc = centre ? x - centre[b0 + i] : x;
        buf[i] = normalise(xc, inv, ORC_MX);
      }
      int e = lsq_block_exp(buf);
      scales[(size_t)r * (D / 32) + b0 / 32] = (uint8_t)(e + 127);
      for (int i = 0; i < 32; i += 2) {
        int c0 = orc_e2m1_code(ldexp((double)buf[i], -e));
        int c1 = orc_e2m1_code(ldexp((double)buf[i + 1], -e));
        codes[(size_t)r * (D / 2) + (b0 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
      }
    }
  }
}

/* Two-term quantisation of rows along channels (section "Second hunt: which
 * operand is to blame": a second FP4 term holds what the first one leaves
 * over, sharing its per-head scale).  Per block: the first term's codes and
 * scale as orc_quant_rows; the residual of each normalised value, fl32(x' -
 * dequantised first term), is then quantised as a block of its own (own
 * exponent or UE4M3 scale).  codes2/scales2 have the layout of
 * codes/scales. */
void orc_quant_rows2(const float* X, int n, int D, float inv, int fmt, uint8_t* codes,
                     uint8_t* scales, uint8_t* codes2, uint8_t* scales2) {
  int Bs = fmt == ORC_NV ? 16 : 32;
  float buf[32], res[32];
  uint8_t cb[32], cb2[32];
  for (int r = 0; r < n; ++r) {
    for (int b0 = 0; b0 < D; b0 += Bs) {
      size_t sidx = (size_t)r * (D / Bs) + b0 / Bs;
      for (int i = 0; i < Bs; ++i) buf[i] = normalise(X[(size_t)r * D + b0 + i], inv, fmt);
      quant_block(buf, Bs, fmt, cb, &scales[sidx]);
      double sv = orc_scale_value(scales[sidx], fmt);
      for (int i = 0; i < Bs; ++i) {
        float deq = (float)(sv * orc_e2m1_value(cb[i])); /* exact: a few bits */
        res[i] = buf[i] - deq;
      }
      quant_block(res, Bs, fmt, cb2, &scales2[sidx]);
      for (int i = 0; i < Bs; i += 2) {
        codes[(size_t)r * (D / 2) + (b0 + i) / 2] = (uint8_t)(cb[i] | (cb[i + 1] << 4));
        codes2[(size_t)r * (D / 2) + (b0 + i) / 2] = (uint8_t)(cb2[i] | (cb2[i + 1] << 4));
      }
    }
  }
}

/* Quantise V along the key axis (the transposed layout the P.V product
 * contracts over).  V: [Nkv][D].  Keys are padded with zeros up to NkvP, a
 * multiple of the tile.  codes: [D][NkvP/2]; scales: [D][NkvP/Bs].  raw: the
 * values enter at their own scale, neither normalised nor clamped (MX: the
 * E8M0 block exponents span the whole range of the inputs, so V's per-head
 * scale is 1; with a scale that is not a power of two it would only move the
 * mantissas of the normalised values); otherwise normalised by inv. */
void orc_quant_vt(const float* V, int Nkv, int NkvP, int D, float inv, int fmt, int raw,
                  uint8_t* codes, uint8_t* scales) {
  int Bs = fmt == ORC_NV ? 16 : 32;
  float buf[32];
  uint8_t cb[32];
  for (int d = 0; d < D; ++d) {
    for (int k0 = 0; k0 < NkvP; k0 += Bs) {
      for (int i = 0; i < Bs; ++i) {
        int k = k0 + i;
        float v = k < Nkv ? V[(size_t)k * D + d] : 0.0f;
        buf[i] = raw ? v : normalise(v, inv, fmt);
      }
      quant_block(buf, Bs, fmt, cb, &scales[(size_t)d * (NkvP / Bs) + k0 / Bs]);
      for (int i = 0; i < Bs; i += 2)
        codes[(size_t)d * (NkvP / 2) + (k0 + i) / 2] = (uint8_t)(cb[i] | (cb[i + 1] << 4));
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Problem geometry                                                          */
/* ------------------------------------------------------------------------ */

static float softmax_sl(const orc_params* p) {
  const float LOG2E32 = 1.44269502162933349609375f; /* fl32(log2 e) */
  float scale = p->scale > 0.0f ? p->scale : (float)(1.0 / sqrt((double)p->D));
  return scale * LOG2E32;
}
float orc_sl(const orc_params* p) { return softmax_sl(p); }

static int n_tiles(const orc_params* p) { return (p->Nkv + p->tile - 1) / p->tile; }

/* Key k is visible from query row r: tail-aligned causal mask (row r sees
 * k <= r + Nkv - Nq), and with a sliding window of W keys only the W most
 * recent of those, k > r + Nkv - Nq - W ("What else is in the box": sliding
 * window). */
static int visible(const orc_params* p, int r, int k) {
  if (k >= p->Nkv) return 0;
  if (!p->causal) return 1;
  int last = r + (p->Nkv - p->Nq);
  if (k > last) return 0;
  return p->window <= 0 || k > last - p->window;
}

/* Visit order of one row group: tile 0 (the sink) first, then from the causal
 * diagonal backwards, "0, d, d-1, ..., 1", where d is the tile holding the
 * last key visible to the group's last row ("Tile order").  With a sliding
 * window whose keys start past tile 0 for the group's first row (first
 * visible tile lo > 0), the sink is not visible and the order is the
 * diagonal backwards alone, "d, d-1, ..., lo".  Returns the count. */
int orc_visit_order(const orc_params* p, int g, int* order) {
  int NT = n_tiles(p);
  int first = g * p->rg;
  int last = (g + 1) * p->rg - 1;
  if (last > p->Nq - 1) last = p->Nq - 1;
  int d, lo = 0;
  if (p->causal) {
    int kmax = last + (p->Nkv - p->Nq);
    if (kmax > p->Nkv - 1) kmax = p->Nkv - 1;
    d = kmax / p->tile;
    if (p->window > 0) {
      int kmin = first + (p->Nkv - p->Nq) - p->window + 1;
      lo = kmin > 0 ? kmin / p->tile : 0;
    }
  } else {
    d = NT - 1;
  }
  int n = 0;
  if (lo == 0) {
    order[n++] = 0;
    for (int t = d; t >= 1; --t) order[n++] = t;
  } else {
    for (int t = d; t >= lo; --t) order[n++] = t;
  }
  return n;
}

/* ------------------------------------------------------------------------ */
/* a4..a7: pass 1 for one row group                                          */
/* ------------------------------------------------------------------------ */

typedef struct {
  const orc_params* p;
  /* quantised operands for this (b, q-head) and its kv-head */
  const uint8_t *qc, *qs;   /* [Nq][D/2], [Nq][D/Bs] */
  const uint8_t *qc2, *qs2; /* the residual term of Q, or NULL */
  const uint8_t *kc, *ks;   /* [Nkv][D/2], [Nkv][D/Bs] */
  const uint8_t *vc, *vs;   /* [D][NkvP/2], [D][NkvP/Bs] */
  int NkvP;
  double alpha;             /* 2^j */
  float g_v;
  /* the unquantised operands (per-operand emulation, see ORC_QUANT_*) */
  const float *Qh, *Kh, *Vh, *kbar; /* [Nq][D], [Nkv][D], [Nkv][D], [D] */
  float inv_q, inv_k, inv_v;
  const float* tw;          /* [NT] value-norm weights of the hot test, or NULL */
} orc_head_ops;

static double code_at(const uint8_t* codes, size_t idx) {
  uint8_t b = codes[idx >> 1];
  int c = (idx & 1) ? (b >> 4) : (b & 15);
  return orc_e2m1_value(c);
}

/* Q and K in normalised units at (row or key, channel d): the dequantised
 * FP4 value, or, with its quantisation switched off, the exact value. */
static double q_value(const orc_head_ops* h, int r, int d) {
  const orc_params* p = h->p;
  int D = p->D, Bs = p->fmt == ORC_NV ? 16 : 32, nb = D / Bs;
  if (!(p->qmask & ORC_QUANT_Q)) return (double)h->Qh[(size_t)r * D + d] * (double)h->inv_q;
  double v = orc_scale_value(h->qs[(size_t)r * nb + d / Bs], p->fmt) *
             code_at(h->qc, (size_t)r * D + d);
  if (h->qc2)
    v += orc_scale_value(h->qs2[(size_t)r * nb + d / Bs], p->fmt) *
         code_at(h->qc2, (size_t)r * D + d);
  return v;
}
static double k_value(const orc_head_ops* h, int k, int d) {
  const orc_params* p = h->p;
  int D = p->D, Bs = p->fmt == ORC_NV ? 16 : 32, nb = D / Bs;
  if (!(p->qmask & ORC_QUANT_K))
    return ((double)h->Kh[(size_t)k * D + d] - (double)h->kbar[d]) * (double)h->inv_k;
  return orc_scale_value(h->ks[(size_t)k * nb + d / Bs], p->fmt) *
         code_at(h->kc, (size_t)k * D + d);
}

/* FP4 score from decoded operands ("Scores in FP4"): s = fl32(alpha *
 * fl32(dot)), dot = the FP64 sum over channels of q'_d k'_d, where q' and k'
 * are the dequantised values (code times block scale; with two Q terms the
 * sum of both terms) or, with an operand's quantisation switched off, its
 * exact value.  With FP4 operands every product is exact and so is the sum
 * (within a block a small multiple of one power of two; blocks combine
 * exactly unless their exponents span more than ~38 octaves), so s is the
 * exact block-scaled dot product rounded once to FP32, then scaled. */
static float fp4_score(const double* q, const double* k, int D, double alpha) {
  double dot = 0.0;
  for (int d = 0; d < D; ++d) dot += q[d] * k[d];
  float d32 = (float)dot;
  return (float)(alpha * (double)d32);
}

/* Dequantised V' (without the per-head g_v) at (key k, channel d); with V's
 * quantisation switched off, the exact v * inv_v (padding keys: 0). */
static double vprime(const orc_head_ops* h, int k, int d) {
  int Bs = h->p->fmt == ORC_NV ? 16 : 32;
  if (!(h->p->qmask & ORC_QUANT_V))
    return k < h->p->Nkv ? (double)h->Vh[(size_t)k * h->p->D + d] * (double)h->inv_v : 0.0;
  double sc = orc_scale_value(h->vs[(size_t)d * (h->NkvP / Bs) + k / Bs], h->p->fmt);
  return sc * code_at(h->vc, (size_t)d * h->NkvP + k);
}

/* 2^x for integer-or-infinite exponent differences (the frames). */
static double pow2d(double x) {
  if (x == -INFINITY) return 0.0;
  return exp2(x);
}
/* fl32(v * 2^x): exact power-of-two rescale of a float (subnormal results
 * round like an FP32 ldexp). */
static float rescale(float v, double x) {
  if (v == 0.0f) return v;
  return (float)((double)v * pow2d(x));
}

typedef struct {
  /* outputs for the group's rows (rows beyond Nq untouched) */
  uint8_t* hot;      /* [NT] 0/1 */
  double* margin;    /* [NT] max_r (l_r - eps*lambda_c)/lambda_c, NaN if not visited */
  double* m;         /* [rg] frame (integer or float; -inf if unset) */
  float* l;          /* [rg] */
  float* lam;        /* [rg] */
  float* o;          /* [rg][D]  o1 = fl32(o * g_v) */
  double* shift_max; /* [rg] largest log2 factor by which lambda was lifted on a hot tile */
} orc_p1_out;

/* Pass 1 of one row group g of one (b, q-head): numbered steps 1-5 of "Pass 1",
 * with the lazy maximum, the visit order and the decoupled cold frame. */
void orc_pass1_group(const orc_head_ops* h, int g, orc_p1_out* out) {
  const orc_params* p = h->p;
  int D = p->D, T = p->tile, R = p->rg, NT = n_tiles(p);
  int Bp = p->fmt == ORC_NV ? 16 : 32; /* keys per P group */
  int r0 = g * R;
  int nr = p->Nq - r0 < R ? p->Nq - r0 : R;
  double m[16];
  float lam[16], l[16];
  float* o = (float*)calloc((size_t)R * D, sizeof(float));
  float* s = (float*)malloc((size_t)R * T * sizeof(float));
  double* ph = (double*)malloc((size_t)R * T * sizeof(double));
  float* tpv = (float*)malloc((size_t)D * sizeof(float));
  int* order = (int*)malloc((size_t)(NT + 1) * sizeof(int));
  /* the operands decoded once: the group's Q rows, and per visited tile its
   * K rows and (for a cold tile) its V rows, zero past Nkv */
  double* qd = (double*)malloc((size_t)R * D * sizeof(double));
  double* kd = (double*)malloc((size_t)T * D * sizeof(double));
  double* vd = (double*)malloc((size_t)T * D * sizeof(double));
  for (int i = 0; i < nr; ++i)
    for (int d = 0; d < D; ++d) qd[(size_t)i * D + d] = q_value(h, r0 + i, d);
  for (int i = 0; i < R; ++i) { m[i] = -INFINITY; lam[i] = 0.0f; l[i] = 0.0f; out->shift_max[i] = 0.0; }
  for (int t = 0; t < NT; ++t) { out->hot[t] = 0; out->margin[t] = NAN; }

  int nvis = orc_visit_order(p, g, order);
  for (int it = 0; it < nvis; ++it) {
    int t = order[it], k0 = t * T;
    /* a tile no row of the group can see is not visited */
    int any = 0;
    for (int i = 0; i < nr && !any; ++i)
      for (int kk = 0; kk < T && !any; ++kk) any = visible(p, r0 + i, k0 + kk);
    if (!any) continue;
    for (int kk = 0; kk < T; ++kk)
      for (int d = 0; d < D; ++d)
        kd[(size_t)kk * D + d] = k0 + kk < p->Nkv ? k_value(h, k0 + kk, d) : 0.0;

    double mc[16];
    float lc[16], lamc[16];
    int fire[16];
    int hot = (p->eps == 0.0f);
    double margin = -INFINITY;
    for (int i = 0; i < nr; ++i) {
      int r = r0 + i;
      /* step 1: scores, causal mask */
      double c = -INFINITY;
      for (int kk = 0; kk < T; ++kk) {
        int k = k0 + kk;
        s[i * T + kk] = visible(p, r, k)
                            ? fp4_score(qd + (size_t)i * D, kd + (size_t)kk * D, D, h->alpha)
                            : -INFINITY;
        if ((double)s[i * T + kk] > c) c = s[i * T + kk];
      }
      /* lazy maximum: move the frame only when the tile max exceeds it by
       * more than tau; the integer frame moves to ceil(c) */
      fire[i] = c > m[i] + (double)p->tau;
      mc[i] = fire[i] ? (p->int_frame ? ceil(c) : c) : m[i];
      /* step 2: P quantised per key group with its own scale */
      double lsum = 0.0;
      for (int q0 = 0; q0 < T; q0 += Bp) {
        double ymax = -INFINITY;
        for (int kk = q0; kk < q0 + Bp; ++kk) {
          double y = (double)s[i * T + kk] - mc[i];
          if (y > ymax) ymax = y;
        }
        if (!(p->qmask & ORC_QUANT_P)) {
          /* emulation: P at its exact value */
          for (int kk = q0; kk < q0 + Bp; ++kk) {
            double y = (double)s[i * T + kk] - mc[i];
            ph[i * T + kk] = (y == -INFINITY || mc[i] == -INFINITY) ? 0.0 : exp2(y);
          }
        } else if (p->fmt == ORC_MX) {
          int E = p_group_exp(ymax);
          for (int kk = q0; kk < q0 + Bp; ++kk) {
            double y = (double)s[i * T + kk] - mc[i];
            double code = (y == -INFINITY || mc[i] == -INFINITY) ? 0.0 : E2M1_VAL[orc_e2m1_mag(exp2(y - E))];
            ph[i * T + kk] = ldexp(code, E);
          }
        } else {
          /* NV: UE4M3 group scale, clamped at 2^-6 to stay a normal value */
          double sg = ymax == -INFINITY ? 0.0 : orc_ue4m3_rn(exp2(ymax) / 6.0);
          if (sg < ldexp(1.0, -6)) sg = ldexp(1.0, -6);
          for (int kk = q0; kk < q0 + Bp; ++kk) {
            double y = (double)s[i * T + kk] - mc[i];
            double code = (y == -INFINITY || mc[i] == -INFINITY) ? 0.0 : E2M1_VAL[orc_e2m1_mag(exp2(y) / sg)];
            ph[i * T + kk] = code * sg;
          }
        }
        for (int kk = q0; kk < q0 + Bp; ++kk) lsum += ph[i * T + kk];
      }
      /* step 3: tile row sum from the same quantised P */
      lc[i] = (float)lsum;
      /* running sum over every tile seen so far, this one included */
      float lam_prev = m[i] == -INFINITY ? 0.0f : rescale(lam[i], m[i] - mc[i]);
      lamc[i] = lam_prev + lc[i];
      /* step 4: the hot test; with value-norm weights the tile's mass
       * counts w_t times (w_t >= 1, one FP32 product) */
      float thr = p->eps * lamc[i];
      float lw = h->tw ? lc[i] * h->tw[t] : lc[i];
      if (lw > thr) hot = 1;
      if (lamc[i] > 0.0f) {
        double mg = ((double)lw - (double)p->eps * (double)lamc[i]) / (double)lamc[i];
        if (mg > margin) margin = mg;
      }
    }
    out->hot[t] = (uint8_t)hot;
    out->margin[t] = margin;

    /* step 5 (cold) or the decoupled frame update (hot) */
    for (int i = 0; i < nr; ++i) {
      double mn;
      if (!hot) {
        mn = mc[i];
        double sh = m[i] - mn;
        if (i == 0)
          for (int kk = 0; kk < T; ++kk)
            for (int d = 0; d < D; ++d) vd[(size_t)kk * D + d] = vprime(h, k0 + kk, d);
        for (int d = 0; d < D; ++d) {
          double acc = 0.0;
          for (int kk = 0; kk < T; ++kk)
            if (ph[i * T + kk] != 0.0) acc += ph[i * T + kk] * vd[(size_t)kk * D + d];
          tpv[d] = (float)acc;
        }
        for (int d = 0; d < D; ++d) {
          float prev = m[i] == -INFINITY ? 0.0f : rescale(o[i * D + d], sh);
          o[i * D + d] = prev + tpv[d];
        }
        float lp = m[i] == -INFINITY ? 0.0f : rescale(l[i], sh);
        l[i] = lp + lc[i];
      } else {
        if (fire[i]) {
          double lift = mc[i] - (double)p->hoff;
          mn = m[i] > lift ? m[i] : lift;
        } else {
          mn = m[i];
        }
        double sh = m[i] - mn;
        for (int d = 0; d < D; ++d) o[i * D + d] = m[i] == -INFINITY ? 0.0f : rescale(o[i * D + d], sh);
        l[i] = m[i] == -INFINITY ? 0.0f : rescale(l[i], sh);
      }
      /* lambda moves from frame mc to the new frame */
      if (mc[i] != -INFINITY && mn != -INFINITY) {
        double up = mc[i] - mn;
        if (up > out->shift_max[i]) out->shift_max[i] = up;
        lam[i] = rescale(lamc[i], up);
      } else {
        lam[i] = lamc[i];
      }
      m[i] = mn;
    }
  }
  for (int i = 0; i < nr; ++i) {
    out->m[i] = m[i];
    out->l[i] = l[i];
    out->lam[i] = lam[i];
    for (int d = 0; d < D; ++d) out->o[(size_t)i * D + d] = o[i * D + d] * h->g_v;
  }
  free(o); free(s); free(ph); free(tpv); free(order); free(qd); free(kd); free(vd);
}

/* ------------------------------------------------------------------------ */
/* a9: exact pass 2 (FP64) over the hot tiles of one row group               */
/* ------------------------------------------------------------------------ */

/* For each row of group g: the keys are the visible keys in the group's hot
 * tiles; scores s2 = sl*q.k - c_r in log2 units with c_r = sl*q.kbar, the same
 * constant the centred keys subtract in pass 1 ("Mean-centred K"); FP64
 * online-softmax state m2 = max s2, l2 = sum 2^(s2-m2), o2 = sum 2^(s2-m2) v.
 * Rows with no hot key get m2 = -inf, l2 = 0, o2 = 0. */
void orc_pass2_group(const orc_params* p, const float* Qh, const float* Kh, const float* Vh,
                     const float* kbar, const uint8_t* hot, int g, double* m2, double* l2,
                     double* o2, double* cr) {
  int D = p->D, T = p->tile, R = p->rg, NT = n_tiles(p);
  double sl = (double)softmax_sl(p);
  int r0 = g * R;
  int nr = p->Nq - r0 < R ? p->Nq - r0 : R;
  double* sc = (double*)malloc((size_t)NT * T * sizeof(double));
  for (int i = 0; i < nr; ++i) {
    int r = r0 + i;
    const float* q = Qh + (size_t)r * D;
    double c = 0.0;
    for (int d = 0; d < D; ++d) c += (double)q[d] * (double)kbar[d];
    c *= sl;
    cr[i] = c;
    double mx = -INFINITY;
    for (int t = 0; t < NT; ++t) {
      for (int kk = 0; kk < T; ++kk) {
        int k = t * T + kk;
        double v = -INFINITY;
        if (hot[t] && visible(p, r, k)) {
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += (double)q[d] * (double)Kh[(size_t)k * D + d];
          v = sl * dot - c;
        }
        sc[(size_t)t * T + kk] = v;
        if (v > mx) mx = v;
      }
    }
    double ls = 0.0;
    for (int d = 0; d < D; ++d) o2[(size_t)i * D + d] = 0.0;
    if (mx != -INFINITY) {
      for (int k = 0; k < NT * T; ++k) {
        if (sc[k] == -INFINITY) continue;
        double w = exp2(sc[k] - mx);
        ls += w;
        for (int d = 0; d < D; ++d) o2[(size_t)i * D + d] += w * (double)Vh[(size_t)k * D + d];
      }
    }
    m2[i] = mx;
    l2[i] = ls;
  }
  free(sc);
}

/* ------------------------------------------------------------------------ */
/* a10: exact merge of two online-softmax states (FP64)                      */
/* ------------------------------------------------------------------------ */

/* "The merge that makes it exact": M = max(m1, m2) over non-empty states,
 * w_i = 2^(m_i - M), O = (w1 o1 + w2 o2) / (w1 l1 + w2 l2); in log2 units.
 * An empty state (l = 0) has weight 0; both empty gives O = 0 and
 * LSE = -inf.  LSE (natural log of sum_k exp(scale q.k)) = ln2 (c + M + log2 L). */
void orc_merge_row(int D, double m1, double l1, const double* o1, double m2, double l2,
                   const double* o2, double c, double* O, double* lse) {
  int e1 = l1 > 0.0, e2 = l2 > 0.0;
  if (!e1 && !e2) {
    for (int d = 0; d < D; ++d) O[d] = 0.0;
    *lse = -INFINITY;
    return;
  }
  double M = -INFINITY;
  if (e1 && m1 > M) M = m1;
  if (e2 && m2 > M) M = m2;
  double w1 = e1 ? exp2(m1 - M) : 0.0, w2 = e2 ? exp2(m2 - M) : 0.0;
  double L = w1 * l1 + w2 * l2;
  for (int d = 0; d < D; ++d) O[d] = ((e1 ? w1 * o1[d] : 0.0) + (e2 ? w2 * o2[d] : 0.0)) / L;
  *lse = log(2.0) * (c + M + log2(L));
}

/* ------------------------------------------------------------------------ */
/* Reference: exact attention in FP64                                        */
/* ------------------------------------------------------------------------ */

/* softmax(scale q K^T) V over the visible keys of row r, FP64. */
void orc_exact_row(const orc_params* p, const float* Qh, const float* Kh, const float* Vh, int r,
                   double* O, double* lse) {
  int D = p->D;
  double scale = p->scale > 0.0f ? (double)p->scale : 1.0 / sqrt((double)D);
  const float* q = Qh + (size_t)r * D;
  double mx = -INFINITY;
  double* sc = (double*)malloc((size_t)(p->Nkv > 0 ? p->Nkv : 1) * sizeof(double));
  for (int k = 0; k < p->Nkv; ++k) {
    double v = -INFINITY;
    if (visible(p, r, k)) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += (double)q[d] * (double)Kh[(size_t)k * D + d];
      v = scale * dot;
    }
    sc[k] = v;
    if (v > mx) mx = v;
  }
  for (int d = 0; d < D; ++d) O[d] = 0.0;
  if (mx == -INFINITY) { *lse = -INFINITY; free(sc); return; }
  double L = 0.0;
  for (int k = 0; k < p->Nkv; ++k) {
    if (sc[k] == -INFINITY) continue;
    double w = exp(sc[k] - mx);
    L += w;
    for (int d = 0; d < D; ++d) O[d] += w * (double)Vh[(size_t)k * D + d];
  }
  for (int d = 0; d < D; ++d) O[d] /= L;
  *lse = mx + log(L);
  free(sc);
}

/* ------------------------------------------------------------------------ */
/* Whole-problem driver over a list of row groups, with worker threads       */
/* ------------------------------------------------------------------------ */

typedef struct {
  const orc_params* p;
  /* inputs (float32 values of the fp16/bf16 tensors) */
  const float *Q, *K, *V;
  /* quantised operands and per-head scales (from the quantise step) */
  const uint8_t *qc, *qs, *kc, *ks, *vc, *vs;
  const uint8_t *qc2, *qs2;  /* the residual term of Q, or NULL */
  const float *kbar, *g_v;
  const int32_t* jq;
  const float *inv_q, *inv_k, *inv_v; /* per-head scales (unquantised operands) */
  const float* vw;   /* [B][Hkv][NT] value-norm weights (used with p->vweight) */
  /* per (b, q-head) score factor when Q has a scale of its own (an ablation
   * of the tied scale: Q normalised by 6 / max|Q|), or NULL: alpha = 2^jq */
  const double* alpha_q;
  /* work list: triplets (b, h, g) */
  const int32_t* groups;
  int ngroups;
  /* outputs, full size */
  uint8_t* hot;      /* [B][Hq][NG][NT] */
  double* margin;    /* [B][Hq][NG][NT] */
  double* m1;        /* [B][Hq][Nq] */
  float* l1;
  float* lam;
  float* o1;         /* [B][Hq][Nq][D] */
  double* shift;     /* [B][Hq][Nq] */
  double* m2;        /* [B][Hq][Nq] */
  double* l2;
  double* o2;        /* [B][Hq][Nq][D] */
  double* cr;        /* [B][Hq][Nq] */
  double* O;         /* [B][Hq][Nq][D] merged, FP64 */
  double* lse;       /* [B][Hq][Nq] */
  int do_pass2;
  /* scheduling */
  int next;
  pthread_mutex_t mu;
} orc_job;

static void run_group(orc_job* J, int w) {
  const orc_params* p = J->p;
  int b = J->groups[3 * w], h = J->groups[3 * w + 1], g = J->groups[3 * w + 2];
  int D = p->D, G = p->Hq / p->Hkv, hk = h / G, NT = n_tiles(p), R = p->rg;
  int Bs = p->fmt == ORC_NV ? 16 : 32;
  int NG = (p->Nq + R - 1) / R, NkvP = NT * p->tile;
  size_t bh = (size_t)b * p->Hq + h, bk = (size_t)b * p->Hkv + hk;
  orc_head_ops ops;
  ops.p = p;
  ops.qc = J->qc + bh * p->Nq * (D / 2);
  ops.qs = J->qs + bh * p->Nq * (D / Bs);
  ops.qc2 = J->qc2 ? J->qc2 + bh * p->Nq * (D / 2) : NULL;
  ops.qs2 = J->qs2 ? J->qs2 + bh * p->Nq * (D / Bs) : NULL;
  ops.kc = J->kc + bk * p->Nkv * (D / 2);
  ops.ks = J->ks + bk * p->Nkv * (D / Bs);
  ops.vc = J->vc + bk * D * (NkvP / 2);
  ops.vs = J->vs + bk * D * (NkvP / Bs);
  ops.NkvP = NkvP;
  ops.alpha = J->alpha_q ? J->alpha_q[bh] : ldexp(1.0, J->jq[bh]);
  ops.g_v = J->g_v[bk];
  ops.Qh = J->Q + bh * p->Nq * D;
  ops.Kh = J->K + bk * p->Nkv * D;
  ops.Vh = J->V + bk * p->Nkv * D;
  ops.kbar = J->kbar + bk * D;
  ops.inv_q = J->inv_q[bh];
  ops.inv_k = J->inv_k[bk];
  ops.inv_v = J->inv_v[bk];
  ops.tw = p->vweight && J->vw ? J->vw + bk * NT : NULL;
  int r0 = g * R;
  orc_p1_out out;
  out.hot = J->hot + (bh * NG + g) * NT;
  out.margin = J->margin + (bh * NG + g) * NT;
  out.m = J->m1 + bh * p->Nq + r0;
  out.l = J->l1 + bh * p->Nq + r0;
  out.lam = J->lam + bh * p->Nq + r0;
  out.o = J->o1 + (bh * p->Nq + r0) * D;
  out.shift_max = J->shift + bh * p->Nq + r0;
  double shift_tmp[16];
  if (p->Nq - r0 < R) out.shift_max = shift_tmp; /* partial group: copy back below */
  orc_pass1_group(&ops, g, &out);
  int nr = p->Nq - r0 < R ? p->Nq - r0 : R;
  if (out.shift_max == shift_tmp)
    for (int i = 0; i < nr; ++i) J->shift[bh * p->Nq + r0 + i] = shift_tmp[i];
  if (!J->do_pass2) return;
  const float* Qh = J->Q + bh * p->Nq * D;
  const float* Kh = J->K + bk * p->Nkv * D;
  const float* Vh = J->V + bk * p->Nkv * D;
  double* m2 = J->m2 + bh * p->Nq + r0;
  double* l2 = J->l2 + bh * p->Nq + r0;
  double* o2 = J->o2 + (bh * p->Nq + r0) * D;
  double* cr = J->cr + bh * p->Nq + r0;
  orc_pass2_group(p, Qh, Kh, Vh, J->kbar + bk * D, out.hot, g, m2, l2, o2, cr);
  double* o1d = (double*)malloc((size_t)D * sizeof(double));
  for (int i = 0; i < nr; ++i) {
    for (int d = 0; d < D; ++d) o1d[d] = (double)out.o[(size_t)i * D + d];
    orc_merge_row(D, out.m[i], (double)out.l[i], o1d, m2[i], l2[i], o2 + (size_t)i * D, cr[i],
                  J->O + (bh * p->Nq + r0 + i) * D, J->lse + bh * p->Nq + r0 + i);
  }
  free(o1d);
}

static void* worker(void* arg) {
  orc_job* J = (orc_job*)arg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int w = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (w >= J->ngroups) break;
    run_group(J, w);
  }
  return NULL;
}

/* Runs pass 1 (and, if do_pass2, the exact pass 2 and the merge) for the
 * listed row groups on nthreads threads.  Each group is computed by one thread
 * in a fixed order, so results do not depend on the thread count. */
int orc_run_groups(orc_job* J, int nthreads) {
  J->next = 0;
  pthread_mutex_init(&J->mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J->mu);
  return 0;
}

size_t orc_job_size(void) { return sizeof(orc_job); }
size_t orc_params_size(void) { return sizeof(orc_params); }

/* Reference attention for a list of (b, h, r) rows, threaded the same way. */
typedef struct {
  const orc_params* p;
  const float *Q, *K, *V;
  const int32_t* rows;
  int nrows;
  double* O;   /* [nrows][D] */
  double* lse; /* [nrows] */
  int next;
  pthread_mutex_t mu;
} orc_exact_job;

static void* exact_worker(void* arg) {
  orc_exact_job* J = (orc_exact_job*)arg;
  const orc_params* p = J->p;
  int D = p->D, G = p->Hq / p->Hkv;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int w = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (w >= J->nrows) break;
    int b = J->rows[3 * w], h = J->rows[3 * w + 1], r = J->rows[3 * w + 2];
    size_t bh = (size_t)b * p->Hq + h, bk = (size_t)b * p->Hkv + h / G;
    orc_exact_row(p, J->Q + bh * p->Nq * D, J->K + bk * p->Nkv * D, J->V + bk * p->Nkv * D, r,
                  J->O + (size_t)w * D, J->lse + w);
  }
  return NULL;
}

int orc_exact_rows(const orc_params* p, const float* Q, const float* K, const float* V,
                   const int32_t* rows, int nrows, double* O, double* lse, int nthreads) {
  orc_exact_job J;
  J.p = p; J.Q = Q; J.K = K; J.V = V; J.rows = rows; J.nrows = nrows; J.O = O; J.lse = lse;
  J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, exact_worker, &J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J.mu);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Reports against exact attention (FP64)                                   */
/* ------------------------------------------------------------------------ */

/* Where one row's exact softmax mass and output sit relative to a hot mask:
 * the exact FP64 weights w_k = exp(scale q.k - max) / L over the visible keys,
 * summed per key tile; hot_share and cold_share are the mass on the tiles the
 * mask marks hot and not hot; cold_tile_max is the largest mass of a single
 * tile not marked hot, at tile *cold_tile_arg (-1 if none) -- the "true share
 * of a cold tile" the page compares with eps ("Pass 1", on safe cold
 * verdicts); O_hot and O_cold are the reference output's parts over the hot
 * and the other keys (the diagnostic split of "The bug"), O_ref their sum
 * computed directly, lse the natural log-sum-exp.  hot: [NT] bytes of the
 * row's 16-row group. */
void orc_report_row(const orc_params* p, const float* Qh, const float* Kh, const float* Vh,
                    const uint8_t* hot, int r, double* O_ref, double* O_hot, double* O_cold,
                    double* lse, double* hot_share, double* cold_share, double* cold_tile_max,
                    int* cold_tile_arg) {
  int D = p->D, T = p->tile, NT = n_tiles(p);
  double scale = p->scale > 0.0f ? (double)p->scale : 1.0 / sqrt((double)D);
  const float* q = Qh + (size_t)r * D;
  double* sc = (double*)malloc((size_t)(p->Nkv > 0 ? p->Nkv : 1) * sizeof(double));
  double mx = -INFINITY;
  for (int k = 0; k < p->Nkv; ++k) {
    double v = -INFINITY;
    if (visible(p, r, k)) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += (double)q[d] * (double)Kh[(size_t)k * D + d];
      v = scale * dot;
    }
    sc[k] = v;
    if (v > mx) mx = v;
  }
  for (int d = 0; d < D; ++d) O_ref[d] = O_hot[d] = O_cold[d] = 0.0;
  *hot_share = *cold_share = *cold_tile_max = 0.0;
  *cold_tile_arg = -1;
  if (mx == -INFINITY) { *lse = -INFINITY; free(sc); return; }
  double L = 0.0;
  for (int k = 0; k < p->Nkv; ++k)
    if (sc[k] != -INFINITY) L += exp(sc[k] - mx);
  for (int t = 0; t < NT; ++t) {
    double tile_mass = 0.0;
    for (int k = t * T; k < p->Nkv && k < (t + 1) * T; ++k) {
      if (sc[k] == -INFINITY) continue;
      double w = exp(sc[k] - mx) / L;
      tile_mass += w;
      for (int d = 0; d < D; ++d) {
        double wv = w * (double)Vh[(size_t)k * D + d];
        O_ref[d] += wv;
        if (hot[t]) O_hot[d] += wv; else O_cold[d] += wv;
      }
    }
    if (hot[t]) {
      *hot_share += tile_mass;
    } else {
      *cold_share += tile_mass;
      if (tile_mass > *cold_tile_max) { *cold_tile_max = tile_mass; *cold_tile_arg = t; }
    }
  }
  *lse = mx + log(L);
  free(sc);
}

typedef struct {
  const orc_params* p;
  const float *Q, *K, *V;
  const uint8_t* hot;   /* [B][Hq][NG][NT] */
  const int32_t* rows;  /* [nrows][3] (b, q-head, r) */
  int nrows;
  double *O_ref, *O_hot, *O_cold; /* [nrows][D] */
  double *lse, *hot_share, *cold_share, *cold_tile_max; /* [nrows] */
  int32_t* cold_tile_arg;
  int next;
  pthread_mutex_t mu;
} orc_report_job;

static void* report_worker(void* arg) {
  orc_report_job* J = (orc_report_job*)arg;
  const orc_params* p = J->p;
  int D = p->D, G = p->Hq / p->Hkv, NT = n_tiles(p), NG = (p->Nq + p->rg - 1) / p->rg;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int w = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (w >= J->nrows) break;
    int b = J->rows[3 * w], h = J->rows[3 * w + 1], r = J->rows[3 * w + 2];
    size_t bh = (size_t)b * p->Hq + h, bk = (size_t)b * p->Hkv + h / G;
    orc_report_row(p, J->Q + bh * p->Nq * D, J->K + bk * p->Nkv * D, J->V + bk * p->Nkv * D,
                   J->hot + (bh * NG + r / p->rg) * NT, r, J->O_ref + (size_t)w * D,
                   J->O_hot + (size_t)w * D, J->O_cold + (size_t)w * D, J->lse + w,
                   J->hot_share + w, J->cold_share + w, J->cold_tile_max + w,
                   J->cold_tile_arg + w);
  }
  return NULL;
}

/* orc_report_row for a list of rows on nthreads threads (each row computed
 * by one thread: results do not depend on the thread count). */
int orc_report_rows(orc_report_job* J, int nthreads) {
  J->next = 0;
  pthread_mutex_init(&J->mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, report_worker, J);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  pthread_mutex_destroy(&J->mu);
  return 0;
}

size_t orc_report_job_size(void) { return sizeof(orc_report_job); }
