/*
 * apa.h -- C ABI of the MI355X (gfx950) adaptive-precision attention prefill
 * library (libapa.so).
 *
 * The method is APA as described in "APA: sloppy attention, exact where it
 * counts" (rfriedmann.de/blog/apa-adaptive-precision-attention): pass 1 runs
 * every key tile of a causal GQA prefill in block-scaled FP4 and marks a tile
 * "hot" for a 16-row group when any row's tile mass exceeds eps of its running
 * sum; pass 2 recomputes only the hot tiles in exact FP16; one log-sum-exp
 * merge combines the two online-softmax states ("The merge that makes it
 * exact").  Tensor layout and masking follow the FFPA documentation
 * (ffpa-attn.readthedocs.io, note on cross-attention, GQA and causal):
 * Q [B, Hq, Nq, D], K and V [B, Hkv, Nkv, D], contiguous, row-major; query
 * head h uses KV head h / (Hq / Hkv); with is_causal, query row r sees keys
 * k <= r + (Nkv - Nq) (the last query row sits at the last key; needs Nkv >= Nq).
 *
 * Conventions for every call:
 *   - All tensor pointers are caller-owned DEVICE pointers.  The library never
 *     allocates device memory, frees or synchronises; calls are enqueued on
 *     `stream` (a hipStream_t passed as void*, NULL = the null stream) and run
 *     in stream order.  apa_ring_pass1 alone also enqueues work on a second
 *     stream the library creates once per device, ordered against `stream`
 *     by events it creates and releases within the call.
 *   - The return value is synchronous validation plus launch status.  On any
 *     non-APA_OK return nothing was enqueued, except APA_ERR_HIP, which reports
 *     a failed launch (earlier kernels of the same call may have run).
 *   - Optional pointers are marked "may be NULL".
 *   - Empty problems (B, Hq or Nq equal to 0) return APA_OK and do nothing.
 */
#ifndef APA_H
#define APA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum apa_status {
  APA_OK = 0,
  APA_ERR_INVALID_ARG = 1, /* NULL required pointer, bad shape or parameter */
  APA_ERR_UNSUPPORTED = 2, /* valid, but not implemented on this device     */
  APA_ERR_WORKSPACE = 3,   /* workspace too small (see apa_workspace_bytes)  */
  APA_ERR_HIP = 4          /* a kernel launch failed                         */
} apa_status;

enum { APA_F16 = 0, APA_BF16 = 1 };        /* input / output element type */
enum { APA_MXFP4 = 0, APA_NVFP4 = 1 };     /* FP4 block format             */
/* How apa_pass1 maps 32-row blocks of one query head to wavefronts when it
 * is given a workspace (see apa_pass1).  AUTO picks from the shape. */
enum { APA_SCHED_AUTO = 0, APA_SCHED_WHOLE = 1, APA_SCHED_PAIRS = 2, APA_SCHED_TRIPLES = 3 };

/* Problem descriptor.  Fill it with apa_problem_init() and override fields. */
typedef struct apa_problem {
  int32_t B, Hq, Hkv, Nq, Nkv, D; /* D in {64, 128, 256, 512}; Hq % Hkv == 0;
                                     apa_pass2 and apa_exact also need the group
                                     size Hq / Hkv in {1, 2, 3, 4, 6, 8}
                                     (else APA_ERR_UNSUPPORTED)                  */
  int32_t dtype;                  /* APA_F16 or APA_BF16 (Q, K, V and the output) */
  int32_t is_causal;              /* 1: tail-aligned causal mask; 0: none        */
  float scale;                    /* softmax scale; <= 0 selects 1/sqrt(D)       */
  int32_t tile;                   /* keys per tile; must be 64 ("tiles of 64")  */
  int32_t row_group;              /* rows per hot verdict; must be 16            */
  int32_t fmt;                    /* APA_MXFP4 (NVFP4 exists only in the oracle) */
  float tau;                      /* lazy-max threshold in log2 units, in [0, 32]
                                     (4)                                         */
  float hot_frame_offset;         /* H: a hot tile lifts the frame to at most
                                     max(m, c - H); an integer in [0, 64] (32)  */
  int32_t pass1_schedule;         /* APA_SCHED_*: scheduling only, the results
                                     agree up to FP32 summation order (AUTO)   */
  int32_t q_terms;                /* FP4 terms of Q in pass 1: 1, or 2 (the
                                     APA page's "Second hunt" fix: Q1, then the
                                     FP4 residual Q - Q1 in the same per-head
                                     scale, both against the same K codes;
                                     D <= 256, else APA_ERR_UNSUPPORTED) (1)  */
  int32_t k_scale_lsq;            /* 1: each 32-channel block exponent of K is
                                     picked from {e, e-1, e+1} (e: the smallest
                                     that does not clip) by least squared error,
                                     the APA page's other "Second hunt" fix;
                                     the error is summed in FP32 in a fixed
                                     order; 0: the nearest rule (0)           */
  int32_t window;                 /* > 0: causal sliding window of this many keys
                                     (the APA page's "What else is in the box"):
                                     row r sees keys r + Nkv - Nq - window < k
                                     <= r + Nkv - Nq; a row group whose first
                                     row no longer sees tile 0 visits its tiles
                                     from the diagonal backwards; needs
                                     is_causal.  0: the full causal mask (0)   */
  int32_t kv_capacity;            /* keys the FP4 buffer's K/V sections hold (a
                                     persistent FP4 K/V cache for chunked
                                     prefill: every chunk's problem names the
                                     same capacity, so those sections keep their
                                     size and place); >= Nkv.  0: Nkv (0)       */
  int32_t stat_keys;              /* > 0: the K/V statistics (key mean, per-head
                                     scales) cover the keys before this one --
                                     chunked prefill keeps them from its last
                                     restat (the APA page restats once the
                                     context has grown by 1.125x); later keys
                                     beyond their range clamp at the FP4
                                     maximum.  0: all keys (0)                */
  const int32_t* block_table;     /* paged 16-bit K/V (the APA page: pass 2 reads
                                     through a block table): NULL, or a DEVICE
                                     array [B][block_table_stride] of page
                                     indices; then k and v of every call are
                                     pools [pages][Hkv][64][D] and key k of
                                     batch b is row k % 64 of page
                                     block_table[b * stride + k / 64] (NULL) */
  int32_t block_table_stride;     /* entries per batch row, >= ceil(Nkv / 64) */
  int32_t hot_weight;             /* 1: the hot test weighs each tile's mass by
                                     its value-norm weight w_t (the APA page's
                                     "Honest limits": a cold tile's small mass
                                     can still carry a large output part; the
                                     page proposes a test weighted by value
                                     norm): w_t = max(1, nu_t / nu_bar), nu_t
                                     the largest L2 norm of a value vector in
                                     tile t, nu_bar the mean norm over the keys
                                     the statistics cover (w_t = 1 when nu_bar
                                     is 0).  A row's tile counts as hot when
                                     l_t * w_t > eps * lambda, so a cold tile
                                     adds at most eps * lambda * nu_bar to the
                                     row's unnormalised output and keeps its
                                     mass share under eps.  apa_quantize writes
                                     the weights into the FP4 buffer; every call
                                     on one FP4 buffer must name the same value.
                                     0: the mass test (0)                       */
  int32_t ring_tiles;             /* KV window ring (the APA page's "What else
                                     is in the box"): 0, or the key tiles R of
                                     each of two ring halves, a multiple of 32
                                     (the page uses 96).  The FP4 buffer then
                                     holds 1 + 2R tile blobs per (b, kv-head):
                                     the sink tile 0 and the halves, and only
                                     apa_ring_pass1 fills and walks them;
                                     apa_quantize, apa_quantize_tiles,
                                     apa_quantize_static and apa_pass1 return
                                     APA_ERR_UNSUPPORTED.  Needs D <= 256, no
                                     window and the mass test (0)              */
} apa_problem;

/* Defaults: scale 1/sqrt(D), tile 64, row_group 16, MXFP4, tau 4, H 32,
 * fp16, causal, APA_SCHED_AUTO, one Q term, nearest K block exponents, no
 * window, capacity Nkv, statistics over all keys, flat K/V, the mass-only
 * hot test. */
void apa_problem_init(apa_problem* p, int32_t B, int32_t Hq, int32_t Hkv, int32_t Nq,
                      int32_t Nkv, int32_t D);

/* Byte offsets of the sections of the FP4 buffer written by apa_quantize,
 * the K/V sections first (kv_blobs, kbar, kv_head, tile_w, status: sized by the
 * capacity, so a persistent cache keeps them), then the query sections.
 * NqP = Nq rounded up to 32, NkvP = Nkv rounded up to 64, NTc = the capacity
 * in 64-key tiles; padding rows and keys hold zero codes.  Codes pack two 4-bit E2M1 values per byte, element
 * 2i in the low nibble; a scale byte is an E8M0 exponent (value 2^(byte-127))
 * of one 32-element block.
 *   q_codes  [B][Hq][NqP][D/2]       Q along D
 *   q_scales [B][Hq][NqP][D/32]
 *   kv_blobs [B][Hkv][NTc][68*D]  one blob per 64-key tile, in the
 *            operand order of the pass-1 MFMAs:
 *              [0, 32D)    K - kbar codes, [64 keys][D/2], along D
 *              [32D, 34D)  K scales, [64 keys][D/32]
 *              [34D, 66D)  V codes along keys, [D channels][32]: 16 bytes
 *                          per 32-key half whose eight 4-key runs are
 *                          stored in the order 0,2,4,6,1,3,5,7 (the lane
 *                          order of the P operand of the P.V product)
 *              [66D, 68D)  V scales, channel 32*db + n and key half hh at
 *                          byte (2n + hh) * D/32 + db
 *   kbar     [B][Hkv][D] float       per-channel key mean
 *   kv_head  [B][Hkv][8] float       amax_K, g_K, inv_K, amax_V, 1, 1 (V's scale),
 *                                    nu_bar (with hot_weight, else 0), 0;
 *                                    amax_V is max |V| over every key coded
 *                                    (a call with frozen statistics raises it
 *                                    to cover its tiles): the 16-bit pass
 *                                    shifts bf16 V into the fp16 range by it
 *   tile_w   [B][Hkv][NTc] float     with hot_weight: the value-norm weight
 *                                    w_t of every tile some row sees (the
 *                                    rest untouched)
 *   q_head   [B][Hq][4]  float       amax_Q, inv_Q, j (as float: alpha = 2^j), 0
 *   q_frame  [B][Hq][NqP] float      c_r = sl * q.kbar, sl = fl32(scale*log2 e)
 *   status   uint32                  bit 0: a non-finite input was seen;
 *                                    bit 1: a wait of apa_fused gave up
 *   q2_codes, q2_scales               with q_terms = 2: the residual term of Q,
 *            laid out as q_codes and q_scales: per 32-channel block, the
 *            FP32 residual of the normalised values after the first term's
 *            dequantised values, with its own E8M0 exponent (empty sections
 *            with one term)                                                  */
typedef struct apa_fp4_layout {
  size_t q_codes, q_scales, kv_blobs;
  size_t kbar, kv_head, tile_w, q_head, q_frame, status, q2_codes, q2_scales, total;
} apa_fp4_layout;

apa_status apa_fp4_layout_of(const apa_problem* p, apa_fp4_layout* out);
size_t apa_fp4_bytes(const apa_problem* p);

/* Hot mask: uint32 words [B][Hq][ceil(Nq/16)][ceil(ceil(Nkv/64)/32)];
 * bit (t % 32) of word (t / 32) is tile t of that 16-row group. */
size_t apa_hotmask_bytes(const apa_problem* p);

enum { APA_CALL_QUANTIZE = 0, APA_CALL_PASS1 = 1, APA_CALL_PASS2 = 2, APA_CALL_MERGE = 3,
       APA_CALL_EXACT = 4, APA_CALL_RING_PASS1 = 5, APA_CALL_FUSED = 6 };
/* Scratch bytes the given call needs in its `ws` argument (0: pass NULL). */
size_t apa_workspace_bytes(const apa_problem* p, int32_t which_call);

const char* apa_status_string(apa_status s);

/* Text of the HIP error behind the calling thread's last APA_ERR_HIP. */
const char* apa_last_hip_error(void);

/* a1 + a2: statistics and block-scaled FP4 quantisation ("Mean-centred K" and
 * the format paragraph of "Pass 1: FP4 everywhere, with a hot test").
 * Reads q, k, v (dtype of p), writes the whole FP4 buffer `fp4`
 * (apa_fp4_bytes(p) bytes, 256-byte aligned).  Per (b, kv-head): kbar = the
 * per-channel mean of K (FP64 sum in a fixed order), K is centred, and
 * K - kbar is normalised by one FP32 scale per head that maps the head's
 * largest magnitude to 6; Q's per-head scale is tied to K's so the score
 * factor is a power of two 2^j; V keeps its own scale (per-head scale 1:
 * the E8M0 block exponents hold its range).  Blocks of 32 (Q, K along D; V
 * along keys) get an E8M0 exponent, the smallest that fits the block maximum
 * under 6, and E2M1 codes rounded to nearest even.  With hot_weight it also
 * writes nu_bar (FP64 sums of the FP32 key norms, keys ascending per tile,
 * then runs of tiles) and the weight of every tile some row sees.  The status
 * word reports non-finite values among Q and every K/V tile it quantises.
 * ws: apa_workspace_bytes(p, APA_CALL_QUANTIZE) bytes. */
apa_status apa_quantize(const apa_problem* p, const void* q, const void* k, const void* v,
                        void* fp4, void* ws, size_t ws_bytes, void* stream);

/* Chunked prefill over a persistent FP4 K/V cache (the APA page, "What else
 * is in the box": chunked prefill keeps the quantised tiles and only
 * quantises new keys): quantises Q, and the K/V tiles [tile_begin, tile_end)
 * of p, with the K/V statistics the FP4 buffer already holds (kbar and the
 * per-head scales of an earlier apa_quantize of the same cache, i.e. the same
 * kv_capacity and stat_keys), leaving every other blob and the statistics as
 * they are.  Q's per-head scale ties to the cache's K scale as in
 * apa_quantize.  A chunk whose keys are [0, Nkv) after a previous chunk
 * ending at key N0 passes tile_begin = N0 / 64 (re-quantising a partly
 * filled last tile).  With hot_weight, the new tiles' weights use the
 * cache's nu_bar.  The status word reports non-finite values among Q and
 * the quantised tiles.  0 <= tile_begin <= tile_end <= ceil(Nkv / 64) (from
 * the window's first tile with a window).  ws: apa_workspace_bytes(p,
 * APA_CALL_QUANTIZE) bytes. */
apa_status apa_quantize_tiles(const apa_problem* p, const void* q, const void* k, const void* v,
                              void* fp4, int32_t tile_begin, int32_t tile_end, void* ws,
                              size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory or call hipMalloc (code
 * under HIP graph capture, tight serving loops, harnesses that forbid it):
 * apa_quantize without a workspace argument.  Its scratch is a fixed device
 * array inside the library, 16 MiB per GPU, held until the process ends;
 * the call allocates nothing.  Problems
 * whose apa_workspace_bytes(p, APA_CALL_QUANTIZE) exceeds that get
 * APA_ERR_WORKSPACE (about B * Hkv * ceil(Nkv / 1024) * D * 16 bytes plus
 * 8 bytes per 64-key tile and 128-channel slice: 960000 keys at 8 KV heads
 * and D = 128 fit).  Every call on one GPU uses
 * that GPU's one array, and each call writes all of the scratch it reads, so
 * nothing carries over between calls; calls that overlap on one GPU (on
 * different streams without ordering) race and must not be issued.  Same
 * arguments and results as apa_quantize otherwise. */
apa_status apa_quantize_static(const apa_problem* p, const void* q, const void* k, const void* v,
                               void* fp4, void* stream);

/* a3..a7: pass 1 ("Pass 1: FP4 everywhere, with a hot test", steps 1-5;
 * "Tile order"; the lazy maximum; the decoupled cold frame of "The bug").
 * Every row group of 16 rows visits its tiles in the order 0, d, d-1, ..., 1
 * (d = its causal diagonal tile), scores them from the FP4 buffer, quantises
 * P per 32-key group, takes the tile row sums with a ones-operand MFMA, and
 * marks the tile hot when any row's sum (times the tile's value-norm weight
 * with hot_weight) exceeds eps times its running sum (eps == 0: every
 * visited tile hot).  Cold tiles accumulate P.V in FP4.
 * Outputs (all [B][Hq][Nq], FP32 unless noted):
 *   cold_m  int32 log2 frame of the cold state (INT32_MIN: empty row)
 *   cold_l  cold row sum in that frame
 *   cold_o  [B][Hq][Nq][D] cold unnormalised output times g_V
 *   hot_bits  apa_hotmask_bytes(p) bytes (every word written)
 *   lambda_out  may be NULL: final running sum in the frame cold_m
 * eps must be >= 0 and not NaN (+inf allowed).  Requires the FP4 buffer of
 * apa_quantize for the same problem.
 * ws: NULL, or apa_workspace_bytes(p, APA_CALL_PASS1) bytes (0 for problems
 * whose 32-row blocks already fill the GPU, and at D = 512, where every
 * block runs as two wavefronts, each holding half of the output channels).
 * With a workspace, each long visit order (64 tiles or more) is cut in two:
 * a head wavefront walks its first part while a tail wavefront of the same
 * work group walks the rest.  APA_SCHED_PAIRS gives every block its own tail
 * wavefront (two per block); APA_SCHED_TRIPLES runs three blocks on four
 * wavefronts, one tail wavefront walking the three shorter tails one after
 * the other; APA_SCHED_WHOLE keeps one wavefront per block.  AUTO takes
 * PAIRS while two waves per block fit the GPU's wave slots at once, TRIPLES
 * while four per three blocks do, else WHOLE; at D = 512 every request runs
 * as WHOLE.  The
 * workspace holds the tiles a tail cannot decide until its head is done
 * (at most 512 per 32-row block, 292 bytes each) and room to hand the
 * head's state to a re-walk of the tail, for blocks with more undecided
 * tiles than that.  Without one, every block runs as one wavefront (slower
 * when the blocks do not fill the GPU).  The verdicts and the state are
 * those of a single walk up to FP32 summation order; the returned frame
 * cold_m is then the larger of the two parts' frames (the state is scaled
 * to match, so cold_l * 2^cold_m and cold_o / cold_l do not depend on it). */
apa_status apa_pass1(const apa_problem* p, const void* fp4, float eps, int32_t* cold_m,
                     float* cold_l, float* cold_o, uint32_t* hot_bits, float* lambda_out,
                     void* ws, size_t ws_bytes, void* stream);

/* Host-only query of how apa_pass1 with a workspace cuts visit orders (no
 * device work).  Returns the schedule such a launch runs for p
 * (APA_SCHED_WHOLE, _PAIRS or _TRIPLES; -1 for an invalid p).  For a visit
 * order of npos >= 0 positions, *cut (may be NULL) receives the first
 * position the tail wavefront walks: npos when the order runs whole, else a
 * value with 32 <= cut <= npos - 8 (the tail first replays positions
 * [0, 32)).  *records (may be NULL) receives the undecided tail tiles kept
 * per 32-row block (0 under APA_SCHED_WHOLE). */
int32_t apa_pass1_split(const apa_problem* p, int32_t npos, int32_t* cut, int32_t* records);

/* f3: pass 1 over a KV window ring ("What else is in the box": a sink tile
 * plus two ring halves of R = p->ring_tiles FP4 tiles per KV head, the next
 * key segment quantised while pass 1 walks the current one).  Does what
 * apa_quantize then apa_pass1 do, with the FP4 K/V copy bounded to 1 + 2R
 * tiles per KV head whatever Nkv is: the statistics over every key (one read
 * of K and V), Q's codes, the sink tile; then, per segment of R tiles from the
 * top down, that segment's FP4 codes into the ring half it alternates to (on
 * a second stream the library keeps per device, ordered by events so that a
 * half is rewritten only after the walk that reads it is done) and one launch
 * of pass 1 over the segment for every 32-row block, carrying each block's
 * state through the workspace.  Every row walks its tiles in the same order
 * as apa_pass1 with one wave per block (APA_SCHED_WHOLE), so the outputs
 * (cold state, hot mask, lambda) equal that call's bit for bit; apa_pass2
 * then runs as usual on the same FP4 buffer (its Q frames and scales) and the
 * 16-bit K/V.  The status word ORs the non-finite checks of every read.
 * Arguments as apa_quantize and apa_pass1; ws: apa_workspace_bytes(p,
 * APA_CALL_RING_PASS1) bytes (the quantise scratch, then per 32-row block
 * and query head 128 D + 1040 bytes rounded up to 256).  Calls on one device
 * must not overlap (they share its second stream's order). */
apa_status apa_ring_pass1(const apa_problem* p, const void* q, const void* k, const void* v,
                          void* fp4, float eps, int32_t* cold_m, float* cold_l, float* cold_o,
                          uint32_t* hot_bits, float* lambda_out, void* ws, size_t ws_bytes,
                          void* stream);

/* a8..a10: pass 2 ("Pass 2: exact FP16 on the hot tiles").  Compacts the hot
 * mask into per-work-group lists of tiles hot for any of its row groups, then
 * runs FP16 MFMA flash attention (FP32 online softmax) over those tiles only,
 * scoring s = sl*q.k - c_r so both passes share the centred logit frame.
 * fuse_merge = 1: merges with the pass-1 state (see apa_merge) and writes
 * out [B][Hq][Nq][D] (dtype of p) and lse [B][Hq][Nq] (natural log, may be
 * NULL).  fuse_merge = 0: writes the hot state hot_m (log2 units, -inf for an
 * empty row), hot_l, hot_o [..][D] (unnormalised) instead.
 * ws: apa_workspace_bytes(p, APA_CALL_PASS2) bytes. */
apa_status apa_pass2(const apa_problem* p, const void* q, const void* k, const void* v,
                     const void* fp4, const uint32_t* hot_bits, const int32_t* cold_m,
                     const float* cold_l, const float* cold_o, int32_t fuse_merge, void* out,
                     float* lse, float* hot_m, float* hot_l, float* hot_o, void* ws,
                     size_t ws_bytes, void* stream);

/* f1: pass 1 and pass 2 (with the fused merge) in one persistent launch
 * ("Pass 2: exact FP16 on the hot tiles": one work group per compute unit
 * takes ordered tickets, the pass-1 work first, then pass-2 work, whose waits
 * are only on tickets that running work groups hold).  Does what apa_pass1
 * (with its workspace) and then apa_pass2 with fuse_merge = 1 do, in one
 * kernel launch (plus a clear of its control words): the same cold state,
 * hot mask, lambda, output and lse, bit for bit.  A pass-2 work group starts
 * as soon as the pass-1 units of its row blocks are done, while other work
 * groups are still in pass 1.  Arguments as apa_pass1 and apa_pass2 (out is
 * required); ws: apa_workspace_bytes(p, APA_CALL_FUSED) bytes (control
 * words, the pass-1 workspace, the split states).  Covers D = 64 and 128
 * (fp16 or bf16, one or two Q terms, with or without value-norm weights; no
 * ring),
 * the GQA groups of apa_pass2 and at most 4096 key tiles (Nkv <= 262144);
 * other problems get APA_ERR_UNSUPPORTED.  Every wait inside the launch is bounded: one that
 * gives up (it cannot while the GPU runs the launch's work groups) sets bit 1
 * of the FP4 buffer's status word, and the outputs are then invalid.  Calls
 * sharing a workspace must not overlap. */
apa_status apa_fused(const apa_problem* p, const void* q, const void* k, const void* v,
                     const void* fp4, float eps, int32_t* cold_m, float* cold_l, float* cold_o,
                     uint32_t* hot_bits, float* lambda_out, void* out, float* lse, void* ws,
                     size_t ws_bytes, void* stream);

/* a10: exact merge of the cold and hot states ("The merge that makes it
 * exact"): M = max(m1, m2) over non-empty states, w_i = 2^(m_i - M),
 * O = (w1 o1 + w2 o2) / (w1 l1 + w2 l2); a state with l = 0 is empty and
 * skipped; both empty gives O = 0 and lse = -inf ("Half the bytes, exactly
 * merged", section "The merge").  lse = ln2 (c_r + M + log2 L) with c_r from
 * the FP4 buffer; lse may be NULL. */
apa_status apa_merge(const apa_problem* p, const void* fp4, const int32_t* cold_m,
                     const float* cold_l, const float* cold_o, const float* hot_m,
                     const float* hot_l, const float* hot_o, void* out, float* lse,
                     void* stream);

/* a11: all-exact FP16 flash attention over every visible tile (the baseline
 * APA is compared against in the post's introduction, where it takes
 * 13.023 ms for the 2048 x 122880 case on that post's GPU).  Same masking and GQA rules; out in dtype of
 * p, lse natural log (may be NULL).  ws: apa_workspace_bytes(p,
 * APA_CALL_EXACT) bytes. */
apa_status apa_exact(const apa_problem* p, const void* q, const void* k, const void* v,
                     void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* APA_H */
