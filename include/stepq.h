/*
 * stepq.h — C ABI of the quantized recurrent-state decode library (gfx950).
 *
 * One decode step of gated delta-rule linear attention with a packed, low-bit
 * recurrent state per (request slot, head), as described by
 *   [SQ]  "STEPQuant: When and Where Errors Matter in Delta-Rule Recurrent
 *          State Quantization" (Sec. 3, Sec. 4, appendices A-F), and
 *   [LQ]  the reading notes on "LeapQuant" (Sec. 2.1-2.6, 4.5), for the
 *          per-window variant.
 *
 * Conventions for every entry point:
 *   - all functions are `extern "C"`, return an sq_status and never throw;
 *     on failure `sq_last_error()` (thread-local) describes the cause;
 *   - "device" pointers are device memory owned by the caller (for example
 *     torch tensors); the library never allocates device memory;
 *   - device-side calls are asynchronous on the given stream (0 = the null
 *     stream); a kernel fault surfaces at the next synchronisation, as in HIP;
 *   - fp32 arrays are dense, row-major, with the shapes given per argument;
 *   - slot ids are int32 device arrays; ids in one call must be distinct
 *     (one workgroup owns one (slot, head) tile and updates it in place) and
 *     lie in [0, n_slots).  Kernels skip a tile whose id is out of range and
 *     write NaN to its outputs, so a bad id never touches memory outside the
 *     pool.  With the environment variable SQ_VALIDATE=1 the host also copies
 *     the ids back and returns SQ_ESLOT_RANGE / SQ_EDUP_SLOT before launching;
 *   - one pool must not be used by two streams at once (caller's duty).
 *
 * ------------------------------------------------------------------------
 * Packed slot layout (all multi-byte values little-endian)
 * ------------------------------------------------------------------------
 * A slot holds the H heads in order; head h starts at byte head_off[h]
 * (sq_plan_desc.head_off) and every head is padded with zero bytes to a
 * multiple of 256; slot_bytes = sum of the padded head sizes.  Slot s of a
 * pool starts at byte s * slot_bytes.
 *
 * Codes are symmetric b-bit two's-complement integers z in [-q_b, q_b],
 * q_b = 2^(b-1) - 1 (so q = 1, 7, 31, 127 for b = 2, 4, 6, 8; [SQ] App. B.5
 * gives [-31, 31] at six bits).  "b = 16" stores IEEE binary16 values.
 *
 * Column-pair blocked code region (uniform heads, STEP GDN heads incl. FP16
 * pivot heads, window boundary codes).  The d_k x d_v tile is cut into row
 * blocks of 32 rows (rb) and column pairs (p = 0 .. d_v/2-1).  The chunk of
 * (rb, p) holds 64 values, value n = 2m + c being element
 * (row 32 rb + m, column 2 p + c), m in [0, 32), c in {0, 1}; as a
 * little-endian bit stream value n occupies bits [n b, n b + b).  A chunk is
 * 8 b bytes = b/2 pieces of 16 bytes; piece q of chunk (rb, p) is stored at
 * byte (rb * (b/2) * (d_v/2) + q * (d_v/2) + p) * 16 of the region.  The
 * region takes d_k d_v b / 8 bytes.
 *
 * Head kinds:
 *   uniform   : code region (b = plan bits), then d_k FP16 row scales s_i.
 *               Dequantised value s_i z_ij.
 *   STEP GDN  : b in {2,4,6,8}: code region, d_k FP16 row scales r_i, d_v
 *               FP16 column scales c_j.  Dequantised value r_i c_j z_ij / q_b.
 *               b = 16 (FP16 pivot head): the region holds the values
 *               themselves and nothing follows.
 *   STEP KDA  : storage rows in order of (width ascending, key row
 *               ascending) — FP16 pivot rows come last; storage row s holds
 *               key row perm[s] as d_v b / 8 bytes (code j at bits
 *               [j b, j b + b)), or 2 d_v bytes of FP16 values for a pivot
 *               row; then d_k FP16 r in storage order (0 for pivot rows),
 *               then d_v FP16 c shared by all rows of the head.
 *   window    : int32 l (records held) at byte 0, bytes 4..15 zero; float32
 *               alpha[p] at byte 16; INT8 boundary codes Z in the blocked
 *               layout (b = 8) at byte round_up(16 + 4p, 128); then float32
 *               C[d_k] (key-row smoothing), float32 B[d_v] (value-column
 *               scales), float32 Kt[p][d_k] (records beta_i k_i), float32
 *               U[p][d_v] (records u_i); with r compensator pairs, then
 *               FP16 Kc[r][d_k] and FP16 Uc[r][d_v].  Boundary state
 *               S0_aj = C_a (Z_aj / 127) B_j + sum_h Kc[h][a] Uc[h][j]
 *               ([LQ] Sec. 2.4-2.5, Eq. 7, App. B.3).
 *
 * All FP16 scales are stored after clamping to [2^-14, 65504] and rounding
 * to nearest even ([SQ] App. B.5 states this clamp for its INT6 baseline;
 * the library applies it to every FP16 scale).
 */
#ifndef STEPQ_H
#define STEPQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point returns a status and never throws.  A call with an empty
 * batch (B = 0, T = 0 or n_tiles = 0) is a no-op that launches nothing; its
 * batch-sized arrays may then be null, while the plan, device tables and pool
 * must still be valid. */
typedef int32_t sq_status;
enum {
  SQ_OK = 0,
  SQ_EINVAL = 1,          /* null pointer, non-positive size, bad enum        */
  SQ_EUNSUPPORTED = 2,    /* d_k, d_v not in {64, 128}; bits not supported    */
  SQ_ESLOT_RANGE = 3,     /* a slot id outside [0, n_slots) (SQ_VALIDATE=1)   */
  SQ_EDUP_SLOT = 4,       /* a slot id repeated in one call (SQ_VALIDATE=1)   */
  SQ_EPLAN_MISMATCH = 5,  /* call does not fit the plan's mode or kind        */
  SQ_EBUDGET = 6,         /* calibration budget below the smallest width      */
  SQ_EHIP = 7,            /* a HIP call or kernel launch failed               */
  SQ_ENOMEM = 8,          /* host allocation failed                           */
  SQ_ENONFINITE = 9       /* NaN or Inf in calibration statistics             */
};

enum { SQ_MODE_UNIFORM = 0, SQ_MODE_STEP = 1, SQ_MODE_WINDOW = 2 };
enum { SQ_KIND_GDN = 0, SQ_KIND_KDA = 1 };
#define SQ_PIVOT_BITS 16
#define SQ_MAX_COMP_RANK 8      /* compensator pairs per window head            */
#define SQ_MAX_POWER_ITERS 32   /* power iterations per compensator pair        */

typedef struct sq_plan sq_plan; /* opaque host object owned by the library */

/* Read-only view of a plan.  Pointers stay valid until sq_plan_destroy. */
typedef struct {
  int32_t mode, kind, heads, d_k, d_v;
  int32_t uniform_bits;     /* uniform mode: code width                         */
  int32_t window;           /* window mode: p                                    */
  int32_t n_units;          /* STEP: H (GDN) or H*d_k (KDA); else 0              */
  int64_t slot_bytes;       /* padded bytes per slot                             */
  int64_t payload_bytes;    /* unpadded codes + scales + pivots (+ window data)  */
  int64_t analytic_bytes;   /* payload if pivot units also kept scale slots      */
  const int64_t* head_off;  /* [H] byte offset of each head in a slot            */
  const int32_t* unit_bits; /* STEP: [n_units] width per unit, 16 = FP16 pivot   */
  const float* w;           /* STEP: [H*d_k] row impact factors; else NULL       */
  float window_c_floor;     /* window: smoothing floor                           */
  int32_t window_rank;      /* window: compensator pairs per head (0 = none)     */
  int32_t window_iters;     /* window: power iterations per compensator pair     */
} sq_plan_desc;

/* Calibration statistics, one entry per unit u (a GDN head, or a KDA key row
 * in head-major order), collected offline on a calibration stream.
 * [SQ] Sec. 4 (Eqs. 6-8): mean log retention ell_u, distortion d_u(b) of the
 * unit quantised at width b; Sec. 4.1: row-impact score omega_i. */
typedef struct {
  int32_t kind, heads, d_k, d_v;
  int32_t n_cand;
  const int32_t* cand_bits; /* [n_cand] ascending candidate widths (2,4,6,8)      */
  const double* ell;        /* [n_units] mean log retention (<= 0)                */
  const double* dist;       /* [n_units * n_cand] distortion at each width        */
  const double* omega;      /* [heads * d_k] row-impact scores (>= 0)             */
} sq_calib_stats;

typedef struct {
  double nominal_bits;      /* average bit budget b_bar                           */
  double pivot_frac;        /* fraction of units kept as FP16 pivots              */
  double gamma;             /* impact relaxation (0.25); w = (omega/gm)^(gamma/2) */
  int32_t horizon;          /* H of the lifetime weight (2048)                    */
  double omega_floor_rel;   /* relative floor of omega (1e-12)                    */
} sq_calib_opts;

/* ------------------------------------------------- calibration statistics */

/* The statistics sq_calibrate_bits takes, accumulated on the GPU over a
 * calibration stream ([SQ] Sec. 4, Eqs. 6-8; Sec. 4.1, App. B-C).  The caller
 * owns every buffer and zeroes the float64 accumulators before the first call;
 * each call adds to them, and the caller divides by the number of samples.
 *
 * sq_calib_gate_stats adds one step of n sequences: log_sum[u] += sum_s
 * log r_{s,u} (r = alpha[s][h] for a GDN unit u = h; d[s][h][i] for a KDA unit
 * u = h d_k + i) and omega_sum[h][i] += sum_s g_{s,h,i}^2 with the transported
 * query g = D (q - beta k (k . q)) (A_t^T q_t, [SQ] Sec. 4.1).  q, k, gate as in
 * sq_decode_step with batch n; device pointers; float64 arithmetic.  Divided
 * by the sample count: ell_u and omega_i of sq_calib_stats.
 * Errors: SQ_EINVAL, SQ_EUNSUPPORTED (d_k not 64 or 128), SQ_EHIP. */
sq_status sq_calib_gate_stats(int32_t kind, int32_t heads, int32_t d_k, int32_t n,
                              const float* q, const float* k, const float* beta,
                              const float* gate, double* log_sum, double* omega_sum,
                              hipStream_t stream);

/* Row impact factors from omega [heads][d_k] (host memory): w = (omega' /
 * geomean_head(omega'))^(gamma / 2) with omega' = max(omega, floor_rel *
 * max_head(omega)); a head whose omega are all zero gets w = 1 ([SQ] App. B,
 * C; the same function sq_calibrate_bits applies).  w: host [heads][d_k].
 * Errors: SQ_EINVAL, SQ_ENONFINITE. */
sq_status sq_impact_factors(int32_t heads, int32_t d_k, const double* omega, double gamma,
                            double floor_rel, float* w);

/* Distortion d_u(b) of one snapshot ([SQ] Sec. 4, Eq. 8: the error of unit u
 * quantised at width b): the plan's quantizer (a STEP plan of GDN heads, all
 * at width b, no FP16 heads, with the impact factors w) packs the dense tiles
 * S[n][H][d_k][d_v] (tile t = sequence t / H, head t % H) into `packed`
 * (n H sq_max_head_bytes bytes of caller-owned device scratch), then
 * dist_sum[u] += sum over the n sequences of the squared error
 * sum (r_i c_j z_ij / q_b - S_ij)^2 of unit u: a whole head (per_row = 0,
 * u = h) or one key row (per_row = 1, u = h d_k + i).  float64 accumulation
 * with atomic adds (the order of the additions is not fixed).
 * Errors: SQ_EINVAL, SQ_EPLAN_MISMATCH, SQ_EHIP. */
sq_status sq_calib_distortion(const sq_plan* plan, const void* dev_plan, int32_t n,
                              const float* S, void* packed, int32_t per_row, double* dist_sum,
                              hipStream_t stream);

/* sq_calib_distortion for callers that cannot allocate device memory (code
 * under HIP graph capture, serving loops, harnesses that forbid hipMalloc):
 * the packed heads go to a device array inside the library instead of a
 * caller buffer.  The array holds 16 MiB on each GPU the library runs on,
 * from the first call on that GPU until the process ends; calls needing more
 * than that (n H sq_max_head_bytes > 16 MiB) fail with SQ_EINVAL before
 * launching anything.  The call allocates nothing.  Every call on one GPU
 * shares that GPU's array, so calls that overlap on one GPU (on different
 * streams, or from several threads without ordering) race; calls ordered on
 * one stream do not.  Arguments, results and the other errors as
 * sq_calib_distortion. */
sq_status sq_calib_distortion_noalloc(const sq_plan* plan, const void* dev_plan, int32_t n,
                                      const float* S, int32_t per_row, double* dist_sum,
                                      hipStream_t stream);

/* ---------------------------------------------------------------- plans */

/* Lifetime-aware bit allocation with sparse FP16 pivots ([SQ] Sec. 4, Eq. 8;
 * App. D), plus the row impact factors of key-row-aware dual-axis fitting
 * ([SQ] Sec. 4.1, 4.3, App. C).  Host only.  Units with the largest
 * L_u d_u(b_max) become pivots (ceil(pivot_frac * U) of them, ties to the
 * lower index) and are charged 8 bits per element; every other unit starts
 * at the smallest width and the greedy repeatedly takes the affordable
 * upgrade to the next width with the largest L_u (d_u(b) - d_u(b+)) /
 * (n_u (b+ - b)) (ties to the lower index) until none fits the budget
 * b_bar * sum n_u.  L_u = sum_{j<horizon} exp(2 j ell_u).
 * Errors: SQ_EINVAL, SQ_EUNSUPPORTED, SQ_ENONFINITE, SQ_EBUDGET, SQ_ENOMEM. */
sq_status sq_calibrate_bits(const sq_calib_stats* stats, const sq_calib_opts* opts,
                            sq_plan** out);

/* STEP plan from an explicit allocation: unit_bits[n_units] in {2,4,6,8,16}
 * (16 = FP16 pivot unit), w[heads*d_k] > 0 row impact factors. */
sq_status sq_plan_create_step(int32_t kind, int32_t heads, int32_t d_k, int32_t d_v,
                              const int32_t* unit_bits, const float* w, sq_plan** out);

/* Uniform symmetric rowwise quantizer ([SQ] Sec. 5.1 baselines, App. B.5):
 * s_i = FP16(absmax_i / q_b), codes = nearest integer of X / s_i.
 * bits in {2,4,6,8}. */
sq_status sq_plan_create_uniform(int32_t heads, int32_t d_k, int32_t d_v, int32_t bits,
                                 sq_plan** out);

/* Per-window variant, GDN scalar gate ([LQ] Sec. 2.3, 2.5, 2.6): INT8 boundary
 * with key-row smoothing, float32 records, dense rebuild every p tokens.
 * 1 <= p <= 32; c_floor > 0 is the smoothing floor (1e-6 by default). */
sq_status sq_plan_create_window(int32_t heads, int32_t d_k, int32_t d_v, int32_t p,
                                float c_floor, sq_plan** out);

/* Per-window variant with compensator tokens ([LQ] Sec. 2.4-2.5, Eqs. 5-7
 * and 10): each head also keeps `rank` FP16 factor pairs (Kc[h], Uc[h]) that
 * join the boundary (S0 = C (Z/127) B + Kc^T Uc) with identity decay and then
 * decay with it; their readout term Uc (Kc Gamma x) rides with the records.
 * At every rebuild (a full window, sq_window_flush) and at pack the pairs
 * are refitted by power iteration on the dense state, one after another on
 * the residual left by the earlier ones: from b = the pair's stored Uc[h]
 * (the all-ones vector at pack, or when Uc[h] is zero), `power_iters` times
 * a = M b / |M b|, b = M^T a; then Kc[h] = FP16(sqrt|b| a),
 * Uc[h] = FP16(b / sqrt|b|), and M -= Kc[h] Uc[h]^T.  Only the residual is
 * smoothed and quantised.  1 <= p <= 32, 0 <= rank <= SQ_MAX_COMP_RANK
 * (rank 0 is sq_plan_create_window), 1 <= power_iters <= SQ_MAX_POWER_ITERS,
 * and p <= 16 unless d_v = 128; SQ_EUNSUPPORTED otherwise. */
sq_status sq_plan_create_window_lowrank(int32_t heads, int32_t d_k, int32_t d_v, int32_t p,
                                        float c_floor, int32_t rank, int32_t power_iters,
                                        sq_plan** out);

sq_status sq_plan_query(const sq_plan* plan, sq_plan_desc* desc);
sq_status sq_plan_destroy(sq_plan* plan);

/* Device copy of the plan's tables (head offsets, widths, impact factors,
 * KDA storage order).  The caller allocates sq_plan_device_bytes() bytes of
 * device memory (256-byte aligned) and keeps it alive while kernels use it;
 * sq_plan_upload copies the tables with an async host-to-device copy from
 * library-owned host memory. */
sq_status sq_plan_device_bytes(const sq_plan* plan, size_t* bytes);
sq_status sq_plan_upload(const sq_plan* plan, void* dev_plan, hipStream_t stream);

/* ----------------------------------------------------------------- pools */

/* Bytes of a pool of n_slots slots (n_slots * slot_bytes). */
sq_status sq_pool_bytes(const sq_plan* plan, int64_t n_slots, size_t* bytes);

/* Zero a whole pool (an all-zero slot is the zero state in every mode). */
sq_status sq_pool_init(const sq_plan* plan, const void* dev_plan, void* pool,
                       int64_t n_slots, hipStream_t stream);

/* Prefill boundary ([SQ] App. F.1: the boundary states of a prefill are
 * packed into the pool): quantise dense fp32 states S[B][H][d_k][d_v] with
 * the plan's quantizer (the same device code as the decode step) and store
 * them into the given slots.  Window mode stores the boundary with l = 0. */
sq_status sq_pool_pack(const sq_plan* plan, const void* dev_plan, void* pool,
                       int64_t n_slots, const int32_t* slots, int32_t batch,
                       const float* S, hipStream_t stream);

/* Dequantise the given slots into S_out[B][H][d_k][d_v] (fp32).  Window mode
 * returns the dense state of the open window, S_l = Gamma_{1:l} S0 +
 * sum_j Gamma_{j+1:l} Kt_j U_j^T ([LQ] Sec. 2.3, Eq. 4; S0 includes the
 * compensator pairs, Eq. 7). */
sq_status sq_pool_unpack(const sq_plan* plan, const void* dev_plan, const void* pool,
                         int64_t n_slots, const int32_t* slots, int32_t batch,
                         float* S_out, hipStream_t stream);

/* ------------------------------------------------------------ the step */

/* One fused decode step for `batch` live requests, in place on their slots.
 * Per (slot, head): reconstruct the packed tile, apply the gated delta rule
 *   X = D S + beta k (v - (D S)^T k)^T      ([SQ] Sec. 3, Eq. 1; D = alpha I
 *                                             for GDN, diag(d) for KDA),
 * read the head output from X before quantisation, y = X^T q ([SQ] App. A),
 * and store Q(X) ([SQ] Sec. 3, Eq. 4): uniform rowwise codes; or STEP
 * dual-axis codes with r_i = FP16(sqrt(m_i / w_i)), m_i = mean_j |X_ij|,
 * c0_j = FP16(max_i |X_ij| / r_i), z = nearest integer of
 * q_b X_ij / (r_i c0_j), and the fixed-code weighted least-squares column
 * refit c_j = FP16(sum_i w_i^2 r_i zt_ij X_ij / sum_i w_i^2 r_i^2 zt_ij^2),
 * zt = z / q_b ([SQ] Sec. 4.3, App. C), FP16 pivot units stored as
 * FP16(X).  Window mode appends the token's record (alpha, beta k, u) with
 * u = v - S^T (alpha k), emits o = S^T q from the windowed expansion and
 * rebuilds + requantises the boundary when the window holds p records
 * ([LQ] Sec. 2.3-2.6).
 *   q, k   : [B][H][d_k] fp32 (k L2-normalised for the method's guarantees)
 *   v      : [B][H][d_v] fp32
 *   beta   : [B][H] fp32 in [0, 1]
 *   gate   : GDN alpha [B][H]; KDA d [B][H][d_k]; values in [0, 1]
 *   y      : [B][H][d_v] fp32 output
 * Errors: SQ_EINVAL, SQ_EPLAN_MISMATCH, SQ_ESLOT_RANGE / SQ_EDUP_SLOT
 * (SQ_VALIDATE=1), SQ_EHIP. */
sq_status sq_decode_step(const sq_plan* plan, const void* dev_plan, void* pool,
                         int64_t n_slots, const int32_t* slots, int32_t batch,
                         const float* q, const float* k, const float* v,
                         const float* beta, const float* gate, float* y,
                         hipStream_t stream);

/* Window mode: rebuild and requantise the boundary of every given slot whose
 * heads hold 0 < l < p records (l = 0 heads are left untouched) ([LQ]
 * Sec. 2.6). */
sq_status sq_window_flush(const sq_plan* plan, const void* dev_plan, void* pool,
                          int64_t n_slots, const int32_t* slots, int32_t batch,
                          hipStream_t stream);

/* Test hook: run only the plan's quantizer on fp32 tiles X[n][d_k][d_v],
 * tile t using head head_ids[t]'s widths and factors, and write each packed
 * head (padded head bytes of that head) to packed_out at t * max_head_bytes,
 * max_head_bytes = the largest padded head size of the plan. */
sq_status sq_quantize_tiles(const sq_plan* plan, const void* dev_plan, const float* X,
                            int32_t n_tiles, const int32_t* head_ids, void* packed_out,
                            hipStream_t stream);
sq_status sq_max_head_bytes(const sq_plan* plan, size_t* bytes);

/* Prefill of one chunk ([SQ] App. F.1: a prefill unpacks the active states,
 * runs the chunk and packs the boundary states; with sq_pool_unpack before
 * and sq_pool_pack after, this is the middle step): T tokens of the
 * unquantised gated delta rule, X = D S + beta k (v - (D S)^T k)^T,
 * y = X^T q, S <- X ([SQ] Sec. 3, Eq. 1), for B sequences, in place on dense
 * fp32 states S[B][H][d_k][d_v] (device, caller-owned; the state stays in
 * registers for the whole chunk).  Inputs are sequence-major:
 * q, k [B][T][H][d_k], v [B][T][H][d_v], beta [B][T][H], gate GDN alpha
 * [B][T][H] or KDA d [B][T][H][d_k]; y [B][T][H][d_v] receives every token's
 * output.  This form runs the tokens one after another on the vector units;
 * sq_prefill_chunkwise below computes the same chunk in matrix form and is the
 * faster one (2.5-3.2x on 64-512 sequences of 16-48 heads at d = 128).
 * Errors: SQ_EINVAL (bad kind, negative or oversized batch or T, a null array
 * when batch and T are positive), SQ_EUNSUPPORTED (d_k or d_v not 64 or 128),
 * SQ_EHIP.  batch = 0 or T = 0 does nothing (the arrays may be null). */
sq_status sq_prefill_chunk(int32_t kind, int32_t heads, int32_t d_k, int32_t d_v,
                           int32_t batch, int32_t T, float* S, const float* q, const float* k,
                           const float* v, const float* beta, const float* gate, float* y,
                           hipStream_t stream);

/* The same chunk in matrix form ([SQ] App. F.1's chunk kernel; the
 * recurrence of [SQ] Sec. 3, Eq. 1 unrolled over blocks of 16 tokens): per
 * block, the decay products, the strictly lower A_ts = beta_t sum_c k_tc
 * G_tsc k_sc, the lower L_ts = sum_c q_tc G_tsc k_sc (G_ts = prod_{s<r<=t}
 * d_r) and T = (I+A)^-1; then U = T (diag(beta) V - diag(beta)(K o g) S),
 * Y = (Q o g) S + L U and S <- diag(g_end) S + (K o G_end)^T U on the fp32
 * matrix cores.  Same arguments, layouts, ownership and errors as
 * sq_prefill_chunk; the results equal it up to rounding order (no
 * intermediate leaves the chip: the workgroup of a (sequence, head) keeps
 * the state in registers and the block's intermediates in LDS). */
sq_status sq_prefill_chunkwise(int32_t kind, int32_t heads, int32_t d_k, int32_t d_v,
                               int32_t batch, int32_t T, float* S, const float* q, const float* k,
                               const float* v, const float* beta, const float* gate, float* y,
                               hipStream_t stream);

/* Full-precision reference step on fp32 states S[n_slots][H][d_k][d_v]
 * (the FP32-state baseline of [SQ] Sec. 5.1 and [LQ] Sec. 3.3):
 * X = D S + beta k (v - (D S)^T k)^T stored in place, y = X^T q.
 * kind = SQ_KIND_GDN (gate [B][H]) or SQ_KIND_KDA (gate [B][H][d_k]). */
sq_status sq_dense_step(int32_t kind, int32_t heads, int32_t d_k, int32_t d_v,
                        float* S, int64_t n_slots, const int32_t* slots, int32_t batch,
                        const float* q, const float* k, const float* v,
                        const float* beta, const float* gate, float* y,
                        hipStream_t stream);

const char* sq_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* STEPQ_H */
