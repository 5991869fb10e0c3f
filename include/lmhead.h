/*
 * lmhead.h - batch-invariant LM head for AMD Instinct MI355X (gfx950).
 *
 * The output projection of final hidden states against the vocabulary matrix,
 * followed by greedy top-2 (with the top-2 logit margin) or by the log-softmax
 * probability of a given token, in two arithmetic modes:
 *
 *   LMHEAD_MODE_BF16  bf16 hidden x bf16 vocab matrix, products accumulated in
 *                     float32 in one fixed order, float32 logits.
 *                     ("Greedy Decoding Has a Precision Clause", section
 *                     "Correct the vulnerable token decisions, not every
 *                     calculation": the final output projection recomputed in
 *                     FP32; "12 Exactness", section 12.2: the head returns
 *                     fp32 logits.)
 *   LMHEAD_MODE_INT8  int8 hidden x int8 vocab matrix, exact int32 logits.
 *                     ("Eliminating Nondeterminism in LLM Inference with
 *                     Integer-Only Arithmetic", sections "What if we don't use
 *                     floats at all?" and "DetLLM": int8 x int8 -> int32
 *                     matmul; integer sums are exact in any order.)
 *   LMHEAD_MODE_BF16_PACKED  LMHEAD_MODE_BF16 with w in the packed layout that
 *                     lmhead_pack_w writes.  Same arithmetic, same order: every
 *                     output has the bits it has in LMHEAD_MODE_BF16 with the
 *                     row-major w it was packed from.  Only where W is read
 *                     from differs; small batches run faster from it.
 *
 * Batch invariance.  Every logit is reduced over k in one order fixed by H
 * alone (one MFMA shape, one accumulator; k ascending in MODE_BF16, and in
 * MODE_INT8 from a start fixed by the column, which cannot change an exact
 * integer sum), never by the number of rows or a row's position in the batch;
 * the softmax partial sums are fixed by V alone.  A row's outputs are
 * therefore bitwise identical at every batch size.  ("12 Exactness", section
 * 12.2: the summation order of a product is a function of the weight's
 * dimensions alone, so the batch's row count cannot change it; "Integer-Only
 * Arithmetic", section "Why kernels don't always add in the same order":
 * split reductions chosen by batch size break batch invariance.)
 *
 * Layout.  x is [B, H] row-major, w is [V, H] row-major (each vocabulary row
 * contiguous in k), or packed (LMHEAD_MODE_BF16_PACKED, see lmhead_pack_w).
 * bf16 tensors are raw 16-bit patterns.  x, w and the
 * workspace must be 16-byte aligned, every other array aligned to its element
 * size.  All data pointers are DEVICE pointers owned by the caller; the
 * library never allocates, frees or synchronises, and keeps no pointer after a
 * call returns.  Every call is
 * asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 *
 * Errors.  Arguments are validated on the host, synchronously, before any work
 * is queued; on a validation error nothing is queued and the status says why.
 * A failed launch returns LMHEAD_E_HIP (lmhead_last_error() has the HIP
 * message).  The reducing calls (greedy, gated, sampling, log-prob) launch two
 * kernels, the tiled contraction and then the per-row fold; if the second
 * launch fails, the first may already be queued.  No exception or abort
 * crosses this interface.  Inputs are assumed finite.
 */
#ifndef LMHEAD_H_
#define LMHEAD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMHEAD_OK = 0,
  LMHEAD_E_NULL = 1,      /* a required pointer is NULL */
  LMHEAD_E_SHAPE = 2,     /* B < 1, V < 2, H not a positive multiple of 64, or too large:
                             B > 2^24, V > 2^30, H > 2^20, or B and V together beyond
                             one launch grid (2^32 threads; about B * V > 2^38) */
  LMHEAD_E_ALIGN = 3,     /* x, w or workspace not 16-byte aligned, or another array
                             not aligned to its element size */
  LMHEAD_E_MODE = 4,      /* unknown mode / rounding, or rounding not valid for the mode */
  LMHEAD_E_OVERFLOW = 5,  /* int8: H * 128^2 could exceed int32 (H > 131071) */
  LMHEAD_E_WORKSPACE = 6, /* workspace NULL or smaller than lmhead_workspace_bytes() */
  LMHEAD_E_HIP = 7,       /* the HIP runtime refused the launch */
  LMHEAD_E_VALUE = 8      /* a scalar argument is out of range (e.g. a NaN or negative tau) */
} lmhead_status;

typedef enum {
  LMHEAD_MODE_BF16 = 0,
  LMHEAD_MODE_INT8 = 1,
  LMHEAD_MODE_BF16_PACKED = 2
} lmhead_mode;

/* Rounding of the logits before they are stored or ranked.  LMHEAD_ROUND_BF16
 * is the ordinary 16-bit head (float32 accumulation, then round-to-nearest-even
 * to bf16), kept to compare decisions against the float32 head; it is valid
 * only in the bf16 modes.  ("Greedy Decoding Has a Precision Clause":
 * BF16-output head versus the FP32-recomputed head.) */
typedef enum { LMHEAD_ROUND_F32 = 0, LMHEAD_ROUND_BF16 = 1 } lmhead_round;

/* Bytes of device workspace lmhead_greedy_top2 / lmhead_logprob need for this
 * shape (0 if the shape is invalid).  Its contents on entry do not matter (no
 * clearing is needed); each call overwrites what it uses.  One workspace must
 * not be shared by two calls that can run at the same time. */
size_t lmhead_workspace_bytes(int mode, int64_t B, int64_t H, int64_t V);

/* Full logits.  logits[b, v] = sum_k x[b, k] * w[v, k], stored row-major [B, V]
 * as float32 (the bf16 modes, ROUND_F32), bf16 bits (the bf16 modes,
 * ROUND_BF16) or int32 (MODE_INT8, exact).  ("Greedy Decoding Has a Precision Clause", section
 * "Token-ranking margins explain why numerical error sometimes matters": the
 * lm_head turns the final representation into one score per token.) */
lmhead_status lmhead_logits(int mode, int round, const void *x, const void *w, int64_t B,
                            int64_t H, int64_t V, void *logits, void *stream);

/* Greedy decision per row, logits never written to memory.
 *   top_id[b, 0..1]  ids of the best and second-best logit; ties go to the
 *                    lowest token id ("Integer-Only Arithmetic", section
 *                    "DetLLM": argmax breaks ties toward the lowest token id);
 *                    an exactly tied maximum makes top_id[b,1] the next tied id.
 *   top_val[b, 0..1] their values: float32 logits (ROUND_BF16: the bf16-rounded
 *                    logits); MODE_INT8: float32(raw * row_scale[b]), one
 *                    rounding of the exact product.
 *   margin[b]        top-2 logit margin z(1) - z(2) >= 0 ("Greedy Decoding Has
 *                    a Precision Clause", section "Token-ranking margins": the
 *                    top-two logit margin); MODE_INT8: float32((raw1 - raw2) *
 *                    row_scale[b]).
 *   top_raw[b, 0..1] MODE_INT8 only, optional (NULL to skip): exact int32 logits.
 *   row_scale[b]     MODE_INT8 only, optional (NULL = 1): per-row positive
 *                    float32 scale applied after the integer argmax; a
 *                    non-positive or non-finite scale makes that row's values
 *                    and margin NaN (ids and raw values stay exact).
 * ws / ws_bytes: device workspace, see lmhead_workspace_bytes. */
lmhead_status lmhead_greedy_top2(int mode, int round, const void *x, const void *w, int64_t B,
                                 int64_t H, int64_t V, const float *row_scale, int32_t *top_id,
                                 float *top_val, float *margin, int32_t *top_raw, void *ws,
                                 size_t ws_bytes, void *stream);

/* lmhead_greedy_top2 for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, outputs and kernels, with the workspace taken from a
 * static device array of LMHEAD_STATIC_WORKSPACE_BYTES in the library (one per
 * GPU, resolved on the first call on that device and held until the process
 * ends).  Shapes whose workspace exceeds it (lmhead_workspace_bytes() >
 * LMHEAD_STATIC_WORKSPACE_BYTES, e.g. B * ceil(V / 128) above about a million
 * records) give LMHEAD_E_WORKSPACE.  Nothing is allocated.  Every call on one
 * GPU shares that array: calls that can overlap on one GPU (concurrent
 * streams, several host threads) race and must not be issued. */
#define LMHEAD_STATIC_WORKSPACE_BYTES ((size_t)16 << 20)
lmhead_status lmhead_greedy_top2_noalloc(int mode, int round, const void *x, const void *w,
                                         int64_t B, int64_t H, int64_t V, const float *row_scale,
                                         int32_t *top_id, float *top_val, float *margin,
                                         int32_t *top_raw, void *stream);

/* log p(target[b]) under the softmax (temperature 1) of row b's logits, float32,
 * logits never written to memory ("batch-logprob-gap": the log probability a
 * model gives a token; "Inference and Decoding", section 3, temperature
 * softmax).  MODE_INT8 uses the scaled logits row_scale[b] * z (NULL = 1).  A
 * target outside [0, V) or an invalid scale gives NaN for that row. */
lmhead_status lmhead_logprob(int mode, const void *x, const void *w, int64_t B, int64_t H,
                             int64_t V, const float *row_scale, const int32_t *target,
                             float *logprob, void *ws, size_t ws_bytes, void *stream);

/* Margin-gated float32 recompute of the greedy decision ("Greedy Decoding Has
 * a Precision Clause", section "Correct the vulnerable token decisions, not
 * every calculation": ordinary inference decides unless the top-2 logit margin
 * is below a calibrated threshold; such steps recompute the output projection
 * in FP32, and recomputing the two leading candidates sufficed).  The bf16
 * modes only (LMHEAD_E_MODE otherwise).
 *   1. greedy top-2 of the bf16-output head, exactly as lmhead_greedy_top2 with
 *      LMHEAD_ROUND_BF16 (ids, bf16-rounded values, margin);
 *   2. every row whose margin is below tau recomputes the logits of its two
 *      candidates with the float32 head (bitwise the values lmhead_logits gives
 *      them: same MFMA instruction and k order) and re-ranks them, lowest id on
 *      a tie; top_val and margin of that row then hold float32 logits.
 *   gated[b] = 1 for a recomputed row, 0 otherwise.
 * Step 2 runs inside the fold of step 1 (no extra launch).
 * tau >= 0 (0 recomputes nothing, +inf every row); NaN or negative tau gives
 * LMHEAD_E_VALUE.  ws / ws_bytes as for lmhead_greedy_top2. */
lmhead_status lmhead_greedy_gated(int mode, const void *x, const void *w, int64_t B, int64_t H,
                                  int64_t V, float tau, int32_t *top_id, float *top_val,
                                  float *margin, int32_t *gated, void *ws, size_t ws_bytes,
                                  void *stream);

/* Seeded Gumbel-max sampling ("12 Exactness", section 12.5: adding Gumbel
 * noise, drawn from a generator keyed by the seed and the position, to every
 * token's log-probability and taking the largest sum is an exact draw from
 * the distribution).  Since log p_t differs from
 * z / T by a constant per row:
 *   token[b] = argmax_v ( z[b, v] / temperature + G(seed[b], position[b], v) ),
 *              the lowest id on a tie;
 *   G(s, t, v) = -ln(-ln U), U = (2u + 1) 2^-24, u the top 23 bits of word
 *              (v >> 5) & 3 of Philox4x32-10 (Salmon et al., SC 2011) at counter
 *              (32 (v >> 7) + (v & 31), 0, t mod 2^32, t div 2^32) under key
 *              (s mod 2^32, s div 2^32), t taken as an unsigned 64-bit value.
 * A row's draw depends on its own (seed, position) and logits only, never on
 * the batch.  value[b] (optional) = the winning score, gap[b] (optional) = its
 * lead over the runner-up (small gaps are where float32 rounding could pick
 * the other token).  MODE_INT8 uses the scaled logits row_scale[b] * z (NULL =
 * 1); a non-positive or non-finite scale draws token -1 with NaN value and gap.
 * temperature must be positive and finite (LMHEAD_E_VALUE otherwise).  seed and
 * position: device arrays of B, 8-byte aligned.  ws / ws_bytes as for
 * lmhead_greedy_top2. */
lmhead_status lmhead_sample_gumbel(int mode, const void *x, const void *w, int64_t B, int64_t H,
                                   int64_t V, float temperature, const float *row_scale,
                                   const uint64_t *seed, const int64_t *position, int32_t *token,
                                   float *value, float *gap, void *ws, size_t ws_bytes,
                                   void *stream);

/* The all-integer front and back of the int8 head ("Eliminating Nondeterminism
 * in LLM Inference with Integer-Only Arithmetic", section "DetLLM": every
 * tensor carries a dyadic scale m / 2^k, rescaled by an integer multiply and a
 * shift with one fixed rounding rule; exp and softmax are integer algorithms;
 * each token's activations are quantised from that token's own values, so its
 * bits cannot depend on the batch).  The pages give no algorithm; this one
 * rounds every rescale half up.
 *
 * lmhead_quantize_rows: per-token int8 quantisation of int32 rows x[B, H]
 * (row-major, any H >= 1).  For row b, a = max |x|; the step D = M 2^E is the
 * least number with a 15-bit mantissa (2^14 <= M < 2^15) such that 127 D >= a;
 * q[b, k] = sign(x) floor(|x| / D + 1/2), so |q| <= 127 and the largest |x|
 * maps to 127.  A zero row gives q = 0, M = 2^14, E = -14 (D = 1).  Outputs
 * q[B, H] int8, step_m[B], step_e[B] int32; x, step_m, step_e 4-byte aligned.
 *
 * lmhead_logprob_int: log p(target[b]) in fixed point Q.24 (int64, units of
 * 2^-24 nats) from the exact int32 logits z = x w^T of int8 x[B, H], w[V, H].
 * Row b's real logits are z * unit * D_b with the tensor unit um 2^ue (the real
 * value of one unit of the hidden input times one unit of w) and the row step
 * D_b = step_m[b] 2^step_e[b] (as lmhead_quantize_rows gives it).  The scale
 * is taken as m / 2^k, the mantissa product rounded to 31 bits, valid when
 * 24 <= k <= 86.  With T(d) = round(d m / 2^(k - 24)) (Q.24 nats):
 *   exp   e(T) = e^(-T / 2^24) in Q.30: T = q L + r with L = round(ln 2 2^24),
 *         e^(-r) by its Taylor series to degree 10 (coefficients
 *         round(2^30 / n!), Horner form), then times 2^-q;
 *   sum   per block of 128 columns (fixed by V): m_c = max z, S_c = sum of
 *         e(T(m_c - z)); S = sum over blocks of round(S_c e(T(z_max - m_c)) /
 *         2^30), every sum exact;
 *   ln    ln(S / 2^30) in Q.30 by 2 atanh(f / (2 + f)) on the 30-bit mantissa
 *         1 + f of S, plus the exponent times round(ln 2 2^30);
 *   out   logprob_q[b] = -(T(z_max - z_target) + round(ln / 2^6)).
 * Integer arithmetic only, so the result is the same on every device.  A
 * target outside [0, V) or a row scale that is not valid gives INT64_MIN.
 * The error against the exact log-softmax of the real logits is a few units of
 * 2^-24 plus 3 V 2^-30 relative to the sum of exps.  unit_m must be positive
 * (LMHEAD_E_VALUE otherwise).  ws / ws_bytes as for lmhead_greedy_top2 with
 * MODE_INT8.  logprob_q 8-byte aligned. */
lmhead_status lmhead_quantize_rows(const int32_t *x, int64_t B, int64_t H, int8_t *q,
                                   int32_t *step_m, int32_t *step_e, void *stream);
lmhead_status lmhead_logprob_int(const void *x, const void *w, int64_t B, int64_t H, int64_t V,
                                 int32_t unit_m, int32_t unit_e, const int32_t *step_m,
                                 const int32_t *step_e, const int32_t *target,
                                 int64_t *logprob_q, void *ws, size_t ws_bytes, void *stream);

/* Device self-check of the row property ("12 Exactness", section 12.8: a
 * load-time self-check proves on the device that every row gets the same bits
 * whatever the number of rows).  Computes the logits of x[0..B) as one batch,
 * of every row alone, and of the rows in reverse order, and adds the number of
 * logits whose bits differ to *mismatches (a device uint64 the caller zeroes,
 * 8-byte aligned; LMHEAD_E_ALIGN otherwise).  scratch: device memory of
 * lmhead_self_check_bytes() bytes, 16-byte aligned; it is overwritten. */
size_t lmhead_self_check_bytes(int mode, int64_t B, int64_t H, int64_t V);
lmhead_status lmhead_self_check(int mode, const void *x, const void *w, int64_t B, int64_t H,
                                int64_t V, void *scratch, size_t scratch_bytes,
                                uint64_t *mismatches, void *stream);

/* The packed layout of a bf16 vocabulary matrix, for LMHEAD_MODE_BF16_PACKED.
 * A weight is packed once and then read by every call; packing changes where
 * each byte sits, not any value or the order of any sum.  W is cut into blocks
 * of 128 rows x 128 bytes; each block is stored row by row (16 KB, contiguous),
 * the blocks of a group of 128 rows one after another in k order followed by
 * one unused 16 KB block (zeros), and the groups in order.  With R = 2 H bytes
 * per row, byte k of vocabulary row v is at byte
 *     (v / 128) * (128 R + 16384) + (k / 128) * 16384 + (v % 128) * 128 + k % 128
 * (integer division), so the contraction's pipeline stages read contiguous
 * blocks, and the unused block keeps the groups from all starting at one
 * offset modulo a large power of two.  The layout has ceil(V / 128) groups,
 * ceil(V / 128) * (128 R + 16384) bytes; the rows from V on are zero.  (The
 * pages fix the arithmetic, not the storage of the weight; this layout is
 * this library's own.)
 *   lmhead_packed_w_bytes  its size in bytes (0 if H or V is not valid);
 *   lmhead_pack_w          writes it from row-major bf16 w [V, H] into
 *                          `packed` (device, 16-byte aligned, at least
 *                          lmhead_packed_w_bytes(H, V) bytes, not overlapping
 *                          w: LMHEAD_E_VALUE if the two ranges meet),
 *                          asynchronously on `stream`.
 * Shape rules and errors as for the other calls with B = 1. */
size_t lmhead_packed_w_bytes(int64_t H, int64_t V);
lmhead_status lmhead_pack_w(const void *w, int64_t H, int64_t V, void *packed, void *stream);

/* Text of a status code, and of the last HIP error seen by this thread. */
const char *lmhead_status_string(int status);
const char *lmhead_last_error(void);

/* The first 16 hex digits of the SHA-256 of the sources this library was built
 * from (a static string), so a caller can refuse a library built from other
 * sources. */
const char *lmhead_source_digest(void);

#ifdef __cplusplus
}
#endif
#endif /* LMHEAD_H_ */
