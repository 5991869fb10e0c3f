// C-ABI of the batch-invariant LM head (declared in include/lmhead.h).
//
// Everything here runs on the host: argument validation (synchronous, before
// anything is queued), workspace layout, choice of the grid tiling and the
// kernel launch on the caller's stream.  No allocation, no synchronisation.
#include "lmhead.h"

#include <hip/hip_runtime_api.h>
#include <stdio.h>
#include <string.h>

#include "lmhead_internal.h"

namespace {

#ifndef LMH_SOURCE_DIGEST
#error "the build passes the sources' digest as LMH_SOURCE_DIGEST"
#endif

thread_local char g_last_error[256] = "no HIP error";

constexpr int64_t kMaxRows = (int64_t)1 << 24;   // B bound (int indexing of rows)
constexpr int64_t kMaxVocab = (int64_t)1 << 30;  // V bound
constexpr int64_t kMaxHidden = (int64_t)1 << 20; // H bound
constexpr int64_t kInt8MaxHidden = 131071;       // H * 128^2 < 2^31

// the kernels' arithmetic (0 float head, 1 int8 head) and W's layout of a mode
int arith_of(int mode) { return mode == LMHEAD_MODE_INT8 ? 1 : 0; }
bool packed_of(int mode) { return mode == LMHEAD_MODE_BF16_PACKED; }
int64_t row_bytes(int mode, int64_t H) { return mode == LMHEAD_MODE_INT8 ? H : 2 * H; }
lmh::Plan plan_of(int mode, int64_t B, int64_t H, int64_t V) {
  return lmh::plan_for(arith_of(mode), B, row_bytes(mode, H), V, packed_of(mode));
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

lmhead_status check_common(int mode, int round, const void *x, const void *w, int64_t B,
                           int64_t H, int64_t V) {
  if (mode != LMHEAD_MODE_BF16 && mode != LMHEAD_MODE_INT8 && mode != LMHEAD_MODE_BF16_PACKED)
    return LMHEAD_E_MODE;
  if (round != LMHEAD_ROUND_F32 && round != LMHEAD_ROUND_BF16) return LMHEAD_E_MODE;
  if (mode == LMHEAD_MODE_INT8 && round != LMHEAD_ROUND_F32) return LMHEAD_E_MODE;
  if (!x || !w) return LMHEAD_E_NULL;
  if (B < 1 || B > kMaxRows || V < 2 || V > kMaxVocab || H < 64 || H % 64 != 0 ||
      H > kMaxHidden)
    return LMHEAD_E_SHAPE;
  if (mode == LMHEAD_MODE_INT8 && H > kInt8MaxHidden) return LMHEAD_E_OVERFLOW;
  // the tile grid is one x dimension of at most 2^32 - 1 threads (256 or 512
  // per workgroup, by plan), which bounds B x V jointly
  const lmh::Plan pl = plan_of(mode, B, H, V);
  if ((uint64_t)pl.grid_m * (uint64_t)pl.grid_n * (uint64_t)pl.nt > 0xFFFFFFFFull)
    return LMHEAD_E_SHAPE;
  if (!aligned16(x) || !aligned16(w)) return LMHEAD_E_ALIGN;
  return LMHEAD_OK;
}

lmhead_status launched(hipError_t e) {
  if (e == hipSuccess) return LMHEAD_OK;
  snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
  return LMHEAD_E_HIP;
}

lmh::Params base_params(int mode, const void *x, const void *w, int64_t B, int64_t H, int64_t V,
                        const lmh::Plan &plan) {
  lmh::Params p;
  memset(&p, 0, sizeof p);
  p.x = (const char *)x;
  p.w = (const char *)w;
  p.rowbytes = row_bytes(mode, H);
  p.w_packed = packed_of(mode) ? 1 : 0;
  p.B = (int)B;
  p.V = (int)V;
  p.nblocks = (int)((V + lmh::kBlockCols - 1) / lmh::kBlockCols);
  p.grid_m = plan.grid_m;
  p.grid_n = plan.grid_n;
  p.div_group = lmh::div_magic((uint64_t)lmh::kTileGroup * (uint64_t)plan.grid_n);
  p.div_units = lmh::div_magic(p.rowbytes >= 256 ? (uint64_t)(p.rowbytes >> 8) : 1);
  return p;
}

}  // namespace

namespace lmh {
size_t workspace_layout(int64_t B, int64_t V, size_t *off_zt, size_t *off_records) {
  auto up = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const size_t zt = up(sizeof(int32_t) * (size_t)B);
  const size_t nblocks = (size_t)((V + kBlockCols - 1) / kBlockCols);
  const size_t records = 16 * (size_t)B * nblocks;
  if (off_zt) *off_zt = 0;
  if (off_records) *off_records = zt;
  return zt + records;
}
}  // namespace lmh

extern "C" {

size_t lmhead_workspace_bytes(int mode, int64_t B, int64_t H, int64_t V) {
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  if (check_common(mode, LMHEAD_ROUND_F32, dummy, dummy, B, H, V) != LMHEAD_OK) return 0;
  return lmh::workspace_layout(B, V, nullptr, nullptr);
}

lmhead_status lmhead_logits(int mode, int round, const void *x, const void *w, int64_t B,
                            int64_t H, int64_t V, void *logits, void *stream) {
  lmhead_status st = check_common(mode, round, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (!logits) return LMHEAD_E_NULL;
  if (((uintptr_t)logits & (round == LMHEAD_ROUND_BF16 ? 1u : 3u)) != 0) return LMHEAD_E_ALIGN;
  const lmh::Plan plan = plan_of(mode, B, H, V);
  lmh::Params p = base_params(mode, x, w, B, H, V, plan);
  p.round_bf16 = round == LMHEAD_ROUND_BF16;
  p.logits = logits;
  return launched(lmh::launch(arith_of(mode), lmh::kStore, plan, p, (hipStream_t)stream));
}

static lmhead_status bind_workspace(lmh::Params &p, void *ws, size_t ws_bytes, int64_t B,
                                    int64_t V) {
  size_t off_zt, off_rec;
  const size_t need = lmh::workspace_layout(B, V, &off_zt, &off_rec);
  if (!ws || ws_bytes < need) return LMHEAD_E_WORKSPACE;
  if (!aligned16(ws)) return LMHEAD_E_ALIGN;
  p.zt = (int32_t *)((char *)ws + off_zt);
  p.records = (uint4 *)((char *)ws + off_rec);
  return LMHEAD_OK;
}

namespace {
// greedy top-2; with gated != null (bf16-output head only) the fold re-ranks
// rows whose margin is below tau on their candidates' float32-head logits
lmhead_status greedy(int mode, int round, const void *x, const void *w, int64_t B, int64_t H,
                     int64_t V, const float *row_scale, int32_t *top_id, float *top_val,
                     float *margin, int32_t *top_raw, float tau, int32_t *gated, void *ws,
                     size_t ws_bytes, void *stream) {
  lmhead_status st = check_common(mode, round, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (!top_id || !top_val || !margin) return LMHEAD_E_NULL;
  if (!aligned4(top_id) || !aligned4(top_val) || !aligned4(margin) ||
      (top_raw && !aligned4(top_raw)) || (row_scale && !aligned4(row_scale)))
    return LMHEAD_E_ALIGN;
  const lmh::Plan plan = plan_of(mode, B, H, V);
  lmh::Params p = base_params(mode, x, w, B, H, V, plan);
  st = bind_workspace(p, ws, ws_bytes, B, V);
  if (st != LMHEAD_OK) return st;
  p.round_bf16 = round == LMHEAD_ROUND_BF16;
  p.scale = mode == LMHEAD_MODE_INT8 ? row_scale : nullptr;
  p.top_id = top_id;
  p.top_val = top_val;
  p.margin = margin;
  p.top_raw = mode == LMHEAD_MODE_INT8 ? top_raw : nullptr;
  p.tau = tau;
  p.gated = gated;
  return launched(lmh::launch(arith_of(mode), lmh::kTop2, plan, p, (hipStream_t)stream));
}
}  // namespace

lmhead_status lmhead_greedy_top2(int mode, int round, const void *x, const void *w, int64_t B,
                                 int64_t H, int64_t V, const float *row_scale, int32_t *top_id,
                                 float *top_val, float *margin, int32_t *top_raw, void *ws,
                                 size_t ws_bytes, void *stream) {
  return greedy(mode, round, x, w, B, H, V, row_scale, top_id, top_val, margin, top_raw, 0.0f,
                nullptr, ws, ws_bytes, stream);
}

lmhead_status lmhead_greedy_top2_noalloc(int mode, int round, const void *x, const void *w,
                                         int64_t B, int64_t H, int64_t V, const float *row_scale,
                                         int32_t *top_id, float *top_val, float *margin,
                                         int32_t *top_raw, void *stream) {
  static_assert(LMHEAD_STATIC_WORKSPACE_BYTES == lmh::kStaticWorkspaceBytes, "static workspace");
  lmhead_status st = check_common(mode, round, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (lmh::workspace_layout(B, V, nullptr, nullptr) > lmh::kStaticWorkspaceBytes)
    return LMHEAD_E_WORKSPACE;
  void *ws = nullptr;
  if ((st = launched(lmh::static_workspace(&ws))) != LMHEAD_OK) return st;
  return greedy(mode, round, x, w, B, H, V, row_scale, top_id, top_val, margin, top_raw, 0.0f,
                nullptr, ws, lmh::kStaticWorkspaceBytes, stream);
}

lmhead_status lmhead_logprob(int mode, const void *x, const void *w, int64_t B, int64_t H,
                             int64_t V, const float *row_scale, const int32_t *target,
                             float *logprob, void *ws, size_t ws_bytes, void *stream) {
  lmhead_status st = check_common(mode, LMHEAD_ROUND_F32, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (!target || !logprob) return LMHEAD_E_NULL;
  if (!aligned4(target) || !aligned4(logprob) || (row_scale && !aligned4(row_scale)))
    return LMHEAD_E_ALIGN;
  const lmh::Plan plan = plan_of(mode, B, H, V);
  lmh::Params p = base_params(mode, x, w, B, H, V, plan);
  st = bind_workspace(p, ws, ws_bytes, B, V);
  if (st != LMHEAD_OK) return st;
  p.scale = mode == LMHEAD_MODE_INT8 ? row_scale : nullptr;
  p.target = target;
  p.logprob = logprob;
  return launched(lmh::launch(arith_of(mode), lmh::kLse, plan, p, (hipStream_t)stream));
}

lmhead_status lmhead_quantize_rows(const int32_t *x, int64_t B, int64_t H, int8_t *q,
                                   int32_t *step_m, int32_t *step_e, void *stream) {
  if (!x || !q || !step_m || !step_e) return LMHEAD_E_NULL;
  if (B < 1 || H < 1 || B > kMaxRows || H > kMaxHidden) return LMHEAD_E_SHAPE;
  if (!aligned4(x) || !aligned4(step_m) || !aligned4(step_e)) return LMHEAD_E_ALIGN;
  return launched(lmh::launch_quantize(x, B, H, q, step_m, step_e, (hipStream_t)stream));
}

lmhead_status lmhead_logprob_int(const void *x, const void *w, int64_t B, int64_t H, int64_t V,
                                 int32_t unit_m, int32_t unit_e, const int32_t *step_m,
                                 const int32_t *step_e, const int32_t *target,
                                 int64_t *logprob_q, void *ws, size_t ws_bytes, void *stream) {
  const int mode = LMHEAD_MODE_INT8;
  lmhead_status st = check_common(mode, LMHEAD_ROUND_F32, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (!step_m || !step_e || !target || !logprob_q) return LMHEAD_E_NULL;
  if (!aligned4(step_m) || !aligned4(step_e) || !aligned4(target) ||
      ((uintptr_t)logprob_q & 7) != 0)
    return LMHEAD_E_ALIGN;
  if (unit_m <= 0) return LMHEAD_E_VALUE;
  const lmh::Plan plan = plan_of(mode, B, H, V);
  lmh::Params p = base_params(mode, x, w, B, H, V, plan);
  st = bind_workspace(p, ws, ws_bytes, B, V);
  if (st != LMHEAD_OK) return st;
  p.target = target;
  p.unit_m = unit_m;
  p.unit_e = unit_e;
  p.step_m = step_m;
  p.step_e = step_e;
  p.logprob_q = logprob_q;
  return launched(lmh::launch(arith_of(mode), lmh::kLseInt, plan, p, (hipStream_t)stream));
}

lmhead_status lmhead_greedy_gated(int mode, const void *x, const void *w, int64_t B, int64_t H,
                                  int64_t V, float tau, int32_t *top_id, float *top_val,
                                  float *margin, int32_t *gated, void *ws, size_t ws_bytes,
                                  void *stream) {
  lmhead_status st = check_common(mode, LMHEAD_ROUND_BF16, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (!gated) return LMHEAD_E_NULL;
  if (!aligned4(gated)) return LMHEAD_E_ALIGN;
  if (!(tau >= 0.0f)) return LMHEAD_E_VALUE;  // NaN or negative
  return greedy(mode, LMHEAD_ROUND_BF16, x, w, B, H, V, nullptr, top_id, top_val, margin,
                nullptr, tau, gated, ws, ws_bytes, stream);
}

lmhead_status lmhead_sample_gumbel(int mode, const void *x, const void *w, int64_t B, int64_t H,
                                   int64_t V, float temperature, const float *row_scale,
                                   const uint64_t *seed, const int64_t *position, int32_t *token,
                                   float *value, float *gap, void *ws, size_t ws_bytes,
                                   void *stream) {
  lmhead_status st = check_common(mode, LMHEAD_ROUND_F32, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (!seed || !position || !token) return LMHEAD_E_NULL;
  if (((uintptr_t)seed & 7u) || ((uintptr_t)position & 7u) || !aligned4(token) ||
      (value && !aligned4(value)) || (gap && !aligned4(gap)) ||
      (row_scale && !aligned4(row_scale)))
    return LMHEAD_E_ALIGN;
  if (!(temperature > 0.0f) || !(temperature <= 3.4e38f)) return LMHEAD_E_VALUE;
  const lmh::Plan plan = plan_of(mode, B, H, V);
  lmh::Params p = base_params(mode, x, w, B, H, V, plan);
  st = bind_workspace(p, ws, ws_bytes, B, V);
  if (st != LMHEAD_OK) return st;
  p.scale = mode == LMHEAD_MODE_INT8 ? row_scale : nullptr;
  p.inv_t = 1.0f / temperature;
  p.seed = seed;
  p.position = position;
  p.token = token;
  p.value = value;
  p.gap = gap;
  return launched(lmh::launch(arith_of(mode), lmh::kSample, plan, p, (hipStream_t)stream));
}

// scratch: [B, V] batch logits | [V] one-row logits | [B, V] reversed-batch logits |
//          [B, H] reversed rows; every region 256-byte aligned
static size_t self_check_layout(int mode, int64_t B, int64_t H, int64_t V, size_t off[4]) {
  auto up = [](size_t n) { return (n + 255) & ~(size_t)255; };
  const size_t lb = up(4 * (size_t)B * (size_t)V), l1 = up(4 * (size_t)V);
  off[0] = 0;
  off[1] = lb;
  off[2] = lb + l1;
  off[3] = lb + l1 + lb;
  return off[3] + up((size_t)B * (size_t)row_bytes(mode, H));
}

size_t lmhead_self_check_bytes(int mode, int64_t B, int64_t H, int64_t V) {
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  if (check_common(mode, LMHEAD_ROUND_F32, dummy, dummy, B, H, V) != LMHEAD_OK) return 0;
  size_t off[4];
  return self_check_layout(mode, B, H, V, off);
}

lmhead_status lmhead_self_check(int mode, const void *x, const void *w, int64_t B, int64_t H,
                                int64_t V, void *scratch, size_t scratch_bytes,
                                uint64_t *mismatches, void *stream) {
  lmhead_status st = check_common(mode, LMHEAD_ROUND_F32, x, w, B, H, V);
  if (st != LMHEAD_OK) return st;
  if (!scratch || !mismatches) return LMHEAD_E_NULL;
  size_t off[4];
  if (scratch_bytes < self_check_layout(mode, B, H, V, off)) return LMHEAD_E_WORKSPACE;
  if (!aligned16(scratch) || ((uintptr_t)mismatches & 7u) != 0) return LMHEAD_E_ALIGN;
  char *sc = (char *)scratch;
  hipStream_t s = (hipStream_t)stream;
  const int64_t rb = row_bytes(mode, H);
  unsigned long long *mm = (unsigned long long *)mismatches;
  // the whole batch
  if ((st = lmhead_logits(mode, LMHEAD_ROUND_F32, x, w, B, H, V, sc + off[0], stream)))
    return st;
  // every row alone, compared with its row of the batch
  for (int64_t r = 0; r < B; ++r) {
    if ((st = lmhead_logits(mode, LMHEAD_ROUND_F32, (const char *)x + r * rb, w, 1, H, V,
                            sc + off[1], stream)))
      return st;
    if ((st = launched(lmh::launch_compare(sc + off[0] + 4 * r * V, sc + off[1], V, mm, s))))
      return st;
  }
  // the rows in reverse order (every row at another position, other neighbours)
  if ((st = launched(lmh::launch_reverse_rows(x, sc + off[3], B, rb, s)))) return st;
  if ((st = lmhead_logits(mode, LMHEAD_ROUND_F32, sc + off[3], w, B, H, V, sc + off[2], stream)))
    return st;
  for (int64_t r = 0; r < B; ++r)
    if ((st = launched(lmh::launch_compare(sc + off[0] + 4 * r * V,
                                           sc + off[2] + 4 * (B - 1 - r) * V, V, mm, s))))
      return st;
  return LMHEAD_OK;
}

size_t lmhead_packed_w_bytes(int64_t H, int64_t V) {
  static const char dummy[16] __attribute__((aligned(16))) = {0};
  if (check_common(LMHEAD_MODE_BF16_PACKED, LMHEAD_ROUND_F32, dummy, dummy, 1, H, V) != LMHEAD_OK)
    return 0;
  return (size_t)((V + lmh::kPackRows - 1) / lmh::kPackRows) *
         (size_t)lmh::packed_group_bytes(row_bytes(LMHEAD_MODE_BF16_PACKED, H));
}

lmhead_status lmhead_pack_w(const void *w, int64_t H, int64_t V, void *packed, void *stream) {
  lmhead_status st = check_common(LMHEAD_MODE_BF16_PACKED, LMHEAD_ROUND_F32, w, w, 1, H, V);
  if (st != LMHEAD_OK) return st;
  if (!packed) return LMHEAD_E_NULL;
  if (!aligned16(packed)) return LMHEAD_E_ALIGN;
  // the layout is written while w is read: the two ranges must not meet
  const uintptr_t w0 = (uintptr_t)w, w1 = w0 + (uintptr_t)V * (uintptr_t)row_bytes(LMHEAD_MODE_BF16_PACKED, H);
  const uintptr_t p0 = (uintptr_t)packed, p1 = p0 + (uintptr_t)lmhead_packed_w_bytes(H, V);
  if (p0 < w1 && w0 < p1) return LMHEAD_E_VALUE;
  return launched(lmh::launch_pack_w(w, packed, V, row_bytes(LMHEAD_MODE_BF16_PACKED, H),
                                     (hipStream_t)stream));
}

const char *lmhead_status_string(int status) {
  switch (status) {
    case LMHEAD_OK: return "ok";
    case LMHEAD_E_NULL: return "a required pointer is NULL";
    case LMHEAD_E_SHAPE:
      return "invalid shape (need B >= 1, V >= 2, H a positive multiple of 64, sizes within bounds)";
    case LMHEAD_E_ALIGN: return "a pointer is not aligned as required";
    case LMHEAD_E_MODE: return "unknown mode or rounding, or rounding not valid for the mode";
    case LMHEAD_E_OVERFLOW: return "int8 head: H too large for exact int32 accumulation";
    case LMHEAD_E_WORKSPACE: return "workspace missing or too small";
    case LMHEAD_E_HIP: return "HIP launch failed (see lmhead_last_error)";
    case LMHEAD_E_VALUE: return "a scalar argument is out of range";
    default: return "unknown status";
  }
}

const char *lmhead_last_error(void) { return g_last_error; }

const char *lmhead_source_digest(void) { return LMH_SOURCE_DIGEST; }

}  // extern "C"
