// Internal interface between the C-ABI layer (lmhead_abi.cpp) and the gfx950
// kernels (lmhead_kernels.hip, lmhead_tiles.hip).  Not installed; not part of the public ABI.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace lmh {

enum Epilogue { kStore = 0, kTop2 = 1, kLse = 2, kSample = 3, kLseInt = 4 };

// Softmax partial sums and top-2 partial records are kept per block of 128
// vocabulary columns; the block grid depends on V only.
constexpr int kBlockCols = 128;

// The packed layout of a bf16 vocabulary matrix (lmhead_pack_w): W cut into
// blocks of kPackRows rows x kPackBytes bytes, each block contiguous (row by
// row), the blocks of a row group in k order, then one unused block (zeros),
// row groups in order.  A pipeline stage of a 128-row tile (128 bytes of each
// row, or a multiple) then reads whole contiguous 16 KB blocks instead of 128
// pieces a row apart.  The unused block staggers the groups: without it every
// group starts on a multiple of 128 * rowbytes (512 KB at H = 2048), so the
// stage that all workgroups read at once sits at one offset modulo that power
// of two in every group; with it, greedy calls from this layout measured
// 0.8-0.9 us faster at batches 1 and 8 and no slower at 256 and 512.  Rows from V
// up to the group's end are zero.
constexpr int kPackRows = 128, kPackBytes = 128;
constexpr int kPackBlock = kPackRows * kPackBytes;  // bytes of one block (16 KB)
// bytes from one row group to the next: its rowbytes / kPackBytes blocks and
// the unused one
__host__ __device__ inline int64_t packed_group_bytes(int64_t rowbytes) {
  return kPackRows * rowbytes + kPackBlock;
}
// byte offset of byte kb of row `row` (row-major: row * rowbytes + kb)
__host__ __device__ inline int64_t w_packed_offset(int64_t row, int64_t kb, int64_t rowbytes) {
  return (row / kPackRows) * packed_group_bytes(rowbytes) + (kb / kPackBytes) * kPackBlock +
         (row % kPackRows) * kPackBytes + kb % kPackBytes;
}

// m = ceil(2^63 / d) for an exact division of n < 2^31 by 1 <= d <= 2^31 with
// a multiply-high (div_exact in lmhead_device.h)
constexpr uint64_t div_magic(uint64_t d) { return ((uint64_t)1 << 63) / d + (((uint64_t)1 << 63) % d != 0); }

// Workgroups per group of the tile raster: kTileGroup row tiles are walked per
// vocabulary tile.
constexpr int kTileGroup = 8;

struct Params {
  const char *x;      // [B, H] row-major (bf16 bits or int8)
  const char *w;      // [V, H] row-major
  int64_t rowbytes;   // H * element size
  int B, V, nblocks;  // nblocks = ceil(V / kBlockCols)
  int grid_m, grid_n; // workgroup tiles over rows and vocabulary columns
  uint64_t div_group; // div_magic(kTileGroup * grid_n)
  uint64_t div_units; // div_magic(rowbytes / 256) (int8 k rotation; 1 if rowbytes < 256)
  int round_bf16;     // 1: round logits to bf16 before storing / ranking
  int w_packed;       // 1: w is in the packed layout (bf16 head; w_packed_offset)
  void *logits;       // kStore output [B, V]
  const float *scale;     // int8 per-row scale (may be null)
  const int32_t *target;  // kLse targets [B]
  int32_t *top_id;        // [B, 2]
  float *top_val;         // [B, 2]
  float *margin;          // [B]
  int32_t *top_raw;       // [B, 2] int8 only (may be null)
  // kTop2, bf16-output head: rows with margin < tau are re-ranked on their two
  // candidates' float32-head logits when gated is not null
  float tau;
  int32_t *gated;         // [B] 1 = re-ranked
  float *logprob;         // [B]
  int32_t *zt;            // [B] target logit bits (float32 or int32)
  uint4 *records;         // [B][nblocks] per-block partials
  // kSample: seeded Gumbel-max draw of every row
  float inv_t;                // 1 / temperature
  const uint64_t *seed;       // [B]
  const int64_t *position;    // [B]
  int32_t *token;             // [B]
  float *value, *gap;         // [B] (each may be null)
  // kLseInt: integer log-softmax; row r's logit scale is unit * step_r
  int32_t unit_m, unit_e;     // tensor unit um 2^ue
  const int32_t *step_m;      // [B] row step mantissa M
  const int32_t *step_e;      // [B] row step exponent E
  int64_t *logprob_q;         // [B] log p(target) in Q.24
};

// One tiling of the grid: which kernel instance runs and its grid shape.
struct Plan {
  int variant;  // tile shape index (see lmhead_kernels.hip)
  int bkb;      // bytes of every row staged per pipeline stage
  int bm, bn;   // rows and vocabulary columns per workgroup
  int nt;       // threads per workgroup
  int grid_m, grid_n;
};

// mode: 0 float head, 1 int8 head; w_packed: W in the packed layout
Plan plan_for(int mode, int64_t B, int64_t rowbytes, int64_t V, bool w_packed);

// Size of the static device workspace of lmhead_greedy_top2_noalloc.
constexpr size_t kStaticWorkspaceBytes = (size_t)16 << 20;

// The current device's copy of that workspace (resolved once per device).
hipError_t static_workspace(void **ptr);

// Byte offsets of the workspace regions; returns the total size.
size_t workspace_layout(int64_t B, int64_t V, size_t *off_zt, size_t *off_records);

hipError_t launch(int mode, int epilogue, const Plan &plan, const Params &p, hipStream_t s);

// The tile and fold kernels of one (mode, epilogue) pair for a plan (one
// instance per object file of lmhead_tiles.hip).
template <int MODE, int EPI>
hipError_t launch_epi(const Plan &plan, const Params &p, hipStream_t s);


// Per-token int8 quantisation of int32 rows (one workgroup per row).
hipError_t launch_quantize(const int32_t *x, int64_t B, int64_t H, int8_t *q, int32_t *step_m,
                           int32_t *step_e, hipStream_t s);

hipError_t launch_compare(const void *a, const void *b, int64_t nwords,
                          unsigned long long *mismatches, hipStream_t s);
hipError_t launch_reverse_rows(const void *src, void *dst, int64_t rows, int64_t rowbytes,
                               hipStream_t s);
// Row-major W [V, rowbytes] to the packed layout (ceil(V / kPackRows) groups,
// unused blocks zeroed).
hipError_t launch_pack_w(const void *w, void *out, int64_t V, int64_t rowbytes, hipStream_t s);

}  // namespace lmh
