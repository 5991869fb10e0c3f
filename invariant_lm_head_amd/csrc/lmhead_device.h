// Batch-invariant LM head kernels for gfx950 (CDNA4, MI355X).
//
// One tiled MFMA kernel computes logits Z[b, v] = sum_k X[b, k] * W[v, k] for a
// tile of rows x vocabulary columns and reduces them in its epilogue:
//   kStore  writes Z (float32, bf16-rounded, or int32);
//   kTop2   per-row top-2 (value, id) of every 128-column vocabulary block;
//   kLse    per-row (block max, sum of exp) of every block, and the target logit;
//   kSample per-row top-2 of z / T + Gumbel noise (seeded Gumbel-max draw);
//   kLseInt (int8) per-row block max and the exact sum of integer exps, for
//           the all-integer log-softmax (see "integer front and back").
// The block partials of a row are then folded into the outputs by a second,
// row-parallel kernel (merge_rows for the log-prob folds, whose slot order it
// fixes; one wave per row for the top-2 folds, which are exact in any order).
//
// Batch invariance (one reduction order per logit, fixed by H only):
//   * every logit is acc = 0; for s = 0 .. H*esize/32 - 1: acc = MFMA(A_s, B_s, acc)
//     with ONE instruction for every batch size (v_mfma_f32_32x32x16_bf16 or
//     v_mfma_i32_32x32x32_i8); k-step s covers bytes [32 s, 32 s + 32) of a row,
//     lane half h holding bytes [32 s + 16 h, +16); no split-K; rows of an MFMA
//     are independent, so a row's bits do not depend on its neighbours; the
//     int8 head takes the k-steps from a column-dependent start (k_rotation),
//     which cannot change a bit of its exact int32 sums;
//   * tile shapes change with B only in how many rows and columns a workgroup
//     covers, which does not change any logit's arithmetic;
//   * a block's softmax partial is m_b = max over the block (exact), then
//     s_b = sum exp(z - m_b): for each column offset j (0..31) a balanced binary
//     tree over the block's four 32-column tiles, then a fixed pairing tree over
//     j (j^16, j^15, j^7, j^2, j^1), the same for every row; the row total folds
//     blocks in 16 slots (block b into slot b mod 16, ascending), then a fixed
//     pairing tree over the slots.  All of it depends on V only.  Top-2 with
//     lowest-id ties is exact in any order.
// ("12 Exactness", section 12.2: a product's summation order follows from the
// weight's dimensions alone, not from the batch's row count; "Integer-Only
// Arithmetic", section "Why kernels don't always add in the same order":
// split-K chosen by batch size.)
//
// Data movement: operand tiles are staged HBM -> LDS with global_load_lds_dwordx4
// (no register round trip), in rings of stages whose W loads are spread over
// the k-steps, issued at the boundary, or issued in pairs (Tile), with 16-byte
// chunks XOR-swizzled by row so the MFMA fragment reads (ds_read_b128) are
// bank-conflict free.  The workgroup -> tile map is XCD-aware: workgroups that
// share operand tiles run on the same XCD (same L2).  Cross-lane reductions use
// v_permlane16_swap, DPP and ds_swizzle.
//
// This header holds the device code; lmhead_tiles.hip instantiates the tile and
// fold kernels of one (mode, epilogue) pair per object file, and
// lmhead_kernels.hip holds the plan choice and the small kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "lmhead_internal.h"

namespace lmh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kSlots = 64;  // slots (lanes) of the log-prob fold per row: one wave
constexpr int kChunk = 16;  // records per slot loaded per round of the fold

template <class V> __device__ __forceinline__ V lowest_of();
template <> __device__ __forceinline__ float lowest_of<float>() { return -__builtin_inff(); }
template <> __device__ __forceinline__ int lowest_of<int>() { return INT_MIN; }

// ------------------------------------------------------------- arithmetic
template <int MODE> struct Arith;
template <> struct Arith<0> {  // bf16 x bf16 -> float32
  using acc_t = f32x16;
  using val_t = float;
  static __device__ __forceinline__ acc_t mfma(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Arith<1> {  // int8 x int8 -> int32 (exact)
  using acc_t = i32x16;
  using val_t = int;
  static __device__ __forceinline__ acc_t mfma(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// float32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ unsigned bf16_bits(float f) {
  unsigned u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float(bf16_bits(f) << 16); }

__device__ __forceinline__ bool scale_ok(float s) { return s > 0.0f && s <= 3.0e38f; }

template <class V> __device__ __forceinline__ int vbits(V v) { return __builtin_bit_cast(int, v); }
template <class V> __device__ __forceinline__ V vfrom(int b) { return __builtin_bit_cast(V, b); }

// row of value v (0..15) of a 32x32 MFMA accumulator held by lane half h
__device__ __forceinline__ int acc_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// ------------------------------------------------------ lane permutations
// Involutions on the 32 lanes of a wave half: X16 pairs j with j^16 (ds_swizzle);
// Mirror, HalfMirror, QuadX2, QuadX1 pair j with j^15, j^7, j^2, j^1 (DPP).
enum Perm { kX16 = 0, kMirror = 1, kHalfMirror = 2, kQuadX2 = 3, kQuadX1 = 4 };
template <int P> __device__ __forceinline__ int perm_i(int x) {
  if constexpr (P == kX16) return __builtin_amdgcn_ds_swizzle(x, 0x401F);
  else if constexpr (P == kMirror) return __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false);
  else if constexpr (P == kHalfMirror) return __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false);
  else if constexpr (P == kQuadX2) return __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);
  else return __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);
}
// the lane bit that differs between partners, which decides who keeps the lower half
template <int P> constexpr int kKeepBit = P == kX16 ? 16 : P == kMirror ? 8 : P == kHalfMirror ? 4
                                                         : P == kQuadX2 ? 2 : 1;
template <int P, class V> __device__ __forceinline__ V perm(V x) {
  return vfrom<V>(perm_i<P>(vbits(x)));
}

// --------------------------------------------------------------- tiling
// A workgroup computes a BM x BN tile of logits (BM hidden rows, BN vocabulary
// rows) with WAVES_M x WAVES_N waves.  The k dimension is staged BKB bytes of
// every row at a time, in two LDS rings: NSX stages of the X rows (read from
// L2: every vocabulary tile re-reads them) and NSW > NSX stages of the W rows
// (streamed from HBM once), so W loads are issued NSW - 1 stages ahead of use.
// WSHARED: the plan's row tiles can share W tiles (batches above BM), the later
// workgroups reading them from L2; otherwise each W byte is read by one
// workgroup, and W is loaded with the non-temporal policy (WNT).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BKB_, int NSX_, int NSW_,
          bool WPAIR_ = false, bool WSHARED_ = false>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int BKB = BKB_, NSX = NSX_, NSW = NSW_;
  static constexpr bool WPAIR = WPAIR_, WNT = !WSHARED_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;
  static constexpr int WM = BM / WAVES_M / 32;  // 32-row MFMA tiles per wave
  static constexpr int WN = BN / WAVES_N / 32;  // 32-column MFMA tiles per wave
  static constexpr int STEPS = BKB / 32;        // MFMA k-steps per stage
  static constexpr int XSTAGE = BM * BKB;       // LDS bytes per X stage
  static constexpr int WSTAGE = BN * BKB;       // LDS bytes per W stage
  static constexpr int XSPANS = XSTAGE / 1024;  // 1 KB wave loads per X stage
  static constexpr int WSPANS = WSTAGE / 1024;
  static constexpr int SPWX_MAX = (XSPANS + NW - 1) / NW, SPWX_MIN = XSPANS / NW;
  static constexpr int SPWW_MAX = (WSPANS + NW - 1) / NW, SPWW_MIN = WSPANS / NW;
  static constexpr int WRING = NSX * XSTAGE;    // LDS offset of the W ring
  static constexpr int LDS = NSX * XSTAGE + NSW * WSTAGE;
  static constexpr int WCOLS = WN * 32;         // vocabulary columns per wave
  static constexpr int TPB = kBlockCols / 32;   // column tiles per block (4)
  // a wave covers BPW whole blocks, or PARTS waves share one block
  static constexpr int BPW = WN >= TPB ? WN / TPB : 1;
  static constexpr int PARTS = WN >= TPB ? 1 : TPB / WN;
  static constexpr int NTB = WN >= TPB ? TPB : WN;  // column tiles per block in one wave
  static_assert(BM % (32 * WAVES_M) == 0 && BN % (32 * WAVES_N) == 0, "tile shape");
  static_assert(XSTAGE % 1024 == 0 && WSTAGE % 1024 == 0, "1 KB load spans");
  static_assert(BN % kBlockCols == 0 && (WN % TPB == 0 || TPB % WN == 0), "blocks");
  static_assert(BKB == 64 || BKB == 128 || BKB == 256 || BKB == 512, "stage width");
  static_assert(NSX >= 2 && NSW >= NSX, "ring depths");
  // NSW > NSX: W stage b + NSW is issued spread over the k-steps after boundary
  // b, ahead of the X stage it is consumed with.  NSW == NSX: both are issued at
  // the boundary, and each boundary waits for every load of the next stage.
  // WPAIR (NSX 2, NSW 4): W stages are issued two at a time at every other
  // boundary, span by span (span i of stage s, then span i of stage s + 1), so
  // the two halves of each row's 2 x BKB bytes reach memory back to back.
  static constexpr bool WSPREAD = NSW > NSX && !WPAIR;
  static_assert(!WPAIR || (NSX == 2 && NSW == 4), "paired W stages: rings of 2 and 4");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  // loads of one wave in flight at once (after a boundary's issue) stay below
  // the 6-bit vmcnt counter
  static_assert((NSX - 1) * SPWX_MAX + (NSW - 1) * SPWW_MAX < 64, "vmcnt range");
  // this wave's loads issued after X stage s by the time stage s is awaited
  // (steady state; fewer near the last stages)
  static constexpr int AFTER_MAX =
      WSPREAD ? SPWW_MIN + (NSX - 2) * (SPWX_MIN + SPWW_MIN) : WPAIR ? 2 * SPWW_MIN : 0;
  static_assert(STEPS % 2 == 0, "fragment double buffer parity");
  // epilogue exchange areas (one 32-row tile per wave row at a time) fit in LDS
  static_assert(WAVES_M * 32 * WAVES_N * (4 + 32 * 4) <= LDS && BM * WAVES_N * 16 <= LDS,
                "exchange");
};

// 16-byte chunk swizzle within a staged row.  LDS has 64 banks of 4 bytes and
// serves a ds_read_b128 16 lanes at a time; the fragment reads of 16 lanes touch
// 16 consecutive rows at one logical chunk, and the swizzle spreads them over all
// 64 banks (BKB / 4 banks per row: rows that share bank offsets get different
// chunks).
template <int BKB> __device__ __forceinline__ int swz(int row) {
  if constexpr (BKB == 64) return (row >> 2) & 3;
  else if constexpr (BKB == 128) return (row >> 1) & 7;
  else return row & 15;
}

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most n (0 <= n <= K) of this wave's loads are in flight, n
// rounded down to a value with its own s_waitcnt (waiting for more is safe)
template <int K> __device__ __forceinline__ void wait_vm_le(int n) {
  if constexpr (K <= 0) {
    wait_vm<0>();
  } else {
    if (n >= K) wait_vm<K>();
    else wait_vm_le<K - 1>(n);
  }
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// 16 bytes per lane global -> LDS (global_load_lds_dwordx4, scalar base + 32-bit
// lane offset): lane i writes LDS bytes [lds + 16 i, +16).  Issued as inline asm
// so the compiler does not guard every later LDS read with a full vmcnt(0)
// drain; completion is tracked by the pipeline's explicit vmcnt waits instead.
// m0 (the copy's LDS base) is saved and restored around it; the s_nop is the
// one wait state required between an SALU write of m0 and its use.  NT: the
// non-temporal cache policy, for bytes that no other workgroup reads again.
template <bool NT = false>
__device__ __forceinline__ void dma16(unsigned voff, const void *sbase, unsigned lds) {
  unsigned saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sbase), "s"(lds)
        : "memory");
}

__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
}

__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// floor(n / d) for 0 <= n < 2^31, 1 <= d <= 2^31, from m = ceil(2^63 / d) (see
// div_magic): q = floor(2n m / 2^64) = floor(n / d + n e / 2^63) with
// 0 <= e < 1, and n e / 2^63 < 2^-32 < 1/d - frac(n/d) unless frac(n/d) = 0,
// so q is the exact quotient.  Integer instructions only (a runtime division
// would be lowered through a float32 reciprocal estimate).
__device__ __forceinline__ uint32_t div_exact(uint32_t n, uint64_t m) {
  return (uint32_t)__umul64hi((uint64_t)n << 1, m);
}
// m of div_exact for the divisors 1..8 (compile-time)
constexpr uint64_t kDivSmall[9] = {0, div_magic(1), div_magic(2), div_magic(3), div_magic(4),
                                   div_magic(5), div_magic(6), div_magic(7), div_magic(8)};

// Start of the int8 head's k order for vocabulary column `col`: the row is
// streamed in 256-byte units in ascending order from unit ((col >> 10) mod
// units), wrapping round.  Workgroups of different column groups then read
// different 256-byte offsets of their W rows at the same moment, which spreads
// the concurrent HBM requests over the address bits below the row stride; with
// every workgroup at the same offset the stream rate depends on where the
// allocation landed (measured on MI355X: 23-36 us for the same 131 MB read).
// Integer sums are exact in any order.  The float head does not rotate: a
// column-dependent order would give two identical W rows different roundings,
// and their exact tie would no longer go to the lower id.  Rows that are not a
// whole number of 256-byte units start at byte 0.
constexpr int kRotShift = 10;  // columns per rotation group: 2^kRotShift
__device__ __forceinline__ int64_t k_rotation(const Params &p, int col) {
  if (p.rowbytes % 256 != 0) return 0;
  const uint32_t g = (uint32_t)col >> kRotShift, units = (uint32_t)(p.rowbytes >> 8);
  return (int64_t)(g - units * div_exact(g, p.div_units)) << 8;
}

// Scheduling hint for one k-step: NR fragment reads (of the next step) spread
// between NM MFMAs, each read after NM / NR MFMAs.  Only the order of issue
// changes; every accumulator still sees its MFMAs in k order.
template <int NR, int NM> __device__ __forceinline__ void interleave_reads() {
  constexpr int per = NM / NR > 0 ? NM / NR : 1;
  constexpr int rounds = NR < NM ? NR : NM;
#pragma unroll
  for (int i = 0; i < rounds; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, per, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // LDS read
  }
  if constexpr (NM > per * rounds) __builtin_amdgcn_sched_group_barrier(0x008, NM - per * rounds, 0);
  if constexpr (NR > rounds) __builtin_amdgcn_sched_group_barrier(0x100, NR - rounds, 0);
}

// ----------------------------------------------------- Gumbel-max noise
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011): ten rounds of two
// 32 x 32 -> 64-bit products of counter words with fixed multipliers, the high
// halves mixed with the other counter words and the key, the key bumped by
// fixed Weyl constants between rounds.  Each product is one v_mad_u64_u32.
__device__ __forceinline__ void philox4x32(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                           uint32_t k0, uint32_t k1, uint32_t (&out)[4]) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  constexpr unsigned kXor3 = 0x96;  // truth table of x ^ y ^ z
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    const uint32_t y0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, kXor3);
    const uint32_t y2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, kXor3);
    c0 = y0; c1 = (uint32_t)p1; c2 = y2; c3 = (uint32_t)p0;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// G = -ln(-ln U), U = (2u + 1) 2^-24 from the top 23 bits u of a Philox word,
// evaluated as G = -ln 2 log2(L) - ln(ln 2) with L = -log2 U = (-ln U) / ln 2.
// For U < 3/4, L comes from the hardware log2 (|log2 U| > 0.41 there, so its
// absolute error stays small relative to L).  For U >= 3/4 it comes from
// d = 1 - U (exact) as (2 / ln 2) atanh(s), s = d / (2 - d) <= 1/7, whose odd
// series is summed to s^9: the first term left out is below 4e-10 of the sum.
// Every multiply-add is an explicit fma (one rounding each).
// x < t ? a : b as one compare and one v_cndmask: both operands are computed
// anyway by a 64-lane wave, and a select written in C++ is turned into a
// branch around the costlier operand
__device__ __forceinline__ float select_lt(float x, float t, float a, float b) {
  float r;
  asm("v_cmp_lt_f32_e32 vcc, %1, %2\n\tv_cndmask_b32_e32 %0, %4, %3, vcc"
      : "=v"(r) : "v"(x), "v"(t), "v"(a), "v"(b) : "vcc");
  return r;
}
constexpr float kLnLn2 = -0.366512920581664327f;  // ln(ln 2)
__device__ __forceinline__ float gumbel_of(uint32_t word) {
  constexpr float c1 = 2.88539008177792681f;  // 2 / ln 2, then c1 / k for s^k
  const float U = (float)((word >> 8) | 1u) * 0x1p-24f;  // (2u + 1) 2^-24, exact
  const float d = 1.0f - U;                               // exact
  const float s = d * __builtin_amdgcn_rcpf(2.0f - d);
  const float s2 = s * s;
  float a = __builtin_fmaf(s2, c1 / 9.0f, c1 / 7.0f);
  a = __builtin_fmaf(a, s2, c1 / 5.0f);
  a = __builtin_fmaf(a, s2, c1 / 3.0f);
  a = __builtin_fmaf(a, s2, c1);
  const float L = select_lt(U, 0.75f, -log2_hw(U), s * a);
  return __builtin_fmaf(-kLn2, log2_hw(L), -kLnLn2);
}

__device__ __forceinline__ uint32_t word_of(const uint32_t (&w)[4], int q) {
  const uint32_t a = (q & 1) ? w[1] : w[0], b = (q & 1) ? w[3] : w[2];
  return (q & 2) ? b : a;
}

// ------------------------------------------------------------ top-2 records
// A candidate is ranked by one 64-bit key: an order-preserving 32-bit image of
// its logit in the high half and the complement of its token id in the low
// half, so a larger key is a larger logit, or an equal logit with a lower id
// (the lowest-id tie rule).  Key 0 ranks below every real candidate.
__device__ __forceinline__ unsigned okey(float z) {
  const unsigned u = __float_as_uint(z + 0.0f);  // -0 and +0 compare equal: one key
  return u ^ ((unsigned)((int)u >> 31) | 0x80000000u);
}
__device__ __forceinline__ unsigned okey(int z) { return (unsigned)z ^ 0x80000000u; }
template <class V> __device__ __forceinline__ V okey_value(unsigned k);
template <> __device__ __forceinline__ float okey_value<float>(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}
template <> __device__ __forceinline__ int okey_value<int>(unsigned k) {
  return (int)(k ^ 0x80000000u);
}
__device__ __forceinline__ uint64_t rank_key(unsigned vk, int id) {
  return ((uint64_t)vk << 32) | (unsigned)~id;
}
__device__ __forceinline__ int key_id(uint64_t k) { return (int)~(unsigned)k; }

struct Top2 {
  uint64_t k1, k2;  // k1 > k2
};
__device__ __forceinline__ Top2 t2_merge(const Top2 &a, const Top2 &b) {
  const bool bw = b.k1 > a.k1;  // b's best is the overall best
  // runner-up: the loser of the two bests against the winner's own second
  const uint64_t l = bw ? a.k1 : b.k1;
  const uint64_t s = bw ? b.k2 : a.k2;
  Top2 r;
  r.k1 = bw ? b.k1 : a.k1;
  r.k2 = l > s ? l : s;
  return r;
}
template <int P> __device__ __forceinline__ uint64_t perm64(uint64_t x) {
  const unsigned lo = (unsigned)perm_i<P>((int)(unsigned)x);
  const unsigned hi = (unsigned)perm_i<P>((int)(unsigned)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}
template <int P> __device__ __forceinline__ Top2 perm(const Top2 &t) {
  return Top2{perm64<P>(t.k1), perm64<P>(t.k2)};
}
__device__ __forceinline__ Top2 pick(bool c, const Top2 &a, const Top2 &b) {
  return Top2{c ? a.k1 : b.k1, c ? a.k2 : b.k2};
}
__device__ __forceinline__ uint4 t2_pack(const Top2 &t) {
  return make_uint4((unsigned)t.k1, (unsigned)(t.k1 >> 32), (unsigned)t.k2, (unsigned)(t.k2 >> 32));
}
__device__ __forceinline__ Top2 t2_unpack(uint4 r) {
  return Top2{((uint64_t)r.y << 32) | r.x, ((uint64_t)r.w << 32) | r.z};
}

// Top-2 of the NTB (1, 2 or 4) logits z[0..NTB) a lane holds for one row, whose
// token ids increase with the index (ties go to the lower index), as keys.
// cbase = ~(id of z[0]); ids step by 32.
template <int NTB, class V>
__device__ __forceinline__ Top2 lane_top2(const V (&z)[NTB], unsigned cbase) {
  auto key = [&](V v, int i) { return ((uint64_t)okey(v) << 32) | (cbase - 32u * (unsigned)i); };
  if constexpr (NTB == 1) {
    return Top2{key(z[0], 0), 0};
  } else if constexpr (NTB == 2) {
    const bool c = z[0] >= z[1];
    return Top2{key(c ? z[0] : z[1], c ? 0 : 1), key(c ? z[1] : z[0], c ? 1 : 0)};
  } else {
    static_assert(NTB == 4, "column tiles per block");
    const bool c01 = z[0] >= z[1], c23 = z[2] >= z[3];
    const V a = c01 ? z[0] : z[1], b = c01 ? z[1] : z[0];
    const int ia = c01 ? 0 : 1, ib = c01 ? 1 : 0;
    const V c = c23 ? z[2] : z[3], d = c23 ? z[3] : z[2];
    const int ic = c23 ? 2 : 3, id = c23 ? 3 : 2;
    const bool cac = a >= c;  // a has the lower id
    const V t1 = cac ? a : c;
    const int i1 = cac ? ia : ic;
    // runner-up: the loser of (a, c) against the winner's partner; the candidate
    // from columns 0..1 has the lower id
    const V pv = cac ? b : a, qv = cac ? c : d;
    const int ip = cac ? ib : ia, iq = cac ? ic : id;
    const bool cpq = pv >= qv;
    return Top2{key(t1, i1), key(cpq ? pv : qv, cpq ? ip : iq)};
  }
}

// f(integral_constant<int, I>) for I = I0 .. N-1, unrolled by the front end
// (for loop bodies too large for the unroller's budget)
template <int I, int N, class F> __device__ __forceinline__ void static_for(F &&f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ------------------------------------------------ integer front and back
// The all-integer head ("Integer-Only Arithmetic", section "DetLLM": every
// tensor carries a dyadic scale m / 2^k, rescaled by an integer multiply and a
// shift under one rounding rule; exp and softmax are integer algorithms; each
// token is quantised from its own values).  The pages give no algorithm; this
// one uses round half up for every rescale, rnd(p, s) = (p + 2^(s-1)) >> s:
//   * exp: T >= 0 in Q.24 nats -> e^(-T) in Q.30.  T = q L + r with L the
//     Q.24 ln 2 and 0 <= r < L; e^(-r) by the Taylor series to degree 10 in
//     Horner form with coefficients round(2^30 / n!); then rnd(., q).
//   * ln: S >= 2^30 (Q.30) -> ln(S / 2^30) in Q.30: S = 2^l (1 + f) with f
//     rounded to 30 bits, ln(1 + f) = 2 atanh(f / (2 + f)) by the odd series
//     to the 25th power (rounded divisions), plus (l - 30) times the Q.30 ln 2.
//   * a row's logit scale: unit um 2^ue times the row step M 2^E, the mantissa
//     product rounded to 31 bits, as m / 2^(24 + sh) with 0 <= sh <= 62.
//   * softmax: per 128-column block (fixed by V) the exact max m_b and the
//     exact sum S_b of exp(T((m_b - z) m)); the row folds
//     S = sum_b rnd(S_b exp(T((z_max - m_b) m)), 30) exactly (in any order),
//     log p(t) = -(T((z_max - z_t) m) + rnd(ln S, 6)) in Q.24.
constexpr int kNatsFrac = 24;
constexpr int kExpFrac = 30;
constexpr uint32_t kLn2Q24 = 11629080u;   // round(ln 2 * 2^24) (ln 2 * 2^24 = 11629079.97)
constexpr int64_t kLn2Q30 = 744261118;    // round(ln 2 * 2^30) (ln 2 * 2^30 = 744261117.95)
constexpr int kExpDegree = 10;
constexpr int kAtanhTerms = 12;

struct TaylorQ30 {  // round(2^30 / n!), n = 0 .. kExpDegree, half up
  uint32_t c[kExpDegree + 1];
  constexpr TaylorQ30() : c() {
    uint64_t f = 1;
    for (int n = 0; n <= kExpDegree; ++n) {
      if (n >= 2) f *= (uint64_t)n;
      c[n] = (uint32_t)((((uint64_t)1 << (kExpFrac + 1)) + f) / (2 * f));
    }
  }
};
constexpr TaylorQ30 kTaylor{};
static_assert(kTaylor.c[0] == (1u << 30) && kTaylor.c[1] == (1u << 30) && kTaylor.c[2] == (1u << 29),
              "Taylor coefficients");

__device__ __forceinline__ uint64_t rnd64(uint64_t p, int s) {  // p < 2^63, 0 <= s <= 63
  return s == 0 ? p : (p + ((uint64_t)1 << (s - 1))) >> s;
}

// e^(-T[i] / 2^24) in Q.30 for N independent T (Q.24 nats), evaluated in
// lockstep so the N Horner chains of dependent multiply-adds interleave (one
// chain alone waits on each multiply-add's latency); each result is the same
// as evaluated alone
template <int N>
__device__ __forceinline__ void iexp_q30_n(const uint64_t (&T)[N], uint32_t (&e)[N]) {
  static_assert(kNatsFrac == 24 && kLn2Q24 < (1u << 24), "r 2^8 fits 32 bits");
  bool zero[N];
  uint32_t q[N], r8[N], y[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    // 2^-q with q >= 32 rounds a Q.30 value to 0 (branch-free: select at the end)
    zero[i] = T[i] >= 32ull * kLn2Q24;
    const uint32_t t = zero[i] ? 0u : (uint32_t)T[i];
    q[i] = t / kLn2Q24;
    // rnd(y r, 24) = floor((y r 2^8 + 2^31) / 2^32): the high word of one
    // 32 x 32 + 64-bit multiply-add (the same value as the 24-bit shift)
    r8[i] = (t - q[i] * kLn2Q24) << 8;
    y[i] = kTaylor.c[kExpDegree];
  }
#pragma unroll
  for (int n = kExpDegree - 1; n >= 0; --n)
#pragma unroll
    for (int i = 0; i < N; ++i)
      y[i] = kTaylor.c[n] - (uint32_t)(((uint64_t)y[i] * r8[i] + (1ull << 31)) >> 32);
  // y <= 2^30 (the partial sums of the alternating series stay in (0, 1]),
  // so the rounding shift by q <= 31 stays within 32 bits
#pragma unroll
  for (int i = 0; i < N; ++i) e[i] = zero[i] ? 0u : (y[i] + ((1u << q[i]) >> 1)) >> q[i];
}
__device__ __forceinline__ uint32_t iexp_q30(uint64_t T) {
  const uint64_t t[1] = {T};
  uint32_t e[1];
  iexp_q30_n<1>(t, e);
  return e[0];
}

// floor(n / d) by restoring binary division, for a quotient below 2^31 (n <
// 2^31 d, d < 2^62): integer instructions only, one step per quotient bit
__device__ __forceinline__ uint64_t udiv_small_quotient(uint64_t n, uint64_t d) {
  uint64_t q = 0;
#pragma unroll 1
  for (int b = 30; b >= 0; --b) {
    const uint64_t t = d << b;
    if (n >= t) {
      n -= t;
      q |= (uint64_t)1 << b;
    }
  }
  return q;
}

// ln(S / 2^30) in Q.30 for S >= 2^30
__device__ int64_t iln_q30(uint64_t S) {
  int l = 63 - __clzll((long long)S);
  uint64_t mant = rnd64(S, l - kExpFrac);
  if (mant == (2ull << kExpFrac)) {
    mant = 1ull << kExpFrac;
    l += 1;
  }
  const uint64_t f = mant - (1ull << kExpFrac);
  const uint64_t den = (2ull << kExpFrac) + f;
  // round(f 2^30 / den): the quotient is below 2^29 (f < 2^30 < den)
  const uint64_t u = udiv_small_quotient(2 * (f << kExpFrac) + den, 2 * den);
  const uint64_t u2 = rnd64(u * u, kExpFrac);
  uint64_t t = u, acc = u;
  for (int j = 1; j <= kAtanhTerms; ++j) {
    t = rnd64(t * u2, kExpFrac);
    const uint64_t d = 2 * j + 1;
    acc += (2 * t + d) / (2 * d);
  }
  return (int64_t)(l - kExpFrac) * kLn2Q30 + 2 * (int64_t)acc;
}

// logit scale m / 2^(24 + sh) of a row; m = 0 when not valid
struct IntScale {
  uint32_t m;
  int sh;
  uint64_t half;  // 2^(sh - 1), 0 when sh = 0: the rounding term of int_nats
};
__device__ __forceinline__ IntScale int_row_scale(int um, int ue, int M, int E) {
  if (um <= 0 || M <= 0) return IntScale{0u, 0, 0};
  const uint64_t P = (uint64_t)um * (uint64_t)M;  // < 2^62
  int sh = (64 - __clzll((long long)P)) - 31;     // bits beyond 31
  uint64_t mm;
  if (sh > 0) {
    mm = (P + (1ull << (sh - 1))) >> sh;
    if (mm == (1ull << 31)) {
      mm = 1ull << 30;
      sh += 1;
    }
  } else {
    mm = P << (-sh);
  }
  const int64_t k = -((int64_t)sh + ue + E);  // real = mm 2^-k
  if (k < kNatsFrac || k > kNatsFrac + 62) return IntScale{0u, 0, 0};
  const int sh2 = (int)(k - kNatsFrac);
  return IntScale{(uint32_t)mm, sh2, sh2 > 0 ? 1ull << (sh2 - 1) : 0ull};
}

// T(d) = rnd(d m, sh): a logit difference d >= 0 in Q.24 nats
__device__ __forceinline__ uint64_t int_nats(uint32_t d, const IntScale &s) {
  // d m + 2^(sh - 1) < 2^63 + 2^61: one multiply-add, then the shift
  return ((uint64_t)d * s.m + s.half) >> s.sh;
}

// integer softmax partial carried through the lane tree: the block max and
// the exact sum as two 32-bit halves (no padding, so it stays in registers)
struct LseI {
  int m;
  unsigned lo, hi;
  __device__ __forceinline__ uint64_t sum() const { return ((uint64_t)hi << 32) | lo; }
};
__device__ __forceinline__ LseI lse_i(int m, uint64_t s) {
  return LseI{m, (unsigned)s, (unsigned)(s >> 32)};
}

// softmax partial carried through the lane tree: the block max (identical on
// both partners of every pairing) and the partial sum
struct Lse {
  int m;  // bits of the block max (float32 or int32)
  float s;
};

__device__ __forceinline__ Top2 combine(const Top2 &a, const Top2 &b) { return t2_merge(a, b); }
__device__ __forceinline__ Lse combine(const Lse &a, const Lse &b) { return Lse{a.m, a.s + b.s}; }
template <int P> __device__ __forceinline__ Lse perm(const Lse &x) { return Lse{x.m, perm<P>(x.s)}; }
__device__ __forceinline__ Lse pick(bool c, const Lse &a, const Lse &b) {
  return Lse{c ? a.m : b.m, c ? a.s : b.s};
}
__device__ __forceinline__ LseI combine(const LseI &a, const LseI &b) {
  return lse_i(a.m, a.sum() + b.sum());
}
template <int P> __device__ __forceinline__ LseI perm(const LseI &x) {
  return LseI{x.m, (unsigned)perm_i<P>((int)x.lo), (unsigned)perm_i<P>((int)x.hi)};
}
__device__ __forceinline__ LseI pick(bool c, const LseI &a, const LseI &b) {
  return LseI{c ? a.m : b.m, c ? a.lo : b.lo, c ? a.hi : b.hi};
}

// One halving step of the reduce-scatter over the 32 column lanes: R row
// values per lane become R/2; the partner under P receives the half this lane
// does not keep.
template <int P, int R, class T> __device__ __forceinline__ void rs_step(T (&a)[16], int j) {
  const bool keep_low = (j & kKeepBit<P>) == 0;
#pragma unroll
  for (int i = 0; i < R / 2; ++i) {
    const T send = pick(keep_low, a[i + R / 2], a[i]);
    const T keep = pick(keep_low, a[i], a[i + R / 2]);
    a[i] = combine(keep, perm<P>(send));
  }
}
// The first step (partners j and j^16, the two 16-lane rows of a wave half)
// without selects: v_permlane16_swap exchanges the odd rows of its first
// operand with the even rows of its second.  With x = a[i], y = a[i + 8] it
// leaves, in an even-row lane, its own a[i] and its partner's a[i]; in an
// odd-row lane, its partner's a[i + 8] and its own a[i + 8].  combine() is
// symmetric (an exact top-2 of a union, or a commutative sum), so the result
// equals rs_step<kX16, 16> bit for bit.
template <class T> __device__ __forceinline__ void swap_rows16(T &x, T &y) {
  static_assert(sizeof(T) % 4 == 0, "32-bit words");
  constexpr int N = sizeof(T) / 4;
  unsigned xw[N], yw[N];
  __builtin_memcpy(xw, &x, sizeof(T));
  __builtin_memcpy(yw, &y, sizeof(T));
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const auto r = __builtin_amdgcn_permlane16_swap(xw[k], yw[k], false, false);
    xw[k] = r[0];
    yw[k] = r[1];
  }
  __builtin_memcpy(&x, xw, sizeof(T));
  __builtin_memcpy(&y, yw, sizeof(T));
}
template <class T> __device__ __forceinline__ void rs_rows16(T (&a)[16]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    swap_rows16(a[i], a[i + 8]);
    a[i] = combine(a[i], a[i + 8]);
  }
}

// 16 row values on each of the 32 column lanes -> lane j holds row value
// u(j) = 8 b4 + 4 b3 + 2 b2 + b1 (b = bits of j) combined over all 32 columns,
// in the pairing order j^16, j^15, j^7, j^2, j^1 (the same for every row).
template <class T> __device__ __forceinline__ T reduce_scatter(T (&a)[16], int j) {
  rs_rows16(a);
  rs_step<kMirror, 8>(a, j);
  rs_step<kHalfMirror, 4>(a, j);
  rs_step<kQuadX2, 2>(a, j);
  return combine(a[0], perm<kQuadX1>(a[0]));
}
__device__ __forceinline__ int rs_value_index(int j) {
  return 8 * ((j >> 4) & 1) + 4 * ((j >> 3) & 1) + 2 * ((j >> 2) & 1) + ((j >> 1) & 1);
}

// max over the 32 column lanes, left in every lane (exact in any order)
template <class V> __device__ __forceinline__ V allmax32(V x) {
  V o;
  o = perm<kX16>(x); x = o > x ? o : x;
  o = perm<kMirror>(x); x = o > x ? o : x;
  o = perm<kHalfMirror>(x); x = o > x ? o : x;
  o = perm<kQuadX2>(x); x = o > x ? o : x;
  o = perm<kQuadX1>(x); x = o > x ? o : x;
  return x;
}

// balanced binary tree sum of N values (left + right at every level)
template <int N> __device__ __forceinline__ float tree_sum(const float *e) {
  if constexpr (N == 1) {
    return e[0];
  } else {
    return tree_sum<N / 2>(e) + tree_sum<N / 2>(e + N / 2);
  }
}

// ------------------------------------------------------- final row folds
// Rows [row0, row0 + nrows) of the records, 16 lanes (slots) per row; the
// caller's threads [0, nthreads) take rows 16 lanes at a time.  Block b goes to
// slot b mod 16, slots fold ascending, then slots pair j^1, j^2, j^7, j^15.
// ------------------------------------------------------ gated recompute
// Margin-gated recompute ("Greedy Decoding Has a Precision Clause", section
// "Correct the vulnerable token decisions, not every calculation"), run by the
// fold right after it has written the bf16-output head's top-2 of rows
// [row0, row0 + nrows), nrows <= 64.  Rows whose margin is below tau are
// listed; each wave takes up to 16 of them and recomputes their candidates'
// logits with the float32 head in one MFMA chain: A row i (and i + 16) is
// listed row i's hidden row, B column 2i / 2i + 1 its first / second
// candidate's W row, k ascending, the instruction and lane layout of the tile
// kernel.  An MFMA result depends only on its own A row and B column, so each
// value equals the float32 head's bits.  The two are then ranked, lowest id on
// a tie, and the row's outputs replaced.
// lds: kGateLdsInts ints of LDS the caller's workgroup does not otherwise use
// meanwhile (the listed rows, then their count)
constexpr int kGateLdsInts = 65;
__device__ void gate_rows(const Params &p, int row0, int nrows, int tid, int nthreads, int *lds) {
  int *s_rows = lds;
  int &s_count = lds[64];
  __syncthreads();  // the fold's writes of these rows are visible to every wave
  if (tid < 64) {
    const bool in = tid < nrows;
    const int row = row0 + (in ? tid : 0);
    const bool gate = in && p.margin[row] < p.tau;
    if (in) p.gated[row] = gate ? 1 : 0;
    const unsigned long long m = __ballot(gate);
    if (gate) s_rows[__popcll(m & ((1ull << tid) - 1))] = row;
    if (tid == 0) s_count = __popcll(m);
  }
  __syncthreads();
  const int G = s_count;
  const int lane = tid & 63, j = lane & 31, h = lane >> 5;
  for (int b = tid >> 6; 16 * b < G; b += nthreads >> 6) {
    const int n = min(16, G - 16 * b);
    const int ra = s_rows[16 * b + min(j & 15, n - 1)];
    const int rb = s_rows[16 * b + min(j >> 1, n - 1)];
    const int cand = p.top_id[2 * rb + (j & 1)];
    const char *xr = p.x + (int64_t)ra * p.rowbytes + 16 * h;
    // byte kb of W row `cand`, row-major or packed
    auto wat = [&](int kb) -> const char * {
      return p.w + (p.w_packed ? w_packed_offset(cand, kb, p.rowbytes)
                               : (int64_t)cand * p.rowbytes + kb);
    };
    f32x16 acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
    // the chain is latency-bound: the fragments of GK k-steps are loaded
    // before their MFMAs, GK = 32 while they last, then 4 (H is a multiple of 64)
    const int nsteps = (int)(p.rowbytes / 32);
    auto steps = [&](int k0, auto gk) {
      constexpr int GK = decltype(gk)::value;
      i32x4 fa[GK], fb[GK];
#pragma unroll
      for (int k = 0; k < GK; ++k) {
        fa[k] = *(const i32x4 *)(xr + 32 * (k0 + k));
        fb[k] = *(const i32x4 *)wat(32 * (k0 + k) + 16 * h);
      }
      __builtin_amdgcn_sched_barrier(0);  // every load issued before the first MFMA waits
#pragma unroll
      for (int k = 0; k < GK; ++k) acc = Arith<0>::mfma(fa[k], fb[k], acc);
    };
    int k0 = 0;
    for (; k0 + 32 <= nsteps; k0 += 32) steps(k0, std::integral_constant<int, 32>{});
    for (; k0 < nsteps; k0 += 4) steps(k0, std::integral_constant<int, 4>{});
    // (A row i, B column c) is value 4 (i >> 3) + (i & 3) of lane 32 ((i >> 2) & 1) + c
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int v = 4 * (i >> 3) + (i & 3), base = 32 * ((i >> 2) & 1) + 2 * i;
      const float z1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[v]), base));
      const float z2 =
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc[v]), base + 1));
      if (lane == 0 && i < n) {
        const int row = s_rows[16 * b + i];
        const int c1 = p.top_id[2 * row], c2 = p.top_id[2 * row + 1];
        const bool second = (z2 > z1) | ((z2 == z1) & (c2 < c1));
        p.top_id[2 * row] = second ? c2 : c1;
        p.top_id[2 * row + 1] = second ? c1 : c2;
        const float t1 = second ? z2 : z1, t2 = second ? z1 : z2;
        p.top_val[2 * row] = t1;
        p.top_val[2 * row + 1] = t2;
        p.margin[row] = t1 - t2;
      }
    }
  }
}

// A row's outputs from its folded top-2 (greedy) or Gumbel top-2 (sampling).
template <int MODE, int EPI>
__device__ __forceinline__ void put_top2(const Params &p, int row, const Top2 &t) {
  using val_t = typename Arith<MODE>::val_t;
  if constexpr (EPI == kSample) {
    bool ok = true;
    if constexpr (MODE == 1) ok = scale_ok(p.scale ? p.scale[row] : 1.0f);
    const float y1 = okey_value<float>((unsigned)(t.k1 >> 32));
    const float y2 = okey_value<float>((unsigned)(t.k2 >> 32));
    const float nan = __builtin_nanf("");
    p.token[row] = ok ? key_id(t.k1) : -1;
    if (p.value) p.value[row] = ok ? y1 : nan;
    if (p.gap) p.gap[row] = ok ? y1 - y2 : nan;
  } else {
    const val_t v1 = okey_value<val_t>((unsigned)(t.k1 >> 32));
    const val_t v2 = okey_value<val_t>((unsigned)(t.k2 >> 32));
    p.top_id[2 * row] = key_id(t.k1);
    p.top_id[2 * row + 1] = key_id(t.k2);
    if constexpr (MODE == 0) {
      p.top_val[2 * row] = v1;
      p.top_val[2 * row + 1] = v2;
      p.margin[row] = v1 - v2;
    } else {
      const float s = p.scale ? p.scale[row] : 1.0f;
      if (p.top_raw) {
        p.top_raw[2 * row] = v1;
        p.top_raw[2 * row + 1] = v2;
      }
      const bool ok = scale_ok(s);
      const float nan = __builtin_nanf("");
      // one rounding of an exact float64 product (|raw| < 2^31, 24-bit scale)
      p.top_val[2 * row] = ok ? (float)((double)v1 * (double)s) : nan;
      p.top_val[2 * row + 1] = ok ? (float)((double)v2 * (double)s) : nan;
      // v1 >= v2 and v1 - v2 < 2^32: exact as an unsigned 32-bit difference
      const uint32_t dv = (uint32_t)v1 - (uint32_t)v2;
      p.margin[row] = ok ? (float)((double)dv * (double)s) : nan;
    }
  }
}

// The log-prob fold of rows row0 .. row0 + nrows - 1: one wave (kSlots lanes)
// per row, so a row's records are loaded in one round up to 1024 blocks and
// its latency is paid once, not once per 256 blocks.
template <int MODE, int EPI, int CH>
__device__ void merge_rows_ch(const Params &p, int row0, int nrows, int tid, int nthreads) {
  static_assert(EPI == kLse || EPI == kLseInt, "top-2 folds use lmhead_merge_top2_kernel");
  using val_t = typename Arith<MODE>::val_t;
  const int slot = tid & (kSlots - 1);
  const int nb = p.nblocks;
  for (int g = tid / kSlots; g < nrows; g += nthreads / kSlots) {
    const int row = row0 + g;
    const uint4 *rec = p.records + (int64_t)row * nb;
    // The row max (exact), then the sum of the rescaled block sums in slot
    // order, then an xor butterfly over the slots.  CH records per slot
    // are in flight per round of loads (one memory latency per round).  When
    // one round covers the row (nb <= CH * kSlots), its records stay in
    // registers for the sum; otherwise they are read again.  The row's own
    // inputs are loaded first, so their latency overlaps the records'.
    const int tgt = p.target[row];
    int zt;  // the target's logit bits, meaningful only for a target in range
    if constexpr (MODE == 1) {
      // int8 head: the target's int32 logit, exact, from 16-byte pieces of
      // x[row] and w[target] spread over the row's lanes (every partial sum is
      // below 2^31 in magnitude, so any order gives the same integer)
      int dot = 0;
      if (tgt >= 0 && tgt < p.V) {
        const char *xr = p.x + (int64_t)row * p.rowbytes;
        const char *wr = p.w + (int64_t)tgt * p.rowbytes;
#pragma unroll 4
        for (int64_t off = 16 * slot; off < p.rowbytes; off += 16 * kSlots) {
          const int4 a = *(const int4 *)(xr + off), c = *(const int4 *)(wr + off);
          dot = __builtin_amdgcn_sdot4(a.x, c.x, dot, false);
          dot = __builtin_amdgcn_sdot4(a.y, c.y, dot, false);
          dot = __builtin_amdgcn_sdot4(a.z, c.z, dot, false);
          dot = __builtin_amdgcn_sdot4(a.w, c.w, dot, false);
        }
      }
#pragma unroll
      for (int m = 1; m < kSlots; m <<= 1) dot += __shfl_xor(dot, m);
      zt = dot;
    } else {
      zt = p.zt[row];  // the float head's target logit, as its tile computed it
    }
    const bool one_round = nb <= CH * kSlots;
    if constexpr (EPI == kLseInt) {
      const IntScale sc = int_row_scale(p.unit_m, p.unit_e, p.step_m[row], p.step_e[row]);
      uint4 r[CH];
      int mx = INT_MIN;
      for (int b0 = slot; b0 < nb; b0 += CH * kSlots) {
#pragma unroll
        for (int q = 0; q < CH; ++q) r[q] = rec[min(b0 + q * kSlots, nb - 1)];
#pragma unroll
        for (int q = 0; q < CH; ++q) mx = (int)r[q].x > mx ? (int)r[q].x : mx;
      }
#pragma unroll
      for (int m = 1; m < kSlots; m <<= 1) {
        const int o = __shfl_xor(mx, m);
        mx = o > mx ? o : mx;
      }
      // integer terms: the order does not matter
      uint64_t S = 0;
      for (int b0 = slot; b0 < nb; b0 += CH * kSlots) {
        if (!one_round) {
#pragma unroll
          for (int q = 0; q < CH; ++q) r[q] = rec[min(b0 + q * kSlots, nb - 1)];
        }
        // the chunk's rescale factors in lockstep (records past nb repeat the
        // last one and are left out of the exact sum)
        uint64_t tq[CH];
        uint32_t Rq[CH];
#pragma unroll
        for (int q = 0; q < CH; ++q) tq[q] = int_nats((uint32_t)mx - r[q].x, sc);
        iexp_q30_n<CH>(tq, Rq);
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          const uint64_t R = Rq[q];
          // rnd(S_b R, 30) with S_b < 2^38 split at bit 32: both products fit
          const uint64_t term = ((uint64_t)r[q].z * R << 2) + rnd64((uint64_t)r[q].y * R, kExpFrac);
          S += b0 + q * kSlots < nb ? term : 0ull;
        }
      }
#pragma unroll
      for (int m = 1; m < kSlots; m <<= 1) S += __shfl_xor(S, m);
      if (slot == 0) {
        int64_t lp = INT64_MIN;
        if (tgt >= 0 && tgt < p.V && sc.m != 0u) {
          const uint64_t Tt = int_nats((uint32_t)mx - (uint32_t)zt, sc);
          const uint64_t L = rnd64((uint64_t)iln_q30(S), kExpFrac - kNatsFrac);
          const uint64_t nl = Tt + L;  // < 2^63 + 2^40: no wrap
          lp = nl > (uint64_t)INT64_MAX ? -INT64_MAX : -(int64_t)nl;
        }
        p.logprob_q[row] = lp;
      }
    } else {
      float cr = kLog2e, sr = 1.0f;
      if constexpr (MODE == 1) {
        sr = p.scale ? p.scale[row] : 1.0f;
        cr = sr * kLog2e;
      }
      uint2 r[CH];
      val_t mx = lowest_of<val_t>();
      for (int b0 = slot; b0 < nb; b0 += CH * kSlots) {
#pragma unroll
        for (int q = 0; q < CH; ++q) r[q] = *(const uint2 *)&rec[min(b0 + q * kSlots, nb - 1)];
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          const val_t o = vfrom<val_t>((int)r[q].x);  // a repeated last block cannot change a max
          mx = o > mx ? o : mx;
        }
      }
#pragma unroll
      for (int m = 1; m < kSlots; m <<= 1) {
        const val_t o = __shfl_xor(mx, m);
        mx = o > mx ? o : mx;
      }
      float s = 0.0f;
      for (int b0 = slot; b0 < nb; b0 += CH * kSlots) {
        if (!one_round) {
#pragma unroll
          for (int q = 0; q < CH; ++q) r[q] = *(const uint2 *)&rec[min(b0 + q * kSlots, nb - 1)];
        }
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          if (b0 + q * kSlots < nb) {
            float d;
            if constexpr (MODE == 0) d = __uint_as_float(r[q].x) - mx;
            else d = -(float)((uint32_t)mx - r[q].x);  // mx - z < 2^32, one rounding
            s = s + __uint_as_float(r[q].y) * exp2_hw(d * cr);
          }
        }
      }
      // xor butterfly: s + partner is the same sum on both partners, so every
      // lane ends with the same bits
#pragma unroll
      for (int m = 1; m < kSlots; m <<= 1) s = s + __shfl_xor(s, m);
      if (slot == 0) {
        float lp = __builtin_nanf("");
        if (tgt >= 0 && tgt < p.V) {
          if constexpr (MODE == 0) {
            lp = (__int_as_float(zt) - mx) - kLn2 * log2_hw(s);
          } else {
            // (z_t - max) * s in float64 (exact difference, one rounding of the product)
            if (scale_ok(sr))
              lp = (float)(-(double)((uint32_t)mx - (uint32_t)zt) * (double)sr) - kLn2 * log2_hw(s);
          }
        }
        p.logprob[row] = lp;
      }
    }
  }
}

// CH records per slot in flight: 4 when one round of them covers the row
// (up to 256 blocks), else 16.  Each slot still adds its blocks in ascending
// order, so CH changes no bit.
template <int MODE, int EPI>
__device__ void merge_rows(const Params &p, int row0, int nrows, int tid, int nthreads) {
  if (p.nblocks <= 4 * kSlots) merge_rows_ch<MODE, EPI, 4>(p, row0, nrows, tid, nthreads);
  else merge_rows_ch<MODE, EPI, kChunk>(p, row0, nrows, tid, nthreads);
}

// one block record (read by the fold kernel after the tile launch ends)
__device__ __forceinline__ void put_record(uint4 *d, uint4 v) { *d = v; }

// ------------------------------------------------------------------ kernel
template <class T, int MODE, int EPI>
__global__ __launch_bounds__(T::NT) void lmhead_tile_kernel(Params p) {
  using A = Arith<MODE>;
  using acc_t = typename A::acc_t;
  using val_t = typename A::val_t;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int j = lane & 31, h = lane >> 5;  // MFMA column lane, lane half

  // ---- workgroup -> tile, XCD-aware: consecutive workgroups are dealt to the 8
  // XCDs in turn, so renumber them XCD-major, then walk GROUP_M row tiles per
  // vocabulary tile so neighbours on one XCD share X and W tiles in its L2.
  // A grid of one row tile of up to 128 rows shares no W tile; from the
  // packed layout it keeps the plain order (workgroup b, vocabulary tile b),
  // which streamed W 0.2-0.65 us faster per call at batches 1-128 (row-major
  // W, and the 256-row tile of batches 129-256: the XCD-major order, 0.03-0.45
  // and about 0.3 us faster).
  int tm, tn;
  {
    const int G = gridDim.x, bid = blockIdx.x, per = G >> 3;
    const int nb = T::BM <= 128 && p.grid_m == 1 && p.w_packed ? bid
                   : bid < (per << 3)                          ? (bid & 7) * per + (bid >> 3)
                                                               : bid;
    constexpr int GROUP_M = kTileGroup;
    const int in_group = GROUP_M * p.grid_n;
    const int group = (int)div_exact((uint32_t)nb, p.div_group);  // nb / in_group
    const int first_m = group * GROUP_M;
    const int gsz = min(p.grid_m - first_m, GROUP_M);
    const int rem = nb - group * in_group;
    uint64_t mg = kDivSmall[1];
#pragma unroll
    for (int d = 2; d <= GROUP_M; ++d) mg = gsz == d ? kDivSmall[d] : mg;
    tn = (int)div_exact((uint32_t)rem, mg);  // rem / gsz
    tm = first_m + (rem - tn * gsz);
  }
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  // ---- per-lane 32-bit source offset (from the tile's first row) of each 1 KB
  // LDS span this wave fills every stage; rows past B / V re-read the last row
  // (their results are masked in the epilogue)
  const bool wpk = MODE == 0 && p.w_packed;  // W in the packed layout (float head)
  const char *xtile = p.x + (int64_t)m0 * p.rowbytes;
  const char *wtile =
      p.w + (wpk ? (int64_t)(n0 / kPackRows) * packed_group_bytes(p.rowbytes) : (int64_t)n0 * p.rowbytes);
  // stage t holds bytes [koff(t), koff(t) + BKB) of every row: the k order of
  // this tile's columns (a tile never straddles a rotation group, and the
  // rotation is a whole number of stages)
  static_assert(MODE != 1 || ((1LL << kRotShift) % T::BN == 0 && 256 % T::BKB == 0),
                "tile within one rotation group");
  const int64_t rot = MODE == 1 ? k_rotation(p, n0) : 0;
  const int nst = (int)(p.rowbytes / T::BKB);  // stages per row
  auto koff = [&](int stage) -> int64_t {
    const int64_t o = (int64_t)stage * T::BKB + rot;
    return o >= p.rowbytes ? o - p.rowbytes : o;
  };
  auto span_offset = [&](int span, int first, int last) -> unsigned {
    const int off = span * 1024 + lane * 16;
    const int row = off / T::BKB;
    const int chunk = ((off % T::BKB) >> 4) ^ swz<T::BKB>(row);
    return (unsigned)(min(first + row, last) - first) * (unsigned)p.rowbytes + 16u * chunk;
  };
  unsigned xoff[T::SPWX_MAX], woff[T::SPWW_MAX];
#pragma unroll
  for (int i = 0; i < T::SPWX_MAX; ++i)
    xoff[i] = span_offset(min(wave + i * T::NW, T::XSPANS - 1), m0, p.B - 1);
  // the packed W layout (float head): the same bytes of the tile's rows, at
  // their packed offsets; tiles start on a row group (BN is a multiple of 128)
  static_assert(T::BN % kPackRows == 0, "tiles start on a packed row group");
  static_assert(T::BKB % kPackBytes == 0 || kPackBytes % T::BKB == 0, "stages and blocks nest");
  auto span_offset_packed = [&](int span, int first, int last) -> unsigned {
    const int off = span * 1024 + lane * 16;
    const int row = min(first + off / T::BKB, last) - first;
    const int kb = 16 * (((off % T::BKB) >> 4) ^ swz<T::BKB>(off / T::BKB));
    return (unsigned)(row / kPackRows) * (unsigned)packed_group_bytes(p.rowbytes) +
           (unsigned)((kb / kPackBytes) * kPackBlock + (row % kPackRows) * kPackBytes + kb % kPackBytes);
  };
#pragma unroll
  for (int i = 0; i < T::SPWW_MAX; ++i) {
    const int span = min(wave + i * T::NW, T::WSPANS - 1);
    woff[i] = wpk ? span_offset_packed(span, n0, p.V - 1) : span_offset(span, n0, p.V - 1);
  }
  // W source of stage t: the stage's first byte of the tile's first row
  auto wkoff = [&](int stage) -> int64_t {
    const int64_t o = koff(stage);
    return wpk ? (o / kPackBytes) * kPackBlock + o % kPackBytes : o;
  };
  const unsigned lds0 = lds_addr(smem);
  auto issue_x = [&](int stage, int buf) {
    const char *base = xtile + koff(stage);
#pragma unroll
    for (int i = 0; i < T::SPWX_MAX; ++i) {
      const int span = wave + i * T::NW;
      if (T::XSPANS % T::NW == 0 || span < T::XSPANS)
        dma16(xoff[i], base,
              __builtin_amdgcn_readfirstlane(lds0 + buf * T::XSTAGE + span * 1024));
    }
  };
  auto issue_w = [&](int stage, int buf) {
    const char *base = wtile + wkoff(stage);
#pragma unroll
    for (int i = 0; i < T::SPWW_MAX; ++i) {
      const int span = wave + i * T::NW;
      if (T::WSPANS % T::NW == 0 || span < T::WSPANS)
        dma16<T::WNT>(woff[i], base,
                      __builtin_amdgcn_readfirstlane(lds0 + T::WRING + buf * T::WSTAGE + span * 1024));
    }
  };
  // W stages s and s + 1 (those below nst), span by span
  auto issue_w_pair = [&](int s) {
    const char *base0 = wtile + wkoff(s), *base1 = wtile + wkoff(s + 1 < nst ? s + 1 : s);
    const unsigned buf0 = lds0 + T::WRING + (s % T::NSW) * T::WSTAGE;
    const unsigned buf1 = lds0 + T::WRING + ((s + 1) % T::NSW) * T::WSTAGE;
#pragma unroll
    for (int i = 0; i < T::SPWW_MAX; ++i) {
      const int span = wave + i * T::NW;
      if (T::WSPANS % T::NW == 0 || span < T::WSPANS) {
        if (s < nst) dma16<T::WNT>(woff[i], base0, __builtin_amdgcn_readfirstlane(buf0 + span * 1024));
        if (s + 1 < nst)
          dma16<T::WNT>(woff[i], base1, __builtin_amdgcn_readfirstlane(buf1 + span * 1024));
      }
    }
  };

  // ---- fragment offsets (bytes within a stage) of this lane, per k-step:
  // lane (j, h) reads chunk 2 s + h of row j of every 32-row tile
  int a_off[T::STEPS], b_off[T::STEPS];
#pragma unroll
  for (int s = 0; s < T::STEPS; ++s) {
    const int c = (2 * s + h) ^ swz<T::BKB>(j);
    a_off[s] = (wm * T::WM * 32 + j) * T::BKB + 16 * c;
    b_off[s] = (wn * T::WN * 32 + j) * T::BKB + 16 * c;
  }

  acc_t acc[T::WM][T::WN];
#pragma unroll
  for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
    for (int nt = 0; nt < T::WN; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0;

  // ---- main loop: stages in k order (koff), one MFMA chain per logit.
  // Loads: boundary b (after stage b; boundaries -NSW..-1 before the loop)
  // loads, in this order, X stage b + NSX into X buffer b mod NSX and W stage
  // b + NSW into W buffer b mod NSW.  With NSW > NSX, in the loop the X loads
  // are issued at the boundary and the W loads are spread over the next
  // stage's k-steps, so the address unit is not handed a whole stage at once.
  // Stage s is awaited at boundary s - 1, before that boundary's loads: loads
  // complete in issue order and W stage s was issued before X stage s, so it
  // suffices that this wave has at most after(s) loads in flight, the number it
  // issued after X stage s.  With NSW == NSX both stages are issued at the
  // boundary (X, then W) and boundary s - 1 waits for every load in flight,
  // which are exactly stage s's.  With paired W stages (NSX 2, NSW 4) each
  // odd boundary b issues X stage b + 2, then W stages b + 3 and b + 4; W stage
  // s leaves before X stage s, and at most the pair issued after X stage s (s
  // odd) may still be in flight at boundary s - 1.
  // Compute: within a stage, the fragments of k-step s + 1 are read while the
  // MFMAs of step s issue (one read per MFMA, so LDS latency hides behind the
  // matrix pipe); after the stage's last MFMAs every wave waits for stage t + 1,
  // the barrier frees stage t's buffers, boundary t's X loads are issued and the
  // next stage's first fragments are read.
  auto read_frags = [&](const char *xb, const char *wb, int s, i32x4 (&af)[T::WM],
                        i32x4 (&bfr)[T::WN]) {
#pragma unroll
    for (int mt = 0; mt < T::WM; ++mt)
      af[mt] = *(const i32x4 *)(xb + a_off[s] + mt * 32 * T::BKB);
#pragma unroll
    for (int nt = 0; nt < T::WN; ++nt)
      bfr[nt] = *(const i32x4 *)(wb + b_off[s] + nt * 32 * T::BKB);
  };
  auto mfmas = [&](const i32x4 (&af)[T::WM], const i32x4 (&bfr)[T::WN]) {
#pragma unroll
    for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
      for (int nt = 0; nt < T::WN; ++nt) acc[mt][nt] = A::mfma(af[mt], bfr[nt], acc[mt][nt]);
  };
  auto boundary = [&](int b) {  // b >= -NSW; buffers of stages b + NSX, b + NSW
    const int sx = b + T::NSX, sw = b + T::NSW;
    if (sx >= 0 && sx < nst) issue_x(sx, sx % T::NSX);
    if constexpr (T::WPAIR) {
      if (b & 1) issue_w_pair(b + T::NSW - 1);  // odd boundary b: W stages b + 3, b + 4
    } else {
      if (sw < nst) issue_w(sw, sw % T::NSW);
    }
  };
  // loads this wave issued after X stage s, once boundaries <= s - 2 are issued
  // (with W issued at the boundary, after X: wait for everything)
  // (paired W: boundary s - 2, which issued X stage s, then issued W stages
  // s + 1 and s + 2 when s is odd; W stage s went out at boundary s - 3 or s - 4)
  auto after = [&](int s) {
    if constexpr (T::WPAIR) return (s & 1) ? T::SPWW_MIN * ((s + 1 < nst) + (s + 2 < nst)) : 0;
    if constexpr (!T::WSPREAD) return 0;
    int n = s - T::NSX + T::NSW < nst ? T::SPWW_MIN : 0;
    const int lo = s - T::NSX + 1, hi = s - 2;  // whole boundaries after X stage s
    n += T::SPWX_MIN * max(0, min(hi, nst - 1 - T::NSX) - lo + 1);
    n += T::SPWW_MIN * max(0, min(hi, nst - 1 - T::NSW) - lo + 1);
    return n;
  };
#pragma unroll
  for (int b = -T::NSW; b <= -2; ++b) boundary(b);
  wait_vm_le<T::AFTER_MAX>(after(0));  // stage 0 has landed
  lds_barrier();
  boundary(-1);
  i32x4 fa[2][T::WM], fb[2][T::WN];
  read_frags(smem, smem + T::WRING, 0, fa[0], fb[0]);
  // W spans of one boundary, PER of them after each of the first k-steps
  constexpr int PER = (T::SPWW_MAX + T::STEPS - 2) / (T::STEPS - 1);
  auto issue_w_part = [&](int stage, int buf, int i0) {
    const char *base = wtile + wkoff(stage);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int i = i0 + q;
      const int span = wave + i * T::NW;
      if (i < T::SPWW_MAX && (T::WSPANS % T::NW == 0 || span < T::WSPANS))
        dma16<T::WNT>(woff[i < T::SPWW_MAX ? i : 0], base,
                      __builtin_amdgcn_readfirstlane(lds0 + T::WRING + buf * T::WSTAGE + span * 1024));
    }
  };
  // one stage; PEND: this stage carries the W loads of boundary t - 1
  auto stage = [&](int t, auto pend) {
    const int pw = t - 1 + T::NSW;
    const char *xb = smem + (t % T::NSX) * T::XSTAGE;
    const char *wb = smem + T::WRING + (t % T::NSW) * T::WSTAGE;
#pragma unroll
    for (int s = 0; s + 1 < T::STEPS; ++s) {
      const int cur = s & 1;
      read_frags(xb, wb, s + 1, fa[cur ^ 1], fb[cur ^ 1]);
      if constexpr (decltype(pend)::value) issue_w_part(pw, pw % T::NSW, s * PER);
      mfmas(fa[cur], fb[cur]);
      interleave_reads<T::WM + T::WN, T::WM * T::WN>();
    }
    constexpr int last = (T::STEPS - 1) & 1;  // STEPS is even: the next stage starts in slot 0
    mfmas(fa[last], fb[last]);
    if (t + 1 < nst) {
      wait_lgkm0();                            // this wave's reads of stage t
      wait_vm_le<T::AFTER_MAX>(after(t + 1));  // stage t + 1 has landed
      lds_barrier();
      if (t + T::NSX < nst) issue_x(t + T::NSX, t % T::NSX);
      if constexpr (T::WPAIR) {
        if (t & 1) issue_w_pair(t + T::NSW - 1);
      } else if constexpr (!T::WSPREAD) {
        if (t + T::NSW < nst) issue_w(t + T::NSW, t % T::NSW);
      }
      read_frags(smem + ((t + 1) % T::NSX) * T::XSTAGE,
                 smem + T::WRING + ((t + 1) % T::NSW) * T::WSTAGE, 0, fa[last ^ 1], fb[last ^ 1]);
    }
  };
  // stage 0 follows the whole boundary -1; stages 1 .. nst - NSW carry the W
  // loads of the boundary before them (W stages NSW .. nst - 1)
  stage(0, std::false_type{});
  int t = 1;
  if constexpr (T::WSPREAD)
    for (; t <= nst - T::NSW; ++t) stage(t, std::true_type{});
  for (; t < nst; ++t) stage(t, std::false_type{});

  // lane (j, h) of MFMA tile (mt, nt) holds Z[row0 + acc_row(v, h)][col0 + j], v = 0..15
  const int wrow0 = m0 + wm * T::WM * 32;  // first row of this wave
  const int wcol0 = n0 + wn * T::WCOLS;    // first column of this wave

  if constexpr (EPI == kStore) {
#pragma unroll
    for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wrow0 + mt * 32 + acc_row(v, h);
        if (row >= p.B) continue;
#pragma unroll
        for (int nt = 0; nt < T::WN; ++nt) {
          const int col = wcol0 + nt * 32 + j;
          if (col >= p.V) continue;
          const int64_t o = (int64_t)row * p.V + col;
          if constexpr (MODE == 0) {
            const float z = acc[mt][nt][v];
            if (p.round_bf16)
              ((unsigned short *)p.logits)[o] = (unsigned short)bf16_bits(z);
            else
              ((float *)p.logits)[o] = z;
          } else {
            ((int *)p.logits)[o] = acc[mt][nt][v];
          }
        }
      }
    return;
  } else {
    __syncthreads();  // stage buffers are free: reuse LDS for the epilogue exchange
    const int u = rs_value_index(j);  // row value this lane holds after a reduce-scatter
    const bool dup = (j & 1) != 0;    // the two lanes holding a row: write from one

    if constexpr (EPI == kTop2 || EPI == kSample) {
      uint4 *xch = (uint4 *)smem;  // [BM rows][WAVES_N] records
      if constexpr (EPI == kSample) {
        // seeded Gumbel-max: every logit becomes y = z / T + G(seed, position,
        // column) in place (float32 bits), then the y are ranked like logits.
        // One Philox block per (row, 128-column block, column lane) serves the
        // lane's column tiles of that block, word q to the block's tile q.  The
        // loops are unrolled at compile time: a rolled row loop would index the
        // accumulators at run time.
        // The tile's per-row keys and logit factors (1 / T, times the row
        // scale in the int8 head) are staged in LDS first, after the exchange
        // area: one global load per row for the workgroup instead of one
        // dependent load per row value in every lane.
        constexpr int TAB = T::BM * T::WAVES_N * 16;
        static_assert(TAB + T::BM * 20 <= T::LDS, "draw table");
        uint64_t *tseed = (uint64_t *)(smem + TAB);
        uint64_t *tpos = tseed + T::BM;
        float *tcr = (float *)(tpos + T::BM);
        for (int r = tid; r < T::BM; r += T::NT) {
          const int row = m0 + r;
          if (row < p.B) {
            float cr = p.inv_t;
            if constexpr (MODE == 1) cr = (p.scale ? p.scale[row] : 1.0f) * p.inv_t;
            tseed[r] = p.seed[row];
            tpos[r] = (uint64_t)p.position[row];
            tcr[r] = cr;
          }
        }
        __syncthreads();
        static_for<0, T::WM>([&](auto mt_) __attribute__((always_inline)) {
          constexpr int mt = decltype(mt_)::value;
          static_for<0, T::BPW>([&](auto b_) __attribute__((always_inline)) {
            constexpr int b = decltype(b_)::value;
            const int col0 = wcol0 + b * T::NTB * 32 + j;
            const uint32_t ctr = 32u * (uint32_t)(col0 >> 7) + (uint32_t)j;
            // tile of the block this lane's first column falls in (0 unless the
            // block is split over waves)
            const int q0 = (col0 >> 5) & 3;
            static_for<0, 16>([&](auto v_) __attribute__((always_inline)) {
              constexpr int v = decltype(v_)::value;
              const int lr = wm * T::WM * 32 + mt * 32 + acc_row(v, h);
              // rows past B (tile padding) are never ranked: skip their noise
              if (m0 + lr < p.B) {
                const float cr = tcr[lr];
                const uint64_t seed = tseed[lr], pos = tpos[lr];
                uint32_t words[4];
                philox4x32(ctr, 0u, (uint32_t)pos, (uint32_t)(pos >> 32), (uint32_t)seed,
                           (uint32_t)(seed >> 32), words);
#pragma unroll
                for (int k = 0; k < T::NTB; ++k) {
                  const int nt = b * T::NTB + k;
                  const uint32_t wq = T::PARTS == 1 ? words[k] : word_of(words, (q0 + k) & 3);
                  const float y = (float)acc[mt][nt][v] * cr + gumbel_of(wq);
                  acc[mt][nt][v] = vfrom<val_t>(__float_as_int(y));
                }
              }
              // one row value at a time: interleaving the 16 Philox chains would
              // buy nothing here and run out of registers
              __builtin_amdgcn_sched_barrier(0);
            });
          });
        });
#pragma unroll
        for (int mt = 0; mt < T::WM; ++mt) {
          const int lrow = wm * T::WM * 32 + mt * 32 + acc_row(u, h);  // row this lane ends with
#pragma unroll
          for (int b = 0; b < T::BPW; ++b) {
            const int col0 = wcol0 + b * T::NTB * 32 + j;
            Top2 t[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              float y[T::NTB];
#pragma unroll
              for (int k = 0; k < T::NTB; ++k) {
                const float yy = __int_as_float(vbits(acc[mt][b * T::NTB + k][v]));
                y[k] = col0 + 32 * k < p.V ? yy : -__builtin_inff();
              }
              t[v] = lane_top2<T::NTB>(y, ~(unsigned)col0);
            }
            const Top2 r = reduce_scatter(t, j);
            if constexpr (T::PARTS == 1) {
              const int row = m0 + lrow;
              const int blk = wcol0 / kBlockCols + b;
              if (!dup && row < p.B && blk < p.nblocks)
                put_record(&p.records[(int64_t)row * p.nblocks + blk], t2_pack(r));
            } else {
              if (!dup) xch[lrow * T::WAVES_N + wn] = t2_pack(r);
            }
          }
        }
      } else {
        // ROUND: rank the bf16-rounded logits (the bf16-output head)
        auto top2_blocks = [&](auto round) {
#pragma unroll
        for (int mt = 0; mt < T::WM; ++mt) {
          const int lrow = wm * T::WM * 32 + mt * 32 + acc_row(u, h);  // row this lane ends with
#pragma unroll
          for (int b = 0; b < T::BPW; ++b) {
            const int col0 = wcol0 + b * T::NTB * 32 + j;  // this lane's first column of the block
            if (p.B - m0 <= 16) {
              // at most 16 live rows in the tile (batches 1-16, or a last row
              // tile that short): rows 0-15 sit in values v = 0..7 of the first
              // 32-row tile of wave row 0 (row acc_row(v, h)); rows 0-7 in
              // values 0-3, row 0 in value 0 of the lanes with h = 0.  Only the
              // NV values that hold live rows are ranked: the reduce-scatter's
              // halving steps over NV values (j^16, j^15, j^7 in turn; each
              // keeps the bits the earlier ones used), then full merges on the
              // remaining pairings.  The five masks are independent, so each
              // lane merges every other lane once, and a set's top-2 is
              // unique: the records are the ones the full reduce-scatter below
              // writes.
              auto rank_rows = [&](auto nv_) {
                constexpr int NV = decltype(nv_)::value;
                Top2 a[16];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                  val_t z[T::NTB];
#pragma unroll
                  for (int k = 0; k < T::NTB; ++k) {
                    val_t zz = acc[mt][b * T::NTB + k][v];
                    if constexpr (MODE == 0 && decltype(round)::value) zz = bf16_round(zz);
                    z[k] = col0 + 32 * k < p.V ? zz : lowest_of<val_t>();
                  }
                  a[v] = lane_top2<T::NTB>(z, ~(unsigned)col0);
                }
                if constexpr (NV >= 4) rs_step<kX16, NV>(a, j);
                else a[0] = combine(a[0], perm<kX16>(a[0]));
                if constexpr (NV >= 4) rs_step<kMirror, NV / 2>(a, j);
                else a[0] = combine(a[0], perm<kMirror>(a[0]));
                if constexpr (NV >= 8) rs_step<kHalfMirror, NV / 4>(a, j);
                else a[0] = combine(a[0], perm<kHalfMirror>(a[0]));
                Top2 r = combine(a[0], perm<kQuadX2>(a[0]));
                r = combine(r, perm<kQuadX1>(r));
                // the value this lane ends with, and one writer per row
                const int u = NV == 8 ? 4 * ((j >> 4) & 1) + 2 * ((j >> 3) & 1) + ((j >> 2) & 1)
                              : NV == 4 ? 2 * ((j >> 4) & 1) + ((j >> 3) & 1)
                                        : 0;
                const int lr = acc_row(u, h);
                const bool writer = (j & (32 / NV - 1)) == 0 && (NV > 1 || h == 0);
                if (writer && m0 + lr < p.B) {
                  if constexpr (T::PARTS == 1) {
                    const int blk = wcol0 / kBlockCols + b;
                    if (blk < p.nblocks)
                      put_record(&p.records[(int64_t)(m0 + lr) * p.nblocks + blk], t2_pack(r));
                  } else {
                    xch[lr * T::WAVES_N + wn] = t2_pack(r);
                  }
                }
              };
              if (wm == 0 && mt == 0) {
                if (p.B - m0 == 1) rank_rows(std::integral_constant<int, 1>{});
                else if (p.B - m0 <= 8) rank_rows(std::integral_constant<int, 4>{});
                else rank_rows(std::integral_constant<int, 8>{});
              }
              continue;
            }
            Top2 t[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              val_t z[T::NTB];
#pragma unroll
              for (int k = 0; k < T::NTB; ++k) {
                val_t zz = acc[mt][b * T::NTB + k][v];
                if constexpr (MODE == 0 && decltype(round)::value) zz = bf16_round(zz);
                z[k] = col0 + 32 * k < p.V ? zz : lowest_of<val_t>();
              }
              t[v] = lane_top2<T::NTB>(z, ~(unsigned)col0);
            }
            const Top2 r = reduce_scatter(t, j);
            if constexpr (T::PARTS == 1) {
              const int row = m0 + lrow;
              const int blk = wcol0 / kBlockCols + b;
              if (!dup && row < p.B && blk < p.nblocks)
                put_record(&p.records[(int64_t)row * p.nblocks + blk], t2_pack(r));
            } else {
              if (!dup) xch[lrow * T::WAVES_N + wn] = t2_pack(r);
            }
          }
        }
        };
        if (MODE == 0 && p.round_bf16) top2_blocks(std::true_type{});
        else top2_blocks(std::false_type{});
      }
      if constexpr (T::PARTS > 1) {
        __syncthreads();
        if (wn % T::PARTS == 0 && lane < T::WM * 32) {
          const int lrow = wm * T::WM * 32 + lane;
          const int row = m0 + lrow;
          Top2 t = t2_unpack(xch[lrow * T::WAVES_N + wn]);
#pragma unroll
          for (int pp = 1; pp < T::PARTS; ++pp)
            t = t2_merge(t, t2_unpack(xch[lrow * T::WAVES_N + wn + pp]));
          const int blk = wcol0 / kBlockCols;
          if (row < p.B && blk < p.nblocks)
            put_record(&p.records[(int64_t)row * p.nblocks + blk], t2_pack(t));
        }
      }
    } else if constexpr (EPI == kLseInt) {
      // exchange areas for one 32-row tile per wave row: block-part maxima
      // [WAVES_M * 32][WAVES_N] and block-part sums [WAVES_M * 32][WAVES_N]
      int *xmax = (int *)smem;
      uint64_t *xsum = (uint64_t *)(smem + T::WAVES_M * 32 * T::WAVES_N * 4);
      const int xbase = wm * 32;
      // the tile's row logit scales, computed once per row and staged in LDS
      // after the exchange areas (rows past B: scale 0).  The target's logit
      // is not captured here: the fold computes it exactly from x and w.
      constexpr int TAB = (T::WAVES_M * 32 * T::WAVES_N * 12 + 15) / 16 * 16;
      static_assert(TAB + T::BM * (int)sizeof(IntScale) <= T::LDS, "row table");
      IntScale *tsc = (IntScale *)(smem + TAB);
      for (int r = tid; r < T::BM; r += T::NT) {
        const int row = m0 + r;
        IntScale sr{0u, 0, 0};
        if (row < p.B) sr = int_row_scale(p.unit_m, p.unit_e, p.step_m[row], p.step_e[row]);
        tsc[r] = sr;
      }
      __syncthreads();
      static_for<0, T::WM>([&](auto mt_) __attribute__((always_inline)) {
        constexpr int mt = decltype(mt_)::value;
        const int lbase = wm * T::WM * 32 + mt * 32;  // first local row of this m-tile
        // per row value: logit scale
        IntScale sc[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) sc[v] = tsc[lbase + acc_row(v, h)];
        static_for<0, T::BPW>([&](auto b_) __attribute__((always_inline)) {
          constexpr int b = decltype(b_)::value;
          // block max (exact), in every lane
          int mx[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            int m = INT_MIN;
#pragma unroll
            for (int k = 0; k < T::NTB; ++k) {
              const int col = wcol0 + (b * T::NTB + k) * 32 + j;
              const int z = acc[mt][b * T::NTB + k][v];
              if (col < p.V && z > m) m = z;
            }
            mx[v] = allmax32(m);
          }
          if constexpr (T::PARTS > 1) {
            if (j < 16) {
              int mine = mx[0];
#pragma unroll
              for (int v = 1; v < 16; ++v) mine = (j == v) ? mx[v] : mine;
              xmax[(xbase + acc_row(j, h)) * T::WAVES_N + wn] = mine;
            }
            __syncthreads();
            const int g0 = wn - wn % T::PARTS;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int xrow = xbase + acc_row(v, h);
              int m = xmax[xrow * T::WAVES_N + g0];
#pragma unroll
              for (int pp = 1; pp < T::PARTS; ++pp) {
                const int o = xmax[xrow * T::WAVES_N + g0 + pp];
                m = o > m ? o : m;
              }
              mx[v] = m;
            }
          }
          // integer exps of (block max - z), summed exactly; rows past B (tile
          // padding) are never written, so their exps are skipped
          LseI part[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            uint64_t e = 0;
            if (m0 + lbase + acc_row(v, h) < p.B) {
              uint64_t tk[T::NTB];
              uint32_t ek[T::NTB];
#pragma unroll
              for (int k = 0; k < T::NTB; ++k)
                tk[k] = int_nats((uint32_t)mx[v] - (uint32_t)acc[mt][b * T::NTB + k][v], sc[v]);
              iexp_q30_n<T::NTB>(tk, ek);  // the lane's logits of this row value in lockstep
#pragma unroll
              for (int k = 0; k < T::NTB; ++k) {
                const int col = wcol0 + (b * T::NTB + k) * 32 + j;
                e += col < p.V ? ek[k] : 0u;
              }
            }
            part[v] = lse_i(mx[v], e);
          }
          const LseI r = reduce_scatter(part, j);
          const int lrow = lbase + acc_row(u, h);  // local row this lane ends with
          const int blk = wcol0 / kBlockCols + b;
          if constexpr (T::PARTS > 1) {
            if (!dup) xsum[(xbase + acc_row(u, h)) * T::WAVES_N + wn] = r.sum();
            __syncthreads();
            if (wn % T::PARTS == 0 && !dup) {
              uint64_t sum = 0;
#pragma unroll
              for (int pp = 0; pp < T::PARTS; ++pp)
                sum += xsum[(xbase + acc_row(u, h)) * T::WAVES_N + wn + pp];
              const int row = m0 + lrow;
              if (row < p.B && blk < p.nblocks)
                put_record(&p.records[(int64_t)row * p.nblocks + blk],
                           make_uint4((unsigned)r.m, (unsigned)sum, (unsigned)(sum >> 32), 0u));
            }
            __syncthreads();
          } else {
            const int row = m0 + lrow;
            if (!dup && row < p.B && blk < p.nblocks)
              put_record(&p.records[(int64_t)row * p.nblocks + blk],
                         make_uint4((unsigned)r.m, r.lo, r.hi, 0u));
          }
        });
      });
    } else {  // kLse
      // exchange areas for one 32-row tile per wave row: block-part maxima
      // [WAVES_M * 32][WAVES_N] and partial sums [WAVES_M * 32][WAVES_N][32]
      int *xmax = (int *)smem;
      float *xsum = (float *)(smem + T::WAVES_M * 32 * T::WAVES_N * 4);
      const int xbase = wm * 32;  // this wave row's slice of the exchange areas
      // the tile's row targets (float head) and exp2 factors (log2(e) for
      // bf16, s_r log2(e) for int8), staged in LDS once after the exchange areas
      constexpr int TAB = T::WAVES_M * 32 * T::WAVES_N * (4 + 32 * 4);
      static_assert(TAB + T::BM * 8 <= T::LDS, "row table");
      int *ttg = (int *)(smem + TAB);
      float *tcr = (float *)(ttg + T::BM);
      for (int r = tid; r < T::BM; r += T::NT) {
        const int row = m0 + r;
        float c = kLog2e;
        if constexpr (MODE == 1) c = ((p.scale && row < p.B) ? p.scale[row] : 1.0f) * kLog2e;
        if constexpr (MODE == 0) ttg[r] = row < p.B ? p.target[row] : -1;
        tcr[r] = c;
      }
      __syncthreads();
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt) {
        const int lbase = wm * T::WM * 32 + mt * 32;  // first local row of this m-tile
        // per row value: target and exp2 scale
        int tgt[16];
        float cr[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          tgt[v] = MODE == 0 ? ttg[lbase + acc_row(v, h)] : -1;
          cr[v] = tcr[lbase + acc_row(v, h)];
        }
        // target logit capture (the float head; the int8 head's fold computes
        // the exact int32 logit itself)
        if constexpr (MODE == 0) {
#pragma unroll
          for (int nt = 0; nt < T::WN; ++nt) {
            const int col = wcol0 + nt * 32 + j;
#pragma unroll
            for (int v = 0; v < 16; ++v)
              if (col == tgt[v]) p.zt[m0 + lbase + acc_row(v, h)] = vbits(acc[mt][nt][v]);
          }
        }
#pragma unroll
        for (int b = 0; b < T::BPW; ++b) {
          // block max (exact), in every lane
          val_t mx[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            val_t m = lowest_of<val_t>();
#pragma unroll
            for (int k = 0; k < T::NTB; ++k) {
              const int col = wcol0 + (b * T::NTB + k) * 32 + j;
              const val_t z = acc[mt][b * T::NTB + k][v];
              if (col < p.V && z > m) m = z;
            }
            mx[v] = allmax32(m);
          }
          if constexpr (T::PARTS > 1) {
            if (j < 16) {
              // lane j publishes row value j's max (identical in all 32 lanes)
              val_t mine = mx[0];
#pragma unroll
              for (int v = 1; v < 16; ++v) mine = (j == v) ? mx[v] : mine;
              xmax[(xbase + acc_row(j, h)) * T::WAVES_N + wn] = vbits(mine);
            }
            __syncthreads();
            const int g0 = wn - wn % T::PARTS;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
              const int xrow = xbase + acc_row(v, h);
              val_t m = vfrom<val_t>(xmax[xrow * T::WAVES_N + g0]);
#pragma unroll
              for (int pp = 1; pp < T::PARTS; ++pp) {
                const val_t o = vfrom<val_t>(xmax[xrow * T::WAVES_N + g0 + pp]);
                m = o > m ? o : m;
              }
              mx[v] = m;
            }
          }
          // exp terms; tree over this wave's column tiles of the block
          Lse part[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            float e[T::NTB];
#pragma unroll
            for (int k = 0; k < T::NTB; ++k) {
              const int col = wcol0 + (b * T::NTB + k) * 32 + j;
              const val_t z = acc[mt][b * T::NTB + k][v];
              float d;
              if constexpr (MODE == 0) d = z - mx[v];
              else d = -(float)((uint32_t)mx[v] - (uint32_t)z);  // < 2^32, one rounding
              e[k] = col < p.V ? exp2_hw(d * cr[v]) : 0.0f;
            }
            part[v] = Lse{vbits(mx[v]), tree_sum<T::NTB>(e)};
          }
          if constexpr (T::PARTS > 1) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
              xsum[((xbase + acc_row(v, h)) * T::WAVES_N + wn) * 32 + j] = part[v].s;
            __syncthreads();
          }
          if (T::PARTS == 1 || wn % T::PARTS == 0) {
            if constexpr (T::PARTS > 1) {
              // finish the tree over the parts (the upper levels of the 4-tile tree)
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                float ps[T::PARTS];
#pragma unroll
                for (int pp = 0; pp < T::PARTS; ++pp)
                  ps[pp] = xsum[((xbase + acc_row(v, h)) * T::WAVES_N + wn + pp) * 32 + j];
                part[v].s = tree_sum<T::PARTS>(ps);
              }
            }
            const Lse r = reduce_scatter(part, j);
            const int row = m0 + lbase + acc_row(u, h);
            const int blk = wcol0 / kBlockCols + b;
            if (!dup && row < p.B && blk < p.nblocks)
              put_record(&p.records[(int64_t)row * p.nblocks + blk],
                         make_uint4((unsigned)r.m, __float_as_uint(r.s), 0u, 0u));
          }
          if constexpr (T::PARTS > 1) __syncthreads();
        }
      }
    }
  }
}

// the row-parallel log-prob fold: 16 rows per workgroup, in the slot order of
// merge_rows
template <int MODE, int EPI>
__global__ __launch_bounds__(256) void lmhead_merge_kernel(Params p) {
  const int row0 = blockIdx.x * (256 / kSlots);
  merge_rows<MODE, EPI>(p, row0, min(256 / kSlots, p.B - row0), threadIdx.x, 256);
}

// The top-2 fold (greedy and sampling): one wave per row, four rows per
// workgroup, so a batch of 512 spreads over 128 workgroups.  A
// top-2 of a union is exact in any order, so the lane count does not change a
// bit (the log-prob folds keep their fixed slot order in merge_rows).
template <int MODE, int EPI>
__global__ __launch_bounds__(256) void lmhead_merge_top2_kernel(Params p) {
  constexpr int kRowsPerWg = 4;
  const int row0 = blockIdx.x * kRowsPerWg;
  const int row = row0 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int nb = p.nblocks;
  if (row < p.B) {
    const uint4 *rec = p.records + (int64_t)row * nb;
    Top2 t{0, 0};
    // PER records per lane in flight per round: 4 cover rows up to 256
    // blocks in one round, 16 rows up to 1024 blocks (fewer clamped repeats
    // of the last record on short rows)
    auto fold = [&](auto per_) {
      constexpr int PER = decltype(per_)::value;
      for (int b0 = lane; b0 < nb; b0 += 64 * PER) {
        uint4 r[PER];  // all issued (a clamped index stays in bounds), then merged
#pragma unroll
        for (int q = 0; q < PER; ++q) r[q] = rec[min(b0 + 64 * q, nb - 1)];
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if (b0 + 64 * q < nb) t = t2_merge(t, t2_unpack(r[q]));
      }
    };
    if (nb <= 64 * 4) fold(std::integral_constant<int, 4>{});
    else fold(std::integral_constant<int, 16>{});
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) t = t2_merge(t, Top2{__shfl_xor(t.k1, m), __shfl_xor(t.k2, m)});
    if (lane == 0) put_top2<MODE, EPI>(p, row, t);
  }
  if constexpr (MODE == 0 && EPI == kTop2)
    if (p.gated) {
      __shared__ int s_gate[kGateLdsInts];
      gate_rows(p, row0, min(kRowsPerWg, p.B - row0), threadIdx.x, 256, s_gate);
    }
}

// ------------------------------------------------------------ tile plans
// tile shapes, indexed by Plan::variant
//   0: 32 x 128  (batch <= 32)   1: 64 x 128  (<= 64)
//   2: 128 x 128 (<= 128)                    3: 256 x 128 (<= 256)
//   4: 256 x 256 (> 256)
//   5: 32 x 256, 6: 64 x 256 in place of 0 and 1 for the int8 head when the
//      128-column grid would take more than two rounds of the 256 CUs (large
//      vocabularies): half the workgroups, so half the pipeline fills and
//      tails per CU
//   0 with 512-byte stages (V0d) for the float head when rows allow it
//   7: 32 x 512, 8: 64 x 512 in place of 5 and 6 for the int8 head when the
//      512-column grid fits one round of the CUs
//   9: 128 x 256 in place of 2 when ceil(V / 256) >= 256; 10: 128 x 512 for
//      the int8 head where 7 and 8 apply
//   11: 1 with eight waves and an unpaired W ring, for packed W
//   12: 2 with 256-byte stages, for packed W
template <int BKB> using V0w = Tile<32, 256, 1, 4, BKB, 2, 3>;
template <int BKB> using V1w = Tile<64, 256, 2, 2, BKB, 2, 3>;
// int8 head, large vocabularies: 512-column tiles with rings of equal depth
// (2 x 64 KB of W), so the grid takes one round of the CUs where 256-column
// tiles would take two.  Measured on MI355X (4096 x 128256, W from HBM): batch
// 1, 33 and 64 in 98 us against 108-111 us.
template <int BKB> using V0x = Tile<32, 512, 1, 4, BKB, 2, 2>;
template <int BKB> using V1x = Tile<64, 512, 2, 2, BKB, 2, 2>;
constexpr int kCUs = 256;  // MI355X compute units
template <int BKB> using V0 = Tile<32, 128, 1, 4, BKB, 2, 3>;
// V0 with 512 bytes of each row per stage and the W ring as deep as the X ring
// (2 x 16 KB + 2 x 64 KB of LDS): each W row is read 512 contiguous bytes at a
// time.  Measured on MI355X for the 131 MB W stream alone (same pattern, eight
// separately allocated copies): 25.3 us against 28.2 us with 256-byte pieces,
// whose rate also varied from copy to copy (23-31 us).  Float head only: the
// int8 head's rotated k order works in 256-byte units.
using V0d = Tile<32, 128, 1, 4, 512, 2, 2>;
// V1 pairs its W stages (WPAIR): each row's 2 x BKB bytes go out back to back.
// Measured on MI355X (TinyLlama head, W from HBM): batch 33 and 64 in 33.1-33.8
// us against 34.2-35.0 us with a 3-deep spread W ring; the same pairing in
// V3 was 4.5 us slower at batch 256 (its loads are limited by issue, not HBM).
// Eight waves of 32 x 32 (two per SIMD) rather than four of 32 x 64: batch
// 33 / 48 / 64 in 29.64 / 29.58 / 29.66 us against 30.06 / 30.11 / 29.95 us,
// and 30.38 / 30.49 / 30.43 us against 30.49 / 30.64 / 30.51 us on a second box.
template <int BKB> using V1 = Tile<64, 128, 2, 4, BKB, 2, 4, true>;
// V1 reading packed W (float head): every stage is already a contiguous block,
// so the W ring is spread over the k-steps, 3 deep, unpaired.  Measured on
// MI355X (TinyLlama head, packed W from HBM): batch 33 and 64 in 27.1 us against
// 28.7 us with the paired ring (row-major W keeps the paired ring: 30.4 against
// 31.1 us unpaired).  Eight waves of 32 x 32 (two per SIMD) rather than four
// of 32 x 64: batch 33 / 48 / 64 in 27.07 / 26.60 / 26.36 us against 27.25 /
// 27.67 / 27.92 us, and 26.37 / 26.30 / 26.29 us against 26.69 / 28.10 / 28.28
// us on a second box (the 128 x 128 tile with eight waves was 1-2 us slower).
template <int BKB> using V1p = Tile<64, 128, 2, 4, BKB, 2, 3>;
template <int BKB> using V2 = Tile<128, 128, 2, 2, BKB, 2, 4>;
// V2 reading packed W (float head): 256-byte stages, so each stage reads two
// adjacent blocks (32 KB contiguous), with a 3-deep W ring (2 x 32 KB + 3 x
// 32 KB of LDS).  Measured on MI355X (TinyLlama head, packed W from HBM, two
// boxes): batch 65 / 100 / 128 in 29.51 / 29.92 / 30.58 us against 29.66 /
// 30.33 / 31.03 us, and 30.34 / 30.86 / 31.20 us against 31.36 / 31.69 / 32.10 us.
using V2p = Tile<128, 128, 2, 2, 256, 2, 3>;
// batches 65-128 at large vocabularies (ceil(V / 256) >= 256): 256-column
// tiles (and 512-column ones for the int8 head where their grid fits one
// round of the CUs) halve or quarter the X re-reads and the rounds.  Measured
// on MI355X at 4096 x 128256, batch 65-128, bitwise identical: float head
// 183-200 us (65-72% of HBM) against 202-239 us; int8 103-105 us (63%) against
// 128-131 us (51%), 115-117 us with 256-column tiles.
template <int BKB> using V2w = Tile<128, 256, 4, 2, BKB, 2, 3>;
template <int BKB> using V2x = Tile<128, 512, 4, 2, BKB, 2, 2>;
template <int BKB> using V3 = Tile<256, 128, 4, 2, BKB, 2, 4>;
using V4 = Tile<256, 256, 4, 2, 128, 2, 3, false, true>;
// V4 with one row tile (batches 129-256 at large vocabularies): no W tile is
// shared, so W takes the non-temporal policy
using V4n = Tile<256, 256, 4, 2, 128, 2, 3>;
// V4 when the row is not a whole number of its stages
using V4s = Tile<256, 256, 4, 2, 64, 2, 6, false, true>;

}  // namespace
}  // namespace lmh
