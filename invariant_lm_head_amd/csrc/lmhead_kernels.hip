// Batch-invariant LM head kernels for gfx950 (CDNA4, MI355X).
//
// One tiled MFMA kernel computes logits Z[b, v] = sum_k X[b, k] * W[v, k] for a
// tile of rows x vocabulary columns and reduces them in its epilogue:
//   kStore  writes Z (float32, bf16-rounded, or int32);
//   kTop2   per-row top-2 (value, id) of every 128-column vocabulary block;
//   kLse    per-row (block max, sum of exp) of every block, and the target logit.
// The block partials of a row are then folded into the outputs by merge_rows(),
// either by the last workgroup of the launch (atomic ticket, small batches) or
// by a second, row-parallel kernel (larger batches); both run the same code.
//
// Batch invariance (one reduction order per logit, fixed by H only):
//   * every logit is acc = 0; for s = 0 .. H*esize/32 - 1: acc = MFMA(A_s, B_s, acc)
//     with ONE instruction for every batch size (v_mfma_f32_32x32x16_bf16 or
//     v_mfma_i32_32x32x32_i8); k-step s covers bytes [32 s, 32 s + 32) of a row,
//     lane half h holding bytes [32 s + 16 h, +16); no split-K; rows of an MFMA
//     are independent, so a row's bits do not depend on its neighbours;
//   * tile shapes change with B only in how many rows and columns a workgroup
//     covers, which does not change any logit's arithmetic;
//   * a block's softmax partial is m_b = max over the block (exact), then
//     s_b = sum exp(z - m_b): for each column offset j (0..31) a balanced binary
//     tree over the block's four 32-column tiles, then a fixed pairing tree over
//     j (j^16, j^15, j^7, j^2, j^1), the same for every row; the row total folds
//     blocks in 16 slots (block b into slot b mod 16, ascending), then a fixed
//     pairing tree over the slots.  All of it depends on V only.  Top-2 with
//     lowest-id ties is exact in any order.
// ("12 Exactness", section 12.2: the reduction order is fixed by the weight's
// shape and never by the row count; "Integer-Only Arithmetic", section "Why
// kernels don't always add in the same order": split-K chosen by batch size.)
//
// Data movement: operand tiles are staged HBM -> LDS with global_load_lds_dwordx4
// (no register round trip), NS stages in flight, 16-byte chunks XOR-swizzled by
// row so the MFMA fragment reads (ds_read_b128) are bank-conflict free.  The
// workgroup -> tile map is XCD-aware: workgroups that share operand tiles run
// on the same XCD (same L2).  Cross-lane reductions use DPP and ds_swizzle.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "lmhead_internal.h"

namespace lmh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;
constexpr int kSlots = 16;  // slots of the final per-row fold
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
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BKB_, int NS_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int BKB = BKB_, NS = NS_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;
  static constexpr int WM = BM / WAVES_M / 32;  // 32-row MFMA tiles per wave
  static constexpr int WN = BN / WAVES_N / 32;  // 32-column MFMA tiles per wave
  static constexpr int STEPS = BKB / 32;        // MFMA k-steps per stage
  static constexpr int STAGE = (BM + BN) * BKB; // LDS bytes per stage
  static constexpr int SPANS = STAGE / 1024;    // 1 KB wave loads per stage
  static constexpr int SPW_MAX = (SPANS + NW - 1) / NW;
  static constexpr int SPW_MIN = SPANS / NW;
  static constexpr int LDS = NS * STAGE;
  static constexpr int WCOLS = WN * 32;         // vocabulary columns per wave
  static constexpr int TPB = kBlockCols / 32;   // column tiles per block (4)
  // a wave covers BPW whole blocks, or PARTS waves share one block
  static constexpr int BPW = WN >= TPB ? WN / TPB : 1;
  static constexpr int PARTS = WN >= TPB ? 1 : TPB / WN;
  static constexpr int NTB = WN >= TPB ? TPB : WN;  // column tiles per block in one wave
  static_assert(BM % (32 * WAVES_M) == 0 && BN % (32 * WAVES_N) == 0, "tile shape");
  static_assert(STAGE % 1024 == 0 && (BM * BKB) % 1024 == 0, "1 KB load spans");
  static_assert(BN % kBlockCols == 0 && (WN % TPB == 0 || TPB % WN == 0), "blocks");
  static_assert(BKB == 64 || BKB == 128 || BKB == 256, "stage width");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(SPW_MIN * (NS - 1) < 64, "vmcnt range");
  static_assert(STEPS % 2 == 0, "fragment double buffer parity");
  // epilogue exchange areas (one 32-row tile per wave row at a time) fit in LDS
  static_assert(WAVES_M * 32 * WAVES_N * (4 + 32 * 4) <= LDS && BM * WAVES_N * 16 <= LDS,
                "exchange");
};

// 16-byte chunk swizzle within a staged row (conflict-free ds_read_b128)
template <int BKB> __device__ __forceinline__ int swz(int row) {
  return BKB >= 128 ? (row & 7) : ((row >> 1) & 3);
}

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));
}

// wait until at most `ahead` (<= K) stages of this wave's loads are still in flight
template <class T, int K> __device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (K <= 0) {
    wait_vm<0>();
  } else {
    if (ahead >= K) {
      wait_vm<K * T::SPW_MIN>();
    } else {
      wait_stages<T, K - 1>(ahead);
    }
  }
}

// 16 bytes per lane global -> LDS (global_load_lds_dwordx4): lane i writes LDS
// bytes [lds + 16 i, +16).  Issued as inline asm so the compiler does not guard
// every later LDS read with a full vmcnt(0) drain; completion is tracked by the
// explicit vmcnt waits of the pipeline (wait_stages) instead.  m0 (the copy's LDS
// base) is saved and restored around it; the s_nop is the one wait state
// required between an SALU write of m0 and its use.
__device__ __forceinline__ void dma16(const void *gptr, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds)
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

// ------------------------------------------------------------ top-2 records
template <class V> struct Top2 {
  V v1, v2;
  int i1, i2;
};
// (a, ia) ranks above (b, ib): larger value, or equal value and lower id
template <class V> __device__ __forceinline__ bool better(V a, int ia, V b, int ib) {
  return (a > b) | ((a == b) & (ia < ib));
}
template <class V> __device__ __forceinline__ Top2<V> t2_neutral() {
  Top2<V> t;
  t.v1 = t.v2 = lowest_of<V>();
  t.i1 = t.i2 = INT_MAX;
  return t;
}
// branch-free: every lane runs the same selects
template <class V> __device__ __forceinline__ void t2_insert(Top2<V> &t, V v, int i) {
  const bool w1 = better(v, i, t.v1, t.i1);
  const bool w2 = better(v, i, t.v2, t.i2);
  const V v2 = w1 ? t.v1 : (w2 ? v : t.v2);
  const int i2 = w1 ? t.i1 : (w2 ? i : t.i2);
  t.v1 = w1 ? v : t.v1;
  t.i1 = w1 ? i : t.i1;
  t.v2 = v2;
  t.i2 = i2;
}
template <class V> __device__ __forceinline__ Top2<V> t2_merge(const Top2<V> &a, const Top2<V> &b) {
  const bool bw = better(b.v1, b.i1, a.v1, a.i1);  // b's best is the overall best
  // runner-up: the loser of the two bests against the winner's own second
  const V lv = bw ? a.v1 : b.v1;
  const int li = bw ? a.i1 : b.i1;
  const V sv = bw ? b.v2 : a.v2;
  const int si = bw ? b.i2 : a.i2;
  const bool lw = better(lv, li, sv, si);
  Top2<V> r;
  r.v1 = bw ? b.v1 : a.v1;
  r.i1 = bw ? b.i1 : a.i1;
  r.v2 = lw ? lv : sv;
  r.i2 = lw ? li : si;
  return r;
}
template <int P, class V> __device__ __forceinline__ Top2<V> perm(const Top2<V> &t) {
  Top2<V> o;
  o.v1 = perm<P>(t.v1); o.i1 = perm_i<P>(t.i1);
  o.v2 = perm<P>(t.v2); o.i2 = perm_i<P>(t.i2);
  return o;
}
template <class V> __device__ __forceinline__ Top2<V> pick(bool c, const Top2<V> &a, const Top2<V> &b) {
  Top2<V> r;
  r.v1 = c ? a.v1 : b.v1; r.i1 = c ? a.i1 : b.i1;
  r.v2 = c ? a.v2 : b.v2; r.i2 = c ? a.i2 : b.i2;
  return r;
}
template <class V> __device__ __forceinline__ uint4 t2_pack(const Top2<V> &t) {
  return make_uint4((unsigned)vbits(t.v1), (unsigned)t.i1, (unsigned)vbits(t.v2), (unsigned)t.i2);
}
template <class V> __device__ __forceinline__ Top2<V> t2_unpack(uint4 r) {
  Top2<V> t;
  t.v1 = vfrom<V>((int)r.x); t.i1 = (int)r.y;
  t.v2 = vfrom<V>((int)r.z); t.i2 = (int)r.w;
  return t;
}

template <class V> __device__ __forceinline__ uint4 kNeutralTop2() {
  return make_uint4((unsigned)vbits(lowest_of<V>()), (unsigned)INT_MAX,
                    (unsigned)vbits(lowest_of<V>()), (unsigned)INT_MAX);
}

// softmax partial carried through the lane tree: the block max (identical on
// both partners of every pairing) and the partial sum
struct Lse {
  int m;  // bits of the block max (float32 or int32)
  float s;
};

template <class V> __device__ __forceinline__ Top2<V> combine(const Top2<V> &a, const Top2<V> &b) {
  return t2_merge(a, b);
}
__device__ __forceinline__ Lse combine(const Lse &a, const Lse &b) { return Lse{a.m, a.s + b.s}; }
template <int P> __device__ __forceinline__ Lse perm(const Lse &x) { return Lse{x.m, perm<P>(x.s)}; }
__device__ __forceinline__ Lse pick(bool c, const Lse &a, const Lse &b) {
  return Lse{c ? a.m : b.m, c ? a.s : b.s};
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
// 16 row values on each of the 32 column lanes -> lane j holds row value
// u(j) = 8 b4 + 4 b3 + 2 b2 + b1 (b = bits of j) combined over all 32 columns,
// in the pairing order j^16, j^15, j^7, j^2, j^1 (the same for every row).
template <class T> __device__ __forceinline__ T reduce_scatter(T (&a)[16], int j) {
  rs_step<kX16, 16>(a, j);
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
template <int MODE, int EPI>
__device__ void merge_rows(const Params &p, int row0, int nrows, int tid, int nthreads) {
  using val_t = typename Arith<MODE>::val_t;
  const int slot = tid & (kSlots - 1);
  const int nb = p.nblocks;
  for (int g = tid / kSlots; g < nrows; g += nthreads / kSlots) {
    const int row = row0 + g;
    const uint4 *rec = p.records + (int64_t)row * nb;
    if constexpr (EPI == kTop2) {
      Top2<val_t> t = t2_neutral<val_t>();
      // 16 records per slot in flight per round (one memory latency per round)
      for (int b0 = slot; b0 < nb; b0 += kChunk * kSlots) {
        uint4 r[kChunk];
#pragma unroll
        for (int q = 0; q < kChunk; ++q) {
          const int b = b0 + q * kSlots;
          r[q] = b < nb ? rec[b] : kNeutralTop2<val_t>();
        }
#pragma unroll
        for (int q = 0; q < kChunk; ++q) t = t2_merge(t, t2_unpack<val_t>(r[q]));
      }
      t = t2_merge(t, perm<kQuadX1>(t));
      t = t2_merge(t, perm<kQuadX2>(t));
      t = t2_merge(t, perm<kHalfMirror>(t));
      t = t2_merge(t, perm<kMirror>(t));
      if (slot == 0) {
        p.top_id[2 * row] = t.i1;
        p.top_id[2 * row + 1] = t.i2;
        if constexpr (MODE == 0) {
          p.top_val[2 * row] = t.v1;
          p.top_val[2 * row + 1] = t.v2;
          p.margin[row] = t.v1 - t.v2;
        } else {
          const float s = p.scale ? p.scale[row] : 1.0f;
          if (p.top_raw) {
            p.top_raw[2 * row] = t.v1;
            p.top_raw[2 * row + 1] = t.v2;
          }
          const bool ok = scale_ok(s);
          const float nan = __builtin_nanf("");
          // one rounding of an exact float64 product (|raw| < 2^31, 24-bit scale)
          p.top_val[2 * row] = ok ? (float)((double)t.v1 * (double)s) : nan;
          p.top_val[2 * row + 1] = ok ? (float)((double)t.v2 * (double)s) : nan;
          p.margin[row] = ok ? (float)((double)(t.v1 - t.v2) * (double)s) : nan;
        }
      }
    } else {
      // pass 1: the row max (exact); pass 2: the sum in slot order
      val_t mx = lowest_of<val_t>();
      for (int b0 = slot; b0 < nb; b0 += kChunk * kSlots) {
        int m[kChunk];
#pragma unroll
        for (int q = 0; q < kChunk; ++q) {
          const int b = b0 + q * kSlots;
          m[q] = b < nb ? (int)rec[b].x : vbits(lowest_of<val_t>());
        }
#pragma unroll
        for (int q = 0; q < kChunk; ++q) {
          const val_t o = vfrom<val_t>(m[q]);
          mx = o > mx ? o : mx;
        }
      }
      val_t o;
      o = perm<kQuadX1>(mx); mx = o > mx ? o : mx;
      o = perm<kQuadX2>(mx); mx = o > mx ? o : mx;
      o = perm<kHalfMirror>(mx); mx = o > mx ? o : mx;
      o = perm<kMirror>(mx); mx = o > mx ? o : mx;
      float cr = kLog2e, sr = 1.0f;
      if constexpr (MODE == 1) {
        sr = p.scale ? p.scale[row] : 1.0f;
        cr = sr * kLog2e;
      }
      float s = 0.0f;
      for (int b0 = slot; b0 < nb; b0 += kChunk * kSlots) {
        uint2 r[kChunk];
#pragma unroll
        for (int q = 0; q < kChunk; ++q) {
          const int b = b0 + q * kSlots;
          r[q] = b < nb ? *(const uint2 *)&rec[b] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int q = 0; q < kChunk; ++q) {
          if (b0 + q * kSlots < nb) {
            float d;
            if constexpr (MODE == 0) d = __uint_as_float(r[q].x) - mx;
            else d = (float)((int)r[q].x - mx);
            s = s + __uint_as_float(r[q].y) * exp2_hw(d * cr);
          }
        }
      }
      s = s + perm<kQuadX1>(s);
      s = s + perm<kQuadX2>(s);
      s = s + perm<kHalfMirror>(s);
      s = s + perm<kMirror>(s);
      if (slot == 0) {
        const int tgt = p.target[row];
        float lp = __builtin_nanf("");
        if (tgt >= 0 && tgt < p.V) {
          if constexpr (MODE == 0) {
            lp = (__int_as_float(p.zt[row]) - mx) - kLn2 * log2_hw(s);
          } else {
            if (scale_ok(sr)) lp = (float)(p.zt[row] - mx) * sr - kLn2 * log2_hw(s);
          }
        }
        p.logprob[row] = lp;
      }
    }
  }
}

// ------------------------------------------------------------------ kernel
template <class T, int MODE, int EPI, bool FUSED>
__global__ __launch_bounds__(T::NT) void lmhead_tile_kernel(Params p) {
  using A = Arith<MODE>;
  using acc_t = typename A::acc_t;
  using val_t = typename A::val_t;
  __shared__ __attribute__((aligned(1024))) char smem[T::LDS];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
  const int j = lane & 31, h = lane >> 5;  // MFMA column lane, lane half

  // ---- workgroup -> tile, XCD-aware: consecutive workgroups are dealt to the 8
  // XCDs in turn, so renumber them XCD-major, then walk GROUP_M row tiles per
  // vocabulary tile so neighbours on one XCD share X and W tiles in its L2.
  int tm, tn;
  {
    const int G = gridDim.x, bid = blockIdx.x, per = G >> 3;
    const int nb = bid < (per << 3) ? (bid & 7) * per + (bid >> 3) : bid;
    constexpr int GROUP_M = 8;
    const int in_group = GROUP_M * p.grid_n;
    const int group = nb / in_group;
    const int first_m = group * GROUP_M;
    const int gsz = min(p.grid_m - first_m, GROUP_M);
    const int rem = nb - group * in_group;
    tm = first_m + rem % gsz;
    tn = rem / gsz;
  }
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  // ---- per-lane source of each 1 KB LDS span this wave fills every stage
  const char *src[T::SPW_MAX];
#pragma unroll
  for (int i = 0; i < T::SPW_MAX; ++i) {
    int span = wave + i * T::NW;
    if (span >= T::SPANS) span = T::SPANS - 1;
    int off = span * 1024 + lane * 16;
    const char *base;
    int r0, rmax;
    if (off < T::BM * T::BKB) {
      base = p.x; r0 = m0; rmax = p.B - 1;
    } else {
      off -= T::BM * T::BKB;
      base = p.w; r0 = n0; rmax = p.V - 1;
    }
    const int row = off / T::BKB;
    const int chunk = ((off % T::BKB) >> 4) ^ swz<T::BKB>(row);
    const int r = min(r0 + row, rmax);  // rows past B / V re-read the last row; masked later
    src[i] = base + (int64_t)r * p.rowbytes + chunk * 16;
  }
  auto issue = [&](int stage, int buf) {
    char *dst = smem + buf * T::STAGE;
#pragma unroll
    for (int i = 0; i < T::SPW_MAX; ++i) {
      const int span = wave + i * T::NW;
      if (T::SPANS % T::NW == 0 || span < T::SPANS)
        dma16(src[i] + (int64_t)stage * T::BKB,
              __builtin_amdgcn_readfirstlane(lds_addr(dst + span * 1024)));
    }
  };

  // ---- fragment offsets (bytes within a stage) of this lane, per k-step:
  // lane (j, h) reads chunk 2 s + h of row j of every 32-row tile
  int a_off[T::STEPS], b_off[T::STEPS];
#pragma unroll
  for (int s = 0; s < T::STEPS; ++s) {
    const int c = (2 * s + h) ^ swz<T::BKB>(j);
    a_off[s] = (wm * T::WM * 32 + j) * T::BKB + 16 * c;
    b_off[s] = T::BM * T::BKB + (wn * T::WN * 32 + j) * T::BKB + 16 * c;
  }

  acc_t acc[T::WM][T::WN];
#pragma unroll
  for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
    for (int nt = 0; nt < T::WN; ++nt)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mt][nt][v] = 0;

  // ---- main loop: k ascending, one MFMA chain per logit.  All NS buffers are
  // filled up front; k-step fragments are double-buffered in registers (step
  // s + 1 is read while step s multiplies); at the end of a stage every wave
  // waits for the next stage, the barrier frees the finished buffer for stage
  // t + NS, and the next stage's first fragments are read before the stage's
  // last MFMAs issue.
  auto read_frags = [&](const char *buf, int s, i32x4 (&af)[T::WM], i32x4 (&bfr)[T::WN]) {
#pragma unroll
    for (int mt = 0; mt < T::WM; ++mt)
      af[mt] = *(const i32x4 *)(buf + a_off[s] + mt * 32 * T::BKB);
#pragma unroll
    for (int nt = 0; nt < T::WN; ++nt)
      bfr[nt] = *(const i32x4 *)(buf + b_off[s] + nt * 32 * T::BKB);
  };
  const int nst = (int)(p.rowbytes / T::BKB);
#pragma unroll
  for (int s = 0; s < T::NS; ++s)
    if (s < nst) issue(s, s);
  wait_stages<T, T::NS - 1>(min(T::NS - 1, nst - 1));  // stage 0 has landed
  lds_barrier();
  i32x4 fa[2][T::WM], fb[2][T::WN];
  read_frags(smem, 0, fa[0], fb[0]);
  for (int t = 0; t < nst; ++t) {
    const char *buf = smem + (t % T::NS) * T::STAGE;
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) {
      const int cur = s & 1;  // STEPS is even, so the parity carries across stages
      if (s + 1 < T::STEPS) {
        read_frags(buf, s + 1, fa[cur ^ 1], fb[cur ^ 1]);
      } else if (t + 1 < nst) {
        wait_lgkm0();                                        // this wave's reads of stage t
        wait_stages<T, T::NS - 2>(min(T::NS - 2, nst - 2 - t));  // stage t + 1 has landed
        lds_barrier();
        if (t + T::NS < nst) issue(t + T::NS, t % T::NS);
        read_frags(smem + ((t + 1) % T::NS) * T::STAGE, 0, fa[cur ^ 1], fb[cur ^ 1]);
      }
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
        for (int nt = 0; nt < T::WN; ++nt)
          acc[mt][nt] = A::mfma(fa[cur][mt], fb[cur][nt], acc[mt][nt]);
    }
  }

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

    if constexpr (EPI == kTop2) {
      uint4 *xch = (uint4 *)smem;  // [BM rows][WAVES_N] records
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt) {
        const int lrow = wm * T::WM * 32 + mt * 32 + acc_row(u, h);  // row this lane ends with
#pragma unroll
        for (int b = 0; b < T::BPW; ++b) {
          Top2<val_t> t[16];
#pragma unroll
          for (int v = 0; v < 16; ++v) t[v] = t2_neutral<val_t>();
#pragma unroll
          for (int k = 0; k < T::NTB; ++k) {
            const int nt = b * T::NTB + k;
            const int col = wcol0 + nt * 32 + j;
            if (col < p.V) {
#pragma unroll
              for (int v = 0; v < 16; ++v) {
                val_t z = acc[mt][nt][v];
                if constexpr (MODE == 0)
                  if (p.round_bf16) z = bf16_round(z);
                t2_insert(t[v], z, col);
              }
            }
          }
          const Top2<val_t> r = reduce_scatter(t, j);
          if constexpr (T::PARTS == 1) {
            const int row = m0 + lrow;
            const int blk = wcol0 / kBlockCols + b;
            if (!dup && row < p.B && blk < p.nblocks)
              p.records[(int64_t)row * p.nblocks + blk] = t2_pack(r);
          } else {
            if (!dup) xch[lrow * T::WAVES_N + wn] = t2_pack(r);
          }
        }
      }
      if constexpr (T::PARTS > 1) {
        __syncthreads();
        if (wn % T::PARTS == 0 && lane < T::WM * 32) {
          const int lrow = wm * T::WM * 32 + lane;
          const int row = m0 + lrow;
          Top2<val_t> t = t2_unpack<val_t>(xch[lrow * T::WAVES_N + wn]);
#pragma unroll
          for (int pp = 1; pp < T::PARTS; ++pp)
            t = t2_merge(t, t2_unpack<val_t>(xch[lrow * T::WAVES_N + wn + pp]));
          const int blk = wcol0 / kBlockCols;
          if (row < p.B && blk < p.nblocks) p.records[(int64_t)row * p.nblocks + blk] = t2_pack(t);
        }
      }
    } else {  // kLse
      // exchange areas for one 32-row tile per wave row: block-part maxima
      // [WAVES_M * 32][WAVES_N] and partial sums [WAVES_M * 32][WAVES_N][32]
      int *xmax = (int *)smem;
      float *xsum = (float *)(smem + T::WAVES_M * 32 * T::WAVES_N * 4);
      const int xbase = wm * 32;  // this wave row's slice of the exchange areas
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt) {
        const int lbase = wm * T::WM * 32 + mt * 32;  // first local row of this m-tile
        // per row value: target and exp2 scale
        int tgt[16];
        float cr[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + lbase + acc_row(v, h);
          tgt[v] = row < p.B ? p.target[row] : -1;
          cr[v] = kLog2e;  // log2(e) (bf16) or s_r log2(e) (int8)
          if constexpr (MODE == 1) cr[v] = ((p.scale && row < p.B) ? p.scale[row] : 1.0f) * kLog2e;
        }
        // target logit capture
#pragma unroll
        for (int nt = 0; nt < T::WN; ++nt) {
          const int col = wcol0 + nt * 32 + j;
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (col == tgt[v]) p.zt[m0 + lbase + acc_row(v, h)] = vbits(acc[mt][nt][v]);
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
              else d = (float)(z - mx[v]);
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
              p.records[(int64_t)row * p.nblocks + blk] =
                  make_uint4((unsigned)r.m, __float_as_uint(r.s), 0u, 0u);
          }
          if constexpr (T::PARTS > 1) __syncthreads();
        }
      }
    }

    if constexpr (FUSED) {
      // ---- the last workgroup of this row tile folds every block of its rows.
      // Every wave's record stores are complete (vmcnt 0) before the barrier;
      // one agent-scope release then publishes them to the other XCDs.
      wait_vm<0>();
      __syncthreads();
      if (tid == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const unsigned prev = atomicAdd(&p.tickets[tm], 1u);
        s_last = prev == (unsigned)(p.grid_n - 1);
      }
      __syncthreads();
      if (!s_last) return;
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      merge_rows<MODE, EPI>(p, m0, min(T::BM, p.B - m0), tid, T::NT);
      if (tid == 0) p.tickets[tm] = 0u;  // leave the workspace zeroed for the next call
    }
  }
}

// the row-parallel fold for larger batches: 16 rows per workgroup
template <int MODE, int EPI>
__global__ __launch_bounds__(256) void lmhead_merge_kernel(Params p) {
  const int row0 = blockIdx.x * (256 / kSlots);
  merge_rows<MODE, EPI>(p, row0, min(256 / kSlots, p.B - row0), threadIdx.x, 256);
}

// ---------------------------------------------------------- small kernels
__global__ void compare_words_kernel(const unsigned *a, const unsigned *b, int64_t n,
                                     unsigned long long *mismatches) {
  unsigned long long c = 0;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    c += a[i] != b[i];
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m);
  if ((threadIdx.x & 63) == 0 && c) atomicAdd(mismatches, c);
}

__global__ void reverse_rows_kernel(const char *src, char *dst, int64_t rows, int64_t rowbytes) {
  const int64_t total = rows * rowbytes;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / rowbytes, c = i % rowbytes;
    dst[(rows - 1 - r) * rowbytes + c] = src[i];
  }
}

// ------------------------------------------------------------ dispatch
// tile shapes, indexed by Plan::variant
//   0: 32 x 128 (batch <= 32, fold fused)   1: 64 x 128 (<= 64)
//   2: 128 x 128 (<= 256)                   3: 256 x 256 (> 256)
#ifndef LMH_V3_TILE
#define LMH_V3_TILE 256, 256, 4, 2, 128, 2
#endif
#ifndef LMH_V2_TILE
#define LMH_V2_TILE 128, 128, 2, 2, BKB, 4
#endif
template <int BKB> using V0 = Tile<32, 128, 1, 4, BKB, 3>;
template <int BKB> using V1 = Tile<64, 128, 2, 2, BKB, 3>;
template <int BKB> using V2 = Tile<LMH_V2_TILE>;
using V3 = Tile<LMH_V3_TILE>;
// V3 when the row is not a whole number of its stages
using V3s = Tile<256, 256, 2, 2, 64, 4>;

template <class T, int MODE, bool FUSED>
hipError_t launch_tile(int epi, const Params &p, hipStream_t s) {
  const dim3 grid(p.grid_m * p.grid_n), block(T::NT);
  switch (epi) {
    case kStore:
      hipLaunchKernelGGL((lmhead_tile_kernel<T, MODE, kStore, false>), grid, block, 0, s, p);
      return hipGetLastError();
    case kTop2:
      hipLaunchKernelGGL((lmhead_tile_kernel<T, MODE, kTop2, FUSED>), grid, block, 0, s, p);
      break;
    default:
      hipLaunchKernelGGL((lmhead_tile_kernel<T, MODE, kLse, FUSED>), grid, block, 0, s, p);
      break;
  }
  if constexpr (!FUSED) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 mgrid((p.B + 256 / kSlots - 1) / (256 / kSlots));
    if (epi == kTop2)
      hipLaunchKernelGGL((lmhead_merge_kernel<MODE, kTop2>), mgrid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((lmhead_merge_kernel<MODE, kLse>), mgrid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int epi, const Plan &plan, const Params &p, hipStream_t s) {
  switch (plan.variant) {
    case 0:
      if (plan.bkb == 256) return launch_tile<V0<256>, MODE, true>(epi, p, s);
      if (plan.bkb == 128) return launch_tile<V0<128>, MODE, true>(epi, p, s);
      return launch_tile<V0<64>, MODE, true>(epi, p, s);
    case 1:
      if (plan.bkb == 256) return launch_tile<V1<256>, MODE, false>(epi, p, s);
      if (plan.bkb == 128) return launch_tile<V1<128>, MODE, false>(epi, p, s);
      return launch_tile<V1<64>, MODE, false>(epi, p, s);
    case 2:
      if (plan.bkb == 128) return launch_tile<V2<128>, MODE, false>(epi, p, s);
      return launch_tile<V2<64>, MODE, false>(epi, p, s);
    default:
      if (plan.bkb == V3::BKB) return launch_tile<V3, MODE, false>(epi, p, s);
      return launch_tile<V3s, MODE, false>(epi, p, s);
  }
}

}  // namespace

Plan plan_for(int64_t B, int64_t rowbytes, int64_t V) {
  Plan pl;
  const int bkb256 = rowbytes % 256 == 0 ? 256 : rowbytes % 128 == 0 ? 128 : 64;
  const int bkb128 = rowbytes % 128 == 0 ? 128 : 64;
  if (B <= 32) {
    pl.variant = 0; pl.bm = 32; pl.bn = 128; pl.bkb = bkb256;
  } else if (B <= 64) {
    pl.variant = 1; pl.bm = 64; pl.bn = 128; pl.bkb = bkb256;
  } else if (B <= 256) {
    pl.variant = 2; pl.bm = V2<128>::BM; pl.bn = V2<128>::BN; pl.bkb = bkb128;
  } else if (rowbytes % V3::BKB == 0) {
    pl.variant = 3; pl.bm = V3::BM; pl.bn = V3::BN; pl.bkb = V3::BKB;
  } else {
    pl.variant = 3; pl.bm = V3s::BM; pl.bn = V3s::BN; pl.bkb = V3s::BKB;
  }
  pl.grid_m = (int)((B + pl.bm - 1) / pl.bm);
  pl.grid_n = (int)((V + pl.bn - 1) / pl.bn);
  return pl;
}

hipError_t launch(int mode, int epi, const Plan &plan, const Params &p, hipStream_t s) {
  return mode == 0 ? launch_mode<0>(epi, plan, p, s) : launch_mode<1>(epi, plan, p, s);
}

hipError_t launch_compare(const void *a, const void *b, int64_t nwords,
                          unsigned long long *mismatches, hipStream_t s) {
  int64_t blocks = (nwords + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(compare_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const unsigned *)a, (const unsigned *)b, nwords, mismatches);
  return hipGetLastError();
}

hipError_t launch_reverse_rows(const void *src, void *dst, int64_t rows, int64_t rowbytes,
                               hipStream_t s) {
  int64_t blocks = (rows * rowbytes + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(reverse_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const char *)src, (char *)dst, rows, rowbytes);
  return hipGetLastError();
}

}  // namespace lmh
