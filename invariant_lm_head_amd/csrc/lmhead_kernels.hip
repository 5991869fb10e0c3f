// Batch-invariant LM head kernels for gfx950 (CDNA4, MI355X).
//
// One tiled MFMA kernel computes logits Z[b, v] = sum_k X[b, k] * W[v, k] for a
// tile of rows x vocabulary columns and reduces them in its epilogue:
//   kStore  writes Z (float32, bf16-rounded, or int32);
//   kTop2   per-row top-2 (value, id) per 128-column vocabulary block;
//   kLse    per-row (block max, sum of exp) per block and the target's logit;
// the last workgroup of a row tile (atomic ticket) folds the block partials of
// its rows into the outputs, in the same launch.
//
// Batch invariance (one reduction order per logit, fixed by H only):
//   * every logit is acc = 0; for s = 0 .. H*esize/64 - 1: acc = MFMA(A_s, B_s, acc)
//     with ONE instruction (v_mfma_f32_16x16x32_bf16 or v_mfma_i32_16x16x64_i8),
//     k-step s covering bytes [64 s, 64 s + 64) of the row, lane group g holding
//     bytes [64 s + 16 g, +16); no split-K, nothing depends on B or on the row's
//     position (rows are independent in the MFMA);
//   * tile shapes change with B only in how many rows / columns a workgroup
//     covers, which does not change any logit's arithmetic;
//   * a block's softmax partial is m_b = max over the block (exact), then
//     s_b = sum exp(z - m_b) over a fixed tree: for each column offset j in
//     0..15 a balanced binary tree over the block's 8 column tiles, then an
//     xor-butterfly over j; the row total folds blocks lane-strided (block b on
//     lane b mod 64, ascending) then an xor-butterfly over the 64 lanes.  Both
//     trees depend on V only.  Top-2 with lowest-id ties is exact in any order.
// ("12 Exactness", section 12.2: the reduction order is fixed by the weight's
// shape and never by the row count; "Integer-Only Arithmetic", section "Why
// kernels don't always add in the same order": split-K chosen by batch size.)
//
// Data movement: operand tiles are staged HBM -> LDS with global_load_lds_dwordx4
// (no register round trip), NS stages in flight, 16-byte chunks XOR-swizzled by
// row so the MFMA fragment reads (ds_read_b128) are bank-conflict free.  The
// workgroup -> tile map is XCD-aware: workgroups that share operand tiles run
// on the same XCD (same L2).
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "lmhead_internal.h"

namespace lmh {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.693147180559945309417f;

// ------------------------------------------------------------- arithmetic
template <int MODE> struct Arith;
template <> struct Arith<0> {  // bf16 x bf16 -> float32
  using acc_t = f32x4;
  using val_t = float;
  static __device__ __forceinline__ acc_t mfma(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ float lowest() { return -__builtin_inff(); }
};
template <> struct Arith<1> {  // int8 x int8 -> int32 (exact)
  using acc_t = i32x4;
  using val_t = int;
  static __device__ __forceinline__ acc_t mfma(i32x4 a, i32x4 b, acc_t c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ int lowest() { return INT_MIN; }
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

// --------------------------------------------------------------- tiling
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BKB_, int NS_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int BKB = BKB_, NS = NS_;
  static constexpr int NW = WAVES_M * WAVES_N, NT = NW * 64;
  static constexpr int WM = BM / WAVES_M / 16;  // 16-row MFMA tiles per wave
  static constexpr int WN = BN / WAVES_N / 16;  // 16-column MFMA tiles per wave
  static constexpr int STEPS = BKB / 64;        // MFMA k-steps per stage
  static constexpr int STAGE = (BM + BN) * BKB; // LDS bytes per stage
  static constexpr int SPANS = STAGE / 1024;    // 1 KB wave loads per stage
  static constexpr int SPW_MAX = (SPANS + NW - 1) / NW;
  static constexpr int SPW_MIN = SPANS / NW;
  static constexpr int LDS = NS * STAGE;
  static constexpr int WCOLS = WN * 16;  // vocabulary columns per wave
  // a wave covers whole 128-column blocks (BPW of them), or PARTS waves share one
  static constexpr int BPW = WCOLS >= kBlockCols ? WCOLS / kBlockCols : 1;
  static constexpr int PARTS = WCOLS >= kBlockCols ? 1 : kBlockCols / WCOLS;
  static constexpr int NTB = WCOLS >= kBlockCols ? kBlockCols / 16 : WN;  // tiles per block-part
  static_assert(BM % (16 * WAVES_M) == 0 && BN % (16 * WAVES_N) == 0, "tile shape");
  static_assert(STAGE % 1024 == 0 && (BM * BKB) % 1024 == 0, "1 KB load spans");
  static_assert(BN % kBlockCols == 0, "workgroup covers whole vocabulary blocks");
  static_assert(BKB == 64 || BKB == 128 || BKB == 256, "stage width");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(SPW_MIN * (NS - 2) < 64, "vmcnt range");
};

// 16-byte chunk swizzle within a staged row (conflict-free ds_read_b128)
template <int BKB> __device__ __forceinline__ int swz(int row) {
  return BKB >= 128 ? (row & 7) : ((row >> 1) & 3);
}

template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait until at most `ahead` stages of this wave's loads are still in flight
template <class T, int K = T::NS - 2> __device__ __forceinline__ void wait_stages(int ahead) {
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

// 16 bytes per lane global -> LDS (global_load_lds_dwordx4): lane i writes
// LDS bytes [lds + 16 i, +16).  Issued as inline asm so the compiler does not
// guard every later LDS read with a full vmcnt(0) drain; completion is tracked
// by the explicit vmcnt waits of the pipeline (wait_stages) instead.
// m0 (the LDS base of the copy) is saved and restored around it; the s_nop is
// the one wait state required between an SALU write of m0 and its use.
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
template <class V> __device__ __forceinline__ bool better(V a, int ia, V b, int ib) {
  return a > b || (a == b && ia < ib);
}
template <class V> __device__ __forceinline__ void t2_init(Top2<V> &t, V lowest) {
  t.v1 = t.v2 = lowest;
  t.i1 = t.i2 = INT_MAX;
}
template <class V> __device__ __forceinline__ void t2_insert(Top2<V> &t, V v, int i) {
  if (better(v, i, t.v1, t.i1)) {
    t.v2 = t.v1; t.i2 = t.i1;
    t.v1 = v; t.i1 = i;
  } else if (better(v, i, t.v2, t.i2)) {
    t.v2 = v; t.i2 = i;
  }
}
template <class V> __device__ __forceinline__ void t2_merge(Top2<V> &a, const Top2<V> &b) {
  if (better(b.v1, b.i1, a.v1, a.i1)) {
    Top2<V> r;
    r.v1 = b.v1; r.i1 = b.i1;
    if (better(a.v1, a.i1, b.v2, b.i2)) { r.v2 = a.v1; r.i2 = a.i1; }
    else { r.v2 = b.v2; r.i2 = b.i2; }
    a = r;
  } else if (better(b.v1, b.i1, a.v2, a.i2)) {
    a.v2 = b.v1; a.i2 = b.i1;
  }
}
template <class V> __device__ __forceinline__ int vbits(V v) { return __builtin_bit_cast(int, v); }
template <class V> __device__ __forceinline__ V vfrom(int b) { return __builtin_bit_cast(V, b); }

template <class V> __device__ __forceinline__ Top2<V> t2_shfl_xor(const Top2<V> &t, int m) {
  Top2<V> o;
  o.v1 = vfrom<V>(__shfl_xor(vbits(t.v1), m));
  o.v2 = vfrom<V>(__shfl_xor(vbits(t.v2), m));
  o.i1 = __shfl_xor(t.i1, m);
  o.i2 = __shfl_xor(t.i2, m);
  return o;
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

// balanced binary tree sum of N values (left + right at every level)
template <int N> __device__ __forceinline__ float tree_sum(const float *e) {
  if constexpr (N == 1) {
    return e[0];
  } else {
    return tree_sum<N / 2>(e) + tree_sum<N / 2>(e + N / 2);
  }
}

// ------------------------------------------------------------------ kernel
template <class T, int MODE, int EPI>
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
  const int fr = lane & 15, fg = lane >> 4;

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

  // ---- fragment offsets (bytes within a stage) of this lane, per k-step
  int a_off[T::STEPS], b_off[T::STEPS];
#pragma unroll
  for (int s = 0; s < T::STEPS; ++s) {
    const int c = (4 * s + fg) ^ swz<T::BKB>(fr);
    a_off[s] = (wm * T::WM * 16 + fr) * T::BKB + 16 * c;
    b_off[s] = T::BM * T::BKB + (wn * T::WN * 16 + fr) * T::BKB + 16 * c;
  }

  acc_t acc[T::WM][T::WN];
#pragma unroll
  for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
    for (int nt = 0; nt < T::WN; ++nt) acc[mt][nt] = acc_t{0, 0, 0, 0};

  // ---- main loop: k ascending, one MFMA chain per logit
  const int nst = (int)(p.rowbytes / T::BKB);
#pragma unroll
  for (int s = 0; s < T::NS - 1; ++s)
    if (s < nst) issue(s, s);
  for (int t = 0; t < nst; ++t) {
    wait_stages<T>(min(T::NS - 2, nst - 1 - t));
    lds_barrier();
    if (t + T::NS - 1 < nst) issue(t + T::NS - 1, (t + T::NS - 1) % T::NS);
    const char *buf = smem + (t % T::NS) * T::STAGE;
#pragma unroll
    for (int s = 0; s < T::STEPS; ++s) {
      i32x4 af[T::WM], bfr[T::WN];
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt)
        af[mt] = *(const i32x4 *)(buf + a_off[s] + mt * 16 * T::BKB);
#pragma unroll
      for (int nt = 0; nt < T::WN; ++nt)
        bfr[nt] = *(const i32x4 *)(buf + b_off[s] + nt * 16 * T::BKB);
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
        for (int nt = 0; nt < T::WN; ++nt) acc[mt][nt] = A::mfma(af[mt], bfr[nt], acc[mt][nt]);
    }
  }

  // lane (fr, fg) of MFMA tile (mt, nt) holds Z[row0 + 4 fg + q][col0 + fr], q = 0..3
  const int wrow0 = m0 + wm * T::WM * 16;        // first row of this wave
  const int wcol0 = n0 + wn * T::WCOLS;          // first column of this wave

  if constexpr (EPI == kStore) {
#pragma unroll
    for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wrow0 + mt * 16 + 4 * fg + q;
        if (row >= p.B) continue;
#pragma unroll
        for (int nt = 0; nt < T::WN; ++nt) {
          const int col = wcol0 + nt * 16 + fr;
          if (col >= p.V) continue;
          const int64_t o = (int64_t)row * p.V + col;
          if constexpr (MODE == 0) {
            const float z = acc[mt][nt][q];
            if (p.round_bf16)
              ((unsigned short *)p.logits)[o] = (unsigned short)bf16_bits(z);
            else
              ((float *)p.logits)[o] = z;
          } else {
            ((int *)p.logits)[o] = acc[mt][nt][q];
          }
        }
      }
    return;
  } else {
    __syncthreads();  // stage buffers are free: reuse LDS for the epilogue exchange

    if constexpr (EPI == kTop2) {
      // exchange area: [BM rows][WAVES_N] records
      uint4 *xch = (uint4 *)smem;
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lrow = wm * T::WM * 16 + mt * 16 + 4 * fg + q;
          const int row = m0 + lrow;
#pragma unroll
          for (int b = 0; b < T::BPW; ++b) {
            Top2<val_t> t;
            t2_init(t, A::lowest());
#pragma unroll
            for (int k = 0; k < T::NTB; ++k) {
              const int nt = b * T::NTB + k;
              const int col = wcol0 + nt * 16 + fr;
              val_t z = acc[mt][nt][q];
              if constexpr (MODE == 0)
                if (p.round_bf16) z = bf16_round(z);
              if (col < p.V) t2_insert(t, z, col);
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) t2_merge(t, t2_shfl_xor(t, m));
            if constexpr (T::PARTS == 1) {
              const int blk = wcol0 / kBlockCols + b;
              if (fr == 0 && row < p.B && blk < p.nblocks)
                p.records[(int64_t)row * p.nblocks + blk] = t2_pack(t);
            } else {
              if (fr == 0) xch[lrow * T::WAVES_N + wn] = t2_pack(t);
            }
          }
        }
      if constexpr (T::PARTS > 1) {
        __syncthreads();
        if (wn % T::PARTS == 0 && lane < T::WM * 16) {
          const int lrow = wm * T::WM * 16 + lane;
          const int row = m0 + lrow;
          Top2<val_t> t = t2_unpack<val_t>(xch[lrow * T::WAVES_N + wn]);
#pragma unroll
          for (int pp = 1; pp < T::PARTS; ++pp)
            t2_merge(t, t2_unpack<val_t>(xch[lrow * T::WAVES_N + wn + pp]));
          const int blk = wcol0 / kBlockCols;
          if (row < p.B && blk < p.nblocks) p.records[(int64_t)row * p.nblocks + blk] = t2_pack(t);
        }
      }
    } else {  // kLse
      // exchange areas: block-part maxima [BM][WAVES_N], partial sums [BM][WAVES_N][16]
      int *xmax = (int *)smem;
      float *xsum = (float *)(smem + T::BM * T::WAVES_N * 4);
#pragma unroll
      for (int mt = 0; mt < T::WM; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lrow = wm * T::WM * 16 + mt * 16 + 4 * fg + q;
          const int row = m0 + lrow;
          const int tgt = row < p.B ? p.target[row] : -1;
          float cr = kLog2e;  // exp2 scale: log2(e) (bf16) or s_r log2(e) (int8)
          if constexpr (MODE == 1) {
            const float sr = (p.scale && row < p.B) ? p.scale[row] : 1.0f;
            cr = sr * kLog2e;
          }
          // target logit capture
#pragma unroll
          for (int nt = 0; nt < T::WN; ++nt) {
            const int col = wcol0 + nt * 16 + fr;
            if (col == tgt) p.zt[row] = vbits(acc[mt][nt][q]);
          }
#pragma unroll
          for (int b = 0; b < T::BPW; ++b) {
            // block max (exact)
            val_t mx = A::lowest();
#pragma unroll
            for (int k = 0; k < T::NTB; ++k) {
              const int col = wcol0 + (b * T::NTB + k) * 16 + fr;
              const val_t z = acc[mt][b * T::NTB + k][q];
              if (col < p.V && z > mx) mx = z;
            }
#pragma unroll
            for (int m = 1; m < 16; m <<= 1) {
              const val_t o = vfrom<val_t>(__shfl_xor(vbits(mx), m));
              mx = o > mx ? o : mx;
            }
            if constexpr (T::PARTS > 1) {
              if (fr == 0) xmax[lrow * T::WAVES_N + wn] = vbits(mx);
              __syncthreads();
              const int g0 = wn - wn % T::PARTS;
              mx = vfrom<val_t>(xmax[lrow * T::WAVES_N + g0]);
#pragma unroll
              for (int pp = 1; pp < T::PARTS; ++pp) {
                const val_t o = vfrom<val_t>(xmax[lrow * T::WAVES_N + g0 + pp]);
                mx = o > mx ? o : mx;
              }
            }
            // exp terms, tree over this wave's column tiles of the block
            float e[T::NTB];
#pragma unroll
            for (int k = 0; k < T::NTB; ++k) {
              const int col = wcol0 + (b * T::NTB + k) * 16 + fr;
              const val_t z = acc[mt][b * T::NTB + k][q];
              float d;
              if constexpr (MODE == 0) d = z - mx;
              else d = (float)(z - mx);
              e[k] = col < p.V ? exp2_hw(d * cr) : 0.0f;
            }
            float u = tree_sum<T::NTB>(e);
            if constexpr (T::PARTS == 1) {
#pragma unroll
              for (int m = 1; m < 16; m <<= 1) u = u + __shfl_xor(u, m);
              const int blk = wcol0 / kBlockCols + b;
              if (fr == 0 && row < p.B && blk < p.nblocks)
                p.records[(int64_t)row * p.nblocks + blk] =
                    make_uint4((unsigned)vbits(mx), __float_as_uint(u), 0u, 0u);
            } else {
              xsum[(lrow * T::WAVES_N + wn) * 16 + fr] = u;
              // the part-0 wave finishes the tree over parts, then the butterfly
              __syncthreads();
              if (wn % T::PARTS == 0) {
                float parts[T::PARTS];
#pragma unroll
                for (int pp = 0; pp < T::PARTS; ++pp)
                  parts[pp] = xsum[(lrow * T::WAVES_N + wn + pp) * 16 + fr];
                u = tree_sum<T::PARTS>(parts);
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) u = u + __shfl_xor(u, m);
                const int blk = wcol0 / kBlockCols;
                if (fr == 0 && row < p.B && blk < p.nblocks)
                  p.records[(int64_t)row * p.nblocks + blk] =
                      make_uint4((unsigned)vbits(mx), __float_as_uint(u), 0u, 0u);
              }
              __syncthreads();
            }
          }
        }
    }

    // ---- last workgroup of this row tile folds every block of its rows
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = atomicAdd(&p.tickets[tm], 1u);
      s_last = prev == (unsigned)(p.grid_n - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    const int rend = min(m0 + T::BM, p.B);
    for (int row = m0 + wave; row < rend; row += T::NW) {
      const uint4 *rec = p.records + (int64_t)row * p.nblocks;
      if constexpr (EPI == kTop2) {
        Top2<val_t> t;
        t2_init(t, A::lowest());
        for (int b = lane; b < p.nblocks; b += 64) t2_merge(t, t2_unpack<val_t>(rec[b]));
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) t2_merge(t, t2_shfl_xor(t, m));
        if (lane == 0) {
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
        val_t mx = A::lowest();
        for (int b = lane; b < p.nblocks; b += 64) {
          const val_t o = vfrom<val_t>((int)rec[b].x);
          mx = o > mx ? o : mx;
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const val_t o = vfrom<val_t>(__shfl_xor(vbits(mx), m));
          mx = o > mx ? o : mx;
        }
        float cr = kLog2e, sr = 1.0f;
        if constexpr (MODE == 1) {
          sr = p.scale ? p.scale[row] : 1.0f;
          cr = sr * kLog2e;
        }
        float s = 0.0f;
        for (int b = lane; b < p.nblocks; b += 64) {
          const uint4 r = rec[b];
          float d;
          if constexpr (MODE == 0) d = __uint_as_float(r.x) - mx;
          else d = (float)((int)r.x - mx);
          s = s + __uint_as_float(r.y) * exp2_hw(d * cr);
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) s = s + __shfl_xor(s, m);
        if (lane == 0) {
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
    if (tid == 0) p.tickets[tm] = 0u;  // leave the workspace zeroed for the next call
  }
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
//   0: 16 x 128 (batch <= 16)   1: 64 x 128 (<= 64)   2: 128 x 128 (<= 256)   3: 256 x 256
template <int BKB> using V0 = Tile<16, 128, 1, 4, BKB, 4>;
template <int BKB> using V1 = Tile<64, 128, 2, 2, BKB, 4>;
template <int BKB> using V2 = Tile<128, 128, 2, 2, BKB, 4>;
using V3 = Tile<256, 256, 2, 2, 64, 4>;

template <class T, int MODE>
hipError_t launch_tile(int epi, const Params &p, hipStream_t s) {
  const dim3 grid(p.grid_m * p.grid_n), block(T::NT);
  switch (epi) {
    case kStore: hipLaunchKernelGGL((lmhead_tile_kernel<T, MODE, kStore>), grid, block, 0, s, p); break;
    case kTop2: hipLaunchKernelGGL((lmhead_tile_kernel<T, MODE, kTop2>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((lmhead_tile_kernel<T, MODE, kLse>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_mode(int epi, const Plan &plan, const Params &p, hipStream_t s) {
  switch (plan.variant) {
    case 0:
      if (plan.bkb == 256) return launch_tile<V0<256>, MODE>(epi, p, s);
      if (plan.bkb == 128) return launch_tile<V0<128>, MODE>(epi, p, s);
      return launch_tile<V0<64>, MODE>(epi, p, s);
    case 1:
      if (plan.bkb == 128) return launch_tile<V1<128>, MODE>(epi, p, s);
      return launch_tile<V1<64>, MODE>(epi, p, s);
    case 2:
      if (plan.bkb == 128) return launch_tile<V2<128>, MODE>(epi, p, s);
      return launch_tile<V2<64>, MODE>(epi, p, s);
    default:
      return launch_tile<V3, MODE>(epi, p, s);
  }
}

}  // namespace

Plan plan_for(int64_t B, int64_t rowbytes, int64_t V) {
  Plan pl;
  if (B <= 16) {
    pl.variant = 0; pl.bm = 16; pl.bn = 128;
    pl.bkb = rowbytes % 256 == 0 ? 256 : rowbytes % 128 == 0 ? 128 : 64;
  } else if (B <= 64) {
    pl.variant = 1; pl.bm = 64; pl.bn = 128;
    pl.bkb = rowbytes % 128 == 0 ? 128 : 64;
  } else if (B <= 256) {
    pl.variant = 2; pl.bm = 128; pl.bn = 128;
    pl.bkb = rowbytes % 128 == 0 ? 128 : 64;
  } else {
    pl.variant = 3; pl.bm = 256; pl.bn = 256; pl.bkb = 64;
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
