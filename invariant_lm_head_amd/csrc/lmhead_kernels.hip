// Plan choice (grid tiling by batch size and vocabulary), dispatch to the
// tile-kernel instances (lmhead_tiles.hip), per-token quantisation and the
// self-check's small kernels, for gfx950.  The device code and the reasons for
// each tile plan are in lmhead_device.h.
#include "lmhead_device.h"

#include <mutex>

namespace lmh {
namespace {

// The workspace of the no-allocation entry point: one array per GPU, held
// until the process ends.  Host code never uses its name as an address (that
// is a host-side stand-in); static_workspace() resolves each device's copy.
static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];

// ------------------------------------------------ per-token quantisation
// One workgroup per row of int32 values x ("Integer-Only Arithmetic", section
// "DetLLM": each token quantised from its own values, so a row's bits never
// depend on the batch).  a = max |x| (exact); the step D = M 2^E is the least
// number with a 15-bit mantissa (2^14 <= M < 2^15) whose 127 multiple covers
// a; q = sign(x) floor(|x| / D + 1/2) (half away from zero), |q| <= 127.  A
// zero row gives q = 0 and D = 2^14 2^-14 = 1.
__global__ __launch_bounds__(256) void quantize_rows_kernel(const int32_t *x, int64_t H, int8_t *q,
                                                            int32_t *step_m, int32_t *step_e) {
  __shared__ unsigned s_max[4];
  const int64_t row = blockIdx.x;
  const int32_t *xr = x + row * H;
  int8_t *qr = q + row * H;
  const int tid = threadIdx.x;
  auto mag = [](int32_t v) -> uint32_t { return v < 0 ? 0u - (uint32_t)v : (uint32_t)v; };
  uint32_t a = 0;
  for (int64_t i = tid; i < H; i += 256) a = max(a, mag(xr[i]));
  for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
  if ((tid & 63) == 0) s_max[tid >> 6] = a;
  __syncthreads();
  a = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  int M = 1 << 14, E = -14;
  if (a != 0u) {
    // e = floor(log2(a / 127)) from the bit length b of a: 127 2^(b-7) < 2^b <= a
    // always, and 127 2^(b-6) <= a iff 64 a >= 127 2^b
    const int b = 31 - __clz((int)a);
    const int e = ((uint64_t)a << 6) >= ((uint64_t)127 << b) ? b - 6 : b - 7;
    E = e - 14;
    uint64_t mm;
    if (E <= 0) {
      mm = (((uint64_t)a << (-E)) + 126u) / 127u;  // ceil(a 2^-E / 127)
    } else {
      // ceil(a / (127 2^E)) = ceil(ceil(a / 2^E) / 127): a shift and a
      // division by a constant (no runtime divisor)
      mm = ((((uint64_t)a + ((uint64_t)1 << E) - 1) >> E) + 126u) / 127u;
    }
    if (mm == (1u << 15)) {
      mm = 1u << 14;
      E += 1;
    }
    M = (int)mm;
  }
  // q = floor((2 n + D) / (2 D)) with n = |x| 2^max(0, -E), D = M 2^max(0, E);
  // the quotient is at most 127, found bit by bit
  const int ls = E < 0 ? -E : 0;
  const uint64_t D2 = (uint64_t)M << (E > 0 ? E + 1 : 1);
  for (int64_t i = tid; i < H; i += 256) {
    const int32_t v = xr[i];
    const uint64_t num = ((uint64_t)mag(v) << (ls + 1)) + (D2 >> 1);
    uint32_t qq = 0;
#pragma unroll
    for (int bit = 6; bit >= 0; --bit) {
      const uint32_t t = qq | (1u << bit);
      if ((uint64_t)t * D2 <= num) qq = t;
    }
    qr[i] = (int8_t)(v < 0 ? -(int)qq : (int)qq);
  }
  if (tid == 0) {
    step_m[row] = M;
    step_e[row] = E;
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

// Row-major bf16 W [V, H] to the packed layout (w_packed_offset): one
// 16-byte piece of the output per thread and step, read from its row; rows
// from V to the end of the last group and each group's unused block are
// written as zeros.
__global__ __launch_bounds__(256) void pack_w_kernel(const char *w, char *out, int64_t V,
                                                     int64_t rowbytes, int64_t n16) {
  const int64_t group = packed_group_bytes(rowbytes), data = kPackRows * rowbytes;
  for (int64_t u = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; u < n16;
       u += (int64_t)gridDim.x * blockDim.x) {
    const int64_t o = 16 * u;
    const int64_t g = o / group, rem = o % group;
    const int64_t c = rem / kPackBlock, in = rem % kPackBlock;
    const int64_t v = g * kPackRows + in / kPackBytes, k = c * kPackBytes + in % kPackBytes;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (rem < data && v < V) val = *(const uint4 *)(w + v * rowbytes + k);
    *(uint4 *)(out + o) = val;
  }
}

__global__ void reverse_rows_kernel(const char *src, char *dst, int64_t rows, int64_t rowbytes) {
  const int64_t total = rows * rowbytes;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / rowbytes, c = i % rowbytes;
    dst[(rows - 1 - r) * rowbytes + c] = src[i];
  }
}

}  // namespace

Plan plan_for(int mode, int64_t B, int64_t rowbytes, int64_t V, bool w_packed) {
  Plan pl;
  const int bkb256 = rowbytes % 256 == 0 ? 256 : rowbytes % 128 == 0 ? 128 : 64;
  const int bkb128 = rowbytes % 128 == 0 ? 128 : 64;
  // Wide tiles (int8 head only) where the 128-column grid takes more than two
  // rounds of the CUs.  256-column tiles are taken only where their grid fills
  // its rounds at least as well as the 128-column one: at 4096 x 151936 (2.32
  // against 4.64 rounds) 128-column tiles measured 10% faster at batches up to
  // 32.  The float head keeps 128-column tiles at batches up to 64: with W
  // streamed non-temporally they measured as fast at 4096 x 128256 and 16%
  // faster at 4096 x 151936.
  auto fill = [](int64_t n) {  // busy share of the CU slots over a grid's rounds
    return (double)n / (double)(((n + kCUs - 1) / kCUs) * kCUs);
  };
  const int64_t n128 = (V + 127) / 128, n256 = (V + 255) / 256;
  const bool big = mode == 1 && n128 > 2 * kCUs;
  const bool wide = big && fill(n256) >= fill(n128);
  const bool wide512 = big && (V + 511) / 512 <= kCUs;
  if (B <= 32 && wide512) {
    pl.variant = 7; pl.bm = V0x<128>::BM; pl.bn = V0x<128>::BN; pl.nt = V0x<128>::NT; pl.bkb = bkb128;
  } else if (B <= 64 && wide512) {
    pl.variant = 8; pl.bm = V1x<128>::BM; pl.bn = V1x<128>::BN; pl.nt = V1x<128>::NT; pl.bkb = bkb128;
  } else if (B <= 32 && wide) {
    pl.variant = 5; pl.bm = V0w<128>::BM; pl.bn = V0w<128>::BN; pl.nt = V0w<128>::NT; pl.bkb = bkb128;
  } else if (B <= 32) {
    pl.variant = 0; pl.bm = V0<256>::BM; pl.bn = V0<256>::BN; pl.nt = V0<256>::NT; pl.bkb = bkb256;
    // 512-byte stages help a row-major W stream; from the packed layout
    // 256-byte stages with a 3-deep ring measured 1.4-1.9 us faster (batch 1-8)
    if (mode == 0 && !w_packed && rowbytes % V0d::BKB == 0) pl.bkb = V0d::BKB;
  } else if (B <= 64 && wide) {
    pl.variant = 6; pl.bm = V1w<128>::BM; pl.bn = V1w<128>::BN; pl.nt = V1w<128>::NT; pl.bkb = bkb128;
  } else if (B <= 64) {
    pl.variant = 1; pl.bm = V1<256>::BM; pl.bn = V1<256>::BN; pl.nt = V1<256>::NT; pl.bkb = bkb256;
    if (mode == 0 && w_packed) { pl.variant = 11; pl.nt = V1p<256>::NT; }  // same tile, 8 waves, W ring unpaired
  } else if (B <= 128 && wide512) {
    pl.variant = 10; pl.bm = V2x<128>::BM; pl.bn = V2x<128>::BN; pl.nt = V2x<128>::NT; pl.bkb = bkb128;
  } else if (B <= 128 && (V + 255) / 256 >= kCUs) {
    pl.variant = 9; pl.bm = V2w<128>::BM; pl.bn = V2w<128>::BN; pl.nt = V2w<128>::NT; pl.bkb = bkb128;
  } else if (B <= 128) {
    pl.variant = 2; pl.bm = V2<128>::BM; pl.bn = V2<128>::BN; pl.nt = V2<128>::NT; pl.bkb = bkb128;
    if (mode == 0 && w_packed && rowbytes % V2p::BKB == 0) { pl.variant = 12; pl.nt = V2p::NT; pl.bkb = V2p::BKB; }
  } else if (B <= 256 && (V + 255) / 256 < kCUs) {
    // 256-column tiles would leave CUs idle: 256 x 128.  Where they fill the
    // CUs (V >= 65281) the 256 x 256 tile below reads X half as often; measured
    // on MI355X at 4096 x 128256, batch 129-256: 10-15% faster (float head),
    // 11-14% (int8).  At batch 65-128 it was 13-30% slower (padded rows).
    pl.variant = 3; pl.bm = V3<128>::BM; pl.bn = V3<128>::BN; pl.nt = V3<128>::NT; pl.bkb = bkb128;
  } else if (rowbytes % V4::BKB == 0) {
    pl.variant = 4; pl.bm = V4::BM; pl.bn = V4::BN; pl.nt = V4::NT; pl.bkb = V4::BKB;
  } else {
    pl.variant = 4; pl.bm = V4s::BM; pl.bn = V4s::BN; pl.nt = V4s::NT; pl.bkb = V4s::BKB;
  }
  pl.grid_m = (int)((B + pl.bm - 1) / pl.bm);
  pl.grid_n = (int)((V + pl.bn - 1) / pl.bn);
  return pl;
}

hipError_t launch(int mode, int epi, const Plan &plan, const Params &p, hipStream_t s) {
  if (mode == 0) {
    switch (epi) {
      case kStore: return launch_epi<0, kStore>(plan, p, s);
      case kTop2: return launch_epi<0, kTop2>(plan, p, s);
      case kLse: return launch_epi<0, kLse>(plan, p, s);
      case kSample: return launch_epi<0, kSample>(plan, p, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (epi) {
    case kStore: return launch_epi<1, kStore>(plan, p, s);
    case kTop2: return launch_epi<1, kTop2>(plan, p, s);
    case kLse: return launch_epi<1, kLse>(plan, p, s);
    case kSample: return launch_epi<1, kSample>(plan, p, s);
    case kLseInt: return launch_epi<1, kLseInt>(plan, p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t static_workspace(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex lock;
  static void *addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(lock);
  if (!addr[dev]) {
    // once per device, with that device current: its copy of the array
    void *a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_quantize(const int32_t *x, int64_t B, int64_t H, int8_t *q, int32_t *step_m,
                           int32_t *step_e, hipStream_t s) {
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)B), dim3(256), 0, s, x, H, q, step_m,
                     step_e);
  return hipGetLastError();
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

hipError_t launch_pack_w(const void *w, void *out, int64_t V, int64_t rowbytes, hipStream_t s) {
  const int64_t n16 = (V + kPackRows - 1) / kPackRows * packed_group_bytes(rowbytes) / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(pack_w_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const char *)w,
                     (char *)out, V, rowbytes, n16);
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
