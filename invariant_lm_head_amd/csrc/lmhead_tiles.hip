// The tile kernel and its fold kernel for one (mode, epilogue) pair.  The
// build compiles this file once per pair, with LMH_INST_MODE (0: bf16 x bf16
// -> float32, 1: int8 x int8 -> int32) and LMH_INST_EPI (an Epilogue value)
// set on the command line, so the instances compile in parallel.
#include "lmhead_device.h"

#if !defined(LMH_INST_MODE) || !defined(LMH_INST_EPI)
#error "compile with -DLMH_INST_MODE=<0|1> -DLMH_INST_EPI=<epilogue>"
#endif

namespace lmh {
namespace {

// The contraction, then (reducing epilogues) the per-row fold of its records.
template <class T, int MODE, int EPI>
hipError_t launch_tile(const Params &p, hipStream_t s) {
  hipLaunchKernelGGL((lmhead_tile_kernel<T, MODE, EPI>), dim3(p.grid_m * p.grid_n), dim3(T::NT),
                     0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (EPI == kStore) {
    return e;
  } else if constexpr (EPI == kTop2 || EPI == kSample) {
    // four rows per workgroup
    hipLaunchKernelGGL((lmhead_merge_top2_kernel<MODE, EPI>), dim3((p.B + 3) / 4), dim3(256), 0,
                       s, p);
  } else {
    // 256 / kSlots rows per workgroup (one wave per row)
    hipLaunchKernelGGL((lmhead_merge_kernel<MODE, EPI>),
                       dim3((p.B + 256 / kSlots - 1) / (256 / kSlots)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

template <int MODE, int EPI>
hipError_t launch_epi(const Plan &plan, const Params &p, hipStream_t s) {
  static_assert(MODE == 1 || EPI != kLseInt, "the integer log-softmax is an int8 epilogue");
  switch (plan.variant) {
    case 0:
      if constexpr (MODE == 0)
        if (plan.bkb == V0d::BKB) return launch_tile<V0d, MODE, EPI>(p, s);
      if (plan.bkb == 256) return launch_tile<V0<256>, MODE, EPI>(p, s);
      if (plan.bkb == 128) return launch_tile<V0<128>, MODE, EPI>(p, s);
      return launch_tile<V0<64>, MODE, EPI>(p, s);
    case 1:
      if (plan.bkb == 256) return launch_tile<V1<256>, MODE, EPI>(p, s);
      if (plan.bkb == 128) return launch_tile<V1<128>, MODE, EPI>(p, s);
      return launch_tile<V1<64>, MODE, EPI>(p, s);
    case 2:
      if (plan.bkb == 128) return launch_tile<V2<128>, MODE, EPI>(p, s);
      return launch_tile<V2<64>, MODE, EPI>(p, s);
    case 3:
      if (plan.bkb == 128) return launch_tile<V3<128>, MODE, EPI>(p, s);
      return launch_tile<V3<64>, MODE, EPI>(p, s);
    case 5:
    case 6:
      if constexpr (MODE == 1) {
        if (plan.variant == 5) {
          if (plan.bkb == 128) return launch_tile<V0w<128>, MODE, EPI>(p, s);
          return launch_tile<V0w<64>, MODE, EPI>(p, s);
        }
        if (plan.bkb == 128) return launch_tile<V1w<128>, MODE, EPI>(p, s);
        return launch_tile<V1w<64>, MODE, EPI>(p, s);
      }
      return hipErrorInvalidValue;  // int8 plans only
    case 7:
    case 8:
      if constexpr (MODE == 1) {
        if (plan.variant == 7) {
          if (plan.bkb == 128) return launch_tile<V0x<128>, MODE, EPI>(p, s);
          return launch_tile<V0x<64>, MODE, EPI>(p, s);
        }
        if (plan.bkb == 128) return launch_tile<V1x<128>, MODE, EPI>(p, s);
        return launch_tile<V1x<64>, MODE, EPI>(p, s);
      }
      return hipErrorInvalidValue;  // int8 plans only
    case 11:
      if constexpr (MODE == 0) {
        if (plan.bkb == 256) return launch_tile<V1p<256>, MODE, EPI>(p, s);
        return launch_tile<V1p<128>, MODE, EPI>(p, s);
      }
      return hipErrorInvalidValue;  // packed W: float head only
    case 12:
      if constexpr (MODE == 0) return launch_tile<V2p, MODE, EPI>(p, s);
      return hipErrorInvalidValue;  // packed W: float head only
    case 9:
      if (plan.bkb == 128) return launch_tile<V2w<128>, MODE, EPI>(p, s);
      return launch_tile<V2w<64>, MODE, EPI>(p, s);
    case 10:
      if constexpr (MODE == 1) {
        if (plan.bkb == 128) return launch_tile<V2x<128>, MODE, EPI>(p, s);
        return launch_tile<V2x<64>, MODE, EPI>(p, s);
      }
      return hipErrorInvalidValue;  // int8 plan only
    default:
      if (plan.bkb == V4::BKB) {
        if (p.grid_m == 1) return launch_tile<V4n, MODE, EPI>(p, s);
        return launch_tile<V4, MODE, EPI>(p, s);
      }
      return launch_tile<V4s, MODE, EPI>(p, s);
  }
}

template hipError_t launch_epi<LMH_INST_MODE, LMH_INST_EPI>(const Plan &, const Params &,
                                                            hipStream_t);

}  // namespace lmh
