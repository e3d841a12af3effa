// Scans and reductions over the 64 lanes of a wave by DPP register moves. A lane shuffle is an LDS round trip
// (about 100 clocks), so a six-step shuffle scan is several hundred clocks of dependent latency; these moves stay
// in the vector unit. The scan shifts by 1, 2, 4 and 8 lanes inside each row of 16 lanes, then adds the row
// broadcasts of lanes 15 and 31; lanes a move has no source for take the operation's identity. The reductions
// return lane 63's total to every lane. All 64 lanes of the wave must be active.
#pragma once

#include "pa_common.h"

namespace pa {

#define PA_DPP(id, x, ctrl, rmask) __builtin_amdgcn_update_dpp((id), (x), (ctrl), (rmask), 0xf, false)

// Inclusive prefix sum over the lanes.
__device__ __forceinline__ int dpp_incl_scan_i(int v) {
  v += PA_DPP(0, v, 0x111, 0xf);  // row_shr:1
  v += PA_DPP(0, v, 0x112, 0xf);  // row_shr:2
  v += PA_DPP(0, v, 0x114, 0xf);  // row_shr:4
  v += PA_DPP(0, v, 0x118, 0xf);  // row_shr:8
  v += PA_DPP(0, v, 0x142, 0xa);  // row_bcast:15 into rows 1 and 3
  v += PA_DPP(0, v, 0x143, 0xc);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ int dpp_sum_i(int v) { return __builtin_amdgcn_readlane(dpp_incl_scan_i(v), 63); }

__device__ __forceinline__ float dpp_sum_f(float x) {
  int v = __float_as_int(x);
  const int z = __float_as_int(0.f);
  v = __float_as_int(__int_as_float(v) + __int_as_float(PA_DPP(z, v, 0x111, 0xf)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(PA_DPP(z, v, 0x112, 0xf)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(PA_DPP(z, v, 0x114, 0xf)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(PA_DPP(z, v, 0x118, 0xf)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(PA_DPP(z, v, 0x142, 0xa)));
  v = __float_as_int(__int_as_float(v) + __int_as_float(PA_DPP(z, v, 0x143, 0xc)));
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

__device__ __forceinline__ float dpp_max_f(float x) {
  int v = __float_as_int(x);
  const int ninf = __float_as_int(-INFINITY);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(PA_DPP(ninf, v, 0x111, 0xf))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(PA_DPP(ninf, v, 0x112, 0xf))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(PA_DPP(ninf, v, 0x114, 0xf))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(PA_DPP(ninf, v, 0x118, 0xf))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(PA_DPP(ninf, v, 0x142, 0xa))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(PA_DPP(ninf, v, 0x143, 0xc))));
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}

#undef PA_DPP

// Lane j's value (j wave-uniform), in every lane.
__device__ __forceinline__ float lane_of(float v, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

}  // namespace pa
