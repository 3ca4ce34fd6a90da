// Device helpers shared by the decode and quantizer kernels: raw activation
// loads that are widened to fp32 later, and wave-wide DPP reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bitnet {

// The same four values loaded raw and widened later, so that the load can be
// issued well before its first use.
template <typename XT>
struct Raw4;
template <>
struct Raw4<float> {
  float4 d;
};
template <>
struct Raw4<uint16_t> {
  uint2 d;
};
__device__ __forceinline__ void raw_load4(const float* x, size_t i, Raw4<float>& r) {
  r.d = *reinterpret_cast<const float4*>(x + i);
}
__device__ __forceinline__ void raw_load4(const uint16_t* x, size_t i, Raw4<uint16_t>& r) {
  r.d = *reinterpret_cast<const uint2*>(x + i);
}
__device__ __forceinline__ void widen4(const Raw4<float>& r, float (&v)[4]) {
  v[0] = r.d.x; v[1] = r.d.y; v[2] = r.d.z; v[3] = r.d.w;
}
__device__ __forceinline__ void widen4(const Raw4<uint16_t>& r, float (&v)[4]) {
  v[0] = __uint_as_float(r.d.x << 16);
  v[1] = __uint_as_float(r.d.x & 0xFFFF0000u);
  v[2] = __uint_as_float(r.d.y << 16);
  v[3] = __uint_as_float(r.d.y & 0xFFFF0000u);
}

// Wave-wide max or sum of non-negative values with DPP row shifts and row
// broadcasts (zero is the identity of both); the fixed order keeps sums
// bitwise reproducible. Every lane gets the result.
template <bool IS_MAX>
__device__ __forceinline__ float wave_reduce(float v) {
#define BITNET_DPP_STEP(ctrl, rmask, bc)                                                      \
  {                                                                                           \
    const float o = __int_as_float(                                                           \
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, rmask, 0xF, bc));             \
    v = IS_MAX ? fmaxf(v, o) : v + o;                                                         \
  }
  BITNET_DPP_STEP(0x111, 0xF, true)   // row_shr:1
  BITNET_DPP_STEP(0x112, 0xF, true)   // row_shr:2
  BITNET_DPP_STEP(0x114, 0xF, true)   // row_shr:4
  BITNET_DPP_STEP(0x118, 0xF, true)   // row_shr:8  -> lane 15 of each row: row total
  BITNET_DPP_STEP(0x142, 0xA, false)  // row_bcast:15 -> lane 31 / 63: two rows
  BITNET_DPP_STEP(0x143, 0xC, false)  // row_bcast:31 -> lane 63: whole wave
#undef BITNET_DPP_STEP
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Wave-wide sum of integers of any sign (zero is the identity), exact, in
// the same DPP steps; every lane gets the result.
__device__ __forceinline__ int wave_sum_int(int v) {
#define BITNET_DPP_ISTEP(ctrl, rmask, bc) v += __builtin_amdgcn_update_dpp(0, v, ctrl, rmask, 0xF, bc);
  BITNET_DPP_ISTEP(0x111, 0xF, true)
  BITNET_DPP_ISTEP(0x112, 0xF, true)
  BITNET_DPP_ISTEP(0x114, 0xF, true)
  BITNET_DPP_ISTEP(0x118, 0xF, true)
  BITNET_DPP_ISTEP(0x142, 0xA, false)
  BITNET_DPP_ISTEP(0x143, 0xC, false)
#undef BITNET_DPP_ISTEP
  return __builtin_amdgcn_readlane(v, 63);
}

}  // namespace bitnet
