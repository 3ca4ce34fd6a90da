// Device helpers shared by the ternary product kernels.
//
// Weight expansion: a 16-B block-64 word holds, in bit pair j of byte b, the
// weight at block offset 16j + b. (w >> 2j) & 0x03030303 therefore gives the
// codes of four consecutive weights in byte order, and one v_perm_b32 with
// the byte table {0xFF, 0x00, 0x01} turns codes {0, 1, 2} into int8
// {-1, 0, +1}. Each MFMA lane feeds 16 consecutive k of its row of codes and
// the same 16 k of its weight column, so both operands share one k order and
// the product is the plain dot product whatever the hardware's k order inside
// a lane is.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr unsigned kCodeLut = 0x000100FFu;      // code 0 -> -1, 1 -> 0, 2 -> +1
constexpr unsigned kZeroWeights = 0x55555555u;  // every field holds code 1 (t = 0)
constexpr float kScaleInt8 = 127.0f;
constexpr float kScaleInt4 = 2.6457513110645906f;  // sqrt 7

__device__ __forceinline__ unsigned expand_word(unsigned w, int j) {
  return __builtin_amdgcn_perm(0u, kCodeLut, (w >> (2 * j)) & 0x03030303u);
}

// Weights 16j .. 16j+15 of a packed 64-weight block as 16 int8 lanes.
__device__ __forceinline__ v4i expand_quarter(const uint4 p, int j) {
  v4i r;
  r.x = (int)expand_word(p.x, j);
  r.y = (int)expand_word(p.y, j);
  r.z = (int)expand_word(p.z, j);
  r.w = (int)expand_word(p.w, j);
  return r;
}

__device__ __forceinline__ uint4 zero_weight_block() {
  return make_uint4(kZeroWeights, kZeroWeights, kZeroWeights, kZeroWeights);
}

// Workgroup barrier that orders LDS traffic only (s_waitcnt lgkmcnt(0) +
// s_barrier). __syncthreads() would also wait for every global load in
// flight, which would drain the loads a kernel issues ahead of their use.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Dequantization factor alpha * s_m / c of output row m.
__device__ __forceinline__ float dequant_factor(float alpha, float s, float c) {
  return (alpha * s) / c;
}

}  // namespace bitnet
