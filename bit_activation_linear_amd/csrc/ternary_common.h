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

// ---------------------------------------------------------------------------
// Direct-to-LDS staging shared by the MFMA GEMM kernels.
// ---------------------------------------------------------------------------

constexpr int kLdsMax = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kXcds = 8;             // XCDs; workgroup L is dispatched to XCD L % 8
constexpr int kBand = 4;             // M-tiles per band of the XCD-aware tile walk

typedef unsigned u4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): raw (stride 0) dword access;
// loads at or past `bytes` return zero and touch no memory.
__device__ __forceinline__ u4 make_rsrc(const void* base, unsigned bytes) {
  const size_t a = reinterpret_cast<size_t>(base);
  u4 r;
  r.x = (unsigned)a;
  r.y = (unsigned)(a >> 32) & 0xFFFFu;
  r.z = bytes;
  r.w = 0x00020000u;
  return r;
}

// LDS byte address of a pointer into the dynamic shared array.
__device__ __forceinline__ unsigned lds_address(const char* p) {
  typedef const __attribute__((address_space(3))) char lds_char;
  return (unsigned)(size_t)(lds_char*)p;
}

// 16 bytes per lane from buffer offset voff straight into LDS at
// lds + 16 * lane (lds is wave-uniform; the instruction takes it from M0,
// which is saved and restored around it). Written as inline assembly so that
// the compiler, which cannot tell which LDS bytes such a load writes, does not
// wait for it before every LDS read: completion is tracked by hand with
// s_waitcnt vmcnt before the workgroup barrier that publishes a stage.
__device__ __forceinline__ void load_lds16(const u4 rsrc, int voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds)
      : "memory");
}

// 4 bytes per lane from buffer offset voff into LDS at lds + 4 * lane (same
// conventions as load_lds16).
__device__ __forceinline__ void load_lds4(const u4 rsrc, int voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dword %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds)
      : "memory");
}

// XOR applied to the 16-byte chunk index of code row r in LDS.
__device__ __forceinline__ int chunk_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define BITNET_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

}  // namespace bitnet
