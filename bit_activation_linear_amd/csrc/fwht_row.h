// Per-row Walsh-Hadamard transform and per-token quantization, as device
// code shared by the quantizer kernels and by the batched-decode kernel that
// overlaps the transform with its weight stream.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py): fast_hadamard_transform /
// Eq. 3-4 (log2 K stages of (u, v) -> ((u + v)/sqrt2, (u - v)/sqrt2)),
// quantize_act_int8 / Eq. 5 and quantize_act_int4 / Eq. 6.
//
// Every barrier here orders LDS traffic only (lds_barrier): no thread reads
// global memory that another thread of the workgroup wrote, and a kernel
// that has weight loads in flight while it transforms a row must not drain
// them at each barrier.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "decode_common.h"
#include "kernels.h"
#include "ternary_common.h"

namespace bitnet {
namespace fwrow {

constexpr float kEps = 1e-7f;

__device__ __forceinline__ int pad_idx(int i) { return i + (i >> 5); }
// For a and b with no set bit in common (a + b == a | b),
// pad_idx(a + b) == pad_idx(a) + pad_idx(b): with b a compile-time constant
// the second term becomes an immediate LDS offset.

__device__ __forceinline__ void load8(const float* p, float* v) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// bf16 -> fp32 widening is a 16-bit left shift.
__device__ __forceinline__ void load8(const uint16_t* p, float* v) {
  const uint4 a = reinterpret_cast<const uint4*>(p)[0];
  const unsigned w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// Unnormalized butterflies over all log2(N) index bits of a register array.
template <int N>
__device__ __forceinline__ void fwht_regs(float* v) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
}

// Butterfly reductions over groups of W lanes (W = 64, or the whole
// workgroup when it is smaller than a wave, so no lane outside it is read).
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, W));
  return v;
}
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, W);
  return v;
}

// Workgroup reduction of the per-thread statistic (fixed order), T threads.
template <int BITS, int T>
__device__ __forceinline__ float block_stat(float s, float* red) {
  constexpr int W = T < 64 ? T : 64;
  if constexpr (T >= 64)
    s = wave_reduce<BITS == 8>(s);
  else
    s = (BITS == 8) ? group_max<W>(s) : group_sum<W>(s);
  constexpr int NW = (T + 63) / 64;
  if (T >= 64) {
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  } else {
    // fewer than 64 threads: the whole group is one (partial) wave
    if (threadIdx.x == 0) red[0] = s;
  }
  lds_barrier();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = (BITS == 8) ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

// Workgroup reduction of the statistic and of a sum of squares together
// (one barrier), fixed order.
template <int BITS, int T>
__device__ __forceinline__ float2 block_stat2(float s, float q, float* red) {
  constexpr int W = T < 64 ? T : 64;
  if constexpr (T >= 64) {
    s = wave_reduce<BITS == 8>(s);
    q = wave_reduce<false>(q);
  } else {
    s = (BITS == 8) ? group_max<W>(s) : group_sum<W>(s);
    q = group_sum<W>(q);
  }
  constexpr int NW = (T + 63) / 64;
  if (T >= 64) {
    if ((threadIdx.x & 63) == 0) {
      red[threadIdx.x >> 6] = s;
      red[NW + (threadIdx.x >> 6)] = q;
    }
  } else if (threadIdx.x == 0) {
    red[0] = s;
    red[1] = q;
  }
  lds_barrier();
  float r = red[0], rq = red[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    r = (BITS == 8) ? fmaxf(r, red[w]) : r + red[w];
    rq += red[NW + w];
  }
  return make_float2(r, rq);
}

// Input prologue on the 8 consecutive elements at idx of one row (v holds
// x): SwiGLU product silu(x) * up (engine page BitNetV2FFN.forward), the
// sum of squares RMSNorm needs (taken before its weight), then the RMSNorm
// weight (engine page HBitLinear.forward step 1, nn.RMSNorm). The 1/rms
// factor itself is applied through the quantization scale: per-token
// quantization only sees x / stat(x).
template <typename XT>
__device__ __forceinline__ void apply_prologue8(const Prologue& pro, const XT* up_row, int idx,
                                                float* v, float& sq) {
  if (pro.up) {
    float u[8];
    load8(up_row + idx, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = silu(v[e]) * u[e];
  }
  if (pro.rms) {
#pragma unroll
    for (int e = 0; e < 8; ++e) sq += v[e] * v[e];
    if (pro.gamma) {
      float g[8];
      load8(pro.gamma + idx, g);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= g[e];
    }
  }
}

// Eight codes packed into two words: adding 1.5 * 2^23 to the rounded
// product leaves rint(p) (ties to even) in the low bits of the sum, med3
// clamps it, and the code is the sum's low byte -- the same code as
// clip(rint(v * mult)) in three operations. The empty asm keeps the multiply
// from fusing into the add (the product is rounded first).
template <int BITS>
__device__ __forceinline__ uint2 quant_pack8(const float* v, float mult) {
  constexpr float kMagic = 12582912.0f;
  constexpr float lo = kMagic + ((BITS == 8) ? -128.0f : -8.0f);
  constexpr float hi = kMagic + ((BITS == 8) ? 127.0f : 7.0f);
  unsigned b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float pr = v[i] * mult;
    asm volatile("" : "+v"(pr));
    b[i] = __float_as_uint(__builtin_amdgcn_fmed3f(pr + kMagic, lo, hi));
  }
  const unsigned w0 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u) |
                      __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
  const unsigned w1 = __builtin_amdgcn_perm(b[5], b[4], 0x0C0C0400u) |
                      __builtin_amdgcn_perm(b[7], b[6], 0x04000C0Cu);
  return make_uint2(w0, w1);
}

// Nibble form of the eight codes of quant_pack8 (low words: codes 0-3 and
// 4-7 as int8): byte b gets code b in its high nibble and code 4 + b in its
// low nibble.
__device__ __forceinline__ unsigned nibble_word(uint2 w) {
  return ((w.x << 4) & 0xF0F0F0F0u) | (w.y & 0x0F0F0F0Fu);
}

template <int BITS>
struct QConst {
  static constexpr float c = (BITS == 8) ? 127.0f : 2.6457513110645906f;
  static constexpr float lo = (BITS == 8) ? -128.0f : -8.0f;
  static constexpr float hi = (BITS == 8) ? 127.0f : 7.0f;
};

// 4-bit codes as fp8 pairs (the prefill product's code form): bytes P ..
// P + E - 1 of a row (P a multiple of E, E = 8, 16 or 32), where byte
// 32 g + 2 i + h of every 64-weight block holds the code of the block's
// weight 16 g + i + 32 h. lds holds the row (padded index) and mult is the
// code multiplier: the codes clip(rint(v * mult)), the same as quant_pack8's,
// are exact in fp8 E4M3 and in the float sum returned (their sum). The two
// runs of E / 2 elements never cross a padding step.
template <int E>
__device__ __forceinline__ int store_fp8_pairs(const float* lds, int P, float mult, int8_t* crow) {
  static_assert(E == 8 || E == 16 || E == 32, "fp8-pair chunk");
  const int k0 = (P & ~63) + 16 * ((P >> 5) & 1) + ((P & 31) >> 1);
  const int q0 = pad_idx(k0), q1 = pad_idx(k0 + 32);
  float fs = 0.0f;
  unsigned wd[E / 4];
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {
    // word j: elements 2 j and 2 j + 1 of the two runs
    const float z[4] = {lds[q0 + 2 * j], lds[q1 + 2 * j], lds[q0 + 2 * j + 1], lds[q1 + 2 * j + 1]};
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = __builtin_amdgcn_fmed3f(__builtin_rintf(z[e] * mult), QConst<4>::lo, QConst<4>::hi);
      fs += r[e];
    }
    const int lo2 = __builtin_amdgcn_cvt_pk_fp8_f32(r[0], r[1], 0, false);
    wd[j] = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(r[2], r[3], lo2, true);
  }
  if constexpr (E == 8) {
    *reinterpret_cast<uint2*>(crow + P) = make_uint2(wd[0], wd[1]);
  } else {
#pragma unroll
    for (int q = 0; q < E / 16; ++q)
      *reinterpret_cast<uint4*>(crow + P + 16 * q) =
          make_uint4(wd[4 * q], wd[4 * q + 1], wd[4 * q + 2], wd[4 * q + 3]);
  }
  return (int)fs;
}

// One middle chunk: butterflies over index bits [B0, B0 + NB). Thread t owns
// the groups g = t + T*gi (gi < E >> NB); a group is the 2^NB elements
// base(g) + (j << B0). LAST: quantize from registers and store the codes,
// or, with BITS = 0 (transform only), store the normalized fp32 values to frow.
// Workgroup sum of one int per thread (fixed order), T threads; every
// thread gets the total. ired holds one int per wave.
template <int T>
__device__ __forceinline__ int block_isum(int v, int* ired) {
  constexpr int W = T < 64 ? T : 64;
  if constexpr (T >= 64) {
    v = wave_sum_int(v);
  } else {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, W);
  }
  constexpr int NW = (T + 63) / 64;
  if ((threadIdx.x & 63) == 0) ired[threadIdx.x >> 6] = v;
  lds_barrier();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += ired[w];
  return r;
}

template <int L, int LT, int B0, int NB, bool LAST, int BITS, bool PRO>
__device__ __forceinline__ void mid_pass(float* v, float* lds, float* red, int8_t* crow,
                                         float* scale_out, float sq, const Prologue& pro,
                                         float* frow = nullptr, int* ired = nullptr,
                                         int32_t* rs_out = nullptr, bool nib = false,
                                         bool f8 = false) {
  constexpr int T = 1 << LT;
  constexpr int E = 1 << (L - LT);
  constexpr int R = 1 << NB;
  constexpr int G = E / R;
  const int t = threadIdx.x;
  // group base: the bits [B0, B0 + NB) are clear, so base + (j << B0) is
  // base | (j << B0) and its padded index is pad_idx(base) + pad_idx(j << B0)
  int base[G], pbase[G];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = t + T * gi;
    base[gi] = (g & ((1 << B0) - 1)) | ((g >> B0) << (B0 + NB));
    pbase[gi] = pad_idx(base[gi]);
  }
#define BITNET_PJ(j) ((j << B0) + ((j << B0) >> 5))
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int j = 0; j < R; ++j) v[gi * R + j] = lds[pbase[gi] + BITNET_PJ(j)];
#pragma unroll
  for (int gi = 0; gi < G; ++gi) fwht_regs<R>(v + gi * R);

  if (!LAST) {
    // A thread writes back exactly the elements it read, so only the next
    // pass needs the barrier.
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int j = 0; j < R; ++j) lds[pbase[gi] + BITNET_PJ(j)] = v[gi * R + j];
    lds_barrier();
    return;
  }

  // prod of L factors 1/sqrt2 = 2^(-L/2)
  float norm = __builtin_ldexpf(1.0f, -(L >> 1));
  if (L & 1) norm *= 0.70710678118654752f;
  if constexpr (BITS == 0) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int j = 0; j < R; ++j) frow[base[gi] + (j << B0)] = v[gi * R + j] * norm;
    return;
  }
  // The transformed row goes back to LDS (the statistic's barrier below
  // publishes it), so that each thread then quantizes E contiguous elements
  // and writes them with 16-byte stores instead of E single-byte stores.
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int j = 0; j < R; ++j) lds[pbase[gi] + BITNET_PJ(j)] = v[gi * R + j];
#undef BITNET_PJ
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < E; ++i) s = (BITS == 8) ? fmaxf(s, fabsf(v[i])) : s + fabsf(v[i]);
  float sc, mult;
  if constexpr (PRO) {
    // stat of H(x) / rms + eps, and codes c H(x) / (stat of H(x) + eps rms):
    // the same numbers as normalizing first (H is linear).
    const float2 r = block_stat2<BITS, T>(s, sq, red);
    float stat = r.x;
    if (BITS == 4) stat = stat / (float)(1 << L);
    if (pro.rms) {
      const float sraw = stat * norm;
      const float rms = sqrtf(r.y / (float)(1 << L) + pro.norm_eps);
      sc = sraw / rms + kEps;
      mult = (QConst<BITS>::c * norm) / (sraw + kEps * rms);
    } else {  // the plain path's arithmetic, operation for operation
      sc = stat * norm + kEps;
      mult = (QConst<BITS>::c * norm) / sc;
    }
  } else {
    float stat = block_stat<BITS, T>(s, red);
    if (BITS == 4) stat = stat / (float)(1 << L);
    sc = stat * norm + kEps;
    mult = (QConst<BITS>::c * norm) / sc;
  }
  if (t == 0) *scale_out = sc;
  const int e0 = t * E;
  const int pe0 = pad_idx(e0);  // e0 is a multiple of E, c + i < E
  int qs = 0;  // this thread's share of the code sum
  if (BITS == 4 && E <= 32 && f8) {
    qs = store_fp8_pairs<(E <= 32 ? E : 32)>(lds, e0, mult, crow);
  } else {
#pragma unroll
    for (int c = 0; c < E; c += 8) {
      float u[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = lds[pe0 + (c + i) + ((c + i) >> 5)];
      const uint2 w = quant_pack8<BITS>(u, mult);
      if (nib)
        *reinterpret_cast<unsigned*>(crow + ((e0 + c) >> 1)) = nibble_word(w);
      else
        *reinterpret_cast<uint2*>(crow + e0 + c) = w;
      qs = __builtin_amdgcn_sdot4((int)w.y, 0x01010101, __builtin_amdgcn_sdot4((int)w.x, 0x01010101, qs, false), false);
    }
  }
  if (rs_out) {
    const int total = block_isum<T>(qs, ired);
    if (t == 0) *rs_out = total;
  }
}

template <int A, int B>
struct Min {
  static constexpr int value = A < B ? A : B;
};
// Phase A loads of one row: thread t takes the 8-element vectors at
// 8 t + 8 T r, r < E / 8 (T = 2^LT threads, E = 2^(L - LT) elements each).
template <typename XT, int L, int LT>
__device__ __forceinline__ void load_row(const XT* xr, float* v) {
  constexpr int T = 1 << LT;
  constexpr int E = 1 << (L - LT);
  const int t = threadIdx.x;
#pragma unroll
  for (int rh = 0; rh < E / 8; ++rh) load8(xr + 8 * t + 8 * T * rh, v + 8 * rh);
}

// The same loads as load_row, kept raw (no widening) so that a caller can
// issue other loads behind them before it first uses the row.
template <typename XT, int L, int LT>
struct RawRow;
template <int L, int LT>
struct RawRow<uint16_t, L, LT> {
  static constexpr int kVecs = (1 << (L - LT)) / 8;
  uint4 d[kVecs];
  __device__ __forceinline__ void load(const uint16_t* xr) {
#pragma unroll
    for (int rh = 0; rh < kVecs; ++rh)
      d[rh] = *reinterpret_cast<const uint4*>(xr + 8 * threadIdx.x + 8 * (1 << LT) * rh);
  }
  __device__ __forceinline__ void widen(float* v) const {
#pragma unroll
    for (int rh = 0; rh < kVecs; ++rh) {
      const unsigned w[4] = {d[rh].x, d[rh].y, d[rh].z, d[rh].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * rh + 2 * i] = __uint_as_float(w[i] << 16);
        v[8 * rh + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    }
  }
};
template <int L, int LT>
struct RawRow<float, L, LT> {
  static constexpr int kVecs = (1 << (L - LT)) / 8;
  float4 d[2 * kVecs];
  __device__ __forceinline__ void load(const float* xr) {
#pragma unroll
    for (int rh = 0; rh < kVecs; ++rh) {
      const float4* q = reinterpret_cast<const float4*>(xr + 8 * threadIdx.x + 8 * (1 << LT) * rh);
      d[2 * rh] = q[0];
      d[2 * rh + 1] = q[1];
    }
  }
  __device__ __forceinline__ void widen(float* v) const {
#pragma unroll
    for (int i = 0; i < 2 * kVecs; ++i) {
      v[4 * i] = d[i].x; v[4 * i + 1] = d[i].y; v[4 * i + 2] = d[i].z; v[4 * i + 3] = d[i].w;
    }
  }
};

// LDS a row needs: the padded row, then the statistic's reduction slots,
// then the code sum's.
template <int L, int LT>
struct RowLds {
  static constexpr int kRowFloats = (1 << L) + (1 << L) / 32;
  static constexpr int kWaves = ((1 << LT) + 63) / 64;
  static constexpr int kRedFloats = 2 * kWaves + 2;
  static constexpr size_t kBytes = (size_t)(kRowFloats + kRedFloats + kWaves) * 4;
};

// The rest of row `row`, on the E values load_row left in v: the prologue,
// the butterflies of the register bits, the LDS passes of the middle bits and
// the quantization from the last pass. smem holds RowLds<L, LT>::kBytes.
// BITS = 0: transform only, the normalized fp32 row written to fout's row.
template <typename XT, int BITS, int L, int LT, bool PRO>
__device__ __forceinline__ void transform_row(float* v, int row, int8_t* codes, float* scales,
                                              const Prologue& pro, float* fout, int32_t* rowsum,
                                              bool nib, float* smem, bool f8 = false) {
  constexpr int K = 1 << L;
  constexpr int T = 1 << LT;
  constexpr int E = K / T;
  constexpr int e = L - LT;
  static_assert(E >= 8, "at least one 8-element vector per thread");
  float* lds = smem;
  float* red = smem + RowLds<L, LT>::kRowFloats;
  int* ired = reinterpret_cast<int*>(red + RowLds<L, LT>::kRedFloats);
  const int t = threadIdx.x;
  int8_t* crow = BITS ? codes + (size_t)row * (nib ? K / 2 : K) : nullptr;
  float* frow = BITS ? nullptr : fout + (size_t)row * K;
  int32_t* rso = (BITS && rowsum) ? rowsum + row : nullptr;
  float sq = 0.0f;
  if constexpr (PRO) {
    const XT* ur = pro.up ? reinterpret_cast<const XT*>(pro.up) + (size_t)row * K : nullptr;
#pragma unroll
    for (int rh = 0; rh < E / 8; ++rh) apply_prologue8(pro, ur, 8 * t + 8 * T * rh, v + 8 * rh, sq);
  }
  fwht_regs<E>(v);
#pragma unroll
  for (int rh = 0; rh < E / 8; ++rh)
#pragma unroll
    for (int lo = 0; lo < 8; ++lo)
      lds[pad_idx(8 * t) + 8 * T * rh + ((8 * T * rh) >> 5) + lo] = v[8 * rh + lo];
  lds_barrier();

  // Middle bits [3, 3 + LT) in chunks of up to e bits.
  constexpr int NB0 = Min<e, LT>::value;
  constexpr int R1 = LT - NB0;
  constexpr int NB1 = Min<e, (R1 > 0 ? R1 : 1)>::value;
  constexpr int R2 = R1 - NB1;
  constexpr int NB2 = Min<e, (R2 > 0 ? R2 : 1)>::value;
  constexpr int R3 = R2 - NB2;
  constexpr int NB3 = Min<e, (R3 > 0 ? R3 : 1)>::value;
  static_assert(R3 <= NB3, "at most four middle chunks");
  float* sc = BITS ? scales + row : nullptr;
  if constexpr (R1 <= 0) {
    mid_pass<L, LT, 3, NB0, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib, f8);
  } else {
    mid_pass<L, LT, 3, NB0, false, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib, f8);
    if constexpr (R2 <= 0) {
      mid_pass<L, LT, 3 + NB0, NB1, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib, f8);
    } else {
      mid_pass<L, LT, 3 + NB0, NB1, false, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib, f8);
      if constexpr (R3 <= 0) {
        mid_pass<L, LT, 3 + NB0 + NB1, NB2, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib, f8);
      } else {
        mid_pass<L, LT, 3 + NB0 + NB1, NB2, false, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib, f8);
        mid_pass<L, LT, 3 + NB0 + NB1 + NB2, R3, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib, f8);
      }
    }
  }
}

}  // namespace fwrow
}  // namespace bitnet
