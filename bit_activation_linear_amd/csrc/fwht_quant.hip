// Fused online Walsh-Hadamard transform + per-token activation quantization.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py):
//   - fast_hadamard_transform / Eq. 3-4: the orthonormal Sylvester transform,
//     log2 K stages of (u, v) -> ((u + v)/sqrt2, (u - v)/sqrt2).
//   - quantize_act_int8 / Eq. 5: s = max|x| + eps, q = RoundClip(127 x / s, -128, 127).
//   - quantize_act_int4 / Eq. 6: s = mean|x| + eps, q = RoundClip(sqrt7 x / s, -8, 7).
//
// One workgroup per token row; the row is widened to fp32 and never rounded
// to a narrower type or written back to HBM. The transform's stages commute
// (H_K is a Kronecker product of H_2 factors), so they are grouped by index
// bit:
//   phase A  each thread loads 16-B vectors (8 consecutive elements) from E/8
//            places spread K/(E/8) apart, and runs the butterflies of index
//            bits 0-2 and of the top log2(E)-3 bits in registers;
//   middle   the remaining index bits (those that tell threads apart) are
//            covered in chunks of up to log2(E) bits: the row goes through
//            LDS, each thread pulls the groups of elements that differ only
//            in the chunk's bits, and runs those butterflies in registers;
//   last     the final chunk stays in registers: the per-token statistic is
//            reduced over the workgroup and the codes are written straight
//            from there.
// The 1/sqrt2 of every stage is folded into one multiplier applied with the
// quantization scale. LDS layout: element i at float index i + i/32.
//
// Without the transform the row stays in registers end to end.
//
// Optional input prologue (PRO): the SwiGLU product silu(x) * up and the
// RMSNorm of the engine page's HBitLinear.forward, applied as each vector is
// loaded. The norm's 1/rms never touches the elements: its sum of squares is
// reduced together with the statistic (one barrier), and it enters only the
// scale and the code multiplier.
#include "kernels.h"
#include "decode_common.h"

namespace bitnet {
namespace {

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
  __syncthreads();
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
  __syncthreads();
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
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) r += ired[w];
  return r;
}

template <int L, int LT, int B0, int NB, bool LAST, int BITS, bool PRO>
__device__ __forceinline__ void mid_pass(float* v, float* lds, float* red, int8_t* crow,
                                         float* scale_out, float sq, const Prologue& pro,
                                         float* frow = nullptr, int* ired = nullptr,
                                         int32_t* rs_out = nullptr, bool nib = false) {
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
    __syncthreads();
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
  if (rs_out) {
    const int total = block_isum<T>(qs, ired);
    if (t == 0) *rs_out = total;
  }
}

template <int A, int B>
struct Min {
  static constexpr int value = A < B ? A : B;
};

// BITS = 0: transform only, the normalized fp32 row written to fout (which
// may alias x: a row is read whole before any of it is written).
template <typename XT, int BITS, int L, int LT, bool PRO>
__global__ __launch_bounds__(1 << LT) void fwht_quant_kernel(const XT* x, int8_t* __restrict__ codes,
                                                             float* __restrict__ scales,
                                                             Prologue pro, float* fout,
                                                             int32_t* __restrict__ rowsum,
                                                             bool nib) {
  constexpr int K = 1 << L;
  constexpr int T = 1 << LT;
  constexpr int E = K / T;
  constexpr int e = L - LT;
  static_assert(E >= 8, "at least one 8-element vector per thread");
  extern __shared__ float lds[];
  __shared__ float red[2 * ((T + 63) / 64) + 2];
  __shared__ int ired[(T + 63) / 64];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const XT* xr = x + (size_t)row * K;
  int8_t* crow = BITS ? codes + (size_t)row * (nib ? K / 2 : K) : nullptr;
  float* frow = BITS ? nullptr : fout + (size_t)row * K;
  int32_t* rso = (BITS && rowsum) ? rowsum + row : nullptr;

  // Phase A: vectors of 8 from E/8 places, butterflies of the register bits.
  float v[E];
#pragma unroll
  for (int rh = 0; rh < E / 8; ++rh) load8(xr + 8 * t + 8 * T * rh, v + 8 * rh);
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
  __syncthreads();

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
    mid_pass<L, LT, 3, NB0, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib);
  } else {
    mid_pass<L, LT, 3, NB0, false, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib);
    if constexpr (R2 <= 0) {
      mid_pass<L, LT, 3 + NB0, NB1, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib);
    } else {
      mid_pass<L, LT, 3 + NB0, NB1, false, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib);
      if constexpr (R3 <= 0) {
        mid_pass<L, LT, 3 + NB0 + NB1, NB2, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib);
      } else {
        mid_pass<L, LT, 3 + NB0 + NB1, NB2, false, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib);
        mid_pass<L, LT, 3 + NB0 + NB1 + NB2, R3, true, BITS, PRO>(v, lds, red, crow, sc, sq, pro, frow, ired, rso, nib);
      }
    }
  }
}

// No transform: thread t owns the 8-element vectors at 8t + 2048c, c < CH.
template <typename XT, int BITS, int CH, bool PRO>
__global__ __launch_bounds__(256) void quant_rows_kernel(const XT* __restrict__ x, int K,
                                                         int8_t* __restrict__ codes,
                                                         float* __restrict__ scales, Prologue pro,
                                                         int32_t* __restrict__ rowsum,
                                                         bool nib) {
  constexpr int T = 256;
  __shared__ float red[8];
  __shared__ int ired[4];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const XT* xr = x + (size_t)row * K;
  const XT* ur = (PRO && pro.up) ? reinterpret_cast<const XT*>(pro.up) + (size_t)row * K : nullptr;
  float v[CH][8];
  float s = 0.0f, sq = 0.0f;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = 8 * t + 8 * T * c;
    if (idx < K) {
      load8(xr + idx, v[c]);
      if constexpr (PRO) apply_prologue8(pro, ur, idx, v[c], sq);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) s = (BITS == 8) ? fmaxf(s, fabsf(v[c][e])) : s + fabsf(v[c][e]);
  }
  float sc, mult;
  if constexpr (PRO) {
    // stat(x) / rms + eps, codes c x / (stat(x) + eps rms): the numbers of
    // normalizing first.
    const float2 r = block_stat2<BITS, T>(s, sq, red);
    const float sraw = (BITS == 4) ? r.x / (float)K : r.x;
    if (pro.rms) {
      const float rms = sqrtf(r.y / (float)K + pro.norm_eps);
      sc = sraw / rms + kEps;
      mult = QConst<BITS>::c / (sraw + kEps * rms);
    } else {  // the plain path's arithmetic, operation for operation
      sc = sraw + kEps;
      mult = QConst<BITS>::c / sc;
    }
  } else {
    float stat = block_stat<BITS, T>(s, red);
    if (BITS == 4) stat = stat / (float)K;
    sc = stat + kEps;
    mult = QConst<BITS>::c / sc;
  }
  if (t == 0) scales[row] = sc;
  int8_t* crow = codes + (size_t)row * (nib ? K / 2 : K);
  int qs = 0;  // this thread's share of the code sum
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = 8 * t + 8 * T * c;
    if (idx < K) {
      const uint2 w = quant_pack8<BITS>(v[c], mult);
      if (nib)
        *reinterpret_cast<unsigned*>(crow + (idx >> 1)) = nibble_word(w);
      else
        *reinterpret_cast<uint2*>(crow + idx) = w;
      qs = __builtin_amdgcn_sdot4((int)w.y, 0x01010101,
                                  __builtin_amdgcn_sdot4((int)w.x, 0x01010101, qs, false), false);
    }
  }
  if (rowsum) {
    const int total = block_isum<T>(qs, ired);
    if (t == 0) rowsum[row] = total;
  }
}

template <typename Kern>
hipError_t ensure_lds(Kern kern, size_t bytes) {
  if (bytes <= 48 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename XT, int BITS, int L, int LT, bool PRO>
hipError_t launch_fwht(const void* x, int64_t M, int8_t* codes, float* scales, const Prologue& pro,
                       hipStream_t stream, float* fout = nullptr, int32_t* rowsum = nullptr,
                       bool nib = false) {
  constexpr int K = 1 << L;
  const size_t lds = (size_t)(K + K / 32) * sizeof(float);
  auto kern = fwht_quant_kernel<XT, BITS, L, LT, PRO>;
  hipError_t e = ensure_lds(kern, lds);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)M), dim3(1 << LT), lds, stream>>>(reinterpret_cast<const XT*>(x), codes,
                                                          scales, pro, fout, rowsum, nib);
  return hipGetLastError();
}

// log2 of the threads per row. Elements per thread E = K / threads: more of
// them means fewer LDS passes and barriers per row, but more registers and
// fewer waves to hide latency. Measured on bf16 rows with int4 codes: for a
// batch (all rows resident together) E = 8 is best up to K = 512, E = 16 at
// K = 1024 - 4096 and E = 32 from K = 8192 on, at most 1024 threads
// (K = 16384: 17.1 us for 1024 rows against 24.9 with E = 64; K = 32768:
// 20.9 against 37.9 with E = 128). For a handful of long rows (M <= 64,
// decode) E = 8 up to K = 2048, E = 16 at K = 4096 and 8192 (M = 16,
// K = 8192: 4.30 us against 4.93 with E = 8) and E = 32 from K = 16384 on
// (M = 16, K = 16384: 5.09 us against 5.65 with E = 16).
constexpr int fwht_lt_batch(int L) { return L <= 9 ? L - 3 : (L <= 12 ? L - 4 : (L - 5 < 10 ? L - 5 : 10)); }
constexpr int fwht_lt_few(int L) {
  return L <= 11 ? (L - 3 < 10 ? L - 3 : 10) : (L <= 13 ? L - 4 : (L - 5 < 10 ? L - 5 : 10));
}

template <typename XT, int BITS, int L, bool PRO>
hipError_t launch_fwht_l(const void* x, int64_t M, int8_t* codes, float* scales,
                         const Prologue& pro, hipStream_t stream, float* fout = nullptr,
                         int32_t* rowsum = nullptr, bool nib = false) {
  constexpr int LT_BATCH = fwht_lt_batch(L);
  constexpr int LT_FEW = fwht_lt_few(L);
  if (M <= 64 && LT_FEW != LT_BATCH)
    return launch_fwht<XT, BITS, L, LT_FEW, PRO>(x, M, codes, scales, pro, stream, fout, rowsum, nib);
  return launch_fwht<XT, BITS, L, LT_BATCH, PRO>(x, M, codes, scales, pro, stream, fout, rowsum, nib);
}

// Transform only (fp32 rows in and out, in place allowed).
template <int L>
hipError_t launch_fwht_f32_l(const float* x, int64_t M, float* out, hipStream_t stream) {
  const Prologue none{nullptr, nullptr, 0.0f, 0};
  return launch_fwht_l<float, 0, L, false>(x, M, nullptr, nullptr, none, stream, out);
}

template <typename XT, int BITS, bool PRO>
hipError_t launch_had(const void* x, int64_t M, int K, int8_t* codes, float* scales,
                      const Prologue& pro, hipStream_t stream, int32_t* rowsum, bool nib) {
  switch (K) {
    case 1 << 6: return launch_fwht_l<XT, BITS, 6, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 7: return launch_fwht_l<XT, BITS, 7, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 8: return launch_fwht_l<XT, BITS, 8, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 9: return launch_fwht_l<XT, BITS, 9, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 10: return launch_fwht_l<XT, BITS, 10, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 11: return launch_fwht_l<XT, BITS, 11, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 12: return launch_fwht_l<XT, BITS, 12, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 13: return launch_fwht_l<XT, BITS, 13, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 14: return launch_fwht_l<XT, BITS, 14, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    case 1 << 15: return launch_fwht_l<XT, BITS, 15, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib);
    default: return hipErrorInvalidValue;
  }
}

template <typename XT, int BITS, int CH, bool PRO>
hipError_t launch_rows_ch(const void* x, int64_t M, int K, int8_t* codes, float* scales,
                          const Prologue& pro, hipStream_t stream, int32_t* rowsum, bool nib) {
  quant_rows_kernel<XT, BITS, CH, PRO><<<dim3((unsigned)M), dim3(256), 0, stream>>>(
      reinterpret_cast<const XT*>(x), K, codes, scales, pro, rowsum, nib);
  return hipGetLastError();
}

template <typename XT, int BITS, bool PRO>
hipError_t launch_rows(const void* x, int64_t M, int K, int8_t* codes, float* scales,
                       const Prologue& pro, hipStream_t stream, int32_t* rowsum, bool nib) {
  const int ch = (K + 2047) / 2048;
  if (ch <= 1) return launch_rows_ch<XT, BITS, 1, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib);
  if (ch <= 2) return launch_rows_ch<XT, BITS, 2, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib);
  if (ch <= 4) return launch_rows_ch<XT, BITS, 4, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib);
  if (ch <= 8) return launch_rows_ch<XT, BITS, 8, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib);
  return launch_rows_ch<XT, BITS, 16, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib);
}

template <typename XT, bool PRO>
hipError_t launch_dtype(const void* x, int64_t M, int K, int bits, int hadamard, int8_t* codes,
                        float* scales, const Prologue& pro, hipStream_t stream, int32_t* rowsum,
                        bool nib) {
  if (hadamard) {
    return bits == 8 ? launch_had<XT, 8, PRO>(x, M, K, codes, scales, pro, stream, rowsum, false)
                     : launch_had<XT, 4, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib);
  }
  return bits == 8 ? launch_rows<XT, 8, PRO>(x, M, K, codes, scales, pro, stream, rowsum, false)
                   : launch_rows<XT, 4, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib);
}

}  // namespace

hipError_t launch_fwht_f32(const float* x, int64_t M, int K, float* out, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  switch (K) {
    case 1 << 6: return launch_fwht_f32_l<6>(x, M, out, stream);
    case 1 << 7: return launch_fwht_f32_l<7>(x, M, out, stream);
    case 1 << 8: return launch_fwht_f32_l<8>(x, M, out, stream);
    case 1 << 9: return launch_fwht_f32_l<9>(x, M, out, stream);
    case 1 << 10: return launch_fwht_f32_l<10>(x, M, out, stream);
    case 1 << 11: return launch_fwht_f32_l<11>(x, M, out, stream);
    case 1 << 12: return launch_fwht_f32_l<12>(x, M, out, stream);
    case 1 << 13: return launch_fwht_f32_l<13>(x, M, out, stream);
    case 1 << 14: return launch_fwht_f32_l<14>(x, M, out, stream);
    case 1 << 15: return launch_fwht_f32_l<15>(x, M, out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_quantize(const void* x, int x_dtype, int64_t M, int K, int bits, int hadamard,
                           int8_t* codes, float* scales, hipStream_t stream, const Prologue* pro,
                           int32_t* rowsum, bool nibbles) {
  if (nibbles && (bits != 4 || K % 8 != 0)) return hipErrorInvalidValue;
  const Prologue none{nullptr, nullptr, 0.0f, 0};
  if (pro) {
    if (x_dtype == 1)
      return launch_dtype<uint16_t, true>(x, M, K, bits, hadamard, codes, scales, *pro, stream, rowsum, nibbles);
    return launch_dtype<float, true>(x, M, K, bits, hadamard, codes, scales, *pro, stream, rowsum, nibbles);
  }
  if (x_dtype == 1)
    return launch_dtype<uint16_t, false>(x, M, K, bits, hadamard, codes, scales, none, stream, rowsum, nibbles);
  return launch_dtype<float, false>(x, M, K, bits, hadamard, codes, scales, none, stream, rowsum, nibbles);
}

}  // namespace bitnet
