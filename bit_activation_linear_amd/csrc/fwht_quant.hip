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
#include "fwht_row.h"

namespace bitnet {
namespace {

using namespace fwrow;

// BITS = 0: transform only, the normalized fp32 row written to fout (which
// may alias x: a row is read whole before any of it is written).
template <typename XT, int BITS, int L, int LT, bool PRO>
__global__ __launch_bounds__(1 << LT) void fwht_quant_kernel(const XT* x, int8_t* __restrict__ codes,
                                                             float* __restrict__ scales,
                                                             Prologue pro, float* fout,
                                                             int32_t* __restrict__ rowsum,
                                                             bool nib) {
  extern __shared__ float lds[];
  const int row = blockIdx.x;
  float v[1 << (L - LT)];
  load_row<XT, L, LT>(x + (size_t)row * (1 << L), v);
  transform_row<XT, BITS, L, LT, PRO>(v, row, codes, scales, pro, fout, rowsum, nib, lds);
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
  const size_t lds = RowLds<L, LT>::kBytes;
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
