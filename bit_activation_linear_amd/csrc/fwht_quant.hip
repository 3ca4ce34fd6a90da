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
#include <type_traits>

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
                                                             bool nib, bool f8) {
  extern __shared__ float lds[];
  const int row = blockIdx.x;
  float v[1 << (L - LT)];
  load_row<XT, L, LT>(x + (size_t)row * (1 << L), v);
  transform_row<XT, BITS, L, LT, PRO>(v, row, codes, scales, pro, fout, rowsum, nib, lds, f8);
}

// No transform: thread t owns the 8-element vectors at 8t + 2048c, c < CH.
template <typename XT, int BITS, int CH, bool PRO>
__global__ __launch_bounds__(256) void quant_rows_kernel(const XT* __restrict__ x, int K,
                                                         int8_t* __restrict__ codes,
                                                         float* __restrict__ scales, Prologue pro,
                                                         int32_t* __restrict__ rowsum,
                                                         bool nib, bool tl2) {
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
  // TL2 order (the batched TL2 product's code form): rows of whole 384-code
  // blocks, the code of weight 3 j + p of a block at its byte 128 p + j, the
  // codes past K zero.
  const int ktl2 = (K + kTl2BlockK - 1) / kTl2BlockK * kTl2BlockK;
  int8_t* crow = codes + (size_t)row * (tl2 ? ktl2 : (nib ? K / 2 : K));
  int qs = 0;  // this thread's share of the code sum
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int idx = 8 * t + 8 * T * c;
    if (idx < K) {
      const uint2 w = quant_pack8<BITS>(v[c], mult);
      if (tl2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = idx + e, kb = k / kTl2BlockK, r = k - kb * kTl2BlockK;
          crow[kb * kTl2BlockK + 128 * (r % 3) + r / 3] =
              (int8_t)(((e < 4 ? w.x : w.y) >> (8 * (e & 3))) & 0xFFu);
        }
      } else if (nib)
        *reinterpret_cast<unsigned*>(crow + (idx >> 1)) = nibble_word(w);
      else
        *reinterpret_cast<uint2*>(crow + idx) = w;
      qs = __builtin_amdgcn_sdot4((int)w.y, 0x01010101,
                                  __builtin_amdgcn_sdot4((int)w.x, 0x01010101, qs, false), false);
    }
  }
  if (tl2) {
    for (int k = K + t; k < ktl2; k += T) {
      const int kb = k / kTl2BlockK, r = k - kb * kTl2BlockK;
      crow[kb * kTl2BlockK + 128 * (r % 3) + r / 3] = 0;
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
                       bool nib = false, bool f8 = false) {
  const size_t lds = RowLds<L, LT>::kBytes;
  auto kern = fwht_quant_kernel<XT, BITS, L, LT, PRO>;
  hipError_t e = ensure_lds(kern, lds);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)M), dim3(1 << LT), lds, stream>>>(reinterpret_cast<const XT*>(x), codes,
                                                          scales, pro, fout, rowsum, nib, f8);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 rows, K >= 2048: six index bits on the matrix cores.
//
// The 64-point factor of H_K over index bits 0-2 and 8-10 (engine page
// Eq. 3-4: H_K is a Kronecker product of one factor per index bit, applied in
// any order) is a dense 64 x 64 matrix of +-1, exact in bf16, and so are the
// bf16 inputs: each wave multiplies its 32 groups of 64 elements by it with
// v_mfma_f32_32x32x16_bf16 (exact products, fp32 sums), straight from the
// loaded rows. That replaces six of the log2 K butterfly stages, the
// widening of the inputs and one LDS pass. The rest: index bits 3, 4, 6, 7
// sit in each lane's accumulator registers and are butterflied there; bit 5
// (the lane half) and the wave bits 11 .. L-1 go through one LDS pass; the
// last pass quantizes as the other quantizer does. Values stay unnormalized
// until the code multiplier. The sums run in another order than the
// butterflies', so a code may differ by one where its pre-round value sits
// within about 1e-6 of a rounding boundary. Measured against the butterfly
// kernel: M = 16, K = 16384: 5.60 -> 4.80 us; M = 2048, K = 8192: 16.0 us
// either way (that batch streams 48 MB). Loading each group's elements from
// 32-byte pieces of 32 rows instead of 1 KB runs cost 1.5 us at M = 2048.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int cpad(int i) { return i + (i >> 5); }                     // pad_idx of a constant
constexpr int deposit10(int g) { return (g & 0x1F) | ((g >> 5) << 6); }  // clear bit 5

// B operands of H_64 for v_mfma_f32_32x32x16_bf16: entry [kc * 2 + nb][lane]
// holds, for lane (c = lane % 32, g = lane / 32), the eight entries
// H[16 kc + 8 g + e][32 nb + c], e < 8, as bf16 bit patterns (+1 = 0x3F80,
// -1 = 0xBF80), two to a word; H[k][j] = (-1)^popcount(k & j).
struct alignas(16) H64Operands {
  unsigned w[8][64][4];
};
constexpr H64Operands make_h64_operands() {
  H64Operands t{};
  for (int kc = 0; kc < 4; ++kc)
    for (int nb = 0; nb < 2; ++nb)
      for (int l = 0; l < 64; ++l)
        for (int p = 0; p < 4; ++p) {
          unsigned word = 0;
          for (int h = 0; h < 2; ++h) {
            const int k = 16 * kc + 8 * (l / 32) + 2 * p + h;
            const int j = 32 * nb + l % 32;
            unsigned par = 0;
            for (int b = 0; b < 6; ++b) par ^= (unsigned)((k & j) >> b) & 1u;
            word |= (0x3F80u | (par << 15)) << (16 * h);
          }
          t.w[kc * 2 + nb][l][p] = word;
        }
  return t;
}
__constant__ H64Operands kH64 = make_h64_operands();

template <int BITS, int L, bool F8>
__global__ __launch_bounds__(64 << (L - 11)) void fwht_mfma_quant_kernel(
    const uint16_t* __restrict__ x, int8_t* __restrict__ codes, float* __restrict__ scales,
    int32_t* __restrict__ rowsum, bool nib, int M) {
  constexpr int K = 1 << L;
  constexpr int W = 1 << (L - 11);  // waves, 2048 elements each
  constexpr int T = 64 * W;
  constexpr int LT = L - 5;         // 32 elements per thread
  constexpr int E = 32;
  constexpr int G = 1 << (L - 10);  // a group: the elements that differ in bits 8, 11 .. L-1
  constexpr int Q = E / G;          // groups per thread
  static_assert(L >= 11 && L <= 15, "2048 <= K <= 32768");
  static_assert(!F8 || BITS == 4, "fp8 pairs hold 4-bit codes");
  extern __shared__ float lds[];
  float* red = lds + RowLds<L, LT>::kRowFloats;
  int* ired = reinterpret_cast<int*>(red + RowLds<L, LT>::kRedFloats);
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  // A operands: lane (s = lane % 32, g = lane / 32), chunk kc holds the 8
  // consecutive elements 2048 w + 8 s + 256 g + 512 kc + [0, 8): the MFMA's
  // k runs over element bits 0-2, 8, 9, 10 and its rows over bits 3-7, so
  // every load instruction reads 1 KB of consecutive bytes.
  const uint16_t* xl = x + 2048 * w + 8 * (lane & 31) + 256 * (lane >> 5);
  uint4 a[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
    a[kc] = *reinterpret_cast<const uint4*>(xl + (size_t)blockIdx.x * K + 512 * kc);
  uint4 b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = *reinterpret_cast<const uint4*>(kH64.w[i][lane]);
  for (int row = blockIdx.x; row < M; row += gridDim.x) {
    // the next row's input is loaded while this one is transformed (the last
    // row reloads itself: the load count stays unconditional)
    const int nrow = row + (int)gridDim.x < M ? row + (int)gridDim.x : row;
    uint4 an[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
      an[kc] = *reinterpret_cast<const uint4*>(xl + (size_t)nrow * K + 512 * kc);
    v16f acc[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[nb][v] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a[kc]), __builtin_bit_cast(bf16x8, b[kc * 2 + nb]), acc[nb],
            0, 0, 0);
    }
    // acc[nb][v] is output row s = 8 (v / 4) + 4 (lane / 32) + v % 4 (the
    // 32 x 32 output layout; element bits 3-7) and output column
    // j = 32 nb + lane % 32, whose bits 0-2, 3, 4, 5 are element bits 0-2, 8,
    // 9, 10: register bits 0, 1, 2, 3 are element bits 3, 4, 6, 7, the lane
    // half element bit 5.
    float v[2][16];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) v[nb][r] = acc[nb][r];
      fwht_regs<16>(v[nb]);
    }
    {
      // the lane's part (bits 0-2, 5, 8, 9, 11 ..) and the register's part
      // (bits 3, 4, 6, 7, 10) share no bit, so their padded indices add up
      const int c = lane & 31;
      const int p0 = pad_idx(2048 * w + (c & 7) + ((c >> 3) << 8) + 32 * (lane >> 5));
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          lds[p0 + cpad(8 * (r & 3) + 64 * (r >> 2) + 1024 * nb)] = v[nb][r];
    }
    lds_barrier();

    // Bits 5 and 11 .. L-1: thread t owns groups t + T q, q < Q; a group's base
    // has those bits clear and its element m sits at base + off(m).
    // Group index g (< 1024) maps to base (g & 0x1F) | ((g >> 5) << 6); t and
    // T q share no bit, nor do a base and an offset, so every padded index is
    // the thread's padded base plus a constant.
    float u[E];
    const int pt = pad_idx(deposit10(t));
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
      for (int m = 0; m < G; ++m)
        u[q * G + m] = lds[pt + cpad(deposit10(T * q)) + cpad(((m & 1) << 5) + ((m >> 1) << 11))];
      fwht_regs<G>(u + q * G);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q)
#pragma unroll
      for (int m = 0; m < G; ++m)
        lds[pt + cpad(deposit10(T * q)) + cpad(((m & 1) << 5) + ((m >> 1) << 11))] = u[q * G + m];

    // The row is transformed (unnormalized): statistic, scale and codes as in
    // the other quantizer's last pass.
    float norm = __builtin_ldexpf(1.0f, -(L >> 1));
    if (L & 1) norm *= 0.70710678118654752f;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) s = (BITS == 8) ? fmaxf(s, fabsf(u[i])) : s + fabsf(u[i]);
    float stat = block_stat<BITS, T>(s, red);  // its barrier also publishes the row
    if (BITS == 4) stat = stat / (float)K;
    const float sc = stat * norm + kEps;
    const float mult = (QConst<BITS>::c * norm) / sc;
    if (t == 0) scales[row] = sc;
    int8_t* crow = codes + (size_t)row * (nib && !F8 ? K / 2 : K);
    int qs = 0;
    if constexpr (F8) {
      qs = store_fp8_pairs<E>(lds, t * E, mult, crow);  // the row's bytes 32 t .. 32 t + 31
    } else {
      const int e0 = t * E;
      const int pe0 = pad_idx(e0);  // e0 is a multiple of 32: the padding of e0 + i is e0's
#pragma unroll
      for (int c = 0; c < E; c += 8) {
        float z[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = lds[pe0 + c + i];
        const uint2 wq = quant_pack8<BITS>(z, mult);
        if (nib)
          *reinterpret_cast<unsigned*>(crow + ((e0 + c) >> 1)) = nibble_word(wq);
        else
          *reinterpret_cast<uint2*>(crow + e0 + c) = wq;
        qs = __builtin_amdgcn_sdot4((int)wq.y, 0x01010101,
                                    __builtin_amdgcn_sdot4((int)wq.x, 0x01010101, qs, false), false);
      }
    }
    if (rowsum) {
      const int total = block_isum<T>(qs, ired);
      if (t == 0) rowsum[row] = total;
    }
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) a[kc] = an[kc];
    lds_barrier();  // this row's LDS reads are done before the next row's writes
  }
}

constexpr size_t kLdsPerCu = 160 * 1024;  // LDS of one CU
constexpr int64_t kCus = 256;

template <int BITS, int L>
hipError_t launch_fwht_mfma(const void* x, int64_t M, int8_t* codes, float* scales,
                            hipStream_t stream, int32_t* rowsum, bool nib, bool f8) {
  constexpr int LT = L - 5;
  const size_t lds = RowLds<L, LT>::kBytes;
  if (f8 && BITS != 4) return hipErrorInvalidValue;
  auto kern = f8 ? fwht_mfma_quant_kernel<BITS, L, BITS == 4> : fwht_mfma_quant_kernel<BITS, L, false>;
  hipError_t e = ensure_lds(kern, lds);
  if (e != hipSuccess) return e;
  // as many workgroups as fit on the chip at once (LDS bounds them), each
  // walking rows and loading its next row's input while it transforms one
  // (M = 2048, K = 8192: 15.6 -> 14.9 us; with half as many workgroups, 15.7)
  const int64_t per_cu = (int64_t)(kLdsPerCu / lds) > 0 ? (int64_t)(kLdsPerCu / lds) : 1;
  const int64_t grid = M < kCus * per_cu ? M : kCus * per_cu;
  kern<<<dim3((unsigned)grid), dim3(1 << LT), lds, stream>>>(reinterpret_cast<const uint16_t*>(x),
                                                             codes, scales, rowsum, nib, (int)M);
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
                         int32_t* rowsum = nullptr, bool nib = false, bool f8 = false) {
  // bf16 rows of 2048 or more elements take the matrix cores for index bits 0-5
  if constexpr (std::is_same<XT, uint16_t>::value && BITS != 0 && !PRO && L >= 11)
    return launch_fwht_mfma<BITS, L>(x, M, codes, scales, stream, rowsum, nib, f8);
  constexpr int LT_BATCH = fwht_lt_batch(L);
  constexpr int LT_FEW = fwht_lt_few(L);
  if (f8 && (BITS != 4 || (1 << (L - LT_BATCH)) > 32 || (1 << (L - LT_FEW)) > 32))
    return hipErrorInvalidValue;  // fp8 pairs: 4-bit codes, at most 32 elements per thread
  if (M <= 64 && LT_FEW != LT_BATCH)
    return launch_fwht<XT, BITS, L, LT_FEW, PRO>(x, M, codes, scales, pro, stream, fout, rowsum, nib, f8);
  return launch_fwht<XT, BITS, L, LT_BATCH, PRO>(x, M, codes, scales, pro, stream, fout, rowsum, nib, f8);
}

// Transform only (fp32 rows in and out, in place allowed).
template <int L>
hipError_t launch_fwht_f32_l(const float* x, int64_t M, float* out, hipStream_t stream) {
  const Prologue none{nullptr, nullptr, 0.0f, 0};
  return launch_fwht_l<float, 0, L, false>(x, M, nullptr, nullptr, none, stream, out);
}

template <typename XT, int BITS, bool PRO>
hipError_t launch_had(const void* x, int64_t M, int K, int8_t* codes, float* scales,
                      const Prologue& pro, hipStream_t stream, int32_t* rowsum, bool nib,
                      bool f8) {
  switch (K) {
    case 1 << 6: return launch_fwht_l<XT, BITS, 6, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 7: return launch_fwht_l<XT, BITS, 7, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 8: return launch_fwht_l<XT, BITS, 8, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 9: return launch_fwht_l<XT, BITS, 9, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 10: return launch_fwht_l<XT, BITS, 10, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 11: return launch_fwht_l<XT, BITS, 11, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 12: return launch_fwht_l<XT, BITS, 12, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 13: return launch_fwht_l<XT, BITS, 13, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 14: return launch_fwht_l<XT, BITS, 14, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    case 1 << 15: return launch_fwht_l<XT, BITS, 15, PRO>(x, M, codes, scales, pro, stream, nullptr, rowsum, nib, f8);
    default: return hipErrorInvalidValue;
  }
}

template <typename XT, int BITS, int CH, bool PRO>
hipError_t launch_rows_ch(const void* x, int64_t M, int K, int8_t* codes, float* scales,
                          const Prologue& pro, hipStream_t stream, int32_t* rowsum, bool nib,
                          bool tl2 = false) {
  quant_rows_kernel<XT, BITS, CH, PRO><<<dim3((unsigned)M), dim3(256), 0, stream>>>(
      reinterpret_cast<const XT*>(x), K, codes, scales, pro, rowsum, nib, tl2);
  return hipGetLastError();
}

template <typename XT, int BITS, bool PRO>
hipError_t launch_rows(const void* x, int64_t M, int K, int8_t* codes, float* scales,
                       const Prologue& pro, hipStream_t stream, int32_t* rowsum, bool nib,
                       bool tl2 = false) {
  const int ch = (K + 2047) / 2048;
  if (ch <= 1) return launch_rows_ch<XT, BITS, 1, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib, tl2);
  if (ch <= 2) return launch_rows_ch<XT, BITS, 2, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib, tl2);
  if (ch <= 4) return launch_rows_ch<XT, BITS, 4, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib, tl2);
  if (ch <= 8) return launch_rows_ch<XT, BITS, 8, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib, tl2);
  return launch_rows_ch<XT, BITS, 16, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib, tl2);
}

template <typename XT, bool PRO>
hipError_t launch_dtype(const void* x, int64_t M, int K, int bits, int hadamard, int8_t* codes,
                        float* scales, const Prologue& pro, hipStream_t stream, int32_t* rowsum,
                        bool nib, bool f8) {
  if (hadamard) {
    return bits == 8
               ? launch_had<XT, 8, PRO>(x, M, K, codes, scales, pro, stream, rowsum, false, f8)
               : launch_had<XT, 4, PRO>(x, M, K, codes, scales, pro, stream, rowsum, nib, f8);
  }
  if (f8) return hipErrorInvalidValue;
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

hipError_t launch_quantize_tl2_order(const void* x, int x_dtype, int64_t M, int K, int bits,
                                     int8_t* codes, float* scales, int32_t* rowsum,
                                     hipStream_t stream) {
  const Prologue none{nullptr, nullptr, 0.0f, 0};
  if (x_dtype == 1)
    return bits == 8 ? launch_rows<uint16_t, 8, false>(x, M, K, codes, scales, none, stream, rowsum, false, true)
                     : launch_rows<uint16_t, 4, false>(x, M, K, codes, scales, none, stream, rowsum, false, true);
  return bits == 8 ? launch_rows<float, 8, false>(x, M, K, codes, scales, none, stream, rowsum, false, true)
                   : launch_rows<float, 4, false>(x, M, K, codes, scales, none, stream, rowsum, false, true);
}

hipError_t launch_quantize(const void* x, int x_dtype, int64_t M, int K, int bits, int hadamard,
                           int8_t* codes, float* scales, hipStream_t stream, const Prologue* pro,
                           int32_t* rowsum, bool nibbles, bool fp8_pairs) {
  if (nibbles && (bits != 4 || K % 8 != 0)) return hipErrorInvalidValue;
  if (fp8_pairs && (nibbles || !fp8_pair_quant_ok(bits, hadamard))) return hipErrorInvalidValue;
  const Prologue none{nullptr, nullptr, 0.0f, 0};
  if (pro && !pro->up && !pro->rms) pro = nullptr;  // nothing to apply: the plain quantizer
  if (pro) {
    if (x_dtype == 1)
      return launch_dtype<uint16_t, true>(x, M, K, bits, hadamard, codes, scales, *pro, stream, rowsum, nibbles, fp8_pairs);
    return launch_dtype<float, true>(x, M, K, bits, hadamard, codes, scales, *pro, stream, rowsum, nibbles, fp8_pairs);
  }
  if (x_dtype == 1)
    return launch_dtype<uint16_t, false>(x, M, K, bits, hadamard, codes, scales, none, stream, rowsum, nibbles, fp8_pairs);
  return launch_dtype<float, false>(x, M, K, bits, hadamard, codes, scales, none, stream, rowsum, nibbles, fp8_pairs);
}

}  // namespace bitnet
