// Prefill-shape (M > 16 tokens) ternary mpGEMM on v_mfma_i32_32x32x32_i8 with
// exact int32 accumulation and a fused dequantization epilogue.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), HBitLinear.forward: the
// output F.linear(Q_act(x_r), alpha * t) equals (q . t^T) * alpha * s / c
// with integer codes q (Eq. 5-6) and ternary t (Eq. 1); the BitNet blog
// page's BitLinear_b158 takes the same integer-product-then-rescale form.
// |q| <= 128 and K <= 32768 keep every int32 sum exact.
//
// Work decomposition. A workgroup of four waves (2 x 2) owns a
// (64 RT) x (64 CT) output tile; each wave owns (32 RT) x (32 CT), i.e.
// RT x CT accumulators of 32x32 int32 (AGPRs). K advances 128 per stage:
// the stage's codes (BM x 128 B) and packed weights (BN x 32 B: two 16-B
// blocks of 64 weights per column) are fetched with coalesced 16-B loads into
// registers at the top of an iteration; halfway through the current stage's
// MFMAs each thread expands its packed weights to int8 (a shift, a mask and
// one v_perm_b32 per 4 weights, done once per workgroup rather than once per
// wave) and writes codes and weights to the other half of a double-buffered
// LDS tile. The MFMA loop itself then only reads LDS.
//
// MFMA operands. For the 32x32x32 instruction lane l supplies row (or column)
// l % 32 and the 16 consecutive k of group g = l / 32. Sub-step h (k32) of a
// stage uses k = 32h + 16g + [0, 16) for both operands, read as 16 bytes from
// the LDS row of the code tile and of the expanded weight tile.
//
// Tile order. Workgroups are dispatched round-robin over the eight XCDs
// (each with its own L2), so workgroup L runs on XCD L % 8. Each XCD gets a
// contiguous range of tiles walked band by band (four M-tiles wide), so the
// workgroups resident on one XCD at a time share code rows and weight columns
// through its L2.
#include "kernels.h"
#include "ternary_common.cuh"

namespace bitnet {
namespace {

constexpr int BK = 128;
constexpr int kAStride = BK + 16;  // bytes per LDS row (codes and expanded weights):
                                   // the pad puts consecutive rows on distinct banks
constexpr int kXcds = 8;
constexpr int kBand = 4;

// A 16-B global load that stays where it is written: a volatile access is
// neither sunk towards its use nor merged, so a prefetch issued before the
// compute stays in flight during it.
__device__ __forceinline__ uint4 ld_pinned(const void* p) {
  const volatile uint4* vp = reinterpret_cast<const volatile uint4*>(p);
  uint4 r;
  r.x = vp->x;
  r.y = vp->y;
  r.z = vp->z;
  r.w = vp->w;
  return r;
}

template <int RT, int CT, int WMW, int WNW, bool OUT_I32>
__global__ __launch_bounds__(64 * WMW * WNW) void ternary_gemm_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ scales, int M, int K,
    const uint8_t* __restrict__ Wp, int N, const float* __restrict__ alpha_p, float c,
    float* __restrict__ y, int32_t* __restrict__ acc_out, int tiles_m, int tiles_n) {
  constexpr int NT = 64 * WMW * WNW;              // threads
  constexpr int BM = 32 * RT * WMW, BN = 32 * CT * WNW;
  constexpr int A_CHUNKS = BM * (BK / 16) / NT;   // 16-B code chunks per thread per stage
  constexpr int B_CHUNKS = BN * 2 / NT;           // 16-B weight chunks per thread per stage
  static_assert(A_CHUNKS >= 1 && B_CHUNKS >= 1, "tile too small for the workgroup");
  static_assert(A_CHUNKS * NT == BM * (BK / 16) && B_CHUNKS * NT == BN * 2, "uneven staging");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int8_t* As = reinterpret_cast<int8_t*>(smem);  // [2][BM][kAStride] codes
  int8_t* Bs = As + 2 * BM * kAStride;           // [2][BN][kAStride] weights as int8

  // XCD-aware tile order.
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int tile = (L % kXcds) * per_xcd + L / kXcds;
  if (tile >= tiles) return;
  const int band = tile / (kBand * tiles_n);
  const int band_m = (tiles_m - band * kBand) < kBand ? (tiles_m - band * kBand) : kBand;
  const int in_band = tile - band * kBand * tiles_n;
  const int tm = band * kBand + in_band % band_m;
  const int tn = in_band / band_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int nKB = K >> 6;
  const int wrow_bytes = K >> 2;

  // Global -> register staging. Uniform tile bases plus 32-bit lane offsets;
  // rows past M are clamped to a valid row (their outputs are not stored) and
  // k past K is clamped: with an odd number of 64-weight blocks the last
  // stage is a half stage whose second block is never read.
  const int a_col = (tid & 7) * 16;
  const int a_row0 = tid >> 3;
  const int b_half = tid & 1;  // which 64-weight block of the stage this thread fetches
  const int b_col0 = tid >> 1;
  const int full = nKB >> 1;   // stages with both blocks
  const int8_t* a_base = codes + (size_t)m0 * K;
  const uint8_t* b_base = Wp + (size_t)n0 * wrow_bytes;
  int a_off[A_CHUNKS];
#pragma unroll
  for (int i = 0; i < A_CHUNKS; ++i) {
    const int r = a_row0 + (NT / 8) * i;
    a_off[i] = (m0 + r < M ? r : M - 1 - m0) * K;
  }
  int b_off[B_CHUNKS];
#pragma unroll
  for (int i = 0; i < B_CHUNKS; ++i) {
    const int cidx = b_col0 + (NT / 2) * i;
    b_off[i] = (n0 + cidx < N ? cidx : N - 1 - n0) * wrow_bytes;
  }

  v16i acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0;

  uint4 ar[A_CHUNKS], br[B_CHUNKS];
  // (Macros rather than lambdas: a lambda capturing these register arrays by
  // reference makes the compiler keep them in scratch memory.)
#define BITNET_FETCH(ks_)                                                                      \
  {                                                                                            \
    const int k_ = (ks_) * BK + a_col;                                                         \
    const int kc_ = k_ < K ? k_ : K - 16;                                                      \
    _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i) ar[i] =                               \
        ld_pinned(a_base + a_off[i] + kc_);                                                    \
    const int kb_ = (ks_) * 2 + b_half;                                                        \
    const int kbc_ = kb_ < nKB ? kb_ : nKB - 1;                                                \
    _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i) br[i] =                               \
        ld_pinned(b_base + b_off[i] + kbc_ * 16);                                              \
  }
#define BITNET_STASH(buf_)                                                                     \
  {                                                                                            \
    int8_t* an_ = As + (buf_) * BM * kAStride;                                                 \
    _Pragma("unroll") for (int i = 0; i < A_CHUNKS; ++i)                                       \
        *reinterpret_cast<uint4*>(an_ + (a_row0 + (NT / 8) * i) * kAStride + a_col) = ar[i];   \
    int8_t* bn_ = Bs + (buf_) * BN * kAStride;                                                 \
    _Pragma("unroll") for (int i = 0; i < B_CHUNKS; ++i) {                                     \
      int8_t* row_ = bn_ + (b_col0 + (NT / 2) * i) * kAStride + b_half * 64;                   \
      _Pragma("unroll") for (int j = 0; j < 4; ++j)                                            \
          *reinterpret_cast<v4i*>(row_ + 16 * j) = expand_quarter(br[i], j);                   \
    }                                                                                          \
  }

  // MFMAs of k32 sub-steps [H0, H1) of the stage in LDS buffer buf_.
#define BITNET_COMPUTE(buf_, H0, H1)                                                           \
  {                                                                                            \
    const int8_t* a_ = As + (buf_) * BM * kAStride + (wm * 32 * RT + l32) * kAStride + 16 * g; \
    const int8_t* b_ = Bs + (buf_) * BN * kAStride + (wn * 32 * CT + l32) * kAStride + 16 * g; \
    _Pragma("unroll") for (int h = (H0); h < (H1); ++h) {                                       \
      v4i af[RT];                                                                              \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) af[rt] =                               \
          *reinterpret_cast<const v4i*>(a_ + rt * 32 * kAStride + 32 * h);                     \
      v4i bf[CT];                                                                              \
      _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) bf[ct] =                               \
          *reinterpret_cast<const v4i*>(b_ + ct * 32 * kAStride + 32 * h);                     \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                        \
          _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) acc[rt][ct] =                      \
              __builtin_amdgcn_mfma_i32_32x32x32_i8(af[rt], bf[ct], acc[rt][ct], 0, 0, 0);     \
    }                                                                                          \
  }

  BITNET_FETCH(0)
  BITNET_STASH(0)
  lds_barrier();

  // Full stages (both blocks). Each iteration prefetches the next stage into
  // registers (the last one re-reads a clamped stage into the idle buffer),
  // runs half of the current stage's MFMAs, expands and stores the prefetch
  // into the other buffer, then runs the second half. sched_barrier keeps the
  // loads at the top, their first use in the middle, and the MFMA halves on
  // either side.
  for (int ks = 0; ks < full; ++ks) {
    BITNET_FETCH(ks + 1)
    __builtin_amdgcn_sched_barrier(0);
    BITNET_COMPUTE(ks & 1, 0, 2)
    __builtin_amdgcn_sched_barrier(0);
    BITNET_STASH((ks + 1) & 1)
    __builtin_amdgcn_sched_barrier(0);
    BITNET_COMPUTE(ks & 1, 2, 4)
    lds_barrier();
  }
  // With an odd number of blocks the last stage holds one block (two k32
  // sub-steps).
  if (nKB & 1) BITNET_COMPUTE(full & 1, 0, 2)
#undef BITNET_FETCH
#undef BITNET_STASH
#undef BITNET_COMPUTE

  // 32x32 output layout: lane holds column l32 and, for v = 0..15, row
  // 8*(v/4) + 4*g + v%4 of its 32x32 block.
  const float alpha = OUT_I32 ? 0.0f : *alpha_p;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 32 * RT + rt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (m >= M) continue;
      const float f = OUT_I32 ? 0.0f : dequant_factor(alpha, scales[m], c);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int n = n0 + wn * 32 * CT + ct * 32 + l32;
        if (n >= N) continue;
        const size_t o = (size_t)m * N + n;
        if (OUT_I32) {
          acc_out[o] = acc[rt][ct][v];
        } else {
          y[o] = (float)acc[rt][ct][v] * f;
        }
      }
    }
  }
}

template <int RT, int CT, int WMW, int WNW, bool OUT_I32>
hipError_t launch_tile(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, float c, float* y,
                       int32_t* acc, hipStream_t stream) {
  constexpr int BM = 32 * RT * WMW, BN = 32 * CT * WNW;
  const int tiles_m = (int)((M + BM - 1) / BM);
  const int tiles_n = (int)((N + BN - 1) / BN);
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const size_t lds = 2 * (size_t)(BM + BN) * kAStride;
  auto kern = ternary_gemm_kernel<RT, CT, WMW, WNW, OUT_I32>;
  if (lds > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3((unsigned)(per_xcd * kXcds)), dim3(64 * WMW * WNW), lds, stream>>>(
      codes, scales, (int)M, K, Wpacked, (int)N, alpha, c, y, acc, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, hipStream_t stream) {
  const float c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  // 256 x 256 tiles when there are enough of them to fill every CU twice;
  // 128 x 128 otherwise.
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles >= 512) {
    return acc ? launch_tile<4, 4, 2, 2, true>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, stream)
               : launch_tile<4, 4, 2, 2, false>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, stream);
  }
  return acc ? launch_tile<2, 2, 2, 2, true>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, stream)
             : launch_tile<2, 2, 2, 2, false>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, stream);
}

hipError_t launch_ternary_matmul(const int8_t* codes, const float* scales, int64_t M, int K,
                                 const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                                 float* y, int32_t* acc, hipStream_t stream) {
  if (M <= kDecodeMaxM)
    return launch_gemv(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream);
  return launch_gemm(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream);
}

}  // namespace bitnet
