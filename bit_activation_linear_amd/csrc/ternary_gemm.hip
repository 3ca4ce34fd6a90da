// Prefill-shape (M > 16 tokens) ternary mpGEMM on v_mfma_i32_32x32x32_i8 with
// exact int32 accumulation and a fused dequantization epilogue.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), HBitLinear.forward: the
// output F.linear(Q_act(x_r), alpha * t) equals (q . t^T) * alpha * s / c
// with integer codes q (Eq. 5-6) and ternary t (Eq. 1); the BitNet blog
// page's BitLinear_b158 takes the same integer-product-then-rescale form.
// |q| <= 128 and K <= 32768 keep every int32 sum exact.
//
// 128x128 output tile per workgroup, four waves of 64x64, K step 128. Codes
// go through a double-buffered LDS tile; packed weights go straight from HBM
// to registers (a quarter of the bytes of an int8 tile) and are expanded
// there.
#include "kernels.h"
#include "ternary_common.cuh"

namespace bitnet {
namespace {

// ------------------------------------------------------------------ GEMM --

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kLdsStride = BK + 16;  // bytes per LDS row; the pad spreads rows over banks

template <bool OUT_I32>
__global__ __launch_bounds__(256) void ternary_gemm_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ scales, int M, int K,
    const uint8_t* __restrict__ Wp, int N, const float* __restrict__ alpha_p, float c,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) int8_t As[2][BM * kLdsStride];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const int nKB = K >> 6;
  const int nks = (nKB + 1) >> 1;
  const size_t wrow_bytes = (size_t)(K >> 2);

  // A tile loader: eight threads cover one 128-B row slice, 32 rows per round.
  const int a_row = tid >> 3;
  const int a_col = (tid & 7) * 16;
  // B loader: lane owns one column of each of the wave's two 32-column tiles
  // and one of the two 64-k blocks of a K step.
  const int b_grp = lane >> 5;
  int b_col[2];
  bool b_ok[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    b_col[ct] = n0 + wn * 64 + ct * 32 + (lane & 31);
    b_ok[ct] = b_col[ct] < N;
  }

  auto load_a = [&](int ks, uint4 (&r)[4]) {
    const int k = ks * BK + a_col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + a_row + 32 * i;
      if (m < M && k < K) {
        r[i] = *reinterpret_cast<const uint4*>(codes + (size_t)m * K + k);
      } else {
        r[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_a = [&](int buf, const uint4 (&r)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&As[buf][(a_row + 32 * i) * kLdsStride + a_col]) = r[i];
    }
  };
  auto load_b = [&](int ks, uint4 (&r)[2]) {
    const int kb = ks * 2 + b_grp;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      if (b_ok[ct] && kb < nKB) {
        r[ct] = *reinterpret_cast<const uint4*>(Wp + (size_t)b_col[ct] * wrow_bytes + (size_t)kb * 16);
      } else {
        r[ct] = make_uint4(kZeroWeights, kZeroWeights, kZeroWeights, kZeroWeights);
      }
    }
  };

  v16i acc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0;

  uint4 areg[4];
  uint4 bcur[2], bnext[2];
  load_a(0, areg);
  load_b(0, bcur);
  store_a(0, areg);
  __syncthreads();

  for (int ks = 0; ks < nks; ++ks) {
    const bool more = ks + 1 < nks;
    if (more) {
      load_a(ks + 1, areg);
      load_b(ks + 1, bnext);
    }
    v4i bx[2][4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int j = 0; j < 4; ++j) bx[ct][j] = expand_quarter(bcur[ct], j);
    const int8_t* abuf = As[ks & 1];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int8_t* arow = abuf + (wm * 64 + rt * 32 + (lane & 31)) * kLdsStride + b_grp * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const v4i af = *reinterpret_cast<const v4i*>(arow + 16 * j);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, bx[ct][j], acc[rt][ct], 0, 0, 0);
      }
    }
    if (more) {
      store_a((ks + 1) & 1, areg);
      bcur[0] = bnext[0];
      bcur[1] = bnext[1];
    }
    __syncthreads();
  }

  // 32x32 output layout: lane holds column lane % 32 and, for v = 0..15,
  // row 8*(v/4) + 4*(lane/32) + v%4.
  const float alpha = OUT_I32 ? 0.0f : *alpha_p;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 64 + rt * 32 + 8 * (v >> 2) + 4 * b_grp + (v & 3);
      if (m >= M) continue;
      const float f = OUT_I32 ? 0.0f : dequant_factor(alpha, scales[m], c);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        if (!b_ok[ct]) continue;
        const size_t o = (size_t)m * N + b_col[ct];
        if (OUT_I32) {
          acc_out[o] = acc[rt][ct][v];
        } else {
          y[o] = (float)acc[rt][ct][v] * f;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, hipStream_t stream) {
  const float c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (acc) {
    ternary_gemm_kernel<true><<<grid, dim3(256), 0, stream>>>(codes, scales, (int)M, K, Wpacked,
                                                             (int)N, alpha, c, y, acc);
  } else {
    ternary_gemm_kernel<false><<<grid, dim3(256), 0, stream>>>(codes, scales, (int)M, K, Wpacked,
                                                              (int)N, alpha, c, y, acc);
  }
  return hipGetLastError();
}

hipError_t launch_ternary_matmul(const int8_t* codes, const float* scales, int64_t M, int K,
                                 const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                                 float* y, int32_t* acc, hipStream_t stream) {
  if (M <= kDecodeMaxM)
    return launch_gemv(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream);
  return launch_gemm(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream);
}

}  // namespace bitnet
