// Ternary mpGEMM / GEMV on int8 MFMA with exact int32 accumulation and a
// fused dequantization epilogue.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), HBitLinear.forward: the
// layer output is F.linear(Q_act(x_r), alpha * t). By linearity that equals
// (q . t^T) * alpha * s / c with integer codes q (Eq. 5-6) and ternary t
// (Eq. 1), the integer-product-then-rescale form the BitNet blog page's
// BitLinear_b158 uses. The products of codes (|q| <= 128) and ternary weights
// are summed exactly in int32 (|acc| <= 128 * 32768 < 2^31).
//
// Weight expansion: a 16-B block-64 word W holds, in bit pair j of byte b,
// the weight at block offset 16j + b. (W >> 2j) & 0x03030303 therefore gives
// the codes of weights 16j .. 16j+15 in byte order, and one v_perm_b32 with
// the byte table {0xFF, 0x00, 0x01} turns codes {0, 1, 2} into int8
// {-1, 0, +1}. Each MFMA lane feeds 16 consecutive k of its row of codes and
// 16 consecutive k of its weight column, so both operands follow the same k
// order and the sum is the plain dot product whatever the hardware's k
// order inside a lane is.
//
// Two shapes:
//   - M <= 16 (decode): v_mfma_i32_16x16x64_i8 with tokens as the 16-row side.
//     One workgroup = 16 output columns, its four waves split K and combine
//     through LDS. HBM-bound on the packed weights.
//   - M > 16 (prefill): 128x128 output tile per workgroup, four waves of
//     64x64 on v_mfma_i32_32x32x32_i8, K step 128. Codes go through a
//     double-buffered LDS tile; packed weights go straight from HBM to
//     registers (a quarter of the bytes of an int8 tile) and are expanded
//     there.
#include "kernels.h"

namespace bitnet {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr unsigned kCodeLut = 0x000100FFu;   // code 0 -> -1, 1 -> 0, 2 -> +1
constexpr unsigned kZeroWeights = 0x55555555u;  // every field code 1 (t = 0)

__device__ __forceinline__ unsigned expand_word(unsigned w, int j) {
  return __builtin_amdgcn_perm(0u, kCodeLut, (w >> (2 * j)) & 0x03030303u);
}

// 64 weights (one packed block) -> four 16-byte int8 vectors, out[j] holding
// block offsets 16j .. 16j+15.
__device__ __forceinline__ void expand_block(const uint4 p, v4i (&out)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[j].x = (int)expand_word(p.x, j);
    out[j].y = (int)expand_word(p.y, j);
    out[j].z = (int)expand_word(p.z, j);
    out[j].w = (int)expand_word(p.w, j);
  }
}

__device__ __forceinline__ float dequant_factor(const float* scales, int m, float alpha, float c) {
  return (alpha * scales[m]) / c;
}

// ------------------------------------------------------------------ GEMV --

template <bool OUT_I32>
__global__ __launch_bounds__(256) void ternary_gemv_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ scales, int M, int K,
    const uint8_t* __restrict__ Wp, int N, const float* __restrict__ alpha_p, float c,
    float* __restrict__ y, int32_t* __restrict__ acc_out) {
  __shared__ v4i red[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;   // B column / A row within the 16x16 tile
  const int grp = lane >> 4;   // which 64-weight block of a 256-k super-block
  const int n = blockIdx.x * 16 + col;
  const int nKB = K >> 6;
  const int nSB = (nKB + 3) >> 2;
  const uint4* wrow = reinterpret_cast<const uint4*>(Wp + (size_t)(n < N ? n : 0) * (size_t)(K >> 2));
  const int8_t* arow = codes + (size_t)(col < M ? col : 0) * (size_t)K;
  const bool n_ok = n < N;
  const bool m_ok = col < M;

  v4i acc = {0, 0, 0, 0};
  for (int sb = wave; sb < nSB; sb += 4) {
    const int kb = sb * 4 + grp;
    const bool k_ok = kb < nKB;
    uint4 p = make_uint4(kZeroWeights, kZeroWeights, kZeroWeights, kZeroWeights);
    if (n_ok && k_ok) p = wrow[kb];
    v4i a[4];
    if (m_ok && k_ok) {
      const v4i* ap = reinterpret_cast<const v4i*>(arow + (size_t)kb * 64);
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = ap[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) a[j] = v4i{0, 0, 0, 0};
    }
    v4i b[4];
    expand_block(p, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], b[j], acc, 0, 0, 0);
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  v4i total = red[0][lane];
#pragma unroll
  for (int w = 1; w < 4; ++w) total += red[w][lane];
  // 16x16 output layout: lane holds rows 4*(lane/16) + v, column lane % 16.
  if (!n_ok) return;
  const float alpha = OUT_I32 ? 0.0f : *alpha_p;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * grp + v;
    if (m < M) {
      if (OUT_I32) {
        acc_out[(size_t)m * N + n] = total[v];
      } else {
        y[(size_t)m * N + n] = (float)total[v] * dequant_factor(scales, m, alpha, c);
      }
    }
  }
}

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
    for (int ct = 0; ct < 2; ++ct) expand_block(bcur[ct], bx[ct]);
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
      const float f = OUT_I32 ? 0.0f : dequant_factor(scales, m, alpha, c);
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

hipError_t launch_ternary_matmul(const int8_t* codes, const float* scales, int64_t M, int K,
                                 const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                                 float* y, int32_t* acc, hipStream_t stream) {
  const float c = (bits == 8) ? 127.0f : 2.6457513110645906f;
  if (M <= 16) {
    const dim3 grid((unsigned)((N + 15) / 16));
    if (acc) {
      ternary_gemv_kernel<true><<<grid, dim3(256), 0, stream>>>(codes, scales, (int)M, K, Wpacked,
                                                               (int)N, alpha, c, y, acc);
    } else {
      ternary_gemv_kernel<false><<<grid, dim3(256), 0, stream>>>(codes, scales, (int)M, K, Wpacked,
                                                                (int)N, alpha, c, y, acc);
    }
  } else {
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    if (acc) {
      ternary_gemm_kernel<true><<<grid, dim3(256), 0, stream>>>(codes, scales, (int)M, K, Wpacked,
                                                               (int)N, alpha, c, y, acc);
    } else {
      ternary_gemm_kernel<false><<<grid, dim3(256), 0, stream>>>(codes, scales, (int)M, K, Wpacked,
                                                                (int)N, alpha, c, y, acc);
    }
  }
  return hipGetLastError();
}

}  // namespace bitnet
