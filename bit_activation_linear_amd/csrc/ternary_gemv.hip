// Decode-shape (M <= 16 tokens) ternary product on v_mfma_i32_16x16x64_i8,
// with exact int32 accumulation and a fused dequantization epilogue.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), HBitLinear.forward: the
// output F.linear(Q_act(x_r), alpha * t) equals (q . t^T) * alpha * s / c
// with integer codes q (Eq. 5-6) and ternary t (Eq. 1).
//
// The kernel is bound by the packed weights streaming from HBM (N*K/4 bytes).
// Every lane issues its 16-B weight loads before anything else, and the grid
// holds enough waves that all of a decode layer's weights are in flight at
// once: tokens are the 16-row side of the MFMA (rows >= M are zero), one
// wave owns one 256-k super-block of `ct` 16-column tiles (its four 16-lane
// groups take one 64-weight block each), the waves of a workgroup cover
// consecutive super-blocks and add up through LDS, and when K has more
// super-blocks than a workgroup has waves, `kz` workgroups split K: each
// writes its int32 partial tile, and the last to arrive (an agent-scope
// ticket counter) sums the partials in split order and applies the epilogue.
// Integer sums are exact, so the result does not depend on the split.
//
// With hadamard = 0 and a small batch the per-token quantization (Eq. 5-6)
// runs inside the same kernel: every workgroup reads the whole (tiny) x,
// reduces the per-token statistic, writes the codes to LDS and feeds the MFMA
// from there, so the decode forward is a single launch.
#include "kernels.h"
#include "ternary_common.cuh"

namespace bitnet {
namespace {

constexpr float kEps = 1e-7f;

struct GemvArgs {
  const int8_t* codes;
  const float* scales;
  const void* x;
  const uint8_t* Wp;
  const float* alpha;
  float* y;
  int32_t* acc_out;
  int32_t* partials;
  unsigned* counters;
  int M, K, N, sb_waves, kz;
  float c;
};

template <int CT>
__device__ __forceinline__ void load_weights(const GemvArgs& a, int kb, bool k_ok, int col,
                                             uint4 (&p)[CT]) {
  const size_t row_bytes = (size_t)(a.K >> 2);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int n = (blockIdx.x * CT + ct) * 16 + col;
    if (k_ok && n < a.N) {
      p[ct] = *reinterpret_cast<const uint4*>(a.Wp + (size_t)n * row_bytes + (size_t)kb * 16);
    } else {
      p[ct] = zero_weight_block();
    }
  }
}

template <int CT>
__device__ __forceinline__ void wave_mma(const v4i (&av)[4], const uint4 (&p)[CT], v4i (&acc)[CT]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[j], expand_quarter(p[ct], j), acc[ct], 0,
                                                       0, 0);
}

// Combine the waves' 16x16 tiles, then (split K) the workgroups' partials,
// then store. 16x16 MFMA layout: lane l holds rows 4*(l/16) + v, column l%16.
template <int CT, bool OUT_I32>
__device__ void gemv_finish(const GemvArgs& a, const v4i (&acc)[CT], v4i* red, int* flag,
                            const float* s_rows) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int nw = blockDim.x >> 6;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) red[(wave * CT + ct) * 64 + lane] = acc[ct];
  __syncthreads();

  const bool active = t < CT * 64;
  const int ct = t >> 6, l = t & 63;
  const int n = (blockIdx.x * CT + ct) * 16 + (l & 15);
  const int m0 = 4 * (l >> 4);
  v4i total = {0, 0, 0, 0};
  if (active) {
    for (int w = 0; w < nw; ++w) total += red[(w * CT + ct) * 64 + l];
  }

  if (a.kz > 1) {
    if (active && n < a.N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + v;
        if (m < a.M) a.partials[((size_t)blockIdx.y * a.M + m) * a.N + n] = total[v];
      }
    }
    __threadfence();
    __syncthreads();
    if (t == 0) {
      const unsigned old = __hip_atomic_fetch_add(&a.counters[blockIdx.x], 1u, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      *flag = (old == (unsigned)(a.kz - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (*flag == 0) return;
    __threadfence();
    if (active && n < a.N) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + v;
        if (m < a.M) {
          int s = 0;
          for (int z = 0; z < a.kz; ++z)
            s += __hip_atomic_load(&a.partials[((size_t)z * a.M + m) * a.N + n], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          total[v] = s;
        }
      }
    }
    if (t == 0)
      __hip_atomic_store(&a.counters[blockIdx.x], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (!active || n >= a.N) return;
  const float alpha = OUT_I32 ? 0.0f : *a.alpha;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = m0 + v;
    if (m >= a.M) continue;
    const size_t o = (size_t)m * a.N + n;
    if (OUT_I32) {
      a.acc_out[o] = total[v];
    } else {
      a.y[o] = (float)total[v] * dequant_factor(alpha, s_rows[m], a.c);
    }
  }
}

template <int CT, bool OUT_I32>
__global__ __launch_bounds__(1024) void ternary_gemv_kernel(GemvArgs a) {
  extern __shared__ v4i red[];
  __shared__ int flag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nKB = a.K >> 6, nSB = (nKB + 3) >> 2;
  const int sb = blockIdx.y * a.sb_waves + wave;
  const bool wave_ok = wave < a.sb_waves && sb < nSB;
  const int kb = sb * 4 + grp;
  const bool k_ok = wave_ok && kb < nKB;

  uint4 p[CT];
  load_weights<CT>(a, kb, k_ok, col, p);
  v4i av[4];
  if (k_ok && col < a.M) {
    const v4i* ap = reinterpret_cast<const v4i*>(a.codes + (size_t)col * a.K + (size_t)kb * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = ap[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = v4i{0, 0, 0, 0};
  }
  v4i acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v4i{0, 0, 0, 0};
  if (wave_ok) wave_mma<CT>(av, p, acc);
  gemv_finish<CT, OUT_I32>(a, acc, red, &flag, a.scales);
}

__device__ __forceinline__ void load4(const float* x, size_t i, float (&v)[4]) {
  const float4 f = *reinterpret_cast<const float4*>(x + i);
  v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
}
__device__ __forceinline__ void load4(const uint16_t* x, size_t i, float (&v)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(x + i);
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xFFFF0000u);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Decode forward with the quantization fused in. Requires K/4 <= blockDim.x
// (each thread owns at most one 4-element chunk per token row) and kz == 1.
template <typename XT, int BITS>
__global__ __launch_bounds__(1024) void fused_decode_kernel(GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  __shared__ int flag;
  const int nw = blockDim.x >> 6;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int col = lane & 15, grp = lane >> 4;
  v4i* red = reinterpret_cast<v4i*>(smem);
  int8_t* qlds = reinterpret_cast<int8_t*>(smem + (size_t)nw * 1024);
  const int mk16 = ((a.M * a.K) + 15) & ~15;
  float* part = reinterpret_cast<float*>(qlds + mk16);  // [nw][16]
  float* srow = part + nw * 16;                         // [16]

  const int nKB = a.K >> 6, nSB = (nKB + 3) >> 2;
  const int sb = wave;
  const bool wave_ok = wave < a.sb_waves && sb < nSB;
  const int kb = sb * 4 + grp;
  const bool k_ok = wave_ok && kb < nKB;

  // Weights first: their HBM latency overlaps the quantization below.
  uint4 p[1];
  load_weights<1>(a, kb, k_ok, col, p);

  // x: thread t owns elements 4t .. 4t+3 of every token row.
  const XT* x = reinterpret_cast<const XT*>(a.x);
  const int K4 = a.K >> 2;
  const bool own = t < K4;
  float v[16][4];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m < a.M && own) {
      load4(x, (size_t)m * a.K + 4 * t, v[m]);
    } else {
      v[m][0] = v[m][1] = v[m][2] = v[m][3] = 0.0f;
    }
  }
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m < a.M) {
      float s;
      if (BITS == 8) {
        s = fmaxf(fmaxf(fabsf(v[m][0]), fabsf(v[m][1])), fmaxf(fabsf(v[m][2]), fabsf(v[m][3])));
        s = wave_max(s);
      } else {
        s = (fabsf(v[m][0]) + fabsf(v[m][1])) + (fabsf(v[m][2]) + fabsf(v[m][3]));
        s = wave_sum(s);
      }
      if (lane == 0) part[wave * 16 + m] = s;
    }
  }
  __syncthreads();
  if (t < a.M) {
    float s = 0.0f;
    for (int w = 0; w < nw; ++w) s = (BITS == 8) ? fmaxf(s, part[w * 16 + t]) : s + part[w * 16 + t];
    if (BITS == 4) s = s / (float)a.K;
    srow[t] = s + kEps;
  }
  __syncthreads();
  const float lo = (BITS == 8) ? -128.0f : -8.0f;
  const float hi = (BITS == 8) ? 127.0f : 7.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    if (m < a.M && own) {
      const float mult = a.c / srow[m];
      unsigned word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float q = __builtin_rintf(v[m][e] * mult);
        q = fminf(fmaxf(q, lo), hi);
        word |= ((unsigned)(int)q & 0xFFu) << (8 * e);
      }
      *reinterpret_cast<unsigned*>(qlds + (size_t)m * a.K + 4 * t) = word;
    }
  }
  __syncthreads();

  v4i av[4];
  if (k_ok && col < a.M) {
    const v4i* ap = reinterpret_cast<const v4i*>(qlds + (size_t)col * a.K + (size_t)kb * 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = ap[j];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = v4i{0, 0, 0, 0};
  }
  v4i acc[1] = {v4i{0, 0, 0, 0}};
  if (wave_ok) wave_mma<1>(av, p, acc);
  gemv_finish<1, false>(a, acc, red, &flag, srow);
}

template <typename Kern>
hipError_t ensure_lds(Kern kern, size_t bytes) {
  if (bytes <= 48 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int CT, bool OUT_I32>
hipError_t launch_gemv_ct(const GemvPlan& p, const GemvArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)(p.threads / 64) * CT * 1024;
  auto kern = ternary_gemv_kernel<CT, OUT_I32>;
  hipError_t e = ensure_lds(kern, lds);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)p.col_groups, (unsigned)p.kz), dim3(p.threads), lds, stream>>>(a);
  return hipGetLastError();
}

template <typename XT, int BITS>
hipError_t launch_fused_t(const GemvPlan& p, const GemvArgs& a, hipStream_t stream) {
  const int nw = p.threads / 64;
  const size_t lds = (size_t)nw * 1024 + (size_t)((a.M * a.K + 15) & ~15) + (size_t)nw * 16 * 4 + 64;
  auto kern = fused_decode_kernel<XT, BITS>;
  hipError_t e = ensure_lds(kern, lds);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)p.col_groups, 1), dim3(p.threads), lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, int32_t* partials, unsigned* counters, hipStream_t stream) {
  const GemvPlan p = plan_gemv(M, K, N, false, false);
  GemvArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.Wp = Wpacked;
  a.alpha = alpha;
  a.y = y;
  a.acc_out = acc;
  a.partials = partials;
  a.counters = counters;
  a.M = (int)M;
  a.K = K;
  a.N = (int)N;
  a.sb_waves = p.sb_waves;
  a.kz = p.kz;
  a.c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  if (p.ct == 4) return acc ? launch_gemv_ct<4, true>(p, a, stream) : launch_gemv_ct<4, false>(p, a, stream);
  return acc ? launch_gemv_ct<1, true>(p, a, stream) : launch_gemv_ct<1, false>(p, a, stream);
}

hipError_t launch_fused_decode(const void* x, int x_dtype, int64_t M, int K,
                               const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                               float* y, hipStream_t stream) {
  const GemvPlan p = plan_gemv(M, K, N, true, false);
  if (!p.fused) return hipErrorInvalidValue;
  GemvArgs a{};
  a.x = x;
  a.Wp = Wpacked;
  a.alpha = alpha;
  a.y = y;
  a.M = (int)M;
  a.K = K;
  a.N = (int)N;
  a.sb_waves = p.sb_waves;
  a.kz = 1;
  a.c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  if (x_dtype == 1) {
    return bits == 8 ? launch_fused_t<uint16_t, 8>(p, a, stream)
                     : launch_fused_t<uint16_t, 4>(p, a, stream);
  }
  return bits == 8 ? launch_fused_t<float, 8>(p, a, stream) : launch_fused_t<float, 4>(p, a, stream);
}

}  // namespace bitnet
