// Absmean ternarization and block-64 2-bit packing of the weights.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), Eq. 1-2,
// quantize_weight_ternary: alpha = mean|W| over the tensor and
// t = RoundClip(W / (alpha + eps), -1, 1). Round-half-even sends |p| <= 0.5 to
// zero and everything above to +-1 after the clip, so the decision reduces to
// |W| > (alpha + eps) / 2, taken here in fp64.
//
// Both passes are HBM-bound (8 B of fp32 reads per weight over the two passes,
// 0.25 B written). Work mapping of the packing pass: four lanes own one 16-B
// packed block (64 weights). Lane c of the four reads the float4 at block
// offset 16j + 4c for j = 0..3 and emits packed dword c, whose byte i carries
// the code of weight 16j + 4c + i in bit pair j.
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr double kEps = 1e-7;
constexpr int64_t kPackMaxBlocks = 2048;

__device__ inline double warp_sum(double v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Fixed-order block reduction of one double per thread (256 threads).
__device__ inline double block_sum(double v, double* red) {
  v = warp_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double total = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(const float4* __restrict__ W4,
                                                                   int64_t n4,
                                                                   double* __restrict__ partials) {
  __shared__ double red[4];
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  // Four independent loads in flight per iteration.
  for (; i + 3 * stride < n4; i += 4 * stride) {
    const float4 v0 = W4[i], v1 = W4[i + stride], v2 = W4[i + 2 * stride], v3 = W4[i + 3 * stride];
    a0 += ((double)fabsf(v0.x) + (double)fabsf(v0.y)) + ((double)fabsf(v0.z) + (double)fabsf(v0.w));
    a1 += ((double)fabsf(v1.x) + (double)fabsf(v1.y)) + ((double)fabsf(v1.z) + (double)fabsf(v1.w));
    a2 += ((double)fabsf(v2.x) + (double)fabsf(v2.y)) + ((double)fabsf(v2.z) + (double)fabsf(v2.w));
    a3 += ((double)fabsf(v3.x) + (double)fabsf(v3.y)) + ((double)fabsf(v3.z) + (double)fabsf(v3.w));
  }
  for (; i < n4; i += stride) {
    const float4 v = W4[i];
    a0 += ((double)fabsf(v.x) + (double)fabsf(v.y)) + ((double)fabsf(v.z) + (double)fabsf(v.w));
  }
  const double total = block_sum((a0 + a1) + (a2 + a3), red);
  if (threadIdx.x == 0) partials[blockIdx.x] = total;
}

__device__ inline unsigned code_of(float w, double thr) {
  // 2-bit code t + 1: 0 for -1, 1 for 0, 2 for +1.
  return ((double)fabsf(w) > thr) ? (w > 0.0f ? 2u : 0u) : 1u;
}

__global__ __launch_bounds__(kThreads) void ternarize_pack_kernel(
    const float* __restrict__ W, int64_t n_dwords, double numel,
    const double* __restrict__ partials, int n_partials, unsigned* __restrict__ out,
    float* __restrict__ alpha) {
  __shared__ double red[4];
  // Every workgroup reduces the partials in the same order, so all of them
  // see the same alpha bit for bit.
  double s = 0.0;
  for (int i = threadIdx.x; i < n_partials; i += kThreads) s += partials[i];
  const double a64 = block_sum(s, red) / numel;
  const double thr = 0.5 * (a64 + kEps);
  if (blockIdx.x == 0 && threadIdx.x == 0) *alpha = (float)a64;

  // Grid-stride over packed dwords (the grid is capped so the redundant
  // partial reduction above stays a small fraction of the traffic).
  for (int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x; d < n_dwords;
       d += (int64_t)gridDim.x * kThreads) {
    const float* src = W + (d >> 2) * 64 + (d & 3) * 4;
    unsigned word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(src + 16 * j);
      const unsigned c = code_of(v.x, thr) | (code_of(v.y, thr) << 8) |
                         (code_of(v.z, thr) << 16) | (code_of(v.w, thr) << 24);
      word |= c << (2 * j);
    }
    out[d] = word;
  }
}

__device__ inline unsigned code_of_sign(int v) { return v > 0 ? 2u : (v < 0 ? 0u : 1u); }

__global__ __launch_bounds__(kThreads) void pack_2bit_kernel(const int8_t* __restrict__ T,
                                                             int64_t n_dwords,
                                                             unsigned* __restrict__ out) {
  const int64_t d = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (d >= n_dwords) return;
  const int8_t* src = T + (d >> 2) * 64 + (d & 3) * 4;
  unsigned word = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const char4 v = *reinterpret_cast<const char4*>(src + 16 * j);
    const unsigned c = code_of_sign(v.x) | (code_of_sign(v.y) << 8) | (code_of_sign(v.z) << 16) |
                       (code_of_sign(v.w) << 24);
    word |= c << (2 * j);
  }
  out[d] = word;
}

}  // namespace

hipError_t launch_absmean_partial(const float* W, int64_t n, double* partials, int* n_partials,
                                  hipStream_t stream) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + kThreads - 1) / kThreads;
  if (blocks > kAbsPartials) blocks = kAbsPartials;
  if (blocks < 1) blocks = 1;
  *n_partials = (int)blocks;
  absmean_partial_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
      reinterpret_cast<const float4*>(W), n4, partials);
  return hipGetLastError();
}

hipError_t launch_ternarize_pack(const float* W, int64_t N, int64_t K, const double* partials,
                                 int n_partials, uint8_t* Wpacked, float* alpha,
                                 hipStream_t stream) {
  const int64_t n_dwords = N * (K / 16);
  int64_t blocks = (n_dwords + kThreads - 1) / kThreads;
  if (blocks > kPackMaxBlocks) blocks = kPackMaxBlocks;
  ternarize_pack_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
      W, n_dwords, (double)N * (double)K, partials, n_partials,
      reinterpret_cast<unsigned*>(Wpacked), alpha);
  return hipGetLastError();
}

hipError_t launch_pack_2bit(const int8_t* T, int64_t N, int64_t K, uint8_t* Wpacked,
                            hipStream_t stream) {
  const int64_t n_dwords = N * (K / 16);
  const int64_t blocks = (n_dwords + kThreads - 1) / kThreads;
  pack_2bit_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, stream>>>(
      T, n_dwords, reinterpret_cast<unsigned*>(Wpacked));
  return hipGetLastError();
}

}  // namespace bitnet
