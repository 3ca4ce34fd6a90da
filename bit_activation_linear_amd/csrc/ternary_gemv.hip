// Decode-shape (M <= 16 tokens) ternary product on v_mfma_i32_16x16x64_i8,
// with exact int32 accumulation and a fused dequantization epilogue.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), HBitLinear.forward: the
// output F.linear(Q_act(x_r), alpha * t) equals (q . t^T) * alpha * s / c
// with integer codes q (Eq. 5-6) and ternary t (Eq. 1).
//
// The kernel is bound by the packed weights streaming from HBM (N*K/4 bytes)
// and, at decode sizes, by the latency of that stream. Tokens are the 16-row
// side of the MFMA (rows >= M are zero). A workgroup owns 16-column tiles
// and the whole of K: its waves take interleaved 256-k super-blocks (four
// 64-weight blocks), issue every load of up to four super-blocks before the
// first MFMA, and add their tiles up through LDS.
// Workgroups never exchange data: on this chip the eight XCD L2 caches are
// not coherent with one another, so a cross-workgroup reduction inside one
// kernel would need an L2 write-back per wave.
//
// Barriers between waves wait for LDS traffic only (s_waitcnt lgkmcnt(0) +
// s_barrier); the default __syncthreads() would also wait for every global
// load in flight, draining the weight stream at each barrier.
//
// The product reads the whole code matrix once per workgroup, so for int4
// codes the forward hands them over two to a byte (nibble codes, see
// kernels.h): the lanes widen them to 16 q on their way to LDS and the tile
// is divided by 16 at the end, exactly. At M = 16, K = 16384, N = 4096 the
// product traces at 8.9 us on nibble codes against 10.0 us on int8 codes.
//
// With hadamard = 0 and a small batch the per-token quantization (Eq. 5-6)
// runs in the same kernel: each wave quantizes the slice of the (tiny) x that
// its own MFMAs consume, with one workgroup barrier to combine the per-token
// statistic, all while its weight loads are in flight, so the decode forward
// is one launch.
#include "kernels.h"
#include "ternary_common.h"
#include "decode_common.h"

namespace bitnet {
namespace {

constexpr float kEps = 1e-7f;
constexpr int kRoundsInFlight = 4;  // super-blocks whose loads a lane issues together
constexpr int kFusedCt = 2;         // 16-column tiles per workgroup in the fused decode kernel
constexpr int kFusedSbw = 1;        // 256-k super-blocks per wave in the fused decode kernel
constexpr int kFusedHadCt = 1;      // ... with the transform (K <= 256: one wave, no idle second)

struct GemvArgs {
  const int8_t* codes;
  const float* scales;
  const void* x;
  const uint8_t* Wp;
  const float* alpha;
  float* y;
  int32_t* acc_out;
  int M, K, N, sb_waves;
  float c;
};

// With the codes' row sums known, the B operand is the stored field u = t + 1
// masked in place (fields 0, 1, 2 worth u, 4u, 16u: one AND per dword) and
// field 3 shifted down to 16u; three accumulators keep the scales apart, and
// q . t = q . u - sum(q) is taken in the epilogue. Without row sums each
// field is expanded to t in {-1, 0, 1} (a shift, a mask and a byte lookup).
template <int CT>
__device__ __forceinline__ void mma_round_u(const v4i (&av)[4], const uint4 (&p)[CT], v4i (&a1)[CT],
                                            v4i (&a4)[CT], v4i (&a16)[CT]) {
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const uint4 w = p[ct];
    v4i u;
    u.x = (int)(w.x & 0x03030303u); u.y = (int)(w.y & 0x03030303u);
    u.z = (int)(w.z & 0x03030303u); u.w = (int)(w.w & 0x03030303u);
    a1[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[0], u, a1[ct], 0, 0, 0);
    u.x = (int)(w.x & 0x0C0C0C0Cu); u.y = (int)(w.y & 0x0C0C0C0Cu);
    u.z = (int)(w.z & 0x0C0C0C0Cu); u.w = (int)(w.w & 0x0C0C0C0Cu);
    a4[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[1], u, a4[ct], 0, 0, 0);
    u.x = (int)(w.x & 0x30303030u); u.y = (int)(w.y & 0x30303030u);
    u.z = (int)(w.z & 0x30303030u); u.w = (int)(w.w & 0x30303030u);
    a16[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[2], u, a16[ct], 0, 0, 0);
    u.x = (int)((w.x >> 2) & 0x30303030u); u.y = (int)((w.y >> 2) & 0x30303030u);
    u.z = (int)((w.z >> 2) & 0x30303030u); u.w = (int)((w.w >> 2) & 0x30303030u);
    a16[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[3], u, a16[ct], 0, 0, 0);
  }
}

template <int CT>
__device__ __forceinline__ void mma_round(const v4i (&av)[4], const uint4 (&p)[CT], v4i (&acc)[CT]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[j], expand_quarter(p[ct], j), acc[ct], 0,
                                                       0, 0);
}

// Codes of one super-block are staged through a wave-private LDS area with
// this row pitch (256 B of k plus 16 B of padding, so the 16 token rows an
// MFMA operand read touches start on distinct banks).
constexpr int kCodePitch = 272;

__device__ __forceinline__ uint4 as_u4(const v4i v) {
  return uint4{(unsigned)v.x, (unsigned)v.y, (unsigned)v.z, (unsigned)v.w};
}

// The wave's share of the product; codes_base is the [M, K] code matrix.
//
// Codes: the MFMA wants row col, block 4 sb + grp, k-quarter j from lane
// (col, grp), a pattern that touches 64 separate 16-byte pieces per load
// instruction; every workgroup streams the whole code matrix, and at that
// rate the L2 -> CU path serves such scattered loads at well under half the
// rate of contiguous ones. So the codes are loaded as 4 rows x 256
// contiguous bytes per instruction, written to the wave's LDS area and read
// back in MFMA order (the same wave writes and reads, so no barrier is
// needed).
//
// With NIB the codes are nibble codes (K % 256 == 0): a lane loads 16 bytes
// (32 codes) of token row 8 i + lane / 8, the two loads of a super-block
// cover its 16 rows, and the lane widens them to 16 x the codes (a mask and
// a shift per four codes) on their way to LDS; the wave's tile is divided
// by 16 at the end, exactly.
//
// Weights, by single super-blocks: lane (col, grp) loads the packed block
// 4 sb + grp of its column straight into its MFMA operand, so one load
// instruction touches 16 rows x 64 bytes, half of 16 cache lines.
// By pairs of super-blocks (PAIR; nibble codes, K % 512 == 0): a wave owns
// 128 bytes of each of its 16 rows and loads them as 8 rows x 128 bytes per
// instruction, whole cache lines (at M = 16, K = 16384, N = 4096 the
// product takes about 0.7 us less than with half lines). Lane L of
// instruction h fetches row 8 h + L / 8, 16-byte block (L % 8) ^ (L / 8) ^ h
// of the 128, and the wave passes them through its own 2 KiB of LDS (in lane
// order, so an operand read of block b of row r finds it at slot
// b ^ (r % 8) ^ (r / 8) of that row: 16 lanes, 64 distinct banks) into MFMA
// order.
//
// Every workgroup reads the whole code matrix; workgroup b starts its walk
// over the super-blocks (or pairs) at b mod their count, so that the
// workgroups of an XCD do not all request the same code lines of its L2 at
// the same moment.
//
// RSG: the codes' row sums are given (u-field operands, see mma_round_u).
template <int CT, bool NIB, bool RSG, bool PAIR>
__device__ __forceinline__ void wave_product(const GemvArgs& a, const int8_t* codes_base,
                                             int8_t* stage, v4i* wstage, v4i (&acc)[CT]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nKB = a.K >> 6, nSB = (nKB + 3) >> 2;
  // work units: super-blocks, or pairs of them
  const int nU = PAIR ? nSB >> 1 : nSB;
  const int rounds = (nU + a.sb_waves - 1) / a.sb_waves;
  __builtin_assume(rounds >= 1);  // at least sb_waves units
  const int rot = (int)(blockIdx.x % (unsigned)nU);
  // units whose loads a lane issues together (four super-blocks either way)
  constexpr int kUnitsInFlight = PAIR ? kRoundsInFlight / 2 : kRoundsInFlight;
  constexpr int kSbPerUnit = PAIR ? 2 : 1;
  v4i a4[CT], a16[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) a4[ct] = a16[ct] = v4i{0, 0, 0, 0};
  const size_t row_bytes = (size_t)(a.K >> 2);
  // contiguous code chunk i of this lane: token row 4 i + lane / 16, byte 16 (lane % 16) of the
  // super-block; nibble codes: token row 8 i + lane / 8, packed byte 16 (lane % 8)
  const int crow = NIB ? lane >> 3 : lane >> 4;
  const int cbyte = NIB ? 16 * (lane & 7) : 16 * (lane & 15);
  constexpr int kCodeLoads = NIB ? 2 : 4;
  constexpr int kRowsPerLoad = NIB ? 8 : 4;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v4i{0, 0, 0, 0};
  if (wave >= a.sb_waves) return;

  // Unconditional loads from clamped addresses; what is out of range is
  // zeroed with a mask (a branch would force a wait on the load).
  auto load_codes = [&](const int sbc, const bool live, v4i (&cv)[4]) {
    const int k = NIB ? sbc * 128 + cbyte : sbc * 256 + cbyte;  // byte in the code row
    const int rb = NIB ? a.K >> 1 : a.K;                        // code row bytes
    const bool k_ok = live && k < rb;
    const int kc = k < rb ? k : rb - 16;
#pragma unroll
    for (int i = 0; i < kCodeLoads; ++i) {
      const int m = kRowsPerLoad * i + crow;
      const int mc = m < a.M ? m : a.M - 1;
      const int mask = (k_ok && m < a.M) ? -1 : 0;
      cv[i] = *reinterpret_cast<const v4i*>(codes_base + (size_t)mc * rb + kc) & mask;
    }
  };
  // One super-block: its codes through LDS into MFMA order, then the MFMAs.
  auto multiply = [&](const v4i (&cv)[4], const uint4 (&pw)[CT]) {
    if constexpr (NIB) {
#pragma unroll
      for (int i = 0; i < kCodeLoads; ++i) {
        const v4i w = cv[i];
        const v4i w4 = w << 4;
        // codes 0-15 and 16-31 of the lane's 32, times 16
        const v4i c0 = v4i{w.x & (int)0xF0F0F0F0u, w4.x & (int)0xF0F0F0F0u,
                           w.y & (int)0xF0F0F0F0u, w4.y & (int)0xF0F0F0F0u};
        const v4i c1 = v4i{w.z & (int)0xF0F0F0F0u, w4.z & (int)0xF0F0F0F0u,
                           w.w & (int)0xF0F0F0F0u, w4.w & (int)0xF0F0F0F0u};
        // codes 32 c .. 32 c + 15 of the row at byte 16 c, the next 16 at
        // 128 + 16 c: eight lanes of a row then write 128 contiguous bytes
        int8_t* dst = stage + (kRowsPerLoad * i + crow) * kCodePitch + cbyte;
        *reinterpret_cast<v4i*>(dst) = c0;
        *reinterpret_cast<v4i*>(dst + 128) = c1;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kCodeLoads; ++i)
        *reinterpret_cast<v4i*>(stage + (kRowsPerLoad * i + crow) * kCodePitch + cbyte) = cv[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    v4i av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // codes 64 grp + 16 j .. + 15 of row col
      const int at = NIB ? 128 * (j & 1) + 32 * grp + 16 * (j >> 1) : 64 * grp + 16 * j;
      av[j] = *reinterpret_cast<const v4i*>(stage + col * kCodePitch + at);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    if constexpr (RSG) mma_round_u<CT>(av, pw, acc, a4, a16);
    else mma_round<CT>(av, pw, acc);
  };

  // One round: the loads of up to four super-blocks, then their MFMAs.
  auto round = [&](const int r0) {
    // (vector-typed, so that the compiler keeps them in registers)
    v4i p[kUnitsInFlight][CT][kSbPerUnit];
    v4i cv[kUnitsInFlight][kSbPerUnit][4];
#pragma unroll
    for (int u = 0; u < kUnitsInFlight; ++u) {
      const int ul = wave + a.sb_waves * (r0 + u);  // place in the walk
      const bool live = (r0 + u < rounds) && ul < nU;
      const int uc = live ? (ul + rot < nU ? ul + rot : ul + rot - nU) : nU - 1;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if constexpr (PAIR) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int n = (blockIdx.x * CT + ct) * 16 + 8 * h + (lane >> 3);
            const int nc = n < a.N ? n : a.N - 1;
            const int blk = (lane & 7) ^ (lane >> 3) ^ h;
            p[u][ct][h] = *reinterpret_cast<const v4i*>(a.Wp + (size_t)nc * row_bytes +
                                                        (size_t)uc * 128 + 16 * blk);
          }
        } else {
          const int kb = uc * 4 + grp;
          const int kbc = kb < nKB ? kb : nKB - 1;
          const int n = (blockIdx.x * CT + ct) * 16 + col;
          const int nc = n < a.N ? n : a.N - 1;
          p[u][ct][0] =
              *reinterpret_cast<const v4i*>(a.Wp + (size_t)nc * row_bytes + (size_t)kbc * 16);
        }
      }
#pragma unroll
      for (int s = 0; s < kSbPerUnit; ++s) load_codes(kSbPerUnit * uc + s, live, cv[u][s]);
    }
    // every load of the round is issued before the first use of one (the
    // scheduler would otherwise pull the weights' LDS writes up between them)
    if constexpr (PAIR) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kUnitsInFlight; ++u) {
      if (r0 + u < rounds) {
        if constexpr (PAIR) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int h = 0; h < 2; ++h) wstage[(ct * 2 + h) * 64 + lane] = p[u][ct][h];
          __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
          const int r8 = col & 7, hi = col >> 3;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            uint4 pw[CT];
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              pw[ct] = as_u4(wstage[(ct * 2 + hi) * 64 + r8 * 8 + ((4 * s + grp) ^ r8 ^ hi)]);
            multiply(cv[u][s], pw);
          }
        } else {
          uint4 pw[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) pw[ct] = as_u4(p[u][ct][0]);
          multiply(cv[u][0], pw);
        }
      }
    }
  };
  // The first round is not inside the loop: at a loop header the compiler waits for every
  // load in flight (a later round's unused loads may target the registers it reuses), which
  // on entry would hold the weight stream back until alpha, the scales and the row sums land.
  round(0);
  for (int r0 = kUnitsInFlight; r0 < rounds; r0 += kUnitsInFlight) round(r0);
  if constexpr (RSG) {
    // q . u over the three scales (exact: a4 holds multiples of 4, a16 of 16)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = acc[ct] + (a4[ct] >> 2) + (a16[ct] >> 4);
  }
  if constexpr (NIB) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] >>= 4;  // every product was 16 q u (or 16 q t)
  }
}

// Add the waves' 16x16 tiles and store. 16x16 MFMA layout: lane l holds rows
// 4*(l/16) + v, column l%16.
// s_row[v] is the scale of output row 4 (l / 16) + v of the finishing lane
// and rs[v] its code row sum when the tiles hold q . u (loaded ahead by the
// caller, like alpha; zero otherwise).
template <int CT, bool OUT_I32>
__device__ __forceinline__ void gemv_finish(const GemvArgs& a, const v4i (&acc)[CT], v4i* red,
                                            const float (&s_row)[4], const int (&rs)[4], int nw,
                                            float alpha) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) red[(wave * CT + ct) * 64 + lane] = acc[ct];
  lds_barrier();
  if (t >= CT * 64) return;
  const int ct = t >> 6, l = t & 63;
  const int n = (blockIdx.x * CT + ct) * 16 + (l & 15);
  if (n >= a.N) return;
  v4i total = red[ct * 64 + l];
  for (int w = 1; w < nw; ++w) total += red[(w * CT + ct) * 64 + l];
  const int m0 = 4 * (l >> 4);
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = m0 + v;
    if (m >= a.M) continue;
    const size_t o = (size_t)m * a.N + n;
    if (OUT_I32) {
      a.acc_out[o] = total[v];
    } else {
      a.y[o] = (float)(total[v] - rs[v]) * dequant_factor(alpha, s_row[v], a.c);
    }
  }
}

// LDS of the product per wave: its tile for the final sum, its code staging
// area and, with PAIR, its weight staging area.
template <int CT, bool PAIR>
constexpr size_t gemv_lds_per_wave() {
  return (size_t)CT * 1024 + 16 * kCodePitch + (PAIR ? (size_t)CT * 2048 : 0);
}

// Scalar arguments: the first two (the weight and code addresses) are
// preloaded into SGPRs (see the single-token kernels below).
template <int CT, bool OUT_I32, bool NIB, bool RSG, bool PAIR>
__global__ __launch_bounds__(1024) void ternary_gemv_kernel(
    const uint8_t* Wp, const int8_t* codes, const float* scales, const float* alpha_p, float* y,
    int32_t* acc_out, const int32_t* rowsum, int M, int K, int N, int sb_waves, float c) {
  GemvArgs a{};
  a.Wp = Wp;
  a.codes = codes;
  a.scales = scales;
  a.alpha = alpha_p;
  a.y = y;
  a.acc_out = acc_out;
  a.M = M;
  a.K = K;
  a.N = N;
  a.sb_waves = sb_waves;
  a.c = c;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6;
  v4i* red = reinterpret_cast<v4i*>(smem);  // [nw][CT][64]
  int8_t* stage = reinterpret_cast<int8_t*>(smem + (size_t)nw * CT * 1024) +
                  (size_t)wave * 16 * kCodePitch;
  v4i* wstage = reinterpret_cast<v4i*>(smem + (size_t)nw * (CT * 1024 + 16 * kCodePitch) +
                                       (size_t)wave * CT * 2048);
  // Scalars, alpha and the finishing lanes' row scales are fetched before
  // the weight stream: a small load issued behind it waits about a
  // microsecond.
  asm volatile("" ::"s"(a.M), "s"(a.K), "s"(a.N), "s"(a.c), "s"(a.y), "s"(a.sb_waves), "s"(a.Wp),
               "s"(a.codes), "s"(nw));
  float alpha = 0.0f;
  float s_row[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int rs[4] = {0, 0, 0, 0};
  if (!OUT_I32) {
    alpha = *a.alpha;
    const int m0 = 4 * ((threadIdx.x & 63) >> 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + v < a.M ? m0 + v : a.M - 1;
      s_row[v] = a.scales[m];
      if (RSG) rs[v] = rowsum[m];
    }
  }
  v4i acc[CT];
  wave_product<CT, NIB, RSG, PAIR>(a, a.codes, stage, wstage, acc);
  gemv_finish<CT, OUT_I32>(a, acc, red, s_row, rs, nw, alpha);
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

// Decode forward with the quantization fused in. Requires M <= MG and
// 256 * SBW * waves >= K: wave w owns the SBW super-blocks w * SBW + r,
// r < SBW (k in [256 (w SBW + r), +256)), for the statistic, for the codes
// and for the product.
//
// Each lane loads 4 consecutive x values per token row and super-block, then
// its packed weights; the per-row statistic (Eq. 5: absmax, or Eq. 6: mean
// |x|) of the wave's share is reduced in the wave with DPP, and a single
// barrier publishes the waves' partial statistics. Every wave then combines
// them in the same fixed order, quantizes its own values and hands them to
// the lanes that feed them to the MFMA through a wave-private LDS region (no
// further barrier), so little work separates the arrival of the data from
// the product.
template <typename XT, int BITS, int MG, int CT, int SBW, bool PRO, bool HAD>
__global__ __launch_bounds__(1024) void fused_decode_kernel(
    const void* x_in, const uint8_t* Wp, const float* alpha_p, float* y, int M, int K, int N,
    float c, const void* up, const float* gamma, float norm_eps, int rms) {
  // scalar arguments, the x and weight addresses preloaded into SGPRs
  GemvArgs a{};
  a.x = x_in;
  a.Wp = Wp;
  a.alpha = alpha_p;
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.c = c;
  const Prologue pro{up, gamma, norm_eps, rms};
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // The scalars the kernel needs (kernel arguments and alpha) are fetched
  // before the weight stream goes out, and pinned there: a small load issued
  // once the stream is in flight waits behind it, about a microsecond, on
  // the path from the statistic to the store. The wave count follows from K
  // as in the launcher, with no read of the dispatch packet.
  asm volatile("" ::"s"(a.M), "s"(a.K), "s"(a.N), "s"(a.c), "s"(a.y), "s"(a.x), "s"(a.Wp));
  if constexpr (PRO)
    asm volatile("" ::"s"(pro.up), "s"(pro.gamma), "s"(pro.norm_eps), "s"(pro.rms));
  const float alpha = *a.alpha;
  const int nsb = ((a.K >> 6) + 3) >> 2;
  const int nw = (nsb + SBW - 1) / SBW > CT ? (nsb + SBW - 1) / SBW : CT;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  v4i* red = reinterpret_cast<v4i*>(smem);                                // [nw][CT][64]
  float* part = reinterpret_cast<float*>(smem + (size_t)nw * CT * 1024);  // [nw][16]
  // [nw][16] row scales: each wave writes its own copy and reads only that,
  // so no wave depends on another's write (every wave computes the same
  // values, bit for bit, from the same partials in the same order)
  float* srow = part + nw * 16;
  float* psq = srow + nw * 16;  // [nw][16] partial sums of squares (prologue with RMSNorm)
  // this wave's codes: [SBW][M][256]
  int8_t* qw = reinterpret_cast<int8_t*>(psq + (PRO ? nw * 16 : 0)) +
               (size_t)wave * SBW * a.M * 256;

  const int col = lane & 15, grp = lane >> 4;
  const int nKB = a.K >> 6;
  // x (and the prologue's inputs) first, then the packed weights. Vector
  // loads complete in issue order, so with this order the statistic, the
  // barrier and the quantization wait for x alone and run while the weight
  // stream (the long pole, HBM) is still arriving. The loads are
  // unconditional from clamped, always-valid addresses (a load inside a
  // branch would be waited for inside it) and are widened only after the
  // weight loads have gone out. Each lane takes 4 consecutive x values of
  // every token row in each super-block.
  const XT* x = reinterpret_cast<const XT*>(a.x);
  const XT* upp = (PRO && pro.up) ? reinterpret_cast<const XT*>(pro.up) : x;
  const bool use_g = PRO && pro.rms && pro.gamma;
  const float* gp = use_g ? pro.gamma : reinterpret_cast<const float*>(a.x);
  bool own[SBW];
  Raw4<XT> xraw[MG][SBW];
  Raw4<XT> uraw[PRO ? MG : 1][SBW];
  float4 graw[SBW];
#pragma unroll
  for (int r = 0; r < SBW; ++r) {
    const int k0 = 256 * (wave * SBW + r) + 4 * lane;
    own[r] = k0 < a.K;
    const int kc = own[r] ? k0 : 0;
#pragma unroll
    for (int m = 0; m < MG; ++m) {
      const size_t i = (size_t)(m < a.M ? m : 0) * a.K + kc;
      raw_load4(x, i, xraw[m][r]);
      if (PRO) raw_load4(upp, i, uraw[PRO ? m : 0][r]);
    }
    if (PRO) graw[r] = *reinterpret_cast<const float4*>(gp + (use_g ? kc : 0));
  }
  // Packed weights; unconditional loads from clamped, always-valid addresses.
  uint4 p[SBW][CT];
  {
    const size_t row_bytes = (size_t)(a.K >> 2);
#pragma unroll
    for (int r = 0; r < SBW; ++r) {
      const int kb = (wave * SBW + r) * 4 + grp;
      const int kbc = kb < nKB ? kb : nKB - 1;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int n = (blockIdx.x * CT + ct) * 16 + col;
        const int nc = n < a.N ? n : a.N - 1;
        // an out-of-range block meets all-zero codes below
        p[r][ct] = *reinterpret_cast<const uint4*>(a.Wp + (size_t)nc * row_bytes + (size_t)kbc * 16);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Rows past M hold row 0's values and are never used.
  float v[MG][SBW][4];
  float u[PRO ? MG : 1][SBW][4];
  float g[SBW][4];
#pragma unroll
  for (int r = 0; r < SBW; ++r) {
#pragma unroll
    for (int m = 0; m < MG; ++m) {
      widen4(xraw[m][r], v[m][r]);
      if (PRO) widen4(uraw[PRO ? m : 0][r], u[PRO ? m : 0][r]);
    }
    g[r][0] = use_g ? graw[r].x : 1.0f;
    g[r][1] = use_g ? graw[r].y : 1.0f;
    g[r][2] = use_g ? graw[r].z : 1.0f;
    g[r][3] = use_g ? graw[r].w : 1.0f;
  }
  // Input prologue (engine page: BitNetV2FFN's silu(gate) * up, then
  // HBitLinear's RMSNorm weight); the norm's 1/rms enters only the scale and
  // the code multiplier below, its sum of squares rides on the statistic's
  // barrier.
  float sq[MG];
#pragma unroll
  for (int m = 0; m < MG; ++m) sq[m] = 0.0f;
  if constexpr (PRO) {
#pragma unroll
    for (int r = 0; r < SBW; ++r) {
#pragma unroll
      for (int m = 0; m < MG; ++m) {
        if (m < a.M) {
          if (pro.up) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              v[m][r][e] = silu(v[m][r][e]) * u[m][r][e];
          }
          if (pro.rms) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sq[m] += own[r] ? v[m][r][e] * v[m][r][e] : 0.0f;
              v[m][r][e] *= g[r][e];
            }
          }
        }
      }
    }
  }

  // Walsh-Hadamard transform (engine page Eq. 3-4; HAD needs K <= 256, so
  // one wave holds every token row whole: lane l has elements 4 l .. 4 l + 3).
  // Index bits 0-1 are butterflied in registers, bits 2-7 across lanes, in
  // bit order and with the same (a + b, a - b) steps as the transform kernel,
  // so the unnormalized values are the same bit for bit; the 1/sqrt(K) goes
  // into the scale and the code multiplier below.
  if constexpr (HAD) {
#pragma unroll
    for (int m = 0; m < MG; ++m) {
#pragma unroll
      for (int h = 1; h < 4; h <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((e & h) == 0) {
            const float x0 = v[m][0][e], x1 = v[m][0][e + h];
            v[m][0][e] = x0 + x1;
            v[m][0][e + h] = x0 - x1;
          }
    }
    // Lane stages (lane bit i = index bit i + 2), every token row's exchanges
    // of a stage issued together: partners within a row of 16 lanes through
    // DPP (quad permutes for 1 and 2, row shifts for 4 and 8), across rows
    // through ds_bpermute.
#define BITNET_HAD_DPP(mk, lo_ctrl, hi_ctrl)                                                      \
    if (4 * (mk) < a.K) {                                                                        \
      _Pragma("unroll") for (int m = 0; m < MG; ++m)                                             \
      _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                            \
        const int vi = __float_as_int(v[m][0][e]);                                               \
        const float up = __int_as_float(__builtin_amdgcn_update_dpp(0, vi, lo_ctrl, 0xF, 0xF, true)); \
        const float dn = __int_as_float(__builtin_amdgcn_update_dpp(0, vi, hi_ctrl, 0xF, 0xF, true)); \
        v[m][0][e] = (lane & (mk)) ? dn - v[m][0][e] : v[m][0][e] + up;                          \
      }                                                                                          \
    }
    BITNET_HAD_DPP(1, 0xB1, 0xB1)    // quad_perm [1,0,3,2]
    BITNET_HAD_DPP(2, 0x4E, 0x4E)    // quad_perm [2,3,0,1]
    BITNET_HAD_DPP(4, 0x104, 0x114)  // row_shl:4 (partner l + 4), row_shr:4 (l - 4)
    BITNET_HAD_DPP(8, 0x108, 0x118)  // row_shl:8, row_shr:8
#undef BITNET_HAD_DPP
    for (int mk = 16; 4 * mk < a.K; mk <<= 1) {
      float o[MG][4];
#pragma unroll
      for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[m][e] = __shfl_xor(v[m][0][e], mk);
#pragma unroll
      for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) v[m][0][e] = (lane & mk) ? o[m][e] - v[m][0][e] : v[m][0][e] + o[m][e];
    }
  }

  // Partial statistic of this wave's super-blocks, one per token row.
#pragma unroll
  for (int m = 0; m < MG; ++m) {
    if (m < a.M) {
      float s = 0.0f;
#pragma unroll
      for (int r = 0; r < SBW; ++r) {
        float sr;
        if (BITS == 8) {
          sr = fmaxf(fmaxf(fabsf(v[m][r][0]), fabsf(v[m][r][1])),
                     fmaxf(fabsf(v[m][r][2]), fabsf(v[m][r][3])));
          s = fmaxf(s, own[r] ? sr : 0.0f);
        } else {
          sr = (fabsf(v[m][r][0]) + fabsf(v[m][r][1])) + (fabsf(v[m][r][2]) + fabsf(v[m][r][3]));
          s += own[r] ? sr : 0.0f;
        }
      }
      s = (BITS == 8) ? wave_reduce<true>(s) : wave_reduce<false>(s);
      if (lane == 0) part[wave * 16 + m] = s;
      if (PRO && pro.rms) {
        const float q = wave_reduce<false>(sq[m]);
        if (lane == 0) psq[wave * 16 + m] = q;
      }
    }
  }
  lds_barrier();

  // Whole-row statistic (every wave combines the partials in the same
  // order, so all agree bit for bit) and this wave's codes.
  const float lo = (BITS == 8) ? -128.0f : -8.0f;
  const float hi = (BITS == 8) ? 127.0f : 7.0f;
#pragma unroll
  for (int m = 0; m < MG; ++m) {
    if (m < a.M) {
      float s = 0.0f;
      for (int w = 0; w < nw; ++w) s = (BITS == 8) ? fmaxf(s, part[w * 16 + m]) : s + part[w * 16 + m];
      if (BITS == 4) s = s / (float)a.K;
      float mult;
      if constexpr (HAD) {
        // the transform kernel's arithmetic: norm = prod of log2 K factors 1/sqrt2
        const int L = 31 - __builtin_clz(a.K);
        float norm = __builtin_ldexpf(1.0f, -(L >> 1));
        if (L & 1) norm *= 0.70710678118654752f;
        if (PRO && pro.rms) {
          float q = 0.0f;
          for (int w = 0; w < nw; ++w) q += psq[w * 16 + m];
          const float sraw = s * norm;
          const float rms = sqrtf(q / (float)a.K + pro.norm_eps);
          mult = (a.c * norm) / (sraw + kEps * rms);
          s = sraw / rms + kEps;
        } else {
          s = s * norm + kEps;
          mult = (a.c * norm) / s;
        }
      } else if (PRO && pro.rms) {
        float q = 0.0f;
        for (int w = 0; w < nw; ++w) q += psq[w * 16 + m];
        const float rms = sqrtf(q / (float)a.K + pro.norm_eps);
        mult = a.c / (s + kEps * rms);
        s = s / rms + kEps;
      } else {
        s += kEps;
        mult = a.c / s;
      }
      if (lane == m) srow[wave * 16 + m] = s;
#pragma unroll
      for (int r = 0; r < SBW; ++r) {
        unsigned word = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float q = __builtin_rintf(v[m][r][e] * mult);
          q = fminf(fmaxf(q, lo), hi);
          word |= ((unsigned)(int)q & 0xFFu) << (8 * e);
        }
        *reinterpret_cast<unsigned*>(qw + (r * a.M + m) * 256 + 4 * lane) = own[r] ? word : 0u;
      }
    }
  }
  // The codes just written are read back by other lanes of the same wave;
  // LDS serves a wave's accesses in order, so only the compiler needs fencing.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // MFMA operand: lane (col, grp) feeds token row col, block 4 (w SBW + r) + grp.
  v4i acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v4i{0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < SBW; ++r) {
    const int kb = (wave * SBW + r) * 4 + grp;
    const int kmask = (kb < nKB && col < a.M) ? -1 : 0;
    const int8_t* qr = qw + (r * a.M + (col < a.M ? col : 0)) * 256 + grp * 64;
    v4i av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const v4i*>(qr + 16 * j) & kmask;
    mma_round<CT>(av, p[r], acc);
  }
  float s_row[4];
  {
    const int m0 = 4 * (lane >> 4);
#pragma unroll
    for (int v = 0; v < 4; ++v) s_row[v] = srow[wave * 16 + (m0 + v < a.M ? m0 + v : 0)];
  }
  const int no_rs[4] = {0, 0, 0, 0};
  gemv_finish<CT, false>(a, acc, red, s_row, no_rs, nw, alpha);
}

// max(|a|, |b|, c) in one instruction. Written with fmaxf, each operand is
// first quieted (one more instruction per value in IEEE mode), although no
// NaN reaches the statistic.
__device__ __forceinline__ float max3_abs(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Wave-wide max of non-negative values in the DPP steps of wave_reduce, each
// one v_max_f32 with its first operand routed by DPP (wave_reduce moves the
// neighbour first and quiets it before the max). The s_nops are the wait
// states a DPP read of a VALU-written register needs, which the compiler does
// not insert for instructions it does not see; the last one precedes the
// readlane. The max of a set does not depend on its order, so the result is
// wave_reduce<true>'s bit for bit.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  asm volatile(
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_f32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n"
      "s_nop 1"
      : "+v"(v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The product of the single-token decode on the vector ALU: lane (c, g) owns
// column c's 64-weight block 4 sb + g, whose codes lanes 16 g .. 16 g + 15 of
// its own DPP row quantized (four consecutive codes each). Each packed dword
// d of the block holds, in field j of byte e, the weight at 16 j + 4 d + e,
// whose code sits in byte e of row lane 4 j + d's code word: one v_dot4c
// with that lane's word broadcast by DPP (row_newbcast) and the field masked
// in place (worth u, 4u or 16u) per four weights. The four row partials of a
// column are then added across rows.
template <int NSB>
__device__ __forceinline__ void wave_decode_dot(const GemvArgs& a, const uint4 (&p)[NSB],
                                                const unsigned (&cw)[NSB], int qsum, float alpha,
                                                float st, int lane) {
  qsum = wave_sum_int(qsum);
  int acc1 = 0, acc4 = 0, acc16a = 0, acc16b = 0;
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    // One block per super-block, with the wait states the compiler cannot
    // insert for instructions it does not see: every VGPR a DPP instruction
    // reads (the code word, the masked field and the accumulator alike) must
    // have been written at least two instructions earlier, which the leading
    // s_nop gives for whatever the compiler places just before the block
    // (inside it the fields are all masked before the first dot); and a dot
    // product's result must wait three before another instruction reads it,
    // which the trailing s_nop gives (within the block each accumulator is
    // read only by the next dot into it, which needs no wait).
    const uint4 pw = p[sb];
    int t[16];
    asm volatile(
        "s_nop 1\n"
        "v_and_b32 %[t0], 0x03030303, %[px]\n"
        "v_and_b32 %[t1], 0x0c0c0c0c, %[px]\n"
        "v_and_b32 %[t2], 0x30303030, %[px]\n"
        "v_lshrrev_b32 %[t3], 2, %[px]\n"
        "v_and_b32 %[t4], 0x03030303, %[py]\n"
        "v_and_b32 %[t5], 0x0c0c0c0c, %[py]\n"
        "v_and_b32 %[t6], 0x30303030, %[py]\n"
        "v_lshrrev_b32 %[t7], 2, %[py]\n"
        "v_and_b32 %[t8], 0x03030303, %[pz]\n"
        "v_and_b32 %[t9], 0x0c0c0c0c, %[pz]\n"
        "v_and_b32 %[t10], 0x30303030, %[pz]\n"
        "v_lshrrev_b32 %[t11], 2, %[pz]\n"
        "v_and_b32 %[t12], 0x03030303, %[pw]\n"
        "v_and_b32 %[t13], 0x0c0c0c0c, %[pw]\n"
        "v_and_b32 %[t14], 0x30303030, %[pw]\n"
        "v_lshrrev_b32 %[t15], 2, %[pw]\n"
        "v_and_b32 %[t3], 0x30303030, %[t3]\n"
        "v_and_b32 %[t7], 0x30303030, %[t7]\n"
        "v_and_b32 %[t11], 0x30303030, %[t11]\n"
        "v_and_b32 %[t15], 0x30303030, %[t15]\n"
        "v_dot4c_i32_i8_dpp %[a1], %[c], %[t0] row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a4], %[c], %[t1] row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a16], %[c], %[t2] row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[b16], %[c], %[t3] row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a1], %[c], %[t4] row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a4], %[c], %[t5] row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a16], %[c], %[t6] row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[b16], %[c], %[t7] row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a1], %[c], %[t8] row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a4], %[c], %[t9] row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a16], %[c], %[t10] row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[b16], %[c], %[t11] row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a1], %[c], %[t12] row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a4], %[c], %[t13] row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[a16], %[c], %[t14] row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
        "v_dot4c_i32_i8_dpp %[b16], %[c], %[t15] row_newbcast:15 row_mask:0xf bank_mask:0xf\n"
        "s_nop 2"
        : [a1] "+v"(acc1), [a4] "+v"(acc4), [a16] "+v"(acc16a), [b16] "+v"(acc16b),
          [t0] "=&v"(t[0]), [t1] "=&v"(t[1]), [t2] "=&v"(t[2]), [t3] "=&v"(t[3]),
          [t4] "=&v"(t[4]), [t5] "=&v"(t[5]), [t6] "=&v"(t[6]), [t7] "=&v"(t[7]),
          [t8] "=&v"(t[8]), [t9] "=&v"(t[9]), [t10] "=&v"(t[10]), [t11] "=&v"(t[11]),
          [t12] "=&v"(t[12]), [t13] "=&v"(t[13]), [t14] "=&v"(t[14]), [t15] "=&v"(t[15])
        : [c] "v"(cw[sb]), [px] "v"(pw.x), [py] "v"(pw.y), [pz] "v"(pw.z), [pw] "v"(pw.w));
  }
  // each partial is a multiple of its field's weight, so the shifts are exact
  int part = acc1 + (acc4 >> 2) + ((acc16a + acc16b) >> 4);
  part += __shfl_xor(part, 16);
  part += __shfl_xor(part, 32);
  const int n = blockIdx.x * 16 + lane;
  if (lane < 16 && n < a.N) a.y[n] = (float)(part - qsum) * dequant_factor(alpha, st, a.c);
}

// Single-token decode forward, one wave per 16 output columns and all of K
// (NSB 256-k super-blocks, NSB <= 16). Every x value the wave needs fits in
// its registers, so it computes the whole-row statistic itself (DPP),
// quantizes, runs the MFMAs over all of K into one accumulator and stores:
// no workgroup barrier and no cross-wave reduction on the path, which is
// then the latency of the x and weight loads plus this wave's arithmetic.
// Each workgroup is one wave (several independent waves per workgroup
// measured slower). NSB is exact and every load unconditional: a load count
// that depends on a branch makes the compiler wait for every load in
// flight, the weights included, before the first use of x, and padding the
// count with re-read blocks costs ~0.2 us per super-block.
// With RMS, the layer input is RMSNorm'd first (engine page HBitLinear.forward
// step 1; gamma may be null for unit weight): the sum of squares is one more
// DPP reduction and 1/rms enters only the scale and the code multiplier, as
// in the other quantizer kernels. That variant multiplies on the vector ALU
// (wave_decode_dot: no LDS round trip, no MFMA), which measured faster for it
// (3.68 -> 3.60 us at K = 2560, N = 6912) and slower without RMSNorm (3.18 ->
// 3.37 us), where the MFMAs overlap the unpacking better than the extra dot
// instructions do.
template <typename XT, int BITS, int NSB, bool RMS, bool FULL>
__device__ __forceinline__ void wave_decode(const GemvArgs& a, const float* gamma,
                                            float norm_eps) {
  // [sb][256] codes, then 64 zero bytes that the lanes feeding dead MFMA rows
  // (and blocks past K) read instead of masking their operands
  __shared__ __attribute__((aligned(16))) int8_t qw[NSB * 256 + 64];
  asm volatile("" ::"s"(a.K), "s"(a.N), "s"(a.c), "s"(a.y), "s"(a.x), "s"(a.Wp));
  if constexpr (RMS) asm volatile("" ::"s"(gamma), "s"(norm_eps));
  const float alpha = *a.alpha;
  const int lane = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  const int nKB = a.K >> 6;
  // x first (4 consecutive values per super-block), then the weights.
  const XT* x = reinterpret_cast<const XT*>(a.x);
  Raw4<XT> xraw[NSB];
  const bool use_g = RMS && gamma;
  const float* gp = use_g ? gamma : reinterpret_cast<const float*>(a.x);
  float4 graw[RMS ? NSB : 1];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const int k0 = 256 * sb + 4 * lane;
    const int kc = (FULL || k0 < a.K) ? k0 : 0;
    raw_load4(x, (size_t)kc, xraw[sb]);
    if (RMS) graw[RMS ? sb : 0] = *reinterpret_cast<const float4*>(gp + (use_g ? kc : 0));
  }
  uint4 p[NSB];
  {
    const size_t row_bytes = (size_t)(a.K >> 2);
    const int n = blockIdx.x * 16 + col;
    const int nc = n < a.N ? n : a.N - 1;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      const int kb = sb * 4 + grp;
      const int kbc = (FULL || kb < nKB) ? kb : nKB - 1;
      // an out-of-range block meets all-zero codes below
      p[sb] = *reinterpret_cast<const uint4*>(a.Wp + (size_t)nc * row_bytes + (size_t)kbc * 16);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  float v[NSB][4];
  float st = 0.0f, sq = 0.0f;
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const bool own = FULL || 256 * sb + 4 * lane < a.K;
    widen4(xraw[sb], v[sb]);
    if constexpr (RMS) {
      const float g[4] = {use_g ? graw[sb].x : 1.0f, use_g ? graw[sb].y : 1.0f,
                          use_g ? graw[sb].z : 1.0f, use_g ? graw[sb].w : 1.0f};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sq += own ? v[sb][e] * v[sb][e] : 0.0f;
        v[sb][e] *= g[e];
      }
    }
    if (BITS == 8) {
      const float m = max3_abs(v[sb][2], v[sb][3], max3_abs(v[sb][0], v[sb][1], st));
      st = own ? m : st;
    } else {
      const float sr = (fabsf(v[sb][0]) + fabsf(v[sb][1])) + (fabsf(v[sb][2]) + fabsf(v[sb][3]));
      st += own ? sr : 0.0f;
    }
  }
  st = (BITS == 8) ? wave_max_nonneg(st) : wave_reduce<false>(st);
  if (BITS == 4) st = st / (float)a.K;
  float mult;
  if constexpr (RMS) {
    const float rms = sqrtf(wave_reduce<false>(sq) / (float)a.K + norm_eps);
    mult = a.c / (st + kEps * rms);
    st = st / rms + kEps;
  } else {
    st += kEps;
    mult = a.c / st;
  }
  // Codes: adding 1.5 * 2^23 to the rounded product p leaves rint(p) (ties to
  // even, |p| < 2^22) in the low bits of the sum, so one add replaces round
  // and convert, med3 clamps, and the code is the sum's low byte. The product
  // is rounded first, as in the quantizer kernels: the empty asm keeps the
  // compiler from fusing the multiply into the add.
  constexpr float kMagic = 12582912.0f;
  const float lo = kMagic + ((BITS == 8) ? -128.0f : -8.0f);
  const float hi = kMagic + ((BITS == 8) ? 127.0f : 7.0f);
  int qsum = 0;  // this lane's share of the code row sum
  unsigned cw[NSB];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const bool own = FULL || 256 * sb + 4 * lane < a.K;
    unsigned b[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pr = v[sb][e] * mult;
      asm volatile("" : "+v"(pr));
      b[e] = __float_as_uint(__builtin_amdgcn_fmed3f(pr + kMagic, lo, hi));
    }
    // low bytes of b[0..3] -> one word (byte e = code e)
    const unsigned w01 = __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u);
    const unsigned w23 = __builtin_amdgcn_perm(b[3], b[2], 0x04000C0Cu);
    const unsigned word = own ? (w01 | w23) : 0u;
    qsum = __builtin_amdgcn_sdot4((int)word, 0x01010101, qsum, false);
    cw[sb] = word;
    if constexpr (!RMS) *reinterpret_cast<unsigned*>(qw + sb * 256 + 4 * lane) = word;
  }
  if constexpr (RMS) {
    wave_decode_dot<NSB>(a, p, cw, qsum, alpha, st, lane);
    return;
  }
  if (lane < 16) *reinterpret_cast<unsigned*>(qw + NSB * 256 + 4 * lane) = 0u;
  // Codes written by this wave are read back by other lanes of it; LDS serves
  // a wave's accesses in order, so only the compiler needs fencing.
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // Wave-wide code row sum (exact int32 in float-free DPP steps).
  qsum = wave_sum_int(qsum);

  // MFMA operand: lane (col, grp) feeds token row col (only row 0 is live),
  // block 4 sb + grp, times the stored field u = t + 1 in {0, 1, 2};
  // q . t = q . u - sum(q). The fields of quarters 0, 1 and 2 are masked in
  // place, worth u, 4u and 16u, and quarter 3's is shifted down to the
  // 16u position; three accumulators keep the scales apart and are shifted
  // back (exactly: each holds a multiple of its scale) at the end. One
  // operation per four weights for three quarters of the weights.
  // The code operands of the first kPre super-blocks are read from LDS
  // before the first MFMA (16 VGPRs each, which one wave per SIMD can spare
  // up to about ten times over): reading one super-block ahead left each
  // super-block's MFMAs waiting on their LDS reads (3.55 -> 3.47 us at ten
  // super-blocks). Later ones are read in the loop.
  constexpr int kPre = NSB < 10 ? NSB : 10;
  auto operands = [&](const int sb, v4i (&o)[4]) {
    const int kb = sb * 4 + grp;
    const int8_t* qr = ((FULL || kb < nKB) && col == 0) ? qw + sb * 256 + grp * 64 : qw + NSB * 256;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = *reinterpret_cast<const v4i*>(qr + 16 * j);
  };
  v4i av[NSB][4];
#pragma unroll
  for (int sb = 0; sb < kPre; ++sb) operands(sb, av[sb]);
  __builtin_amdgcn_sched_barrier(0);
  v4i acc1 = v4i{0, 0, 0, 0}, acc4 = v4i{0, 0, 0, 0}, acc16 = v4i{0, 0, 0, 0};
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    if (sb >= kPre) operands(sb, av[sb]);
    const uint4 pw = p[sb];
    v4i u;
    u.x = (int)(pw.x & 0x03030303u); u.y = (int)(pw.y & 0x03030303u);
    u.z = (int)(pw.z & 0x03030303u); u.w = (int)(pw.w & 0x03030303u);
    acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[sb][0], u, acc1, 0, 0, 0);
    u.x = (int)(pw.x & 0x0C0C0C0Cu); u.y = (int)(pw.y & 0x0C0C0C0Cu);
    u.z = (int)(pw.z & 0x0C0C0C0Cu); u.w = (int)(pw.w & 0x0C0C0C0Cu);
    acc4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[sb][1], u, acc4, 0, 0, 0);
    u.x = (int)(pw.x & 0x30303030u); u.y = (int)(pw.y & 0x30303030u);
    u.z = (int)(pw.z & 0x30303030u); u.w = (int)(pw.w & 0x30303030u);
    acc16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[sb][2], u, acc16, 0, 0, 0);
    u.x = (int)((pw.x >> 2) & 0x30303030u); u.y = (int)((pw.y >> 2) & 0x30303030u);
    u.z = (int)((pw.z >> 2) & 0x30303030u); u.w = (int)((pw.w >> 2) & 0x30303030u);
    acc16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[sb][3], u, acc16, 0, 0, 0);
  }
  const int dot = acc1[0] + (acc4[0] >> 2) + (acc16[0] >> 4) - qsum;
  // 16x16 layout: lane holds rows 4 (lane / 16) + v, column lane % 16; row 0
  // sits in element 0 of the lanes of group 0.
  const int n = blockIdx.x * 16 + col;
  if (grp == 0 && n < a.N) a.y[n] = (float)dot * dequant_factor(alpha, st, a.c);
}

// Scalar kernel arguments, the first two of which (the x and weight
// addresses) this file is built to have the command processor preload into
// SGPRs before the wave starts, so that the x and weight loads need not wait
// for a load of the argument block. Measured at M = 1, K = 2560, N = 6912
// (cold weights, 200 launches per replay): the forward without RMSNorm takes
// 3.45 us reading the argument block and about 3.1-3.2 us with the first two
// to six arguments preloaded (3.67 us with all seven); with RMSNorm 4.00 ->
// 3.67 us.
template <typename XT, int BITS, int NSB, bool FULL>
__global__ __launch_bounds__(64) void wave_decode_kernel(const void* x_in, const uint8_t* Wp,
                                                         const float* alpha_p, float* y, int K,
                                                         int N, float c) {
  GemvArgs a{};
  a.x = x_in;
  a.Wp = Wp;
  a.alpha = alpha_p;
  a.y = y;
  a.K = K;
  a.N = N;
  a.c = c;
  wave_decode<XT, BITS, NSB, false, FULL>(a, nullptr, 0.0f);
}

template <typename XT, int BITS, int NSB, bool FULL>
__global__ __launch_bounds__(64) void wave_decode_rms_kernel(const void* x_in, const uint8_t* Wp,
                                                             const float* alpha_p, float* y,
                                                             int K, int N, float c,
                                                             const float* gamma, float norm_eps) {
  GemvArgs a{};
  a.x = x_in;
  a.Wp = Wp;
  a.alpha = alpha_p;
  a.y = y;
  a.K = K;
  a.N = N;
  a.c = c;
  wave_decode<XT, BITS, NSB, true, FULL>(a, gamma, norm_eps);
}

template <typename Kern>
hipError_t ensure_lds(Kern kern, size_t bytes) {
  if (bytes <= 48 * 1024) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <int CT, bool OUT_I32, bool NIB, bool RSG>
hipError_t launch_gemv_ct(const GemvPlan& p, const GemvArgs& a, const int32_t* rowsum,
                          hipStream_t stream) {
  // Whole-line weight loads by pairs of super-blocks when every pair is
  // whole (K % 512 == 0) and there are enough pairs to give every wave one;
  // on nibble codes only (int8 codes take twice the registers, and the pair
  // layout would spill them).
  if constexpr (NIB) {
    const int nSB = ((a.K >> 6) + 3) >> 2;
    if (a.K % 512 == 0 && nSB / 2 >= p.sb_waves) {
      const size_t lds = (size_t)(p.threads / 64) * gemv_lds_per_wave<CT, true>();
      auto kern = ternary_gemv_kernel<CT, OUT_I32, NIB, RSG, true>;
      hipError_t e = ensure_lds(kern, lds);
      if (e != hipSuccess) return e;
      kern<<<dim3((unsigned)p.col_groups), dim3(p.threads), lds, stream>>>(
        a.Wp, a.codes, a.scales, a.alpha, a.y, a.acc_out, rowsum, a.M, a.K, a.N, a.sb_waves, a.c);
      return hipGetLastError();
    }
  }
  const size_t lds = (size_t)(p.threads / 64) * gemv_lds_per_wave<CT, false>();
  auto kern = ternary_gemv_kernel<CT, OUT_I32, NIB, RSG, false>;
  hipError_t e = ensure_lds(kern, lds);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)p.col_groups), dim3(p.threads), lds, stream>>>(
        a.Wp, a.codes, a.scales, a.alpha, a.y, a.acc_out, rowsum, a.M, a.K, a.N, a.sb_waves, a.c);
  return hipGetLastError();
}

template <typename XT, int BITS, int MG, int CT, int SBW, bool PRO, bool HAD>
hipError_t launch_fused_ct(const GemvArgs& a, const Prologue& pro, hipStream_t stream) {
  const int nSB = ((a.K >> 6) + 3) >> 2;
  // at least CT waves: the finish stores column tile ct from wave ct
  const int nw = (nSB + SBW - 1) / SBW > CT ? (nSB + SBW - 1) / SBW : CT;
  const size_t lds = (size_t)nw * CT * 1024 + 2 * (size_t)nw * 16 * 4 +
                     (PRO ? (size_t)nw * 16 * 4 : 0) + (size_t)nw * SBW * a.M * 256;
  auto kern = fused_decode_kernel<XT, BITS, MG, CT, SBW, PRO, HAD>;
  hipError_t e = ensure_lds(kern, lds);
  if (e != hipSuccess) return e;
  const unsigned groups = (unsigned)((a.N + 16 * CT - 1) / (16 * CT));
  kern<<<dim3(groups), dim3(64 * nw), lds, stream>>>(a.x, a.Wp, a.alpha, a.y, a.M, a.K, a.N, a.c,
                                                    pro.up, pro.gamma, pro.norm_eps, pro.rms);
  return hipGetLastError();
}

template <typename XT, int BITS, int NSB, bool FULL>
void launch_wave_full(const GemvArgs& a, const Prologue* pro, hipStream_t stream) {
  const dim3 grid((unsigned)((a.N + 15) / 16));
  if (pro && pro->rms)
    wave_decode_rms_kernel<XT, BITS, NSB, FULL><<<grid, dim3(64), 0, stream>>>(
        a.x, a.Wp, a.alpha, a.y, a.K, a.N, a.c, pro->gamma, pro->norm_eps);
  else
    wave_decode_kernel<XT, BITS, NSB, FULL><<<grid, dim3(64), 0, stream>>>(a.x, a.Wp, a.alpha, a.y,
                                                                        a.K, a.N, a.c);
}

// FULL: every super-block is whole (K = 256 NSB), so the kernel drops its
// range checks (703 -> 596 VALU per wave at K = 2560: 3.49 -> 3.45 us).
// With the RMSNorm prologue the same variant measured slower (3.67 ->
// 3.92 us), so that one keeps its checks.
template <typename XT, int BITS, int NSB>
hipError_t launch_wave_nsb(const GemvArgs& a, const Prologue* pro, hipStream_t stream) {
  if (a.K == 256 * NSB && !(pro && pro->rms))
    launch_wave_full<XT, BITS, NSB, true>(a, pro, stream);
  else
    launch_wave_full<XT, BITS, NSB, false>(a, pro, stream);
  return hipGetLastError();
}

// The one-wave kernel for a single token, with or without RMSNorm; the
// SwiGLU product (an exponential per element) is better spread over the
// multi-wave kernel's waves.
template <typename XT, int BITS>
bool try_launch_wave(const GemvArgs& a, const Prologue* pro, hipStream_t stream, hipError_t* err) {
  const int nsb = ((a.K >> 6) + 3) >> 2;
  if (a.M != 1 || (pro && pro->up) || nsb > 16) return false;
  switch (nsb) {
#define BITNET_WAVE_CASE(n) \
  case n: *err = launch_wave_nsb<XT, BITS, n>(a, pro, stream); break;
    BITNET_WAVE_CASE(1) BITNET_WAVE_CASE(2) BITNET_WAVE_CASE(3) BITNET_WAVE_CASE(4)
    BITNET_WAVE_CASE(5) BITNET_WAVE_CASE(6) BITNET_WAVE_CASE(7) BITNET_WAVE_CASE(8)
    BITNET_WAVE_CASE(9) BITNET_WAVE_CASE(10) BITNET_WAVE_CASE(11) BITNET_WAVE_CASE(12)
    BITNET_WAVE_CASE(13) BITNET_WAVE_CASE(14) BITNET_WAVE_CASE(15) BITNET_WAVE_CASE(16)
#undef BITNET_WAVE_CASE
    default: return false;
  }
  return true;
}

template <typename XT, int BITS, int MG>
hipError_t launch_fused_t(const GemvArgs& a, const Prologue* pro, hipStream_t stream, bool had) {
  const Prologue none{nullptr, nullptr, 0.0f, 0};
  if (had) {
    if (pro) return launch_fused_ct<XT, BITS, MG, kFusedHadCt, kFusedSbw, true, true>(a, *pro, stream);
    return launch_fused_ct<XT, BITS, MG, kFusedHadCt, kFusedSbw, false, true>(a, none, stream);
  }
  hipError_t err = hipSuccess;
  if (try_launch_wave<XT, BITS>(a, pro, stream, &err)) return err;
  if (pro) return launch_fused_ct<XT, BITS, MG, kFusedCt, kFusedSbw, true, false>(a, *pro, stream);
  return launch_fused_ct<XT, BITS, MG, kFusedCt, kFusedSbw, false, false>(a, none, stream);
}

}  // namespace

hipError_t launch_gemv(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, hipStream_t stream, bool nibbles, const int32_t* rowsum) {
  if (nibbles && (M > kDecodeMaxM || K % kNibbleKMultiple != 0)) return hipErrorInvalidValue;
  const GemvPlan p = plan_gemv(M, K, N, false, false);
  GemvArgs a{};
  a.codes = codes;
  a.scales = scales;
  a.Wp = Wpacked;
  a.alpha = alpha;
  a.y = y;
  a.acc_out = acc;
  a.M = (int)M;
  a.K = K;
  a.N = (int)N;
  a.sb_waves = p.sb_waves;
  a.c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  if (acc)
    return nibbles ? launch_gemv_ct<1, true, true, false>(p, a, nullptr, stream)
                   : launch_gemv_ct<1, true, false, false>(p, a, nullptr, stream);
  if (rowsum)
    return nibbles ? launch_gemv_ct<1, false, true, true>(p, a, rowsum, stream)
                   : launch_gemv_ct<1, false, false, true>(p, a, rowsum, stream);
  return nibbles ? launch_gemv_ct<1, false, true, false>(p, a, nullptr, stream)
                 : launch_gemv_ct<1, false, false, false>(p, a, nullptr, stream);
}

hipError_t launch_fused_decode(const void* x, int x_dtype, int64_t M, int K,
                               const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                               float* y, hipStream_t stream, const Prologue* pro, int hadamard) {
  const bool had = hadamard != 0;
  const GemvPlan p = plan_gemv(M, K, N, true, had);
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
  a.c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  if (M == 1) {  // single token: the smallest code, which a cold launch fetches fastest
    if (x_dtype == 1)
      return bits == 8 ? launch_fused_t<uint16_t, 8, 1>(a, pro, stream, had)
                       : launch_fused_t<uint16_t, 4, 1>(a, pro, stream, had);
    return bits == 8 ? launch_fused_t<float, 8, 1>(a, pro, stream, had)
                     : launch_fused_t<float, 4, 1>(a, pro, stream, had);
  }
  if (M <= 4) {
    if (x_dtype == 1)
      return bits == 8 ? launch_fused_t<uint16_t, 8, 4>(a, pro, stream, had)
                       : launch_fused_t<uint16_t, 4, 4>(a, pro, stream, had);
    return bits == 8 ? launch_fused_t<float, 8, 4>(a, pro, stream, had)
                     : launch_fused_t<float, 4, 4>(a, pro, stream, had);
  }
  if (x_dtype == 1)
    return bits == 8 ? launch_fused_t<uint16_t, 8, 16>(a, pro, stream, had)
                     : launch_fused_t<uint16_t, 4, 16>(a, pro, stream, had);
  return bits == 8 ? launch_fused_t<float, 8, 16>(a, pro, stream, had)
                   : launch_fused_t<float, 4, 16>(a, pro, stream, had);
}

}  // namespace bitnet
