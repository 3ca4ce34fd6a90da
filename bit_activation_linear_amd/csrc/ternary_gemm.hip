// Prefill-shape (M > 16 tokens) ternary mpGEMM on v_mfma_i32_32x32x32_i8 with
// exact int32 accumulation and a fused dequantization epilogue.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), HBitLinear.forward: the
// output F.linear(Q_act(x_r), alpha * t) equals (q . t^T) * alpha * s / c
// with integer codes q (Eq. 5-6) and ternary t (Eq. 1); the BitNet blog
// page's BitLinear_b158 takes the same integer-product-then-rescale form.
// |q| <= 128 and K <= 32768 keep every int32 sum exact.
//
// Work decomposition. A workgroup owns a BM x BN output tile and has
// WMW x WNW x KS waves: each wave owns a (32 RT) x (32 CT) block of it
// (RT x CT accumulators of 32x32 int32 in AGPRs) and one of KS interleaved
// 128-wide k slices of every stage; with KS > 1 the slices' partial sums are
// added through LDS at the end.
//
// Staging. Codes and packed weights go from global memory straight into LDS
// (buffer_load_dwordx4 with the lds bit: each lane's 16 bytes land at
// base + 16 * lane), so no register holds a tile in transit. LDS is a ring of three stage slots:
// stage s + 2 is being fetched while stage s is multiplied, and one
// workgroup barrier per stage both publishes a stage and frees the slot
// after it. Codes keep their 128-byte k rows, with the 16-byte chunks of a
// row permuted by a row-dependent XOR so that the 32 rows one MFMA operand
// read touches fall on distinct LDS banks; the permutation is applied by
// choosing which global chunk each lane fetches, so every fetch still reads
// whole 128-byte rows. Packed weights keep their 16-byte blocks, laid out so
// that lane l of an operand read takes the block of column l.
//
// Expansion. Each wave expands the packed weights it multiplies in
// registers: a 16-byte block of one column holds 64 weights, of which a lane
// needs the 16 of its k quarter; a shift, a mask and one v_perm_b32 per four
// weights turn the 2-bit codes into int8 {-1, 0, +1}.
//
// MFMA operands. For the 32x32x32 instruction lane l supplies row (or column)
// l % 32 and the 16 consecutive k of group g = l / 32. Sub-step h (k32) of a
// slice uses k = 32h + 16g + [0, 16) for both operands.
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

constexpr int BKW = 128;   // k per wave slice per stage
constexpr int kSlots = 3;  // LDS ring depth
constexpr int kXcds = 8;
constexpr int kBand = 4;

template <int RT, int CT, int WMW, int WNW, int KS>
struct Shape {
  static constexpr int NW = WMW * WNW * KS;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * RT * WMW;
  static constexpr int BN = 32 * CT * WNW;
  static constexpr int SK = BKW * KS;        // k per stage
  static constexpr int A_BYTES = BM * SK;    // codes of a stage
  static constexpr int B_BYTES = BN * SK / 4;  // packed weights of a stage
  static constexpr int SLOT = A_BYTES + B_BYTES;
  static constexpr int NA = A_BYTES / 1024;  // 1-KB direct loads per stage
  static constexpr int NB = B_BYTES / 1024;
  static constexpr int NA_W = NA / NW;       // ... per wave
  static constexpr int NB_W = NB / NW;
  static constexpr int LDS = kSlots * SLOT;
  static constexpr int PART = RT * CT * 4096;  // one wave's accumulators in bytes
  static_assert(NA_W * NW == NA && NB_W * NW == NB && NB_W >= 1, "uneven staging");
  static_assert(KS == 1 || (KS / 2) * WMW * WNW * PART <= LDS, "reduction does not fit");
};

// Buffer resource over [base, base + bytes): raw (stride 0) dword access;
// loads at or past `bytes` return zero.
typedef unsigned u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u4 make_rsrc(const void* base, unsigned bytes) {
  const size_t a = reinterpret_cast<size_t>(base);
  u4 r;
  r.x = (unsigned)a;
  r.y = (unsigned)(a >> 32) & 0xFFFFu;
  r.z = bytes;
  r.w = 0x00020000u;
  return r;
}

// LDS byte address of a pointer into the dynamic shared array.
__device__ __forceinline__ unsigned lds_address(const char* p) {
  typedef const __attribute__((address_space(3))) char lds_char;
  return (unsigned)(size_t)(lds_char*)p;
}

// 16 bytes per lane from buffer offset voff straight into LDS at
// lds + 16 * lane (lds is wave-uniform; the instruction takes it from M0,
// which is saved and restored around it). Written as inline assembly so that
// the compiler, which cannot tell which LDS bytes such a load writes, does not
// wait for it before every LDS read: completion is tracked by hand with
// s_waitcnt vmcnt before the workgroup barrier that publishes a stage.
__device__ __forceinline__ void load_lds16(const u4 rsrc, int voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds)
      : "memory");
}

// XOR applied to the 16-byte chunk index of code row r in LDS.
__device__ __forceinline__ int chunk_swizzle(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define BITNET_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

__device__ __forceinline__ v4i expand_shifted(const uint4 p, int sh) {
  v4i r;
  r.x = (int)__builtin_amdgcn_perm(0u, kCodeLut, (p.x >> sh) & 0x03030303u);
  r.y = (int)__builtin_amdgcn_perm(0u, kCodeLut, (p.y >> sh) & 0x03030303u);
  r.z = (int)__builtin_amdgcn_perm(0u, kCodeLut, (p.z >> sh) & 0x03030303u);
  r.w = (int)__builtin_amdgcn_perm(0u, kCodeLut, (p.w >> sh) & 0x03030303u);
  return r;
}

template <int RT, int CT, int WMW, int WNW, int KS, bool OUT_I32>
__global__ __launch_bounds__(64 * WMW * WNW * KS) void ternary_gemm_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ scales, int M, int K,
    const uint8_t* __restrict__ Wp, int N, const float* __restrict__ alpha_p, float c,
    float* __restrict__ y, int32_t* __restrict__ acc_out, int tiles_m, int tiles_n) {
  using S = Shape<RT, CT, WMW, WNW, KS>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // XCD-aware tile order.
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int tile = (L % kXcds) * per_xcd + L / kXcds;
  if (tile >= tiles) return;
  const int band = tile / (kBand * tiles_n);
  const int band_m = (tiles_m - band * kBand) < kBand ? (tiles_m - band * kBand) : kBand;
  const int in_band = tile - band * kBand * tiles_n;
  const int m0 = (band * kBand + in_band % band_m) * S::BM;
  const int n0 = (in_band / band_m) * S::BN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wave / (WMW * WNW);
  const int wmn = wave % (WMW * WNW);
  const int wm = wmn / WNW, wn = wmn % WNW;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int nKB = K >> 6;
  const int wrow = K >> 2;

  // Direct-load addressing. Load q of a stage (q = wave + NW * i) fills one
  // KB of LDS: for codes, 8 rows of one k slice; for weights, both blocks of
  // one slice for 32 columns. The loads go through buffer resources that end
  // at the tile's last valid row (column): rows past M and columns past N
  // read as zero, and k past K reads either the next row's bytes or zero --
  // in both cases data that is never multiplied, and never a fault.
  const u4 a_rsrc = make_rsrc(codes + (size_t)m0 * K,
                              (unsigned)((M - m0 < S::BM ? M - m0 : S::BM) * K));
  const u4 b_rsrc = make_rsrc(Wp + (size_t)n0 * wrow,
                              (unsigned)((N - n0 < S::BN ? N - n0 : S::BN) * wrow));
  const unsigned lds0 = lds_address(smem);
  int a_voff[S::NA_W], b_voff[S::NB_W];
  unsigned a_lds[S::NA_W], b_lds[S::NB_W];
#pragma unroll
  for (int i = 0; i < S::NA_W; ++i) {
    const int q = wave + S::NW * i;
    const int slice = q / (S::BM / 8), rb = q % (S::BM / 8);
    const int r = rb * 8 + (lane >> 3);
    a_voff[i] = r * K + slice * BKW + 16 * ((lane & 7) ^ chunk_swizzle(r));
    a_lds[i] = lds0 + slice * S::BM * BKW + rb * 1024;
  }
#pragma unroll
  for (int i = 0; i < S::NB_W; ++i) {
    const int q = wave + S::NW * i;
    const int slice = q / (S::BN / 32), cg = q % (S::BN / 32);
    b_voff[i] = (cg * 32 + l32) * wrow + (slice * 2 + g) * 16;
    b_lds[i] = lds0 + S::A_BYTES + slice * (S::BN / 32) * 1024 + cg * 1024;
  }

#define BITNET_ISSUE(ks_, slot_)                                                                \
  {                                                                                             \
    const unsigned so_ = (unsigned)(slot_) * S::SLOT;                                           \
    const int ka_ = (ks_) * S::SK, kb_ = (ks_) * S::SK / 4;                                     \
    _Pragma("unroll") for (int i = 0; i < S::NA_W; ++i)                                         \
        load_lds16(a_rsrc, a_voff[i] + ka_, a_lds[i] + so_);                                    \
    _Pragma("unroll") for (int i = 0; i < S::NB_W; ++i)                                         \
        load_lds16(b_rsrc, b_voff[i] + kb_, b_lds[i] + so_);                                    \
  }

  // Operand reads. Codes: row wm*32RT + rt*32 + l32 of this wave's slice,
  // logical chunk 2h + g (sub-step h) at its swizzled position. Weights:
  // block blk of column wn*32CT + ct*32 + l32.
  int a_rd[4];
  {
    const int r = wm * 32 * RT + l32;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      a_rd[h] = kw * S::BM * BKW + r * BKW + 16 * ((2 * h + g) ^ chunk_swizzle(r));
  }
  const int b_rd = S::A_BYTES + kw * (S::BN / 32) * 1024 + wn * CT * 1024 + 16 * l32;

  v16i acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0;

  // One 64-weight block (two k32 sub-steps) of the slice in slot slot_.
#define BITNET_BLOCK(slot_, blk_)                                                               \
  {                                                                                             \
    const char* sb_ = smem + (slot_) * S::SLOT;                                                 \
    uint4 pw_[CT];                                                                              \
    _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) pw_[ct] =                                 \
        *reinterpret_cast<const uint4*>(sb_ + b_rd + ct * 1024 + (blk_) * 512);                 \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh) {                                          \
      v4i af_[RT];                                                                              \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) af_[rt] =                               \
          *reinterpret_cast<const v4i*>(sb_ + a_rd[2 * (blk_) + hh] + rt * 32 * BKW);           \
      v4i bf_[CT];                                                                              \
      _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) bf_[ct] =                               \
          expand_shifted(pw_[ct], 2 * g + 4 * hh);                                              \
      _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                         \
          _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) acc[rt][ct] =                       \
              __builtin_amdgcn_mfma_i32_32x32x32_i8(af_[rt], bf_[ct], acc[rt][ct], 0, 0, 0);    \
    }                                                                                           \
  }

  constexpr int kLoadsPerStage = S::NA_W + S::NB_W;
  const int nst = (nKB + 2 * KS - 1) / (2 * KS);  // stages, the last possibly partial
  const int nfull = nKB / (2 * KS);               // stages whose every slice is whole

  BITNET_ISSUE(0, 0)
  if (nst > 1) BITNET_ISSUE(1, 1)
  int slot = 0;
  for (int ks = 0; ks < nfull; ++ks) {
    // This wave's loads of stage ks are done once at most the next stage's
    // are outstanding; the barrier then makes every wave's loads visible and
    // guarantees that stage ks - 1's slot is no longer being read.
    if (ks + 1 < nst) {
      BITNET_WAIT_VMCNT(kLoadsPerStage);
    } else {
      BITNET_WAIT_VMCNT(0);
    }
    lds_barrier();
    if (ks + 2 < nst) {
      const int ns = slot == 0 ? 2 : slot - 1;  // (ks + 2) % 3
      BITNET_ISSUE(ks + 2, ns)
    }
    BITNET_BLOCK(slot, 0)
    BITNET_BLOCK(slot, 1)
    slot = slot == 2 ? 0 : slot + 1;
  }
  if (nst > nfull) {
    // Partial last stage: this wave's slice holds vb whole blocks (0..2).
    BITNET_WAIT_VMCNT(0);
    lds_barrier();
    const int vb = nKB - nfull * 2 * KS - 2 * kw;
    if (vb >= 1) BITNET_BLOCK(slot, 0)
    if (vb >= 2) BITNET_BLOCK(slot, 1)
  }
#undef BITNET_ISSUE
#undef BITNET_BLOCK

  if constexpr (KS > 1) {
    // Add the k slices' partial sums through LDS, halving the number of
    // live slices per round; slice 0's waves end up with the full sums.
    BITNET_WAIT_VMCNT(0);
    lds_barrier();
#pragma unroll
    for (int step = KS / 2; step >= 1; step >>= 1) {
      if (kw >= step && kw < 2 * step) {
        char* p = smem + ((kw - step) * WMW * WNW + wmn) * S::PART + 16 * lane;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              v4i t;
              t.x = acc[rt][ct][4 * qd + 0];
              t.y = acc[rt][ct][4 * qd + 1];
              t.z = acc[rt][ct][4 * qd + 2];
              t.w = acc[rt][ct][4 * qd + 3];
              *reinterpret_cast<v4i*>(p + ((rt * CT + ct) * 4 + qd) * 1024) = t;
            }
      }
      lds_barrier();
      if (kw < step) {
        const char* p = smem + (kw * WMW * WNW + wmn) * S::PART + 16 * lane;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
              const v4i t = *reinterpret_cast<const v4i*>(p + ((rt * CT + ct) * 4 + qd) * 1024);
              acc[rt][ct][4 * qd + 0] += t.x;
              acc[rt][ct][4 * qd + 1] += t.y;
              acc[rt][ct][4 * qd + 2] += t.z;
              acc[rt][ct][4 * qd + 3] += t.w;
            }
      }
      lds_barrier();
    }
    if (kw != 0) return;
  } else {
    // No load may still be writing LDS when the workgroup retires.
    BITNET_WAIT_VMCNT(0);
  }

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

template <int RT, int CT, int WMW, int WNW, int KS, bool OUT_I32>
hipError_t launch_tile(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, float c, float* y,
                       int32_t* acc, hipStream_t stream) {
  using S = Shape<RT, CT, WMW, WNW, KS>;
  const int tiles_m = (int)((M + S::BM - 1) / S::BM);
  const int tiles_n = (int)((N + S::BN - 1) / S::BN);
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  auto kern = ternary_gemm_kernel<RT, CT, WMW, WNW, KS, OUT_I32>;
  if (S::LDS > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3((unsigned)(per_xcd * kXcds)), dim3(S::NT), S::LDS, stream>>>(
      codes, scales, (int)M, K, Wpacked, (int)N, alpha, c, y, acc, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int RT, int CT, int WMW, int WNW, int KS>
hipError_t launch_variant(const int8_t* codes, const float* scales, int64_t M, int K,
                          const uint8_t* Wpacked, int64_t N, const float* alpha, float c, float* y,
                          int32_t* acc, hipStream_t stream) {
  return acc ? launch_tile<RT, CT, WMW, WNW, KS, true>(codes, scales, M, K, Wpacked, N, alpha, c,
                                                       y, acc, stream)
             : launch_tile<RT, CT, WMW, WNW, KS, false>(codes, scales, M, K, Wpacked, N, alpha, c,
                                                        y, acc, stream);
}

}  // namespace

hipError_t launch_gemm(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, hipStream_t stream) {
  const float c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  // 256 x 256 tiles (one k slice per stage) when there are enough of them to
  // give every CU several; otherwise 128 x 128 tiles whose four waves split
  // each 256-wide stage into two k slices.
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles >= 1024)
    return launch_variant<4, 4, 2, 2, 1>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, stream);
  return launch_variant<4, 2, 1, 2, 2>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, stream);
}

hipError_t launch_ternary_matmul(const int8_t* codes, const float* scales, int64_t M, int K,
                                 const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                                 float* y, int32_t* acc, hipStream_t stream) {
  if (M <= kDecodeMaxM)
    return launch_gemv(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream);
  return launch_gemm(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream);
}

}  // namespace bitnet
