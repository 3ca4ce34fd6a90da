// Prefill-shape (M > 16 tokens) ternary mpGEMM on v_mfma_i32_32x32x32_i8 with
// exact int32 accumulation and a fused dequantization epilogue.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py), HBitLinear.forward: the
// output F.linear(Q_act(x_r), alpha * t) equals (q . t^T) * alpha * s / c
// with integer codes q (Eq. 5-6) and ternary t (Eq. 1); the BitNet blog
// page's BitLinear_b158 takes the same integer-product-then-rescale form.
// |q| <= 128 and K <= 32768 keep every int32 sum exact.
//
// Weight operand. The MFMA multiplies the codes by the stored 2-bit field
// u = t + 1 in {0, 1, 2} rather than by t itself, and the epilogue subtracts
// the row sum of the codes: q . t = q . u - sum(q), exactly, in int32.
// Unpacking u is a shift and a mask per four weights (no byte remap), and
// the small non-negative operand toggles fewer MFMA input bits than
// {-1, 0, +1} = {0xFF, 0x00, 0x01}, which matters because the matrix cores
// of this chip lower their clock as operand switching activity rises. The
// forward passes the row sums the quantizer computed with the codes (RSG);
// given bare codes, the kernel sums the code fragments the MFMAs read
// anyway (v_dot4 with a vector of ones), which measured 10-19% of the
// kernel's time.
//
// Work decomposition. A workgroup owns a BM x BN output tile and has
// WMW x WNW x KS waves: each wave owns a (32 RT) x (32 CT) block of it
// (RT x CT accumulators of 32x32 int32) and one of KS interleaved
// 128-wide k slices of every stage; with KS > 1 the slices' partial sums are
// added through LDS at the end.
//
// Staging. Codes and packed weights go from global memory straight into LDS
// (buffer_load_dwordx4 with the lds bit: each lane's 16 bytes land at
// base + 16 * lane), so no register holds a tile in transit. LDS is a ring of
// SL stage slots (three, or two when a stage is too big for three): stage
// s + SL is fetched while the stages between are in flight or waiting, and
// one workgroup barrier per stage both publishes a stage and frees the slot
// of the one before it. The fetches are spread
// between MFMAs, since a wave issuing ten of them back to back stalls for
// hundreds of cycles. Codes keep their 128-byte k rows, with the 16-byte
// chunks of a row permuted by a row-dependent XOR so that the rows one MFMA
// operand read touches fall on distinct LDS banks; the permutation is
// applied by choosing which global chunk each lane fetches, so every fetch
// still reads whole 128-byte rows. Packed weights keep their 16-byte
// blocks, laid out so that lane l of an operand read takes the block of
// column l.
//
// Pipeline. Work advances in 64-weight blocks (two k32 sub-steps): while the
// MFMAs of one block run, the next block's operands are read from LDS, its
// weights unpacked and (without given row sums) its code row sums
// accumulated.
//
// Output. With N % 4 == 0 and a 16-byte aligned y, each 32x32 accumulator
// block is turned around through the drained LDS ring so that a lane stores
// 16 contiguous bytes of one row (a quarter of the store instructions, which
// measured 18% of the M=2048 K=8192 N=2048 product); otherwise lanes store
// single values. Large products given the row sums run the streamed-tile
// kernel further down instead, which also overlaps a tile's stores with the
// next tile's work.
//
// MFMA operands. For the 32x32x32 instruction lane l supplies row (or column)
// l % 32 and the 16 consecutive k of group g = l / 32. Sub-step h (k32) of a
// slice uses k = 32h + 16g + [0, 16) for both operands.
//
// FP8 pairs (F8; 4-bit codes the quantizer wrote as fp8 pairs, row sums
// given). The int4 codes are exact in fp8 E4M3 and u = t + 1 is exact in
// fp4 E2M1 as u / 2 (the field itself in a nibble's low bits), so one
// v_mfma_f32_32x32x64_f8f6f4 (fp8 A, fp4 B) multiplies a whole 64-weight
// block, exactly: every partial sum is a multiple of 1/2 below 2^19, and
// 2 acc = q . u. The B operand of lane group g is (p >> 2g) & 0x33333333 per
// packed word: nibble 2i + h of it (i = 4 d + c for byte c of word d) holds
// the weight 16 g + i + 32 h, and the quantizer stores that weight's code at
// byte 32 g + 2i + h of the block. The instruction pairs fp4 nibble e of
// lane group g with fp8 byte e % 16 of lane group (e / 16) when g = 0 and
// with byte 16 + e % 16 of that lane group when g = 1 (measured with a
// layout probe), so lane group g's fp8 operand is the block's bytes 16 g ..
// 16 g + 15 and then 32 + 16 g .. 32 + 16 g + 15: the same two 16-byte
// chunks as its two int8 sub-steps. Measured at M = 2048, K = 8192,
// N = 2048: half as many MFMA instructions and half the unpacking (a shift
// and a mask per eight weights instead of four) take the product from 39 to
// 34 us (a timing variant with fp6 codes, whose MFMA runs twice as fast,
// measured the same: the matrix pipe is not what holds this product).
//
// Tile order. Workgroups are dispatched round-robin over the eight XCDs
// (each with its own L2), so workgroup L runs on XCD L % 8. Each XCD gets a
// contiguous range of tiles walked band by band (four M-tiles wide), so the
// workgroups resident on one XCD at a time share code rows and weight columns
// through its L2.
#include "kernels.h"
#include "ternary_common.h"

namespace bitnet {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int BKW = 128;     // k per wave slice per stage

template <int RT, int CT, int WMW, int WNW, int KS>
struct Shape {
  static constexpr int NW = WMW * WNW * KS;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * RT * WMW;
  static constexpr int BN = 32 * CT * WNW;
  static constexpr int SK = BKW * KS;          // k per stage
  static constexpr int A_BYTES = BM * SK;      // codes of a stage
  static constexpr int B_BYTES = BN * SK / 4;  // packed weights of a stage
  static constexpr int SLOT = A_BYTES + B_BYTES;
  static constexpr int NA = A_BYTES / 1024;    // 1-KB direct loads per stage
  static constexpr int NB = B_BYTES / 1024;
  static constexpr int NA_W = NA / NW;         // ... per wave
  static constexpr int NB_W = NB / NW;
  static constexpr int NL_W = NA_W + NB_W;
  static constexpr int SL = (3 * SLOT <= kLdsMax) ? 3 : 2;  // LDS ring depth (stage slots)
  static constexpr int RING = SL * SLOT;
  static constexpr int ROWSUM = RING - KS * BM * 4;  // int32 row sums [KS][BM], after the ring drains
  static constexpr int LDS = RING;
  static constexpr int PART = RT * CT * 4096;  // one wave's accumulators in bytes
  // MFMA groups per 64-weight block in the interleaved schedule
  static constexpr int CH = (2 * RT * CT) < 8 ? 2 * RT * CT : 8;
  static_assert(NA_W * NW == NA && NB_W * NW == NB && NB_W >= 1, "uneven staging");
  static_assert(SLOT * 2 <= kLdsMax, "two stage slots do not fit in LDS");
  static_assert(KS == 1 || (KS / 2) * WMW * WNW * PART <= ROWSUM, "reduction does not fit");
  static_assert((2 * RT * CT) % CH == 0, "MFMA groups");
};

// The 2-bit fields at bit offset sh of each byte: u = t + 1 for 16 weights.
__device__ __forceinline__ v4i unpack_u(const uint4 p, int sh) {
  v4i r;
  r.x = (int)((p.x >> sh) & 0x03030303u);
  r.y = (int)((p.y >> sh) & 0x03030303u);
  r.z = (int)((p.z >> sh) & 0x03030303u);
  r.w = (int)((p.w >> sh) & 0x03030303u);
  return r;
}

// The fp4 (E2M1) B operand of lane group g: fields g and g + 2 of every byte
// of a packed block, each in a nibble's low bits (the value u / 2).
__device__ __forceinline__ v4i unpack_f4(const uint4 p, int g) {
  v4i r;
  r.x = (int)((p.x >> (2 * g)) & 0x33333333u);
  r.y = (int)((p.y >> (2 * g)) & 0x33333333u);
  r.z = (int)((p.z >> (2 * g)) & 0x33333333u);
  r.w = (int)((p.w >> (2 * g)) & 0x33333333u);
  return r;
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// acc += A (32 fp8 codes per lane, a0 then a1) x B (32 fp4 fields per lane),
// the accumulator kept as the bits of its fp32 values.
__device__ __forceinline__ v16i mma_f8f4(const v4i a0, const v4i a1, const v4i b, const v16i acc) {
  const v8i a = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
  const v8i bb = {b.x, b.y, b.z, b.w, 0, 0, 0, 0};  // fp4 reads the first four words
  return __builtin_bit_cast(
      v16i, __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bb, __builtin_bit_cast(v16f, acc),
                                                              0, 4, 0, 0, 0, 0));
}

// Sum of the 16 signed bytes of a code fragment, added to s.
__device__ __forceinline__ int add_bytes(const v4i a, int s) {
  s = __builtin_amdgcn_sdot4(a.x, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.y, 0x01010101, s, false);
  s = __builtin_amdgcn_sdot4(a.z, 0x01010101, s, false);
  return __builtin_amdgcn_sdot4(a.w, 0x01010101, s, false);
}

template <int RT, int CT, int WMW, int WNW, int KS, bool OUT_I32, bool RSG, bool WIDE, bool F8>
__global__ __launch_bounds__(64 * WMW * WNW * KS) void ternary_gemm_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ scales, int M, int K,
    const uint8_t* __restrict__ Wp, int N, const float* __restrict__ alpha_p, float c,
    float* __restrict__ y, int32_t* __restrict__ acc_out, const int32_t* __restrict__ rowsum_g,
    int tiles_m, int tiles_n) {
  using S = Shape<RT, CT, WMW, WNW, KS>;
  static_assert(!F8 || (RSG && !OUT_I32), "fp8 pairs come with their row sums");
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
  // in both cases data that is never multiplied, and never a fault. Fetches
  // of stages past the last go through empty resources: they write zeros to
  // a free slot and read no memory, which keeps every stage's load count,
  // and so the vmcnt bookkeeping, uniform.
  const u4 a_rsrc = make_rsrc(codes + (size_t)m0 * K,
                              (unsigned)((M - m0 < S::BM ? M - m0 : S::BM) * K));
  const u4 b_rsrc = make_rsrc(Wp + (size_t)n0 * wrow,
                              (unsigned)((N - n0 < S::BN ? N - n0 : S::BN) * wrow));
  u4 a_none = a_rsrc, b_none = b_rsrc;
  a_none.z = 0;
  b_none.z = 0;
  const unsigned lds0 = lds_address(smem);
  // Lane parts of the load offsets; everything else about load i of a stage
  // is wave-uniform. Code row r = 8 rb + lane / 8 takes global chunk
  // (lane % 8) ^ swizzle(r), and swizzle(r) = lane / 8 ^ (rb & 1).
  const int a_lane0 = (lane >> 3) * K + 16 * ((lane & 7) ^ (lane >> 3));
  const int a_lane1 = (lane >> 3) * K + 16 * ((lane & 7) ^ (lane >> 3) ^ 1);
  const int b_lane = l32 * wrow + g * 16;
  // Load i of stage ks_ into slot slot_.
#define BITNET_LOAD(ks_, slot_, i)                                                              \
  {                                                                                             \
    const bool live_ = (ks_) < nst;                                                             \
    if ((i) < S::NA_W) {                                                                        \
      const int q_ = wave + S::NW * (i);                                                        \
      const int slice_ = q_ / (S::BM / 8), rb_ = q_ % (S::BM / 8);                              \
      load_lds16(live_ ? a_rsrc : a_none,                                                       \
                 ((rb_ & 1) ? a_lane1 : a_lane0) + rb_ * 8 * K + slice_ * BKW + (ks_) * S::SK,  \
                 lds0 + (unsigned)((slot_) * S::SLOT + slice_ * S::BM * BKW + rb_ * 1024));     \
    } else {                                                                                    \
      const int q_ = wave + S::NW * ((i) - S::NA_W);                                            \
      const int slice_ = q_ / (S::BN / 32), cg_ = q_ % (S::BN / 32);                            \
      load_lds16(live_ ? b_rsrc : b_none,                                                       \
                 b_lane + cg_ * 32 * wrow + slice_ * 32 + (ks_) * (S::SK / 4),                  \
                 lds0 + (unsigned)((slot_) * S::SLOT + S::A_BYTES +                             \
                                   (slice_ * (S::BN / 32) + cg_) * 1024));                      \
    }                                                                                           \
  }

  // Operand reads. Codes: row wm*32RT + rt*32 + l32 of this wave's slice,
  // logical chunk 2h + g (sub-step h) at its swizzled position (with F8 the
  // two chunks of a block are the two halves of one fp8 operand). Weights:
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
  int rsum[RT];  // this lane's share of the code row sums of its RT rows
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) rsum[rt] = 0;

  // Fragment sets X and Y alternate between the block being multiplied and
  // the block being prepared.
  v4i ax[2][RT], ay[2][RT];  // codes, per sub-step
  v4i bx[2][CT], by[2][CT];  // weight fields u, per sub-step
  uint4 pw[CT];              // packed weights of the block being prepared

#define BITNET_READ(slot_, blk_, A_)                                                            \
  {                                                                                             \
    const char* sb_ = smem + (slot_) * S::SLOT;                                                 \
    _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) pw[ct] =                                  \
        *reinterpret_cast<const uint4*>(sb_ + b_rd + ct * 1024 + (blk_) * 512);                 \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                            \
        _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) A_[hh][rt] =                          \
            *reinterpret_cast<const v4i*>(sb_ + a_rd[2 * (blk_) + hh] + rt * 32 * BKW);         \
  }
#define BITNET_UNPACK(B_)                                                                       \
  _Pragma("unroll") for (int hh = 0; hh < (F8 ? 1 : 2); ++hh)                                   \
      _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) B_[hh][ct] =                            \
          F8 ? unpack_f4(pw[ct], g) : unpack_u(pw[ct], 2 * g + 4 * hh);
#define BITNET_MMA(A_, B_)                                                                      \
  if constexpr (F8) {                                                                           \
    _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                           \
        _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) acc[rt][ct] =                         \
            mma_f8f4(A_[0][rt], A_[1][rt], B_[0][ct], acc[rt][ct]);                             \
  } else {                                                                                      \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                            \
        _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                     \
      if (!RSG) rsum[rt] = add_bytes(A_[hh][rt], rsum[rt]);                                     \
      _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) acc[rt][ct] =                           \
          __builtin_amdgcn_mfma_i32_32x32x32_i8(A_[hh][rt], B_[hh][ct], acc[rt][ct], 0, 0, 0);  \
    }                                                                                           \
  }
  // The empty asm statements pin the next block's operands (codes read and
  // weights unpacked) to the step that prepares them: otherwise the compiler
  // sinks that work to its first use, past the MFMAs it is meant to overlap.
#define BITNET_PIN(A_, B_)                                                                      \
  _Pragma("unroll") for (int hh = 0; hh < 2; ++hh) {                                            \
    _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) if (!F8 || hh == 0)                       \
        asm volatile("" : "+v"(B_[hh][ct]));                                                    \
    _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) asm volatile("" : "+v"(A_[hh][rt]));      \
  }
  // One block's MFMAs (operands A_, B_) cut into S::CH groups separated by
  // scheduling barriers. Group 0 gives the next block's LDS reads (issued
  // just before) time to land; the unpacking of its weights into NB_, the
  // row sums of A_ and, when LD_ is set, this wave's share of the loads of
  // stage lks_ into slot lslot_ are spread over the later groups, so the
  // matrix pipe always has work queued.
  constexpr int kMfmaPerBlock = F8 ? RT * CT : 2 * RT * CT;
  constexpr int kUnpackPerBlock = F8 ? CT : 2 * CT;
  constexpr int kSumPerBlock = 2 * RT;
  constexpr int CHB = kMfmaPerBlock < 8 ? kMfmaPerBlock : 8;  // MFMA groups per block
  static_assert(kMfmaPerBlock % CHB == 0, "MFMA groups");
#define BITNET_STEP(A_, B_, NB_, LD_, lks_, lslot_)                                             \
  _Pragma("unroll") for (int ch = 0; ch < CHB; ++ch) {                                        \
    _Pragma("unroll") for (int e = 0; e < kUnpackPerBlock; ++e) {                               \
      if (1 + e * (CHB - 1) / kUnpackPerBlock == ch) {                                        \
        if constexpr (F8) NB_[0][e] = unpack_f4(pw[e], g);                                      \
        else NB_[e / CT][e % CT] = unpack_u(pw[e % CT], 2 * g + 4 * (e / CT));                  \
      }                                                                                         \
    }                                                                                           \
    _Pragma("unroll") for (int e = 0; e < kSumPerBlock; ++e) {                                  \
      if (!RSG && 1 + e * (CHB - 1) / kSumPerBlock == ch)                                     \
        rsum[e % RT] = add_bytes(A_[e / RT][e % RT], rsum[e % RT]);                             \
    }                                                                                           \
    if (LD_) {                                                                                  \
      _Pragma("unroll") for (int i = 0; i < S::NL_W; ++i) {                                     \
        if (i * CHB / S::NL_W == ch) BITNET_LOAD(lks_, lslot_, i)                             \
      }                                                                                         \
    }                                                                                           \
    _Pragma("unroll") for (int f = ch * (kMfmaPerBlock / CHB);                                \
                           f < (ch + 1) * (kMfmaPerBlock / CHB); ++f) {                       \
      if constexpr (F8) {                                                                       \
        const int rt = f / CT, ct = f % CT;                                                     \
        acc[rt][ct] = mma_f8f4(A_[0][rt], A_[1][rt], B_[0][ct], acc[rt][ct]);                   \
      } else {                                                                                  \
        const int hh = f / (RT * CT), rt = (f / CT) % RT, ct = f % CT;                          \
        acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A_[hh][rt], B_[hh][ct],             \
                                                            acc[rt][ct], 0, 0, 0);              \
      }                                                                                         \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }

  const int nst = (nKB + 2 * KS - 1) / (2 * KS);  // stages, the last possibly partial
  const int nfull = nKB / (2 * KS);               // stages whose every slice is whole

  // Prologue: stages 0..2 in flight, stage 0 published, its block 0 read.
#pragma unroll
  for (int s = 0; s < S::SL; ++s)
#pragma unroll
    for (int i = 0; i < S::NL_W; ++i) BITNET_LOAD(s, s, i)
  BITNET_WAIT_VMCNT((S::SL - 1) * S::NL_W);
  lds_barrier();
  BITNET_READ(0, 0, ax)
  BITNET_UNPACK(bx)

  int slot = 0;
  for (int ks = 0; ks < nfull; ++ks) {
    const int nslot = slot + 1 == S::SL ? 0 : slot + 1;
    // Block 0 of stage ks (set X) runs while block 1 (set Y) is prepared.
    __builtin_amdgcn_sched_barrier(0);
    BITNET_READ(slot, 1, ay)
    BITNET_STEP(ax, bx, by, false, 0, 0)
    BITNET_PIN(ay, by)
    __builtin_amdgcn_sched_barrier(0);
    // Stage boundary. This wave's loads of stage ks + 1 are complete once at
    // most those of the SL - 2 stages after it are outstanding; after the
    // barrier every wave's are visible and no wave reads stage ks any more,
    // so its slot takes stage ks + SL.
    BITNET_WAIT_VMCNT((S::SL - 2) * S::NL_W);
    lds_barrier();
    // Block 1 of stage ks (set Y) runs while block 0 of stage ks + 1 (set X)
    // is prepared (past the last stage this reads a stale slot, unused) and
    // stage ks + SL is fetched.
    __builtin_amdgcn_sched_barrier(0);
    BITNET_READ(nslot, 0, ax)
    BITNET_STEP(ay, by, bx, true, ks + S::SL, slot)
    BITNET_PIN(ax, bx)
    __builtin_amdgcn_sched_barrier(0);
    slot = nslot;
  }
  if (nst > nfull) {
    // Partial last stage (published by the last boundary above, or by the
    // prologue): this wave's slice holds vb whole blocks (0..2).
    const int vb = nKB - nfull * 2 * KS - 2 * kw;
    if (vb >= 1) {
      BITNET_READ(slot, 0, ax)
      BITNET_UNPACK(bx)
      BITNET_MMA(ax, bx)
    }
    if (vb >= 2) {
      BITNET_READ(slot, 1, ay)
      BITNET_UNPACK(by)
      BITNET_MMA(ay, by)
    }
  }
#undef BITNET_READ
#undef BITNET_UNPACK
#undef BITNET_MMA
#undef BITNET_STEP
#undef BITNET_PIN
#undef BITNET_LOAD
  if constexpr (F8) {
    // fp32 sums of q u / 2, exact: q . u = 2 acc, an integer (converted as
    // whole vectors: a bit cast of one vector element read element 0)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const v16f f = __builtin_bit_cast(v16f, acc[rt][ct]);
        acc[rt][ct] = __builtin_convertvector(f * 2.0f, v16i);
      }
  }

  // No load may still be writing LDS past this point, and no wave may still
  // be reading the ring, whose tail now takes the row sums.
  BITNET_WAIT_VMCNT(0);
  lds_barrier();

  // Row sums: add the two k halves (lane groups g = 0, 1) and publish the
  // slice's sums per tile row; every wave of a (wm, kw) pair holds the same
  // values, the one with wn = 0 writes them.
  int* rowsum = reinterpret_cast<int*>(smem + S::ROWSUM);
  if constexpr (!RSG) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int total = rsum[rt] + __shfl_xor(rsum[rt], 32);
      if (wn == 0 && g == 0) rowsum[kw * S::BM + wm * 32 * RT + rt * 32 + l32] = total;
    }
    lds_barrier();
  }

  if constexpr (KS > 1) {
    // Add the k slices' partial products through LDS, halving the number of
    // live slices per round; slice 0's waves end up with the full sums.
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
  }

  // 32x32 output layout: lane holds column l32 and, for v = 0..15, row
  // 8*(v/4) + 4*g + v%4 of its 32x32 block. q . t = q . u - sum(q).
  const float alpha = OUT_I32 ? 0.0f : *alpha_p;
  if constexpr (WIDE && !OUT_I32) {
    // Wide stores (N % 4 == 0, y 16-byte aligned): each 32x32 block is turned
    // around, 16 rows at a time, through this wave's 2.5 KB of the (drained)
    // LDS ring, so that a lane stores 16 contiguous bytes of one row: a
    // quarter of the store instructions. Rows past M fall outside the store
    // resource; groups of four columns past N get an out-of-range offset.
    constexpr int TP = 40;  // row pitch in floats: rows r and r + 4 on opposite bank halves
    float* tb = reinterpret_cast<float*>(smem) + wmn * 16 * TP;
    const int rows = (M - m0 < S::BM) ? M - m0 : S::BM;
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(y + (size_t)m0 * N, (short)0, rows * N * 4, 0x00020000);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int rb = wm * 32 * RT + rt * 32;
      float f[16];
      int rsv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = rb + 8 * (v >> 2) + 4 * g + (v & 3);
        const int m = m0 + r < M ? m0 + r : M - 1;
        int rs = 0;
        if constexpr (RSG) {
          rs = rowsum_g[m];
        } else {
#pragma unroll
          for (int s = 0; s < KS; ++s) rs += rowsum[s * S::BM + r];
        }
        rsv[v] = rs;
        f[v] = dequant_factor(alpha, scales[m], c);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int nc = n0 + wn * 32 * CT + ct * 32 + 4 * (lane & 7);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int vv = 0; vv < 8; ++vv) {
            const int v = 8 * h + vv;
            tb[(8 * (vv >> 2) + 4 * g + (vv & 3)) * TP + l32] = (float)(acc[rt][ct][v] - rsv[v]) * f[v];
          }
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r = 8 * jj + (lane >> 3);
            const v4f o = *reinterpret_cast<const v4f*>(tb + r * TP + 4 * (lane & 7));
            const int off = nc < N ? ((rb + 16 * h + r) * N + nc) * 4 : (int)0x80000000;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, o), yr, off, 0, 0);
          }
        }
      }
    }
    return;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = wm * 32 * RT + rt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      const int m = m0 + r;
      if (m >= M) continue;
      int rs = 0;
      if constexpr (RSG) {
        rs = rowsum_g[m];
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) rs += rowsum[s * S::BM + r];
      }
      const float f = OUT_I32 ? 0.0f : dequant_factor(alpha, scales[m], c);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int n = n0 + wn * 32 * CT + ct * 32 + l32;
        if (n >= N) continue;
        const size_t o = (size_t)m * N + n;
        const int dot = acc[rt][ct][v] - rs;
        if (OUT_I32) {
          acc_out[o] = dot;
        } else {
          y[o] = (float)dot * f;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Streamed tiles: the large-product variant given the quantizer's row sums.
//
// With one workgroup per CU and several 256 x 256 tiles per CU, every CU
// finishes its tile at about the same time, and the fp32 outputs of all of
// them (64 MB at M=8192 N=14336) then go to HBM in one burst while the matrix
// cores idle: measured, the stores cost about a fifth of the kernel. Here one
// workgroup per CU walks its tiles in sequence with one continuous stage
// pipeline: the first stages of tile i + 1 are fetched while tile i is still
// multiplied, and tile i's outputs are stored (without waiting for them)
// while those fetches are in flight and the next tile's MFMAs start.
//
// Output stores. The vector-memory counter covers loads and stores alike and
// drains in issue order, so the stage waits of the next tile's first two
// stages allow for the tile's stores; that needs few, wide stores. The
// accumulators are therefore turned around through a small per-wave LDS
// buffer (16 rows of a 32 x 32 block at a time) so that each lane stores 16
// contiguous bytes of one row: RT * CT * 4 buffer_store_dwordx4 per wave and
// tile. Rows past M fall outside the store resource and columns past N get an
// out-of-range offset, so every store instruction issues (the count stays
// exact) and nothing lands outside y.
//
// Scales and code row sums of a tile travel with its first stage: one more
// direct-to-LDS dword load per wave (waves 0..3 scales, 4..7 row sums) into a
// double-buffered area; every other stage's extra load reads nothing and
// writes zeros to a sink, so every stage has the same load count.
template <int RT, int CT, int WMW, int WNW>
struct StreamShape {
  using S = Shape<RT, CT, WMW, WNW, 1>;
  static constexpr int TPITCH = 40;                   // floats per transpose row (bank offset 32 between row r and r + 4)
  static constexpr int TBUF = 16 * TPITCH * 4;        // one wave's transpose buffer
  static constexpr int TRANS = S::RING;
  static constexpr int META = TRANS + S::NW * TBUF;   // [2][scales BM | row sums BM]
  static constexpr int META_BYTES = 2 * S::BM * 4;
  static constexpr int SINK = META + 2 * META_BYTES;  // 256 B per wave
  static constexpr int LDS = SINK + S::NW * 256;
  static constexpr int NLG = S::NL_W + 1;             // loads per wave and stage
  static constexpr int STORES = RT * CT * 4;          // dwordx4 stores per wave and tile
  static_assert(S::NW * 64 == 2 * S::BM, "one scale or row sum per lane");
  static_assert(LDS <= kLdsMax, "LDS");
  static_assert((S::SL - 1) * NLG + STORES <= 63, "vmcnt range");
};

template <int RT, int CT, int WMW, int WNW>
__global__ __launch_bounds__(64 * WMW * WNW) void ternary_gemm_stream_kernel(
    const int8_t* __restrict__ codes, const float* __restrict__ scales,
    const int32_t* __restrict__ rowsum_g, int M, int K, const uint8_t* __restrict__ Wp, int N,
    const float* __restrict__ alpha_p, float c, float* __restrict__ y, int tiles_m, int tiles_n) {
  using S = Shape<RT, CT, WMW, WNW, 1>;
  using T = StreamShape<RT, CT, WMW, WNW>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WNW, wn = wave % WNW;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int wrow = K >> 2;
  const int nst = K / (2 * 64);  // 128-k stages per tile, all whole

  // This workgroup's tiles. XCD x = blockIdx.x % 8 owns the contiguous range
  // [x per_xcd, (x + 1) per_xcd) of the band-ordered tile walk, which its
  // workgroups take in turn, so the tiles resident on one XCD at a time are
  // neighbours in the walk and share codes and weights in its L2.
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int wg_step = gridDim.x / kXcds;
  const int first = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  const int t_end = min(tiles, (blockIdx.x % kXcds + 1) * per_xcd);
  const int ntiles = first < t_end ? (t_end - first + wg_step - 1) / wg_step : 0;
  if (ntiles == 0) return;
  const int total = ntiles * nst;

  // alpha is used here so that its load completes before the stage loads go
  // out (a later first use would wait for them too).
  const float alpha = *alpha_p;
  asm volatile("" ::"v"(alpha));

  const unsigned lds0 = lds_address(smem);
  const int a_lane0 = (lane >> 3) * K + 16 * ((lane & 7) ^ (lane >> 3));
  const int a_lane1 = (lane >> 3) * K + 16 * ((lane & 7) ^ (lane >> 3) ^ 1);
  const int b_lane = l32 * wrow + g * 16;
  const int meta_lane = 4 * (lane + 64 * (wave & 3));  // row 64 (wave % 4) + lane of the tile

  // Load cursor: stage ld_ks of tile ld_i, and that tile's resources.
  int ld_i = 0, ld_ks = 0;
  u4 a_rsrc, b_rsrc, m_rsrc;
  auto set_load_tile = [&]() {
    if (ld_i < ntiles) {
      const int tile = first + ld_i * wg_step;
      const int band = tile / (kBand * tiles_n);
      const int band_m = min(tiles_m - band * kBand, kBand);
      const int in_band = tile - band * kBand * tiles_n;
      const int m0 = (band * kBand + in_band % band_m) * S::BM;
      const int n0 = (in_band / band_m) * S::BN;
      const int rows = min(M - m0, S::BM);
      a_rsrc = make_rsrc(codes + (size_t)m0 * K, (unsigned)(rows * K));
      b_rsrc = make_rsrc(Wp + (size_t)n0 * wrow, (unsigned)(min(N - n0, S::BN) * wrow));
      m_rsrc = (wave < 4) ? make_rsrc(scales + m0, (unsigned)(rows * 4))
                          : make_rsrc(rowsum_g + m0, (unsigned)(rows * 4));
    } else {
      a_rsrc.z = 0;
      b_rsrc.z = 0;
      m_rsrc.z = 0;
    }
  };
  set_load_tile();
  u4 none = a_rsrc;
  none.z = 0;

  // Load q of the current load stage into slot lslot_ (q < NL_W: codes or
  // weights, as in the per-tile kernel; q == NL_W: the tile's scales or row
  // sums when the stage is its first, else nothing, into the sink).
#define BITNET_SLOAD(lslot_, q)                                                                 \
  {                                                                                             \
    if ((q) < S::NA_W) {                                                                        \
      const int q_ = wave + S::NW * (q);                                                        \
      const int rb_ = q_ % (S::BM / 8);                                                         \
      load_lds16(a_rsrc, ((rb_ & 1) ? a_lane1 : a_lane0) + rb_ * 8 * K + ld_ks * S::SK,         \
                 lds0 + (unsigned)((lslot_) * S::SLOT + rb_ * 1024));                           \
    } else if ((q) < S::NL_W) {                                                                 \
      const int cg_ = wave + S::NW * ((q) - S::NA_W);                                           \
      load_lds16(b_rsrc, b_lane + cg_ * 32 * wrow + ld_ks * (S::SK / 4),                        \
                 lds0 + (unsigned)((lslot_) * S::SLOT + S::A_BYTES + cg_ * 1024));              \
    } else {                                                                                    \
      const bool first_ = ld_ks == 0; /* a select, not a branch */                              \
      load_lds4(first_ ? m_rsrc : none, meta_lane,                                              \
                lds0 + (unsigned)(first_ ? T::META + (ld_i & 1) * T::META_BYTES + 256 * wave    \
                                         : T::SINK + 256 * wave));                              \
    }                                                                                           \
  }
#define BITNET_SADVANCE()                                                                       \
  {                                                                                             \
    if (++ld_ks == nst) {                                                                       \
      ld_ks = 0;                                                                                \
      ++ld_i;                                                                                   \
      set_load_tile();                                                                          \
    }                                                                                           \
  }

  int a_rd[4];
  {
    const int r = wm * 32 * RT + l32;
#pragma unroll
    for (int h = 0; h < 4; ++h) a_rd[h] = r * BKW + 16 * ((2 * h + g) ^ chunk_swizzle(r));
  }
  const int b_rd = S::A_BYTES + wn * CT * 1024 + 16 * l32;

  v16i acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0;
  v4i ax[2][RT], ay[2][RT];
  v4i bx[2][CT], by[2][CT];
  uint4 pw[CT];

#define BITNET_SREAD(slot_, blk_, A_)                                                           \
  {                                                                                             \
    const char* sb_ = smem + (slot_) * S::SLOT;                                                 \
    _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) pw[ct] =                                  \
        *reinterpret_cast<const uint4*>(sb_ + b_rd + ct * 1024 + (blk_) * 512);                 \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                            \
        _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) A_[hh][rt] =                          \
            *reinterpret_cast<const v4i*>(sb_ + a_rd[2 * (blk_) + hh] + rt * 32 * BKW);         \
  }
#define BITNET_SUNPACK(B_)                                                                      \
  _Pragma("unroll") for (int hh = 0; hh < 2; ++hh)                                              \
      _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) B_[hh][ct] =                            \
          unpack_u(pw[ct], 2 * g + 4 * hh);
#define BITNET_SPIN(A_, B_)                                                                     \
  _Pragma("unroll") for (int hh = 0; hh < 2; ++hh) {                                            \
    _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) asm volatile("" : "+v"(B_[hh][ct]));      \
    _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) asm volatile("" : "+v"(A_[hh][rt]));      \
  }
  constexpr int kMfmaPerBlock = 2 * RT * CT;
  constexpr int kUnpackPerBlock = 2 * CT;
#define BITNET_SSTEP(A_, B_, NB_, LD_, lslot_)                                                  \
  _Pragma("unroll") for (int ch = 0; ch < S::CH; ++ch) {                                      \
    _Pragma("unroll") for (int e = 0; e < kUnpackPerBlock; ++e) {                               \
      if (1 + e * (S::CH - 1) / kUnpackPerBlock == ch)                                        \
        NB_[e / CT][e % CT] = unpack_u(pw[e % CT], 2 * g + 4 * (e / CT));                       \
    }                                                                                           \
    if (LD_) {                                                                                  \
      _Pragma("unroll") for (int q = 0; q < T::NLG; ++q) {                                      \
        if (q * S::CH / T::NLG == ch) BITNET_SLOAD(lslot_, q)                                 \
      }                                                                                         \
    }                                                                                           \
    _Pragma("unroll") for (int f = ch * (kMfmaPerBlock / S::CH);                              \
                           f < (ch + 1) * (kMfmaPerBlock / S::CH); ++f) {                     \
      const int hh = f / (RT * CT), rt = (f / CT) % RT, ct = f % CT;                            \
      acc[rt][ct] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A_[hh][rt], B_[hh][ct], acc[rt][ct],  \
                                                          0, 0, 0);                             \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }

  // Epilogue of tile ti: y = (q . u - sum(q)) * alpha * s / c for its rows,
  // turned around 16 rows at a time through this wave's LDS buffer and
  // stored as 16-byte row pieces.
  float* tb = reinterpret_cast<float*>(smem + T::TRANS + wave * T::TBUF);
  auto epilogue = [&](int ti) {
    const int tile = first + ti * wg_step;
    const int band = tile / (kBand * tiles_n);
    const int band_m = min(tiles_m - band * kBand, kBand);
    const int in_band = tile - band * kBand * tiles_n;
    const int m0 = (band * kBand + in_band % band_m) * S::BM;
    const int n0 = (in_band / band_m) * S::BN;
    const int rows = min(M - m0, S::BM);
    const __amdgpu_buffer_rsrc_t yr =
        __builtin_amdgcn_make_buffer_rsrc(y + (size_t)m0 * N, (short)0, rows * N * 4, 0x00020000);
    const float* msc = reinterpret_cast<const float*>(smem + T::META + (ti & 1) * T::META_BYTES);
    const int* mrs = reinterpret_cast<const int*>(msc + S::BM);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      // this lane's rows: rb + 8 q + 4 g + e (q, e = 0..3), the 32x32 MFMA layout
      const int rb = wm * 32 * RT + rt * 32;
      v4f f[4];
      v4i rs[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f sv = *reinterpret_cast<const v4f*>(msc + rb + 8 * q + 4 * g);
        rs[q] = *reinterpret_cast<const v4i*>(mrs + rb + 8 * q + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) f[q][e] = dequant_factor(alpha, sv[e], c);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int nc = n0 + wn * 32 * CT + ct * 32 + 4 * (lane & 7);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int qq = 0; qq < 2; ++qq)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int q = 2 * h + qq, v = 4 * q + e;
              tb[(8 * qq + 4 * g + e) * T::TPITCH + l32] =
                  (float)(acc[rt][ct][v] - rs[q][e]) * f[q][e];
            }
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r = 8 * jj + (lane >> 3);
            const v4f o = *reinterpret_cast<const v4f*>(tb + r * T::TPITCH + 4 * (lane & 7));
            const int off = nc < N ? ((rb + 16 * h + r) * N + nc) * 4 : (int)0x80000000;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, o), yr, off, 0, 0);
          }
        }
      }
    }
  };

  // Prologue: stages 0 .. SL - 1 in flight, stage 0 published, its block 0 read.
#pragma unroll
  for (int s = 0; s < S::SL; ++s) {
#pragma unroll
    for (int q = 0; q < T::NLG; ++q) BITNET_SLOAD(s, q)
    BITNET_SADVANCE()
  }
  BITNET_WAIT_VMCNT((S::SL - 1) * T::NLG);
  lds_barrier();
  BITNET_SREAD(0, 0, ax)
  BITNET_SUNPACK(bx)

  int slot = 0, ks = 0, ti = 0;
  for (int gs = 0; gs < total; ++gs) {
    const int nslot = slot + 1 == S::SL ? 0 : slot + 1;
    __builtin_amdgcn_sched_barrier(0);
    BITNET_SREAD(slot, 1, ay)
    BITNET_SSTEP(ax, bx, by, false, 0)
    BITNET_SPIN(ay, by)
    __builtin_amdgcn_sched_barrier(0);
    // Stage boundary: this wave's loads of stage gs + 1 are complete once at
    // most the loads of stage gs + 2 -- and, in a tile's first two stages, the
    // previous tile's stores, issued after or between them -- are
    // outstanding.
    if (ti > 0 && ks <= 1) {
      BITNET_WAIT_VMCNT((S::SL - 2) * T::NLG + T::STORES);
    } else {
      BITNET_WAIT_VMCNT((S::SL - 2) * T::NLG);
    }
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    BITNET_SREAD(nslot, 0, ax)
    BITNET_SSTEP(ay, by, bx, true, slot)
    BITNET_SPIN(ax, bx)
    __builtin_amdgcn_sched_barrier(0);
    BITNET_SADVANCE()
    slot = nslot;
    if (++ks == nst) {
      epilogue(ti);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0;
      ks = 0;
      ++ti;
    }
  }
  // The fetches past the last stage write zeros into free LDS; let them land
  // before the workgroup ends.
  BITNET_WAIT_VMCNT(0);
#undef BITNET_SLOAD
#undef BITNET_SADVANCE
#undef BITNET_SREAD
#undef BITNET_SUNPACK
#undef BITNET_SPIN
#undef BITNET_SSTEP
}

template <int RT, int CT, int WMW, int WNW, int KS, bool OUT_I32, bool RSG, bool WIDE = false,
          bool F8 = false>
hipError_t launch_tile(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, float c, float* y,
                       int32_t* acc, const int32_t* rowsum, hipStream_t stream) {
  using S = Shape<RT, CT, WMW, WNW, KS>;
  const int tiles_m = (int)((M + S::BM - 1) / S::BM);
  const int tiles_n = (int)((N + S::BN - 1) / S::BN);
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  auto kern = ternary_gemm_kernel<RT, CT, WMW, WNW, KS, OUT_I32, RSG, WIDE, F8>;
  if (S::LDS > 48 * 1024) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
    if (e != hipSuccess) return e;
  }
  kern<<<dim3((unsigned)(per_xcd * kXcds)), dim3(S::NT), S::LDS, stream>>>(
      codes, scales, (int)M, K, Wpacked, (int)N, alpha, c, y, acc, rowsum, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int RT, int CT, int WMW, int WNW, int KS>
hipError_t launch_variant(const int8_t* codes, const float* scales, int64_t M, int K,
                          const uint8_t* Wpacked, int64_t N, const float* alpha, float c, float* y,
                          int32_t* acc, const int32_t* rowsum, hipStream_t stream) {
  if (acc)
    return launch_tile<RT, CT, WMW, WNW, KS, true, false>(codes, scales, M, K, Wpacked, N, alpha,
                                                          c, y, acc, nullptr, stream);
  // wide stores need whole groups of four columns and 16-byte rows
  const bool wide = N % 4 == 0 && N <= (1 << 20) && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  if (rowsum) {
    if (wide)
      return launch_tile<RT, CT, WMW, WNW, KS, false, true, true>(codes, scales, M, K, Wpacked, N,
                                                                  alpha, c, y, nullptr, rowsum,
                                                                  stream);
    return launch_tile<RT, CT, WMW, WNW, KS, false, true>(codes, scales, M, K, Wpacked, N, alpha,
                                                          c, y, nullptr, rowsum, stream);
  }
  if (wide)
    return launch_tile<RT, CT, WMW, WNW, KS, false, false, true>(codes, scales, M, K, Wpacked, N,
                                                                 alpha, c, y, nullptr, nullptr,
                                                                 stream);
  return launch_tile<RT, CT, WMW, WNW, KS, false, false>(codes, scales, M, K, Wpacked, N, alpha, c,
                                                         y, nullptr, nullptr, stream);
}

template <int RT, int CT, int WMW, int WNW>
hipError_t launch_stream(const int8_t* codes, const float* scales, const int32_t* rowsum,
                         int64_t M, int K, const uint8_t* Wpacked, int64_t N, const float* alpha,
                         float c, float* y, hipStream_t stream) {
  using S = Shape<RT, CT, WMW, WNW, 1>;
  using T = StreamShape<RT, CT, WMW, WNW>;
  const int tiles_m = (int)((M + S::BM - 1) / S::BM);
  const int tiles_n = (int)((N + S::BN - 1) / S::BN);
  const int tiles = tiles_m * tiles_n;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  // one workgroup per CU (the LDS footprint admits no second), the same
  // number on every XCD
  int grid = (tiles < cus ? tiles : cus) / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  auto kern = ternary_gemm_stream_kernel<RT, CT, WMW, WNW>;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, T::LDS);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)grid), dim3(S::NT), T::LDS, stream>>>(
      codes, scales, rowsum, (int)M, K, Wpacked, (int)N, alpha, c, y, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* codes, const float* scales, int64_t M, int K,
                       const uint8_t* Wpacked, int64_t N, const float* alpha, int bits, float* y,
                       int32_t* acc, hipStream_t stream, const int32_t* rowsum,
                       bool f8) {
  const float c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  if (f8) {
    if (!fp8_pair_gemm_ok(M, K, N, bits) || !rowsum || acc) return hipErrorInvalidValue;
    if (N % 4 == 0 && N <= (1 << 20) && (reinterpret_cast<uintptr_t>(y) & 15) == 0)
      return launch_tile<2, 2, 2, 2, 2, false, true, true, true>(codes, scales, M, K, Wpacked, N,
                                                                 alpha, c, y, nullptr, rowsum,
                                                                 stream);
    return launch_tile<2, 2, 2, 2, 2, false, true, false, true>(codes, scales, M, K, Wpacked, N,
                                                                alpha, c, y, nullptr, rowsum, stream);
  }
  // Two waves per SIMD (eight per workgroup, 64 x 128 or 128 x 64 per wave,
  // accumulators in VGPRs): while one wave waits on LDS or the stage barrier
  // the other issues MFMAs, which measured 13-18% faster than one wave of
  // 128 x 128 per SIMD. 256 x 256 tiles when there are enough of them to give
  // every CU several; otherwise 128 x 128 tiles whose waves split each
  // 256-wide stage into two k slices.
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  // Many tiles, row sums given: one workgroup per CU streams its tiles, the
  // stores of one overlapping the next one's fetches and products.
  if (big_tiles >= 1024 && rowsum && !acc && K % 128 == 0 && K >= 512 && N % 4 == 0 &&
      N <= (1 << 20) && (reinterpret_cast<uintptr_t>(y) & 15) == 0)
    return launch_stream<2, 4, 4, 2>(codes, scales, rowsum, M, K, Wpacked, N, alpha, c, y, stream);
  if (big_tiles >= 1024)
    return launch_variant<2, 4, 4, 2, 1>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, rowsum,
                                         stream);
  return launch_variant<2, 2, 2, 2, 2>(codes, scales, M, K, Wpacked, N, alpha, c, y, acc, rowsum,
                                       stream);
}

hipError_t launch_ternary_matmul(const int8_t* codes, const float* scales, int64_t M, int K,
                                 const uint8_t* Wpacked, int64_t N, const float* alpha, int bits,
                                 float* y, int32_t* acc, hipStream_t stream,
                                 const int32_t* rowsum, bool nibbles, bool fp8_pairs) {
  if (M <= kDecodeMaxM) {
    if (fp8_pairs) return hipErrorInvalidValue;
    return launch_gemv(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream, nibbles, rowsum);
  }
  if (nibbles) return hipErrorInvalidValue;
  return launch_gemm(codes, scales, M, K, Wpacked, N, alpha, bits, y, acc, stream, rowsum,
                     fp8_pairs);
}

}  // namespace bitnet
