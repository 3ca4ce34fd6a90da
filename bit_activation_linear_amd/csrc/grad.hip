// Backward pass of the H-BitLinear layer.
//
// Engine page (Quillan-Ronin bitnet_v2_engine.py): HBitLinear.forward ends in
// F.linear(x_q, w_q) with x_q = (s / c) q per token (Eq. 5-6) and
// w_q = alpha t (Eq. 1); the quantizers' autograd functions pass gradients
// straight through (STE), and HadamardTransformFunction's backward applies
// the transform to the gradient (Eq. 8). For dL/dy = dy [M, N]:
//   dx = H (alpha dy . t)        [M, K]  (H only with the transform)
//   dw = dy^T . x_q              [N, K]  gradient of the latent weights
//
// Both products are dense floating-point contractions and run on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation:
//   - dx: dy in bf16 (exact when the caller's gradient is bf16; an fp32
//     gradient is split into hi + lo bf16 parts) times t, which
//     bf16 holds exactly. The packed weights are expanded once per call into
//     a bf16 copy of t^T [K, N] so that both operands have the contraction
//     (N) contiguous.
//   - dw: p = dy * s / c per token, split into hi + lo bf16 parts (16
//     significant bits), times the integer codes q, exact in bf16; both are
//     transposed so that the contraction (M) is contiguous.
// Every product in the MFMA is exact; only the fp32 accumulation and the
// 2^-17 relative residual of the hi/lo split round.
//
// GEMM kernel: C[R, Cn] = scale * (A + A2)[R, Kc] . B[Cn, Kc]^T, bf16
// row-major operands with Kc % 64 == 0; with SPLIT the hi and lo parts A and
// A2 are staged side by side and multiplied into the same accumulators, so
// a split operand costs twice the MFMAs but no second pass over C.
// Direct-to-LDS staging as in the forward prefill kernel: a ring of SL stage
// slots, each holding 64 k (128 bytes) of the tile's A (and A2) and B rows,
// 16-byte chunks of every row XOR-permuted so that operand reads are
// bank-conflict-free; one barrier per stage; the next 32-k block's operands
// are read while the current block's MFMAs run.
#include "kernels.h"
#include "ternary_common.h"

namespace bitnet {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kRow = 128;        // bytes of one operand row per stage (64 bf16)
constexpr int kGradChunks = 8;   // MFMA groups per block in the interleaved schedule

template <int RT, int CT, int WM, int WN, bool SPLIT>
struct GShape {
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;
  static constexpr int BM = 32 * RT * WM;
  static constexpr int BN = 32 * CT * WN;
  static constexpr int NAP = SPLIT ? 2 : 1;      // A parts (hi, lo)
  static constexpr int A_BYTES = NAP * BM * kRow;  // part p's rows at p * BM
  static constexpr int B_BYTES = BN * kRow;
  static constexpr int SLOT = A_BYTES + B_BYTES;
  static constexpr int NA = A_BYTES / 1024;  // 1-KB direct loads per stage (8 rows each)
  static constexpr int NB = B_BYTES / 1024;
  static constexpr int NL_W = (NA + NB) / NW;  // ... per wave
  static constexpr int SL = (3 * SLOT <= kLdsMax) ? 3 : 2;
  static constexpr int LDS = SL * SLOT;
  static_assert(NL_W * NW == NA + NB, "uneven staging");
  static_assert(2 * SLOT <= kLdsMax, "two stage slots do not fit in LDS");
  static_assert((2 * NAP * RT * CT) % kGradChunks == 0, "MFMA groups");
  static_assert(BM % 16 == 0, "the parts' rows must keep the swizzle");
};

__device__ __forceinline__ bf16x8 as_bf16x8(const v4i v) {
  return __builtin_bit_cast(bf16x8, v);
}

template <int RT, int CT, int WM, int WN, bool SPLIT>
__global__ __launch_bounds__(64 * WM * WN) void bf16_gemm_nt_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ A2, int64_t lda,
    const uint16_t* __restrict__ B, int64_t ldb, int R, int Cn, int Kc, float* __restrict__ C,
    int64_t ldc, const float* __restrict__ scale_p, float scale_h, int tiles_m, int tiles_n) {
  using S = GShape<RT, CT, WM, WN, SPLIT>;
  extern __shared__ __attribute__((aligned(1024))) char smem[];

  // XCD-aware tile order (workgroup L runs on XCD L % 8; each XCD walks a
  // contiguous range of tiles band by band).
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int L = blockIdx.x;
  const int tile = (L % kXcds) * per_xcd + L / kXcds;
  if (tile >= tiles) return;
  const int band = tile / (kBand * tiles_n);
  const int band_m = (tiles_m - band * kBand) < kBand ? (tiles_m - band * kBand) : kBand;
  const int in_band = tile - band * kBand * tiles_n;
  const int r0 = (band * kBand + in_band % band_m) * S::BM;
  const int c0 = (in_band / band_m) * S::BN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int nst = Kc / 64;
  const int64_t arow = lda * 2, brow = ldb * 2;  // row pitches in bytes

  // Buffer resources end at the tile's last valid row: rows past R (Cn) read
  // as zero. Stages past the last go through empty resources (zeros, no
  // memory touched) so every stage issues the same number of loads.
  const unsigned a_bytes = (unsigned)((R - r0 < S::BM ? R - r0 : S::BM) * arow);
  const unsigned b_bytes = (unsigned)((Cn - c0 < S::BN ? Cn - c0 : S::BN) * brow);
  const u4 a_rsrc = make_rsrc(A + (size_t)r0 * lda, a_bytes);
  const u4 a2_rsrc = make_rsrc((SPLIT ? A2 : A) + (size_t)r0 * lda, a_bytes);
  const u4 b_rsrc = make_rsrc(B + (size_t)c0 * ldb, b_bytes);
  u4 a_none = a_rsrc, b_none = b_rsrc;
  a_none.z = 0;
  b_none.z = 0;
  const unsigned lds0 = lds_address(smem);
  // Load i of a wave fills 1 KB: 8 rows of 128 bytes (row 8 rb + lane / 8),
  // lane taking global chunk (lane % 8) ^ swizzle(row), so that LDS position
  // p of row r holds chunk p ^ swizzle(r); swizzle(r) = lane / 8 ^ (rb & 1).
  const int sw0 = (lane & 7) ^ (lane >> 3);
  const int a_lane0 = (int)((lane >> 3) * arow) + 16 * sw0;
  const int a_lane1 = (int)((lane >> 3) * arow) + 16 * (sw0 ^ 1);
  const int b_lane0 = (int)((lane >> 3) * brow) + 16 * sw0;
  const int b_lane1 = (int)((lane >> 3) * brow) + 16 * (sw0 ^ 1);
#define GRAD_LOAD(ks_, slot_, i)                                                                \
  {                                                                                             \
    const bool live_ = (ks_) < nst;                                                             \
    const int q_ = wave + S::NW * (i);                                                          \
    if (q_ < S::NA) {                                                                           \
      const bool lo_ = SPLIT && q_ >= S::BM / 8;                                                \
      const int qa_ = lo_ ? q_ - S::BM / 8 : q_;                                                \
      load_lds16(live_ ? (lo_ ? a2_rsrc : a_rsrc) : a_none,                                     \
                 ((qa_ & 1) ? a_lane1 : a_lane0) + (int)(qa_ * 8 * arow) + (ks_) * kRow,        \
                 lds0 + (unsigned)((slot_) * S::SLOT + q_ * 1024));                             \
    } else {                                                                                    \
      const int qb_ = q_ - S::NA;                                                               \
      load_lds16(live_ ? b_rsrc : b_none,                                                       \
                 ((qb_ & 1) ? b_lane1 : b_lane0) + (int)(qb_ * 8 * brow) + (ks_) * kRow,        \
                 lds0 + (unsigned)((slot_) * S::SLOT + S::A_BYTES + qb_ * 1024));               \
    }                                                                                           \
  }

  // Operand reads: sub-step h (16 k) takes logical chunk 2h + g of row
  // l32 of each 32-row block (32-row offsets keep the swizzle).
  int a_rd[4], b_rd[4];
  {
    const int ra = wm * 32 * RT + l32;
    const int rb = wn * 32 * CT + l32;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      a_rd[h] = ra * kRow + 16 * ((2 * h + g) ^ chunk_swizzle(ra));
      b_rd[h] = S::A_BYTES + rb * kRow + 16 * ((2 * h + g) ^ chunk_swizzle(rb));
    }
  }

  v16f acc[RT][CT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rt][ct][v] = 0.0f;

  // Fragment sets X and Y alternate between the 32-k block being multiplied
  // and the block being read. A fragment i < RT is part hi's row block i,
  // i >= RT part lo's row block i - RT (same accumulator).
  constexpr int RA = S::NAP * RT;
  v4i ax[2][RA], ay[2][RA], bx[2][CT], by[2][CT];

#define GRAD_READ(slot_, blk_, A_, B_)                                                          \
  {                                                                                             \
    const char* sb_ = smem + (slot_) * S::SLOT;                                                 \
    _Pragma("unroll") for (int hh = 0; hh < 2; ++hh) {                                          \
      _Pragma("unroll") for (int ra = 0; ra < RA; ++ra) A_[hh][ra] =                            \
          *reinterpret_cast<const v4i*>(sb_ + a_rd[2 * (blk_) + hh] +                           \
                                        ((ra / RT) * S::BM + (ra % RT) * 32) * kRow);           \
      _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) B_[hh][ct] =                            \
          *reinterpret_cast<const v4i*>(sb_ + b_rd[2 * (blk_) + hh] + ct * 32 * kRow);          \
    }                                                                                           \
  }
#define GRAD_PIN(A_, B_)                                                                        \
  _Pragma("unroll") for (int hh = 0; hh < 2; ++hh) {                                            \
    _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) asm volatile("" : "+v"(B_[hh][ct]));      \
    _Pragma("unroll") for (int ra = 0; ra < RA; ++ra) asm volatile("" : "+v"(A_[hh][ra]));      \
  }
  // One block's MFMAs in kGradChunks groups separated by scheduling barriers;
  // with LD_ set, this wave's loads of stage lks_ into slot lslot_ are spread
  // over the groups.
  constexpr int kMfmaPerBlock = 2 * RA * CT;
#define GRAD_STEP(A_, B_, LD_, lks_, lslot_)                                                    \
  _Pragma("unroll") for (int ch = 0; ch < kGradChunks; ++ch) {                                  \
    if (LD_) {                                                                                  \
      _Pragma("unroll") for (int i = 0; i < S::NL_W; ++i) {                                     \
        if (i * kGradChunks / S::NL_W == ch) GRAD_LOAD(lks_, lslot_, i)                         \
      }                                                                                         \
    }                                                                                           \
    _Pragma("unroll") for (int f = ch * (kMfmaPerBlock / kGradChunks);                          \
                           f < (ch + 1) * (kMfmaPerBlock / kGradChunks); ++f) {                 \
      const int hh = f / (RA * CT), ra = (f / CT) % RA, ct = f % CT;                            \
      acc[ra % RT][ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                               \
          as_bf16x8(A_[hh][ra]), as_bf16x8(B_[hh][ct]), acc[ra % RT][ct], 0, 0, 0);             \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
  }

  // Prologue: stages 0 .. SL-1 in flight, stage 0 published, its block 0 read.
#pragma unroll
  for (int s = 0; s < S::SL; ++s)
#pragma unroll
    for (int i = 0; i < S::NL_W; ++i) GRAD_LOAD(s, s, i)
  BITNET_WAIT_VMCNT((S::SL - 1) * S::NL_W);
  lds_barrier();
  GRAD_READ(0, 0, ax, bx)

  int slot = 0;
  for (int ks = 0; ks < nst; ++ks) {
    const int nslot = slot + 1 == S::SL ? 0 : slot + 1;
    // Block 0 of stage ks (set X) runs while block 1 (set Y) is read.
    __builtin_amdgcn_sched_barrier(0);
    GRAD_READ(slot, 1, ay, by)
    GRAD_STEP(ax, bx, false, 0, 0)
    GRAD_PIN(ay, by)
    __builtin_amdgcn_sched_barrier(0);
    // Stage boundary: this wave's loads of stage ks + 1 are complete once at
    // most those of the SL - 2 stages after it are outstanding; after the
    // barrier every wave's are visible and no wave reads stage ks any more.
    BITNET_WAIT_VMCNT((S::SL - 2) * S::NL_W);
    lds_barrier();
    // Block 1 of stage ks (set Y) runs while block 0 of stage ks + 1 is read
    // (past the last stage this reads a slot that is never multiplied) and
    // stage ks + SL is fetched into the slot just freed.
    __builtin_amdgcn_sched_barrier(0);
    GRAD_READ(nslot, 0, ax, bx)
    GRAD_STEP(ay, by, true, ks + S::SL, slot)
    GRAD_PIN(ax, bx)
    __builtin_amdgcn_sched_barrier(0);
    slot = nslot;
  }
#undef GRAD_LOAD
#undef GRAD_READ
#undef GRAD_PIN
#undef GRAD_STEP
  // The loads of the stages past the last (zeros) may still be landing.
  BITNET_WAIT_VMCNT(0);

  // 32x32 output layout: lane holds column l32 and, for v = 0..15, row
  // 8 (v / 4) + 4 g + v % 4 of its block.
  const float scale = scale_p ? scale_h * *scale_p : scale_h;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = r0 + wm * 32 * RT + rt * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
      if (r >= R) continue;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int cc = c0 + wn * 32 * CT + ct * 32 + l32;
        if (cc >= Cn) continue;
        C[(size_t)r * ldc + cc] = acc[rt][ct][v] * scale;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Operand preparation (HBM-bound; 64 x 64 tiles through LDS, 256 threads).
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const unsigned u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((unsigned)h << 16); }

// fp32 -> (hi, lo) bf16 with hi + lo = f to 16 significant bits.
__device__ __forceinline__ void split_bf16(float f, uint16_t& hi, uint16_t& lo) {
  hi = bf16_rne(f);
  lo = bf16_rne(f - bf16_to_f32(hi));
}

constexpr int kTilePitch = 72;  // uint16 per LDS tile row (64 + 8: 16-B aligned rows)

// t^T in bf16: Wt[k][n] = t[n][k] in {-1, 0, +1} from the packed weights.
// Tile (n0, k0) = (64 bx, 64 by): thread t takes row n = t % 64 and bit pair
// j = t / 64 of its 16-byte block, i.e. k = 16 j + b for bytes b = 0..15.
__global__ __launch_bounds__(256) void expand_transpose_kernel(const uint8_t* __restrict__ Wp,
                                                               int64_t N, int64_t K,
                                                               uint16_t* __restrict__ Wt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kTilePitch];
  const int t = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
  const int n = t & 63, j = t >> 6;
  const uint4 p = *reinterpret_cast<const uint4*>(Wp + (n0 + n) * (K / 4) + k0 / 4);
  const unsigned w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int b = 0; b < 16; ++b) {
    const unsigned code = (w[b >> 2] >> (8 * (b & 3) + 2 * j)) & 3u;
    // code 0 -> -1 (0xBF80), 1 -> 0, 2 -> +1 (0x3F80)
    const uint16_t v = code == 1u ? (uint16_t)0 : (code == 0u ? (uint16_t)0xBF80 : (uint16_t)0x3F80);
    tile[(16 * j + b) * kTilePitch + n] = v;
  }
  __syncthreads();
  const int k = t >> 2, seg = (t & 3) * 16;
  const uint4* src = reinterpret_cast<const uint4*>(tile + k * kTilePitch + seg);
  uint4* dst = reinterpret_cast<uint4*>(Wt + (k0 + k) * N + n0 + seg);
  dst[0] = src[0];
  dst[1] = src[1];
}

// dy (fp32) -> hi, lo bf16 [M, N], 8 elements per thread (M * N % 8 == 0).
__global__ __launch_bounds__(256) void split_rows_kernel(const float* __restrict__ dy, int64_t n8,
                                                         uint16_t* __restrict__ hi,
                                                         uint16_t* __restrict__ lo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(dy)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(dy)[2 * i + 1];
  const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint16_t h[8], l[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) split_bf16(f[e], h[e], l[e]);
  uint4 hv, lv;
  hv.x = h[0] | ((unsigned)h[1] << 16); hv.y = h[2] | ((unsigned)h[3] << 16);
  hv.z = h[4] | ((unsigned)h[5] << 16); hv.w = h[6] | ((unsigned)h[7] << 16);
  lv.x = l[0] | ((unsigned)l[1] << 16); lv.y = l[2] | ((unsigned)l[3] << 16);
  lv.z = l[4] | ((unsigned)l[5] << 16); lv.w = l[6] | ((unsigned)l[7] << 16);
  reinterpret_cast<uint4*>(hi)[i] = hv;
  reinterpret_cast<uint4*>(lo)[i] = lv;
}

__device__ __forceinline__ void load16(const float* p, float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 a = reinterpret_cast<const float4*>(p)[q];
    v[4 * q] = a.x; v[4 * q + 1] = a.y; v[4 * q + 2] = a.z; v[4 * q + 3] = a.w;
  }
}
__device__ __forceinline__ void load16(const uint16_t* p, float* v) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[q];
    const unsigned w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
      v[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

// p = dy * s / c per token, transposed and split: Phi, Plo [N, Mp] with
// Phi[n][m] + Plo[n][m] = dy[m][n] s[m] / c (zero for m >= M).
// Tile (m0, n0) = (64 bx, 64 by).
template <typename DT>
__global__ __launch_bounds__(256) void scale_transpose_split_kernel(
    const DT* __restrict__ dy, const float* __restrict__ scales, float inv_c, int64_t M,
    int64_t N, int64_t Mp, uint16_t* __restrict__ phi, uint16_t* __restrict__ plo) {
  __shared__ float tile[64 * 65];
  const int t = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * 64, n0 = (int64_t)blockIdx.y * 64;
  {
    const int m = t >> 2, seg = (t & 3) * 16;
    float v[16];
    if (m0 + m < M) {
      load16(dy + (m0 + m) * N + n0 + seg, v);
      const float f = scales[m0 + m] * inv_c;
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] *= f;
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) tile[(seg + e) * 65 + m] = v[e];
  }
  __syncthreads();
  const int n = t >> 2, seg = (t & 3) * 16;
  uint16_t h[16], l[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) split_bf16(tile[n * 65 + seg + e], h[e], l[e]);
  uint4 hv[2], lv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    hv[q].x = h[8 * q] | ((unsigned)h[8 * q + 1] << 16);
    hv[q].y = h[8 * q + 2] | ((unsigned)h[8 * q + 3] << 16);
    hv[q].z = h[8 * q + 4] | ((unsigned)h[8 * q + 5] << 16);
    hv[q].w = h[8 * q + 6] | ((unsigned)h[8 * q + 7] << 16);
    lv[q].x = l[8 * q] | ((unsigned)l[8 * q + 1] << 16);
    lv[q].y = l[8 * q + 2] | ((unsigned)l[8 * q + 3] << 16);
    lv[q].z = l[8 * q + 4] | ((unsigned)l[8 * q + 5] << 16);
    lv[q].w = l[8 * q + 6] | ((unsigned)l[8 * q + 7] << 16);
  }
  uint4* dh = reinterpret_cast<uint4*>(phi + (n0 + n) * Mp + m0 + seg);
  uint4* dl = reinterpret_cast<uint4*>(plo + (n0 + n) * Mp + m0 + seg);
  dh[0] = hv[0];
  dh[1] = hv[1];
  dl[0] = lv[0];
  dl[1] = lv[1];
}

// Codes transposed and widened to bf16 (exact: |q| <= 128): Qt[k][m] = q[m][k]
// (zero for m >= M). Tile (m0, k0) = (64 bx, 64 by).
__global__ __launch_bounds__(256) void codes_transpose_kernel(const int8_t* __restrict__ codes,
                                                              int64_t M, int64_t K, int64_t Mp,
                                                              uint16_t* __restrict__ Qt) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kTilePitch];
  const int t = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
  {
    const int m = t >> 2, seg = (t & 3) * 16;
    uint4 p = make_uint4(0u, 0u, 0u, 0u);
    if (m0 + m < M) p = *reinterpret_cast<const uint4*>(codes + (m0 + m) * K + k0 + seg);
    const unsigned w[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int q = (int)(int8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
      tile[(seg + e) * kTilePitch + m] = bf16_rne((float)q);
    }
  }
  __syncthreads();
  const int k = t >> 2, seg = (t & 3) * 16;
  const uint4* src = reinterpret_cast<const uint4*>(tile + k * kTilePitch + seg);
  uint4* dst = reinterpret_cast<uint4*>(Qt + (k0 + k) * Mp + m0 + seg);
  dst[0] = src[0];
  dst[1] = src[1];
}

template <int RT, int CT, int WM, int WN, bool SPLIT>
hipError_t launch_gemm_t(const uint16_t* A, const uint16_t* A2, int64_t lda, const uint16_t* B,
                         int64_t ldb, int64_t R, int64_t Cn, int64_t Kc, float* C, int64_t ldc,
                         const float* scale_p, float scale_h, hipStream_t stream) {
  using S = GShape<RT, CT, WM, WN, SPLIT>;
  const int tiles_m = (int)((R + S::BM - 1) / S::BM);
  const int tiles_n = (int)((Cn + S::BN - 1) / S::BN);
  const int tiles = tiles_m * tiles_n;
  if (tiles == 0) return hipSuccess;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  auto kern = bf16_gemm_nt_kernel<RT, CT, WM, WN, SPLIT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, S::LDS);
  if (e != hipSuccess) return e;
  kern<<<dim3((unsigned)(per_xcd * kXcds)), dim3(S::NT), S::LDS, stream>>>(
      A, A2, lda, B, ldb, (int)R, (int)Cn, (int)Kc, C, ldc, scale_p, scale_h, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

// Two waves per SIMD (eight per workgroup; measured 6-10% faster than four
// larger waves): 256 x 256 tiles of 64 x 128 per wave for one A part; for a
// split A, 128 x 256 tiles of 64 x 64 per wave, the two parts' rows side by
// side in LDS (same MFMA count per stage).
hipError_t launch_bf16_gemm_nt(const uint16_t* A, const uint16_t* A_lo, int64_t lda,
                               const uint16_t* B, int64_t ldb, int64_t R, int64_t Cn, int64_t Kc,
                               float* C, int64_t ldc, const float* scale_p, float scale_h,
                               hipStream_t stream) {
  if (A_lo)
    return launch_gemm_t<2, 2, 2, 4, true>(A, A_lo, lda, B, ldb, R, Cn, Kc, C, ldc, scale_p,
                                           scale_h, stream);
  return launch_gemm_t<2, 4, 4, 2, false>(A, nullptr, lda, B, ldb, R, Cn, Kc, C, ldc, scale_p,
                                          scale_h, stream);
}

hipError_t launch_expand_transpose(const uint8_t* Wpacked, int64_t N, int64_t K, uint16_t* Wt,
                                   hipStream_t stream) {
  if (N == 0 || K == 0) return hipSuccess;
  expand_transpose_kernel<<<dim3((unsigned)(N / 64), (unsigned)(K / 64)), dim3(256), 0, stream>>>(
      Wpacked, N, K, Wt);
  return hipGetLastError();
}

hipError_t launch_split_rows(const float* x, int64_t n, uint16_t* hi, uint16_t* lo,
                             hipStream_t stream) {
  const int64_t n8 = n / 8;
  if (n8 == 0) return hipSuccess;
  split_rows_kernel<<<dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, stream>>>(x, n8, hi, lo);
  return hipGetLastError();
}

hipError_t launch_scale_transpose_split(const void* dy, int dy_dtype, const float* scales,
                                        float inv_c, int64_t M, int64_t N, int64_t Mp,
                                        uint16_t* phi, uint16_t* plo, hipStream_t stream) {
  if (Mp == 0 || N == 0) return hipSuccess;
  const dim3 grid((unsigned)(Mp / 64), (unsigned)(N / 64));
  if (dy_dtype == 1)
    scale_transpose_split_kernel<uint16_t><<<grid, dim3(256), 0, stream>>>(
        reinterpret_cast<const uint16_t*>(dy), scales, inv_c, M, N, Mp, phi, plo);
  else
    scale_transpose_split_kernel<float><<<grid, dim3(256), 0, stream>>>(
        reinterpret_cast<const float*>(dy), scales, inv_c, M, N, Mp, phi, plo);
  return hipGetLastError();
}

hipError_t launch_codes_transpose(const int8_t* codes, int64_t M, int64_t K, int64_t Mp,
                                  uint16_t* Qt, hipStream_t stream) {
  if (Mp == 0 || K == 0) return hipSuccess;
  codes_transpose_kernel<<<dim3((unsigned)(Mp / 64), (unsigned)(K / 64)), dim3(256), 0, stream>>>(
      codes, M, K, Mp, Qt);
  return hipGetLastError();
}

}  // namespace bitnet
