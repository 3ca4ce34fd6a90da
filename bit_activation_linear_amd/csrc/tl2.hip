// TL2 ternary weight code (1.67 bits per weight): re-encoding, the single-token
// decode forward and the batched product (up to 16 tokens).
//
// Edge page (Quillan-Ronin bitnet_cpp_edge.py), module docstring item 2 and
// class SignedUnsignedWeightPacker: the 27 states of a ternary triplet
// (w0, w1, w2) fold onto 14 base triplets (all zero, or first non-zero
// element +1) and a sign, stored as a 4-bit index and one bit: 5 bits per
// 3 weights. In the page's table the index of a base triplet equals its
// balanced-ternary value 9 w0 + 3 w1 + w2, so a triplet of value v has index
// |v| and sign v < 0.
//
// Device layout, per output column, in blocks of 128 triplets (384 weights):
// 64 bytes of 4-bit indices, then 16 bytes of sign bits. Triplet
// j = 32 g + 4 i + tt (group g, slot i, position tt) keeps its index in
// nibble i % 2 of byte 16 g + 4 (i / 2) + tt and its sign in bit i of byte
// 16 G + 4 g + tt, G = 4 groups in a whole block. A partial last block keeps
// only the G groups (96 weights each) the row reaches, padded with zero
// weights, its 20 G bytes rounded up to 16 with zeros: 1.67 bits per weight
// at K = 16384, 1.70 at K = 2560. So the four triplets of one slot sit in the
// four bytes of one index word (one mask spreads them to byte lanes) and in
// bit i of the four bytes of one sign word.
//
// Decode product. As in the 2-bit single-token kernel, one wave owns 16
// output columns and all of K, quantizes the token itself and runs
// v_mfma_i32_16x16x64_i8 with the token as row 0. A weight byte lane carries
// the stored field u = t + 1 in {0, 1, 2} and q . t = q . u - sum(q). A
// slot's four triplet indices become, through two v_perm byte-table lookups
// (entries 0-7 and 8-13), a byte holding the three fields u0 | u1 << 2 |
// u2 << 4 of the base triplet; a set sign bit mirrors the byte to
// 0x2A - byte (each field u -> 2 - u). Fields 0, 1 and 2 are then masked in
// place (worth u, 4u and 16u) and meet the codes of the triplets' first,
// second and third weights in three MFMAs with three accumulators, which
// are scaled back exactly at the end. The codes are written to LDS in that
// order: lane l owns triplets 4 l .. 4 l + 3 of each 768-weight super-block
// and writes the codes of their first, second and third weights as three
// words.
#include "kernels.h"
#include "ternary_common.h"
#include "decode_common.h"

namespace bitnet {
namespace {

constexpr float kEps = 1e-7f;
constexpr int kTl2SuperK = 768;       // weights per super-block (two blocks)

// One thread per (column, block, group): 32 triplets = 96 weights read from
// the 2-bit layout (weight k of a row: field k / 16 % 4 of byte k % 16 of
// 16-byte block k / 64, holding t + 1), 16 index bytes and 4 sign bytes
// written.
__global__ __launch_bounds__(256) void repack_tl2_kernel(const uint8_t* __restrict__ Wp,
                                                         int64_t N, int K, int nblk,
                                                         int64_t row_bytes,
                                                         uint8_t* __restrict__ Wt) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = N * nblk * 4;
  if (tid >= total) return;
  const int g = (int)(tid & 3);
  const int b = (int)((tid >> 2) % nblk);
  const int64_t n = (tid >> 2) / nblk;
  const int gb = b == nblk - 1 ? tl2_last_groups(K) : 4;  // groups of this block
  uint8_t* out = Wt + n * row_bytes + (int64_t)b * kTl2BlockBytes;
  if (g == 0) {  // the bytes the block is rounded up by are zero
    for (int o = 20 * gb; o < (20 * gb + 15) / 16 * 16; o += 4)
      *reinterpret_cast<unsigned*>(out + o) = 0u;
  }
  if (g >= gb) return;
  const uint8_t* row = Wp + n * (int64_t)(K >> 2);
  unsigned idxw[4] = {0u, 0u, 0u, 0u};
  unsigned signw = 0u;
#pragma unroll 4
  for (int jj = 0; jj < 32; ++jj) {
    const int i = jj >> 2, tt = jj & 3;
    const int k0 = kTl2BlockK * b + 3 * (32 * g + jj);
    int t[3];
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int k = k0 + p;
      if (k < K) {
        const uint8_t byte = row[(k >> 6) * 16 + (k & 15)];
        t[p] = (int)((byte >> (2 * ((k >> 4) & 3))) & 3u) - 1;
      } else {
        t[p] = 0;
      }
    }
    const int v = 9 * t[0] + 3 * t[1] + t[2];
    const unsigned idx = (unsigned)(v < 0 ? -v : v);
    idxw[i >> 1] |= idx << (8 * tt + 4 * (i & 1));
    signw |= (v < 0 ? 1u : 0u) << (8 * tt + i);
  }
  *reinterpret_cast<uint4*>(out + 16 * g) = make_uint4(idxw[0], idxw[1], idxw[2], idxw[3]);
  *reinterpret_cast<unsigned*>(out + 16 * gb + 4 * g) = signw;
}

// Field byte u0 | u1 << 2 | u2 << 4 (u = w + 1) of base triplets 0-7 and
// 8-13, four entries per word (the edge page's table, in its order).
constexpr unsigned kLut0 = 0x19092515u;  // (0,0,0) (0,0,1) (0,1,-1) (0,1,0)
constexpr unsigned kLut1 = 0x22120229u;  // (0,1,1) (1,-1,-1) (1,-1,0) (1,-1,1)
constexpr unsigned kLut2 = 0x0A261606u;  // (1,0,-1) (1,0,0) (1,0,1) (1,1,-1)
constexpr unsigned kLut3 = 0x00002A1Au;  // (1,1,0) (1,1,1)

// 0xFF in each byte of x whose bit `bit` is set.
__device__ __forceinline__ unsigned byte_mask(unsigned x, int bit) {
  const unsigned b = (x >> bit) & 0x01010101u;
  return (b << 8) - b;
}

// Field bytes of the four triplets of one slot: idx4 holds their indices
// (0..13) in its bytes, sign4 their signs in bit `bit` of its bytes.
__device__ __forceinline__ unsigned slot_fields(unsigned idx4, unsigned sign4, int bit) {
  const unsigned sel = idx4 & 0x07070707u;
  const unsigned lo = __builtin_amdgcn_perm(kLut1, kLut0, sel);
  const unsigned hi = __builtin_amdgcn_perm(kLut3, kLut2, sel);
  const unsigned f = (byte_mask(idx4, 3) & hi) | (~byte_mask(idx4, 3) & lo);
  const unsigned neg = byte_mask(sign4, bit);
  return (neg & (0x2A2A2A2Au - f)) | (~neg & f);
}

// Single-token decode forward on TL2 weights: WV waves per 16 columns (NB =
// ceil(K / 384) blocks in NS = ceil(NB / 2) 768-weight super-blocks; wave w
// takes super-blocks w NSW .. w NSW + NSW - 1). Every wave reduces the
// per-token statistic over all of x itself (the same fixed order, so the
// same value) and quantizes only its own super-blocks; with several waves, one
// barrier adds their dot products. Quantization as in the 2-bit single-token
// kernel (Eq. 5 / Eq. 6), with each lane owning 12 consecutive values per
// super-block.
template <typename XT, int BITS, int NB, int WV>
__global__ __launch_bounds__(64 * WV) void tl2_decode_kernel(const void* __restrict__ xv,
                                                             const uint8_t* __restrict__ Wt,
                                                             const float* __restrict__ alpha_p,
                                                             float* __restrict__ y, int K, int N,
                                                             float c) {
  constexpr int NS = (NB + 1) / 2;
  constexpr int NSW = (NS + WV - 1) / WV;  // super-blocks per wave
  // codes per wave and super-block: [bb][g][h][p] 16-byte words (768 B), then
  // 64 zero bytes read by the lanes that feed the dead MFMA rows
  __shared__ __attribute__((aligned(16))) int8_t qw_all[WV * NSW * 768 + 64];
  __shared__ int part[16 * (WV > 1 ? WV - 1 : 1)];
  asm volatile("" ::"s"(K), "s"(N), "s"(c), "s"(y), "s"(xv), "s"(Wt));
  const float alpha = *alpha_p;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int s0 = wave * NSW;  // this wave's first super-block
  int8_t* qw = qw_all + wave * NSW * 768;
  int8_t* const qzero = qw_all + WV * NSW * 768;
  // x first: 12 consecutive values per super-block (all of them for the
  // statistic, and again this wave's own for its codes), then the weights
  const XT* x = reinterpret_cast<const XT*>(xv);
  Raw4<XT> xraw[NS][3];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int k0 = kTl2SuperK * s + 12 * lane + 4 * r;
      raw_load4(x, (size_t)(k0 < K ? k0 : 0), xraw[s][r]);
    }
  Raw4<XT> xown[WV > 1 ? NSW : 1][3];
  if constexpr (WV > 1) {
#pragma unroll
    for (int s = 0; s < NSW; ++s)
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        const int k0 = kTl2SuperK * (s0 + s) + 12 * lane + 4 * r;
        raw_load4(x, (size_t)(k0 < K ? k0 : 0), xown[s][r]);
      }
  }
  uint4 widx[2 * NSW];
  unsigned wsign[2 * NSW];
  {
    const int n = blockIdx.x * 16 + col;
    const int nc = n < N ? n : N - 1;
    const uint8_t* wrow = Wt + (size_t)nc * tl2_row_bytes(K);
    const int glast = tl2_last_groups(K);
#pragma unroll
    for (int b = 0; b < 2 * NSW; ++b) {
      // a block past the row's end, and a group past a partial last block's,
      // meet all-zero codes below
      const int bg = 2 * s0 + b < NB ? 2 * s0 + b : NB - 1;
      const int gb = bg == NB - 1 ? glast : 4;
      const int gs = grp < gb ? grp : gb - 1;
      const uint8_t* blk = wrow + bg * kTl2BlockBytes;
      widx[b] = *reinterpret_cast<const uint4*>(blk + 16 * gs);
      wsign[b] = *reinterpret_cast<const unsigned*>(blk + 16 * gb + 4 * gs);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  float v[NSW][12];
  float st = 0.0f;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const bool own = kTl2SuperK * s + 12 * lane + 4 * r < K;
      float w4[4];
      widen4(xraw[s][r], w4);
      if constexpr (WV == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[s][4 * r + e] = w4[e];
      }
      if (BITS == 8) {
        const float m = fmaxf(fmaxf(fabsf(w4[0]), fabsf(w4[1])), fmaxf(fabsf(w4[2]), fabsf(w4[3])));
        st = fmaxf(st, own ? m : 0.0f);
      } else {
        const float m = (fabsf(w4[0]) + fabsf(w4[1])) + (fabsf(w4[2]) + fabsf(w4[3]));
        st += own ? m : 0.0f;
      }
    }
  if constexpr (WV > 1) {
#pragma unroll
    for (int s = 0; s < NSW; ++s)
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        float w4[4];
        widen4(xown[s][r], w4);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[s][4 * r + e] = w4[e];
      }
  }
  st = (BITS == 8) ? wave_reduce<true>(st) : wave_reduce<false>(st);
  if (BITS == 4) st = st / (float)K;
  st += kEps;
  const float mult = c / st;
  // Codes as in the 2-bit single-token kernel (magic-number rounding, med3
  // clamp, the code in the sum's low byte).
  constexpr float kMagic = 12582912.0f;
  const float lo = kMagic + ((BITS == 8) ? -128.0f : -8.0f);
  const float hi = kMagic + ((BITS == 8) ? 127.0f : 7.0f);
  int qsum = 0;
  // this lane's triplets in the super-block: block half bb, group g, slot i
  const int bb = lane >> 5, g = (lane >> 3) & 3, i = lane & 7;
  const int wbase = ((bb * 4 + g) * 2 + (i >> 2)) * 48 + 4 * (i & 3);
#pragma unroll
  for (int s = 0; s < NSW; ++s) {
    unsigned b[12];
#pragma unroll
    for (int e = 0; e < 12; ++e) {
      const bool own = kTl2SuperK * (s0 + s) + 12 * lane + e < K;
      float pr = v[s][e] * mult;
      asm volatile("" : "+v"(pr));
      b[e] = own ? __float_as_uint(__builtin_amdgcn_fmed3f(pr + kMagic, lo, hi)) : 0u;
    }
    // word p: codes of the triplets' weights p (values p, p + 3, p + 6, p + 9)
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const unsigned word = __builtin_amdgcn_perm(b[p + 3], b[p], 0x0C0C0400u) |
                            __builtin_amdgcn_perm(b[p + 9], b[p + 6], 0x04000C0Cu);
      qsum = __builtin_amdgcn_sdot4((int)word, 0x01010101, qsum, false);
      *reinterpret_cast<unsigned*>(qw + s * 768 + wbase + 16 * p) = word;
    }
  }
  if (lane < 16) *reinterpret_cast<unsigned*>(qzero + 4 * lane) = 0u;  // each wave, before its own reads
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  qsum = wave_sum_int(qsum);

  // MFMA operands: lane (col, grp) feeds column col's slots 4 h .. 4 h + 3 of
  // group grp of each block; lanes of token row 0 (col == 0) feed the codes.
  v4i acc1 = v4i{0, 0, 0, 0}, acc4 = v4i{0, 0, 0, 0}, acc16 = v4i{0, 0, 0, 0};
#pragma unroll
  for (int b = 0; b < 2 * NSW; ++b) {
    if (2 * s0 + b >= NB) break;  // past the row (uniform)
    const unsigned iw[4] = {widx[b].x, widx[b].y, widx[b].z, widx[b].w};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int8_t* qa = col == 0
                             ? qw + (b >> 1) * 768 + (((b & 1) * 4 + grp) * 2 + h) * 48
                             : qzero;
      const int step = col == 0 ? 16 : 0;
      v4i u1, u4, u16;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        const int slot = 4 * h + sl;
        const unsigned idx4 = (iw[slot >> 1] >> (4 * (slot & 1))) & 0x0F0F0F0Fu;
        const unsigned f = slot_fields(idx4, wsign[b], slot);
        u1[sl] = (int)(f & 0x03030303u);
        u4[sl] = (int)(f & 0x0C0C0C0Cu);
        u16[sl] = (int)(f & 0x30303030u);
      }
      acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const v4i*>(qa), u1, acc1,
                                                   0, 0, 0);
      acc4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const v4i*>(qa + step), u4,
                                                   acc4, 0, 0, 0);
      acc16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          *reinterpret_cast<const v4i*>(qa + 2 * step), u16, acc16, 0, 0, 0);
    }
  }
  int dot = acc1[0] + (acc4[0] >> 2) + (acc16[0] >> 4) - qsum;
  if constexpr (WV > 1) {
    if (wave > 0 && grp == 0) part[(wave - 1) * 16 + col] = dot;
    lds_barrier();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < WV; ++w) dot += part[(w - 1) * 16 + col];
  }
  const int n = blockIdx.x * 16 + col;
  if (grp == 0 && n < N) y[n] = (float)dot * dequant_factor(alpha, st, c);
}

// Batched TL2 product (the edge page's TL2 GEMV takes a batch of tokens):
// y[m, n] for M <= 16 token rows from int8 codes in TL2 order (per row,
// blocks of 384 codes, the code of weight 3 j + p of a block at its byte
// 128 p + j, the codes past K zero) with the codes' row sums. A workgroup
// owns 16 output columns and wave w the blocks w, w + NW, ...; per block a
// lane (col, grp) loads its column's index and sign words of group grp and,
// for token row col, the six 16-byte code operands (field p, half h: bytes
// 128 p + 32 grp + 16 h of the block), so that MFMA k = 16 grp + e meets the
// group's triplet 16 h + e in both operands, as in the single-token kernel.
// Up to kTl2Rounds blocks' loads go out together; one barrier adds the
// waves' tiles.
constexpr int kTl2Rounds = 3;

__global__ __launch_bounds__(1024) void tl2_gemv_kernel(const int8_t* __restrict__ codes,
                                                       const float* __restrict__ scales,
                                                       const int32_t* __restrict__ rowsum,
                                                       const uint8_t* __restrict__ Wt,
                                                       const float* __restrict__ alpha_p,
                                                       float* __restrict__ y, int M, int K, int N,
                                                       float c) {
  __shared__ v4i red[16 * 64];
  const int nw = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int nblk = (K + kTl2BlockK - 1) / kTl2BlockK;
  const int ktl2 = nblk * kTl2BlockK;
  const int n = blockIdx.x * 16 + col;
  const uint8_t* wrow = Wt + (size_t)(n < N ? n : N - 1) * tl2_row_bytes(K);
  const int glast = tl2_last_groups(K);
  const int8_t* crow = codes + (size_t)(col < M ? col : M - 1) * ktl2;
  // the epilogue's operands, fetched before the weight stream
  const float alpha = *alpha_p;
  float s_row[4];
  int rs[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * grp + v < M ? 4 * grp + v : M - 1;
    s_row[v] = scales[m];
    rs[v] = rowsum[m];
  }
  v4i acc1 = v4i{0, 0, 0, 0}, acc4 = v4i{0, 0, 0, 0}, acc16 = v4i{0, 0, 0, 0};
  auto round = [&](const int b0) {
    uint4 widx[kTl2Rounds];
    unsigned wsign[kTl2Rounds];
    v4i a[kTl2Rounds][2][3];
#pragma unroll
    for (int r = 0; r < kTl2Rounds; ++r) {
      const int b = b0 + r * nw;
      const int bc = b < nblk ? b : nblk - 1;  // a dead block reloads the last one, unused
      // a group past a partial last block's reloads its last group (its codes are zero)
      const int gb = bc == nblk - 1 ? glast : 4;
      const int gs = grp < gb ? grp : gb - 1;
      widx[r] = *reinterpret_cast<const uint4*>(wrow + (size_t)bc * kTl2BlockBytes + 16 * gs);
      wsign[r] = *reinterpret_cast<const unsigned*>(wrow + (size_t)bc * kTl2BlockBytes + 16 * gb +
                                                    4 * gs);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int p = 0; p < 3; ++p)
          a[r][h][p] = *reinterpret_cast<const v4i*>(crow + (size_t)bc * kTl2BlockK + 128 * p +
                                                     32 * grp + 16 * h);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < kTl2Rounds; ++r) {
      if (b0 + r * nw >= nblk) break;  // uniform
      const unsigned iw[4] = {widx[r].x, widx[r].y, widx[r].z, widx[r].w};
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v4i u1, u4, u16;
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const int slot = 4 * h + sl;
          const unsigned idx4 = (iw[slot >> 1] >> (4 * (slot & 1))) & 0x0F0F0F0Fu;
          const unsigned f = slot_fields(idx4, wsign[r], slot);
          u1[sl] = (int)(f & 0x03030303u);
          u4[sl] = (int)(f & 0x0C0C0C0Cu);
          u16[sl] = (int)(f & 0x30303030u);
        }
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[r][h][0], u1, acc1, 0, 0, 0);
        acc4 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[r][h][1], u4, acc4, 0, 0, 0);
        acc16 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[r][h][2], u16, acc16, 0, 0, 0);
      }
    }
  };
  // The first round is not inside the loop (a loop header would wait for
  // every load in flight before the first one's use).
  round(wave);
  for (int b0 = wave + kTl2Rounds * nw; b0 < nblk; b0 += kTl2Rounds * nw) round(b0);
  // q . u over the three scales (exact: acc4 holds multiples of 4, acc16 of 16)
  red[wave * 64 + lane] = acc1 + (acc4 >> 2) + (acc16 >> 4);
  lds_barrier();
  if (wave != 0 || n >= N) return;
  v4i total = red[lane];
  for (int w = 1; w < nw; ++w) total += red[w * 64 + lane];
  // 16x16 MFMA layout: lane l holds rows 4 (l / 16) + v, column l % 16
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int m = 4 * grp + v;
    if (m < M) y[(size_t)m * N + n] = (float)(total[v] - rs[v]) * dequant_factor(alpha, s_row[v], c);
  }
}

// Waves per 16 columns: one per super-block, at most four (measured at
// K = 2560, four super-blocks: 4.8 us against 5.45 us with two waves of
// two).
template <typename XT, int BITS, int NB, int WV = ((NB + 1) / 2 < 4 ? (NB + 1) / 2 : 4)>
hipError_t launch_tl2_nb(const void* x, const uint8_t* Wt, const float* alpha, float* y, int K,
                         int64_t N, hipStream_t stream) {
  const float c = (BITS == 8) ? kScaleInt8 : kScaleInt4;
  tl2_decode_kernel<XT, BITS, NB, WV><<<dim3((unsigned)((N + 15) / 16)), dim3(64 * WV), 0,
                                        stream>>>(x, Wt, alpha, y, K, (int)N, c);
  return hipGetLastError();
}

template <typename XT, int BITS>
hipError_t launch_tl2_t(const void* x, const uint8_t* Wt, const float* alpha, float* y, int K,
                        int64_t N, hipStream_t stream) {
  switch ((K + kTl2BlockK - 1) / kTl2BlockK) {
#define BITNET_TL2_CASE(nb) \
  case nb: return launch_tl2_nb<XT, BITS, nb>(x, Wt, alpha, y, K, N, stream);
    BITNET_TL2_CASE(1) BITNET_TL2_CASE(2) BITNET_TL2_CASE(3) BITNET_TL2_CASE(4)
    BITNET_TL2_CASE(5) BITNET_TL2_CASE(6) BITNET_TL2_CASE(7) BITNET_TL2_CASE(8)
    BITNET_TL2_CASE(9) BITNET_TL2_CASE(10) BITNET_TL2_CASE(11) BITNET_TL2_CASE(12)
#undef BITNET_TL2_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_repack_tl2(const uint8_t* Wpacked, int64_t N, int K, uint8_t* Wtl2,
                             hipStream_t stream) {
  const int nblk = (K + kTl2BlockK - 1) / kTl2BlockK;
  const int64_t threads = N * nblk * 4;
  if (threads == 0) return hipSuccess;
  repack_tl2_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream>>>(
      Wpacked, N, K, nblk, tl2_row_bytes(K), Wtl2);
  return hipGetLastError();
}

hipError_t launch_tl2_gemv(const int8_t* codes, const float* scales, const int32_t* rowsum,
                           int64_t M, int K, const uint8_t* Wtl2, int64_t N, const float* alpha,
                           int bits, float* y, hipStream_t stream) {
  if (M < 1 || M > 16 || K < 1) return hipErrorInvalidValue;
  const int nblk = (K + kTl2BlockK - 1) / kTl2BlockK;
  const int nw = nblk < 16 ? nblk : 16;
  const float c = (bits == 8) ? kScaleInt8 : kScaleInt4;
  tl2_gemv_kernel<<<dim3((unsigned)((N + 15) / 16)), dim3(64 * nw), 0, stream>>>(
      codes, scales, rowsum, Wtl2, alpha, y, (int)M, K, (int)N, c);
  return hipGetLastError();
}

hipError_t launch_tl2_decode(const void* x, int x_dtype, int K, const uint8_t* Wtl2, int64_t N,
                             const float* alpha, int bits, float* y, hipStream_t stream) {
  if (K > kTl2MaxK) return hipErrorInvalidValue;
  if (x_dtype == 1)
    return bits == 8 ? launch_tl2_t<uint16_t, 8>(x, Wtl2, alpha, y, K, N, stream)
                     : launch_tl2_t<uint16_t, 4>(x, Wtl2, alpha, y, K, N, stream);
  return bits == 8 ? launch_tl2_t<float, 8>(x, Wtl2, alpha, y, K, N, stream)
                   : launch_tl2_t<float, 4>(x, Wtl2, alpha, y, K, N, stream);
}

}  // namespace bitnet
