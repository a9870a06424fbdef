// Bulk encode of fp16 vectors on the matrix cores (gfx950): tq_encode's flat
// records and tq_append_page's bulk appends into pages.
//
// Same per-vector steps as the vector-ALU encoder in encode.hip ("aither-
// kvcache" README, section "Algorithm"; keys' residual sketch from "TurboQuant
// on a 16GB MacBook", sections "Why this caught my eye" and "The QJL detective
// story"): n = ||x||, y = Pi x / n, codes = boundaries below y, and for keys
// r = Pi x - n c[code], ||r||, sign bits of S r.  The two d x d products are
// dense contractions over a tile of vectors and run as MFMA 16x16x32 f16:
//  * Y = Pi X: the fp16 input is exact as an operand; Pi (fp32) is scaled by
//    16 and split into fp16 hi + lo parts (two MFMAs), which keeps ~22 bits;
//  * Z = S R: R is scaled by 64/n and S is split as well; hi*hi + hi*lo +
//    lo*hi (three MFMAs) keep the sign decisions far inside the guard band.
// The matrices live in LDS as ready-made A-operand fragments.  The rows of
// each product are permuted so that lane (n, kg) of a wave ends with the 32
// consecutive coordinates 32kg .. 32kg+31 of vector n: its codes form whole
// 32-bit words of the LSB-first stream and its 32 sign bits are one word,
// so packing needs no communication between lanes.  The contraction order is
// permuted the same way (MFMA k index 8kg + i of step s is coordinate
// 32kg + 8s + i), so every operand a lane feeds is its own data.
// The Hadamard variant rotates with butterflies (five stages inside a lane,
// two across the lane groups) and keeps the dense QJL product.
//
// Bulk append ("TurboQuant Family Design Study", sections "Packed format and
// complete bit accounting" and "Paging, lifecycle, and cache identity"): one
// wave encodes one 32-token value group of one (sequence, KV head) at a time,
// taking its tokens from the FP16 ring (tokens already cached) or from the new
// rows, and writes key records token by token, or the group's value words
// (for each coordinate, the 32 tokens' codes as one bit string), which the
// wave forms with a transpose of the code fields across its lanes.
#include <type_traits>

#include "device_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kEncThreads = 512;
constexpr int kEncWaves = kEncThreads / 64;
// 16-vector MFMA column blocks per wave iteration: two for the dense
// rotation (each matrix fragment read from LDS feeds two MFMAs), one for the
// Hadamard variant (its butterflies keep 32 values per vector in registers)
__host__ __device__ constexpr int cols_for(bool had) { return had ? 1 : 2; }

__device__ inline f4 mfma(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

__device__ inline uint32_t hbits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}
__device__ inline float hval(uint32_t h) { return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h))); }

// Scaled matrix M' = scale * M split into fp16 hi/lo A-operand fragments:
// fragment (t, s, part) of lane l holds M'[row][32kg + 8s + i], i = 0..7, with
// m = l & 15, kg = l >> 4, row = 32 (m >> 2) + 4t + (m & 3).
__device__ void build_frags(u4* frag, const float* M, float scale, int tid) {
  for (int e = tid; e < 8 * 4 * 64; e += kEncThreads) {
    const int l = e & 63, s = (e >> 6) & 3, tt = e >> 8;
    const int m = l & 15, kg = l >> 4;
    const int row = 32 * (m >> 2) + 4 * tt + (m & 3);
    const float4* src = reinterpret_cast<const float4*>(M + row * kD + 32 * kg + 8 * s);
    const float4 v0 = src[0], v1 = src[1];
    const float v[8] = {v0.x * scale, v0.y * scale, v0.z * scale, v0.w * scale,
                        v1.x * scale, v1.y * scale, v1.z * scale, v1.w * scale};
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t h0 = hbits(v[2 * i]), h1 = hbits(v[2 * i + 1]);
      hi[i] = h0 | (h1 << 16);
      lo[i] = hbits(v[2 * i] - hval(h0)) | (hbits(v[2 * i + 1] - hval(h1)) << 16);
    }
    frag[((tt * 4 + s) * 2 + 0) * 64 + l] = u4{hi[0], hi[1], hi[2], hi[3]};
    frag[((tt * 4 + s) * 2 + 1) * 64 + l] = u4{lo[0], lo[1], lo[2], lo[3]};
  }
}

struct EncCodebook {
  float cen[16];
  float bnd[16];
  float cen2[16];  // mixed-channel rate: the (b+1)-bit codebook of the high-rate half
  float bnd2[16];
};

// Code of y: the number of decision boundaries strictly below it.  The
// codebook is symmetric with boundaries 0, +-p_1 < .. < p_{H-1}.  With s the
// sign bit of y and m' the bit pattern of |y| plus s (the next float up for
// y < 0; non-negative floats order like their bit patterns): y > 0 gives
// H + #{p_k < m'}, y < 0 gives H - 1 - #{p_k <= |y|} = H - 1 - #{p_k < m'},
// and both are cnt XOR (H - s).  (y = +0 takes code H rather than H - 1: a
// value on the boundary 0, inside the guard band.)  The count comes from a
// branch-free binary search over the positive boundaries (bit patterns
// pb[1..H-1], uniform): each step compares m' with one boundary through the
// sign of the difference and picks the next boundary with a bit select, so
// no lane masks and no table are involved.
template <int BITS>
__device__ __forceinline__ uint32_t quantize_search(float y, const uint32_t* pb) {
  constexpr uint32_t H = 1u << (BITS - 1);
  const uint32_t bits = __builtin_bit_cast(uint32_t, y);
  const uint32_t sgn = bits >> 31;
  const uint32_t m = (bits & 0x7fffffffu) + sgn;
  // all-ones where m' > p (both below 2^31: the difference cannot wrap)
  auto gt = [&](uint32_t p) { return static_cast<uint32_t>(static_cast<int32_t>(p - m) >> 31); };
  // mask ? a : b, bit by bit (v_bitop3 with truth table 0xCA for operands
  // mask, a, b); written as the instruction so that the compiler keeps the
  // mask arithmetic instead of turning it into compares and lane masks
  auto pick = [](uint32_t mask, uint32_t a, uint32_t b) { return __builtin_amdgcn_bitop3_b32(mask, a, b, 0xCA); };
  uint32_t cnt;
  if constexpr (BITS == 2) {
    cnt = (pb[1] - m) >> 31;
  } else if constexpr (BITS == 3) {
    const uint32_t g2 = gt(pb[2]);
    cnt = ((pick(g2, pb[3], pb[1]) - m) >> 31) - 2u * g2;
  } else {
    const uint32_t g4 = gt(pb[4]);
    const uint32_t g2 = gt(pick(g4, pb[6], pb[2]));
    const uint32_t t1 = pick(g4, pick(g2, pb[7], pb[5]), pick(g2, pb[3], pb[1]));
    cnt = ((t1 - m) >> 31) - 2u * (2u * g4 + g2);
  }
  return cnt ^ (H - sgn);
}

// 32-lane-group sum of a double over the four lanes holding one vector
__device__ inline double sum4(double v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// One stage of a transpose of small fields across lanes: lanes that differ
// in lane bit XOR swap blocks of S bits (mask M selects the blocks a lane
// keeps in place).  Three stages transpose an 8 x 8 matrix of 4-bit fields
// held as one word per lane over 8 lanes, four a 16 x 16 matrix of 2-bit
// fields over 16 lanes: field i of lane r becomes field r of lane i.
template <int XOR, uint32_t M, int S>
__device__ __forceinline__ uint32_t xchg_fields(uint32_t x, int lane) {
  const uint32_t p = static_cast<uint32_t>(__shfl_xor(static_cast<int>(x), XOR, 64));
  return (lane & XOR) ? (((p >> S) & M) | (x & ~M)) : ((x & M) | ((p & M) << S));
}
__device__ __forceinline__ uint32_t transpose_nibbles8(uint32_t x, int lane) {
  x = xchg_fields<1, 0x0F0F0F0Fu, 4>(x, lane);
  x = xchg_fields<2, 0x00FF00FFu, 8>(x, lane);
  return xchg_fields<4, 0x0000FFFFu, 16>(x, lane);
}
__device__ __forceinline__ uint32_t transpose_crumbs16(uint32_t x, int lane) {
  x = xchg_fields<1, 0x33333333u, 2>(x, lane);
  x = xchg_fields<2, 0x0F0F0F0Fu, 4>(x, lane);
  x = xchg_fields<4, 0x00FF00FFu, 8>(x, lane);
  return xchg_fields<8, 0x0000FFFFu, 16>(x, lane);
}
// 8 fields of 3 bits (24 bits) <-> 8 nibbles (the high bit of each zero)
__device__ __forceinline__ uint32_t spread3to4(uint32_t x) {
  x = ((x & 0xFFF000u) << 4) | (x & 0xFFFu);
  x = ((x & 0x0FC00FC0u) << 2) | (x & 0x003F003Fu);
  return ((x & 0x38383838u) << 1) | (x & 0x07070707u);
}
__device__ __forceinline__ uint32_t pack4to3(uint32_t x) {
  x = (x & 0x07070707u) | ((x & 0x70707070u) >> 1);
  x = (x & 0x003F003Fu) | ((x & 0x3F003F00u) >> 2);
  return (x & 0x00000FFFu) | ((x & 0x0FFF0000u) >> 4);
}

// Encodes the COLS x 16 vectors whose fp16 coordinates the lanes hold in xb
// (zeros for dead vectors: they come out as the zero vector's record); lane
// (n, kg) of column block c holds vector 16c + n, coordinates 32kg .. 32kg+31.
// Results go to two callbacks, each called for c = 0 .. COLS-1 as soon as
// they exist (so they need not stay in registers):
//   codes(c, words, words2, nst, nq): the lane's BITS words of the vector's
//     LSB-first code stream, the stored norm (f32 norm, or the u8 log-norm
//     level) and the u8 log-norm code (N8).  With a mixed-channel rate
//     (MIXMOD = M > 0: coordinate j takes BITS + 1 bits and the second
//     codebook when j mod M >= M/2) words holds the low-rate codes and words2
//     the high-rate ones, each in rank order (rank of the lane's coordinate j
//     within its half: (j / M)(M/2) + j mod M/2), 16 codes each;
//   signs(c, rn, sw): ||r|| and the sign bits of coordinates 32kg .. 32kg+31 (QJL).
// frag*: the LDS fragments; ctab: the centroids in LDS (then those of the
// (b+1)-bit codebook, mixed rates); emask: the lane's
// Hadamard signs as fp16 sign-bit masks over its input words (bit 15 or 31
// set where the sign is -1); ntab: the u8 log-norm levels then boundaries (N8).
template <bool QJL, bool HAD, int BITS, bool N8, int COLS, int MIXMOD, class CodesFn, class SignsFn>
__device__ __forceinline__ void encode_tile(const u4* fragP, const u4* fragS, const float* ctab, const u4* emask,
                                            const EncCodebook& cbk, const float* ntab,
                                            const u4 (&xb)[COLS][4], CodesFn&& codes_out, SignsFn&& signs_out) {
  const int l = threadIdx.x & 63;
  // the dense product comes out scaled by 16 (Pi's fragments are): y, the
  // residual and its norm take that factor out where they are formed
  constexpr float kScale = HAD ? 1.0f : 16.0f, kInv = HAD ? 1.0f : 0.0625f;
  // positive boundaries as bit patterns: pbits[k] = p_k, k = 1 .. H-1
  uint32_t pbits[1 << (BITS - 1)];
#pragma unroll
  for (int k = 0; k < (1 << (BITS - 1)); ++k) pbits[k] = __builtin_bit_cast(uint32_t, cbk.bnd[(1 << (BITS - 1)) - 1 + k]);
  uint32_t pbits2[MIXMOD ? (1 << BITS) : 1];
  if constexpr (MIXMOD > 0) {
#pragma unroll
    for (int k = 0; k < (1 << BITS); ++k) pbits2[k] = __builtin_bit_cast(uint32_t, cbk.bnd2[(1 << BITS) - 1 + k]);
  }
  // ---- norms (double accumulation, as the vector-ALU path)
  float n32[COLS], invn[COLS], nstv[COLS];
  int nqv[COLS];
#pragma unroll
  for (int c = 0; c < COLS; ++c) {
    double ss = 0.0;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const double e0 = hval(xb[c][s][w] & 0xffffu), e1 = hval(xb[c][s][w] >> 16);
        ss = fma(e0, e0, ss);
        ss = fma(e1, e1, ss);
      }
    ss = sum4(ss);
    const double nn = sqrt(ss);
    n32[c] = static_cast<float>(nn);
    invn[c] = nn > 0.0 ? static_cast<float>(1.0 / nn) : 0.0f;
    nstv[c] = n32[c];
    nqv[c] = 0;
    if constexpr (N8) {
      const int q = norm_code(n32[c], ntab + kNormCodes);
      nqv[c] = q;
      nstv[c] = ntab[q];
    }
  }
  // ---- y (unnormalised, fp32): lane holds coordinate 32kg + 4tt + r in acc[c][tt][r]
  f4 acc[COLS][8];
  if constexpr (!HAD) {
#pragma unroll
    for (int c = 0; c < COLS; ++c)
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) acc[c][tt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    // one output tile at a time: the scheduling barrier keeps later tiles'
    // fragment reads from being hoisted (they would all be live at once;
    // reading the next tile ahead measured no faster)
    u4 fa[8];
    auto ldP = [&](int tt, u4* f) {
#pragma unroll
      for (int q = 0; q < 8; ++q) f[q] = fragP[(tt * 8 + q) * 64 + l];
    };
    ldP(0, fa);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      u4* cur = fa;
      if (tt > 0) ldP(tt, cur);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int c = 0; c < COLS; ++c) {
          acc[c][tt] = mfma(cur[2 * s], xb[c][s], acc[c][tt]);
          acc[c][tt] = mfma(cur[2 * s + 1], xb[c][s], acc[c][tt]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // y = H (eps . x) / sqrt(d), natural (Sylvester) order
#pragma unroll
    for (int c = 0; c < COLS; ++c) {
      float v[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const uint32_t w = xb[c][j >> 3][(j >> 1) & 3] ^ emask[j >> 3][(j >> 1) & 3];
        v[j] = hval((j & 1) ? (w >> 16) : (w & 0xffffu));
      }
#pragma unroll
      for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int j = 0; j < 32; ++j)
          if (!(j & h)) {
            const float p = v[j], q = v[j + h];
            v[j] = p + q;
            v[j + h] = p - q;
          }
#pragma unroll
      for (int h = 16; h <= 32; h <<= 1)
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const float ov = __shfl_xor(v[j], h, 64);
          v[j] = (l & h) ? (ov - v[j]) : (v[j] + ov);
        }
#pragma unroll
      for (int j = 0; j < 32; ++j) acc[c][j >> 2][j & 3] = v[j] * 0.08838834764831845f;
    }
  }
  // ---- quantise, pack, residual
  u4 rb[COLS][4][2];  // B operands of the residual product (hi / lo)
  float rnv[COLS];
#pragma unroll
  for (int c = 0; c < COLS; ++c) {
    uint32_t words[BITS], words2[MIXMOD ? 2 : 1];
#pragma unroll
    for (int w = 0; w < BITS; ++w) words[w] = 0u;
    words2[0] = 0u;
    if constexpr (MIXMOD > 0) words2[1] = 0u;
    float rv[32];
    float rs = 0.0f;
    // y = acc / (kScale n); residual r kScale = acc - kScale nst c[code]
    const float ys = invn[c] * kInv, nsts = -nstv[c] * kScale, rvs = 64.0f * kInv * invn[c];
    const uint32_t live = n32[c] > 0.0f ? 0xffffffffu : 0u;  // a zero vector keeps all-zero codes
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float accv = acc[c][j >> 2][j & 3];
      const bool hi = MIXMOD > 0 && (j % (MIXMOD > 0 ? MIXMOD : 1)) >= MIXMOD / 2;
      uint32_t code;
      if constexpr (MIXMOD > 0)
        code = hi ? quantize_search<BITS + 1>(accv * ys, pbits2) : quantize_search<BITS>(accv * ys, pbits);
      else
        code = quantize_search<BITS>(accv * ys, pbits);
      code &= live;
      if constexpr (MIXMOD > 0) {
        const int rank = (j / MIXMOD) * (MIXMOD / 2) + (j % MIXMOD) % (MIXMOD / 2);
        const int wd = hi ? BITS + 1 : BITS, pos = rank * wd;
        uint32_t* ws = hi ? words2 : words;
        ws[pos >> 5] |= code << (pos & 31);
        if ((pos & 31) + wd > 32) ws[(pos >> 5) + 1] |= code >> (32 - (pos & 31));
      } else {
        const int pos = j * BITS;
        words[pos >> 5] |= code << (pos & 31);
        if ((pos & 31) + BITS > 32) words[(pos >> 5) + 1] |= code >> (32 - (pos & 31));
      }
      if constexpr (QJL) {
        // the residual against the stored reconstruction nst c[code]
        // (a zero vector has accv = 0 and nst = 0: r = 0 without a branch)
        const float r = fmaf(nsts, ctab[(hi ? 16 : 0) + code], accv);
        rs = fmaf(r, r, rs);
        rv[j] = r * rvs;
      }
    }
    codes_out(c, words, words2, nstv[c], nqv[c]);
    if constexpr (QJL) {
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      rnv[c] = sqrtf(rs) * kInv;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // hi truncated to fp16, lo = the exact fp32 remainder truncated again
          const float r0 = rv[8 * s + 2 * i], r1 = rv[8 * s + 2 * i + 1];
          const auto hp = __builtin_amdgcn_cvt_pkrtz(r0, r1);
          hi[i] = __builtin_bit_cast(uint32_t, hp);
          lo[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0 - static_cast<float>(hp[0]),
                                                                          r1 - static_cast<float>(hp[1])));
        }
        rb[c][s][0] = u4{hi[0], hi[1], hi[2], hi[3]};
        rb[c][s][1] = u4{lo[0], lo[1], lo[2], lo[3]};
      }
    }
  }
  if constexpr (QJL) {
    // ---- z = S r (scaled), one sign word per lane: bit 4tt + r of word kg
    // is set for z >= 0; collected as the sign bits of z, complemented at the
    // end (z = -0 counts as negative: a value on the decision, in the band)
    uint32_t sw[COLS] = {};
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      f4 z[COLS];
#pragma unroll
      for (int c = 0; c < COLS; ++c) z[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u4 sh = fragS[((tt * 4 + s) * 2 + 0) * 64 + l];
        const u4 sl = fragS[((tt * 4 + s) * 2 + 1) * 64 + l];
#pragma unroll
        for (int c = 0; c < COLS; ++c) {
          z[c] = mfma(sh, rb[c][s][0], z[c]);
          z[c] = mfma(sh, rb[c][s][1], z[c]);
          z[c] = mfma(sl, rb[c][s][0], z[c]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < COLS; ++c)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float zr = z[c][r];  // (a scalar first: bit-casting the vector element reads element 0)
          sw[c] |= (__builtin_bit_cast(uint32_t, zr) >> 31) << (4 * tt + r);
        }
    }
#pragma unroll
    for (int c = 0; c < COLS; ++c) signs_out(c, rnv[c], (n32[c] > 0.0f) ? ~sw[c] : 0u);
  }
}

// Builds the work-group's LDS tables (all threads) and the lane's Hadamard
// sign masks (for coordinates 32kg + 8s + 2i, 2i+1: bits 15, 31 of word i of emask[s]).
template <bool QJL, bool HAD>
__device__ __forceinline__ void setup_tables(u4* fragP, u4* fragS, float* ctab, const DevTables& t,
                                             const EncCodebook& cbk, u4* emask) {
  const int tid = threadIdx.x;
  if (!HAD) build_frags(fragP, t.rot, 16.0f, tid);
  if (QJL) build_frags(fragS, t.S, 1.0f, tid);
  if (tid < 32) {
    float cv = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k == tid) cv = cbk.cen[k];
      if (k + 16 == tid) cv = cbk.cen2[k];
    }
    ctab[tid] = cv;
  }
  if constexpr (HAD) {
    const int kg = (tid & 63) >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e0 = t.rot[32 * kg + 8 * s + 2 * i], e1 = t.rot[32 * kg + 8 * s + 2 * i + 1];
        emask[s][i] = (e0 < 0.0f ? 0x8000u : 0u) | (e1 < 0.0f ? 0x80000000u : 0u);
      }
  }
  __syncthreads();
}

// Two work-groups per CU need <= 128 VGPRs; the dense key variant holds both
// matrices (128 KB of LDS) and fits only one anyway.
// MIXMOD > 0: mixed-channel rate (coordinate j at BITS + 1 bits when
// j mod MIXMOD >= MIXMOD/2); a record holds the low-rate codes, then the
// high-rate ones, each in rank order.
template <bool QJL, bool HAD, int BITS, bool N8, int MIXMOD>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu((QJL && !HAD) ? 2 : 4)))
void encode_mma_kernel(EncodeArgs a, DevTables t, EncCodebook cbk) {
  __shared__ u4 fragP[HAD ? 1 : 8 * 4 * 2 * 64];  // 64 KB
  __shared__ u4 fragS[QJL ? 8 * 4 * 2 * 64 : 1];  // 64 KB
  __shared__ float ctab[32];
  u4 emask[4];  // Hadamard signs of this lane's coordinates
  setup_tables<QJL, HAD>(fragP, fragS, ctab, t, cbk, emask);

  constexpr int kCols = cols_for(HAD), kTileVec = 16 * kCols;
  const int tid = threadIdx.x;
  const int l = tid & 63, n = l & 15, kg = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t ntiles = (a.n + kTileVec - 1) / kTileVec;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kEncWaves;
  const _Float16* X = static_cast<const _Float16*>(a.x);

  for (int64_t tile = static_cast<int64_t>(blockIdx.x) * kEncWaves + wave; tile < ntiles; tile += stride) {
    // ---- load: lane (n, kg) of block c takes vector 32 tile + 16 c + n, coordinates 32kg .. 32kg+31
    u4 xb[kCols][4];
    int64_t vid[kCols];
    bool live[kCols];
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      vid[c] = tile * kTileVec + 16 * c + n;
      live[c] = vid[c] < a.n;
      // (rows of d coordinates: the 8-coordinate chunks past d are zero padding)
      const u4* src = reinterpret_cast<const u4*>(X + (live[c] ? vid[c] : 0) * a.row_stride + 32 * kg);
#pragma unroll
      for (int s = 0; s < 4; ++s) xb[c][s] = (live[c] && 32 * kg + 8 * s < a.d) ? src[s] : u4{0u, 0u, 0u, 0u};
    }
    // stores: this lane's BITS words of the code stream, the norm, ||r||, the sign word
    encode_tile<QJL, HAD, BITS, N8, kCols, MIXMOD>(
        fragP, fragS, ctab, emask, cbk, t.ntab, xb,
        [&](int c, const uint32_t* words, const uint32_t* words2, float nst, int) {
          if (!live[c]) return;
          if constexpr (MIXMOD > 0) {
            // record of 16 BITS + 8 bytes: the lane's low-rate piece (2 BITS
            // bytes at 2 BITS kg) and high-rate piece (2 (BITS+1) bytes at
            // 8 BITS + 2 (BITS+1) kg), 16-bit stores
            uint8_t* rec = a.codes + vid[c] * (16 * BITS + 8);
            uint16_t* rl = reinterpret_cast<uint16_t*>(rec + 2 * BITS * kg);
            uint16_t* rh = reinterpret_cast<uint16_t*>(rec + 8 * BITS + 2 * (BITS + 1) * kg);
#pragma unroll
            for (int i = 0; i < BITS; ++i) rl[i] = static_cast<uint16_t>(words[i >> 1] >> (16 * (i & 1)));
#pragma unroll
            for (int i = 0; i < BITS + 1; ++i) rh[i] = static_cast<uint16_t>(words2[i >> 1] >> (16 * (i & 1)));
          } else {
            uint32_t* cw = reinterpret_cast<uint32_t*>(a.codes + vid[c] * (16 * BITS)) + BITS * kg;
#pragma unroll
            for (int w = 0; w < BITS; ++w) cw[w] = words[w];
          }
          if (kg == 0) a.norms[vid[c]] = nst;
        },
        [&](int c, float rn, uint32_t sw) {
          if (!live[c]) return;
          if (kg == 0) a.rnorms[vid[c]] = rn;
          reinterpret_cast<uint32_t*>(a.signs + vid[c] * 16)[kg] = sw;
        });
  }
}

// ---------------------------------------------------------------------------
// Bulk append of one kind (keys or values) of every sequence.  Work item
// (tile) = ((b * H + h) * gmax + gr): the gr-th 32-token value group among
// those whose tokens leave the window in this append, for sequence b and KV
// head h; a wave takes tiles wave, wave + waves in the grid, ...  For each
// sequence: T0 = seq_lens[b], T1 = T0 + count; the tokens at positions
// [max(T0-W, 0), max(T1-W, 0)) are encoded from their FP16 values (the ring
// for positions below T0, else the new rows).  A sequence with an invalid
// count or page id is skipped (left unchanged; the commit kernel reports it).
// MIX: the mixed-channel rate BITS + 1/2 (keys: coordinates j mod 32 >= 16,
// values: j mod 8 >= 4 at BITS + 1 bits); a key record holds the low-rate
// codes then the high-rate ones, a value group a BITS-bit word block for the
// low-rate half then a (BITS+1)-bit block, each indexed by rank.
template <bool KEY, bool QJL, bool HAD, int BITS, bool N8, bool MIX>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu((QJL && !HAD) ? 2 : 4)))
void append_mma_kernel(AppendArgs a, DevTables t, EncCodebook cbk, Layout L, int W, int gmax) {
  __shared__ u4 fragP[HAD ? 1 : 8 * 4 * 2 * 64];  // 64 KB
  __shared__ u4 fragS[QJL ? 8 * 4 * 2 * 64 : 1];  // 64 KB
  __shared__ float ctab[32];
  u4 emask[4];
  setup_tables<QJL, HAD>(fragP, fragS, ctab, t, cbk, emask);

  constexpr int kCols = cols_for(HAD);
  constexpr int kSub = 2 / kCols;  // encode_tile calls per 32-token group
  const int tid = threadIdx.x;
  const int l = tid & 63, n = l & 15, kg = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // (32-bit tile arithmetic: the launcher keeps batch * H * gmax below 2^31)
  const uint32_t ntiles = static_cast<uint32_t>(a.batch) * static_cast<uint32_t>(L.H) * static_cast<uint32_t>(gmax);
  const uint32_t stride = gridDim.x * kEncWaves;
  const uint16_t* win = KEY ? a.k_win : a.v_win;
  const uint16_t* src = KEY ? a.k_new : a.v_new;

  for (uint32_t tile = blockIdx.x * kEncWaves + wave; tile < ntiles; tile += stride) {
    const uint32_t bh32 = tile / static_cast<uint32_t>(gmax);
    const int gr = static_cast<int>(tile - bh32 * static_cast<uint32_t>(gmax));
    const int64_t bh = bh32;
    const int b = static_cast<int>(bh32 / static_cast<uint32_t>(L.H)), h = static_cast<int>(bh32 - b * L.H);
    // ---- the sequence's plan (wave-uniform)
    const int T0 = a.seq_lens[b];
    const int cnt = a.counts ? a.counts[b] : a.n_new;
    if (cnt < 0 || cnt > a.n_new || T0 < 0) continue;
    const int c0 = T0 - W > 0 ? T0 - W : 0;
    const int c1 = T0 + cnt - W > 0 ? T0 + cnt - W : 0;
    const int gpos = (c0 / kVGroup + gr) * kVGroup;
    if (c1 <= c0 || gpos >= c1) continue;
    const int pg0 = c0 / L.P, pg1 = (c1 - 1) / L.P;
    if (pg1 >= a.max_pages) continue;
    // every page the append touches must be valid, or the sequence stays as it is
    bool bad = false;
    for (int pg = pg0 + l; pg <= pg1; pg += 64) {
      const int pid = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg];
      bad = bad || pid < 0 || pid >= a.num_pages;
    }
    if (__ballot(bad)) continue;
    const int lo = c0 > gpos ? c0 : gpos;
    const int hi = c1 < gpos + kVGroup ? c1 : gpos + kVGroup;
    const int pid = a.block_table[static_cast<int64_t>(b) * a.max_pages + gpos / L.P];
    uint8_t* hb = a.pool + static_cast<int64_t>(pid) * L.page_bytes + kBodyOffset + static_cast<int64_t>(h) * L.head_bytes;
    const int slot0 = gpos % L.P;
    // value words of the group: word w of coordinate j at gw[w kD + j] (mixed
    // rate: of rank j in the block at word off, gw[off + 64 w + j]); bits of
    // tokens before lo (earlier appends) are kept, those from hi on are zero
    constexpr int kVStride = MIX ? kD / 2 : kD;
    uint32_t* gw = reinterpret_cast<uint32_t*>(hb + L.v_codes) +
                   static_cast<int64_t>(slot0 / kVGroup) * (MIX ? (2 * BITS + 1) * (kD / 2) : BITS * kD);
    auto put_word = [&](int off, int wd, int w, int j, uint32_t v) {
      const int kb = (lo - gpos) * wd - 32 * w;
      uint32_t* pw = gw + off + w * kVStride + j;
      if (kb > 0) v |= *pw & (kb >= 32 ? 0xffffffffu : ((1u << kb) - 1u));
      *pw = v;
    };
    // the 3-bit block's 24-bit chunks per 16-token block (3-bit values, or
    // the 3-bit half of a mixed rate), joined after the loop
    constexpr int kQ3 = MIX ? 2 : 4;                                // chunks of 8 codes per lane
    constexpr int kOff3 = (MIX && BITS == 2) ? (kD / 2) * BITS : 0;  // word offset of the 3-bit block
    uint32_t ch3[2][4];
    (void)ch3;
#pragma unroll
    for (int sb = 0; sb < kSub; ++sb) {
      // ---- load: lane (n, kg) of block c takes token 16 (kCols sb + c) + n of the group
      u4 xb[kCols][4];
      int tk[kCols];
      bool live[kCols];
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        tk[c] = 16 * (kCols * sb + c) + n;
        const int p = gpos + tk[c];
        live[c] = p >= lo && p < hi;
        // (a dead lane reads row 0 of the new rows, which always exist, and discards it)
        const bool ring = live[c] && p < T0;
        const int64_t row = !live[c] ? 0 : ring ? (bh * W + p % W) : (bh * a.n_new + (p - T0));
        // (rows of d coordinates: the 8-coordinate chunks past d are zero padding)
        const u4* rp = reinterpret_cast<const u4*>((ring ? win : src) + row * L.d + 32 * kg);
#pragma unroll
        for (int s = 0; s < 4; ++s) xb[c][s] = (live[c] && 32 * kg + 8 * s < L.d) ? rp[s] : u4{0u, 0u, 0u, 0u};
      }
      encode_tile<QJL, HAD, BITS, N8, kCols, MIX ? (KEY ? kKeyHiMod : kValHiMod) : 0>(
          fragP, fragS, ctab, emask, cbk, t.ntab, xb,
          [&](int c, const uint32_t* words, const uint32_t* words2, float nst, int nq) {
            const int slot = slot0 + tk[c];
            if constexpr (KEY) {
              if (!live[c]) return;
              if constexpr (MIX) {
                // low-rate piece: 2 BITS bytes at 2 BITS kg; high-rate piece:
                // 2 (BITS+1) bytes at 8 BITS + 2 (BITS+1) kg (16-bit stores)
                uint16_t* rl = reinterpret_cast<uint16_t*>(hb + L.k_codes + static_cast<int64_t>(slot) * L.k_rec +
                                                           2 * BITS * kg);
                uint16_t* rh = reinterpret_cast<uint16_t*>(hb + L.k_codes + static_cast<int64_t>(slot) * L.k_rec +
                                                           8 * BITS + 2 * (BITS + 1) * kg);
#pragma unroll
                for (int i = 0; i < BITS; ++i) rl[i] = static_cast<uint16_t>(words[i >> 1] >> (16 * (i & 1)));
#pragma unroll
                for (int i = 0; i < BITS + 1; ++i) rh[i] = static_cast<uint16_t>(words2[i >> 1] >> (16 * (i & 1)));
              } else {
                uint32_t* cw =
                    reinterpret_cast<uint32_t*>(hb + L.k_codes + static_cast<int64_t>(slot) * L.k_rec) + BITS * kg;
#pragma unroll
                for (int w = 0; w < BITS; ++w) cw[w] = words[w];
              }
              if (kg == 0) {
                if constexpr (N8)
                  (hb + L.k_norm)[slot] = static_cast<uint8_t>(nq);
                else
                  reinterpret_cast<float*>(hb + L.k_norm)[slot] = nst;
              }
            } else {
              if (live[c] && kg == 0) reinterpret_cast<float*>(hb + L.v_norm)[slot] = nst;
              // Token t's code of coordinate j goes to bits [t BITS, (t+1) BITS)
              // of j's string.  The lanes of this 16-token block (tb) hold one
              // token each and 32 coordinates: a transpose of the code fields
              // across lanes gives each lane whole words of the strings (dead
              // tokens carry zero codes).  All lanes take part in the shuffles.
              const int tb = kCols * sb + c;
              // One block of NC codes of width WD per lane (the lane's codes of
              // indices J0 .. J0 + NC - 1 of the block at word OFF):
              //  WD = 4: word q holds indices J0 + 8q .. +7 -> word 2tb + n/8 of
              //          index J0 + 8q + n%8 (tokens 16tb + 8(n/8) .. +7);
              //  WD = 2: word q holds indices J0 + 16q .. +15 -> word tb of index J0 + 16q + n;
              //  WD = 3: 8 codes (24 bits) at a time as nibbles, transposed and
              //          packed back: the 24-bit chunk of tokens 16tb + 8(n/8)
              //          .. +7 of index J0 + 8q + n%8; joined below.
              auto block = [&](auto wd_c, auto nc_c, int off, int j0, const uint32_t* ws) {
                constexpr int WD = decltype(wd_c)::value, NC = decltype(nc_c)::value;
                if constexpr (WD == 4) {
#pragma unroll
                  for (int q = 0; q < NC / 8; ++q)
                    put_word(off, 4, 2 * tb + (n >> 3), j0 + 8 * q + (n & 7), transpose_nibbles8(ws[q], l));
                } else if constexpr (WD == 2) {
#pragma unroll
                  for (int q = 0; q < NC / 16; ++q) put_word(off, 2, tb, j0 + 16 * q + n, transpose_crumbs16(ws[q], l));
                } else {
#pragma unroll
                  for (int q = 0; q < NC / 8; ++q) {
                    const int b0 = 24 * q, wi = b0 >> 5, sh = b0 & 31;
                    uint32_t v = ws[wi] >> sh;
                    if (sh > 8) v |= ws[wi + 1] << (32 - sh);
                    ch3[tb][q] = pack4to3(transpose_nibbles8(spread3to4(v & 0xFFFFFFu), l));
                  }
                }
              };
              if constexpr (MIX) {
                // ranks 16kg .. 16kg+15 of each half
                block(std::integral_constant<int, BITS>{}, std::integral_constant<int, 16>{}, 0, 16 * kg, words);
                block(std::integral_constant<int, BITS + 1>{}, std::integral_constant<int, 16>{}, (kD / 2) * BITS,
                      16 * kg, words2);
              } else {
                block(std::integral_constant<int, BITS>{}, std::integral_constant<int, 32>{}, 0, 32 * kg, words);
              }
            }
          },
          [&](int c, float rn, uint32_t sw) {
            if (!live[c]) return;
            const int slot = slot0 + tk[c];
            if (kg == 0) reinterpret_cast<float*>(hb + L.k_rnorm)[slot] = rn;
            reinterpret_cast<uint32_t*>(hb + L.k_signs + static_cast<int64_t>(slot) * (kD / 8))[kg] = sw;
          });
    }
    if constexpr (!KEY && (BITS == 3 || MIX)) {
      // index j's 96-bit string is chunks 0..3 (tokens 8w .. 8w+7) at bits
      // 24w: lane n < 8 holds chunks 0 and 2, lane n + 8 chunks 1 and 3; each
      // takes the other two from its partner and writes words 0, 1 (n < 8)
      // or word 2
      const bool hi8 = (n & 8) != 0;
#pragma unroll
      for (int q = 0; q < kQ3; ++q) {
        const uint32_t o0 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(ch3[0][q]), 8, 64));
        const uint32_t o1 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(ch3[1][q]), 8, 64));
        const uint32_t c0 = hi8 ? o0 : ch3[0][q], c1 = hi8 ? ch3[0][q] : o0;
        const uint32_t c2 = hi8 ? o1 : ch3[1][q], c3 = hi8 ? ch3[1][q] : o1;
        const int j = (MIX ? 16 : 32) * kg + 8 * q + (n & 7);
        if (!hi8) {
          put_word(kOff3, 3, 0, j, c0 | (c1 << 24));
          put_word(kOff3, 3, 1, j, (c1 >> 8) | (c2 << 16));
        } else {
          put_word(kOff3, 3, 2, j, (c2 >> 16) | (c3 << 8));
        }
      }
    }
  }
}

template <bool QJL, bool HAD, bool N8>
const void* pick_bits(int bits, int mixmod) {
  if (mixmod == kKeyHiMod) {  // mixed rates exist at 2.5 and 3.5 bits
    if (bits == 2) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 2, N8, kKeyHiMod>);
    if (bits == 3) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 3, N8, kKeyHiMod>);
    return nullptr;
  }
  if (mixmod == kValHiMod) {
    if (bits == 2) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 2, N8, kValHiMod>);
    if (bits == 3) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 3, N8, kValHiMod>);
    return nullptr;
  }
  if (bits == 2) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 2, N8, 0>);
  if (bits == 3) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 3, N8, 0>);
  return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 4, N8, 0>);
}

template <bool KEY, bool QJL, bool HAD, bool N8>
const void* pick_append_bits(int bits, bool mix) {
  if (mix) {  // mixed rates exist at 2.5 and 3.5 bits
    if (bits == 2) return reinterpret_cast<const void*>(&append_mma_kernel<KEY, QJL, HAD, 2, N8, true>);
    if (bits == 3) return reinterpret_cast<const void*>(&append_mma_kernel<KEY, QJL, HAD, 3, N8, true>);
    return nullptr;
  }
  if (bits == 2) return reinterpret_cast<const void*>(&append_mma_kernel<KEY, QJL, HAD, 2, N8, false>);
  if (bits == 3) return reinterpret_cast<const void*>(&append_mma_kernel<KEY, QJL, HAD, 3, N8, false>);
  return reinterpret_cast<const void*>(&append_mma_kernel<KEY, QJL, HAD, 4, N8, false>);
}

template <bool QJL, bool HAD>
const void* pick_append_key(int bits, bool n8, bool mix) {
  return n8 ? pick_append_bits<true, QJL, HAD, true>(bits, mix) : pick_append_bits<true, QJL, HAD, false>(bits, mix);
}

// This kind's codebook(s), if the matrix-core path takes them: symmetric
// codebooks (the binary-search quantiser relies on it); a mixed-channel rate
// only where allowed (the bulk append), with its (b+1)-bit codebook too.
bool mma_codebook(const tq_ctx* c, bool key, EncCodebook& cbk, bool allow_mixed) {
  const bool mix = key ? c->p.key_mixed : c->p.value_mixed;
  if (c->lay.D != kD || (mix && !allow_mixed)) return false;
  const int bits = key ? c->p.key_bits : c->p.value_bits;
  for (int k = 0; k < 16; ++k) {
    cbk.cen[k] = key ? c->cb.kc[k] : c->cb.vc[k];
    cbk.bnd[k] = key ? c->cb.kb[k] : c->cb.vb[k];
    cbk.cen2[k] = key ? c->cb.kc2[k] : c->cb.vc2[k];
    cbk.bnd2[k] = key ? c->cb.kb2[k] : c->cb.vb2[k];
  }
  auto symmetric = [](const float* bnd, int levels) {
    if (bnd[levels / 2 - 1] != 0.0f) return false;
    for (int k = 0; k + 1 < levels; ++k)
      if (bnd[k] != -bnd[levels - 2 - k]) return false;
    return true;
  };
  if (!symmetric(cbk.bnd, 1 << bits)) return false;
  if (mix && (bits + 1 > 4 || !symmetric(cbk.bnd2, 1 << (bits + 1)))) return false;
  return true;
}

// Work-groups for a persistent grid over `items` wave-sized items.
int persistent_blocks(const void* f, int64_t items, int64_t* blocks) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kEncThreads, 0) != hipSuccess)
    return -1;
  int64_t bl = (items + kEncWaves - 1) / kEncWaves;
  const int64_t cap = static_cast<int64_t>(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  if (bl > cap) bl = cap;
  *blocks = bl < 1 ? 1 : bl;
  return 0;
}

}  // namespace

// Returns 1 when this path does not apply (input not fp16 or not 16-byte
// rows, or a codebook the binary-search quantiser cannot take); the caller
// then uses the vector-ALU encoder.
int launch_encode_mma(const tq_ctx* c, int kind, int dtype, const EncodeArgs& a, void* stream) {
  if (dtype != TQ_DTYPE_F16 || (a.row_stride % 8) != 0 || (reinterpret_cast<uintptr_t>(a.x) % 16) != 0) return 1;
  const bool key = kind == TQ_KIND_KEY;
  EncCodebook cbk;
  if (!mma_codebook(c, key, cbk, true)) return 1;
  const bool qjl = key && c->p.key_qjl;
  const bool had = c->p.rotation == TQ_ROT_HADAMARD;
  const bool n8 = key && c->p.key_norm_u8;
  const int bits = key ? c->p.key_bits : c->p.value_bits;
  const int mm = (key ? c->p.key_mixed : c->p.value_mixed) ? (key ? kKeyHiMod : kValHiMod) : 0;
  const void* f;
  if (n8)
    f = qjl ? (had ? pick_bits<true, true, true>(bits, mm) : pick_bits<true, false, true>(bits, mm))
            : (had ? pick_bits<false, true, true>(bits, mm) : pick_bits<false, false, true>(bits, mm));
  else
    f = qjl ? (had ? pick_bits<true, true, false>(bits, mm) : pick_bits<true, false, false>(bits, mm))
            : (had ? pick_bits<false, true, false>(bits, mm) : pick_bits<false, false, false>(bits, mm));
  if (!f) return 1;
  const int tv = 16 * cols_for(had);
  int64_t blocks = 0;
  if (persistent_blocks(f, (a.n + tv - 1) / tv, &blocks) != 0) return -1;
  EncodeArgs aa = a;
  DevTables tt = c->t;
  void* args[] = {&aa, &tt, &cbk};
  return hipLaunchKernel(f, dim3(static_cast<unsigned>(blocks)), dim3(kEncThreads), args, 0,
                         static_cast<hipStream_t>(stream)) == hipSuccess
             ? 0
             : -1;
}

// Bulk append of one kind on the matrix cores.  Returns 1 when this path does
// not apply (a codebook the binary-search quantiser cannot take); -1 on a
// launch error.
int launch_append_mma(const tq_ctx* c, int kind, const AppendArgs& a, void* stream) {
  const bool key = kind == TQ_KIND_KEY;
  EncCodebook cbk;
  if (!mma_codebook(c, key, cbk, true)) return 1;
  const bool had = c->p.rotation == TQ_ROT_HADAMARD;
  const bool n8 = key && c->p.key_norm_u8;
  const bool qjl = key && c->p.key_qjl;
  const bool mix = key ? c->p.key_mixed : c->p.value_mixed;
  const int bits = key ? c->p.key_bits : c->p.value_bits;
  const void* f;
  if (key)
    f = qjl ? (had ? pick_append_key<true, true>(bits, n8, mix) : pick_append_key<true, false>(bits, n8, mix))
            : (had ? pick_append_key<false, true>(bits, n8, mix) : pick_append_key<false, false>(bits, n8, mix));
  else
    f = had ? pick_append_bits<false, false, true, false>(bits, mix)
            : pick_append_bits<false, false, false, false>(bits, mix);
  if (!f) return 1;
  // value groups a sequence can touch: ceil(n_new / 32) + 1 (unaligned start)
  const int gmax = (a.n_new + kVGroup - 1) / kVGroup + 1;
  if (static_cast<int64_t>(a.batch) * c->lay.H * gmax >= (int64_t(1) << 31)) return 1;
  int64_t blocks = 0;
  if (persistent_blocks(f, static_cast<int64_t>(a.batch) * c->lay.H * gmax, &blocks) != 0) return -1;
  AppendArgs aa = a;
  DevTables tt = c->t;
  Layout L = c->lay;
  int W = c->p.window, gm = gmax;
  void* args[] = {&aa, &tt, &cbk, &L, &W, &gm};
  return hipLaunchKernel(f, dim3(static_cast<unsigned>(blocks)), dim3(kEncThreads), args, 0,
                         static_cast<hipStream_t>(stream)) == hipSuccess
             ? 0
             : -1;
}

}  // namespace tq
