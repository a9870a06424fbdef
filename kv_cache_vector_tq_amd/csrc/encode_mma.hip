// Bulk encode of fp16 vectors on the matrix cores (tq_encode, gfx950).
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
};

// Code of y for a symmetric codebook of 2^B levels (boundaries b_j = -b_{L-2-j},
// middle boundary 0): the number of boundaries strictly below y.  With
// m = |y| and the positive boundaries p_1 < .. < p_P (P = L/2 - 1): y > 0
// gives L/2 + #{p_k < m}; y <= 0 gives L/2 - 1 - #{p_k <= m}.  Both counts
// are #{p_k < m'} with m' = m or its float successor, found by binary search.
template <int B>
__device__ inline uint32_t quantize_sym(float y, const EncCodebook& cbk) {
  constexpr int H = 1 << (B - 1);  // L/2
  const float* p = cbk.bnd + (H - 1);  // p[k] = k-th positive boundary, p[0] = 0
  const bool pos = y > 0.0f;
  const uint32_t mb = __builtin_bit_cast(uint32_t, y) & 0x7fffffffu;
  const float m = __builtin_bit_cast(float, pos ? mb : mb + 1u);
  uint32_t cnt;
  if constexpr (B == 2) {
    cnt = m > p[1] ? 1u : 0u;
  } else {
    static_assert(B == 3, "binary search written for 2 and 3 bits");
    const bool g2 = m > p[2];
    const bool g1 = m > (g2 ? p[3] : p[1]);
    cnt = (g2 ? 2u : 0u) + (g1 ? 1u : 0u);
  }
  return pos ? H + cnt : H - 1 - cnt;
}

// 32-lane-group sum of a double over the four lanes holding one vector
__device__ inline double sum4(double v) {
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// Two work-groups per CU need <= 128 VGPRs; the dense key variant holds both
// matrices (128 KB of LDS) and fits only one anyway.
template <bool QJL, bool HAD, int BITS>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu((QJL && !HAD) ? 2 : 4)))
void encode_mma_kernel(EncodeArgs a, DevTables t, EncCodebook cbk) {
  __shared__ u4 fragP[HAD ? 1 : 8 * 4 * 2 * 64];  // 64 KB
  __shared__ u4 fragS[QJL ? 8 * 4 * 2 * 64 : 1];  // 64 KB
  __shared__ float ctab[16];
  const int tid = threadIdx.x;
  if (!HAD) build_frags(fragP, t.rot, 16.0f, tid);
  if (QJL) build_frags(fragS, t.S, 1.0f, tid);
  if (tid < 16) {
    float cv = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      if (k == tid) cv = cbk.cen[k];
    ctab[tid] = cv;
  }
  __syncthreads();

  constexpr int kCols = cols_for(HAD), kTileVec = 16 * kCols;
  const int l = tid & 63, n = l & 15, kg = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  float eps[32];  // Hadamard signs of this lane's coordinates
  if constexpr (HAD) {
#pragma unroll
    for (int j = 0; j < 32; ++j) eps[j] = t.rot[32 * kg + j];
  }
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
      const u4* src = reinterpret_cast<const u4*>(X + (live[c] ? vid[c] : 0) * a.row_stride + 32 * kg);
#pragma unroll
      for (int s = 0; s < 4; ++s) xb[c][s] = live[c] ? src[s] : u4{0u, 0u, 0u, 0u};
    }
    // ---- norms (double accumulation, as the vector-ALU path)
    float n32[kCols], invn[kCols];
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
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
    }
    // ---- y (unnormalised, fp32): lane holds coordinate 32kg + 4tt + r in acc[c][tt][r]
    f4 acc[kCols][8];
    if constexpr (!HAD) {
#pragma unroll
      for (int c = 0; c < kCols; ++c)
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
          for (int c = 0; c < kCols; ++c) {
            acc[c][tt] = mfma(cur[2 * s], xb[c][s], acc[c][tt]);
            acc[c][tt] = mfma(cur[2 * s + 1], xb[c][s], acc[c][tt]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int c = 0; c < kCols; ++c)
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) acc[c][tt] *= 0.0625f;
    } else {
      // y = H (eps . x) / sqrt(d), natural (Sylvester) order
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const uint32_t w = xb[c][j >> 3][(j >> 1) & 3];
          v[j] = hval((j & 1) ? (w >> 16) : (w & 0xffffu)) * eps[j];
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
            const float o = __shfl_xor(v[j], h, 64);
            v[j] = (l & h) ? (o - v[j]) : (v[j] + o);
          }
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[c][j >> 2][j & 3] = v[j] * 0.08838834764831845f;
      }
    }
    // ---- quantise, pack, residual
    uint32_t words[kCols][BITS];
    u4 rb[kCols][4][2];  // B operands of the residual product (hi / lo)
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
#pragma unroll
      for (int w = 0; w < BITS; ++w) words[c][w] = 0u;
      float rv[32];
      float rs = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float accv = acc[c][j >> 2][j & 3];
        const float y = accv * invn[c];
        uint32_t code = 0;
        if constexpr (BITS == 3 && !QJL) {
          code = quantize_sym<BITS>(y, cbk);
        } else {
          // a linear count measured faster for 2 and 4 bits and for keys
#pragma unroll
          for (int k = 0; k < (1 << BITS) - 1; ++k) code += (y > cbk.bnd[k]) ? 1u : 0u;
        }
        if (!(n32[c] > 0.0f)) code = 0;
        const int pos = j * BITS;
        words[c][pos >> 5] |= code << (pos & 31);
        if ((pos & 31) + BITS > 32) words[c][(pos >> 5) + 1] |= code >> (32 - (pos & 31));
        if constexpr (QJL) {
          const float r = (n32[c] > 0.0f) ? fmaf(-n32[c], ctab[code], accv) : 0.0f;
          rs = fmaf(r, r, rs);
          rv[j] = r * (64.0f * invn[c]);
        }
      }
      // stores: this lane's BITS words of the code stream, and the norm
      if (live[c]) {
        uint32_t* cw = reinterpret_cast<uint32_t*>(a.codes + vid[c] * (16 * BITS)) + BITS * kg;
#pragma unroll
        for (int w = 0; w < BITS; ++w) cw[w] = words[c][w];
        if (kg == 0) a.norms[vid[c]] = n32[c];
      }
      if constexpr (QJL) {
        rs += __shfl_xor(rs, 16, 64);
        rs += __shfl_xor(rs, 32, 64);
        if (live[c] && kg == 0) a.rnorms[vid[c]] = sqrtf(rs);
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
      uint32_t sw[kCols] = {};
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        f4 z[kCols];
#pragma unroll
        for (int c = 0; c < kCols; ++c) z[c] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const u4 sh = fragS[((tt * 4 + s) * 2 + 0) * 64 + l];
          const u4 sl = fragS[((tt * 4 + s) * 2 + 1) * 64 + l];
#pragma unroll
          for (int c = 0; c < kCols; ++c) {
            z[c] = mfma(sh, rb[c][s][0], z[c]);
            z[c] = mfma(sh, rb[c][s][1], z[c]);
            z[c] = mfma(sl, rb[c][s][0], z[c]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int c = 0; c < kCols; ++c)
#pragma unroll
          for (int r = 0; r < 4; ++r) sw[c] |= (z[c][r] >= 0.0f ? 1u : 0u) << (4 * tt + r);
      }
#pragma unroll
      for (int c = 0; c < kCols; ++c)
        if (live[c]) reinterpret_cast<uint32_t*>(a.signs + vid[c] * 16)[kg] = (n32[c] > 0.0f) ? sw[c] : 0u;
    }
  }
}

template <bool QJL, bool HAD>
const void* pick_bits(int bits) {
  if (bits == 2) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 2>);
  if (bits == 3) return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 3>);
  return reinterpret_cast<const void*>(&encode_mma_kernel<QJL, HAD, 4>);
}

}  // namespace

// Returns 1 when this path does not apply (input not fp16 or not 16-byte
// rows); the caller then uses the vector-ALU encoder.
int launch_encode_mma(const tq_ctx* c, int kind, int dtype, const EncodeArgs& a, void* stream) {
  if (dtype != TQ_DTYPE_F16 || c->p.head_dim != kD || (a.row_stride % 8) != 0 ||
      (reinterpret_cast<uintptr_t>(a.x) % 16) != 0)
    return 1;
  const bool key = kind == TQ_KIND_KEY;
  // mixed-channel rates take the vector-ALU encoder
  if (key ? c->p.key_mixed : c->p.value_mixed) return 1;
  // so do keys with u8 log-norms
  if (key && c->p.key_norm_u8) return 1;
  const bool qjl = key && c->p.key_qjl;
  const bool had = c->p.rotation == TQ_ROT_HADAMARD;
  const int bits = key ? c->p.key_bits : c->p.value_bits;
  const void* f = qjl ? (had ? pick_bits<true, true>(bits) : pick_bits<true, false>(bits))
                      : (had ? pick_bits<false, true>(bits) : pick_bits<false, false>(bits));
  EncCodebook cbk;
  for (int k = 0; k < 16; ++k) {
    cbk.cen[k] = key ? c->cb.kc[k] : c->cb.vc[k];
    cbk.bnd[k] = key ? c->cb.kb[k] : c->cb.vb[k];
  }
  // the quantiser relies on a symmetric codebook with a boundary at 0
  const int L = 1 << bits;
  if (cbk.bnd[L / 2 - 1] != 0.0f) return 1;
  for (int k = 0; k + 1 < L; ++k)
    if (cbk.bnd[k] != -cbk.bnd[L - 2 - k]) return 1;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kEncThreads, 0) != hipSuccess)
    return -1;
  const int tv = 16 * cols_for(had);
  const int64_t ntiles = (a.n + tv - 1) / tv;
  int64_t blocks = (ntiles + kEncWaves - 1) / kEncWaves;
  const int64_t cap = static_cast<int64_t>(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
  if (blocks > cap) blocks = cap;
  EncodeArgs aa = a;
  DevTables tt = c->t;
  void* args[] = {&aa, &tt, &cbk};
  return hipLaunchKernel(f, dim3(static_cast<unsigned>(blocks)), dim3(kEncThreads), args, 0,
                         static_cast<hipStream_t>(stream)) == hipSuccess
             ? 0
             : -1;
}

}  // namespace tq
