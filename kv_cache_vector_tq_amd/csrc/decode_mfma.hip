// Compressed-page scan on the matrix cores (MFMA 16x16x32 f16, gfx950).
//
// Same arithmetic as the VALU scan in decode.hip ("TurboQuant Family Design
// Study", section "CPU and WASM kernel design": transform the query once,
// score packed keys through small per-dimension tables, accumulate values in
// the rotated basis): for the G query heads of one KV head,
//   score_t = n_t <q_rot, c_K[idx_t]> + ||r_t|| <p, 2 sigma_t - 1>
//   acc    += sum_t w_t n^V_t c_V[idx^V_t]
// With G queries sharing every decoded key and value, both sums are small
// matrix products (G x 128 by 128 x tokens, and G x tokens by tokens x 128).
// They run as MFMAs with fp16 operands and fp32 accumulation:
//  * the query side (q_rot, p, and the softmax weights times value norms)
//    is split into fp16 hi + lo parts placed in rows g and g + G of the A
//    operand, so it keeps ~22 bits; rows hi and lo are summed afterwards;
//  * the cache side is exact in fp16 for the sign bits (+-1) and rounded to
//    fp16 (relative error <= 2^-11) for the centroid values;
//  * packed codes are expanded to fp16 B operands through LDS lookup tables
//    (a 6- or 8-bit slice of the code stream yields 2 or 4 fp16 values).
// Each wave streams 32-token chunks (one value group) with its own online
// softmax state; the four waves of a work-group merge at the end.
#include "decode_common.h"
#include "device_common.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 32;
constexpr int kWaves = kScanThreads / 64;

__device__ inline uint32_t h_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

// fp16 hi part and fp16 remainder of x
__device__ inline void split_hl(float x, uint32_t& hi, uint32_t& lo) {
  const _Float16 h = static_cast<_Float16>(x);
  hi = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
  lo = h_bits(x - static_cast<float>(h));
}

__device__ inline f4 mfma(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

__device__ inline void wave_sync() { __builtin_amdgcn_wave_barrier(); }

// Lookup-table entries per bit width: a slice of the code stream -> fp16 values.
//   B=2: 8-bit slice (4 codes) -> 4 fp16 (two words per entry, 256 entries)
//   B=3: 6-bit slice (2 codes) -> 2 fp16 (one word, 64 entries)
//   B=4: 8-bit slice (2 codes) -> 2 fp16 (one word, 256 entries)
template <int B>
struct Lut {
  static constexpr int kEntries = B == 3 ? 64 : 256;
  static constexpr int kWords = B == 2 ? 2 : 1;
  static constexpr int kSlice = B == 3 ? 6 : 8;
};

template <int B>
__device__ void build_lut(uint32_t* lut, const float* cen, int tid) {
  for (int e = tid; e < Lut<B>::kEntries; e += kScanThreads) {
    if constexpr (B == 2) {
      lut[2 * e] = h_bits(cen[e & 3]) | (h_bits(cen[(e >> 2) & 3]) << 16);
      lut[2 * e + 1] = h_bits(cen[(e >> 4) & 3]) | (h_bits(cen[(e >> 6) & 3]) << 16);
    } else if constexpr (B == 3) {
      lut[e] = h_bits(cen[e & 7]) | (h_bits(cen[(e >> 3) & 7]) << 16);
    } else {
      lut[e] = h_bits(cen[e & 15]) | (h_bits(cen[(e >> 4) & 15]) << 16);
    }
  }
}

// 8 consecutive codes (8*B bits, LSB-first in x) -> 8 fp16 values.
template <int B>
__device__ inline u4 dec8(uint32_t x, const uint32_t* lut) {
  u4 r;
  if constexpr (B == 2) {
    const uint2 a = reinterpret_cast<const uint2*>(lut)[x & 255u];
    const uint2 b = reinterpret_cast<const uint2*>(lut)[(x >> 8) & 255u];
    r.x = a.x; r.y = a.y; r.z = b.x; r.w = b.y;
  } else if constexpr (B == 3) {
    r.x = lut[x & 63u]; r.y = lut[(x >> 6) & 63u]; r.z = lut[(x >> 12) & 63u]; r.w = lut[(x >> 18) & 63u];
  } else {
    r.x = lut[x & 255u]; r.y = lut[(x >> 8) & 255u]; r.z = lut[(x >> 16) & 255u]; r.w = lut[x >> 24];
  }
  return r;
}

// Codes 8i .. 8i+7 of a lane's 32-code key slice held in B words.
template <int B>
__device__ inline uint32_t key_slice(const uint32_t* w, int i) {
  if constexpr (B == 4) return w[i];
  else if constexpr (B == 2) return (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
  else return bits_at<24>(w, 24 * i);
}

template <int BK, int BV, bool QJL>
struct Chunk {
  uint32_t kc[2][BK];   // key codes: tile t, lane's 32-coordinate slice
  uint32_t sg[2];       // sign bits of that slice
  float kn[2], rn[2];   // key norms / residual norms of tokens n, 16+n
  float vn;             // value norm of token (lane & 31)
  uint32_t vw[8];       // value words for coordinates 8n..8n+7 (tokens 8kg..)
  uint32_t vw2[8];      // second word when a 3-bit slice straddles words
  int ntok;             // live tokens in the chunk (0 when the page is invalid)
  int64_t pos0;         // position of the chunk's first token
};

template <int G, int BK, int BV, bool QJL>
__global__ __launch_bounds__(kScanThreads) void scan_mfma_kernel(DecodeArgs a, DevTables t, Codebooks cb,
                                                                 KParams k) {
  __shared__ uint32_t lutK[Lut<BK>::kEntries * Lut<BK>::kWords];
  __shared__ uint32_t lutV[Lut<BV>::kEntries * Lut<BV>::kWords];
  __shared__ u4 lutS[QJL ? 256 : 1];
  __shared__ float sc[kWaves][G][kChunk];  // scores, then weights * value norm
  __shared__ float crr[kWaves][G];         // per-chunk rescale factors
  __shared__ float wm[kWaves][G], wl[kWaves][G];
  __shared__ float red[16][kD];

  const int tid = threadIdx.x, split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = tid >> 6, l = tid & 63, n = l & 15, kg = l >> 4;
  const int T = a.seq_lens[b];
  const int C = T - k.W > 0 ? T - k.W : 0;
  const int npages = (C + k.P - 1) / k.P;
  const int pb = split * a.pages_per_split;
  int pe = npages < pb + a.pages_per_split ? npages : pb + a.pages_per_split;
  const int64_t pidx = ((static_cast<int64_t>(b) * k.Hkv + h) * a.splits + split) * G;
  if (pe > a.max_pages) {
    if (tid == 0) atomicOr(t.status, TQ_STATUS_BAD_PAGE);
    pe = a.max_pages;
  }
  if (pb >= pe) {
    if (tid < G) {
      a.pm[pidx + tid] = -INFINITY;
      a.pl[pidx + tid] = 0.0f;
    }
    for (int i = tid; i < G * kD; i += kScanThreads) a.pacc[pidx * kD + i] = 0.0f;
    return;
  }
  // lookup tables (codebooks first copied to LDS: no dynamic indexing of kernel arguments)
  __shared__ float ck[16], cvv[16];
  if (tid < 16) {
    float kv = 0.0f, vv = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i == tid) {
        kv = cb.kc[i];
        vv = cb.vc[i];
      }
    ck[tid] = kv;
    cvv[tid] = vv;
  }
  __syncthreads();
  build_lut<BK>(lutK, ck, tid);
  build_lut<BV>(lutV, cvv, tid);
  if constexpr (QJL) {
    // byte of sign bits -> 8 fp16 values +-1 (bit set = +1)
    const int e = tid;
    u4 v;
    v.x = (e & 1 ? 0x3C00u : 0xBC00u) | ((e & 2 ? 0x3C00u : 0xBC00u) << 16);
    v.y = (e & 4 ? 0x3C00u : 0xBC00u) | ((e & 8 ? 0x3C00u : 0xBC00u) << 16);
    v.z = (e & 16 ? 0x3C00u : 0xBC00u) | ((e & 32 ? 0x3C00u : 0xBC00u) << 16);
    v.w = (e & 64 ? 0x3C00u : 0xBC00u) | ((e & 128 ? 0x3C00u : 0xBC00u) << 16);
    lutS[e] = v;
  }
  // A operands of the key products: row m = n holds query m (hi) or m-G (lo);
  // lane group kg covers coordinates 32kg .. 32kg+31, MFMA i the 8 at 32kg+8i.
  const int64_t qrow = (static_cast<int64_t>(b) * k.Hq + static_cast<int64_t>(h) * G) * kD;
  u4 aq[4], ap[4];
  {
    const int m = n;
    const int g = m < G ? m : m - G;
    const bool live = m < 2 * G;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t wq[4] = {0, 0, 0, 0}, wp[4] = {0, 0, 0, 0};
      if (live) {
        const float4* q4 = reinterpret_cast<const float4*>(a.qs + qrow + g * kD + 32 * kg + 8 * i);
        const float4* p4 = reinterpret_cast<const float4*>(a.ps + qrow + g * kD + 32 * kg + 8 * i);
        float qv[8], pv[8];
        const float4 q0 = q4[0], q1 = q4[1];
        qv[0] = q0.x; qv[1] = q0.y; qv[2] = q0.z; qv[3] = q0.w; qv[4] = q1.x; qv[5] = q1.y; qv[6] = q1.z; qv[7] = q1.w;
        if constexpr (QJL) {
          const float4 p0 = p4[0], p1 = p4[1];
          pv[0] = p0.x; pv[1] = p0.y; pv[2] = p0.z; pv[3] = p0.w; pv[4] = p1.x; pv[5] = p1.y; pv[6] = p1.z; pv[7] = p1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          uint32_t h0, l0, h1, l1;
          split_hl(qv[e], h0, l0);
          split_hl(qv[e + 1], h1, l1);
          wq[e / 2] = m < G ? (h0 | (h1 << 16)) : (l0 | (l1 << 16));
          if constexpr (QJL) {
            split_hl(pv[e], h0, l0);
            split_hl(pv[e + 1], h1, l1);
            wp[e / 2] = m < G ? (h0 | (h1 << 16)) : (l0 | (l1 << 16));
          }
        }
      }
      aq[i] = u4{wq[0], wq[1], wq[2], wq[3]};
      ap[i] = u4{wp[0], wp[1], wp[2], wp[3]};
    }
  }
  __syncthreads();

  // per-wave online-softmax state; lane handles token (l & 31) of queries
  // g = (l >> 5) + 2j (all G for G = 1 is lane < 32 only)
  constexpr int GH = G >= 2 ? G / 2 : 1;  // queries per lane in the softmax phase
  float mrun[GH], lrun[GH];
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    mrun[j] = -INFINITY;
    lrun[j] = 0.0f;
  }
  f4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const int64_t tot = static_cast<int64_t>(C < pe * k.P ? C : pe * k.P) - static_cast<int64_t>(pb) * k.P;
  const int nchunks = static_cast<int>((tot + kChunk - 1) / kChunk);
  const int gpp = k.P / kChunk;  // chunks per page
  const int t32 = l & 31;
  // value words: lane's 8 tokens of coordinate 8n + blk are bits [8*kg*BV, +8*BV)
  const int vbit = 8 * kg * BV;
  const int vw0 = vbit >> 5, vsh = vbit & 31;
  const bool vtwo = (vsh + 8 * BV) > 32;

  auto load = [&](int c, Chunk<BK, BV, QJL>& d) {
    const int64_t tok0 = static_cast<int64_t>(c) * kChunk;
    const int pg = pb + static_cast<int>(tok0 / k.P);
    const int gi = static_cast<int>((tok0 % k.P) / kChunk);
    const int64_t rem = tot - tok0;
    d.ntok = rem < kChunk ? static_cast<int>(rem) : kChunk;
    d.pos0 = static_cast<int64_t>(pg) * k.P + gi * kChunk;
    const int pid = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg];
    if (pid < 0 || pid >= a.num_pages) {
      if (l == 0) atomicOr(t.status, TQ_STATUS_BAD_PAGE);
      d.ntok = 0;
      return;
    }
    const uint8_t* hb = a.pool + static_cast<int64_t>(pid) * k.page_bytes + kBodyOffset + h * k.head_bytes;
    const int s0 = gi * kChunk;
    const float* kn = reinterpret_cast<const float*>(hb + k.k_norm);
    const float* rn = reinterpret_cast<const float*>(hb + k.k_rnorm);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int slot = s0 + 16 * tt + n;
      d.kn[tt] = kn[slot];
      if constexpr (QJL) d.rn[tt] = rn[slot];
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(hb + k.k_codes + static_cast<int64_t>(slot) * 16 * BK) + kg * BK;
      if constexpr (BK == 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(kw);
        d.kc[tt][0] = v.x; d.kc[tt][1] = v.y; d.kc[tt][2] = v.z; d.kc[tt][3] = v.w;
      } else if constexpr (BK == 2) {
        const uint2 v = *reinterpret_cast<const uint2*>(kw);
        d.kc[tt][0] = v.x; d.kc[tt][1] = v.y;
      } else {
#pragma unroll
        for (int w = 0; w < BK; ++w) d.kc[tt][w] = kw[w];
      }
      if constexpr (QJL) d.sg[tt] = reinterpret_cast<const uint32_t*>(hb + k.k_signs)[slot * 4 + kg];
    }
    d.vn = reinterpret_cast<const float*>(hb + k.v_norm)[s0 + t32];
    const uint32_t* vwp = reinterpret_cast<const uint32_t*>(hb + k.v_codes) + static_cast<int64_t>(gi) * BV * kD;
    const uint4* r0 = reinterpret_cast<const uint4*>(vwp + vw0 * kD + 8 * n);
    const uint4 x0 = r0[0], x1 = r0[1];
    d.vw[0] = x0.x; d.vw[1] = x0.y; d.vw[2] = x0.z; d.vw[3] = x0.w;
    d.vw[4] = x1.x; d.vw[5] = x1.y; d.vw[6] = x1.z; d.vw[7] = x1.w;
    if constexpr (BV == 3) {
      const int w1 = vtwo ? vw0 + 1 : vw0;
      const uint4* r1 = reinterpret_cast<const uint4*>(vwp + w1 * kD + 8 * n);
      const uint4 y0 = r1[0], y1 = r1[1];
      d.vw2[0] = y0.x; d.vw2[1] = y0.y; d.vw2[2] = y0.z; d.vw2[3] = y0.w;
      d.vw2[4] = y1.x; d.vw2[5] = y1.y; d.vw2[6] = y1.z; d.vw2[7] = y1.w;
    }
  };

  float* scw = &sc[wave][0][0];
  auto process = [&](const Chunk<BK, BV, QJL>& d) {
    if (d.ntok == 0) return;
    // ---- key scores: two 16-token tiles
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f4 dm = f4{0.0f, 0.0f, 0.0f, 0.0f}, dq = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dm = mfma(aq[i], dec8<BK>(key_slice<BK>(d.kc[tt], i), lutK), dm);
        if constexpr (QJL) dq = mfma(ap[i], lutS[(d.sg[tt] >> (8 * i)) & 255u], dq);
      }
      // rows g (hi) and g + G (lo) -> query g
      float s[4];
      if constexpr (G >= 4) {
        constexpr int off = 16 * (G / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float em = __shfl_down(dm[r], off, 64);
          float v = (dm[r] + em) * d.kn[tt];
          if constexpr (QJL) v = fmaf(dq[r] + __shfl_down(dq[r], off, 64), d.rn[tt], v);
          s[r] = v;
        }
      } else {
#pragma unroll
        for (int r = 0; r < G; ++r) {
          float v = (dm[r] + dm[r + G]) * d.kn[tt];
          if constexpr (QJL) v = fmaf(dq[r] + dq[r + G], d.rn[tt], v);
          s[r] = v;
        }
      }
      const int tok = 16 * tt + n;
      const bool live = tok < d.ntok;
      constexpr int lanes_g = G >= 4 ? G / 4 : 1;  // lane groups holding results
      if (kg < lanes_g) {
#pragma unroll
        for (int r = 0; r < (G >= 4 ? 4 : G); ++r) {
          const int g = (G >= 4 ? 4 * kg : 0) + r;
          const float v = live ? s[r] : -INFINITY;
          scw[g * kChunk + tok] = v;
          if (a.dbg_logits && live)
            a.dbg_logits[(static_cast<int64_t>(b) * k.Hq + h * G + g) * a.logits_stride + d.pos0 + tok] = v * kLn2;
        }
      }
    }
    wave_sync();
    // ---- online softmax over the chunk
    float crow[GH];
    bool any = false;
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      const int g = G >= 2 ? (l >> 5) + 2 * j : 0;
      const bool mine = G >= 2 || l < 32;
      const float x = mine ? scw[g * kChunk + t32] : -INFINITY;
      float cm = x;
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) cm = fmaxf(cm, __shfl_xor(cm, o, 64));
      const float mn = fmaxf(mrun[j], cm);
      const float corr = exp2f(mrun[j] - mn);
      const float w = exp2f(x - mn);
      mrun[j] = mn;
      lrun[j] = fmaf(lrun[j], corr, w);
      crow[j] = corr;
      any |= mine && corr != 1.0f;
      if (mine) scw[g * kChunk + t32] = t32 < d.ntok ? w * d.vn : 0.0f;
      if (mine && t32 == 0) crr[wave][g] = corr;
    }
    wave_sync();
    // rescale the value accumulators if any running max moved
    if (__ballot(any)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = crr[wave][(4 * kg + r) % G];
#pragma unroll
        for (int bl = 0; bl < 8; ++bl) acc[bl][r] *= f;
      }
    }
    // ---- A operand of the value product: row m = n, tokens 8kg .. 8kg+7
    u4 aw = u4{0u, 0u, 0u, 0u};
    if (n < 2 * G) {
      const int g = n < G ? n : n - G;
      const float4* pw = reinterpret_cast<const float4*>(scw + g * kChunk + 8 * kg);
      const float4 w0 = pw[0], w1 = pw[1];
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      uint32_t ww[4];
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        uint32_t h0, l0, h1, l1;
        split_hl(wv[e], h0, l0);
        split_hl(wv[e + 1], h1, l1);
        ww[e / 2] = n < G ? (h0 | (h1 << 16)) : (l0 | (l1 << 16));
      }
      aw = u4{ww[0], ww[1], ww[2], ww[3]};
    }
    wave_sync();
    // ---- value product: block bl covers coordinates 8n' + bl
#pragma unroll
    for (int bl = 0; bl < 8; ++bl) {
      uint32_t x;
      if constexpr (BV == 4) x = d.vw[bl];
      else if constexpr (BV == 2) x = (d.vw[bl] >> vsh) & 0xffffu;
      else x = vtwo ? ((d.vw[bl] >> vsh) | (d.vw2[bl] << (32 - vsh))) & 0xffffffu : (d.vw[bl] >> vsh) & 0xffffffu;
      acc[bl] = mfma(aw, dec8<BV>(x, lutV), acc[bl]);
    }
  };

  int c = wave;
  Chunk<BK, BV, QJL> ca, cb2;
  if (c < nchunks) load(c, ca);
  while (c < nchunks) {
    if (c + kWaves < nchunks) load(c + kWaves, cb2);
    process(ca);
    c += kWaves;
    if (c >= nchunks) break;
    if (c + kWaves < nchunks) load(c + kWaves, ca);
    process(cb2);
    c += kWaves;
  }

  // ---- merge the four waves
  float lsum[GH];
#pragma unroll
  for (int j = 0; j < GH; ++j) {
    float v = (G >= 2 || l < 32) ? lrun[j] : 0.0f;
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) v += __shfl_xor(v, o, 64);
    lsum[j] = v;
  }
  if (t32 == 0) {
#pragma unroll
    for (int j = 0; j < GH; ++j) {
      const int g = G >= 2 ? (l >> 5) + 2 * j : 0;
      if (G >= 2 || l < 32) {
        wm[wave][g] = mrun[j];
        wl[wave][g] = lsum[j];
      }
    }
  }
  __syncthreads();
  // every lane needs M and its wave's factor for rows 4kg + r
  float fac[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int g = (4 * kg + r) % G;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w][g]);
    fac[r] = (M == -INFINITY || wm[wave][g] == -INFINITY) ? 0.0f : exp2f(wm[wave][g] - M);
  }
  for (int w = 0; w < kWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int bl = 0; bl < 8; ++bl)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * kg + r, col = 8 * n + bl;
          const float v = acc[bl][r] * fac[r];
          red[row][col] = (w == 0) ? v : red[row][col] + v;
        }
    }
    __syncthreads();
  }
  for (int i = tid; i < G * kD; i += kScanThreads) {
    const int g = i / kD, j = i % kD;
    a.pacc[(pidx + g) * kD + j] = red[g][j] + red[g + G][j];
  }
  if (tid < G) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w][tid]);
    float L = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (wm[w][tid] != -INFINITY) L = fmaf(exp2f(wm[w][tid] - M), wl[w][tid], L);
    a.pm[pidx + tid] = M;
    a.pl[pidx + tid] = L;
  }
}

template <int G, int BK, int BV>
void launch_bits(bool qjl, dim3 grid, hipStream_t s, const DecodeArgs& a, const DevTables& t, const Codebooks& cb,
                 const KParams& k) {
  if (qjl)
    hipLaunchKernelGGL((scan_mfma_kernel<G, BK, BV, true>), grid, dim3(kScanThreads), 0, s, a, t, cb, k);
  else
    hipLaunchKernelGGL((scan_mfma_kernel<G, BK, BV, false>), grid, dim3(kScanThreads), 0, s, a, t, cb, k);
}

template <int G, int BK>
void launch_bv(int bv, bool qjl, dim3 grid, hipStream_t s, const DecodeArgs& a, const DevTables& t,
               const Codebooks& cb, const KParams& k) {
  if (bv == 2) launch_bits<G, BK, 2>(qjl, grid, s, a, t, cb, k);
  else if (bv == 3) launch_bits<G, BK, 3>(qjl, grid, s, a, t, cb, k);
  else launch_bits<G, BK, 4>(qjl, grid, s, a, t, cb, k);
}

template <int G>
void launch_g(int bk, int bv, bool qjl, dim3 grid, hipStream_t s, const DecodeArgs& a, const DevTables& t,
              const Codebooks& cb, const KParams& k) {
  if (bk == 2) launch_bv<G, 2>(bv, qjl, grid, s, a, t, cb, k);
  else if (bk == 3) launch_bv<G, 3>(bv, qjl, grid, s, a, t, cb, k);
  else launch_bv<G, 4>(bv, qjl, grid, s, a, t, cb, k);
}

}  // namespace

int launch_scan_mfma(const tq_ctx* c, const DecodeArgs& a, const KParams& k, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  dim3 grid(a.splits, k.Hkv, a.batch);
  const int bk = c->p.key_bits, bv = c->p.value_bits;
  const bool qjl = c->p.key_qjl != 0;
  switch (k.G) {
    case 1: launch_g<1>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
    case 2: launch_g<2>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
    case 4: launch_g<4>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
    case 8: launch_g<8>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace tq
