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
// softmax state; the waves of a work-group (four, or sixteen with the wide
// table below) merge at the end.
#include <hip/hip_ext.h>

#include "decode_common.h"
#include "decode_finalize.h"
#include "device_common.h"

namespace tq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u3 __attribute__((ext_vector_type(3)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

constexpr int kChunk = 32;                   // tokens per wave iteration (one value group)
constexpr float kLazy = 8.0f;                // log2 headroom before the running max moves
constexpr uint32_t kRsrcWord3 = 0x00020000;  // raw buffer descriptor flags (gfx9 family)
constexpr int kStream = 2;                   // buffer-load cache policy: non-temporal (pages are read once)

__device__ inline uint32_t h_bits(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}

__device__ inline f4 mfma(u4 a, u4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a), __builtin_bit_cast(h8, b), c, 0, 0, 0);
}

__device__ inline void wave_sync() { __builtin_amdgcn_wave_barrier(); }

template <int CTRL>
__device__ inline float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// max / sum over the 16 lanes of a row (row_ror 8, row_ror 4, quad swaps)
__device__ inline float row_max(float x) {
  x = fmaxf(x, dpp<0x128>(x));
  x = fmaxf(x, dpp<0x124>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  return fmaxf(x, dpp<0xB1>(x));
}
__device__ inline float row_sum(float x) {
  x += dpp<0x128>(x);
  x += dpp<0x124>(x);
  x += dpp<0x4E>(x);
  return x + dpp<0xB1>(x);
}

// fp16 pair (RTZ) of two floats
__device__ inline uint32_t pk_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

// part 0: x truncated to fp16; part 1: x minus that truncation (exact in fp32),
// selected by a per-lane mask (0 for part 0, 0xffffe000 for part 1).  For
// |x| below the fp16 normal range the two parts still add up to x within 2^-24.
__device__ inline float part_of(float x, uint32_t mask) {
  return x - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & mask);
}

// x rounded to fp16, packed pairs: part 0 = hi, part 1 = remainder
__device__ inline uint32_t pack_part(float x0, float x1, int part) {
  const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
  if (part == 0)
    return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
           (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
  return h_bits(x0 - static_cast<float>(h0)) | (h_bits(x1 - static_cast<float>(h1)) << 16);
}

// Lookup tables turning packed codes into fp16 MFMA operands.  A "pair"
// table maps the 2B bits of two consecutive codes to their two fp16 centroids
// (one word).  The LDS serves a 64-lane read as two halves of 32 lanes over
// 32 four-byte banks: a 16-entry table is conflict-free (equal entries
// broadcast) and a 64-entry one costs at most two passes, which measured
// cheaper than replicating it (the replicated address takes one more VALU
// op).  The 256-entry table of 4-bit codes is stored in 32 copies (word e of
// copy c at 32e + c) and lane l reads copy l % 32, so every half-wave touches
// 32 distinct banks whatever the codes are.
// (The high-rate key table of a mixed rate is kept as a single copy: C = 1.)
template <int B, int C = (B == 4 ? 32 : 1)>
struct PairLut {
  static constexpr int kEntries = 1 << (2 * B);
  static constexpr int kCopies = C;
  static constexpr int kWords = kEntries * kCopies;
};

template <int B, int NT, int C = (B == 4 ? 32 : 1)>
__device__ void build_pair_lut(uint32_t* lut, const float* cen, int tid) {
  using L = PairLut<B, C>;
  constexpr int m = (1 << B) - 1;
  for (int w = tid; w < L::kWords; w += NT) {
    const int e = w / L::kCopies;
    lut[w] = h_bits(cen[e & m]) | (h_bits(cen[(e >> B) & m]) << 16);
  }
}

// 8 consecutive codes (8*B bits, LSB-first in x) -> 8 fp16 values; `lut` is
// the lane's copy (already offset by lane % 32 for replicated tables).
template <int B, int C = (B == 4 ? 32 : 1)>
__device__ inline u4 dec8(uint32_t x, const uint32_t* lut) {
  using L = PairLut<B, C>;
  constexpr uint32_t m = (1u << (2 * B)) - 1u;
  u4 r;
  r.x = lut[(x & m) * L::kCopies];
  r.y = lut[((x >> (2 * B)) & m) * L::kCopies];
  r.z = lut[((x >> (4 * B)) & m) * L::kCopies];
  r.w = lut[((x >> (6 * B)) & m) * L::kCopies];
  return r;
}

// sign bits -> fp16 +-1 (bit set = +1): a nibble table of 16 two-word entries
__device__ inline u4 dec_signs8(uint32_t x, const u2* lutN) {
  const u2 a = lutN[x & 15u], c = lutN[(x >> 4) & 15u];
  return u4{a.x, a.y, c.x, c.y};
}

// Work-group shape.  One work-group fills a CU (four SIMDs at the waves per
// SIMD the register budget below allows: 16 or 12 waves); its waves share
// the tables and one chunk counter, so the waves of a CU finish together
// (two eight-wave work-groups per CU ended 15 us apart: the younger one's
// waves lose issue arbitration to the older one's and then run on at half
// occupancy).
// With 4-bit values (and at most four query heads per KV head, for the LDS
// budget) one 64 KB "wide" table serves both the value codes and the sign
// bits, addressed straight from a byte of the code word: row e (256 bytes)
// holds the value pair e in 32 copies (words 64e + c, lane reads copy
// lane % 32: a half-wave touches 32 distinct banks) and, in its second half,
// the eight +-1 fp16 values of sign byte e in 8 copies of 16 bytes (lane
// reads copy lane % 8, one 16-byte read per 8 signs).  One v_perm forms each
// address (byte e into bits 8..15, the lane's copy offset into bits 0..7)
// where the narrow tables take a shift and a mask-or.
// With 2-bit keys and values a "quad" table of the same shape serves both:
// row e holds the four fp16 centroids of code byte e (four 2-bit codes) in
// 16 copies of 8 bytes (lane reads copy lane % 16) and the same sign half,
// so 8 codes take two v_perm addresses and two 8-byte reads, where the
// 16-entry pair table takes a shift and a mask per pair.
// Register budget: 128 VGPRs (four waves per SIMD), except where that would
// spill inside the loop: 3-bit values (two words per value slice) and mixed
// rates (two tables per operand side) get 168 (three waves).  Measured at
// B=16, T=32K with four-wave work-groups: keys 3 / values 3 166 -> 132 us,
// keys 3.5 / values 3 201 -> 136 us.
constexpr bool wide_table(int G, int BV, bool vmix) { return BV == 4 && G <= 8 && !vmix; }
constexpr bool quad_table(int BK, int BV, bool kmix, bool vmix) { return BK == 2 && BV == 2 && !kmix && !vmix; }
constexpr int scan_waves_per_simd(int BV, bool kmix, bool vmix) { return (BV == 3 || kmix || vmix) ? 3 : 4; }
constexpr int scan_threads(int BV, bool kmix, bool vmix) { return 256 * scan_waves_per_simd(BV, kmix, vmix); }

template <int G, int BK, int BV, bool KMIX, bool VMIX>
struct ScanShape {
  static constexpr bool kWide = wide_table(G, BV, VMIX);
  static constexpr bool kQuad = quad_table(BK, BV, KMIX, VMIX);
  static constexpr bool kRows = kWide || kQuad;  // 256-byte rows with the sign half
  static constexpr int kThreads = scan_threads(BV, KMIX, VMIX);
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kLutWords = kRows ? 256 * 64 : PairLut<BV>::kWords;
};

// address of byte K of x in a 256-byte-row table, plus the lane's copy offset
template <int K>
__device__ inline uint32_t row_addr(uint32_t x, uint32_t base) {
  return __builtin_amdgcn_perm(x, base, 0x0C0C0000u | ((4u + K) << 8));
}
__device__ inline uint32_t lds_word(const uint32_t* t, uint32_t byte_addr) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(t) + byte_addr);
}
// 8 consecutive 4-bit codes -> 8 fp16 values from the wide table
__device__ inline u4 dec8_wide(uint32_t x, const uint32_t* t, uint32_t vbase) {
  return u4{lds_word(t, row_addr<0>(x, vbase)), lds_word(t, row_addr<1>(x, vbase)),
            lds_word(t, row_addr<2>(x, vbase)), lds_word(t, row_addr<3>(x, vbase))};
}
// selector of v_perm placing byte K of its first operand in bits 8..15 and
// byte 0 of the second in bits 0..7
constexpr uint32_t row_sel(int K) { return 0x0C0C0000u | ((4u + K) << 8); }
// 8 consecutive 2-bit codes (bytes of x picked by sel0, sel1) -> 8 fp16
// values from the quad table
__device__ inline u4 dec8_quad(uint32_t x, const uint32_t* t, uint32_t qbase, uint32_t sel0, uint32_t sel1) {
  const u2 a = *reinterpret_cast<const u2*>(reinterpret_cast<const char*>(t) + __builtin_amdgcn_perm(x, qbase, sel0));
  const u2 b = *reinterpret_cast<const u2*>(reinterpret_cast<const char*>(t) + __builtin_amdgcn_perm(x, qbase, sel1));
  return u4{a.x, a.y, b.x, b.y};
}
// sign byte K of x -> 8 fp16 +-1 from the wide table
template <int K>
__device__ inline u4 dec_signs_wide(uint32_t x, const uint32_t* t, uint32_t sbase) {
  return *reinterpret_cast<const u4*>(reinterpret_cast<const char*>(t) + row_addr<K>(x, sbase));
}

// Codes 8i .. 8i+7 of a lane's 32-code key slice held in B words.
template <int B>
__device__ inline uint32_t key_slice(const uint32_t* w, int i) {
  if constexpr (B == 4) return w[i];
  else if constexpr (B == 2) return (w[i >> 1] >> (16 * (i & 1))) & 0xffffu;
  else return bits_at<24>(w, 24 * i);
}

// The lane's 8 codes of width W in a value word: bits [sh, sh + 8W), from
// the next word too when a 3-bit slice straddles (two).
template <int W>
__device__ inline uint32_t vslice(uint32_t w0, uint32_t w1, int sh, bool two) {
  if constexpr (W == 4) return w0;
  else if constexpr (W == 2) return (w0 >> sh) & 0xffffu;
  else return two ? ((w0 >> sh) | (w1 << (32 - sh))) & 0xffffffu : (w0 >> sh) & 0xffffffu;
}

// Per-chunk data, split so that key and value words can be loaded at
// different times: a chunk's keys are scored one step before its values are
// accumulated, and both are fetched one step ahead of use.
template <int BK, bool KMIX>
struct KBuf {
  // key codes of tokens n / 16+n, coordinates 32kg .. 32kg+31; mixed rate:
  // words 0-1 the low-rate piece (coordinates 32kg .. +15), 2-3 the high-rate one
  uint32_t kc[2][KMIX ? 4 : BK];
  uint32_t sg[2];      // their sign bits
  uint32_t kn[2];      // key norms: float32 bits, or u8 log-norm codes (decoded when scoring)
  float rn[2];
  float vn[2];         // value norms of tokens n / 16+n (used when scoring)
};
template <int BV, bool VMIX>
struct VBuf {
  uint32_t vw[8];  // value words: coordinates 8n .. 8n+7, tokens 8kg .. 8kg+7
  // next word when a 3-bit slice straddles two words (mixed: either half may be 3-bit)
  uint32_t vw2[(BV == 3 || VMIX) ? 8 : 1];
};
// wave-uniform chunk description (scalar registers)
struct Meta {
  __amdgpu_buffer_rsrc_t rs;
  int s0;    // first token of the chunk inside its page
  int gi;    // value group (32 tokens) inside the page
  int ntok;  // live tokens (0 when the page id is invalid)
  int pos0;  // position of the chunk's first token
};

// A row m of every MFMA holds query g = 2(m/4) + (m%2), part (m/2)%2 (0: fp16
// hi, 1: remainder); the product's rows 4kg + r land in lane group kg, so a
// lane sees query 2kg + i as rows i (hi) and i + 2 (remainder) and adds them.
// KMIX / VMIX: mixed-channel rate BK + 1/2 (BV + 1/2): the high-rate half
// of the coordinates (keys: j mod 32 >= 16, values: j mod 8 >= 4) takes one
// more bit and its own codebook.  A lane's key slice then holds a low-rate
// piece (MFMAs i = 0, 1) and a high-rate piece (i = 2, 3); value MFMA bl
// reads the low-rate word block for bl < 4 and the high-rate one otherwise,
// so every operand slice has one compile-time width.
template <int G, int BK, int BV, bool QJL, bool KMIX, bool VMIX, bool N8>
__global__ __launch_bounds__((ScanShape<G, BK, BV, KMIX, VMIX>::kThreads), (scan_waves_per_simd(BV, KMIX, VMIX))) void
scan_mfma_kernel(DecodeArgs a, DevTables t, Codebooks cb, KParams k) {
  using Sh = ScanShape<G, BK, BV, KMIX, VMIX>;
  constexpr bool kWide = Sh::kWide, kQuad = Sh::kQuad, kRows = Sh::kRows;
  constexpr int kThreads = Sh::kThreads, kWaves = Sh::kWaves;
  // One array: the key table (absent when keys and values share a bit width,
  // hence a codebook) first, so that every table address stays within the
  // 16-bit immediate offset of the LDS instructions.
  // keys read the value table of their width when there is one (the
  // codebook depends on the width only): BK == BV, or the high-rate half of
  // mixed values when BK == BV + 1
  constexpr bool kKeyInVhi = VMIX && BK == BV + 1;
  constexpr int kKeyWords = (BK == BV || kKeyInVhi) ? 0 : PairLut<BK>::kWords;
  constexpr int kKeyHiWords = KMIX ? PairLut<BK + 1, 1>::kWords : 0;  // mixed keys: high-rate table, one copy
  constexpr int kValHiWords = VMIX ? PairLut<BV + 1>::kWords : 0;     // mixed values: high-rate table
  __shared__ __align__(16) uint32_t luts[kKeyWords + kKeyHiWords + Sh::kLutWords + kValHiWords];
  uint32_t* const lutKown = luts;
  uint32_t* const lutKhi = luts + kKeyWords;
  uint32_t* const lutV = luts + kKeyWords + kKeyHiWords;
  uint32_t* const lutVhi = lutV + Sh::kLutWords;
  __shared__ u2 lutN[kRows ? 1 : 16];
  __shared__ float pv[kWaves][2][G][kChunk];  // softmax weights x value norms, two chunks in flight
  __shared__ float wm[kWaves][G], wl[kWaves][G];
  __shared__ float red[G][kD];
  __shared__ float ck[16], cvv[16], ck2[16], cv2[16];
  // scratch of the end phases: the waves' scaled accumulators (one slot of
  // G x kD floats per wave), then the final combine (last work-group of the
  // kv head); the table memory when that is large enough
  constexpr int kFin = finalize_scratch_floats<kThreads, G>();
  constexpr int kEnd = kFin > kWaves * G * kD ? kFin : kWaves * G * kD;
  constexpr bool kEndInLuts = sizeof(luts) >= sizeof(float) * kEnd;
  __shared__ __align__(16) float end_own[kEndInLuts ? 1 : kEnd];
  float* const endbuf = kEndInLuts ? reinterpret_cast<float*>(luts) : end_own;
  __shared__ float fsm[2][G];
  __shared__ int fflag;
  __shared__ int next_chunk;  // the split's next unclaimed chunk
  __shared__ int page_ids[kMaxSplitPages];

  const int tid = threadIdx.x;
  // (b, kv head h, split): the grid position, or with balanced splits plan
  // entry blockIdx.x (whose partial slot it is); idle entries leave at once
  int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, pps = a.pages_per_split, nsplit = a.splits;
  int64_t slot = (static_cast<int64_t>(b) * k.Hkv + h) * a.splits + split;
  if (a.plan) {
    const int4 e = a.plan[blockIdx.x];
    const int bh = __builtin_amdgcn_readfirstlane(e.x);
    if (bh < 0) return;
    b = bh / k.Hkv;
    h = bh - b * k.Hkv;
    split = __builtin_amdgcn_readfirstlane(e.y);
    nsplit = __builtin_amdgcn_readfirstlane(e.z);
    pps = __builtin_amdgcn_readfirstlane(e.w);
    slot = blockIdx.x;
    // an entry out of range (a plan prep did not write) touches nothing
    if (b >= a.batch || split < 0 || split >= nsplit || pps < 1 || pps > kMaxSplitPages) return;
  }
  // the wave index is uniform within a wave; saying so keeps page addresses
  // and buffer descriptors in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, n = l & 15, kg = l >> 4;
  // Loads that do not depend on the sequence length are issued first, so
  // that they land while the length is read and the tables are built: the
  // query operands (A operands of the key products: lane group kg covers
  // coordinates 32kg .. 32kg+31, MFMA i the 8 starting at 32kg + 8i) and the
  // split's page ids (vector loads: a scalar load's out-of-order return would
  // make every later LDS wait a full drain).
  const int64_t qrow = (static_cast<int64_t>(b) * k.Hq + static_cast<int64_t>(h) * G) * kD;
  const int ag = 2 * (n >> 2) + (n & 1), apart = (n >> 1) & 1;
  const int agc = ag < G ? ag : 0;
  float4 qin[4][2], pin[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4* q4 = reinterpret_cast<const float4*>(a.qs + qrow + agc * kD + 32 * kg + 8 * i);
    qin[i][0] = q4[0];
    qin[i][1] = q4[1];
    if constexpr (QJL) {
      const float4* p4 = reinterpret_cast<const float4*>(a.ps + qrow + agc * kD + 32 * kg + 8 * i);
      pin[i][0] = p4[0];
      pin[i][1] = p4[1];
    }
  }
  // the split's page ids (at most kMaxSplitPages), to LDS by the first
  // threads: a chunk reads its page id from there (held in a register, it
  // was spilled, and its reload at the top of every step waited for all
  // loads in flight)
  const int pb = split * pps;
  int pid_in = 0;
  if (tid < kMaxSplitPages)
    pid_in = a.block_table[static_cast<int64_t>(b) * a.max_pages + (pb + tid < a.max_pages ? pb + tid : 0)];
  const int T = a.seq_lens[b];
  const int C = T - k.W > 0 ? T - k.W : 0;
  const int npages = (C + k.P - 1) / k.P;
  int pe = npages < pb + pps ? npages : pb + pps;
  const int64_t pidx = slot * G;
  if (pe > a.max_pages) {
    if (tid == 0) atomicOr(t.status, TQ_STATUS_BAD_PAGE);
    pe = a.max_pages;
  }
  if (pb >= pe) {
    if (tid < G) {
      a.pm[pidx + tid] = -INFINITY;
      a.pl[pidx + tid] = 0.0f;
    }
    for (int i = tid; i < G * kD; i += kThreads) a.pacc[pidx * kD + i] = 0.0f;
    if (a.fuse && arrive_last<kThreads>(a.ctr + static_cast<int64_t>(b) * k.Hkv + h, nsplit, &fflag))
      finalize_bh<kThreads, G>(a, t, k, b, h, 0, red, endbuf, fsm[0], fsm[1], nullptr, nullptr, nullptr,
                               slot - split, nsplit);
    return;
  }
  // codebooks to LDS (no dynamic indexing of kernel arguments), then the tables
  if (tid == 0) next_chunk = kWaves;  // wave w starts with chunk w
  if (tid < kMaxSplitPages) page_ids[tid] = pid_in;
  if (tid < 16) {
    float kv = 0.0f, vv = 0.0f, kv2 = 0.0f, vv2 = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i == tid) {
        kv = cb.kc[i];
        vv = cb.vc[i];
        kv2 = cb.kc2[i];
        vv2 = cb.vc2[i];
      }
    ck[tid] = kv;
    cvv[tid] = vv;
    ck2[tid] = kv2;
    cv2[tid] = vv2;
  }
  __syncthreads();
  if constexpr (kRows) {
    // row e: words 0..31 the value pair of byte e (32 copies; quad table:
    // the four values of byte e, 16 copies of two words), words 32..63 the
    // four sign words of byte e (8 copies); written four words at a time
    auto sgn_word = [](int e, int j) {  // word j of sign byte e: bits 2j (low half) and 2j + 1
      return ((e >> (2 * j)) & 1 ? 0x3C00u : 0xBC00u) | (((e >> (2 * j + 1)) & 1 ? 0x3C00u : 0xBC00u) << 16);
    };
    u4* lut4 = reinterpret_cast<u4*>(lutV);
    for (int w4 = tid; w4 < Sh::kLutWords / 4; w4 += kThreads) {
      const int e = w4 >> 4;
      u4 v;
      if ((w4 & 15) < 8) {
        if constexpr (kQuad) {
          const uint32_t x0 = h_bits(cvv[e & 3]) | (h_bits(cvv[(e >> 2) & 3]) << 16);
          const uint32_t x1 = h_bits(cvv[(e >> 4) & 3]) | (h_bits(cvv[e >> 6]) << 16);
          v = u4{x0, x1, x0, x1};
        } else {
          const uint32_t x = h_bits(cvv[e & 15]) | (h_bits(cvv[e >> 4]) << 16);
          v = u4{x, x, x, x};
        }
      } else {
        v = u4{sgn_word(e, 0), sgn_word(e, 1), sgn_word(e, 2), sgn_word(e, 3)};
      }
      lut4[w4] = v;
    }
  } else {
    build_pair_lut<BV, kThreads>(lutV, cvv, tid);
  }
  if constexpr (BK != BV && !kKeyInVhi) build_pair_lut<BK, kThreads>(lutKown, ck, tid);
  if constexpr (KMIX) build_pair_lut<BK + 1, kThreads, 1>(lutKhi, ck2, tid);
  if constexpr (VMIX) build_pair_lut<BV + 1, kThreads>(lutVhi, cv2, tid);
  if (!kRows && tid < 16) {
    const int e = tid;
    lutN[e] = u2{(e & 1 ? 0x3C00u : 0xBC00u) | ((e & 2 ? 0x3C00u : 0xBC00u) << 16),
                 (e & 4 ? 0x3C00u : 0xBC00u) | ((e & 8 ? 0x3C00u : 0xBC00u) << 16)};
  }
  const uint32_t* lutK = BK == BV ? lutV : kKeyInVhi ? lutVhi : lutKown;
  const uint32_t* lutKl = lutK + (PairLut<BK>::kCopies > 1 ? (tid & 31) : 0);
  const uint32_t* lutVl = lutV + (PairLut<BV>::kCopies > 1 ? (tid & 31) : 0);
  const uint32_t* lutVhil = lutVhi + ((VMIX && PairLut<BV + 1>::kCopies > 1) ? (tid & 31) : 0);
  const uint32_t vbase = static_cast<uint32_t>(tid & 31) * 4u, sbase = 128u + static_cast<uint32_t>(tid & 7) * 16u;
  const uint32_t qbase = static_cast<uint32_t>(tid & 15) * 8u;  // quad table: the lane's copy
  // the query operands, fp16 hi part or remainder per lane (zero for rows
  // past the G queries)
  u4 aq[4], ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 q0 = qin[i][0], q1 = qin[i][1];
    aq[i] = u4{pack_part(q0.x, q0.y, apart), pack_part(q0.z, q0.w, apart), pack_part(q1.x, q1.y, apart),
               pack_part(q1.z, q1.w, apart)};
    ap[i] = u4{0u, 0u, 0u, 0u};
    if constexpr (QJL) {
      const float4 p0 = pin[i][0], p1 = pin[i][1];
      ap[i] = u4{pack_part(p0.x, p0.y, apart), pack_part(p0.z, p0.w, apart), pack_part(p1.x, p1.y, apart),
                 pack_part(p1.z, p1.w, apart)};
    }
    if (ag >= G) {
      aq[i] = u4{0u, 0u, 0u, 0u};
      ap[i] = u4{0u, 0u, 0u, 0u};
    }
  }
  __syncthreads();

  // running state of queries 2kg (i = 0) and 2kg + 1 (i = 1)
  float mrun[2] = {-INFINITY, -INFINITY}, lrun[2] = {0.0f, 0.0f};
  f4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f4{0.0f, 0.0f, 0.0f, 0.0f};

  const int tot = (C < pe * k.P ? C : pe * k.P) - pb * k.P;
  const int nchunks = (tot + kChunk - 1) / kChunk;
  // value words: the lane's 8 tokens of coordinate 8n + bl are bits [8*kg*BV, +8*BV)
  const int vbit = 8 * kg * BV;
  const int vw0 = vbit >> 5, vsh = vbit & 31;
  const bool vtwo = (vsh + 8 * BV) > 32;
  // per-lane byte offsets inside a head block (the chunk adds a uniform offset)
  const uint32_t o_tok0 = 4u * n, o_tok1 = 4u * (16 + n);
  constexpr int kKRec = 16 * BK + (KMIX ? 8 : 0);  // key record bytes
  const uint32_t o_kc0 = static_cast<uint32_t>(n * 16 * BK + 4 * BK * kg);
  const uint32_t o_kc1 = o_kc0 + 16u * 16u * BK;
  // mixed keys: the lane's low-rate piece (2 BK bytes at 2 BK kg) and
  // high-rate piece (2 (BK+1) bytes at 8 BK + 2 (BK+1) kg) of the record, each
  // read as 8 bytes from the 4-byte boundary below and shifted down
  const uint32_t oL = 2u * BK * kg, oH = 8u * BK + 2u * (BK + 1) * kg;
  const uint32_t o_kL0 = n * kKRec + (oL & ~3u), o_kH0 = n * kKRec + (oH & ~3u);
  const uint32_t o_kL1 = o_kL0 + 16u * kKRec, o_kH1 = o_kH0 + 16u * kKRec;
  const uint32_t shL = 8u * (oL & 3u), shH = 8u * (oH & 3u);
  // mixed values: low-rate block [BV][64] then high-rate block [BV+1][64] per
  // group; MFMA bl < 4 reads low-rate ranks 4n .. 4n+3, bl >= 4 high-rate ones
  const int vbitL = 8 * kg * BV, vbitH = 8 * kg * (BV + 1);
  const int vwL = vbitL >> 5, vshL = vbitL & 31, vwH = vbitH >> 5, vshH = vbitH & 31;
  const bool vtwoL = (vshL + 8 * BV) > 32, vtwoH = (vshH + 8 * (BV + 1)) > 32;
  const uint32_t vHiBlock = 64u * BV * 4u;
  const uint32_t o_vwL = static_cast<uint32_t>((vwL * 64 + 4 * n) * 4);
  const uint32_t o_vwL2 = static_cast<uint32_t>(((vtwoL ? vwL + 1 : vwL) * 64 + 4 * n) * 4);
  const uint32_t o_vwH = vHiBlock + static_cast<uint32_t>((vwH * 64 + 4 * n) * 4);
  const uint32_t o_vwH2 = vHiBlock + static_cast<uint32_t>(((vtwoH ? vwH + 1 : vwH) * 64 + 4 * n) * 4);
  const uint32_t o_sg0 = static_cast<uint32_t>(n * 16 + 4 * kg), o_sg1 = o_sg0 + 256u;
  const uint32_t o_vw = static_cast<uint32_t>((vw0 * kD + 8 * n) * 4);
  const uint32_t o_vw2 = static_cast<uint32_t>(((vtwo ? vw0 + 1 : vw0) * kD + 8 * n) * 4);

  auto meta = [&](int c, Meta& m) {
    const int tok0 = c * kChunk;
    const int pg = pb + tok0 / k.P;
    m.gi = (tok0 % k.P) / kChunk;
    m.s0 = m.gi * kChunk;
    const int rem = tot - tok0;
    m.pos0 = pg * k.P + m.s0;
    const int pid0 = __builtin_amdgcn_readfirstlane(page_ids[pg - pb]);
    const bool bad = pid0 < 0 || pid0 >= a.num_pages;  // flagged, then page 0 is read and the chunk masked
    if (bad && l == 0) atomicOr(t.status, TQ_STATUS_BAD_PAGE);
    m.ntok = __builtin_amdgcn_readfirstlane(bad ? 0 : (rem < kChunk ? rem : kChunk));
    const int pid = __builtin_amdgcn_readfirstlane(bad ? 0 : pid0);
    const uint8_t* hb = a.pool + static_cast<int64_t>(pid) * k.page_bytes + kBodyOffset + h * k.head_bytes;
    m.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(hb), 0, static_cast<int>(k.head_bytes), kRsrcWord3);
  };
  auto loadK = [&](const Meta& m, KBuf<BK, KMIX>& d) {
    if constexpr (N8) {
      const int so_kn = static_cast<int>(k.k_norm) + m.s0;
      d.kn[0] = __builtin_amdgcn_raw_buffer_load_b8(m.rs, o_tok0 >> 2, so_kn, kStream);
      d.kn[1] = __builtin_amdgcn_raw_buffer_load_b8(m.rs, o_tok1 >> 2, so_kn, kStream);
    } else {
      const int so_kn = static_cast<int>(k.k_norm) + 4 * m.s0;
      d.kn[0] = __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_tok0, so_kn, kStream);
      d.kn[1] = __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_tok1, so_kn, kStream);
    }
    if constexpr (QJL) {
      const int so_rn = static_cast<int>(k.k_rnorm) + 4 * m.s0;
      d.rn[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_tok0, so_rn, kStream));
      d.rn[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_tok1, so_rn, kStream));
      const int so_sg = static_cast<int>(k.k_signs) + 16 * m.s0;
      d.sg[0] = __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_sg0, so_sg, kStream);
      d.sg[1] = __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_sg1, so_sg, kStream);
    }
    const int so_vn = static_cast<int>(k.v_norm) + 4 * m.s0;
    d.vn[0] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_tok0, so_vn, kStream));
    d.vn[1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(m.rs, o_tok1, so_vn, kStream));
    const int so_kc = static_cast<int>(k.k_codes) + kKRec * m.s0;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint32_t o = tt ? o_kc1 : o_kc0;
      if constexpr (KMIX) {
        const u2 lo = __builtin_amdgcn_raw_buffer_load_b64(m.rs, tt ? o_kL1 : o_kL0, so_kc, kStream);
        const u2 hi = __builtin_amdgcn_raw_buffer_load_b64(m.rs, tt ? o_kH1 : o_kH0, so_kc, kStream);
        d.kc[tt][0] = __builtin_amdgcn_alignbit(lo.y, lo.x, shL);
        d.kc[tt][1] = lo.y >> shL;
        d.kc[tt][2] = __builtin_amdgcn_alignbit(hi.y, hi.x, shH);
        d.kc[tt][3] = hi.y >> shH;
      } else if constexpr (BK == 4) {
        const u4 v = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o, so_kc, kStream);
        d.kc[tt][0] = v.x; d.kc[tt][1] = v.y; d.kc[tt][2] = v.z; d.kc[tt][3] = v.w;
      } else if constexpr (BK == 3) {
        const u3 v = __builtin_amdgcn_raw_buffer_load_b96(m.rs, o, so_kc, kStream);
        d.kc[tt][0] = v.x; d.kc[tt][1] = v.y; d.kc[tt][2] = v.z;
      } else {
        const u2 v = __builtin_amdgcn_raw_buffer_load_b64(m.rs, o, so_kc, kStream);
        d.kc[tt][0] = v.x; d.kc[tt][1] = v.y;
      }
    }
  };
  auto loadV = [&](const Meta& m, VBuf<BV, VMIX>& d) {
    if constexpr (VMIX) {
      const int so_vw = static_cast<int>(k.v_codes) + m.gi * 256 * (2 * BV + 1);
      const u4 x0 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vwL, so_vw, kStream);
      const u4 x1 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vwH, so_vw, kStream);
      d.vw[0] = x0.x; d.vw[1] = x0.y; d.vw[2] = x0.z; d.vw[3] = x0.w;
      d.vw[4] = x1.x; d.vw[5] = x1.y; d.vw[6] = x1.z; d.vw[7] = x1.w;
      if constexpr (BV == 3) {  // the 3-bit low-rate slice may straddle two words
        const u4 y0 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vwL2, so_vw, kStream);
        d.vw2[0] = y0.x; d.vw2[1] = y0.y; d.vw2[2] = y0.z; d.vw2[3] = y0.w;
      } else {  // BV == 2: the 3-bit high-rate slice may
        const u4 y1 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vwH2, so_vw, kStream);
        d.vw2[4] = y1.x; d.vw2[5] = y1.y; d.vw2[6] = y1.z; d.vw2[7] = y1.w;
      }
      return;
    }
    const int so_vw = static_cast<int>(k.v_codes) + m.gi * BV * kD * 4;
    const u4 x0 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vw, so_vw, kStream);
    const u4 x1 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vw + 16u, so_vw, kStream);
    d.vw[0] = x0.x; d.vw[1] = x0.y; d.vw[2] = x0.z; d.vw[3] = x0.w;
    d.vw[4] = x1.x; d.vw[5] = x1.y; d.vw[6] = x1.z; d.vw[7] = x1.w;
    if constexpr (BV == 3) {
      const u4 y0 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vw2, so_vw, kStream);
      const u4 y1 = __builtin_amdgcn_raw_buffer_load_b128(m.rs, o_vw2 + 16u, so_vw, kStream);
      d.vw2[0] = y0.x; d.vw2[1] = y0.y; d.vw2[2] = y0.z; d.vw2[3] = y0.w;
      d.vw2[4] = y1.x; d.vw2[5] = y1.y; d.vw2[6] = y1.z; d.vw2[7] = y1.w;
    }
  };

  float* pvw = &pv[wave][0][0][0];
  const int64_t dbg_row = (static_cast<int64_t>(b) * k.Hq + h * G) * a.logits_stride;
  // ---- scores of one chunk, online softmax, weights x value norms to pv[slot]
  auto keyphase = [&](const Meta& m, const KBuf<BK, KMIX>& d, int slot) {
    float sc[2][2];  // [query i][tile]
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      f4 dm = f4{0.0f, 0.0f, 0.0f, 0.0f}, dq = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KMIX) {
          if (i < 2) dm = mfma(aq[i], dec8<BK>(key_slice<BK>(&d.kc[tt][0], i), lutKl), dm);
          else dm = mfma(aq[i], dec8<BK + 1, 1>(key_slice<BK + 1>(&d.kc[tt][2], i - 2), lutKhi), dm);
        } else if constexpr (kWide && BK == 4) {
          dm = mfma(aq[i], dec8_wide(d.kc[tt][i], lutV, vbase), dm);
        } else if constexpr (kQuad) {
          // codes 8i .. 8i+7: bytes 2(i%2), 2(i%2)+1 of word i/2
          dm = mfma(aq[i], dec8_quad(d.kc[tt][i >> 1], lutV, qbase, row_sel(2 * (i & 1)), row_sel(2 * (i & 1) + 1)), dm);
        } else {
          dm = mfma(aq[i], dec8<BK>(key_slice<BK>(d.kc[tt], i), lutKl), dm);
        }
        if constexpr (QJL && kRows) {
          const uint32_t sgw = d.sg[tt];
          const u4 sb = i == 0 ? dec_signs_wide<0>(sgw, lutV, sbase)
                        : i == 1 ? dec_signs_wide<1>(sgw, lutV, sbase)
                        : i == 2 ? dec_signs_wide<2>(sgw, lutV, sbase)
                                 : dec_signs_wide<3>(sgw, lutV, sbase);
          dq = mfma(ap[i], sb, dq);
        } else if constexpr (QJL) {
          dq = mfma(ap[i], dec_signs8(d.sg[tt] >> (8 * i), lutN), dq);
        }
      }
      const bool live = 16 * tt + n < m.ntok;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        // u8 log-norm code q: level 2^(q/16 - 4), code 0 a zero norm
        const float kn = N8 ? (d.kn[tt] ? __builtin_amdgcn_exp2f(static_cast<float>(d.kn[tt]) * 0.0625f - 4.0f)
                                        : 0.0f)
                            : __builtin_bit_cast(float, d.kn[tt]);
        float v = (dm[i] + dm[i + 2]) * kn;
        if constexpr (QJL) v = fmaf(dq[i] + dq[i + 2], d.rn[tt], v);
        sc[i][tt] = live ? v : -INFINITY;
      }
    }
    if (a.dbg_logits) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (2 * kg + i < G && 16 * tt + n < m.ntok)
            a.dbg_logits[dbg_row + (2 * kg + i) * a.logits_stride + m.pos0 + 16 * tt + n] = sc[i][tt] * kLn2;
    }
    float* pw = pvw + slot * (G * kChunk);
    float corr[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float lm = fmaxf(sc[i][0], sc[i][1]);
      bool move = false;
      float mn = mrun[i];
      if (__ballot(lm > mrun[i] + kLazy)) {  // rare after the first chunk
        const float cm = row_max(lm);
        move = cm > mrun[i] + kLazy;
        mn = move ? cm : mrun[i];
      }
      corr[i] = move ? __builtin_amdgcn_exp2f(mrun[i] - mn) : 1.0f;
      mrun[i] = mn;
      // a dead token has score -inf and weight exp2(-inf) = 0; while mn is
      // still -inf every score is, and the reference 0 keeps them at 0
      const float mref = mn == -INFINITY ? 0.0f : mn;
      const float w0 = __builtin_amdgcn_exp2f(sc[i][0] - mref);
      const float w1 = __builtin_amdgcn_exp2f(sc[i][1] - mref);
      lrun[i] = fmaf(lrun[i], corr[i], w0 + w1);
      const int g = 2 * kg + i;
      if (g < G) {
        // dead tokens may carry garbage norms: select, do not multiply by 0
        pw[g * kChunk + n] = n < m.ntok ? w0 * d.vn[0] : 0.0f;
        pw[g * kChunk + 16 + n] = 16 + n < m.ntok ? w1 * d.vn[1] : 0.0f;
      }
    }
    wave_sync();
    if (corr[0] != 1.0f || corr[1] != 1.0f) {
#pragma unroll
      for (int bl = 0; bl < 8; ++bl) {
        acc[bl][0] *= corr[0];
        acc[bl][2] *= corr[0];
        acc[bl][1] *= corr[1];
        acc[bl][3] *= corr[1];
      }
    }
  };
  // ---- value product of one chunk with the weights in pv[slot]
  auto valuephase = [&](const VBuf<BV, VMIX>& d, int slot) {
    // the lane's weight row (query ag, hi or remainder part, tokens 8kg ..), derived
    // afresh from the lane id each step: an opaque read of the id keeps these
    // values out of the registers held across the loop (a spill there would
    // make every step wait for all loads in flight)
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    const int wn = ln & 15, wkg = ln >> 4;
    const int wag = 2 * (wn >> 2) + (wn & 1);
    const uint32_t wmask = ((wn >> 1) & 1) ? 0xffffe000u : 0u;
    u4 aw = u4{0u, 0u, 0u, 0u};
    if (wag < G) {
      const float4* pw = reinterpret_cast<const float4*>(pvw + slot * (G * kChunk) + wag * kChunk + 8 * wkg);
      const float4 w0 = pw[0], w1 = pw[1];
      aw = u4{pk_rtz(part_of(w0.x, wmask), part_of(w0.y, wmask)), pk_rtz(part_of(w0.z, wmask), part_of(w0.w, wmask)),
              pk_rtz(part_of(w1.x, wmask), part_of(w1.y, wmask)), pk_rtz(part_of(w1.z, wmask), part_of(w1.w, wmask))};
    }
    if constexpr (VMIX) {
#pragma unroll
      for (int bl = 0; bl < 8; ++bl) {
        if (bl < 4)
          acc[bl] = mfma(aw, dec8<BV>(vslice<BV>(d.vw[bl], d.vw2[bl], vshL, vtwoL), lutVl), acc[bl]);
        else
          acc[bl] = mfma(aw, dec8<BV + 1>(vslice<BV + 1>(d.vw[bl], d.vw2[bl], vshH, vtwoH), lutVhil), acc[bl]);
      }
      return;
    }
    if constexpr (kQuad) {
      // the lane's 8 codes are bytes 2(kg%2), 2(kg%2)+1 of each value word
      const uint32_t qs0 = 0x0C0C0400u + ((2u * (static_cast<uint32_t>(wkg) & 1u)) << 8), qs1 = qs0 + 0x100u;
#pragma unroll
      for (int bl = 0; bl < 8; ++bl) acc[bl] = mfma(aw, dec8_quad(d.vw[bl], lutV, qbase, qs0, qs1), acc[bl]);
      return;
    }
#pragma unroll
    for (int bl = 0; bl < 8; ++bl) {
      uint32_t x;
      if constexpr (BV == 4) x = d.vw[bl];
      else if constexpr (BV == 2) x = (d.vw[bl] >> vsh) & 0xffffu;
      else x = vtwo ? ((d.vw[bl] >> vsh) | (d.vw2[bl] << (32 - vsh))) & 0xffffffu : (d.vw[bl] >> vsh) & 0xffffffu;
      if constexpr (kWide) acc[bl] = mfma(aw, dec8_wide(x, lutV, vbase), acc[bl]);
      else acc[bl] = mfma(aw, dec8<BV>(x, lutVl), acc[bl]);
    }
  };

  // Software pipeline over this wave's chunks: each step accumulates the
  // values of the current chunk and scores the next one.  Each buffer is
  // refilled as soon as it is consumed: keys (with the value norms) of the
  // next chunk load while the current chunk's values are accumulated, its
  // values while it is scored.  The weights alternate between two pv slots.
  // Wave w starts with chunk w and then claims the split's next unclaimed
  // chunk (an LDS counter, claimed one step ahead of its loads), so the
  // waves of a work-group finish within about one chunk of each other; the
  // grouping of the sums then varies between calls.  With k.det every wave
  // takes the fixed share w, w + kWaves, ... (bit-reproducible results).
  auto claim = [&]() {
    int c = 0;
    if (l == 0) c = atomicAdd(&next_chunk, 1);
    return __builtin_amdgcn_readfirstlane(c);
  };
  Meta m;
  KBuf<BK, KMIX> kb;
  VBuf<BV, VMIX> vb;
  if (wave < nchunks) {
    meta(wave, m);
    loadK(m, kb);
    loadV(m, vb);
    int cn = k.det ? wave + kWaves : claim();
    keyphase(m, kb, 0);
    int i = 0;
    for (; cn < nchunks; ++i) {
      meta(cn, m);
      loadK(m, kb);
      const int cnn = k.det ? cn + kWaves : claim();
      valuephase(vb, i & 1);
      loadV(m, vb);
      keyphase(m, kb, (i + 1) & 1);
      cn = cnn;
    }
    valuephase(vb, i & 1);
  }

  // ---- merge the waves: per query max M, factors 2^(m_w - M)
  float ls[2];
#pragma unroll
  for (int i2 = 0; i2 < 2; ++i2) ls[i2] = row_sum(lrun[i2]);
  if (n == 0) {
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
      if (2 * kg + i2 < G) {
        wm[wave][2 * kg + i2] = mrun[i2];
        wl[wave][2 * kg + i2] = ls[i2];
      }
  }
  __syncthreads();
  float fac[2];
#pragma unroll
  for (int i2 = 0; i2 < 2; ++i2) {
    const int g = 2 * kg + i2 < G ? 2 * kg + i2 : 0;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wm[w][g]);
    fac[i2] = (M == -INFINITY || wm[wave][g] == -INFINITY) ? 0.0f : exp2f(wm[wave][g] - M);
  }
  {
    // every wave stores its scaled accumulators in a slot of its own (when
    // the slots are the table memory, the tables are not read any more: all
    // waves have passed the barrier above), then each element is summed over
    // the waves in order 0 .. kWaves-1
    float* wslot = endbuf;
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const int g = 2 * kg + i2;
      if (g < G) {
#pragma unroll
        for (int bl = 0; bl < 8; ++bl)
          wslot[(wave * G + g) * kD + 8 * n + bl] = (acc[bl][i2] + acc[bl][i2 + 2]) * fac[i2];
      }
    }
    __syncthreads();
    for (int e = tid; e < G * kD; e += kThreads) {
      float v = wslot[e];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += wslot[w * G * kD + e];
      a.pacc[pidx * kD + e] = v;
    }
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
  // with few splits (a.fuse) the last work-group of this kv head to finish
  // combines every split's partial with the window's and writes the output
  // rows; otherwise the finalize kernel does
  if (a.fuse && arrive_last<kThreads>(a.ctr + static_cast<int64_t>(b) * k.Hkv + h, nsplit, &fflag))
    finalize_bh<kThreads, G>(a, t, k, b, h, 0, red, endbuf, fsm[0], fsm[1], nullptr, nullptr, nullptr,
                             slot - split, nsplit);
}

template <int G, int BK, int BV, bool KMIX, bool VMIX>
const void* pick_bits(bool qjl, bool n8) {
  if (n8)
    return qjl ? reinterpret_cast<const void*>(&scan_mfma_kernel<G, BK, BV, true, KMIX, VMIX, true>)
               : reinterpret_cast<const void*>(&scan_mfma_kernel<G, BK, BV, false, KMIX, VMIX, true>);
  return qjl ? reinterpret_cast<const void*>(&scan_mfma_kernel<G, BK, BV, true, KMIX, VMIX, false>)
             : reinterpret_cast<const void*>(&scan_mfma_kernel<G, BK, BV, false, KMIX, VMIX, false>);
}

// mixed-channel rates exist for 2.5 and 3.5 bits (low width 2 or 3)
template <int G, int BK, bool KMIX>
const void* pick_bv(int bv, bool vmix, bool qjl, bool n8) {
  if (vmix) {
    if (bv == 2) return pick_bits<G, BK, 2, KMIX, true>(qjl, n8);
    if (bv == 3) return pick_bits<G, BK, 3, KMIX, true>(qjl, n8);
    return nullptr;
  }
  if (bv == 2) return pick_bits<G, BK, 2, KMIX, false>(qjl, n8);
  if (bv == 3) return pick_bits<G, BK, 3, KMIX, false>(qjl, n8);
  return pick_bits<G, BK, 4, KMIX, false>(qjl, n8);
}

template <int G>
const void* pick_g(int bk, bool kmix, int bv, bool vmix, bool qjl, bool n8) {
  if (kmix) {
    if (bk == 2) return pick_bv<G, 2, true>(bv, vmix, qjl, n8);
    if (bk == 3) return pick_bv<G, 3, true>(bv, vmix, qjl, n8);
    return nullptr;
  }
  if (bk == 2) return pick_bv<G, 2, false>(bv, vmix, qjl, n8);
  if (bk == 3) return pick_bv<G, 3, false>(bv, vmix, qjl, n8);
  return pick_bv<G, 4, false>(bv, vmix, qjl, n8);
}

}  // namespace

const void* scan_mfma_kernel_ptr(const tq_ctx* c) {
  const int G = c->p.num_q_heads / c->p.num_kv_heads, bk = c->p.key_bits, bv = c->p.value_bits;
  const bool qjl = c->p.key_qjl != 0, kmix = c->p.key_mixed != 0, vmix = c->p.value_mixed != 0;
  const bool n8 = c->p.key_norm_u8 != 0;
  switch (G) {
    case 1: return pick_g<1>(bk, kmix, bv, vmix, qjl, n8);
    case 2: return pick_g<2>(bk, kmix, bv, vmix, qjl, n8);
    case 4: return pick_g<4>(bk, kmix, bv, vmix, qjl, n8);
    case 8: return pick_g<8>(bk, kmix, bv, vmix, qjl, n8);
    default: return nullptr;
  }
}

int scan_mfma_threads(const tq_ctx* c) {
  return scan_threads(c->p.value_bits, c->p.key_mixed != 0, c->p.value_mixed != 0);
}

int launch_scan_mfma(const tq_ctx* c, const DecodeArgs& a, const KParams& k, void* stream, void* ev0, void* ev1) {
  const void* f = scan_mfma_kernel_ptr(c);
  if (!f) return 1;
  DecodeArgs aa = a;
  DevTables tt = c->t;
  Codebooks cc = c->cb;
  KParams kk = k;
  void* args[] = {&aa, &tt, &cc, &kk};
  const dim3 grid = a.plan ? dim3(a.nwg) : dim3(a.splits, k.Hkv, a.batch);
  return hipExtLaunchKernel(f, grid, dim3(scan_mfma_threads(c)), args, 0, static_cast<hipStream_t>(stream),
                            static_cast<hipEvent_t>(ev0), static_cast<hipEvent_t>(ev1), 0) == hipSuccess
             ? 0
             : 1;
}

}  // namespace tq
