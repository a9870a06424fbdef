// Encode kernels: flat records (tq_encode) and paged append (tq_append_page).
//
// Per vector x ("aither-kvcache" README, section "Algorithm"; keys' residual
// sketch from "TurboQuant on a 16GB MacBook", sections "Why this caught my
// eye" and "The QJL detective story"):
//   n = ||x|| (accumulated in double, stored f32); y = Pi x / n;
//   code_j = #{k : y_j > boundary_k} (ties to the lower index);
//   keys: r = Pi x - n c[code], ||r||, sign bit j = [(S r)_j >= 0].
// A work-group of 128 threads (thread = coordinate) handles a tile of 32
// vectors held in LDS; rotations are fp32 VALU matrix-vector products with the
// matrix row in registers and the tile broadcast from LDS, or sign flips plus
// Walsh-Hadamard butterflies (wave shuffles, one LDS exchange for stride 64)
// for the Hadamard variant; sign bits come from wave ballots.
#include "device_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kTile = 32;
constexpr int kThreads = 128;

struct Smem {
  float xs[kTile][kD];   // input tile (f32)
  float rs[kTile][kD];   // residuals / butterfly scratch
  uint8_t code[kTile][kD];
  float n32[kTile], invn[kTile], rn[kTile];
  float nst[kTile];    // the stored norm: n32, or the u8 log-norm level
  int nq[kTile];       // u8 log-norm code
  uint32_t sgn[kTile][4];
  float ctab[32];  // centroids; [16, 32): the (b+1)-bit codebook of a mixed rate
};

struct CoreParams {
  int bits;
  bool qjl;
  bool n8;         // the norm is stored as a u8 log-norm code (keys)
  int hmod;        // mixed-channel rate: coordinate j takes bits + 1 when j mod hmod >= hmod/2; 0: integer rate
  float bnd[16];   // decision boundaries (uniform values)
  float cen[16];   // centroids
  float bnd2[16];  // the (bits+1)-bit codebook of a mixed rate
  float cen2[16];
};

__device__ inline CoreParams make_core(const Codebooks& cb, bool key, int bits, bool qjl, bool mixed,
                                       bool n8 = false) {
  CoreParams cp;
  cp.bits = bits;
  cp.qjl = qjl;
  cp.n8 = n8;
  cp.hmod = mixed ? (key ? kKeyHiMod : kValHiMod) : 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    cp.bnd[k] = key ? cb.kb[k] : cb.vb[k];
    cp.cen[k] = key ? cb.kc[k] : cb.vc[k];
    cp.bnd2[k] = key ? cb.kb2[k] : cb.vb2[k];
    cp.cen2[k] = key ? cb.kc2[k] : cb.vc2[k];
  }
  return cp;
}

// Rotate, quantise and (for keys) sketch the residual of the tile in LDS.
// Only vectors v0 <= v < v1 of the tile are encoded (the others are not
// written by the callers).
template <bool HAD>
__device__ void encode_core(Smem& sm, const DevTables& t, const CoreParams& cp, int v0, int v1) {
  const int tid = threadIdx.x;
  // this thread's coordinate (tid) and its codebook
  const bool hi = cp.hmod != 0 && mixed_hi(tid, cp.hmod);
  const int nb = (1 << (cp.bits + (hi ? 1 : 0))) - 1;
  if (tid < 32) {
    float cv = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k == tid) cv = cp.cen[k];
      if (k + 16 == tid) cv = cp.cen2[k];
    }
    sm.ctab[tid] = cv;
  }
  // norms in double: thread t sums a quarter of vector t/4
  {
    const int v = tid >> 2, part = tid & 3;
    double s = 0.0;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const double e = sm.xs[v][part * 32 + j];
      s = fma(e, e, s);
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (part == 0) {
      const double n = sqrt(s);
      const float n32 = static_cast<float>(n);
      sm.n32[v] = n32;
      sm.invn[v] = n > 0.0 ? static_cast<float>(1.0 / n) : 0.0f;
      float nst = n32;
      if (cp.n8) {
        const int q = norm_code(n32, t.ntab + kNormCodes);
        sm.nq[v] = q;
        nst = t.ntab[q];
      }
      sm.nst[v] = nst;
    }
  }
  __syncthreads();
  // quantise one vector's coordinate (this thread's) and keep the key
  // residual against the stored reconstruction nst c[code]
  auto finish = [&](int v, float accv) {
    const float n = sm.nst[v];
    const float y = accv * sm.invn[v];
    int c = 0;
#pragma unroll
    for (int k = 0; k < 15; ++k)
      if (k < nb) c += (y > (hi ? cp.bnd2[k] : cp.bnd[k])) ? 1 : 0;
    if (!(n > 0.0f)) c = 0;
    sm.code[v][tid] = static_cast<uint8_t>(c);
    if (cp.qjl) sm.rs[v][tid] = (n > 0.0f) ? fmaf(-n, sm.ctab[(hi ? 16 : 0) + c], accv) : 0.0f;
  };
  if constexpr (!HAD) {
    // two passes over halves of the rotation row keep the register count
    // low; the first pass parks its partial sums in this thread's rs slots
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      float pr[kD / 2];
#pragma unroll
      for (int j = 0; j < kD / 2; ++j) pr[j] = t.rotT[(hp * (kD / 2) + j) * kD + tid];
#pragma unroll 1
      for (int v = v0; v < v1; ++v) {
        float s = hp ? sm.rs[v][tid] : 0.0f;
        {
          const float4* xr = reinterpret_cast<const float4*>(sm.xs[v]) + hp * (kD / 8);
#pragma unroll
          for (int j4 = 0; j4 < kD / 8; ++j4) {
            const float4 x = xr[j4];
            s = fmaf(pr[4 * j4 + 0], x.x, s);
            s = fmaf(pr[4 * j4 + 1], x.y, s);
            s = fmaf(pr[4 * j4 + 2], x.z, s);
            s = fmaf(pr[4 * j4 + 3], x.w, s);
          }
        }
        if (hp == 0)
          sm.rs[v][tid] = s;
        else
          finish(v, s);
      }
    }
  } else {
    const float eps = t.rot[tid];
    // strides 1..32 inside the wave, stride 64 through LDS
    for (int v = v0; v < v1; ++v) {
      float val = sm.xs[v][tid] * eps;
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const float o = __shfl_xor(val, s, 64);
        val = (tid & s) ? (o - val) : (val + o);
      }
      sm.rs[v][tid] = val;
    }
    __syncthreads();
    float acc[kTile];
    const float inv_sqrt_d = 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
    for (int v = 0; v < kTile; ++v) {
      const float a = sm.rs[v][tid], b = sm.rs[v][tid ^ 64];
      acc[v] = ((tid & 64) ? (b - a) : (a + b)) * inv_sqrt_d;
    }
    __syncthreads();
#pragma unroll
    for (int v = 0; v < kTile; ++v)
      if (v >= v0 && v < v1) finish(v, acc[v]);
  }
  if (!cp.qjl) return;
  __syncthreads();
  {
    const int v = tid >> 2, part = tid & 3;
    double s = 0.0;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
      const double e = sm.rs[v][part * 32 + j];
      s = fma(e, e, s);
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (part == 0) sm.rn[v] = static_cast<float>(sqrt(s));
  }
  const int wave = tid >> 6, lane = tid & 63;
  __syncthreads();  // xs is free from here on: it holds the first half of S r
#pragma unroll
  for (int hp = 0; hp < 2; ++hp) {
    float sr[kD / 2];
#pragma unroll
    for (int j = 0; j < kD / 2; ++j) sr[j] = t.ST[(hp * (kD / 2) + j) * kD + tid];
#pragma unroll 1
    for (int v = v0; v < v1; ++v) {
      float z = hp ? sm.xs[v][tid] : 0.0f;
      const float4* rr = reinterpret_cast<const float4*>(sm.rs[v]) + hp * (kD / 8);
#pragma unroll
      for (int j4 = 0; j4 < kD / 8; ++j4) {
        const float4 r = rr[j4];
        z = fmaf(sr[4 * j4 + 0], r.x, z);
        z = fmaf(sr[4 * j4 + 1], r.y, z);
        z = fmaf(sr[4 * j4 + 2], r.z, z);
        z = fmaf(sr[4 * j4 + 3], r.w, z);
      }
      if (hp == 0) {
        sm.xs[v][tid] = z;
      } else {
        const bool bit = (z >= 0.0f) && (sm.n32[v] > 0.0f);
        const uint64_t m = __ballot(bit);
        if (lane == 0) {
          sm.sgn[v][2 * wave] = static_cast<uint32_t>(m);
          sm.sgn[v][2 * wave + 1] = static_cast<uint32_t>(m >> 32);
        }
      }
    }
  }
}

// Word w (32 bits) of the LSB-first stream of n codes of `bits` bits each,
// the i-th being code(i).
template <class F>
__device__ inline uint32_t stream_word(F code, int n, int w, int bits) {
  const int first = (32 * w) / bits;
  const int base = first * bits;
  uint64_t acc = 0;
  for (int c = first; c < n && c * bits < 32 * w + 32; ++c) acc |= static_cast<uint64_t>(code(c)) << (c * bits - base);
  return static_cast<uint32_t>(acc >> (32 * w - base));
}

// Word w of vector v's record: the d codes LSB-first, or for a mixed rate
// (hmod != 0) the d/2 low-rate codes at `bits` bits, then the d/2 high-rate
// codes at bits + 1, each half in ascending coordinate order.
template <class SM>
__device__ inline uint32_t code_word(const SM& sm, int v, int w, int bits, int hmod) {
  if (hmod == 0) return stream_word([&](int c) { return sm.code[v][c]; }, kD, w, bits);
  const int lo_words = (kD / 2) * bits / 32;
  if (w < lo_words)
    return stream_word([&](int r) { return sm.code[v][mixed_coord(r, 0, hmod)]; }, kD / 2, w, bits);
  return stream_word([&](int r) { return sm.code[v][mixed_coord(r, 1, hmod)]; }, kD / 2, w - lo_words, bits + 1);
}

template <bool HAD>
__global__ __launch_bounds__(kThreads) void encode_flat_kernel(EncodeArgs a, DevTables t, Codebooks cb, int kind,
                                                              int dtype, int bits, int qjl, int mixed, int n8) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int nv = static_cast<int>(a.n - n0 < kTile ? a.n - n0 : kTile);
  // rows of d coordinates, zero-padded to kD
  for (int v = 0; v < kTile; ++v)
    sm.xs[v][tid] = (v < nv && tid < a.d) ? load_any(a.x, (n0 + v) * a.row_stride + tid, dtype) : 0.0f;
  __syncthreads();
  const CoreParams cp = make_core(cb, kind == TQ_KIND_KEY, bits, qjl != 0, mixed != 0, n8 != 0);
  encode_core<HAD>(sm, t, cp, 0, nv);
  __syncthreads();
  if (tid < nv) {
    a.norms[n0 + tid] = sm.nst[tid];
    if (qjl) a.rnorms[n0 + tid] = sm.rn[tid];
  }
  const int wpv = 4 * bits + (mixed ? 2 : 0);  // 32-bit words per record (d = 128)
  uint32_t* cw = reinterpret_cast<uint32_t*>(a.codes);
  for (int k = tid; k < nv * wpv; k += kThreads) {
    const int v = k / wpv, w = k % wpv;
    cw[(n0 + v) * wpv + w] = code_word(sm, v, w, bits, cp.hmod);
  }
  if (qjl) {
    uint32_t* sw = reinterpret_cast<uint32_t*>(a.signs);
    if (tid < 4 * nv) sw[(n0 + (tid >> 2)) * 4 + (tid & 3)] = sm.sgn[tid >> 2][tid & 3];
  }
}

// ---------------------------------------------------------------------------
// Append.  For sequence b: T0 = seq_lens[b], T1 = T0 + count; the tokens at
// positions [max(T0-W,0), max(T1-W,0)) leave the FP16 window and are encoded
// into their pages (from the ring if they were already cached, else from the
// new input), the new tokens that stay within the last W go to the ring, and
// seq_lens[b] becomes T1 ("TurboQuant Family Design Study", sections "Packed
// format and complete bit accounting" (recent FP16 window, fixed pages) and
// "Paging, lifecycle, and cache identity" (fixed-page append, rollback)).
// A sequence with an invalid count or page id is left untouched.

struct SeqPlan {
  int T0, cnt, c0, c1;
  bool ok;
};

// Called by every thread of the work-group (it ends with a barrier): the
// page ids are checked by all threads at once, since a check that stops at
// the first bad page waits a round trip per page.
__device__ inline SeqPlan plan_seq(const AppendArgs& a, const Layout& L, int W, int b) {
  SeqPlan s;
  s.T0 = a.seq_lens[b];
  s.cnt = a.counts ? a.counts[b] : a.n_new;
  bool ok = !(s.cnt < 0 || s.cnt > a.n_new || s.T0 < 0);
  const int T1 = s.T0 + s.cnt;
  s.c0 = ok && s.T0 - W > 0 ? s.T0 - W : 0;
  s.c1 = ok && T1 - W > 0 ? T1 - W : 0;
  if (ok && s.c1 > s.c0) {
    const int pg0 = s.c0 / L.P, pg1 = (s.c1 - 1) / L.P;
    ok = pg1 < a.max_pages;
    for (int pg = pg0 + static_cast<int>(threadIdx.x); ok && pg <= pg1; pg += static_cast<int>(blockDim.x)) {
      const int pid = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg];
      if (pid < 0 || pid >= a.num_pages) ok = false;
    }
  }
  s.ok = __syncthreads_and(ok) != 0;
  return s;
}

// New tokens that remain among the last W go to the FP16 ring.  With at most
// W new tokens, token q either evicts q - W from its slot, and is written by
// the work-group that encodes q - W (after that one has read the slot), or
// evicts nothing and is written by the first work-group; no slot is read by
// one work-group and written by another.
__device__ inline void ring_owned(const AppendArgs& a, const SeqPlan& sp, int W, int d, int64_t bh, int kv, int gr,
                                  int tid) {
  const int j0 = sp.cnt > W ? sp.cnt - W : 0;
  const int g0 = sp.c0 / kVGroup;
  if (tid >= d) return;  // rows hold d coordinates
  for (int j = j0; j < sp.cnt; ++j) {
    const int q = sp.T0 + j;
    if ((q >= W ? (q - W) / kVGroup - g0 : 0) != gr) continue;
    if (kv == 0)
      a.k_win[(bh * W + q % W) * d + tid] = a.k_new[(bh * a.n_new + j) * d + tid];
    else
      a.v_win[(bh * W + q % W) * d + tid] = a.v_new[(bh * a.n_new + j) * d + tid];
  }
}

// Encode the evicted tokens of one 32-token group of sequence b, head h.
template <bool HAD>
__device__ void encode_group(Smem& sm, const AppendArgs& a, const DevTables& t, const Codebooks& cb, const Layout& L,
                             int W, const SeqPlan& sp, int b, int h, int kv, int gpos) {
  const int tid = threadIdx.x;
  const int lo = sp.c0 > gpos ? sp.c0 : gpos;
  const int hi = sp.c1 < gpos + kVGroup ? sp.c1 : gpos + kVGroup;
  const int pg = gpos / L.P, slot0 = gpos % L.P;
  const int pid = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg];
  uint8_t* hb = a.pool + static_cast<int64_t>(pid) * L.page_bytes + kBodyOffset + static_cast<int64_t>(h) * L.head_bytes;
  const int64_t bh = static_cast<int64_t>(b) * L.H + h;
  {
    const uint16_t* win = kv == 0 ? a.k_win : a.v_win;
    const uint16_t* src = kv == 0 ? a.k_new : a.v_new;
    for (int v = 0; v < kTile; ++v) {
      const int pos = gpos + v;
      float x = 0.0f;  // (coordinates past d: zero padding)
      if (pos >= lo && pos < hi && tid < L.d) {
        const uint16_t bits = pos < sp.T0 ? win[(bh * W + pos % W) * L.d + tid]
                                          : src[(bh * a.n_new + (pos - sp.T0)) * L.d + tid];
        x = half_bits_to_float(bits);
      }
      sm.xs[v][tid] = x;
    }
    __syncthreads();
    const bool key = kv == 0;
    const CoreParams cp = make_core(cb, key, key ? L.bK : L.bV, key && L.qjl, key ? L.kmix : L.vmix, key && L.kn8);
    const int vlo = lo - gpos, vhi = hi - gpos;
    encode_core<HAD>(sm, t, cp, vlo, vhi);
    __syncthreads();
    if (key) {
      if (tid >= vlo && tid < vhi) {
        if (L.kn8)
          (hb + L.k_norm)[slot0 + tid] = static_cast<uint8_t>(sm.nq[tid]);
        else
          reinterpret_cast<float*>(hb + L.k_norm)[slot0 + tid] = sm.n32[tid];
        if (L.qjl) reinterpret_cast<float*>(hb + L.k_rnorm)[slot0 + tid] = sm.rn[tid];
      }
      const int wpv = L.k_rec / 4;
      uint32_t* cw = reinterpret_cast<uint32_t*>(hb + L.k_codes);
      for (int k = tid; k < kTile * wpv; k += kThreads) {
        const int v = k / wpv, w = k % wpv;
        if (v >= vlo && v < vhi) cw[(slot0 + v) * wpv + w] = code_word(sm, v, w, L.bK, cp.hmod);
      }
      if (L.qjl) {
        uint32_t* sw = reinterpret_cast<uint32_t*>(hb + L.k_signs);
        const int v = tid >> 2;
        if (v >= vlo && v < vhi) sw[(slot0 + v) * 4 + (tid & 3)] = sm.sgn[v][tid & 3];
      }
    } else {
      float* vn = reinterpret_cast<float*>(hb + L.v_norm);
      if (tid >= vlo && tid < vhi) vn[slot0 + tid] = sm.n32[tid];
      // group-interleaved value codes: coordinate tid, words w = 0..width-1
      // (mixed rate: a low-rate block [bV][d/2], then a high-rate block [bV+1][d/2])
      uint32_t* gw = reinterpret_cast<uint32_t*>(hb + L.v_codes) + static_cast<int64_t>(slot0 / kVGroup) * 8 * L.v_rec;
      const bool hi = L.vmix && mixed_hi(tid, kValHiMod);
      const int width = L.bV + (hi ? 1 : 0);
      const int stride = L.vmix ? kD / 2 : kD;
      const int at0 = L.vmix ? (hi ? L.bV * (kD / 2) : 0) + mixed_rank(tid, kValHiMod) : tid;
      // bits of tokens not yet written are left zero
#pragma unroll
      for (int w = 0; w < 5; ++w) {
        if (w >= width) break;
        const int keep = vhi * width - 32 * w;  // stream bits of word w below this belong to tokens < vhi
        uint32_t word = vlo == 0 || keep <= 0 ? 0u : gw[at0 + w * stride];
        if (keep < 32) word &= keep > 0 ? (1u << keep) - 1u : 0u;
        for (int v = vlo; v < vhi; ++v) {
          const uint32_t c = sm.code[v][tid];
          for (int k = 0; k < width; ++k) {
            const int p = v * width + k;
            if ((p >> 5) == w) {
              const uint32_t m = 1u << (p & 31);
              word = (word & ~m) | (((c >> k) & 1u) << (p & 31));
            }
          }
        }
        gw[at0 + w * stride] = word;
      }
    }
    __syncthreads();
  }
}

// kinds: bit 0 keys, bit 1 values (the kinds the matrix-core append does not take)
template <bool HAD>
__global__ __launch_bounds__(kThreads) void append_encode_kernel(AppendArgs a, DevTables t, Codebooks cb, Layout L,
                                                                int W, int ring, int kinds) {
  __shared__ Smem sm;
  const int tid = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  // every work-group of b evaluates the same plan; the commit kernel reports
  const SeqPlan sp = plan_seq(a, L, W, b);
  if (!sp.ok) return;
  const int kv = static_cast<int>(blockIdx.x & 1u);  // 0: keys, 1: values
  const int gr = static_cast<int>(blockIdx.x >> 1);
  const int g = sp.c0 / kVGroup + gr;
  const int gpos = g * kVGroup;
  if (sp.c1 > sp.c0 && gpos < sp.c1 && ((kinds >> kv) & 1)) encode_group<HAD>(sm, a, t, cb, L, W, sp, b, h, kv, gpos);
  if (ring) ring_owned(a, sp, W, L.d, static_cast<int64_t>(b) * L.H + h, kv, gr, tid);
}

// ------------------------------------------------------------ few-token append
// Appends of at most kSmallNew tokens per sequence (decode steps) are a chain
// of dependent memory round trips, not a throughput problem: sequence length
// -> window slot and page id -> existing value words.  One work-group of 256
// threads per (sequence, kv head, keys|values) encodes the (at most
// kSmallNew) tokens that leave the window.  Threads 0..127 own coordinate i =
// tid for the rotation and quantiser and hold row i of Pi in registers;
// threads 128..255 own coordinate i = tid - 128 for the norms and the sign
// sketch and hold row i of S.  Both rows are requested before the sequence
// plan, from tables interleaved so that each lane reads 16 contiguous bytes
// ((j/4, i) -> M[i][4(j/4) .. 4(j/4)+3]), and land while the plan and the
// window slots are read.  Every sum is taken in the same order as in the bulk
// kernel above, so one-token and bulk appends write identical bytes.
constexpr int kSmallNew = 4;
constexpr int kSmallThreads = 256;

struct SmallSmem {
  float xs[kSmallNew][kD];   // inputs
  float rs[kSmallNew][kD];   // key residuals in the rotated basis
  float hx[kSmallNew][kD];   // Hadamard stride-64 exchange
  uint8_t code[kSmallNew][kD];
  float n32[kSmallNew], invn[kSmallNew], rn[kSmallNew];
  float nst[kSmallNew];  // the stored norm: n32, or the u8 log-norm level
  int nq[kSmallNew];     // u8 log-norm code
  uint32_t sgn[kSmallNew][4];
  float cbt[64];  // this kind's centroids, boundaries, and the (b+1)-bit ones of a mixed rate
  float ntab[2 * kNormCodes];  // u8 log-norm levels, then boundaries
};

// Double-precision squared norm of row v of `x` as the bulk kernel takes it:
// four partial sums over 32 consecutive coordinates, combined pairwise.
// Called by 16 consecutive lanes of one wave (lane l: vector l >> 2, part l & 3).
__device__ inline double sq_norm_quarters(const float (*x)[kD], int l) {
  const int v = l >> 2, part = l & 3;
  double s = 0.0;
#pragma unroll 8
  for (int j = 0; j < 32; ++j) {
    const double e = x[v][part * 32 + j];
    s = fma(e, e, s);
  }
  s += __shfl_xor(s, 1, 64);
  s += __shfl_xor(s, 2, 64);
  return s;
}

// What the commit of sequence b reads: the plan as plan_seq takes it (both
// per-sequence words, then the ids of the first two pages: a decode step
// touches one page, at most two).
struct CommitLoads {
  int T0, craw, pa, pb;
};

// The append of one (keys | values, kv head, sequence); cl receives the words
// a commit of the sequence reads, as this work-group read them.
template <bool HAD>
__device__ __forceinline__ void append_small_body(const AppendArgs& a, const DevTables& t, const Layout& L, int W,
                                                  int ring, SmallSmem& sm, CommitLoads& cl) {
  const int tid = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int i = tid & (kD - 1), lane = tid & 63;
  const bool lower = tid < kD;
  const bool key = blockIdx.x == 0;
  const bool qjl = key && L.qjl;

  // the plan's two words and this kind's codebook are requested first; the
  // codebook goes to LDS while nothing else is in flight (loads complete in
  // order, so a later wait for it would also wait for the tables), then the
  // table rows, which land while the window slots are read
  const int T0 = a.seq_lens[b];
  int cnt = a.n_new;
  if (a.counts != nullptr) cnt = a.counts[b];
  cl.T0 = T0;
  cl.craw = cnt;
  cl.pa = cl.pb = -1;
  const float cbv = t.cbtab[(key ? 0 : 64) + (tid & 63)];
  const float nt0 = t.ntab[tid], nt1 = t.ntab[kNormCodes + tid];
  if (tid < 64) sm.cbt[tid] = cbv;
  sm.ntab[tid] = nt0;
  sm.ntab[kNormCodes + tid] = nt1;
  // (every thread loads a table, used or not: loads under a branch leave the
  // compiler's wait counting at later uses conservative, i.e. full drains;
  // threads without a row of their own read Pi's, which their wave's other
  // half reads anyway, or a zero table for the Hadamard rotation)
  float4 row[kD / 4];
  const float4* tab = reinterpret_cast<const float4*>(!lower && qjl ? t.S4 : t.rot4);
#pragma unroll
  for (int j4 = 0; j4 < kD / 4; ++j4) row[j4] = tab[j4 * kD + i];
  if (cnt < 0 || cnt > a.n_new || T0 < 0) return;  // reported by the commit kernel
  const int c0 = T0 - W > 0 ? T0 - W : 0;
  const int T1 = T0 + cnt;
  const int c1 = T1 - W > 0 ? T1 - W : 0;
  const int nv = c1 - c0;  // tokens leaving the window: 0 .. kSmallNew
  const int64_t bh = static_cast<int64_t>(b) * L.H + h;
  const uint16_t* win = key ? a.k_win : a.v_win;
  const uint16_t* src = key ? a.k_new : a.v_new;
  uint16_t* wdst = key ? a.k_win : a.v_win;
  // new tokens bound for the ring (the last W of them), loaded now and
  // stored once this thread has read the slots they overwrite
  // (loads in this kernel are unconditional, from clamped indices: a load
  // under a branch makes the branch's join wait for every load in flight)
  const int j0 = cnt > W ? cnt - W : 0;
  // FP16 rows hold d coordinates: threads of coordinates past d read
  // coordinate 0 (discarded) and take zero padding
  const int d = L.d;
  const bool live = i < d;
  const int ic = live ? i : 0;
  uint16_t rnew[kSmallNew];
  if (ring && lower && cnt > 0) {
#pragma unroll
    for (int j = 0; j < kSmallNew; ++j) rnew[j] = src[(bh * a.n_new + (j0 + j < cnt ? j0 + j : cnt - 1)) * d + ic];
  }
  int pid0 = 0, pid1 = 0;
  if (nv > 0) {
    const int pg0 = c0 / L.P, pg1 = (c1 - 1) / L.P;
    if (pg1 >= a.max_pages) return;
    pid0 = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg0];
    pid1 = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg1];
    cl.pa = pid0;
    cl.pb = pid1;  // (the commit takes it only when pg1 = pg0 + 1)
    if (pid0 < 0 || pid0 >= a.num_pages || pid1 < 0 || pid1 >= a.num_pages) return;
  }
  if (nv > 0 && lower) {
    uint16_t xr[kSmallNew];
#pragma unroll
    for (int v = 0; v < kSmallNew; ++v) {
      const int pos = c0 + (v < nv ? v : nv - 1);
      const uint16_t* p = pos < T0 ? win + (bh * W + pos % W) * d : src + (bh * a.n_new + (pos - T0)) * d;
      xr[v] = p[ic];
    }
#pragma unroll
    for (int v = 0; v < kSmallNew; ++v) sm.xs[v][i] = (v < nv && live) ? half_bits_to_float(xr[v]) : 0.0f;
  }
  auto ring_store = [&]() {
    if (ring && lower && live) {
#pragma unroll
      for (int j = 0; j < kSmallNew; ++j)
        if (j0 + j < cnt) wdst[(bh * W + (T0 + j0 + j) % W) * d + i] = rnew[j];
    }
  };
  if (nv == 0) {  // nothing leaves the window: no slot is read
    ring_store();
    return;
  }

  // page addresses of the (at most two) pages and groups the tokens touch
  auto head_base = [&](int pos) {
    const int pid = pos / L.P == c0 / L.P ? pid0 : pid1;
    return a.pool + static_cast<int64_t>(pid) * L.page_bytes + kBodyOffset + static_cast<int64_t>(h) * L.head_bytes;
  };
  const int bits = key ? L.bK : L.bV;
  const int hmod = (key ? L.kmix : L.vmix) ? (key ? kKeyHiMod : kValHiMod) : 0;
  const bool hi = hmod != 0 && mixed_hi(i, hmod);
  const int width = bits + (hi ? 1 : 0);
  // value words hold 32 tokens' codes: the new tokens' bits are stored into
  // a group's first word outright (later tokens are not valid yet) or
  // cleared and set with two no-return atomics (same thread, same word: they
  // take effect in program order), without reading the word
  const int ga = c0 / kVGroup, gb = (c1 - 1) / kVGroup;  // first and last group
  const int vstride = L.vmix ? kD / 2 : kD;
  const int vat0 = L.vmix ? (hi ? L.bV * (kD / 2) : 0) + mixed_rank(i, kValHiMod) : i;
  const int nb = (1 << width) - 1;
  const float* cen = sm.cbt + (hi ? 32 : 0);
  const float* bnd = sm.cbt + (hi ? 48 : 16);
  lds_barrier();  // (1) inputs in LDS

  // norms (upper wave 0) while the lower threads rotate
  float acc[kSmallNew];
  if (!lower) {
    const int l = tid - kD;
    if (l < 4 * kSmallNew) {
      const double sq = sq_norm_quarters(sm.xs, l);
      const int v = l >> 2;
      if ((l & 3) == 0 && v < nv) {
        const double n = sqrt(sq);
        const float n32 = static_cast<float>(n);
        sm.n32[v] = n32;
        sm.invn[v] = n > 0.0 ? static_cast<float>(1.0 / n) : 0.0f;
        float nst = n32;
        if (key && L.kn8) {
          const int q = norm_code(n32, sm.ntab + kNormCodes);
          sm.nq[v] = q;
          nst = sm.ntab[q];
        }
        sm.nst[v] = nst;
      }
    }
  } else if constexpr (!HAD) {
#pragma unroll
    for (int v = 0; v < kSmallNew; ++v) {
      float s = 0.0f;
      if (v < nv) {
        const float4* xr = reinterpret_cast<const float4*>(sm.xs[v]);
#pragma unroll
        for (int j4 = 0; j4 < kD / 4; ++j4) {
          const float4 x = xr[j4];
          s = fmaf(row[j4].x, x.x, s);
          s = fmaf(row[j4].y, x.y, s);
          s = fmaf(row[j4].z, x.z, s);
          s = fmaf(row[j4].w, x.w, s);
        }
      }
      acc[v] = s;
    }
  } else {
    // randomised Hadamard: strides 1..32 in the wave, 64 through LDS
    const float eps = t.rot[i];
#pragma unroll
    for (int v = 0; v < kSmallNew; ++v) {
      if (v >= nv) break;
      float val = sm.xs[v][i] * eps;
#pragma unroll
      for (int st = 1; st < 64; st <<= 1) {
        const float o = __shfl_xor(val, st, 64);
        val = (i & st) ? (o - val) : (val + o);
      }
      sm.hx[v][i] = val;
    }
  }
  lds_barrier();  // (2) norms (and Hadamard halves) in LDS
  if (lower) {
    if constexpr (HAD) {
      const float inv_sqrt_d = 0.08838834764831845f;  // 1/sqrt(128)
#pragma unroll
      for (int v = 0; v < kSmallNew; ++v) {
        const float p = sm.hx[v][i], q = sm.hx[v][i ^ 64];
        acc[v] = ((i & 64) ? (q - p) : (p + q)) * inv_sqrt_d;
      }
    }
    // quantise this coordinate of each vector and keep the key residual
#pragma unroll
    for (int v = 0; v < kSmallNew; ++v) {
      if (v >= nv) break;
      const float n = sm.nst[v];  // the residual is taken against the stored norm
      const float y = acc[v] * sm.invn[v];
      int c = 0;
#pragma unroll
      for (int k = 0; k < 15; ++k)
        if (k < nb) c += (y > bnd[k]) ? 1 : 0;
      if (!(n > 0.0f)) c = 0;
      sm.code[v][i] = static_cast<uint8_t>(c);
      if (qjl) sm.rs[v][i] = (n > 0.0f) ? fmaf(-n, cen[c], acc[v]) : 0.0f;
    }
  }
  lds_barrier();  // (3) codes and residuals in LDS

  if (key) {
    if (qjl && !lower) {
      // ||r|| (upper wave 0) and the sign sketch: bit i = [(S r)_i >= 0]
      const int l = tid - kD, wu = l >> 6;
      if (l < 4 * kSmallNew) {
        const double sq = sq_norm_quarters(sm.rs, l);
        if ((l & 3) == 0 && (l >> 2) < nv) sm.rn[l >> 2] = static_cast<float>(sqrt(sq));
      }
#pragma unroll 1
      for (int v = 0; v < nv; ++v) {
        float z = 0.0f;
        const float4* rr = reinterpret_cast<const float4*>(sm.rs[v]);
#pragma unroll
        for (int j4 = 0; j4 < kD / 4; ++j4) {
          const float4 r = rr[j4];
          z = fmaf(row[j4].x, r.x, z);
          z = fmaf(row[j4].y, r.y, z);
          z = fmaf(row[j4].z, r.z, z);
          z = fmaf(row[j4].w, r.w, z);
        }
        const bool bit = (z >= 0.0f) && (sm.n32[v] > 0.0f);
        const uint64_t m = __ballot(bit);
        if (lane == 0) {
          sm.sgn[v][2 * wu] = static_cast<uint32_t>(m);
          sm.sgn[v][2 * wu + 1] = static_cast<uint32_t>(m >> 32);
        }
      }
    }
    if (lower) {
      // records: code words and norms
      const int wpv = L.k_rec / 4;
      for (int k = tid; k < nv * wpv; k += kD) {
        const int v = k / wpv, w = k % wpv;
        const int pos = c0 + v;
        reinterpret_cast<uint32_t*>(head_base(pos) + L.k_codes)[(pos % L.P) * wpv + w] =
            code_word(sm, v, w, L.bK, hmod);
      }
      if (tid < nv) {
        if (L.kn8)
          (head_base(c0 + tid) + L.k_norm)[(c0 + tid) % L.P] = static_cast<uint8_t>(sm.nq[tid]);
        else
          reinterpret_cast<float*>(head_base(c0 + tid) + L.k_norm)[(c0 + tid) % L.P] = sm.n32[tid];
      }
    }
    if (qjl) {
      lds_barrier();  // (4) signs and ||r||
      const int v = tid >> 2;
      if (v < nv) {
        const int pos = c0 + v;
        reinterpret_cast<uint32_t*>(head_base(pos) + L.k_signs)[(pos % L.P) * 4 + (tid & 3)] = sm.sgn[v][tid & 3];
      }
      if (tid < nv) reinterpret_cast<float*>(head_base(c0 + tid) + L.k_rnorm)[(c0 + tid) % L.P] = sm.rn[tid];
    }
  } else if (lower) {
    if (tid < nv) reinterpret_cast<float*>(head_base(c0 + tid) + L.v_norm)[(c0 + tid) % L.P] = sm.n32[tid];
    // group-interleaved value words of coordinate i: token v of a group takes
    // bits [v width, (v + 1) width) of the stream over words 0 .. width-1
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (ga + q > gb) break;
      const int gpos = (ga + q) * kVGroup;
      const int lo = c0 > gpos ? c0 : gpos;
      const int hi_ = c1 < gpos + kVGroup ? c1 : gpos + kVGroup;
      uint32_t* gw = reinterpret_cast<uint32_t*>(head_base(gpos) + L.v_codes) +
                     static_cast<int64_t>((gpos % L.P) / kVGroup) * 8 * L.v_rec;
#pragma unroll
      for (int w = 0; w < 5; ++w) {
        if (w >= width) break;
        uint32_t bitsw = 0u, maskw = 0u;
        for (int pos = lo; pos < hi_; ++pos) {
          const int v = pos - gpos;
          const uint32_t c = sm.code[pos - c0][i];
          for (int k = 0; k < width; ++k) {
            const int p = v * width + k;
            if ((p >> 5) == w) {
              bitsw |= ((c >> k) & 1u) << (p & 31);
              maskw |= 1u << (p & 31);
            }
          }
        }
        uint32_t* wp = &gw[vat0 + w * vstride];
        if (lo == gpos) {
          *wp = bitsw;  // the group starts here
        } else if (maskw != 0u) {
          atomicAnd(wp, ~maskw);
          atomicOr(wp, bitsw);
        }
      }
    }
  }
  // the inputs are in LDS, so the slots they came from may be overwritten
  // (stored last: an earlier store would wait for the value words in flight)
  ring_store();
}

// What the commit writes into page headers besides the layout.
struct CommitInfo {
  int rotation;
  int qjl_code;  // 0 no QJL, 1 Gaussian S, 2 orthogonal S
  uint64_t seed;
};

// Words 4j .. 4j+3 of the 64-byte header of page pg (valid tokens `valid`).
__device__ inline uint4 header_words(const Layout& L, CommitInfo ci, int pg, int valid, int j) {
  switch (j) {
    case 0:
      // bits bytes: b, or b + 16 for a mixed-channel rate b + 1/2
      return make_uint4(kMagic, 1u | (static_cast<uint32_t>(L.d) << 16),
                        static_cast<uint32_t>(L.bK + 16 * L.kmix) | (static_cast<uint32_t>(ci.qjl_code) << 8) |
                            (static_cast<uint32_t>(L.bV + 16 * L.vmix) << 16) |
                            (static_cast<uint32_t>(ci.rotation) << 24),
                        static_cast<uint32_t>(L.H) | (static_cast<uint32_t>(L.P) << 16));
    case 1:
      return make_uint4(static_cast<uint32_t>(valid), 1u, static_cast<uint32_t>(ci.seed),
                        static_cast<uint32_t>(ci.seed >> 32));
    case 2:
      return make_uint4(static_cast<uint32_t>(pg), static_cast<uint32_t>(L.kn8), 0u, 0u);  // byte 36: key norm format
    default:
      return make_uint4(0u, 0u, 0u, 0u);
  }
}

// Commit of sequence b after its tokens are stored (cl: the words the append
// read, before any of them can change): check the count and the page ids as
// the append took them, rewrite the headers of the pages the append touched
// and advance seq_lens[b].  A bad count or page raises a status bit and
// leaves the sequence as it was.  One thread per sequence.
__device__ inline void commit_store(const AppendArgs& a, const DevTables& t, const Layout& L, int W, CommitInfo ci,
                                    int b, const CommitLoads& cl) {
  SeqPlan sp;
  sp.T0 = cl.T0;
  sp.cnt = a.counts ? cl.craw : a.n_new;
  if (sp.cnt < 0 || sp.cnt > a.n_new || sp.T0 < 0) {
    atomicOr(t.status, TQ_STATUS_BAD_COUNT);
    return;
  }
  const int T1 = sp.T0 + sp.cnt;
  sp.c0 = sp.T0 - W > 0 ? sp.T0 - W : 0;
  sp.c1 = T1 - W > 0 ? T1 - W : 0;
  const int pg0 = sp.c0 / L.P, pg1 = sp.c1 > sp.c0 ? (sp.c1 - 1) / L.P : pg0 - 1;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages;
  const int pa = cl.pa, pb = cl.pb;
  bool ok = sp.c1 <= sp.c0 || pg1 < a.max_pages;
  for (int pg = pg0; ok && pg <= pg1; ++pg) {
    const int pid = pg == pg0 ? pa : pg == pg0 + 1 ? pb : bt[pg];
    if (pid < 0 || pid >= a.num_pages) ok = false;
  }
  if (!ok) {
    atomicOr(t.status, TQ_STATUS_BAD_PAGE);
    return;
  }
  if (sp.c1 > sp.c0) {
    for (int pg = pg0; pg <= pg1; ++pg) {
      const int pid = pg == pg0 ? pa : pg == pg0 + 1 ? pb : bt[pg];
      uint4* hd = reinterpret_cast<uint4*>(a.pool + static_cast<int64_t>(pid) * L.page_bytes);
      const int valid = sp.c1 - pg * L.P < L.P ? sp.c1 - pg * L.P : L.P;
#pragma unroll
      for (int j = 0; j < 4; ++j) hd[j] = header_words(L, ci, pg, valid, j);
    }
  }
  a.seq_lens[b] = sp.T0 + sp.cnt;
}

// One work-group per (keys | values, kv head, sequence) appends at most
// kSmallNew tokens.  With a.ctr, the last of sequence b's 2 H work-groups to
// finish also commits it: every work-group counts its arrival once all its
// threads have read seq_lens[b], so the length is advanced only after its
// last reader (the count is cleared for the next call).  Without a.ctr a
// commit kernel follows.
template <bool HAD>
__global__ __launch_bounds__(kSmallThreads) void append_small_kernel(AppendArgs a, DevTables t, Layout L, int W,
                                                                    int ring, CommitInfo ci) {
  __shared__ SmallSmem sm;
  const int b = blockIdx.z;
  // the words the commit reads come from the append's own loads (taken
  // before any of them can change)
  CommitLoads cl;
  append_small_body<HAD>(a, t, L, W, ring, sm, cl);
  if (a.ctr == nullptr) return;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int n = 2 * static_cast<int>(gridDim.y);
    if (__hip_atomic_fetch_add(a.ctr + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1) {
      __hip_atomic_store(a.ctr + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      commit_store(a, t, L, W, ci, b, cl);
    }
  }
}


// New tokens that remain among the last W go to the FP16 ring, when the
// append of the sequence is valid (its count, and every page it touched:
// checked by all threads at once).  Rows of d fp16 values (d a multiple of
// 8) move as 16-byte pieces spread over the threads.
__global__ __launch_bounds__(kThreads) void append_ring_kernel(AppendArgs a, DevTables t, Layout L, int W) {
  const int tid = threadIdx.x, h = blockIdx.x, b = blockIdx.y;
  const int T0 = a.seq_lens[b];
  const int cnt = a.counts ? a.counts[b] : a.n_new;
  bool ok = !(cnt < 0 || cnt > a.n_new || T0 < 0);
  const int c0 = T0 - W > 0 ? T0 - W : 0;
  const int c1 = T0 + cnt - W > 0 ? T0 + cnt - W : 0;
  if (ok && c1 > c0) {
    const int pg0 = c0 / L.P, pg1 = (c1 - 1) / L.P;
    ok = pg1 < a.max_pages;
    for (int pg = pg0 + tid; ok && pg <= pg1; pg += kThreads) {
      const int pid = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg];
      if (pid < 0 || pid >= a.num_pages) ok = false;
    }
  }
  if (!__syncthreads_and(ok)) return;
  const int64_t bh = static_cast<int64_t>(b) * L.H + h;
  const int j0 = cnt > W ? cnt - W : 0;
  const int r16 = L.d / 8;  // 16-byte pieces per row
  const uint4* kn = reinterpret_cast<const uint4*>(a.k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(a.v_new);
  uint4* kw = reinterpret_cast<uint4*>(a.k_win);
  uint4* vw = reinterpret_cast<uint4*>(a.v_win);
  for (int e = tid; e < (cnt - j0) * r16; e += kThreads) {
    const int j = j0 + e / r16, c = e % r16;
    const int64_t dst = (bh * W + (T0 + j) % W) * r16 + c, src = (bh * a.n_new + j) * r16 + c;
    kw[dst] = kn[src];
    vw[dst] = vn[src];
  }
}

// Commit after a bulk append, one work-group per sequence b: check the
// count and every page id the append took, then rewrite the headers of those
// pages (four 16-byte stores each, spread over the threads) and advance
// seq_lens[b].  A bad count or page raises a status bit and leaves the
// sequence as it was.
constexpr int kCommitThreads = 256;

__global__ __launch_bounds__(kCommitThreads) void append_commit_kernel(AppendArgs a, DevTables t, Layout L, int W,
                                                                      CommitInfo ci) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int T0 = a.seq_lens[b];
  const int cnt = a.counts ? a.counts[b] : a.n_new;
  const bool bad_count = cnt < 0 || cnt > a.n_new || T0 < 0;
  const int T1 = T0 + cnt;
  const int c0 = T0 - W > 0 ? T0 - W : 0;
  const int c1 = T1 - W > 0 ? T1 - W : 0;
  const int pg0 = c0 / L.P, pg1 = c1 > c0 ? (c1 - 1) / L.P : pg0 - 1;
  const int32_t* bt = a.block_table + static_cast<int64_t>(b) * a.max_pages;
  bool ok = !bad_count && (c1 <= c0 || pg1 < a.max_pages);
  for (int pg = pg0 + tid; ok && pg <= pg1; pg += kCommitThreads) {
    const int pid = bt[pg];
    if (pid < 0 || pid >= a.num_pages) ok = false;
  }
  // (every thread has read seq_lens[b] before this barrier)
  ok = __syncthreads_and(ok) != 0;
  if (!ok) {
    if (tid == 0) atomicOr(t.status, bad_count ? TQ_STATUS_BAD_COUNT : TQ_STATUS_BAD_PAGE);
    return;
  }
  const int nw = c1 > c0 ? (pg1 - pg0 + 1) * 4 : 0;
  for (int e = tid; e < nw; e += kCommitThreads) {
    const int pg = pg0 + (e >> 2), j = e & 3;
    const int valid = c1 - pg * L.P < L.P ? c1 - pg * L.P : L.P;
    reinterpret_cast<uint4*>(a.pool + static_cast<int64_t>(bt[pg]) * L.page_bytes)[j] =
        header_words(L, ci, pg, valid, j);
  }
  if (tid == 0) a.seq_lens[b] = T1;
}

}  // namespace

int launch_encode(const tq_ctx* c, int kind, int dtype, const EncodeArgs& a, void* stream) {
  // fp16 rows take the matrix-core encoder; other inputs this one
  const int rc = launch_encode_mma(c, kind, dtype, a, stream);
  if (rc <= 0) return rc == 0 ? 0 : 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bits = kind == TQ_KIND_KEY ? c->p.key_bits : c->p.value_bits;
  const int qjl = (kind == TQ_KIND_KEY && c->p.key_qjl) ? 1 : 0;
  const int mixed = (kind == TQ_KIND_KEY ? c->p.key_mixed : c->p.value_mixed) ? 1 : 0;
  const int n8 = (kind == TQ_KIND_KEY && c->p.key_norm_u8) ? 1 : 0;
  const int64_t tiles = (a.n + kTile - 1) / kTile;
  if (tiles > 0x7fffffff) return 1;
  dim3 grid(static_cast<unsigned>(tiles));
  if (c->p.rotation == TQ_ROT_HADAMARD)
    hipLaunchKernelGGL(encode_flat_kernel<true>, grid, dim3(kThreads), 0, s, a, c->t, c->cb, kind, dtype, bits, qjl,
                       mixed, n8);
  else
    hipLaunchKernelGGL(encode_flat_kernel<false>, grid, dim3(kThreads), 0, s, a, c->t, c->cb, kind, dtype, bits, qjl,
                       mixed, n8);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

int launch_append(const tq_ctx* c, const AppendArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int W = c->p.window;
  const Layout& L = c->lay;
  const bool had = c->p.rotation == TQ_ROT_HADAMARD;
  // the ring update rides along when no slot can be read and written by
  // different work-groups (at most W new tokens)
  int ring = (W > 0 && a.n_new <= W) ? 1 : 0;
  // header byte: 0 no QJL, 1 Gaussian S, 2 orthogonal S
  const CommitInfo ci{c->p.rotation, c->p.key_qjl ? 1 + c->p.qjl_kind : 0, c->p.seed};
  if (a.n_new <= kSmallNew) {
    // decode steps: one work-group per (sequence, kv head, keys|values); with
    // the ring updated here too (or no ring), the last work-group of each
    // sequence commits it, with the next set of arrival counts
    AppendArgs as = a;
    if ((ring || W == 0) && a.batch <= kAppendMaxBatch && c->append_ctr) {
      const unsigned slot = c->append_calls.fetch_add(1u, std::memory_order_relaxed) % kAppendSlots;
      as.ctr = c->append_ctr + static_cast<int64_t>(slot) * kAppendMaxBatch;
    }
    const dim3 grid(2, L.H, a.batch);
    if (had)
      hipLaunchKernelGGL(append_small_kernel<true>, grid, dim3(kSmallThreads), 0, s, as, c->t, L, W, ring, ci);
    else
      hipLaunchKernelGGL(append_small_kernel<false>, grid, dim3(kSmallThreads), 0, s, as, c->t, L, W, ring, ci);
    if (hipGetLastError() != hipSuccess) return 1;
    if (as.ctr) return 0;
  } else {
    // bulk: the matrix-core append for the kinds it takes (every rate with a
    // symmetric codebook), the vector-ALU one for the rest and under
    // TQ_FLAG_VALU_APPEND; the ring is then updated by its own kernel, after
    // every encoded token has been read
    int kinds = 0;
    for (int kind = 0; kind < 2; ++kind) {
      const int rc = (c->p.flags & TQ_FLAG_VALU_APPEND) ? 1 : launch_append_mma(c, kind, a, stream);
      if (rc < 0) return 1;
      if (rc > 0) kinds |= 1 << kind;
    }
    if (kinds != 3) ring = 0;
    if (kinds != 0) {
      // groups a sequence can touch: ceil(n_new / 32) + 1 (unaligned start)
      const int gmax = (a.n_new + kVGroup - 1) / kVGroup + 1;
      const dim3 grid(2 * gmax, L.H, a.batch);  // even x: keys, odd x: values
      if (had)
        hipLaunchKernelGGL(append_encode_kernel<true>, grid, dim3(kThreads), 0, s, a, c->t, c->cb, L, W, ring, kinds);
      else
        hipLaunchKernelGGL(append_encode_kernel<false>, grid, dim3(kThreads), 0, s, a, c->t, c->cb, L, W, ring, kinds);
    }
  }
  if (hipGetLastError() != hipSuccess) return 1;
  if (W > 0 && !ring) {
    hipLaunchKernelGGL(append_ring_kernel, dim3(L.H, a.batch), dim3(kThreads), 0, s, a, c->t, L, W);
    if (hipGetLastError() != hipSuccess) return 1;
  }
  hipLaunchKernelGGL(append_commit_kernel, dim3(a.batch), dim3(kCommitThreads), 0, s, a, c->t, L, W, ci);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace tq
