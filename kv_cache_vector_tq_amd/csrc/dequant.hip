// Dequantise flat records (tq_decode): the inverse of tq_encode's records
// ("aither-kvcache" README, "Algorithm", last step; keys' correction from
// "TurboQuant on a 16GB MacBook", "The QJL detective story"):
//   u = n c[code] (+ a ||r|| S^T (2 sigma - 1) for keys with the sketch),
//   x_hat = Pi^T u  (dense) or eps . H u / sqrt(d)  (Hadamard).
// A work-group of 128 threads (thread = coordinate) takes a tile of 32
// records: codes and sign bits are unpacked into LDS, each thread holds one
// row of S^T and then one row of Pi^T in registers and runs the tile's
// matrix-vector products against LDS broadcasts.  Used for quality
// measurements; the decode path scores the packed cache directly.
#include "decode_common.h"
#include "device_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kTile = 32;
constexpr int kThreads = 128;

struct DequantArgs {
  const uint8_t* codes;
  const uint8_t* signs;
  const float* norms;
  const float* rnorms;
  int64_t n;
  float* out;  // rows of d coordinates (the first d of the D the records hold)
  int d;
  int bits;
  int qjl;
  int hmod;  // mixed-channel rate: coordinate j has bits + 1 when j mod hmod >= hmod/2; 0: integer rate
  float coef;
  float cen[16];
  float cen2[16];  // the (bits+1)-bit codebook of a mixed rate
};

template <bool HAD>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs a, DevTables t) {
  __shared__ float us[kTile][kD];      // rotated-basis vectors
  __shared__ uint32_t sg[kTile][4];    // sign words
  __shared__ float nv[kTile], rv[kTile];
  __shared__ float ctab[32];
  const int tid = threadIdx.x;
  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * kTile;
  const int nvec = static_cast<int>(a.n - v0 < kTile ? a.n - v0 : kTile);
  if (tid < 32) {
    float c = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (k == tid) c = a.cen[k];
      if (k + 16 == tid) c = a.cen2[k];
    }
    ctab[tid] = c;
  }
  if (tid < kTile) {
    nv[tid] = tid < nvec ? a.norms[v0 + tid] : 0.0f;
    rv[tid] = (a.qjl && tid < nvec) ? a.rnorms[v0 + tid] : 0.0f;
  }
  if (a.qjl) {
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(a.signs);
    const int v = tid >> 2;
    sg[v][tid & 3] = v < nvec ? sw[(v0 + v) * 4 + (tid & 3)] : 0u;
  }
  __syncthreads();
  // u[v][j] = n c[code_j] for coordinate j = tid
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(a.codes);
  // record: d codes of `bits` bits, or (mixed rate) the d/2 low-rate codes,
  // then the d/2 high-rate codes of bits + 1, each half in ascending order
  const bool hi = a.hmod != 0 && mixed_hi(tid, a.hmod);
  const int width = a.bits + (hi ? 1 : 0);
  const int wpv = 4 * a.bits + (a.hmod ? 2 : 0);  // 32-bit words per record (d = 128)
  const int bitpos = a.hmod == 0 ? tid * a.bits
                                 : (hi ? (kD / 2) * a.bits : 0) + mixed_rank(tid, a.hmod) * width;
  for (int v = 0; v < nvec; ++v) {
    const uint32_t* w = cw + (v0 + v) * wpv;
    const int wi = bitpos >> 5, bi = bitpos & 31;
    uint32_t c = w[wi] >> bi;
    if (bi + width > 32) c |= w[wi + 1] << (32 - bi);
    c &= (1u << width) - 1u;
    us[v][tid] = nv[v] * ctab[(hi ? 16 : 0) + c];
  }
  if (a.qjl) {
    // + coef ||r|| (S^T pm)_j: this thread's row of S^T is column j of S
    float srow[kD];
#pragma unroll
    for (int i = 0; i < kD; ++i) srow[i] = t.ST[tid * kD + i];
#pragma unroll 1
    for (int v = 0; v < nvec; ++v) {
      float z = 0.0f;
#pragma unroll
      for (int i = 0; i < kD; ++i) z += ((sg[v][i >> 5] >> (i & 31)) & 1u) ? srow[i] : -srow[i];
      us[v][tid] = fmaf(a.coef * rv[v], z, us[v][tid]);
    }
  }
  __syncthreads();
  if constexpr (!HAD) {
    // x_hat[v][i] = sum_j Pi[j][i] u[v][j]: row i of Pi^T
    float prow[kD];
#pragma unroll
    for (int j = 0; j < kD; ++j) prow[j] = t.rotT[tid * kD + j];
#pragma unroll 1
    for (int v = 0; v < nvec; ++v) {
      float x = 0.0f;
      const float4* ur = reinterpret_cast<const float4*>(us[v]);
#pragma unroll
      for (int j4 = 0; j4 < kD / 4; ++j4) {
        const float4 u = ur[j4];
        x = fmaf(prow[4 * j4 + 0], u.x, x);
        x = fmaf(prow[4 * j4 + 1], u.y, x);
        x = fmaf(prow[4 * j4 + 2], u.z, x);
        x = fmaf(prow[4 * j4 + 3], u.w, x);
      }
      if (tid < a.d) a.out[(v0 + v) * a.d + tid] = x;
    }
  } else {
    // x_hat = eps . H u / sqrt(d): butterflies 1..32 in the wave, 64 through LDS
    const float eps = t.rot[tid];
    for (int v = 0; v < nvec; ++v) {
      float val = us[v][tid];
#pragma unroll
      for (int s = 1; s < 64; s <<= 1) {
        const float o = __shfl_xor(val, s, 64);
        val = (tid & s) ? (o - val) : (val + o);
      }
      __syncthreads();
      us[v][tid] = val;
      __syncthreads();
      const float p = us[v][tid], q = us[v][tid ^ 64];
      if (tid < a.d) a.out[(v0 + v) * a.d + tid] = ((tid & 64) ? (q - p) : (p + q)) * 0.08838834764831845f * eps;
    }
  }
}

}  // namespace

int launch_dequant(const tq_ctx* c, int kind, const uint8_t* codes, const uint8_t* signs, const float* norms,
                   const float* rnorms, int64_t n, float* out, void* stream) {
  const bool key = kind == TQ_KIND_KEY;
  DequantArgs a;
  a.codes = codes;
  a.signs = signs;
  a.norms = norms;
  a.rnorms = rnorms;
  a.n = n;
  a.out = out;
  a.d = c->p.head_dim;
  a.bits = key ? c->p.key_bits : c->p.value_bits;
  a.qjl = (key && c->p.key_qjl) ? 1 : 0;
  a.coef = make_kparams(c).qjl_scale;
  a.hmod = (key ? c->p.key_mixed : c->p.value_mixed) ? (key ? kKeyHiMod : kValHiMod) : 0;
  for (int k = 0; k < 16; ++k) {
    a.cen[k] = key ? c->cb.kc[k] : c->cb.vc[k];
    a.cen2[k] = key ? c->cb.kc2[k] : c->cb.vc2[k];
  }
  const int64_t tiles = (n + kTile - 1) / kTile;
  if (tiles > 0x7fffffff) return 1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->p.rotation == TQ_ROT_HADAMARD)
    hipLaunchKernelGGL(dequant_kernel<true>, dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, s, a, c->t);
  else
    hipLaunchKernelGGL(dequant_kernel<false>, dim3(static_cast<unsigned>(tiles)), dim3(kThreads), 0, s, a, c->t);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace tq
