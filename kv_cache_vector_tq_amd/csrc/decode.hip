// Decode attention over the paged compressed cache (tq_decode_attn).
//
// Three kernels ("TurboQuant Family Design Study", sections "Placement
// relative to RoPE and attention" and "CPU and WASM kernel design";
// "aither-kvcache" README, "Zero-buffer fused attention"):
//  1. prep:  per (b, query head) q_rot = Pi q and p = S q_rot, pre-scaled by
//     sm_scale*log2(e) (and sqrt(pi/2)/d for p) so scores come out in log2
//     units; the plain query is kept for the FP16 window.
//  2. scan:  per (b, kv head, page split) stream the packed pages once:
//     score_t = n_t <q_rot, c_K[idx_t]> + ||r_t|| (2 <p, sigma_t> - sum p)
//     for the G query heads of the group, online softmax (exp2), and
//     acc += w_t n^V_t c_V[idx^V_t] in the rotated basis; write (m, l, acc).
//  3. merge: per (b, query head) combine the split partials in fixed order,
//     score the FP16 window exactly in the original basis, apply Pi^T to the
//     rotated accumulator once and normalise.
#include "decode_common.h"
#include "device_common.h"
#include "tq_internal.h"

namespace tq {
namespace {

// ---------------------------------------------------------------- prep
__global__ __launch_bounds__(kD) void prep_kernel(DecodeArgs a, DevTables t, KParams k, int qjl) {
  __shared__ float qv[kD], qr[kD], red[2];
  const int j = threadIdx.x, g = blockIdx.x, b = blockIdx.y;
  const int64_t row = (static_cast<int64_t>(b) * k.Hq + g) * kD;
  const float c2 = a.sm_scale * kLog2e;
  const float q = load_any(a.q, row + j, a.q_dtype);
  a.qwin[row + j] = q * c2;
  qv[j] = q;
  __syncthreads();
  float y;
  if (k.rotation == TQ_ROT_DENSE) {
    y = 0.0f;
#pragma unroll 8
    for (int i = 0; i < kD; ++i) y = fmaf(t.rotT[i * kD + j], qv[i], y);
  } else {
    float val = qv[j] * t.rot[j];
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const float o = __shfl_xor(val, s, 64);
      val = (j & s) ? (o - val) : (val + o);
    }
    qr[j] = val;
    __syncthreads();
    const float a0 = qr[j], b0 = qr[j ^ 64];
    y = ((j & 64) ? (b0 - a0) : (a0 + b0)) * 0.08838834764831845f;
    __syncthreads();
  }
  qr[j] = y;
  a.qs[row + j] = y * c2;
  if (!qjl) return;
  __syncthreads();
  float p = 0.0f;
#pragma unroll 8
  for (int i = 0; i < kD; ++i) p = fmaf(t.ST[i * kD + j], qr[i], p);
  const float ps = p * k.qjl_scale * c2;
  a.ps[row + j] = ps;
  const float w = wave_sum(ps);
  if ((j & 63) == 0) red[j >> 6] = w;
  __syncthreads();
  if (j == 0) a.psum[static_cast<int64_t>(b) * k.Hq + g] = red[0] + red[1];
}

// ---------------------------------------------------------------- scan
template <int G, int BK, int BV, bool QJL>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(DecodeArgs a, DevTables t, Codebooks cb, KParams k) {
  __shared__ float kct[16], vct[16];
  __shared__ float wv[kScanThreads][G];
  __shared__ float red[4][G];
  __shared__ float comb[kD][G];
  const int tid = threadIdx.x, split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = tid >> 6;
  const int T = a.seq_lens[b];
  const int C = T - k.W > 0 ? T - k.W : 0;
  const int npages = (C + k.P - 1) / k.P;
  const int pb = split * a.pages_per_split;
  const int pe = npages < pb + a.pages_per_split ? npages : pb + a.pages_per_split;
  const int64_t pidx = ((static_cast<int64_t>(b) * k.Hkv + h) * a.splits + split) * G;
  if (pb >= pe) {
    if (tid < G) {
      a.pm[pidx + tid] = -INFINITY;
      a.pl[pidx + tid] = 0.0f;
    }
    for (int i = tid; i < G * kD; i += kScanThreads) a.pacc[pidx * kD + i] = 0.0f;
    return;
  }
  if (tid < 16) {
    float kv = 0.0f, vv = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i == tid) {
        kv = cb.kc[i];
        vv = cb.vc[i];
      }
    kct[tid] = kv;
    vct[tid] = vv;
  }
  const int64_t qrow = (static_cast<int64_t>(b) * k.Hq + static_cast<int64_t>(h) * G) * kD;
  const float* __restrict__ qs = a.qs + qrow;
  const float* __restrict__ ps = a.ps + qrow;
  float psum[G];
#pragma unroll
  for (int g = 0; g < G; ++g) psum[g] = QJL ? a.psum[static_cast<int64_t>(b) * k.Hq + h * G + g] : 0.0f;
  float m[G], l[G], acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.0f;
    acc[g] = 0.0f;
  }
  const int j = tid & (kD - 1), half = tid >> 7;
  __syncthreads();
  for (int pg = pb; pg < pe; ++pg) {
    if (pg >= a.max_pages) {  // more compressed tokens than the block table can name
      if (tid == 0) atomicOr(t.status, TQ_STATUS_BAD_PAGE);
      break;
    }
    const int pid = a.block_table[static_cast<int64_t>(b) * a.max_pages + pg];
    if (pid < 0 || pid >= a.num_pages) {
      if (tid == 0) atomicOr(t.status, TQ_STATUS_BAD_PAGE);
      continue;
    }
    const uint8_t* hb = a.pool + static_cast<int64_t>(pid) * k.page_bytes + kBodyOffset + h * k.head_bytes;
    const int nval = C - pg * k.P < k.P ? C - pg * k.P : k.P;
    for (int s0 = 0; s0 < nval; s0 += kScanThreads) {
      const int tk = s0 + tid;
      const bool valid = tk < nval;
      float sc[G];
      float vnorm = 0.0f;
      if (valid) {
        const float kn = reinterpret_cast<const float*>(hb + k.k_norm)[tk];
        vnorm = reinterpret_cast<const float*>(hb + k.v_norm)[tk];
        uint32_t cw[4 * BK];
        const uint4* cp4 = reinterpret_cast<const uint4*>(hb + k.k_codes + static_cast<int64_t>(tk) * 16 * BK);
#pragma unroll
        for (int i = 0; i < BK; ++i) {
          const uint4 v = cp4[i];
          cw[4 * i + 0] = v.x;
          cw[4 * i + 1] = v.y;
          cw[4 * i + 2] = v.z;
          cw[4 * i + 3] = v.w;
        }
        float dot[G];
#pragma unroll
        for (int g = 0; g < G; ++g) dot[g] = 0.0f;
#pragma unroll
        for (int jj = 0; jj < kD; ++jj) {
          const float c = kct[bits_at<BK>(cw, jj * BK)];
#pragma unroll
          for (int g = 0; g < G; ++g) dot[g] = fmaf(qs[g * kD + jj], c, dot[g]);
        }
        if constexpr (QJL) {
          const float rn = reinterpret_cast<const float*>(hb + k.k_rnorm)[tk];
          const uint4 sv = reinterpret_cast<const uint4*>(hb + k.k_signs)[tk];
          const uint32_t sw[4] = {sv.x, sv.y, sv.z, sv.w};
          float sd[G];
#pragma unroll
          for (int g = 0; g < G; ++g) sd[g] = 0.0f;
#pragma unroll
          for (int jj = 0; jj < kD; ++jj) {
            const float f = static_cast<float>((sw[jj >> 5] >> (jj & 31)) & 1u);
#pragma unroll
            for (int g = 0; g < G; ++g) sd[g] = fmaf(ps[g * kD + jj], f, sd[g]);
          }
#pragma unroll
          for (int g = 0; g < G; ++g) sc[g] = fmaf(kn, dot[g], rn * fmaf(2.0f, sd[g], -psum[g]));
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g) sc[g] = kn * dot[g];
        }
        if (a.dbg_logits) {
#pragma unroll
          for (int g = 0; g < G; ++g)
            a.dbg_logits[(static_cast<int64_t>(b) * k.Hq + h * G + g) * a.logits_stride + pg * k.P + tk] =
                sc[g] * kLn2;
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = -INFINITY;
      }
      // tile max
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mx = wave_max(sc[g]);
        if ((tid & 63) == 0) red[wave][g] = mx;
      }
      __syncthreads();
      float corr[G], w[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float tm = fmaxf(fmaxf(red[0][g], red[1][g]), fmaxf(red[2][g], red[3][g]));
        const float mn = fmaxf(m[g], tm);
        corr[g] = exp2f(m[g] - mn);
        m[g] = mn;
        w[g] = valid ? exp2f(sc[g] - mn) : 0.0f;
        wv[tid][g] = valid ? w[g] * vnorm : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float sw = wave_sum(w[g]);
        if ((tid & 63) == 0) red[wave][g] = sw;
      }
      __syncthreads();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        l[g] = fmaf(l[g], corr[g], (red[0][g] + red[1][g]) + (red[2][g] + red[3][g]));
        acc[g] *= corr[g];
      }
      // value accumulation: thread (coordinate j, half) takes every other 32-token group
      const int tile_tokens = nval - s0 < kScanThreads ? nval - s0 : kScanThreads;
      const int ngroups = (tile_tokens + kVGroup - 1) / kVGroup;
      const uint32_t* vw = reinterpret_cast<const uint32_t*>(hb + k.v_codes);
      for (int gi = half; gi < ngroups; gi += 2) {
        const int64_t grp = s0 / kVGroup + gi;
        uint32_t wd[BV + 1];
#pragma unroll
        for (int w2 = 0; w2 < BV; ++w2) wd[w2] = vw[(grp * BV + w2) * kD + j];
        wd[BV] = 0u;
#pragma unroll
        for (int i = 0; i < kVGroup; ++i) {
          const float c = vct[bits_at<BV>(wd, i * BV)];
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g] = fmaf(wv[gi * kVGroup + i][g], c, acc[g]);
        }
      }
      __syncthreads();
    }
  }
  if (half == 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) comb[j][g] = acc[g];
  }
  __syncthreads();
  if (half == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) a.pacc[(pidx + g) * kD + j] = acc[g] + comb[j][g];
  }
  if (tid < G) {
    float mv = 0.0f, lv = 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g == tid) {
        mv = m[g];
        lv = l[g];
      }
    a.pm[pidx + tid] = mv;
    a.pl[pidx + tid] = lv;
  }
}

// ---------------------------------------------------------------- merge
__global__ __launch_bounds__(kD) void merge_kernel(DecodeArgs a, DevTables t, KParams k) {
  __shared__ float accr[kD];
  __shared__ float ls[kMaxWindow];
  __shared__ float qw[kD];
  __shared__ float red[2];
  const int j = threadIdx.x, g = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int gq = h * k.G + g;
  const int T = a.seq_lens[b];
  const int nwin = T < k.W ? T : k.W;
  const int64_t qrow = (static_cast<int64_t>(b) * k.Hq + gq) * kD;
  // 1. combine split partials (fixed order)
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) {
    const int64_t pi = ((static_cast<int64_t>(b) * k.Hkv + h) * a.splits + s) * k.G + g;
    if (a.pl[pi] > 0.0f) M = fmaxf(M, a.pm[pi]);
  }
  float acc = 0.0f, L = 0.0f;
  for (int s = 0; s < a.splits; ++s) {
    const int64_t pi = ((static_cast<int64_t>(b) * k.Hkv + h) * a.splits + s) * k.G + g;
    const float lv = a.pl[pi];
    if (lv > 0.0f) {
      const float f = exp2f(a.pm[pi] - M);
      L = fmaf(f, lv, L);
      acc = fmaf(f, a.pacc[pi * kD + j], acc);
    }
  }
  accr[j] = acc;
  qw[j] = a.qwin[qrow + j];
  __syncthreads();
  // 2. window scores (original basis, FP16 keys), log2 units
  const int64_t bh = static_cast<int64_t>(b) * k.Hkv + h;
  float lmax = -INFINITY;
  for (int tk = j; tk < nwin; tk += kD) {
    const uint4* kr = reinterpret_cast<const uint4*>(a.k_win + (bh * k.W + tk) * kD);
    float s = 0.0f;
#pragma unroll 4
    for (int i = 0; i < kD / 8; ++i) {
      const uint4 v = kr[i];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = fmaf(qw[8 * i + 2 * e], half_bits_to_float(static_cast<uint16_t>(u[e] & 0xffffu)), s);
        s = fmaf(qw[8 * i + 2 * e + 1], half_bits_to_float(static_cast<uint16_t>(u[e] >> 16)), s);
      }
    }
    ls[tk] = s;
    lmax = fmaxf(lmax, s);
    if (a.dbg_logits) {
      // slot tk holds the largest position p < T with p = tk (mod W)
      const int pos = tk + k.W * ((T - 1 - tk) / k.W);
      a.dbg_logits[(static_cast<int64_t>(b) * k.Hq + gq) * a.logits_stride + pos] = s * kLn2;
    }
  }
  lmax = wave_max(lmax);
  if ((j & 63) == 0) red[j >> 6] = lmax;
  __syncthreads();
  const float M2 = fmaxf(M, fmaxf(red[0], red[1]));
  __syncthreads();
  const float corr = (M == -INFINITY) ? 0.0f : exp2f(M - M2);
  float lw = 0.0f;
  for (int tk = j; tk < nwin; tk += kD) {
    const float w = exp2f(ls[tk] - M2);
    ls[tk] = w;
    lw += w;
  }
  lw = wave_sum(lw);
  if ((j & 63) == 0) red[j >> 6] = lw;
  __syncthreads();
  const float Ltot = fmaf(L, corr, red[0] + red[1]);
  float accw = 0.0f;
  for (int tk = 0; tk < nwin; ++tk)
    accw = fmaf(ls[tk], half_bits_to_float(a.v_win[(bh * k.W + tk) * kD + j]), accw);
  // 3. one inverse rotation of the rotated accumulator
  float o;
  if (k.rotation == TQ_ROT_DENSE) {
    o = 0.0f;
#pragma unroll 8
    for (int i = 0; i < kD; ++i) o = fmaf(t.rot[i * kD + j], accr[i], o);
  } else {
    float val = accr[j];
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
      const float ov = __shfl_xor(val, s, 64);
      val = (j & s) ? (ov - val) : (val + ov);
    }
    __syncthreads();
    accr[j] = val;
    __syncthreads();
    const float a0 = accr[j], b0 = accr[j ^ 64];
    o = ((j & 64) ? (b0 - a0) : (a0 + b0)) * 0.08838834764831845f * t.rot[j];
  }
  const float res = Ltot > 0.0f ? fmaf(o, corr, accw) / Ltot : 0.0f;
  a.out[qrow + j] = res;
}

template <int G, int BK, int BV>
void launch_scan_bits(bool qjl, dim3 grid, hipStream_t s, const DecodeArgs& a, const DevTables& t, const Codebooks& cb,
                      const KParams& k) {
  if (qjl)
    hipLaunchKernelGGL((scan_kernel<G, BK, BV, true>), grid, dim3(kScanThreads), 0, s, a, t, cb, k);
  else
    hipLaunchKernelGGL((scan_kernel<G, BK, BV, false>), grid, dim3(kScanThreads), 0, s, a, t, cb, k);
}

template <int G, int BK>
void launch_scan_bv(int bv, bool qjl, dim3 grid, hipStream_t s, const DecodeArgs& a, const DevTables& t,
                    const Codebooks& cb, const KParams& k) {
  if (bv == 2) launch_scan_bits<G, BK, 2>(qjl, grid, s, a, t, cb, k);
  else if (bv == 3) launch_scan_bits<G, BK, 3>(qjl, grid, s, a, t, cb, k);
  else launch_scan_bits<G, BK, 4>(qjl, grid, s, a, t, cb, k);
}

template <int G>
void launch_scan_g(int bk, int bv, bool qjl, dim3 grid, hipStream_t s, const DecodeArgs& a, const DevTables& t,
                   const Codebooks& cb, const KParams& k) {
  if (bk == 2) launch_scan_bv<G, 2>(bv, qjl, grid, s, a, t, cb, k);
  else if (bk == 3) launch_scan_bv<G, 3>(bv, qjl, grid, s, a, t, cb, k);
  else launch_scan_bv<G, 4>(bv, qjl, grid, s, a, t, cb, k);
}

}  // namespace

int launch_decode(const tq_ctx* c, const DecodeArgs& a, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const KParams k = make_kparams(c);
  const int qjl = c->p.key_qjl;
  hipLaunchKernelGGL(prep_kernel, dim3(k.Hq, a.batch), dim3(kD), 0, s, a, c->t, k, qjl);
  if (hipGetLastError() != hipSuccess) return 1;
  dim3 grid(a.splits, k.Hkv, a.batch);
  const int bk = c->p.key_bits, bv = c->p.value_bits;
  void* ev0 = profile_slot(c, 0);
  if (ev0 && hipEventRecord(static_cast<hipEvent_t>(ev0), s) != hipSuccess) return 1;
  if (c->p.flags & TQ_FLAG_VALU_SCAN) {
    switch (k.G) {
      case 1: launch_scan_g<1>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
      case 2: launch_scan_g<2>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
      case 4: launch_scan_g<4>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
      case 8: launch_scan_g<8>(bk, bv, qjl, grid, s, a, c->t, c->cb, k); break;
      default: return 1;
    }
    if (hipGetLastError() != hipSuccess) return 1;
  } else if (launch_scan_mfma(c, a, k, stream) != 0) {
    return 1;
  }
  if (ev0 && hipEventRecord(static_cast<hipEvent_t>(profile_slot(c, 1)), s) != hipSuccess) return 1;
  hipLaunchKernelGGL(merge_kernel, dim3(k.G, k.Hkv, a.batch), dim3(kD), 0, s, a, c->t, k);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace tq
