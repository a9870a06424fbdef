// Final step of tq_decode_attn for one (sequence b, kv head h), run by the
// last scan work-group of the pair to finish (or by a finalize kernel after
// the vector-ALU scan): combine the split partials (m_s, l_s, acc_s, rotated
// basis, s = 0 .. splits-1 in order) with the FP16 window's partial (m_w,
// l_w, acc_w, original basis), apply Pi^T once and normalise
// ("TurboQuant Family Design Study", section "CPU and WASM kernel design":
// values accumulated in the rotated basis, one inverse transform per head):
//   M = max(m_s, m_w),  L = sum_s 2^(m_s - M) l_s + 2^(m_w - M) l_w,
//   o = (Pi^T sum_s 2^(m_s - M) acc_s + 2^(m_w - M) acc_w) / L.
// Every sum is taken in a fixed order, so the result does not depend on
// which work-group finalizes.
#pragma once

#include "decode_common.h"
#include "device_common.h"

namespace tq {

// LDS floats the finalize needs besides acc[GW][kD]: NT * max(GW, 4) for the
// partial sums, and the per-group maxima and normalisers.
template <int NT, int GW>
constexpr int finalize_scratch_floats() { return NT * (GW > 4 ? GW : 4) + 2 * NT; }

// Splits up to which the matrix-core scan's last work-group of a kv head
// finalizes it; with more (long contexts, few sequences) a finalize kernel
// spreads the heads over more work-groups.
constexpr int kFuseMaxSplits = 4;

// Called after this work-group's partial is in global memory; every thread
// calls it.  Returns true in the work-group that arrives last among the
// splits of (b, h), which then sees every split's partial.  Each wave waits
// for its own stores to be acknowledged; one thread then counts the arrival
// with an agent-scope acquire-release add (its release writes back this
// XCD's L2 so that the partial reaches a finalizer on another XCD; its
// acquire invalidates the caches the finalizer reads through).  One such
// pair per work-group: a device fence in every wave measured twice the scan
// time.
template <int NT>
__device__ inline bool arrive_last(int* ctr, int splits, int* flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == splits - 1;
  __syncthreads();
  return *flag != 0;
}

// Combines query heads g0 .. g0+GW-1 of kv head h of sequence b (GW of the
// group's k.G heads; acc: LDS [GW][kD]; fin: LDS, finalize_scratch_floats;
// sL, sW: LDS [GW]).  The window's partial comes from global memory (prep
// wrote it), or with lw_m non-null from LDS (lw_m, lw_l [GW], lw_acc
// [GW][kD]: the finalize kernel took the window itself).  Every load of a
// step is issued before any is used: empty splits hold zero accumulators
// and get factor 0, so they are read like the others.  base_in >= 0 gives
// the kv head's first partial slot and S_in its split count (a scan
// work-group knows both from its own plan entry); else they are read.
template <int NT, int GW>
__device__ void finalize_bh(const DecodeArgs& a, const DevTables& t, const KParams& k, int b, int h, int g0,
                            float (*acc)[kD], float* fin, float* sL, float* sW, const float* lw_m = nullptr,
                            const float* lw_l = nullptr, const float (*lw_acc)[kD] = nullptr,
                            int64_t base_in = -1, int S_in = 0) {
  const int tid = threadIdx.x;
  const int64_t bh = static_cast<int64_t>(b) * k.Hkv + h;
  const int64_t q0 = static_cast<int64_t>(b) * k.Hq + static_cast<int64_t>(h) * k.G + g0;  // first query row
  // this kv head's partial slots: base .. base + S - 1, in split order
  // (slots outside the plan's are never read)
  const int64_t base = base_in >= 0 ? base_in : a.sbase ? a.sbase[bh] : bh * a.splits;
  int S = base_in >= 0 ? S_in : a.sbase ? a.sbase[bh + 1] - a.sbase[bh] : a.splits;
  if (a.sbase && (base < 0 || S < 0 || base + S > a.nwg)) S = 0;
  const int G = k.G;
  const bool dense = k.rotation == TQ_ROT_DENSE;
  auto win_m = [&](int g) { return lw_m ? lw_m[g] : a.wm[q0 + g]; };
  auto win_l = [&](int g) { return lw_l ? lw_l[g] : a.wl[q0 + g]; };
  // (a) this thread's slice of a row of Pi^T (dense): thread (j, part p),
  //     P parts (a power of two; threads past P * kD take no part)
  constexpr int P = (NT / kD) >= 8 ? 8 : (NT / kD) >= 4 ? 4 : (NT / kD) >= 2 ? 2 : 1;
  constexpr int kSlice = kD / P;
  const int j = tid % kD, p = tid / kD;
  float4 rrow[kSlice / 4];
  if (dense && p < P) {
    const float4* row = reinterpret_cast<const float4*>(t.rotT + j * kD + p * kSlice);
#pragma unroll
    for (int i4 = 0; i4 < kSlice / 4; ++i4) rrow[i4] = row[i4];
  }
  // (b) the window accumulator elements this thread finishes in step 3
  constexpr int kOut = (GW * kD + NT - 1) / NT;
  float wa[kOut];
#pragma unroll
  for (int r = 0; r < kOut; ++r) {
    const int e = tid + r * NT;
    const int g = e / kD, i = e % kD;
    wa[r] = e >= GW * kD ? 0.0f : lw_acc ? lw_acc[g][i] : a.wacc[(q0 + g) * kD + i];
  }
  // 1. thread (item = query g, coordinates c4 .. c4+3; group grp) merges
  //    splits grp, grp + NG, ... online (running maximum m, rescaled sums);
  //    the groups are merged in order below
  constexpr int kItems = GW * (kD / 4);
  constexpr int NG = NT / kItems > 0 ? NT / kItems : 1;
  constexpr int kRounds = (kItems * NG + NT - 1) / NT;
  float* gm = fin + NG * GW * kD;  // [NG][GW] group maxima
  float* gl = gm + NG * GW;        // [NG][GW] group sums of l
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int e = tid + r * NT;
    if (e >= kItems * NG) continue;
    const int item = e % kItems, grp = e / kItems;
    const int g = item / (kD / 4), c4 = 4 * (item % (kD / 4));
    float m = -INFINITY, L = 0.0f;
    float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
    for (int s2 = grp; s2 < S; s2 += NG) {
      const int64_t pi = (base + s2) * G + g0 + g;
      const float ls = a.pl[pi], ms = a.pm[pi];
      const float4 pa = *reinterpret_cast<const float4*>(a.pacc + pi * kD + c4);
      const bool ok = ls > 0.0f;
      const float mn = ok ? fmaxf(m, ms) : m;
      const float cf = m == mn ? 1.0f : exp2f(m - mn);
      const float f = ok ? exp2f(ms - mn) : 0.0f;
      v.x = fmaf(f, pa.x, v.x * cf);
      v.y = fmaf(f, pa.y, v.y * cf);
      v.z = fmaf(f, pa.z, v.z * cf);
      v.w = fmaf(f, pa.w, v.w * cf);
      L = fmaf(f, ls, L * cf);
      m = mn;
    }
    *reinterpret_cast<float4*>(fin + (grp * GW + g) * kD + c4) = v;
    if (c4 == 0) {
      gm[grp * GW + g] = m;
      gl[grp * GW + g] = L;
    }
  }
  __syncthreads();
  // per query: M over the groups and the window, the factors, L
  if (tid < GW) {
    const float wl = win_l(tid), wmv = win_m(tid);
    float M = wl > 0.0f ? wmv : -INFINITY;
    for (int r = 0; r < NG; ++r) M = fmaxf(M, gm[r * GW + tid]);
    float L = 0.0f;
    for (int r = 0; r < NG; ++r) {
      const float mr = gm[r * GW + tid];
      const float f = mr == -INFINITY ? 0.0f : exp2f(mr - M);
      gm[r * GW + tid] = f;  // the group's factor from here on
      L = fmaf(f, gl[r * GW + tid], L);
    }
    const float fw = wl > 0.0f ? exp2f(wmv - M) : 0.0f;
    sW[tid] = fw;
    sL[tid] = fmaf(fw, wl, L);
  }
  __syncthreads();
  for (int e = tid; e < GW * kD; e += NT) {
    const int g = e / kD, i = e % kD;
    float x = 0.0f;
    for (int r = 0; r < NG; ++r) x = fmaf(gm[r * GW + g], fin[(r * GW + g) * kD + i], x);
    acc[g][i] = x;
  }
  __syncthreads();
  // 2. back to the original basis
  if (dense) {
    // o[g][j] = sum_i Pi[i][j] acc[g][i] = sum_i PiT[j][i] acc[g][i]
    if (p < P) {
      float o[GW];
#pragma unroll
      for (int g = 0; g < GW; ++g) o[g] = 0.0f;
#pragma unroll
      for (int i4 = 0; i4 < kSlice / 4; ++i4) {
        const float4 r = rrow[i4];
        const int i = p * kSlice + 4 * i4;
#pragma unroll
        for (int g = 0; g < GW; ++g) {
          o[g] = fmaf(r.x, acc[g][i], o[g]);
          o[g] = fmaf(r.y, acc[g][i + 1], o[g]);
          o[g] = fmaf(r.z, acc[g][i + 2], o[g]);
          o[g] = fmaf(r.w, acc[g][i + 3], o[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GW; ++g) fin[(p * GW + g) * kD + j] = o[g];
    }
    __syncthreads();
    for (int e = tid; e < GW * kD; e += NT) {
      const int g = e / kD, jj = e % kD;
      float x = fin[g * kD + jj];
      for (int r = 1; r < P; ++r) x += fin[(r * GW + g) * kD + jj];
      acc[g][jj] = x;
    }
    __syncthreads();
  } else {
    // x = eps . H y / sqrt(kD): butterflies at strides 1 .. 64 in LDS
    for (int hs = 1; hs < kD; hs <<= 1) {
      for (int e = tid; e < GW * (kD / 2); e += NT) {
        const int g = e / (kD / 2), r = e % (kD / 2);
        const int i0 = (r / hs) * 2 * hs + r % hs, i1 = i0 + hs;
        const float x0 = acc[g][i0], x1 = acc[g][i1];
        acc[g][i0] = x0 + x1;
        acc[g][i1] = x0 - x1;
      }
      __syncthreads();
    }
    for (int e = tid; e < GW * kD; e += NT) {
      const int g = e / kD, i = e % kD;
      acc[g][i] *= t.rot[i] * 0.08838834764831845f;  // 1/sqrt(128)
    }
    __syncthreads();
  }
  // 3. plus the window's share, normalised; rows of d coordinates
#pragma unroll
  for (int r = 0; r < kOut; ++r) {
    const int e = tid + r * NT;
    const int g = e / kD, jj = e % kD;
    if (e >= GW * kD || jj >= k.d) continue;
    const float L = sL[g];
    const float x = fmaf(sW[g], wa[r], acc[g][jj]);
    a.out[(q0 + g) * k.d + jj] = L > 0.0f ? x / L : 0.0f;
  }
}

}  // namespace tq
