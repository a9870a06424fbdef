// Shared by the decode kernels.
#pragma once

#include <cmath>

#include "tq_internal.h"

namespace tq {

struct KParams {
  int Hq, Hkv, G, P, W;
  int d;  // head size: coordinates of q, out and the FP16 window rows (the rest use D)
  int64_t page_bytes, head_bytes, k_norm, k_rnorm, k_codes, k_signs, v_norm, v_codes;
  int rotation;
  float qjl_scale;
  int det;  // fixed (bit-reproducible) share of chunks per scan wave
};

inline KParams make_kparams(const tq_ctx* c) {
  KParams k;
  k.Hq = c->p.num_q_heads;
  k.Hkv = c->p.num_kv_heads;
  k.G = k.Hq / k.Hkv;
  k.P = c->p.page_tokens;
  k.W = c->p.window;
  k.d = c->p.head_dim;
  k.page_bytes = c->lay.page_bytes;
  k.head_bytes = c->lay.head_bytes;
  k.k_norm = c->lay.k_norm;
  k.k_rnorm = c->lay.k_rnorm;
  k.k_codes = c->lay.k_codes;
  k.k_signs = c->lay.k_signs;
  k.v_norm = c->lay.v_norm;
  k.v_codes = c->lay.v_codes;
  k.rotation = c->p.rotation;
  k.det = (c->p.flags & TQ_FLAG_DETERMINISTIC) ? 1 : 0;
  // QJL coefficient: sqrt(pi/2)/D for Gaussian S, sqrt(pi/2)/sqrt(D) for
  // orthogonal S (S has D rows), times the shrinkage factor
  const double dd = static_cast<double>(c->lay.D);
  const double base = c->p.qjl_kind == TQ_QJL_ORTHOGONAL ? 1.2533141373155003 / std::sqrt(dd)
                                                          : 1.2533141373155003 / dd;
  k.qjl_scale = static_cast<float>(base * static_cast<double>(c->p.qjl_shrink));
  return k;
}


constexpr int kScanThreads = 256;

// MFMA-based compressed-page scan (decode_mfma.hip).
// ev0 / ev1 (may be null): HIP events updated with the scan kernel's own start and stop times
int launch_scan_mfma(const tq_ctx* c, const DecodeArgs& a, const KParams& k, void* stream, void* ev0, void* ev1);

}  // namespace tq
