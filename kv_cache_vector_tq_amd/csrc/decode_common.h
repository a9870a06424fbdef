// Shared by the decode kernels.
#pragma once

#include "tq_internal.h"

namespace tq {

struct KParams {
  int Hq, Hkv, G, P, W;
  int64_t page_bytes, head_bytes, k_norm, k_rnorm, k_codes, k_signs, v_norm, v_codes;
  int rotation;
  float qjl_scale;
};

inline KParams make_kparams(const tq_ctx* c) {
  KParams k;
  k.Hq = c->p.num_q_heads;
  k.Hkv = c->p.num_kv_heads;
  k.G = k.Hq / k.Hkv;
  k.P = c->p.page_tokens;
  k.W = c->p.window;
  k.page_bytes = c->lay.page_bytes;
  k.head_bytes = c->lay.head_bytes;
  k.k_norm = c->lay.k_norm;
  k.k_rnorm = c->lay.k_rnorm;
  k.k_codes = c->lay.k_codes;
  k.k_signs = c->lay.k_signs;
  k.v_norm = c->lay.v_norm;
  k.v_codes = c->lay.v_codes;
  k.rotation = c->p.rotation;
  k.qjl_scale = 1.2533141373155003f / static_cast<float>(c->p.head_dim);  // sqrt(pi/2)/d
  return k;
}


constexpr int kScanThreads = 256;

// MFMA-based compressed-page scan (decode_mfma.hip).
int launch_scan_mfma(const tq_ctx* c, const DecodeArgs& a, const KParams& k, void* stream);

}  // namespace tq
