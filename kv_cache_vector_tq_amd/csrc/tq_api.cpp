// C ABI of the library: argument validation, context tables, workspace
// sizing and kernel launches.  See include/tq.h for the contract.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <limits>
#include <new>
#include <vector>

#include "decode_common.h"
#include "tq_internal.h"

namespace {

bool params_ok(const tq_params* p) {
  if (!p) return false;
  if (p->head_dim <= 0 || p->head_dim % 8 || p->head_dim > 4096) return false;
  if (p->key_bits < 2 || p->key_bits > 4 || p->value_bits < 2 || p->value_bits > 4) return false;
  if (p->key_qjl != 0 && p->key_qjl != 1) return false;
  if (p->rotation != TQ_ROT_DENSE && p->rotation != TQ_ROT_HADAMARD) return false;
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads) return false;
  if (p->page_tokens <= 0 || p->page_tokens % tq::kVGroup || p->page_tokens > tq::kMaxPage) return false;
  if (p->window < 0 || p->window > tq::kMaxWindow) return false;
  if (p->flags & ~(TQ_FLAG_VALU_SCAN | TQ_FLAG_VALU_APPEND | TQ_FLAG_DETERMINISTIC)) return false;
  if (p->qjl_kind != TQ_QJL_GAUSSIAN && p->qjl_kind != TQ_QJL_ORTHOGONAL) return false;
  if (!(p->qjl_shrink > 0.0f && p->qjl_shrink <= 4.0f)) return false;  // also rejects NaN
  // mixed-channel rates: 2.5 and 3.5 bits, halves of a multiple of 32 transform coordinates
  if (p->key_mixed != 0 && p->key_mixed != 1) return false;
  if (p->value_mixed != 0 && p->value_mixed != 1) return false;
  const int D = tq::transform_dim(p->head_dim);
  if (p->key_mixed && (p->key_bits < 2 || p->key_bits > 3 || D % 32)) return false;
  if (p->value_mixed && (p->value_bits < 2 || p->value_bits > 3 || D % 32)) return false;
  if (p->key_norm_u8 != 0 && p->key_norm_u8 != 1) return false;
  return true;
}

// What the kernels in this build cover.
bool params_supported(const tq_params* p) {
  const int G = p->num_q_heads / p->num_kv_heads;
  // the vector-ALU scan covers integer rates only
  if ((p->flags & TQ_FLAG_VALU_SCAN) && (p->key_mixed || p->value_mixed || p->key_norm_u8)) return false;
  // head sizes 72 .. 128 (transform size 128)
  return tq::transform_dim(p->head_dim) == tq::kD && (G == 1 || G == 2 || G == 4 || G == 8) &&
         p->num_kv_heads <= 65535;
}

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

void transpose(const float* a, float* at, int d) {
  for (int i = 0; i < d; ++i)
    for (int j = 0; j < d; ++j) at[j * d + i] = a[i * d + j];
}

// Pages per split-K work-group.  Automatic choice (pages_per_split = 0): the
// split count s minimising rounds(s) * (ceil(max_pages / s) + 2), where
// rounds(s) is how many waves of `slots` resident work-groups the
// batch * hkv * s work-groups take and the 2 pages stand for a work-group's
// fixed cost (tables, pipeline fill, final merge); ties go to the smaller s.
int decode_splits(int batch, int hkv, int max_pages, int pages_per_split, int slots, int* pps_out) {
  int pps = pages_per_split;
  if (pps <= 0) {
    const long long bh = static_cast<long long>(batch) * hkv;
    const long long sl = slots > 0 ? slots : 1;
    long long best = -1;
    pps = max_pages > 0 ? max_pages : 1;
    for (int s = 1; s <= (max_pages > 0 ? max_pages : 1); ++s) {
      const long long per = (max_pages + s - 1) / s;
      if (per > tq::kMaxSplitPages) continue;  // a split reads at most kMaxSplitPages pages
      if (s > 1 && per == (max_pages + s - 2) / (s - 1)) continue;  // same pages per split as s - 1
      const long long rounds = (bh * s + sl - 1) / sl;
      const long long cost = rounds * (per + 2);
      if (best < 0 || cost < best) {
        best = cost;
        pps = static_cast<int>(per);
      }
    }
  }
  if (pps > max_pages) pps = max_pages;
  if (pps > tq::kMaxSplitPages) pps = tq::kMaxSplitPages;
  if (pps < 1) pps = 1;
  if (pps_out) *pps_out = pps;
  const int splits = (max_pages + pps - 1) / pps;
  return splits < 1 ? 1 : splits;
}

struct WsLayout {
  size_t qs, ps, psum, wm, wl, wacc, pm, pl, pacc, ctr, plan, sbase, total;
};

// Splits of one tq_decode_attn call.  Automatic split size with the
// matrix-core scan: balanced splits, planned on the device from the
// sequence lengths (nwg work-groups, one partial slot each); otherwise a
// fixed number of splits per kv head (nparts = batch * hkv * splits).
struct SplitPlan {
  bool balanced;
  int pps, splits;  // fixed splits
  int nwg;          // balanced: work-groups launched
  size_t nparts;    // partial slots
};

SplitPlan split_plan(const tq_ctx* c, int batch, int max_pages, int pages_per_split) {
  SplitPlan sp{};
  const long long bh = static_cast<long long>(batch) * c->p.num_kv_heads;
  // (prep gives the plan a grid row of its own: batch + 1 rows)
  sp.balanced = pages_per_split == 0 && max_pages > 0 && (c->p.flags & TQ_FLAG_VALU_SCAN) == 0 && batch < 65535;
  sp.splits = decode_splits(batch, c->p.num_kv_heads, max_pages, pages_per_split, c->scan_slots, &sp.pps);
  if (sp.balanced) {
    // every kv head gets at least one split and a split at most
    // kMaxSplitPages pages, so bh * ceil(max_pages / kMaxSplitPages) bounds the plan
    const long long per = (max_pages + tq::kMaxSplitPages - 1) / tq::kMaxSplitPages;
    const long long n = std::max<long long>(c->scan_slots > 0 ? c->scan_slots : 1, bh * std::max<long long>(per, 1));
    sp.nwg = static_cast<int>(std::min<long long>(n, 1LL << 30));
    sp.nparts = static_cast<size_t>(sp.nwg);
  } else {
    sp.nparts = static_cast<size_t>(bh) * sp.splits;
  }
  return sp;
}

WsLayout ws_layout(const tq_params& p, int batch, const SplitPlan& sp) {
  const int G = p.num_q_heads / p.num_kv_heads;
  const size_t d = tq::transform_dim(p.head_dim);  // workspace rows hold D coordinates
  const size_t bq = static_cast<size_t>(batch) * p.num_q_heads;
  const size_t nbh = static_cast<size_t>(batch) * p.num_kv_heads;
  const size_t nb = sp.nparts * G;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  WsLayout w{};
  size_t off = 0;
  w.qs = off; off += up(bq * d * 4);
  w.ps = off; off += up(bq * d * 4);
  w.psum = off; off += up(bq * 4);
  w.wm = off; off += up(bq * 4);
  w.wl = off; off += up(bq * 4);
  w.wacc = off; off += up(bq * d * 4);
  w.pm = off; off += up(nb * 4);
  w.pl = off; off += up(nb * 4);
  w.pacc = off; off += up(nb * d * 4);
  w.ctr = off; off += up(nbh * 4);
  w.plan = off; off += sp.balanced ? up(static_cast<size_t>(sp.nwg) * 16) : 0;
  w.sbase = off; off += sp.balanced ? up((nbh + 1) * 4) : 0;
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

TQ_API const char* tq_strerror(int err) {
  switch (err) {
    case TQ_OK: return "ok";
    case TQ_ERR_INVALID_ARG: return "invalid argument";
    case TQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case TQ_ERR_WORKSPACE: return "workspace too small";
    case TQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown error";
  }
}

TQ_API int64_t tq_page_bytes(const tq_params* p) {
  if (!params_ok(p)) return TQ_ERR_INVALID_ARG;
  return tq::make_layout(*p).page_bytes;
}

TQ_API int tq_seed_draws(uint64_t seed, int stream, int64_t n, double* out) {
  if (!out || n < 0 || n > (int64_t(1) << 40)) return TQ_ERR_INVALID_ARG;
  if (stream != TQ_DRAWS_ROTATION && stream != TQ_DRAWS_QJL && stream != TQ_DRAWS_HADAMARD)
    return TQ_ERR_INVALID_ARG;
  tq::seed_normals(seed, stream, n, out);
  return TQ_OK;
}

TQ_API int tq_host_tables(const tq_params* p, const double* rot_draws, const double* qjl_draws, float* rotation,
                          float* qjl, float* key_centroids, float* key_boundaries, float* value_centroids,
                          float* value_boundaries) {
  if (!params_ok(p)) return TQ_ERR_INVALID_ARG;
  // tables act on the transform size D (rows zero-padded from head_dim)
  const int d = tq::transform_dim(p->head_dim);
  // draws not given: the seeded generator's streams
  std::vector<double> gen_rot, gen_qjl;
  if (!rot_draws && rotation) {
    gen_rot.resize(p->rotation == TQ_ROT_DENSE ? static_cast<size_t>(d) * d : d);
    tq::seed_normals(p->seed, p->rotation == TQ_ROT_DENSE ? TQ_DRAWS_ROTATION : TQ_DRAWS_HADAMARD,
                     static_cast<int64_t>(gen_rot.size()), gen_rot.data());
    rot_draws = gen_rot.data();
  }
  if (!qjl_draws && qjl) {
    gen_qjl.resize(static_cast<size_t>(d) * d);
    tq::seed_normals(p->seed, TQ_DRAWS_QJL, static_cast<int64_t>(gen_qjl.size()), gen_qjl.data());
    qjl_draws = gen_qjl.data();
  }
  if (rotation) {
    if (p->rotation == TQ_ROT_DENSE) {
      tq::haar_rotation_f32(rot_draws, d, rotation);
    } else {
      for (int i = 0; i < d; ++i) rotation[i] = rot_draws[i] < 0.0 ? -1.0f : 1.0f;
    }
  }
  if (qjl) {
    if (p->qjl_kind == TQ_QJL_ORTHOGONAL)
      tq::haar_rotation_f32(qjl_draws, d, qjl);  // Haar orthogonal S from the draws
    else
      for (int i = 0; i < d * d; ++i) qjl[i] = static_cast<float>(qjl_draws[i]);
  }
  tq::codebook_f32(p->key_bits, d, key_centroids, key_boundaries);
  tq::codebook_f32(p->value_bits, d, value_centroids, value_boundaries);
  // mixed-channel rates: the (b+1)-bit codebook follows the b-bit one
  auto after = [](float* a, int n) { return a ? a + n : nullptr; };
  if (p->key_mixed)
    tq::codebook_f32(p->key_bits + 1, d, after(key_centroids, 1 << p->key_bits),
                     after(key_boundaries, (1 << p->key_bits) - 1));
  if (p->value_mixed)
    tq::codebook_f32(p->value_bits + 1, d, after(value_centroids, 1 << p->value_bits),
                     after(value_boundaries, (1 << p->value_bits) - 1));
  return TQ_OK;
}

}  // extern "C"

namespace {

// Caller-given levels of one kind, rounded to the stored half-precision
// values, with the boundaries between them (midpoints, float32); 2^b levels,
// or 2^b then 2^(b+1) for a mixed rate (two ascending runs).  False for a
// non-finite level or a run that is not strictly increasing once rounded.
bool caller_codebook(const float* cen, int bits, bool mixed, float* c, float* bnd) {
  int off = 0, boff = 0;
  for (int part = 0; part < (mixed ? 2 : 1); ++part) {
    const int L = 1 << (bits + part);
    for (int k = 0; k < L; ++k) {
      if (!std::isfinite(cen[off + k])) return false;
      c[off + k] = static_cast<float>(static_cast<_Float16>(cen[off + k]));
      if (k > 0 && !(c[off + k] > c[off + k - 1])) return false;
    }
    for (int k = 0; k + 1 < L; ++k)
      bnd[boff + k] =
          static_cast<float>(0.5 * (static_cast<double>(c[off + k]) + static_cast<double>(c[off + k + 1])));
    off += L;
    boff += L - 1;
  }
  return true;
}

// A context from finished tables: the rotation (Pi row-major, or the
// Hadamard signs), the QJL matrix S as used (ignored without QJL) and the
// codebooks with their boundaries, laid out as tq_host_tables writes them.
int init_ctx(tq_ctx** out, const tq_params* p, const float* rot_in, const float* S_in, const float* kc,
             const float* kb, const float* vc, const float* vb, void* stream) {
  *out = nullptr;
  const int d = tq::transform_dim(p->head_dim);  // table size D
  tq_ctx* c = new (std::nothrow) tq_ctx();
  if (!c) return TQ_ERR_HIP;
  c->p = *p;
  c->lay = tq::make_layout(*p);
  std::vector<float> rot(d * d, 0.0f), rotT(d * d, 0.0f), S(d * d, 0.0f), ST(d * d, 0.0f);
  std::memcpy(rot.data(), rot_in, (p->rotation == TQ_ROT_DENSE ? d * d : d) * sizeof(float));
  if (p->key_qjl) std::memcpy(S.data(), S_in, d * d * sizeof(float));
  std::memset(&c->cb, 0, sizeof(c->cb));
  const int nk = 1 << p->key_bits, nv = 1 << p->value_bits;
  std::memcpy(c->cb.kc, kc, nk * sizeof(float));
  std::memcpy(c->cb.kb, kb, (nk - 1) * sizeof(float));
  std::memcpy(c->cb.vc, vc, nv * sizeof(float));
  std::memcpy(c->cb.vb, vb, (nv - 1) * sizeof(float));
  if (p->key_mixed) {
    std::memcpy(c->cb.kc2, kc + nk, 2 * nk * sizeof(float));
    std::memcpy(c->cb.kb2, kb + nk - 1, (2 * nk - 1) * sizeof(float));
  }
  if (p->value_mixed) {
    std::memcpy(c->cb.vc2, vc + nv, 2 * nv * sizeof(float));
    std::memcpy(c->cb.vb2, vb + nv - 1, (2 * nv - 1) * sizeof(float));
  }
  if (p->rotation == TQ_ROT_DENSE) transpose(rot.data(), rotT.data(), d);
  transpose(S.data(), ST.data(), d);
  // row-owner layouts for the few-token append: lane i reads M[i][4 j4 .. 4 j4 + 3] as one float4
  std::vector<float> rot4(d * d, 0.0f), S4(d * d, 0.0f);
  for (int j4 = 0; j4 < d / 4; ++j4)
    for (int i = 0; i < d; ++i)
      for (int q = 0; q < 4; ++q) {
        if (p->rotation == TQ_ROT_DENSE) rot4[(j4 * d + i) * 4 + q] = rot[i * d + 4 * j4 + q];
        S4[(j4 * d + i) * 4 + q] = S[i * d + 4 * j4 + q];
      }
  c->h_rot = rot;
  c->h_S = S;
  const size_t mat = static_cast<size_t>(d) * d * sizeof(float);
  // codebooks as a device table (the few-token append reads them into LDS)
  float cbtab[128] = {};
  for (int k = 0; k < 16; ++k) {
    cbtab[k] = c->cb.kc[k];
    cbtab[16 + k] = c->cb.kb[k];
    cbtab[32 + k] = c->cb.kc2[k];
    cbtab[48 + k] = c->cb.kb2[k];
    cbtab[64 + k] = c->cb.vc[k];
    cbtab[80 + k] = c->cb.vb[k];
    cbtab[96 + k] = c->cb.vc2[k];
    cbtab[112 + k] = c->cb.vb2[k];
  }
  // u8 log-norm: levels 2^(q/16 - 4) (level 0 = 0) and the boundaries
  // between levels q and q + 1 (entry 0: 0, entry 255: +inf), in float32
  float ntab[2 * tq::kNormCodes];
  for (int q = 0; q < tq::kNormCodes; ++q) {
    ntab[q] = q == 0 ? 0.0f : static_cast<float>(std::exp2(q / 16.0 - 4.0));
    ntab[tq::kNormCodes + q] = q == 0 ? 0.0f
                               : q == tq::kNormCodes - 1 ? std::numeric_limits<float>::infinity()
                                                         : static_cast<float>(std::exp2((q + 0.5) / 16.0 - 4.0));
  }
  const size_t ctr_bytes = sizeof(int) * static_cast<size_t>(tq::kAppendSlots) * tq::kAppendMaxBatch;
  const size_t total = 6 * mat + sizeof(cbtab) + sizeof(ntab) + 256 + ctr_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipGetDevice(&c->device) != hipSuccess || hipMalloc(&c->dmem, total) != hipSuccess) {
    delete c;
    return TQ_ERR_HIP;
  }
  char* base = static_cast<char*>(c->dmem);
  c->t.rot = reinterpret_cast<float*>(base);
  c->t.rotT = reinterpret_cast<float*>(base + mat);
  c->t.S = reinterpret_cast<float*>(base + 2 * mat);
  c->t.ST = reinterpret_cast<float*>(base + 3 * mat);
  c->t.rot4 = reinterpret_cast<float*>(base + 4 * mat);
  c->t.S4 = reinterpret_cast<float*>(base + 5 * mat);
  c->t.cbtab = reinterpret_cast<float*>(base + 6 * mat);
  c->t.ntab = reinterpret_cast<float*>(base + 6 * mat + sizeof(cbtab));
  c->t.status = reinterpret_cast<int*>(base + 6 * mat + sizeof(cbtab) + sizeof(ntab));
  c->append_ctr = reinterpret_cast<int*>(base + 6 * mat + sizeof(cbtab) + sizeof(ntab) + 256);
  bool ok = hipMemcpyAsync(base, rot.data(), mat, hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemcpyAsync(base + mat, rotT.data(), mat, hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemcpyAsync(base + 2 * mat, S.data(), mat, hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemcpyAsync(base + 3 * mat, ST.data(), mat, hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemcpyAsync(base + 4 * mat, rot4.data(), mat, hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemcpyAsync(base + 5 * mat, S4.data(), mat, hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemcpyAsync(base + 6 * mat, cbtab, sizeof(cbtab), hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemcpyAsync(base + 6 * mat + sizeof(cbtab), ntab, sizeof(ntab), hipMemcpyHostToDevice, s) == hipSuccess &&
            hipMemsetAsync(base + 6 * mat + sizeof(cbtab) + sizeof(ntab), 0, 256 + ctr_bytes, s) == hipSuccess &&
            hipStreamSynchronize(s) == hipSuccess;
  // resident scan work-groups per device, for the automatic split count
  const bool valu = (p->flags & TQ_FLAG_VALU_SCAN) != 0;
  const void* kf = valu ? tq::scan_valu_kernel_ptr(c) : tq::scan_mfma_kernel_ptr(c);
  const int threads = valu ? tq::kScanThreads : tq::scan_mfma_threads(c);
  int per_cu = 0, cus = 0;
  ok = ok && kf && hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kf, threads, 0) == hipSuccess &&
       hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device) == hipSuccess;
  if (!ok) {
    (void)hipFree(c->dmem);
    delete c;
    return TQ_ERR_HIP;
  }
  c->scan_slots = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  // the static scratch of the allocation-free decode: its address on this device
  if (tq::static_scratch_init(c->device) != 0) {
    (void)hipFree(c->dmem);
    delete c;
    return TQ_ERR_HIP;
  }
  *out = c;
  return TQ_OK;
}

}  // namespace

extern "C" {

TQ_API int tq_codebook_init(tq_ctx** out, const tq_params* p, const double* rot_draws, const double* qjl_draws,
                            void* stream) {
  if (!out || !params_ok(p)) return TQ_ERR_INVALID_ARG;
  if (!params_supported(p)) return TQ_ERR_UNSUPPORTED;
  *out = nullptr;
  const int d = tq::transform_dim(p->head_dim);  // table size D
  std::vector<float> rot(d * d, 0.0f), S(d * d, 0.0f);
  float kc[48] = {}, kb[48] = {}, vc[48] = {}, vb[48] = {};
  const int rc =
      tq_host_tables(p, rot_draws, qjl_draws, rot.data(), p->key_qjl ? S.data() : nullptr, kc, kb, vc, vb);
  if (rc != TQ_OK) return rc;
  return init_ctx(out, p, rot.data(), S.data(), kc, kb, vc, vb, stream);
}

TQ_API int tq_codebook_init_tables(tq_ctx** out, const tq_params* p, const tq_tables* tables, void* stream) {
  if (!out || !params_ok(p)) return TQ_ERR_INVALID_ARG;
  if (!params_supported(p)) return TQ_ERR_UNSUPPORTED;
  *out = nullptr;
  const int d = tq::transform_dim(p->head_dim);  // table size D
  const tq_tables none = {nullptr, nullptr, nullptr, nullptr};
  const tq_tables& t = tables ? *tables : none;
  // the seeded tables for whatever the caller leaves out
  std::vector<float> rot(d * d, 0.0f), S(d * d, 0.0f);
  float kc[48] = {}, kb[48] = {}, vc[48] = {}, vb[48] = {};
  const int rc = tq_host_tables(p, nullptr, nullptr, t.rotation ? nullptr : rot.data(),
                                (p->key_qjl && !t.qjl) ? S.data() : nullptr, kc, kb, vc, vb);
  if (rc != TQ_OK) return rc;
  if (t.rotation) {
    const int n = p->rotation == TQ_ROT_DENSE ? d * d : d;
    for (int i = 0; i < n; ++i) {
      const float v = t.rotation[i];
      if (!std::isfinite(v) || (p->rotation == TQ_ROT_HADAMARD && v != 1.0f && v != -1.0f))
        return TQ_ERR_INVALID_ARG;
      rot[i] = v;
    }
  }
  if (p->key_qjl && t.qjl) {
    for (int i = 0; i < d * d; ++i) {
      if (!std::isfinite(t.qjl[i])) return TQ_ERR_INVALID_ARG;
      S[i] = t.qjl[i];
    }
  }
  if (t.key_centroids && !caller_codebook(t.key_centroids, p->key_bits, p->key_mixed != 0, kc, kb))
    return TQ_ERR_INVALID_ARG;
  if (t.value_centroids && !caller_codebook(t.value_centroids, p->value_bits, p->value_mixed != 0, vc, vb))
    return TQ_ERR_INVALID_ARG;
  return init_ctx(out, p, rot.data(), S.data(), kc, kb, vc, vb, stream);
}

TQ_API int tq_destroy(tq_ctx* c) {
  if (!c) return TQ_ERR_INVALID_ARG;
  int rc = TQ_OK;
  if (c->dmem && hipFree(c->dmem) != hipSuccess) rc = TQ_ERR_HIP;
  delete c;
  return rc;
}

TQ_API int tq_profile_begin(tq_ctx* c, int max_calls) {
  if (!c || max_calls < 0 || max_calls > 100000) return TQ_ERR_INVALID_ARG;
  int rc = TQ_OK;
  for (void* e : c->prof_events)
    if (hipEventDestroy(static_cast<hipEvent_t>(e)) != hipSuccess) rc = TQ_ERR_HIP;
  c->prof_events.clear();
  c->prof_next = 0;
  for (int i = 0; i < 2 * max_calls; ++i) {
    hipEvent_t e;
    // timing-only events: no system-scope fence (cache writeback and
    // invalidate) when they are recorded, which would lengthen the interval
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return TQ_ERR_HIP;
    c->prof_events.push_back(e);
  }
  return rc;
}

TQ_API int tq_profile_end(tq_ctx* c, double* scan_ms_total, int* calls) {
  if (!c || !scan_ms_total || !calls) return TQ_ERR_INVALID_ARG;
  double tot = 0.0;
  int rc = TQ_OK;
  for (int i = 0; i < c->prof_next; ++i) {
    hipEvent_t a = static_cast<hipEvent_t>(c->prof_events[2 * i]);
    hipEvent_t b = static_cast<hipEvent_t>(c->prof_events[2 * i + 1]);
    float ms = 0.0f;
    if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&ms, a, b) != hipSuccess) rc = TQ_ERR_HIP;
    tot += ms;
  }
  *scan_ms_total = tot;
  *calls = c->prof_next;
  for (void* e : c->prof_events)
    if (hipEventDestroy(static_cast<hipEvent_t>(e)) != hipSuccess) rc = TQ_ERR_HIP;
  c->prof_events.clear();
  c->prof_next = 0;
  return rc;
}

TQ_API int tq_get_status(tq_ctx* c, int* code) {
  if (!c || !code) return TQ_ERR_INVALID_ARG;
  int prev = 0;
  if (hipSetDevice(c->device) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
      hipMemcpy(&prev, c->t.status, sizeof(int), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemset(c->t.status, 0, sizeof(int)) != hipSuccess || hipDeviceSynchronize() != hipSuccess)
    return TQ_ERR_HIP;
  *code = prev;
  return TQ_OK;
}

TQ_API int tq_encode(const tq_ctx* c, int kind, const void* x, int dtype, int64_t n, int64_t row_stride,
                     uint8_t* codes, uint8_t* signs, float* norms, float* rnorms, void* stream) {
  if (!c || (kind != TQ_KIND_KEY && kind != TQ_KIND_VALUE)) return TQ_ERR_INVALID_ARG;
  if (dtype != TQ_DTYPE_F16 && dtype != TQ_DTYPE_BF16 && dtype != TQ_DTYPE_F32) return TQ_ERR_INVALID_ARG;
  if (n < 0 || row_stride < c->p.head_dim) return TQ_ERR_INVALID_ARG;
  if (n == 0) return TQ_OK;
  const bool qjl = kind == TQ_KIND_KEY && c->p.key_qjl;
  if (!x || !codes || !norms || (qjl && (!signs || !rnorms))) return TQ_ERR_INVALID_ARG;
  const size_t esz = dtype == TQ_DTYPE_F32 ? 4 : 2;
  if (!aligned(x, esz) || !aligned(codes, 4) || !aligned(norms, 4) || (qjl && (!aligned(signs, 4) || !aligned(rnorms, 4))))
    return TQ_ERR_INVALID_ARG;
  if (n > (int64_t(1) << 40)) return TQ_ERR_INVALID_ARG;
  tq::EncodeArgs a{x, n, row_stride, c->p.head_dim, codes, qjl ? signs : nullptr, norms, qjl ? rnorms : nullptr};
  return tq::launch_encode(c, kind, dtype, a, stream) == 0 ? TQ_OK : TQ_ERR_HIP;
}

TQ_API int tq_decode(const tq_ctx* c, int kind, const uint8_t* codes, const uint8_t* signs, const float* norms,
                     const float* rnorms, int64_t n, float* out, void* stream) {
  if (!c || (kind != TQ_KIND_KEY && kind != TQ_KIND_VALUE) || n < 0) return TQ_ERR_INVALID_ARG;
  if (n == 0) return TQ_OK;
  const bool qjl = kind == TQ_KIND_KEY && c->p.key_qjl;
  if (!codes || !norms || !out || (qjl && (!signs || !rnorms))) return TQ_ERR_INVALID_ARG;
  if (!aligned(codes, 4) || !aligned(norms, 4) || !aligned(out, 16) || (qjl && (!aligned(signs, 4) || !aligned(rnorms, 4))))
    return TQ_ERR_INVALID_ARG;
  if (n > (int64_t(1) << 40)) return TQ_ERR_INVALID_ARG;
  return tq::launch_dequant(c, kind, codes, qjl ? signs : nullptr, norms, qjl ? rnorms : nullptr, n, out, stream) == 0
             ? TQ_OK
             : TQ_ERR_HIP;
}

TQ_API int tq_append_page(const tq_ctx* c, uint8_t* pool, int64_t num_pages, const int32_t* block_table,
                          int max_pages, int batch, int32_t* seq_lens, const uint16_t* k_new, const uint16_t* v_new,
                          int n_new, const int32_t* new_counts, uint16_t* k_win, uint16_t* v_win, void* stream) {
  if (!c || batch < 0 || n_new < 0 || max_pages < 0 || num_pages < 0) return TQ_ERR_INVALID_ARG;
  if (batch == 0 || n_new == 0) return TQ_OK;
  if (batch > 65535) return TQ_ERR_INVALID_ARG;
  if (!seq_lens || !k_new || !v_new || !block_table || !pool) return TQ_ERR_INVALID_ARG;
  if (c->p.window > 0 && (!k_win || !v_win)) return TQ_ERR_INVALID_ARG;
  if (!aligned(pool, 256) || !aligned(k_new, 16) || !aligned(v_new, 16) ||
      (c->p.window > 0 && (!aligned(k_win, 16) || !aligned(v_win, 16))))
    return TQ_ERR_INVALID_ARG;
  tq::AppendArgs a{pool, num_pages, block_table, max_pages, batch, seq_lens, k_new, v_new, n_new, new_counts, k_win, v_win};
  return tq::launch_append(c, a, stream) == 0 ? TQ_OK : TQ_ERR_HIP;
}

TQ_API int64_t tq_decode_workspace_bytes(const tq_ctx* c, int batch, int max_pages, int pages_per_split) {
  if (!c || batch < 0 || max_pages < 0 || pages_per_split < 0) return TQ_ERR_INVALID_ARG;
  return static_cast<int64_t>(ws_layout(c->p, batch, split_plan(c, batch, max_pages, pages_per_split)).total);
}

TQ_API int tq_decode_attn(const tq_ctx* c, const void* q, int q_dtype, const uint8_t* pool, int64_t num_pages,
                          const int32_t* block_table, int max_pages, int batch, const int32_t* seq_lens,
                          const uint16_t* k_win, const uint16_t* v_win, float sm_scale, float* out, void* workspace,
                          size_t workspace_bytes, int pages_per_split, float* dbg_logits, int64_t logits_stride,
                          void* stream) {
  if (!c || batch < 0 || max_pages < 0 || num_pages < 0 || pages_per_split < 0) return TQ_ERR_INVALID_ARG;
  if (q_dtype != TQ_DTYPE_F16 && q_dtype != TQ_DTYPE_BF16 && q_dtype != TQ_DTYPE_F32) return TQ_ERR_INVALID_ARG;
  if (!std::isfinite(sm_scale)) return TQ_ERR_INVALID_ARG;
  if (batch == 0) return TQ_OK;
  if (batch > 65535) return TQ_ERR_INVALID_ARG;
  if (!q || !seq_lens || !out || !workspace) return TQ_ERR_INVALID_ARG;
  if (max_pages > 0 && (!pool || !block_table)) return TQ_ERR_INVALID_ARG;
  if (c->p.window > 0 && (!k_win || !v_win)) return TQ_ERR_INVALID_ARG;
  if (dbg_logits && logits_stride < 1) return TQ_ERR_INVALID_ARG;
  if ((pool && !aligned(pool, 256)) || !aligned(out, 16) || !aligned(workspace, 256) ||
      !aligned(q, q_dtype == TQ_DTYPE_F32 ? 16 : 8))
    return TQ_ERR_INVALID_ARG;
  const SplitPlan sp = split_plan(c, batch, max_pages, pages_per_split);
  const WsLayout w = ws_layout(c->p, batch, sp);
  if (workspace_bytes < w.total) return TQ_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  tq::DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.pool = pool;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.batch = batch;
  a.seq_lens = seq_lens;
  a.k_win = k_win;
  a.v_win = v_win;
  a.sm_scale = sm_scale;
  a.out = out;
  a.dbg_logits = dbg_logits;
  a.logits_stride = logits_stride;
  a.pages_per_split = sp.pps;
  a.splits = sp.splits;
  a.slots = c->scan_slots > 0 ? c->scan_slots : 1;
  if (sp.balanced) {
    a.nwg = sp.nwg;
    a.plan = reinterpret_cast<int4*>(base + w.plan);
    a.sbase = reinterpret_cast<int*>(base + w.sbase);
  }
  a.qs = reinterpret_cast<float*>(base + w.qs);
  a.ps = reinterpret_cast<float*>(base + w.ps);
  a.psum = reinterpret_cast<float*>(base + w.psum);
  a.wm = reinterpret_cast<float*>(base + w.wm);
  a.wl = reinterpret_cast<float*>(base + w.wl);
  a.wacc = reinterpret_cast<float*>(base + w.wacc);
  a.ctr = reinterpret_cast<int*>(base + w.ctr);
  a.pm = reinterpret_cast<float*>(base + w.pm);
  a.pl = reinterpret_cast<float*>(base + w.pl);
  a.pacc = reinterpret_cast<float*>(base + w.pacc);
  return tq::launch_decode(c, a, stream) == 0 ? TQ_OK : TQ_ERR_HIP;
}

TQ_API int tq_decode_attn_noalloc(const tq_ctx* c, const void* q, int q_dtype, const uint8_t* pool,
                                  int64_t num_pages, const int32_t* block_table, int max_pages, int batch,
                                  const int32_t* seq_lens, const uint16_t* k_win, const uint16_t* v_win,
                                  float sm_scale, float* out, int pages_per_split, void* stream) {
  if (!c || batch < 0 || max_pages < 0 || pages_per_split < 0) return TQ_ERR_INVALID_ARG;
  const int64_t need = tq_decode_workspace_bytes(c, batch, max_pages, pages_per_split);
  if (need < 0) return static_cast<int>(need);
  if (need > static_cast<int64_t>(TQ_NOALLOC_SCRATCH_BYTES)) return TQ_ERR_WORKSPACE;
  void* ws = tq::static_scratch_ptr(c->device);
  if (!ws) return TQ_ERR_HIP;
  return tq_decode_attn(c, q, q_dtype, pool, num_pages, block_table, max_pages, batch, seq_lens, k_win, v_win,
                        sm_scale, out, ws, static_cast<size_t>(TQ_NOALLOC_SCRATCH_BYTES), pages_per_split, nullptr, 0,
                        stream);
}

}  // extern "C"

namespace tq {
// which = 0: start event of this call's scan (claims a slot), 1: its stop event.
void* profile_slot(const tq_ctx* c, int which) {
  if (which == 0) {
    if (2 * (c->prof_next + 1) > static_cast<int>(c->prof_events.size())) return nullptr;
    return c->prof_events[2 * c->prof_next];
  }
  void* e = c->prof_events[2 * c->prof_next + 1];
  ++c->prof_next;
  return e;
}
}  // namespace tq
