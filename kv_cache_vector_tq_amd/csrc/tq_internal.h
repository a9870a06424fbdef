// Internal declarations shared by the host API and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <vector>

#include "../../include/tq.h"

namespace tq {

constexpr int kD = 128;           // transform size D the kernels are built for (head_dim 72..128)
constexpr int kBodyOffset = 256;  // page body starts after the 64-byte header and padding
constexpr int kVGroup = 32;       // value codes are interleaved in 32-token groups
constexpr uint32_t kMagic = 0x564B5154u;  // "TQKV"
constexpr int kMaxWindow = 1024;
constexpr int kMaxPage = 1024;
constexpr int kMaxSplitPages = 64;  // pages one decode split reads (its page ids fill one wave's lanes)
constexpr int kNormCodes = 256;   // u8 log-norm codes

// u8 log-norm code of a float32 norm n >= 0 against the boundary table nb
// (nb[q]: between levels q and q + 1; nb[255] = +inf): 0 for n = 0, else the
// level nearest in log2.  A first guess from log2 (off by at most one near a
// boundary) is settled by comparing n with the two boundaries around it.
__host__ __device__ inline int norm_code(float n, const float* nb) {
  if (!(n > 0.0f)) return 0;
  int q = static_cast<int>(floorf(16.0f * (log2f(n) + 4.0f) + 0.5f));
  q = q < 1 ? 1 : (q > kNormCodes - 1 ? kNormCodes - 1 : q);
  if (n > nb[q]) ++q;
  else if (q > 1 && !(n > nb[q - 1])) --q;
  return q;
}

// Transform size D for head size d: the next power of two >= d.  A head
// size that is not a power of two is zero-padded to D for the rotation and
// its records hold all D transform coordinates ("TurboQuant Family Design
// Study", section "Dense and structured transform comparison": temporary
// zero-padding during append and the query transform); FP16 rows, queries
// and outputs keep d coordinates.
__host__ __device__ inline int transform_dim(int d) {
  int D = 1;
  while (D < d) D *= 2;
  return D;
}

// Host table builders (tables.cpp).
std::vector<double> lloyd_max_normal(int bits);
void codebook_f32(int bits, int d, float* centroids, float* boundaries);
void haar_rotation_f32(const double* g, int d, float* out);
// Philox4x32-10 block function (in place on the counter) and the seeded
// N(0,1) draws built on it (stream: TQ_DRAWS_*).
void philox4x32_10(uint32_t ctr[4], const uint32_t key[2]);
void seed_normals(uint64_t seed, int stream, int64_t n, double* out);

// Byte offsets of one head's streams inside its head block, and page sizes.
// kmix / vmix: mixed-channel rate b + 1/2 (half the coordinates at b + 1 bits).
struct Layout {
  int P, bK, bV, qjl, H, kmix, vmix;
  int d;             // head size: FP16 rows (new tokens, ring) hold d coordinates
  int D;             // transform size: records hold D coordinates
  int kn8;           // key norms as u8 log-norm codes
  int k_rec, v_rec;  // code bytes of one key record / one token's value codes
  int64_t k_norm, k_rnorm, k_codes, k_signs, v_norm, v_codes;
  int64_t head_bytes, page_bytes;
};

// Mixed-channel rates: coordinate j takes b + 1 bits when j mod M >= M / 2,
// with M = 32 for keys and 8 for values; a key record (and a value group)
// holds the low-rate half first.  Rank of coordinate j within its half:
constexpr int kKeyHiMod = 32, kValHiMod = 8;
__host__ __device__ inline bool mixed_hi(int j, int mod) { return (j % mod) >= mod / 2; }
__host__ __device__ inline int mixed_rank(int j, int mod) { return (j / mod) * (mod / 2) + (j % mod) % (mod / 2); }
// Coordinate of rank r in the low (hi = 0) or high half.
__host__ __device__ inline int mixed_coord(int r, int hi, int mod) {
  return (r / (mod / 2)) * mod + (hi ? mod / 2 : 0) + r % (mod / 2);
}

inline Layout make_layout(const tq_params& p) {
  Layout l{};
  l.P = p.page_tokens;
  l.bK = p.key_bits;
  l.bV = p.value_bits;
  l.qjl = p.key_qjl ? 1 : 0;
  l.H = p.num_kv_heads;
  l.d = p.head_dim;
  l.D = transform_dim(p.head_dim);
  l.kmix = p.key_mixed ? 1 : 0;
  l.vmix = p.value_mixed ? 1 : 0;
  l.kn8 = p.key_norm_u8 ? 1 : 0;
  l.k_rec = l.D * l.bK / 8 + (l.kmix ? l.D / 16 : 0);
  l.v_rec = l.D * l.bV / 8 + (l.vmix ? l.D / 16 : 0);
  int64_t off = 0;
  l.k_norm = off;
  off += (l.kn8 ? 1LL : 4LL) * l.P;
  l.k_rnorm = off;
  if (l.qjl) off += 4LL * l.P;
  l.k_codes = off;
  off += int64_t(l.P) * l.k_rec;
  l.k_signs = off;
  if (l.qjl) off += int64_t(l.P) * l.D / 8;
  l.v_norm = off;
  off += 4LL * l.P;
  l.v_codes = off;
  off += int64_t(l.P) * l.v_rec;
  l.head_bytes = off;
  l.page_bytes = (kBodyOffset + int64_t(l.H) * off + 255) / 256 * 256;
  return l;
}

// Device-resident constant tables (one allocation owned by the context).
struct DevTables {
  const float* rot;    // DENSE: Pi [D][D] row-major; HADAMARD: signs [D]
  const float* rotT;   // DENSE: Pi^T [D][D] row-major
  const float* S;      // QJL matrix [D][D] row-major (sign bit i from row i)
  const float* ST;     // S^T [D][D] row-major
  const float* rot4;   // DENSE: Pi interleaved by 4 columns: float4 (j4, i) = Pi[i][4 j4 .. 4 j4 + 3]
  const float* S4;     // S interleaved the same way
  const float* cbtab;  // [keys, values][64]: centroids[16], boundaries[16], then the (b+1)-bit pair of a mixed rate
  const float* ntab;   // u8 log-norm: levels[kNormCodes], then boundaries[kNormCodes] (entry q: between q and q+1)
  int* status;         // status word (TQ_STATUS_* bits)
};

// Codebook values passed by value to kernels (uniform across lanes); the
// "2" arrays are the (b+1)-bit codebooks of mixed-channel rates.
struct Codebooks {
  float kc[16], kb[16], vc[16], vb[16];
  float kc2[16], kb2[16], vc2[16], vb2[16];
};

struct EncodeArgs {
  const void* x;
  int64_t n, row_stride;
  int d;  // coordinates per input row (zero-padded to D)
  uint8_t* codes;
  uint8_t* signs;
  float* norms;
  float* rnorms;
};

struct AppendArgs {
  uint8_t* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int max_pages;
  int batch;
  int32_t* seq_lens;
  const uint16_t* k_new;
  const uint16_t* v_new;
  int n_new;
  const int32_t* counts;
  uint16_t* k_win;
  uint16_t* v_win;
  // per-sequence arrival counts of the one-token append that commits itself
  // (null: a commit kernel follows)
  int* ctr = nullptr;
};

// Arrival counts of the self-committing append: kAppendSlots sets of one
// count per sequence (batch <= 65535), taken in turn by successive calls,
// each count back at zero once its sequence is committed.
constexpr int kAppendSlots = 8;
constexpr int kAppendMaxBatch = 65536;

struct DecodeArgs {
  const void* q;
  int q_dtype;
  const uint8_t* pool;
  int64_t num_pages;
  const int32_t* block_table;
  int max_pages;
  int batch;
  const int32_t* seq_lens;
  const uint16_t* k_win;
  const uint16_t* v_win;
  float sm_scale;
  float* out;
  float* dbg_logits;
  int64_t logits_stride;
  int pages_per_split;
  int splits;     // fixed splits per kv head (plan == nullptr)
  int fuse;       // the matrix-core scan's last work-group per kv head finalizes it
  // balanced splits (matrix-core scan, automatic split size): prep sizes the
  // splits from the sequence lengths; scan work-group j takes plan entry j
  int4* plan;     // [nwg] {b * Hkv + h, split, splits of that kv head, pages per split}; b * Hkv + h < 0: idle
  int* sbase;     // [B * Hkv + 1] first plan entry (= partial slot) of each kv head; last: entries in use
  int nwg;        // scan work-groups launched (plan entries)
  int slots;      // scan work-groups resident at once
  // workspace carve-up
  // (rows of D coordinates; q and out rows hold d)
  float* qs;      // [B][Hq][D] rotated query * sm_scale * log2(e)
  float* ps;      // [B][Hq][D] S q_rot * qjl_scale * sm_scale * log2(e)
  float* psum;    // [B][Hq] sum of ps
  float* wm;      // [B][Hq] FP16 window: max score (log2 units)
  float* wl;      // [B][Hq] FP16 window: sum of 2^(s - wm)
  float* wacc;    // [B][Hq][D] FP16 window: weighted values, original basis
  // split partials: slot (b * Hkv + h) * splits + split, or the plan entry
  float* pm;      // [slots][G] running max (log2 units)
  float* pl;      // [slots][G] running sum
  float* pacc;    // [slots][G][D] rotated-basis accumulator
  int* ctr;       // [B][Hkv] scan work-groups finished (cleared by prep)
};

struct Ctx;  // tq_ctx

// Launchers (return hipError_t as int).
int launch_encode(const tq_ctx* ctx, int kind, int dtype, const EncodeArgs& a, void* stream);
// Matrix-core encoder for fp16 rows (encode_mma.hip): 0 launched, 1 not
// applicable (the caller falls back to the vector-ALU encoder), -1 error.
int launch_encode_mma(const tq_ctx* ctx, int kind, int dtype, const EncodeArgs& a, void* stream);
int launch_append(const tq_ctx* ctx, const AppendArgs& a, void* stream);
// Matrix-core bulk append of one kind (encode_mma.hip): 0 launched, 1 not
// applicable (mixed-channel rate), -1 error.
int launch_append_mma(const tq_ctx* ctx, int kind, const AppendArgs& a, void* stream);
int launch_decode(const tq_ctx* ctx, const DecodeArgs& a, void* stream);
int launch_dequant(const tq_ctx* ctx, int kind, const uint8_t* codes, const uint8_t* signs, const float* norms,
                   const float* rnorms, int64_t n, float* out, void* stream);
// The scan kernel a context's decode launches (MFMA or vector-ALU variant),
// for occupancy queries; nullptr for an unsupported parameter set.
const void* scan_mfma_kernel_ptr(const tq_ctx* ctx);
const void* scan_valu_kernel_ptr(const tq_ctx* ctx);
// Threads per work-group of the MFMA scan for this context's parameters.
int scan_mfma_threads(const tq_ctx* ctx);
// Events to record around the scan kernel of this call (nullptr when not profiling).
void* profile_slot(const tq_ctx* ctx, int which);
// Device address of the allocation-free decode's static scratch
// (decode.hip): static_scratch_init records it for the current device
// (0 on success), static_scratch_ptr returns it (nullptr before init).
int static_scratch_init(int device);
void* static_scratch_ptr(int device);

}  // namespace tq

struct tq_ctx {
  tq_params p;
  // measurement hooks (tq_profile_begin / tq_profile_end)
  mutable std::vector<void*> prof_events;  // hipEvent_t pairs
  mutable int prof_next = 0;
  tq::Layout lay;
  int device;
  void* dmem;
  tq::DevTables t;
  tq::Codebooks cb;
  std::vector<float> h_rot, h_S;
  // scan work-groups resident at once on the device (compute units x
  // work-groups per unit); the automatic split count fills one such round
  int scan_slots = 0;
  // the self-committing append's counts (kAppendSlots x kAppendMaxBatch, in
  // dmem) and the call counter that picks their set
  int* append_ctr = nullptr;
  mutable std::atomic<unsigned> append_calls{0};
};
