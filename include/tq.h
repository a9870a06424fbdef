/*
 * tq.h - C ABI of the TurboQuant compressed KV-cache library for AMD MI355X
 * (gfx950).  Plain pointers and sizes only; every device pointer is memory the
 * caller owns (the library owns only the constant tables inside a tq_ctx).
 *
 * Method sources (web pages this library implements):
 *  - "aither-kvcache" PyPI README, section "Algorithm": normalise (L2 norm
 *    stored as f32), rotate by a fixed random orthogonal matrix, quantise each
 *    coordinate with a precomputed Lloyd-Max codebook, pack the indices.
 *  - "TurboQuant on a 16GB MacBook" (yashrajpandey.com), sections "Why this
 *    caught my eye" and "The QJL detective story": for keys, a 1-bit QJL sketch
 *    sign(S r) of the quantisation residual r with Gaussian S, dequantised
 *    with scale sqrt(pi/2)/d.
 *  - "TurboQuant Family Design Study for CPU and Browser WASM KV Caches"
 *    (iarpg.com): post-RoPE placement and the query transformed into the same
 *    basis (section "Placement relative to RoPE and attention"), fixed-size
 *    pages with a 64-byte header and a recent FP16 window (sections "Packed
 *    format and complete bit accounting", "Paging, lifecycle, and cache
 *    identity"), compressed-domain key scan and rotated-domain value
 *    accumulation with one inverse transform per head (section "CPU and WASM
 *    kernel design"), the randomized Hadamard transform (section "Dense and
 *    structured transform comparison").
 *
 * Conventions
 *  - All calls return 0 (TQ_OK) or a negative TQ_ERR_* code; arguments are
 *    validated on the host before anything is launched, and a failing call
 *    launches nothing.  No exceptions cross the ABI.
 *  - Calls that take a stream enqueue asynchronous work on it (a hipStream_t
 *    passed as void*; NULL is the default stream) and do not synchronise,
 *    except tq_codebook_init (uploads tables, then synchronises the stream)
 *    and tq_get_status (reads the status word back).  No device memory is
 *    allocated in hot calls.  A tq_ctx is immutable after init apart from its
 *    status word, its profiling slots (tq_profile_begin) and the arrival
 *    counts of decode-step appends (8 sets, taken in turn, each back at zero
 *    when its call ends), so calls on different streams may share it while
 *    profiling is off, with at most 8 appends in flight at once.
 *  - Head size d and transform size D: D is the next power of two >= d.  A
 *    head size that is not a power of two is zero-padded to D for the
 *    rotation and the QJL sketch, and its records hold all D transform
 *    coordinates ("TurboQuant Family Design Study", "Dense and structured
 *    transform comparison": temporary zero-padding during append and the
 *    query transform; storing all D coordinates keeps the transform
 *    invertible, so q.k = (Tq).(Tk) still holds).  FP16 rows, queries and
 *    outputs hold d coordinates.  The kernels are built for D = 128: head
 *    sizes 72..128 in steps of 8; tq_codebook_init returns
 *    TQ_ERR_UNSUPPORTED for other sizes, which the host-only calls accept.
 *
 * Page format (one page = one layer x one sequence x P tokens x all H_kv heads):
 *   page_bytes = roundup(256 + H_kv * head_bytes, 256); 64-byte header at 0
 *   (u32 magic 0x564B5154, u16 version 1, u16 d (the head size), u8 key_bits, u8 key QJL
 *   (0 none, 1 Gaussian S, 2 orthogonal S),
 *   u8 value_bits, u8 rotation, u16 H_kv, u16 P, u32 valid tokens, u32
 *   codebook version 1, u64 seed, u32 page index, u8 key norm format (0 f32,
 *   1 u8 log-norm), zeros); head h's body at 256 + h * head_bytes holds, in
 *   order: key norms f32[P] (u8[P] codes with key_norm_u8); key residual norms
 *   f32[P] (QJL only); key codes u8[P][D*bK/8] token-major, LSB-first; key
 *   signs u8[P][D/8] (QJL only); value norms f32[P]; value codes
 *   u32[P/32][bV][D], where for each 32-token group and coordinate j the bV
 *   words w = 0..bV-1 form a little-endian 32*bV-bit string holding token i's
 *   code at bits [i*bV, (i+1)*bV).
 *   Mixed-channel rates (key_mixed / value_mixed): the header bits byte holds
 *   b + 16; a key record is D*b/8 + D/16 bytes (the D/2 low-rate codes at b
 *   bits, then the D/2 high-rate codes at b + 1 bits, each half in ascending
 *   coordinate order); a value group is a low-rate block u32[bV][D/2] then a
 *   high-rate block u32[bV+1][D/2], coordinates of each half in ascending
 *   order, each coordinate's words forming its 32-token string as above.
 * FP16 window: k_win, v_win [B][H_kv][W][d] fp16; the token at position t
 *   lives in slot t mod W while it is among the last W tokens of its sequence.
 *   A sequence of length T has max(T - W, 0) compressed tokens (positions
 *   0 .. T-W-1, position t in page block_table[b][t / P], slot t mod P).
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_API __attribute__((visibility("default")))

enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = -1, /* null pointer, size out of range, inconsistent shapes */
  TQ_ERR_UNSUPPORTED = -2, /* valid request that this build has no kernel for */
  TQ_ERR_WORKSPACE = -3,   /* workspace smaller than tq_decode_workspace_bytes() */
  TQ_ERR_HIP = -4,         /* a HIP runtime call failed (no device, launch error) */
};

enum { TQ_ROT_DENSE = 0, TQ_ROT_HADAMARD = 1 };
enum { TQ_QJL_GAUSSIAN = 0, TQ_QJL_ORTHOGONAL = 1 };
enum { TQ_DTYPE_F16 = 0, TQ_DTYPE_BF16 = 1, TQ_DTYPE_F32 = 2 };
enum { TQ_KIND_KEY = 0, TQ_KIND_VALUE = 1 };
/* tq_params.flags: TQ_FLAG_VALU_SCAN selects the vector-ALU decode scan
 * instead of the matrix-core one, TQ_FLAG_VALU_APPEND the vector-ALU encoder
 * for bulk appends instead of the matrix-core one (same results to the stated
 * tolerance and guard band; kept for measurement and cross-checking).
 * TQ_FLAG_DETERMINISTIC makes tq_decode_attn bit-reproducible: by default
 * the waves of a matrix-core scan work-group claim the tokens of their page
 * split as they free up, which balances the waves but lets the grouping of
 * the floating-point sums, hence the last bits of the output, vary from call
 * to call (within about 1e-6 relative); with the flag every wave takes a
 * fixed share and repeated calls on the same inputs give identical bits.
 * The vector-ALU scan is always bit-reproducible. */
enum { TQ_FLAG_VALU_SCAN = 1, TQ_FLAG_VALU_APPEND = 2, TQ_FLAG_DETERMINISTIC = 4 };
/* Streams of the library's seeded generator (tq_seed_draws): the Gaussian
 * matrix the dense rotation is built from, the QJL draws, and the draws whose
 * signs are the Hadamard variant's Rademacher stage. */
enum { TQ_DRAWS_ROTATION = 1, TQ_DRAWS_QJL = 2, TQ_DRAWS_HADAMARD = 3 };
/* Size of the static device scratch tq_decode_attn_noalloc works in (32 MiB
 * per device). */
#define TQ_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Bits of the device status word (tq_get_status). */
enum {
  TQ_STATUS_BAD_PAGE = 1, /* a block-table entry needed by a call was < 0 or >= num_pages;
                             that sequence was left unchanged (append) or skipped (decode) */
  TQ_STATUS_BAD_COUNT = 2 /* a per-sequence new-token count was < 0 or > n_new */
};

typedef struct tq_params {
  int32_t head_dim;     /* d, a multiple of 8 (kernels: 72..128) */
  int32_t key_bits;     /* MSE bits per key coordinate, 2..4 */
  int32_t key_qjl;      /* 1: keys carry the QJL sign sketch and residual norm */
  int32_t value_bits;   /* bits per value coordinate, 2..4 */
  int32_t rotation;     /* TQ_ROT_DENSE or TQ_ROT_HADAMARD */
  int32_t num_q_heads;  /* H_q */
  int32_t num_kv_heads; /* H_kv; H_q % H_kv == 0, query head g reads kv head g / (H_q/H_kv) */
  int32_t page_tokens;  /* P, a multiple of 32, at most 1024 */
  int32_t window;       /* W, FP16 recent tokens per sequence, 0..1024 */
  int32_t flags;        /* TQ_FLAG_* bits, 0 for the default kernels and schedule */
  uint64_t seed;        /* recorded in page headers (cache identity); keys the library's generator
                           when the caller gives no draws or tables */
  int32_t qjl_kind;     /* TQ_QJL_GAUSSIAN (the paper's S, coefficient sqrt(pi/2)/D) or
                           TQ_QJL_ORTHOGONAL (S = Haar orthogonal matrix from the same draws,
                           matched coefficient sqrt(pi/2)/sqrt(D)): "TurboQuant on a 16GB
                           MacBook", "The QJL detective story" */
  float qjl_shrink;     /* factor on the QJL correction term in decode, (0, 4]; 1 = unbiased,
                           2/pi = the MMSE shrinkage for orthogonal S (same section, the 0.7
                           damping of the ablation) */
  int32_t key_mixed;    /* 1: mixed-channel rate key_bits + 1/2 (key_bits 2 or 3): the rotated
                           coordinates j with j mod 32 >= 16 take key_bits + 1 bits with their
                           own Lloyd-Max codebook; a record holds the low-rate codes, then the
                           high-rate ones ("TurboQuant Family Design Study", "Packed format and
                           complete bit accounting": 2.5 / 3.5 bits per channel for d = 128) */
  int32_t value_mixed;  /* 1: the same for values, high-rate coordinates j mod 8 >= 4 */
  int32_t key_norm_u8;  /* 1: key norms stored as u8 log-norm codes, one byte per token-head
                           ("TurboQuant Family Design Study", "Packed format and complete bit
                           accounting": the low-overhead modes, 0.0625 bits per channel):
                           code 0 for a zero norm, else the level 2^(q/16 - 4), q = 1..255,
                           nearest in log2 (float32 boundaries 2^((q + 1/2)/16 - 4)); the QJL
                           residual is taken against the stored level */
} tq_params;

typedef struct tq_ctx tq_ctx;

/* Seeded draws ("aither-kvcache" README, "API Reference": a quantiser is
 * built from head_dim, bits and a seed; "Algorithm" step 2: a fixed random
 * orthogonal matrix; "TurboQuant on a 16GB MacBook", "The QJL detective
 * story": a Gaussian QJL matrix).  Writes n N(0,1) values (host double[n]) of
 * one stream (TQ_DRAWS_*) of the generator the library uses when a caller
 * gives it only a seed: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) with key (seed mod
 * 2^32, seed / 2^32); draws 2j and 2j+1 come from the block with counter
 * (j mod 2^32, j / 2^32, stream, 0), whose words w0..w3 give the uniforms
 * u1 = ((w0 >> 5) 2^26 + (w1 >> 6)) 2^-53 and u2 likewise from w2, w3, and
 * Box-Muller gives sqrt(-2 ln(1 - u1)) cos(2 pi u2), then ... sin(2 pi u2).
 * Host only.  TQ_ERR_INVALID_ARG for a null out, n < 0 or an unknown stream. */
TQ_API int tq_seed_draws(uint64_t seed, int stream, int64_t n, double* out);

/* Host-only: compute the constant tables exactly as tq_codebook_init stores
 * them, without touching a GPU ("aither-kvcache" README, "Algorithm":
 * rotation and precomputed Lloyd-Max codebooks; "TurboQuant Family Design
 * Study", "Dense and structured transform comparison": the Rademacher-sign
 * stage of the Hadamard variant; "TurboQuant on a 16GB MacBook", "The QJL
 * detective story": Gaussian S, or the orthogonal S built by QR).
 * Every table acts on the D = next power of two >= d transform coordinates.
 * rot_draws: DENSE: D*D i.i.d. N(0,1) values (row-major) whose QR Q factor,
 * with the signs of diag(R) folded in, is the rotation Pi (y = Pi x);
 * HADAMARD: D values whose signs (x < 0 -> -1, else +1) are the Rademacher
 * stage.  qjl_draws: D*D N(0,1) values: the QJL matrix S itself
 * (TQ_QJL_GAUSSIAN; row i gives sign bit i) or the draws its Haar orthogonal S
 * is built from, like the dense rotation (TQ_QJL_ORTHOGONAL).  Either draw
 * pointer may be NULL: the draws then come from the seeded generator
 * (tq_seed_draws with params->seed; streams TQ_DRAWS_ROTATION or
 * TQ_DRAWS_HADAMARD, and TQ_DRAWS_QJL).
 * Outputs (each nullable): rotation D*D f32 (DENSE: Pi row-major; HADAMARD:
 * the D signs), qjl D*D f32, key/value centroids 2^b f32 (Lloyd-Max levels of
 * N(0,1) times 1/sqrt(D), rounded to half-precision values), key/value
 * boundaries 2^b - 1 f32 (midpoints of the stored levels); with a
 * mixed-channel rate the b-bit arrays are followed by the (b+1)-bit ones
 * (2^b + 2^(b+1) centroids, 2^b - 1 + 2^(b+1) - 1 boundaries).
 * Returns TQ_ERR_INVALID_ARG for bad params. */
TQ_API int tq_host_tables(const tq_params* params, const double* rot_draws, const double* qjl_draws,
                          float* rotation, float* qjl, float* key_centroids, float* key_boundaries,
                          float* value_centroids, float* value_boundaries);

/* Build a context on the current HIP device ("aither-kvcache" README, "API
 * Reference": TurboQuant(head_dim, bits, seed) builds the quantiser once and
 * is shared by encode and decode; "TurboQuant Family Design Study", "Paging,
 * lifecycle, and cache identity": the seed and codebook version identify a
 * cache): computes the tables of tq_host_tables (host, double precision,
 * rounded to f32) from the given draws, or from params->seed where a draw
 * pointer is NULL, and uploads them.  *out receives the context, to be
 * released with tq_destroy.  Host pointers; the stream is used for the
 * upload and synchronised before return.  TQ_ERR_INVALID_ARG for bad
 * params, TQ_ERR_UNSUPPORTED for a parameter set without kernels, TQ_ERR_HIP
 * if the device allocation or upload fails (nothing is left allocated). */
TQ_API int tq_codebook_init(tq_ctx** out, const tq_params* params, const double* rot_draws,
                            const double* qjl_draws, void* stream);

/* Finished tables given as data (host f32 arrays, read during the call). */
typedef struct tq_tables {
  const float* rotation;        /* DENSE: Pi, D*D row-major (y = Pi x); HADAMARD: D signs, each +1 or -1 */
  const float* qjl;             /* S as used, D*D row-major (sign bit i from row i); ignored without QJL */
  const float* key_centroids;   /* 2^bK ascending levels (2^bK then 2^(bK+1) for a mixed key rate) */
  const float* value_centroids; /* likewise for values */
} tq_tables;

/* Build a context from tables given as data ("aither-kvcache" README, "API
 * Reference" and "Algorithm": the quantiser is a rotation, a QJL matrix and
 * precomputed codebooks; a caller that already holds them, for instance to
 * decode a cache written elsewhere ("TurboQuant Family Design Study",
 * "Paging, lifecycle, and cache identity"), passes them in).  Every member of
 * *tables, and tables itself, may be NULL: what is missing is built from
 * params->seed as tq_codebook_init does without draws.  Levels are stored
 * rounded to half precision and the decision boundaries are the midpoints
 * of the stored levels; the rotation and S are used as given (their
 * orthogonality is the caller's responsibility).  TQ_ERR_INVALID_ARG for bad
 * params, a non-finite table entry, a Hadamard sign other than +-1 or levels
 * that are not strictly increasing once rounded; otherwise as
 * tq_codebook_init. */
TQ_API int tq_codebook_init_tables(tq_ctx** out, const tq_params* params, const tq_tables* tables, void* stream);

/* Release a context and its device tables ("aither-kvcache" README, "API
 * Reference": the quantiser object's lifetime).  TQ_ERR_INVALID_ARG for
 * NULL, TQ_ERR_HIP if freeing the device memory fails (the context is
 * released either way). */
TQ_API int tq_destroy(tq_ctx* ctx);

/* Bytes of one page for these params ("TurboQuant Family Design Study",
 * "Packed format and complete bit accounting": fixed-size pages with a
 * 64-byte header, 16-byte aligned streams; the layout is given at the top of
 * this file); TQ_ERR_INVALID_ARG on bad params. */
TQ_API int64_t tq_page_bytes(const tq_params* params);

/* Dequantise n flat records (device pointers) back to vectors ("aither-
 * kvcache" README, "Algorithm", last step; "TurboQuant on a 16GB MacBook",
 * "The QJL detective story" for the key correction):
 *   out[i] = Pi^T ( norms[i] c[codes[i]] + a rnorms[i] S^T (2 sigma_i - 1) )
 * with the correction only for keys with key_qjl and a the context's QJL
 * coefficient: qjl_shrink * sqrt(pi/2)/D for Gaussian S, qjl_shrink *
 * sqrt(pi/2)/sqrt(D) for orthogonal S.  Record layouts as in
 * tq_encode; out: [n][d] f32, the first d of the D coordinates of
 * Pi^T (...).  For quality measurements against exact
 * attention; the decode path never dequantises. */
TQ_API int tq_decode(const tq_ctx* ctx, int kind, const uint8_t* codes, const uint8_t* signs, const float* norms,
                     const float* rnorms, int64_t n, float* out, void* stream);

/* Encode n vectors (device pointers) into flat records ("aither-kvcache"
 * README, "Algorithm": norm, rotation, Lloyd-Max codes, LSB-first packing;
 * "TurboQuant on a 16GB MacBook", "Why this caught my eye": the keys' 1-bit
 * QJL sketch of the residual, with the residual's norm):
 *   x: [n][row_stride] elements of dtype (F16, BF16 or F32), first d used
 *   (zero-padded to D);
 *   codes: [n][D*b/8] u8 LSB-first, b = key_bits or value_bits by kind
 *   ([n][D*b/8 + D/16] for a mixed-channel rate, layout as in the page);
 *   norms: [n] f32 L2 norms (keys with key_norm_u8: the u8 log-norm level each norm is
 *   stored as, 2^(q/16 - 4) or 0, against which the key's QJL residual is taken);
 *   signs: [n][D/8] u8 and rnorms: [n] f32, required iff kind == KEY and key_qjl.
 * A vector with zero norm gets all-zero codes, signs and rnorm ("TurboQuant
 * on a 16GB MacBook", "Round 2: the llama.cpp bug hunt": the zero-block fix).
 * TQ_ERR_INVALID_ARG for null or misaligned pointers (x to its element size,
 * the outputs to 4 bytes) or row_stride < d; TQ_ERR_HIP if a launch fails. */
TQ_API int tq_encode(const tq_ctx* ctx, int kind, const void* x, int dtype, int64_t n, int64_t row_stride,
                     uint8_t* codes, uint8_t* signs, float* norms, float* rnorms, void* stream);

/* Append new tokens to every sequence of one layer's cache (device
 * pointers; "TurboQuant Family Design Study", "Paging, lifecycle, and cache
 * identity": token-order append into fixed pages reserved by the caller,
 * rollback of an append that fails; "Packed format and complete bit
 * accounting": the recent-token FP16 window).
 *   page_pool: num_pages * tq_page_bytes bytes; block_table: [batch][max_pages] page ids;
 *   seq_lens: [batch] tokens held so far, advanced by this call;
 *   k_new, v_new: [batch][H_kv][n_new][d] fp16 (bit patterns as uint16);
 *   new_counts: [batch] tokens to take from each sequence's rows (<= n_new), or NULL for n_new each;
 *   k_win, v_win: [batch][H_kv][W][d] fp16 rings (may be NULL when W == 0).
 * For each sequence, tokens that leave the last-W window are encoded (from their
 * FP16 values) into their page slots, the page headers are rewritten, the new
 * tokens still inside the window go to the ring, and seq_lens[b] grows by its
 * count.  The caller reserves pages: every page a token lands in must be a valid
 * id in block_table.  A sequence whose pages or count are invalid is left
 * unchanged and raises a status bit (tq_get_status).  TQ_ERR_INVALID_ARG
 * for null or misaligned pointers (pool 256 bytes, token rows and rings 16
 * bytes) or negative sizes; TQ_ERR_HIP if a launch fails.  A decode-step
 * append (n_new <= 4, n_new <= W or W == 0) is one kernel: the last of a
 * sequence's work-groups commits it, counting arrivals in one of 8 sets of
 * counters in the context, taken in turn by successive calls; at most 8
 * append calls on one context may therefore be in flight at once (calls on
 * one stream never overlap). */
TQ_API int tq_append_page(const tq_ctx* ctx, uint8_t* page_pool, int64_t num_pages, const int32_t* block_table,
                          int max_pages, int batch, int32_t* seq_lens, const uint16_t* k_new,
                          const uint16_t* v_new, int n_new, const int32_t* new_counts, uint16_t* k_win,
                          uint16_t* v_win, void* stream);

/* Workspace bytes tq_decode_attn needs for this batch, block-table width
 * and split size (rotated queries and the split partials of the online
 * softmax, "TurboQuant Family Design Study", "CPU and WASM kernel design");
 * TQ_ERR_INVALID_ARG for negative sizes. */
TQ_API int64_t tq_decode_workspace_bytes(const tq_ctx* ctx, int batch, int max_pages, int pages_per_split);

/* Decode attention for one query token per sequence (device pointers;
 * "TurboQuant Family Design Study", "Placement relative to RoPE and
 * attention": the query goes through the same transform so q.k = (Tq).(Tk),
 * and "CPU and WASM kernel design": packed keys scored in the compressed
 * domain, values accumulated in the rotated basis, one inverse transform per
 * head; "TurboQuant on a 16GB MacBook", "The QJL detective story": the QJL
 * correction at scale sqrt(pi/2)/D).
 *   q: [batch][H_q][d] post-RoPE queries, dtype F16, BF16 or F32;
 *   cache arguments as in tq_append_page (seq_lens[b] tokens, at most
 *   max_pages * P + W);
 *   sm_scale: logit scale (1/sqrt(d) for standard attention);
 *   out: [batch][H_q][d] f32, softmax(q.k * sm_scale) weighted sum of values
 *   over all seq_lens[b] tokens (zeros for an empty sequence);
 *   workspace: >= tq_decode_workspace_bytes(ctx, batch, max_pages, pages_per_split);
 *   pages_per_split: compressed pages per work-group (at most 64; larger values
 *   are taken as 64); 0 lets the library choose
 *   from the batch, the block-table width and how many scan work-groups the
 *   device holds at once (the fewest rounds of resident work-groups, each
 *   work-group as long as possible);
 *   dbg_logits: NULL, or [batch][H_q][logits_stride] f32 receiving each token's
 *   logit q.k*sm_scale at its position index (for tests).
 * TQ_ERR_INVALID_ARG for null or misaligned pointers (pool and workspace 256
 * bytes, out 16, q 8 or 16) or a non-finite sm_scale, TQ_ERR_WORKSPACE for a
 * workspace below tq_decode_workspace_bytes, TQ_ERR_HIP if a launch fails;
 * invalid page ids met on the device set a status bit (tq_get_status). */
TQ_API int tq_decode_attn(const tq_ctx* ctx, const void* q, int q_dtype, const uint8_t* page_pool, int64_t num_pages,
                          const int32_t* block_table, int max_pages, int batch, const int32_t* seq_lens,
                          const uint16_t* k_win, const uint16_t* v_win, float sm_scale, float* out,
                          void* workspace, size_t workspace_bytes, int pages_per_split, float* dbg_logits,
                          int64_t logits_stride, void* stream);

/* tq_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and kernels, with the workspace taken from a static
 * device array of TQ_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device it runs on until the process ends (its address is looked up once
 * per device, at tq_codebook_init).  The caller passes inputs and outputs as
 * for tq_decode_attn; no logits are captured.  Allocates nothing.  Calls on
 * one device share the array and keep nothing from one call to the next
 * (every word a call reads, it has written): calls that overlap on one device,
 * from different streams or threads, race and must not be made.
 * TQ_ERR_WORKSPACE when tq_decode_workspace_bytes for these sizes exceeds
 * TQ_NOALLOC_SCRATCH_BYTES; otherwise the errors of tq_decode_attn. */
TQ_API int tq_decode_attn_noalloc(const tq_ctx* ctx, const void* q, int q_dtype, const uint8_t* page_pool,
                                  int64_t num_pages, const int32_t* block_table, int max_pages, int batch,
                                  const int32_t* seq_lens, const uint16_t* k_win, const uint16_t* v_win,
                                  float sm_scale, float* out, int pages_per_split, void* stream);

/* Kernel timing for measurement.  tq_profile_begin(ctx, n) arms the context:
 * the next n tq_decode_attn calls record a pair of HIP events on their stream
 * around the compressed-page scan kernel (the kernel that streams the packed
 * cache).  tq_profile_end waits for those events, writes the summed scan time
 * in milliseconds and the number of recorded calls, and disarms the context.
 * While armed, the context must not be used by two threads at once.
 * Returns TQ_ERR_HIP if events cannot be created or read. */
TQ_API int tq_profile_begin(tq_ctx* ctx, int max_calls);
TQ_API int tq_profile_end(tq_ctx* ctx, double* scan_ms_total, int* calls);

/* Streaming-read reference for the bandwidth roofline (no context needed):
 * reads the whole device buffer `buf` (`bytes` > 0, a multiple of 16,
 * 16-byte aligned, caller-owned) with coalesced 16-byte loads and an XOR fold,
 * `reps` times (1..1000) on `stream`, each launch bracketed by HIP events, and
 * writes the fastest launch's time in milliseconds to *best_ms (host).
 * `sink` is a caller-owned 4-byte device word the kernel may write (once in
 * 2^32 fold values).  Synchronises on the events.  The device's read rate is
 * bytes / best_ms; it is the practical ceiling the scan's rate is compared
 * with, beside the nominal HBM peak.  Returns TQ_ERR_INVALID_ARG for bad
 * arguments, TQ_ERR_HIP if a launch or an event fails. */
TQ_API int tq_read_probe(const void* buf, int64_t bytes, uint32_t* sink, int reps, double* best_ms, void* stream);

/* Read and clear the device status word (synchronises the context's device):
 * the device-side error report of appends and decodes ("TurboQuant Family
 * Design Study", "Paging, lifecycle, and cache identity": an append that
 * cannot complete leaves its sequence unchanged).  TQ_ERR_HIP if the read
 * fails. */
TQ_API int tq_get_status(tq_ctx* ctx, int* code);

/* Text for a TQ_ERR_* code (the library's own error convention). */
TQ_API const char* tq_strerror(int err);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
