"""Python binding of the TurboQuant KV-cache library (libtq.so, HIP for gfx950).

Argument marshalling only: every step of encode, append and decode runs in
the library's HIP kernels; PyTorch supplies device memory and the stream.
The function names mirror the C ABI in include/tq.h.  Importing this module
does not build anything; ``kv_cache_vector_tq_amd.build.build()`` does.
"""

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libtq.so")

TQ_OK = 0
TQ_ERR_INVALID_ARG = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_WORKSPACE = -3
TQ_ERR_HIP = -4
TQ_ROT_DENSE, TQ_ROT_HADAMARD = 0, 1
TQ_QJL_GAUSSIAN, TQ_QJL_ORTHOGONAL = 0, 1
TQ_DTYPE_F16, TQ_DTYPE_BF16, TQ_DTYPE_F32 = 0, 1, 2
TQ_KIND_KEY, TQ_KIND_VALUE = 0, 1
TQ_STATUS_BAD_PAGE, TQ_STATUS_BAD_COUNT = 1, 2
TQ_FLAG_VALU_SCAN = 1
TQ_FLAG_VALU_APPEND = 2
TQ_FLAG_DETERMINISTIC = 4
TQ_DRAWS_ROTATION, TQ_DRAWS_QJL, TQ_DRAWS_HADAMARD = 1, 2, 3
TQ_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = [
    "tq_host_tables", "tq_codebook_init", "tq_destroy", "tq_page_bytes", "tq_encode",
    "tq_append_page", "tq_decode_workspace_bytes", "tq_decode_attn", "tq_get_status", "tq_strerror",
    "tq_profile_begin", "tq_profile_end", "tq_decode", "tq_read_probe", "tq_seed_draws",
    "tq_codebook_init_tables", "tq_decode_attn_noalloc",
]


class TQError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what} failed: {code} ({strerror(code)})")
        self.code = code


class tq_params(ctypes.Structure):
    _fields_ = [
        ("head_dim", ctypes.c_int32), ("key_bits", ctypes.c_int32), ("key_qjl", ctypes.c_int32),
        ("value_bits", ctypes.c_int32), ("rotation", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("page_tokens", ctypes.c_int32), ("window", ctypes.c_int32),
        ("flags", ctypes.c_int32), ("seed", ctypes.c_uint64), ("qjl_kind", ctypes.c_int32),
        ("qjl_shrink", ctypes.c_float), ("key_mixed", ctypes.c_int32), ("value_mixed", ctypes.c_int32),
        ("key_norm_u8", ctypes.c_int32),
    ]


class tq_tables(ctypes.Structure):
    _fields_ = [("rotation", ctypes.c_void_p), ("qjl", ctypes.c_void_p), ("key_centroids", ctypes.c_void_p),
                ("value_centroids", ctypes.c_void_p)]


def make_params(head_dim=128, key_bits=3, key_qjl=1, value_bits=4, rotation=TQ_ROT_DENSE, num_q_heads=1,
                num_kv_heads=1, page_tokens=256, window=128, seed=0, flags=0, qjl_kind=0, qjl_shrink=1.0,
                key_mixed=0, value_mixed=0, key_norm_u8=0):
    """key_mixed / value_mixed: mixed-channel rate bits + 1/2 (bits 2 or 3);
    key_norm_u8: key norms stored as u8 log-norm codes."""
    return tq_params(head_dim, key_bits, key_qjl, value_bits, rotation, num_q_heads, num_kv_heads,
                     page_tokens, window, flags, seed, qjl_kind, qjl_shrink, key_mixed, value_mixed,
                     int(key_norm_u8))


_lib = None


def lib():
    """Load libtq.so.  torch is imported first so the library binds to the HIP
    runtime torch already loaded.  Raises if the library was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: run kv_cache_vector_tq_amd.build.build() first")
    import torch  # noqa: F401  (shares its libamdhip64 with the library)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f32, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    pp = ctypes.POINTER(tq_params)
    sig = {
        "tq_host_tables": (i32, [pp, P, P, P, P, P, P, P, P]),
        "tq_codebook_init": (i32, [ctypes.POINTER(P), pp, P, P, P]),
        "tq_destroy": (i32, [P]),
        "tq_page_bytes": (i64, [pp]),
        "tq_encode": (i32, [P, i32, P, i32, i64, i64, P, P, P, P, P]),
        "tq_decode": (i32, [P, i32, P, P, P, P, i64, P, P]),
        "tq_append_page": (i32, [P, P, i64, P, i32, i32, P, P, P, i32, P, P, P, P]),
        "tq_decode_workspace_bytes": (i64, [P, i32, i32, i32]),
        "tq_decode_attn": (i32, [P, P, i32, P, i64, P, i32, i32, P, P, P, f32, P, P, sz, i32, P, i64, P]),
        "tq_get_status": (i32, [P, ctypes.POINTER(ctypes.c_int)]),
        "tq_strerror": (ctypes.c_char_p, [i32]),
        "tq_profile_begin": (i32, [P, i32]),
        "tq_profile_end": (i32, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]),
        "tq_read_probe": (i32, [P, i64, P, i32, ctypes.POINTER(ctypes.c_double), P]),
        "tq_seed_draws": (i32, [ctypes.c_uint64, i32, i64, P]),
        "tq_codebook_init_tables": (i32, [ctypes.POINTER(P), pp, ctypes.POINTER(tq_tables), P]),
        "tq_decode_attn_noalloc": (i32, [P, P, i32, P, i64, P, i32, i32, P, P, P, f32, P, i32, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def strerror(code):
    try:
        return lib().tq_strerror(code).decode()
    except Exception:  # library not loadable
        return str(code)


def _check(rc, what):
    if rc != TQ_OK:
        raise TQError(rc, what)


def _ptr(t):
    """Device (or host) address of a tensor / numpy array, or None."""
    if t is None:
        return None
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


_DT = {}


def _dtype_code(t):
    import torch
    if not _DT:
        _DT.update({torch.float16: TQ_DTYPE_F16, torch.bfloat16: TQ_DTYPE_BF16, torch.float32: TQ_DTYPE_F32})
    return _DT[t.dtype]


def tq_seed_draws(seed, stream, n):
    """n N(0,1) draws of one stream of the library's seeded generator (host)."""
    out = np.zeros(n, np.float64)
    _check(lib().tq_seed_draws(int(seed), int(stream), int(n), _ptr(out)), "tq_seed_draws")
    return out


def transform_dim(head_dim):
    """D: the next power of two >= head_dim (records and tables hold D coordinates)."""
    D = 1
    while D < head_dim:
        D *= 2
    return D


def tq_host_tables(params, rot_draws=None, qjl_draws=None, qjl=True):
    """Library-side tables computed on the host (no GPU): dict of numpy arrays.
    Draws left as None come from the library's seeded generator (the QJL
    matrix only when ``qjl``).  The tables act on D = transform_dim(head_dim)
    coordinates."""
    d = transform_dim(params.head_dim)
    rot = np.zeros(d * d if params.rotation == TQ_ROT_DENSE else d, np.float32)
    S = np.zeros(d * d, np.float32) if (qjl_draws is not None or qjl) else None
    # a mixed-channel rate appends the (b+1)-bit codebook to the b-bit one
    nk = (1 << params.key_bits) * (3 if params.key_mixed else 1)
    nv = (1 << params.value_bits) * (3 if params.value_mixed else 1)
    kc = np.zeros(nk, np.float32)
    kb = np.zeros(nk - (2 if params.key_mixed else 1), np.float32)
    vc = np.zeros(nv, np.float32)
    vb = np.zeros(nv - (2 if params.value_mixed else 1), np.float32)
    rd = None if rot_draws is None else np.ascontiguousarray(rot_draws, dtype=np.float64)
    qd = None if qjl_draws is None else np.ascontiguousarray(qjl_draws, dtype=np.float64)
    rc = lib().tq_host_tables(ctypes.byref(params), _ptr(rd), _ptr(qd), _ptr(rot), _ptr(S),
                              _ptr(kc), _ptr(kb), _ptr(vc), _ptr(vb))
    _check(rc, "tq_host_tables")
    return {"rotation": rot.reshape(d, d) if params.rotation == TQ_ROT_DENSE else rot,
            "qjl": None if S is None else S.reshape(d, d), "key_centroids": kc, "key_boundaries": kb,
            "value_centroids": vc, "value_boundaries": vb}


def tq_page_bytes(params):
    n = lib().tq_page_bytes(ctypes.byref(params))
    if n < 0:
        raise TQError(int(n), "tq_page_bytes")
    return int(n)


class Context:
    """Owns a tq_ctx (constant tables on the current device).  Built from
    draws (None: the library's seeded generator) or, with ``tables``, from
    finished tables given as data (a dict with any of "rotation", "qjl",
    "key_centroids", "value_centroids"; missing ones come from the seed)."""

    def __init__(self, params, rot_draws=None, qjl_draws=None, stream=None, tables=None):
        self.params = params
        self._h = ctypes.c_void_p()
        if tables is None:
            rd = None if rot_draws is None else np.ascontiguousarray(rot_draws, dtype=np.float64)
            qd = None if qjl_draws is None else np.ascontiguousarray(qjl_draws, dtype=np.float64)
            rc = lib().tq_codebook_init(ctypes.byref(self._h), ctypes.byref(params), _ptr(rd), _ptr(qd),
                                        _stream(stream))
            _check(rc, "tq_codebook_init")
            return
        keep = {k: np.ascontiguousarray(v, dtype=np.float32) for k, v in tables.items() if v is not None}
        t = tq_tables(*[_ptr(keep.get(k)) for k in ("rotation", "qjl", "key_centroids", "value_centroids")])
        rc = lib().tq_codebook_init_tables(ctypes.byref(self._h), ctypes.byref(params), ctypes.byref(t),
                                           _stream(stream))
        _check(rc, "tq_codebook_init_tables")

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h and self._h.value:
            lib().tq_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tq_codebook_init(params, rot_draws=None, qjl_draws=None, stream=None):
    return Context(params, rot_draws, qjl_draws, stream)


def tq_codebook_init_tables(params, tables=None, stream=None):
    return Context(params, stream=stream, tables=tables or {})


def tq_encode(ctx, kind, x, codes, norms, signs=None, rnorms=None, stream=None):
    """x: [n, >=d] cuda tensor (f16/bf16/f32, rows contiguous); outputs preallocated."""
    n = x.shape[0]
    rc = lib().tq_encode(ctx.handle, kind, _ptr(x), _dtype_code(x), n, x.stride(0), _ptr(codes), _ptr(signs),
                         _ptr(norms), _ptr(rnorms), _stream(stream))
    _check(rc, "tq_encode")


def tq_decode(ctx, kind, codes, norms, out, signs=None, rnorms=None, stream=None):
    """Dequantise n flat records (cuda tensors as written by tq_encode) into
    out: [n, d] float32."""
    n = codes.shape[0]
    rc = lib().tq_decode(ctx.handle, kind, _ptr(codes), _ptr(signs), _ptr(norms), _ptr(rnorms), n, _ptr(out),
                         _stream(stream))
    _check(rc, "tq_decode")


def tq_append_page(ctx, page_pool, block_table, seq_lens, k_new, v_new, k_win, v_win, new_counts=None,
                   num_pages=None, stream=None):
    """k_new, v_new: [B, H_kv, n_new, d] float16 cuda tensors."""
    import torch
    assert k_new.dtype == torch.float16 and v_new.dtype == torch.float16
    assert k_new.is_contiguous() and v_new.is_contiguous()
    B, _, n_new, _ = k_new.shape
    npg = num_pages if num_pages is not None else page_pool.numel() // tq_page_bytes(ctx.params)
    rc = lib().tq_append_page(ctx.handle, _ptr(page_pool), npg, _ptr(block_table), block_table.shape[1], B,
                              _ptr(seq_lens), _ptr(k_new), _ptr(v_new), n_new, _ptr(new_counts), _ptr(k_win),
                              _ptr(v_win), _stream(stream))
    _check(rc, "tq_append_page")


def tq_decode_workspace_bytes(ctx, batch, max_pages, pages_per_split=0):
    n = lib().tq_decode_workspace_bytes(ctx.handle, batch, max_pages, pages_per_split)
    if n < 0:
        raise TQError(int(n), "tq_decode_workspace_bytes")
    return int(n)


def tq_decode_attn(ctx, q, page_pool, block_table, seq_lens, k_win, v_win, out, workspace, sm_scale,
                   pages_per_split=0, dbg_logits=None, num_pages=None, stream=None):
    B = q.shape[0]
    npg = num_pages if num_pages is not None else page_pool.numel() // tq_page_bytes(ctx.params)
    stride = 0 if dbg_logits is None else dbg_logits.shape[-1]
    rc = lib().tq_decode_attn(ctx.handle, _ptr(q), _dtype_code(q), _ptr(page_pool), npg, _ptr(block_table),
                              block_table.shape[1], B, _ptr(seq_lens), _ptr(k_win), _ptr(v_win), float(sm_scale),
                              _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              pages_per_split, _ptr(dbg_logits), stride, _stream(stream))
    _check(rc, "tq_decode_attn")


def tq_decode_attn_noalloc(ctx, q, page_pool, block_table, seq_lens, k_win, v_win, out, sm_scale,
                           pages_per_split=0, num_pages=None, stream=None):
    """tq_decode_attn with the library's static device scratch as workspace
    (no allocation)."""
    B = q.shape[0]
    npg = num_pages if num_pages is not None else page_pool.numel() // tq_page_bytes(ctx.params)
    rc = lib().tq_decode_attn_noalloc(ctx.handle, _ptr(q), _dtype_code(q), _ptr(page_pool), npg, _ptr(block_table),
                                      block_table.shape[1], B, _ptr(seq_lens), _ptr(k_win), _ptr(v_win),
                                      float(sm_scale), _ptr(out), pages_per_split, _stream(stream))
    _check(rc, "tq_decode_attn_noalloc")


def tq_get_status(ctx):
    code = ctypes.c_int(0)
    _check(lib().tq_get_status(ctx.handle, ctypes.byref(code)), "tq_get_status")
    return code.value


def tq_profile_begin(ctx, max_calls):
    _check(lib().tq_profile_begin(ctx.handle, max_calls), "tq_profile_begin")


def tq_profile_end(ctx):
    """Returns (summed scan-kernel milliseconds, number of recorded decode calls)."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int(0)
    _check(lib().tq_profile_end(ctx.handle, ctypes.byref(ms), ctypes.byref(n)), "tq_profile_end")
    return ms.value, n.value


def tq_read_probe(buf, sink, reps=5, stream=None):
    """Fastest of `reps` streaming reads of the device tensor `buf` (bytes a
    multiple of 16), in milliseconds; `sink` is a 4-byte device tensor."""
    ms = ctypes.c_double(0.0)
    nbytes = buf.numel() * buf.element_size()
    _check(lib().tq_read_probe(_ptr(buf), nbytes, _ptr(sink), reps, ctypes.byref(ms), _stream(stream)),
           "tq_read_probe")
    return ms.value
