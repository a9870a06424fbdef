"""Per-vector TurboQuant encode and dequantise (test oracle only).

Encode of one post-RoPE vector x (float values, taken exactly as float64):
1. n = ||x||_2, stored as float32 (or, for keys in the low-overhead mode,
   as a u8 log-norm code, ``oracle.lognorm``); u = x / n ("aither-kvcache"
   README, "Algorithm" step 1).  A zero vector stores n = 0 and all-zero codes, signs
   and residual norm, so it decodes to exact zeros ("TurboQuant on a 16GB
   MacBook", "Round 2: the llama.cpp bug hunt", the zero-block fix).
2. y = Pi u (step 2).
3. Each coordinate of y, rounded to float32 (the precision the GPU decides
   in), is mapped to its Lloyd-Max code by boundary comparison (step 3).
4. Codes are bit-packed LSB-first: code j occupies bits [j*b, (j+1)*b) of the
   vector's bitstream, bit i of the stream is bit (i mod 8) of byte i//8
   (step 4; d*b/8 bytes, e.g. 64 bytes at d=128, b=4, from the README's
   "Where This Fits" example).  A mixed-channel rate b + 1/2 quantises and
   packs each half of the coordinates with its own width (``oracle.mixed``).
5. Keys only: the residual of the MSE reconstruction in the rotated basis,
   r = Pi x - n32 * c[idx]; its norm ||r|| (float32); and the 1-bit QJL sketch
   sigma_j = [ (S r)_j >= 0 ], packed LSB-first like the codes ("TurboQuant on
   a 16GB MacBook", "Why this caught my eye": 1-bit QJL transform on the
   quantisation residual; "The QJL detective story": Gaussian S).

Dequantise (reverses the steps, README "Algorithm" last line):
  k_hat = Pi^T ( n c_K[idx] + a * ||r|| * S^T (2 sigma - 1) )
  v_hat = Pi^T ( n_V c_V[idx_V] )
with the QJL coefficient a = sqrt(pi/2)/d for Gaussian S (the paper's pair)
or a = alpha * sqrt(pi/2)/sqrt(d) for an orthogonal S with shrinkage alpha
(the variance-reduced variant; "The QJL detective story": orthogonal matrix
and the matched 1/sqrt(d) scale are one coupled substitution, damping 0.7 is
close to the MMSE shrinkage 2/pi).
"""

import math

import numpy as np

QJL_SCALE_NUM = math.sqrt(math.pi / 2.0)


def qjl_scale(head_dim: int, kind: str = "gaussian", shrink: float = 1.0) -> float:
    """QJL dequantisation coefficient.  Gaussian S with d rows: sqrt(pi/2)/d
    (unbiased).  Orthogonal S: sqrt(pi/2)/sqrt(d) (the matched scale; rows of
    unit norm), times the shrinkage factor."""
    if kind == "gaussian":
        return shrink * QJL_SCALE_NUM / head_dim
    if kind == "orthogonal":
        return shrink * QJL_SCALE_NUM / math.sqrt(head_dim)
    raise ValueError(kind)


def pack_bits(codes: np.ndarray, bits: int) -> np.ndarray:
    """Pack integer codes [..., d] into uint8 [..., d*bits/8], LSB-first."""
    codes = np.asarray(codes, dtype=np.int64)
    d = codes.shape[-1]
    if (d * bits) % 8:
        raise ValueError("d*bits must be a multiple of 8")
    bitpos = np.arange(bits)
    stream = ((codes[..., :, None] >> bitpos) & 1).reshape(codes.shape[:-1] + (d * bits,))
    stream = stream.reshape(codes.shape[:-1] + (d * bits // 8, 8))
    weights = 1 << np.arange(8)
    return (stream * weights).sum(axis=-1).astype(np.uint8)


def unpack_bits(packed: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of ``pack_bits``: uint8 [..., d*bits/8] -> int64 codes [..., d]."""
    packed = np.asarray(packed, dtype=np.uint8)
    stream = ((packed[..., :, None].astype(np.int64) >> np.arange(8)) & 1)
    stream = stream.reshape(packed.shape[:-1] + (d, bits))
    return (stream << np.arange(bits)).sum(axis=-1).astype(np.int64)


class Encoded:
    """Flat records for n vectors: codes uint8 [n, d*b/8], norms f32 [n],
    and for keys with QJL signs uint8 [n, d/8] and rnorms f32 [n]."""

    def __init__(self, codes, norms, signs=None, rnorms=None, idx=None, norm_codes=None):
        self.codes = codes
        self.norms = norms
        self.signs = signs
        self.rnorms = rnorms
        self.idx = idx  # unpacked code indices, kept for tests
        self.norm_codes = norm_codes  # u8 log-norm codes, when the norms are stored that way


def encode(x: np.ndarray, rotation, codebook, qjl_S=None, norm_u8=False) -> Encoded:
    """Encode row vectors x [n, d]; keys pass the QJL matrix, values pass None.
    The records hold the D = rotation.D transform coordinates (d zero-padded
    to D when d is not a power of two); codebook and S are built for D.
    ``norm_u8``: the norm is stored as a u8 log-norm code (``oracle.lognorm``);
    the record's float32 norm is then that code's level and the QJL residual
    is taken against it."""
    x = np.asarray(x, dtype=np.float64)
    n_vec, d = x.shape
    norm = np.sqrt(np.sum(x * x, axis=1))
    norm32 = norm.astype(np.float32).astype(np.float64)
    nonzero = norm > 0.0
    safe = np.where(nonzero, norm, 1.0)
    y = rotation.forward(x / safe[:, None])
    y32 = y.astype(np.float32).astype(np.float64)
    idx = codebook.quantize(y32)
    idx[~nonzero] = 0
    ncode = None
    if norm_u8:
        from . import lognorm
        ncode = lognorm.encode(norm32.astype(np.float32))
        norm32 = lognorm.decode(ncode).astype(np.float32).astype(np.float64)
    rec = Encoded(codebook.pack(idx), norm32.astype(np.float32), idx=idx)
    rec.norm_codes = ncode
    if qjl_S is not None:
        r = rotation.forward(x) - norm32[:, None] * codebook.values(idx)
        r[~nonzero] = 0.0
        rnorm = np.sqrt(np.sum(r * r, axis=1))
        z = r @ qjl_S.T
        sigma = (z >= 0.0).astype(np.int64)
        sigma[~nonzero] = 0
        rec.signs = pack_bits(sigma, 1)
        rec.rnorms = rnorm.astype(np.float32)
    return rec


def residual_from_codes(x: np.ndarray, rotation, codebook, norms32, idx) -> np.ndarray:
    """r = Pi x - n32 * c[idx] for given codes (used to check sign bits against
    codes produced elsewhere)."""
    x = np.asarray(x, dtype=np.float64)
    r = rotation.forward(x) - np.asarray(norms32, dtype=np.float64)[:, None] * codebook.values(idx)
    r[np.asarray(norms32) == 0] = 0.0
    return r


def dequantize_rotated(codes, norms, codebook, d, signs=None, rnorms=None, qjl_S=None, qjl_coef=None):
    """Reconstruction in the rotated basis: n c[idx] (+ QJL term for keys,
    coefficient ``qjl_coef``, default the Gaussian sqrt(pi/2)/d)."""
    idx = codebook.unpack(codes, d)
    out = np.asarray(norms, dtype=np.float64)[:, None] * codebook.values(idx)
    if signs is not None:
        coef = qjl_scale(d) if qjl_coef is None else qjl_coef
        pm = 2.0 * unpack_bits(signs, 1, d) - 1.0
        out = out + coef * np.asarray(rnorms, dtype=np.float64)[:, None] * (pm @ qjl_S)
    return out


def dequantize(codes, norms, rotation, codebook, signs=None, rnorms=None, qjl_S=None, qjl_coef=None):
    """k_hat / v_hat in the original basis (d coordinates; the records hold
    the D = rotation.D transform coordinates)."""
    D = rotation.D
    return rotation.inverse(dequantize_rotated(codes, norms, codebook, D, signs, rnorms, qjl_S, qjl_coef))


def qjl_reconstruct(r: np.ndarray, S: np.ndarray, coef: float) -> np.ndarray:
    """The residual as the sketch gives it back: coef * ||r|| * S^T sign(S r)
    (sign(0) = +1), for rows r."""
    r = np.asarray(r, dtype=np.float64)
    pm = np.where(r @ S.T >= 0.0, 1.0, -1.0)
    return coef * np.linalg.norm(r, axis=-1, keepdims=True) * (pm @ S)


def qjl_inner_product(q: np.ndarray, r_norm: float, signs_pm: np.ndarray, S: np.ndarray, coef=None) -> float:
    """QJL estimate of <q, r> from the sketch: a * ||r|| * <S q, sigma>, with
    a = sqrt(pi/2)/m for Gaussian S with m rows (m = d in the cache) unless
    another coefficient is given."""
    a = qjl_scale(S.shape[0]) if coef is None else coef
    return a * r_norm * float(np.dot(S @ q, signs_pm))
