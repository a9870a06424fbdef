"""u8 log-norm storage of key norms (test oracle only).

"TurboQuant Family Design Study", section "Packed format and complete bit
accounting": in the low-overhead modes a key norm takes one byte per
token-head, which adds 0.0625 bits per channel at d = 128; the page's
recommended first mode stores keys with a u8 log-norm.

Readings taken here (the page fixes the width and the logarithmic domain, not
the grid, the rounding or the range):
* code 0 stands for a zero norm; codes 1..255 are levels uniform in log2
  with 16 levels per octave, code 128 at 2^4:
      level(q) = 2^(q/16 - 4),  q = 1..255  (2^-3.9375 .. 2^11.9375);
* a norm is rounded to the nearest level in the log domain: the boundary
  between levels k and k+1 is their geometric midpoint 2^((k + 1/2)/16 - 4),
  taken as a float32 value, and the float32 norm is compared with it (the
  precision the GPU decides in; a norm equal to a boundary takes the lower
  level).  Norms below the first boundary take code 1, above the last one
  code 255;
* the stored reconstruction of a key is level(q) * c[idx], and its QJL
  residual is taken against that: r = Pi x - level(q) c[idx], so the sketch
  also carries the norm's rounding and the estimator stays unbiased;
* value norms stay float32 (the page gives their size only as "norms or
  gains, if the value mode requires them").
"""

import numpy as np

STEPS_PER_OCTAVE = 16
CENTER_LOG2 = 4.0
CENTER_CODE = 128


def levels() -> np.ndarray:
    """float64 [256]: level(q) for q = 0..255 (level(0) = 0)."""
    q = np.arange(256, dtype=np.float64)
    out = 2.0 ** ((q - CENTER_CODE) / STEPS_PER_OCTAVE + CENTER_LOG2)
    out[0] = 0.0
    return out


def boundaries() -> np.ndarray:
    """float32 [254]: B_k, k = 1..254, the geometric midpoint of levels k and k+1."""
    k = np.arange(1, 255, dtype=np.float64)
    return (2.0 ** ((k + 0.5 - CENTER_CODE) / STEPS_PER_OCTAVE + CENTER_LOG2)).astype(np.float32)


def encode(norm32) -> np.ndarray:
    """u8 codes of float32 norms: 0 for a zero norm, else 1 + #{k : n > B_k}."""
    n = np.asarray(norm32, dtype=np.float32)
    q = 1 + np.sum(n[..., None] > boundaries(), axis=-1)
    return np.where(n > 0, q, 0).astype(np.uint8)


def decode(codes) -> np.ndarray:
    """float64 levels of u8 codes."""
    return levels()[np.asarray(codes, dtype=np.int64)]


def bits_per_channel(head_dim: int) -> float:
    return 8.0 / head_dim
