"""Mixed-channel fractional rates (test oracle only).

"TurboQuant Family Design Study", section "Packed format and complete bit
accounting": fractional nominal rates come from splitting the channels, not
from entropy coding; for d = 128, 2.5 bits per channel is 64 channels at 2
bits and 64 at 3 bits, 3.5 bits is 64 at 3 and 64 at 4, with fixed offsets
and no decoder state.  The same page's recommended first mode stores keys at
3.5 bits per channel.

Readings taken here (the page fixes the counts, not which channels):
* the split applies to the rotated coordinates, half at ``bits`` and half at
  ``bits + 1``, each half with its own Lloyd-Max codebook for the same
  N(0, 1/d) density; after the rotation every coordinate has the same
  distribution, so which half takes the extra bit does not change the
  expected error;
* the high-rate half is fixed per kind: keys {j : j mod 32 >= 16}, values
  {j : j mod 8 >= 4}; these are the sets the matrix-core decode reads as
  whole operand slices;
* a record stores the codes of the low-rate coordinates first, then those of
  the high-rate ones, each in ascending coordinate order and packed LSB-first
  like the integer-rate codes: (d/2) b + (d/2)(b + 1) bits.
"""

import numpy as np

from . import codebook as cbm


def hi_mask(head_dim: int, kind: str) -> np.ndarray:
    """Boolean [d]: coordinates coded with bits + 1."""
    j = np.arange(head_dim)
    if kind == "key":
        return (j % 32) >= 16
    if kind == "value":
        return (j % 8) >= 4
    raise ValueError(kind)


class MixedCodebook:
    """Codebook of a mixed-channel rate bits + 1/2 (bits in {2, 3})."""

    mixed = True

    def __init__(self, bits: int, head_dim: int, kind: str):
        if bits not in (2, 3):
            raise ValueError("mixed-channel rates are 2.5 and 3.5 bits")
        if head_dim % 32:
            raise ValueError("head_dim must be a multiple of 32")
        self.bits, self.head_dim, self.kind = bits, head_dim, kind
        self.lo = cbm.Codebook(bits, head_dim)
        self.hi = cbm.Codebook(bits + 1, head_dim)
        self.hi_mask = hi_mask(head_dim, kind)
        self.lo_idx = np.nonzero(~self.hi_mask)[0]
        self.hi_idx = np.nonzero(self.hi_mask)[0]

    def quantize(self, y32: np.ndarray) -> np.ndarray:
        """Per coordinate, the code of its half's codebook (ties to the lower index)."""
        y32 = np.asarray(y32, dtype=np.float64)
        return np.where(self.hi_mask, self.hi.quantize(y32), self.lo.quantize(y32)).astype(np.int64)

    def nearest(self, y: np.ndarray) -> np.ndarray:
        """Exhaustive nearest level per coordinate in its half's codebook."""
        y = np.asarray(y, dtype=np.float64)
        return np.where(self.hi_mask, self.hi.nearest(y), self.lo.nearest(y)).astype(np.int64)

    def values(self, idx: np.ndarray) -> np.ndarray:
        """Level values c[idx] per coordinate."""
        idx = np.asarray(idx, dtype=np.int64)
        lo = self.lo.centroids[np.minimum(idx, len(self.lo.centroids) - 1)]
        return np.where(self.hi_mask, self.hi.centroids[idx], lo)

    def record_bytes(self, d: int) -> int:
        return (d // 2) * (2 * self.bits + 1) // 8

    def pack(self, idx: np.ndarray) -> np.ndarray:
        from . import codec
        idx = np.asarray(idx, dtype=np.int64)
        return np.concatenate([codec.pack_bits(idx[..., self.lo_idx], self.bits),
                               codec.pack_bits(idx[..., self.hi_idx], self.bits + 1)], axis=-1)

    def unpack(self, packed: np.ndarray, d: int) -> np.ndarray:
        from . import codec
        packed = np.asarray(packed, dtype=np.uint8)
        nlo = (d // 2) * self.bits // 8
        out = np.zeros(packed.shape[:-1] + (d,), dtype=np.int64)
        out[..., self.lo_idx] = codec.unpack_bits(packed[..., :nlo], self.bits, d // 2)
        out[..., self.hi_idx] = codec.unpack_bits(packed[..., nlo:], self.bits + 1, d // 2)
        return out

    def width(self) -> np.ndarray:
        """Bits per coordinate, [d]."""
        return np.where(self.hi_mask, self.bits + 1, self.bits)


def make_codebook(bits: int, head_dim: int, kind: str, mixed: bool):
    """Integer-rate codebook, or the mixed-channel one for bits + 1/2."""
    return MixedCodebook(bits, head_dim, kind) if mixed else cbm.Codebook(bits, head_dim)
