"""Lloyd-Max scalar codebooks for the rotated coordinates (test oracle only).

After a random rotation every coordinate of a unit vector is close to
N(0, 1/d), so each coordinate is quantised independently with a fixed,
precomputed MSE-optimal scalar quantiser and no per-block scale
("TurboQuant on a 16GB MacBook", section "Why this caught my eye", the
PolarQuant/MSE stage; "aither-kvcache" README, section "Algorithm", steps 2-3).

Reading taken here (the pages do not spell out the construction):
* target density: standard normal, levels then scaled by 1/sqrt(d);
* Lloyd iteration (centroid = conditional mean of the cell, boundary =
  midpoint of neighbouring centroids), started from evenly spaced levels,
  stopped when no level moves by 1e-14; the quantiser is kept exactly
  symmetric by iterating the positive half and mirroring it;
* the stored codebook is the scaled levels rounded (once, from double) to
  IEEE half precision; the pages do not fix the storage precision, and the
  package README's decode returns float16 vectors ("aither-kvcache",
  "Where This Fits"), so reconstructions are half-precision values either
  way.  Decision boundaries are the midpoints of the stored levels (exact in
  float32); a value equal to a boundary takes the lower index.
"""

import math

import numpy as np

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def normal_pdf(x: float) -> float:
    """Standard normal density, 0 at +-inf."""
    if math.isinf(x):
        return 0.0
    return math.exp(-0.5 * x * x) * _INV_SQRT_2PI


def normal_upper_tail(x: float) -> float:
    """P(X > x) for X ~ N(0,1), via erfc so that tails keep full precision."""
    if x == math.inf:
        return 0.0
    if x == -math.inf:
        return 1.0
    return 0.5 * math.erfc(x / _SQRT2)


def cell_mass(a: float, b: float) -> float:
    """P(a < X <= b) for X ~ N(0,1), computed from the tail nearer the cell."""
    if a >= 0.0:
        return normal_upper_tail(a) - normal_upper_tail(b)
    if b <= 0.0:
        return normal_upper_tail(-b) - normal_upper_tail(-a)
    return 1.0 - normal_upper_tail(b) - normal_upper_tail(-a)


def lloyd_max_normal(bits: int, tol: float = 1e-14, max_iter: int = 1_000_000):
    """MSE-optimal 2**bits-level quantiser of N(0,1) by Lloyd iteration.

    Returns the levels in increasing order (float64 list).  A cell [a, b]
    gets the conditional mean (pdf(a) - pdf(b)) / P(a < X <= b).
    """
    if bits < 1:
        raise ValueError("bits must be >= 1")
    levels = 1 << bits
    half = levels // 2
    pos = [(k + 0.5) * 2.0 / half for k in range(half)]
    for _ in range(max_iter):
        full = [-x for x in reversed(pos)] + pos
        mids = [(full[k] + full[k + 1]) * 0.5 for k in range(levels - 1)]
        edges = [0.0] + mids[half:] + [math.inf]
        new = [
            (normal_pdf(edges[k]) - normal_pdf(edges[k + 1])) / cell_mass(edges[k], edges[k + 1])
            for k in range(half)
        ]
        delta = max(abs(x - y) for x, y in zip(new, pos))
        pos = new
        if delta < tol:
            break
    return [-x for x in reversed(pos)] + pos


def gaussian_distortion(levels) -> float:
    """E[(X - Q(X))^2] for X ~ N(0,1) and nearest-level quantiser Q (closed form).

    Per cell [a, b] with level c: M2 - 2 c M1 + c^2 M0 where M0 = P(cell),
    M1 = pdf(a) - pdf(b), M2 = M0 - (b pdf(b) - a pdf(a)).
    """
    lv = [float(x) for x in levels]
    n = len(lv)
    edges = [-math.inf] + [(lv[k] + lv[k + 1]) * 0.5 for k in range(n - 1)] + [math.inf]
    total = 0.0
    for k in range(n):
        a, b = edges[k], edges[k + 1]
        m0 = cell_mass(a, b)
        m1 = normal_pdf(a) - normal_pdf(b)
        bpb = 0.0 if math.isinf(b) else b * normal_pdf(b)
        apa = 0.0 if math.isinf(a) else a * normal_pdf(a)
        m2 = m0 - (bpb - apa)
        c = lv[k]
        total += m2 - 2.0 * c * m1 + c * c * m0
    return total


class Codebook:
    """Stored codebook for one bit width and head dimension.

    ``centroids`` are half-precision values and ``boundaries`` float32 values,
    held as float64 so that every later step uses them as exact numbers.
    """

    def __init__(self, bits: int, head_dim: int, storage: str = "half"):
        """``storage``: precision the scaled levels are rounded to, "half"
        (the reading used throughout) or "single" (float32; kept only so a
        test can show the choice does not move results at the parity bar)."""
        self.bits = bits
        self.head_dim = head_dim
        unit = lloyd_max_normal(bits)
        scale = 1.0 / math.sqrt(head_dim)
        rnd = {"half": np.float16, "single": np.float32}[storage]
        self.centroids = np.array([rnd(c * scale) for c in unit], dtype=np.float64)
        c = self.centroids
        self.boundaries = np.array(
            [np.float32((c[k] + c[k + 1]) * 0.5) for k in range(len(c) - 1)], dtype=np.float64
        )

    def quantize(self, y32: np.ndarray) -> np.ndarray:
        """Code index of each (float32-valued) coordinate: number of boundaries
        strictly below it, so a tie goes to the lower index."""
        return np.searchsorted(self.boundaries, np.asarray(y32, dtype=np.float64), side="left").astype(np.int64)

    def nearest(self, y: np.ndarray) -> np.ndarray:
        """Exhaustive nearest-centroid index (first minimum), the plain definition."""
        y = np.asarray(y, dtype=np.float64)
        return np.argmin(np.abs(y[..., None] - self.centroids), axis=-1).astype(np.int64)

    # the record interface shared with the mixed-channel codebook (oracle.mixed)
    mixed = False

    def values(self, idx: np.ndarray) -> np.ndarray:
        """Level values c[idx]."""
        return self.centroids[np.asarray(idx, dtype=np.int64)]

    def record_bytes(self, d: int) -> int:
        return d * self.bits // 8

    def pack(self, idx: np.ndarray) -> np.ndarray:
        from . import codec
        return codec.pack_bits(idx, self.bits)

    def unpack(self, packed: np.ndarray, d: int) -> np.ndarray:
        from . import codec
        return codec.unpack_bits(packed, self.bits, d)

    def width(self) -> np.ndarray:
        """Bits per coordinate, [d]."""
        return np.full(self.head_dim, self.bits, dtype=np.int64)
