"""Rotations and the QJL projection (test oracle only).

* Dense rotation: a fixed, data-oblivious random orthogonal d x d matrix
  ("aither-kvcache" README, section "Algorithm", step 2).  Built from a d x d
  matrix of i.i.d. N(0,1) draws by QR with the signs of diag(R) folded into Q,
  which gives the Haar distribution; stored as float32.
* Randomized Hadamard: one seeded Rademacher sign stage followed by a fast
  Walsh-Hadamard transform, scaled by 1/sqrt(d) so it is orthogonal
  ("TurboQuant Family Design Study", section "Dense and structured transform
  comparison").  Sylvester (natural) ordering.
* QJL projection S: d x d i.i.d. N(0,1) entries, as in the paper's QJL
  definition quoted in "TurboQuant on a 16GB MacBook", section "The QJL
  detective story"; stored as float32.  The variance-reduced variant from
  the same section replaces it by an orthogonal matrix obtained by QR, here
  the Haar construction of the dense rotation applied to the S draws.

Head sizes that are not a power of two ("TurboQuant Family Design Study",
same section: zero-pad temporarily during append and the query transform):
the transform acts on D = the next power of two >= d coordinates; a vector is
padded with zeros to D, transformed, and all D transform coordinates are
quantised and stored.  (The page asks not to store padded payload unless a
kernel proves it worthwhile; keeping only d of the D coordinates would make
the transform non-invertible and break q.k = (Tq).(Tk), so this reading
stores them: the padding is what stays temporary, the FP16 vectors and the
outputs keep d coordinates.)  The dense rotation is padded the same way, a
Haar D x D matrix applied to the padded vector, i.e. its first d columns, an
isometry of R^d into R^D.  The inverse transform returns the first d
coordinates.

The random draws are inputs (they come from ``tq_inputs``); this module only
does the arithmetic that turns them into the stored matrices.
"""

import numpy as np


def dense_rotation(gauss_draws: np.ndarray) -> np.ndarray:
    """Pi = Q diag(sign(diag R)) for QR of the draws, rounded to float32.

    Returned as float64 holding float32 values.  y = Pi @ x rotates x.
    """
    g = np.asarray(gauss_draws, dtype=np.float64)
    if g.ndim != 2 or g.shape[0] != g.shape[1]:
        raise ValueError("draws must be square")
    q, r = np.linalg.qr(g)
    s = np.sign(np.diag(r))
    s[s == 0] = 1.0
    return (q * s[None, :]).astype(np.float32).astype(np.float64)


def sylvester_hadamard(d: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix H_d (entries +-1), d a power of two."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rademacher_signs(draws: np.ndarray) -> np.ndarray:
    """+-1 from draws: the sign of each draw, 0 and positive map to +1."""
    return np.where(np.asarray(draws, dtype=np.float64) < 0, -1.0, 1.0)


def fwht(x: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform along the last axis
    (butterflies a+b, a-b at strides 1, 2, 4, ...); equals x @ H_d."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def transform_dim(head_dim: int) -> int:
    """D: the next power of two >= head_dim (the transform's size)."""
    D = 1
    while D < head_dim:
        D *= 2
    return D


class Rotation:
    """The orthogonal transform Pi used for keys, values and queries, on
    D = transform_dim(d) coordinates (inputs zero-padded from d to D).

    kind "dense": explicit D x D matrix (draws D x D).  kind "hadamard":
    y = H_D (eps * x) / sqrt(D) (draws: D values), inverse
    x = eps * (H_D y) / sqrt(D).
    """

    def __init__(self, kind: str, draws: np.ndarray, head_dim: int):
        self.kind = kind
        self.d = head_dim
        self.D = D = transform_dim(head_dim)
        if kind == "dense":
            self.matrix = dense_rotation(np.asarray(draws).reshape(D, D))
        elif kind == "hadamard":
            self.eps = rademacher_signs(np.asarray(draws).reshape(D))
            self.matrix = sylvester_hadamard(D) * self.eps[None, :] / np.sqrt(D)
        else:
            raise ValueError(kind)

    def pad(self, x: np.ndarray) -> np.ndarray:
        """Row vectors of d coordinates, zero-padded to D."""
        x = np.asarray(x, dtype=np.float64)
        if x.shape[-1] == self.D:
            return x
        out = np.zeros(x.shape[:-1] + (self.D,))
        out[..., :x.shape[-1]] = x
        return out

    def forward(self, x: np.ndarray) -> np.ndarray:
        """Rotate row vectors of d coordinates: returns the D coordinates of
        Pi [x; 0] for each row."""
        x = self.pad(x)
        if self.kind == "dense":
            return x @ self.matrix.T
        return fwht(x * self.eps) / np.sqrt(self.D)

    def inverse(self, y: np.ndarray) -> np.ndarray:
        """Undo ``forward`` on row vectors of D coordinates: the first d
        coordinates of Pi^T y."""
        y = np.asarray(y, dtype=np.float64)
        if self.kind == "dense":
            full = y @ self.matrix
        else:
            full = fwht(y) * self.eps / np.sqrt(self.D)
        return full[..., :self.d]


def qjl_matrix(gauss_draws: np.ndarray, head_dim: int, kind: str = "gaussian") -> np.ndarray:
    """S, shape (d, d) (one row per sign bit), float32 values: the draws
    themselves ("gaussian") or the Haar orthogonal matrix built from them
    ("orthogonal")."""
    g = np.asarray(gauss_draws, dtype=np.float64).reshape(head_dim, head_dim)
    if kind == "gaussian":
        return g.astype(np.float32).astype(np.float64)
    if kind == "orthogonal":
        return dense_rotation(g)
    raise ValueError(kind)
