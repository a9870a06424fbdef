"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module holds none of the cache's arithmetic: it only draws random
numbers and shapes them into the workloads (post-RoPE keys with heavy-tailed
channel scales, Gaussian values and queries, ragged lengths) and the random
draws the method consumes (the Gaussian matrix that the rotation is built
from, the Rademacher signs of the Hadamard variant, the QJL Gaussian matrix).
Every stream comes from ``numpy.random.SeedSequence([seed, tag, ...])`` so a
slice (one sequence, one head) can be regenerated on its own.

Key recipe: z ~ N(0,1) per channel, times per-channel scales exp(N(0, 0.5^2))
with 4 of the d channels (drawn without replacement) multiplied by 20, then
RoPE with interleaved pairs (2i, 2i+1), theta_i = base^(-2i/d), base 10000,
at the token's absolute position.  Values and queries are N(0,1).
"""

import numpy as np

TAG_ROT = 1
TAG_QJL = 2
TAG_HAD = 3
TAG_SCALE = 10
TAG_KEY = 11
TAG_VAL = 12
TAG_QUERY = 13
TAG_LENS = 14
TAG_MISC = 15


def rng(seed, *path):
    return np.random.default_rng(np.random.SeedSequence([int(seed)] + [int(p) for p in path]))


def rotation_draws(seed, d):
    """d x d i.i.d. N(0,1) draws (float64) for the dense rotation."""
    return rng(seed, TAG_ROT).standard_normal((d, d))


def hadamard_draws(seed, d):
    """d Rademacher values (+-1.0) for the randomized Hadamard transform."""
    return rng(seed, TAG_HAD).integers(0, 2, d).astype(np.float64) * 2.0 - 1.0


def qjl_draws(seed, d):
    """d x d i.i.d. N(0,1) draws (float64) for the QJL projection."""
    return rng(seed, TAG_QJL).standard_normal((d, d))


def channel_scales(seed, d, layer=0, head=0, n_outliers=4, outlier_gain=20.0, sigma=0.5):
    r = rng(seed, TAG_SCALE, layer, head)
    s = np.exp(r.normal(0.0, sigma, d))
    out = r.choice(d, size=n_outliers, replace=False)
    s[out] *= outlier_gain
    return s


def rope_interleaved(x, positions, base=10000.0):
    """Rotate pairs (2i, 2i+1) of each row by positions * base^(-2i/d)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def keys(seed, d, positions, layer=0, head=0, seq=0):
    """Post-RoPE keys [len(positions), d] (float64, not yet rounded)."""
    positions = np.asarray(positions)
    z = rng(seed, TAG_KEY, layer, head, seq, int(positions[0]) if len(positions) else 0).standard_normal(
        (len(positions), d))
    return rope_interleaved(z * channel_scales(seed, d, layer, head)[None, :], positions)


def values(seed, d, n, layer=0, head=0, seq=0, start=0):
    return rng(seed, TAG_VAL, layer, head, seq, start).standard_normal((n, d))


def queries(seed, shape, layer=0, step=0):
    return rng(seed, TAG_QUERY, layer, step).standard_normal(shape)


def ragged_lengths(seed, n, lo, hi):
    """n integer lengths uniform in [lo, hi]."""
    return rng(seed, TAG_LENS).integers(lo, hi + 1, n)


def fp16(x):
    """Round to IEEE half (the cache's input precision)."""
    return np.asarray(x).astype(np.float16)


def bf16_round(x):
    """Round float64/float32 values to bfloat16 (nearest-even), returned as float32."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32)


def kv_block(seed, d, T, layer=0, head=0, seq=0, start=0):
    """FP16 keys and values for positions start..start+T-1 of one (seq, head)."""
    pos = np.arange(start, start + T)
    k = fp16(keys(seed, d, pos, layer, head, seq))
    v = fp16(values(seed, d, T, layer, head, seq, start))
    return k, v


def torch_kv(seed, B, H, T, d, device, layer=0, start=0, out_dtype=None):
    """The same key/value recipe drawn with torch's generator on a device (for
    benchmark-sized workloads; a different random stream from ``keys`` /
    ``values``).  Returns fp16 tensors [B, H, T, d]."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([int(seed), TAG_KEY, layer]).generate_state(1)[0]))
    scales = torch.tensor(np.stack([channel_scales(seed, d, layer, h) for h in range(H)]), dtype=torch.float32,
                          device=device)
    pos = torch.arange(start, start + T, device=device, dtype=torch.float64)
    inv = torch.tensor(10000.0 ** (-np.arange(0, d, 2, dtype=np.float64) / d), device=device)
    ang = (pos[:, None] * inv[None, :])
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    k = torch.empty((B, H, T, d), dtype=torch.float16, device=device)
    v = torch.empty((B, H, T, d), dtype=torch.float16, device=device)
    for b in range(B):
        z = torch.randn((H, T, d), generator=g, device=device, dtype=torch.float32) * scales[:, None, :]
        a, c = z[..., 0::2], z[..., 1::2]
        r = torch.empty_like(z)
        r[..., 0::2] = a * cos - c * sin
        r[..., 1::2] = a * sin + c * cos
        k[b] = r.half()
        v[b] = torch.randn((H, T, d), generator=g, device=device, dtype=torch.float32).half()
    return k, v


def torch_queries(seed, shape, device, dtype, step=0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([int(seed), TAG_QUERY, step]).generate_state(1)[0]))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)
