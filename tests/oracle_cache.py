"""Builds oracle caches from the seeded synthetic inputs (tests only)."""

import numpy as np

from oracle import codebook as cbm
from oracle import mixed
from oracle import codec
from oracle import pages
from oracle import rotation as rot
import tq_inputs


class Setup:
    def __init__(self, d=128, key_bits=3, key_qjl=1, value_bits=4, rotation="dense", seed=0,
                 Hq=1, Hkv=1, P=256, W=128, qjl_kind="gaussian", qjl_shrink=1.0, key_mixed=False,
                 value_mixed=False, key_norm_u8=False):
        self.d, self.bK, self.qjl, self.bV = d, key_bits, key_qjl, value_bits
        self.kmix, self.vmix = key_mixed, value_mixed
        self.kn8 = key_norm_u8
        self.qjl_kind, self.qjl_shrink = qjl_kind, qjl_shrink
        self.rotation, self.seed, self.Hq, self.Hkv, self.P, self.W = rotation, seed, Hq, Hkv, P, W
        # the transform, codebooks and S act on D = next power of two >= d
        # coordinates (inputs zero-padded); D = d for the power-of-two sizes
        self.D = D = rot.transform_dim(d)
        if rotation == "dense":
            self.rot_draws = tq_inputs.rotation_draws(seed, D)
        else:
            self.rot_draws = tq_inputs.hadamard_draws(seed, D)
        self.qjl_draws = tq_inputs.qjl_draws(seed, D)
        self.R = rot.Rotation(rotation, self.rot_draws, d)
        self.kcb = mixed.make_codebook(key_bits, D, "key", key_mixed)
        self.vcb = mixed.make_codebook(value_bits, D, "value", value_mixed)
        self.S = rot.qjl_matrix(self.qjl_draws, D, qjl_kind) if key_qjl else None
        self.qjl_coef = codec.qjl_scale(D, qjl_kind, qjl_shrink)
        # page-header QJL byte: 0 none, 1 Gaussian S, 2 orthogonal S
        self.lay = pages.Layout(d, key_bits, (1 + (qjl_kind == "orthogonal")) if key_qjl else 0, value_bits, Hkv, P,
                                key_mixed, value_mixed, key_norm_u8)

    def cache(self, batch, max_tokens):
        max_pages = max(1, -(-max(max_tokens - self.W, 0) // self.P))
        c = pages.PagedCache(self.lay, self.R, self.kcb, self.vcb, self.S, self.W,
                             num_pages=batch * max_pages + 3, batch=batch, max_pages=max_pages,
                             rotation_kind=0 if self.rotation == "dense" else 1, seed=self.seed,
                             qjl_coef=self.qjl_coef)
        # scatter pages over the pool (not in sequence order) so block tables matter
        perm = np.random.default_rng(123).permutation(batch * max_pages) + 3
        c.block_table[:] = perm.reshape(batch, max_pages)
        return c


def fill(setup, cache, lens, layer=0, chunked=False):
    """Prefill each sequence b with lens[b] tokens of config-0-style K/V."""
    B = len(lens)
    Tm = int(max(lens))
    k = np.zeros((B, setup.Hkv, Tm, setup.d), np.float16)
    v = np.zeros_like(k)
    for b in range(B):
        for h in range(setup.Hkv):
            kk, vv = tq_inputs.kv_block(setup.seed, setup.d, int(lens[b]), layer, h, b)
            k[b, h, :lens[b]] = kk
            v[b, h, :lens[b]] = vv
    if not chunked:
        cache.append(k, v, counts=np.asarray(lens))
    else:
        for t in range(Tm):
            cnt = (np.asarray(lens) > t).astype(np.int64)
            cache.append(k[:, :, t:t + 1], v[:, :, t:t + 1], counts=cnt)
    return k, v
