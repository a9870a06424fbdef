"""Pins of the u8 log-norm key-norm storage (oracle.lognorm; "TurboQuant
Family Design Study", section "Packed format and complete bit accounting").

The page fixes the width (one byte per token-head, 0.0625 bpc at d = 128)
and the log domain; the grid (16 levels per octave, code 128 at 2^4, code 0
for a zero norm) and nearest-level rounding are this build's reading.  The
pins check the width against the page's printed figure, the rounding against
a brute-force nearest level, the error bound of the grid, the unbiasedness of
the QJL estimator when the residual is taken against the stored level, and
the page layout."""

import math

import numpy as np
import pytest

import tq_inputs
from oracle import codebook as cbm
from oracle import codec, lognorm, mixed, pages
from oracle import rotation as rot
from oracle_cache import Setup, fill


def test_bits_per_channel_printed(golden):
    g = golden["design_study_u8_norm"]
    assert lognorm.bits_per_channel(g["head_dim"]) == g["added_bpc"]
    # the page stream: one byte per token instead of four
    a = pages.Layout(128, 3, 1, 3, 8, 32, key_mixed=True)
    b = pages.Layout(128, 3, 1, 3, 8, 32, key_mixed=True, key_norm_u8=True)
    assert a.head_bytes - b.head_bytes == 3 * 32
    assert b.k_rnorm - b.k_norm == g["norm_bytes_per_token_head"] * 32


def test_levels_map_to_themselves():
    lv = lognorm.levels()
    assert lv[0] == 0.0 and lv[128] == 16.0 and lv[144] == 32.0 and lv[112] == 8.0
    q = np.arange(1, 256)
    assert np.array_equal(lognorm.encode(lv[q].astype(np.float32)), q)
    assert lognorm.encode(np.float32(0.0)) == 0


def test_nearest_level_brute_force():
    """Away from the boundaries (within float32 rounding of them the
    comparison decides), the code is the level nearest in log2."""
    rng = np.random.default_rng(3)
    n = np.exp2(rng.uniform(-6.0, 14.0, 20000)).astype(np.float32)
    q = lognorm.encode(n).astype(np.int64)
    lv = lognorm.levels()[1:]
    dist = np.abs(np.log2(n.astype(np.float64))[:, None] - np.log2(lv)[None, :])
    q_bf = 1 + np.argmin(dist, axis=1)
    # distance to the nearest boundary in log2 units
    bl = np.log2(lognorm.boundaries().astype(np.float64))
    near = np.min(np.abs(np.log2(n.astype(np.float64))[:, None] - bl[None, :]), axis=1) < 1e-6
    assert np.array_equal(q[~near], q_bf[~near])
    assert near.sum() < 10


def test_relative_error_bound_and_clamp():
    rng = np.random.default_rng(4)
    lv = lognorm.levels()
    n = np.exp2(rng.uniform(math.log2(lv[1]), math.log2(lv[255]), 50000)).astype(np.float32)
    nh = lognorm.decode(lognorm.encode(n))
    rel = np.abs(nh / n.astype(np.float64) - 1.0)
    bound = 2.0 ** (1.0 / 32.0) - 1.0   # half a step of 2^(1/16)
    assert rel.max() <= bound * (1 + 1e-6)
    assert rel.max() > 0.95 * bound
    big = np.array([lv[255] * 1.5, 1e30], dtype=np.float32)
    small = np.array([lv[1] / 1.5, 1e-30], dtype=np.float32)
    assert np.all(lognorm.encode(big) == 255) and np.all(lognorm.encode(small) == 1)
    s = np.sort(n)
    assert np.all(np.diff(lognorm.encode(s).astype(np.int64)) >= 0)


def test_flat_record_and_zero_vector():
    d = 128
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    cb = cbm.Codebook(3, d)
    S = rot.qjl_matrix(tq_inputs.qjl_draws(0, d), d, "gaussian")
    x = tq_inputs.keys(1, d, np.arange(40)).astype(np.float64)
    x[7] = 0.0
    e = codec.encode(x, R, cb, S, norm_u8=True)
    n32 = np.sqrt(np.sum(x * x, axis=1)).astype(np.float32)
    assert np.array_equal(e.norm_codes, lognorm.encode(n32))
    assert np.array_equal(e.norms, lognorm.decode(e.norm_codes).astype(np.float32))
    assert e.norm_codes[7] == 0 and e.norms[7] == 0 and e.rnorms[7] == 0
    # direction codes do not depend on how the norm is stored
    assert np.array_equal(e.idx, codec.encode(x, R, cb, S).idx)
    # residual against the stored level
    r = codec.residual_from_codes(x, R, cb, e.norms, e.idx)
    assert np.allclose(e.rnorms, np.linalg.norm(r, axis=1), rtol=1e-6)


def test_qjl_unbiased_with_rounded_norm():
    """Averaged over draws of S the key score with the sketch is unbiased for
    q.k even though the stored norm is rounded (the residual holds the
    rounding); a residual against the unrounded norm would leave the
    rounding's bias (about 2% of the score here), many standard errors away."""
    d = 64
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    cb = cbm.Codebook(2, d)
    r0 = np.random.default_rng(8)
    k = r0.standard_normal((1, d))
    # put the norm 0.45 of a step above a level: close to the largest rounding
    target = 2.0 ** ((150 + 0.45) / 16 - 4)
    k *= target / np.linalg.norm(k)
    q = k[0] + 0.5 * r0.standard_normal(d)
    truth = float(q @ k[0])
    rng = np.random.default_rng(9)
    full, wrong = [], []
    for _ in range(3000):
        S = rng.standard_normal((d, d))
        e = codec.encode(k, R, cb, S, norm_u8=True)
        full.append(q @ codec.dequantize(e.codes, e.norms, R, cb, e.signs, e.rnorms, S)[0])
        # the plausible mistake: sketch of the residual against the exact norm
        n = np.linalg.norm(k[0])
        rr = R.forward(k)[0] - n * cb.values(e.idx)[0]
        sig = codec.pack_bits(((S @ rr) >= 0).astype(np.int64)[None, :], 1)
        wrong.append(q @ codec.dequantize(e.codes, e.norms, R, cb, sig, np.array([np.linalg.norm(rr)]), S)[0])
    full, wrong = np.array(full), np.array(wrong)
    se = full.std(ddof=1) / math.sqrt(full.size)
    assert abs(full.mean() - truth) < 4 * se
    assert abs(wrong.mean() - truth) > 8 * se


def test_page_round_trip_and_header():
    s = Setup(Hq=2, Hkv=2, W=8, P=32, key_bits=3, value_bits=3, key_mixed=True, key_norm_u8=True)
    c = s.cache(2, 100)
    k, v = fill(s, c, [100, 45])
    for b, T in ((0, 100), (1, 45)):
        for pg in range(-(-(T - s.W) // s.P)):
            page = c.pool[int(c.block_table[b, pg])]
            assert page[36] == 1
        for h in range(s.Hkv):
            kr, vn, vi = c.compressed(b, h)
            x = k[b, h, :T - s.W].astype(np.float64)
            n32 = np.sqrt(np.sum(x * x, axis=1)).astype(np.float32)
            assert np.array_equal(kr.norm_codes, lognorm.encode(n32))
            assert np.array_equal(kr.norms, lognorm.decode(kr.norm_codes).astype(np.float32))
            ref = codec.encode(x, s.R, s.kcb, s.S, norm_u8=True)
            assert np.array_equal(kr.codes, ref.codes) and np.array_equal(kr.signs, ref.signs)
            assert np.array_equal(kr.rnorms, ref.rnorms)
