"""Pins for the oracle's per-vector codec: record sizes (README "Compression
Ratios" and the 64-byte example in "Where This Fits"), bit packing, zero
vectors ("TurboQuant on a 16GB MacBook", zero-block fix), and the QJL
estimator's unbiasedness, variance and reconstruction error, derived from
the Gaussian-S definition and scale sqrt(pi/2)/d ("The QJL detective story")."""

import math

import numpy as np
import pytest

from oracle import codebook as cbm
from oracle import codec
from oracle import rotation as rot
import tq_inputs


@pytest.mark.parametrize("bits,nbytes", [(4, 64), (3, 48), (2, 32)])
def test_packed_sizes(golden, bits, nbytes):
    d = 128
    cb = cbm.Codebook(bits, d)
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    x = np.random.default_rng(0).standard_normal((7, d))
    enc = codec.encode(x, R, cb)
    assert enc.codes.shape == (7, nbytes) and enc.codes.dtype == np.uint8
    assert enc.norms.dtype == np.float32
    g = golden["compression_ratios"]
    assert enc.codes.shape[1] + 4 == g["bytes_per_vector"][g["bits"].index(bits)]


def test_pack_lsb_first():
    # b=4: code j in the low nibble when j is even
    codes = np.arange(16)[None, :]
    p = codec.pack_bits(codes, 4)
    assert list(p[0]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    # b=3: codes 1..8 -> bitstream
    c3 = np.array([[1, 2, 3, 4, 5, 6, 7, 0]])
    p3 = codec.pack_bits(c3, 3)
    bits = ''.join(format(c, '03b')[::-1] for c in c3[0])  # LSB-first per code
    want = [int(bits[i:i + 8][::-1], 2) for i in range(0, 24, 8)]
    assert list(p3[0]) == want
    # b=1
    assert list(codec.pack_bits(np.array([[1, 0, 0, 0, 0, 0, 0, 1, 1, 1, 0, 0, 0, 0, 0, 0]]), 1)[0]) == [0x81, 0x03]


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_pack_round_trip(bits):
    c = np.random.default_rng(bits).integers(0, 1 << bits, (50, 128))
    assert np.array_equal(codec.unpack_bits(codec.pack_bits(c, bits), bits, 128), c)


def test_zero_vector_decodes_to_zero():
    d = 128
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    cb = cbm.Codebook(3, d)
    S = rot.qjl_matrix(tq_inputs.qjl_draws(0, d), d)
    x = np.zeros((2, d))
    x[1] = np.random.default_rng(0).standard_normal(d)
    enc = codec.encode(x, R, cb, S)
    assert enc.norms[0] == 0 and enc.rnorms[0] == 0
    assert not enc.codes[0].any() and not enc.signs[0].any()
    kh = codec.dequantize(enc.codes, enc.norms, R, cb, enc.signs, enc.rnorms, S)
    assert np.array_equal(kh[0], np.zeros(d))
    assert np.linalg.norm(kh[1] - x[1]) < 0.5 * np.linalg.norm(x[1])


def test_encode_steps_match_definition():
    """Norm, rotation, code choice and residual follow the stated steps."""
    d = 128
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    cb = cbm.Codebook(3, d)
    S = rot.qjl_matrix(tq_inputs.qjl_draws(0, d), d)
    x = tq_inputs.fp16(tq_inputs.keys(0, d, np.arange(64))).astype(np.float64)
    enc = codec.encode(x, R, cb, S)
    n = np.linalg.norm(x, axis=1)
    assert np.array_equal(enc.norms, n.astype(np.float32))
    y = (R.matrix @ (x / n[:, None]).T).T
    idx = cb.nearest(y)
    assert np.mean(idx == enc.idx) > 0.999
    r = (R.matrix @ x.T).T - enc.norms.astype(np.float64)[:, None] * cb.centroids[enc.idx]
    assert np.allclose(enc.rnorms, np.linalg.norm(r, axis=1).astype(np.float32), rtol=1e-6)
    sig = codec.unpack_bits(enc.signs, 1, d)
    assert np.array_equal(sig, ((r @ S.T) >= 0).astype(np.int64))


def test_qjl_unbiased_and_variance():
    """Over many draws of S: the estimate's mean is <q, r> (within 4 SE) and its
    variance is [(pi/2)|q|^2|r|^2 - <q,r>^2]/m for m Gaussian rows."""
    m = 64
    r0 = np.random.default_rng(1)
    q = r0.standard_normal(m)
    r = 0.3 * q + r0.standard_normal(m)
    truth = float(q @ r)
    rng = np.random.default_rng(2)
    est = []
    for _ in range(20):
        S = rng.standard_normal((1000, m, m))
        sig = np.where(np.einsum('nij,j->ni', S, r) >= 0, 1.0, -1.0)
        sq = np.einsum('nij,j->ni', S, q)
        est.append(codec.qjl_scale(m) * np.linalg.norm(r) * np.sum(sq * sig, axis=1))
    est = np.concatenate(est)
    se = est.std(ddof=1) / math.sqrt(est.size)
    assert abs(est.mean() - truth) < 4 * se
    var_theory = ((math.pi / 2) * (q @ q) * (r @ r) - truth ** 2) / m
    assert est.var(ddof=1) == pytest.approx(var_theory, rel=0.05)
    # same estimator through the oracle's helper on one draw
    S1 = rng.standard_normal((m, m))
    s1 = np.where(S1 @ r >= 0, 1.0, -1.0)
    assert codec.qjl_inner_product(q, np.linalg.norm(r), s1, S1) == pytest.approx(
        codec.qjl_scale(m) * np.linalg.norm(r) * float((S1 @ q) @ s1))


def test_qjl_reconstruction_error():
    """E||r_hat - r||^2 = (pi/2 - 1/d) ||r||^2 for Gaussian S (derived from the
    estimator's definition), using the oracle's dequantiser."""
    d = 32
    cb = cbm.Codebook(2, d)
    r = np.random.default_rng(4).standard_normal(d)
    rng = np.random.default_rng(5)
    errs = []
    for _ in range(4000):
        S = rng.standard_normal((d, d))
        sig = codec.pack_bits(((S @ r) >= 0).astype(np.int64)[None, :], 1)
        zero_codes = codec.pack_bits(np.zeros((1, d), dtype=np.int64), 2)
        rh = codec.dequantize_rotated(zero_codes, np.zeros(1), cb, d, sig,
                                      np.array([np.linalg.norm(r)]), S)[0]
        errs.append(np.sum((rh - r) ** 2))
    want = (math.pi / 2 - 1 / d) * (r @ r)
    assert np.mean(errs) == pytest.approx(want, rel=0.05)


def test_qjl_correction_unbiases_key_scores():
    """Averaged over draws of S, key scores with the QJL term are unbiased for
    q.k while the MSE-only score is not (the reason keys carry the sketch)."""
    d = 64
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    cb = cbm.Codebook(2, d)
    r0 = np.random.default_rng(8)
    k = r0.standard_normal((1, d))
    q = k[0] + 0.5 * r0.standard_normal(d)
    truth = float(q @ k[0])
    rng = np.random.default_rng(9)
    full, mse = [], []
    for _ in range(3000):
        S = rng.standard_normal((d, d))
        e = codec.encode(k, R, cb, S)
        full.append(q @ codec.dequantize(e.codes, e.norms, R, cb, e.signs, e.rnorms, S)[0])
        mse.append(q @ codec.dequantize(e.codes, e.norms, R, cb)[0])
    full = np.array(full)
    se = full.std(ddof=1) / math.sqrt(full.size)
    assert abs(full.mean() - truth) < 4 * se
    assert abs(mse[0] - truth) > 4 * se
