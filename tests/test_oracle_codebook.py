"""Pins for the oracle's Lloyd-Max codebooks and scalar quantiser.

Printed pins come from tests/golden/printed_values.json ("aither-kvcache"
README, table "Validated MSE").  The rest are closed forms (1-bit level
sqrt(2/pi), distortion 1 - 2/pi), independent numerical integration, the
Lloyd fixed-point conditions and brute force.
"""

import itertools
import math

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cbm
from oracle import codec
from oracle import rotation as rot
import tq_inputs


def test_one_bit_closed_form():
    lv = cbm.lloyd_max_normal(1)
    assert lv[1] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-14)
    assert lv[0] == -lv[1]
    assert cbm.gaussian_distortion(lv) == pytest.approx(1 - 2 / math.pi, abs=1e-14)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_printed_gaussian_distortion(golden, bits):
    g = golden["validated_mse"]
    i = g["bits"].index(bits)
    D = cbm.gaussian_distortion(cbm.lloyd_max_normal(bits))
    # printed to 4 decimals
    assert abs(D - g["mse"][i]) <= 0.5e-4 + 1e-12
    # brackets printed beside it
    assert g["theory_lower"][i] - 0.5e-4 <= D <= g["theory_upper"][i]
    assert D >= 4.0 ** -bits


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_by_quadrature(bits):
    """The closed-form distortion equals direct numerical integration."""
    lv = np.array(cbm.lloyd_max_normal(bits))
    edges = np.concatenate([[-np.inf], (lv[1:] + lv[:-1]) / 2, [np.inf]])
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    tot = 0.0
    for k in range(len(lv)):
        a, b = max(edges[k], -40.0), min(edges[k + 1], 40.0)
        val, _ = integrate.quad(lambda x: (x - lv[k]) ** 2 * pdf(x), a, b, epsabs=1e-15, epsrel=1e-13)
        tot += val
    assert cbm.gaussian_distortion(lv) == pytest.approx(tot, rel=1e-10)


# Max (1960), "Quantizing for minimum distortion", table of optimum levels for
# the unit normal (positive half), to 4 decimals.
MAX_1960 = {
    2: [0.4528, 1.5104],
    3: [0.2451, 0.7560, 1.3439, 2.1520],
    4: [0.1284, 0.3881, 0.6568, 0.9424, 1.2562, 1.6181, 2.0690, 2.7326],
}


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_textbook_levels(bits):
    lv = cbm.lloyd_max_normal(bits)
    pos = lv[len(lv) // 2:]
    assert np.allclose(pos, MAX_1960[bits], atol=1.5e-4)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_lloyd_fixed_point(bits):
    """Each level is the conditional mean of its cell under N(0,1), by quadrature."""
    lv = np.array(cbm.lloyd_max_normal(bits))
    edges = np.concatenate([[-np.inf], (lv[1:] + lv[:-1]) / 2, [np.inf]])
    pdf = lambda x: math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    for k in range(len(lv)):
        a, b = max(edges[k], -40.0), min(edges[k + 1], 40.0)
        m1, _ = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-15)
        m0, _ = integrate.quad(pdf, a, b, epsabs=1e-15)
        assert m1 / m0 == pytest.approx(lv[k], abs=1e-9)
    assert np.all(np.diff(lv) > 0)
    assert np.array_equal(lv, -lv[::-1])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_scaled_codebook_half_and_boundaries(bits):
    cb = cbm.Codebook(bits, 128)
    unit = np.array(cbm.lloyd_max_normal(bits))
    assert np.array_equal(cb.centroids, (unit / math.sqrt(128)).astype(np.float16).astype(np.float64))
    # rounding to half moves each level by at most 2^-11 relative
    assert np.all(np.abs(cb.centroids * math.sqrt(128) / unit - 1) <= 2.0 ** -11)
    # boundaries are exact midpoints
    assert np.array_equal(cb.boundaries, (cb.centroids[1:] + cb.centroids[:-1]) / 2)
    assert np.array_equal(cb.centroids, -cb.centroids[::-1])
    assert cb.boundaries[len(cb.boundaries) // 2] == 0.0
    assert np.all(cb.boundaries > cb.centroids[:-1]) and np.all(cb.boundaries < cb.centroids[1:])


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_boundary_search_equals_exhaustive_argmin(bits):
    """10^6 scalars: boundary comparison == nearest centroid, except within
    float32 rounding of a midpoint (none expected at this sample size)."""
    cb = cbm.Codebook(bits, 128)
    r = np.random.default_rng(7)
    y = (r.standard_normal(1_000_000) / math.sqrt(128)).astype(np.float32).astype(np.float64)
    a = cb.quantize(y)
    b = cb.nearest(y)
    mids = (cb.centroids[1:] + cb.centroids[:-1]) / 2
    near = np.min(np.abs(y[:, None] - mids[None, :]), axis=1) < 1e-7
    assert np.array_equal(a[~near], b[~near])
    # ties: exactly on a boundary goes to the lower index
    assert np.array_equal(cb.quantize(cb.boundaries), np.arange(len(cb.boundaries)))


@pytest.mark.parametrize("bits,d", [(2, 3), (3, 2), (2, 4)])
def test_brute_force_vector_nearest(bits, d):
    """Over all (2^b)^d code vectors the nearest reconstruction is the
    per-coordinate nearest (separability of the squared error)."""
    cb = cbm.Codebook(bits, 128)
    r = np.random.default_rng(3)
    allc = np.array(list(itertools.product(range(1 << bits), repeat=d)))
    recon = cb.centroids[allc]
    for _ in range(200):
        y = (r.standard_normal(d) * 0.12).astype(np.float32).astype(np.float64)
        best = allc[np.argmin(np.sum((recon - y) ** 2, axis=1))]
        assert np.array_equal(best, cb.quantize(y))


@pytest.mark.slow
@pytest.mark.parametrize("bits", [4, 3, 2])
def test_unit_vector_mse_50k(golden, bits):
    """50K random unit vectors at d=128, rotated and quantised: E||u - u_hat||^2
    matches the printed MSE (README "Validated MSE", 50K vectors) within 3%."""
    from oracle import codec
    d = 128
    g = golden["validated_mse"]
    printed = g["mse"][g["bits"].index(bits)]
    r = np.random.default_rng(11)
    x = r.standard_normal((50_000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    cb = cbm.Codebook(bits, d)
    enc = codec.encode(u, R, cb)
    uh = codec.dequantize(enc.codes, enc.norms, R, cb)
    mse = np.mean(np.sum((u - uh) ** 2, axis=1))
    assert abs(mse - printed) / printed < 0.03


def test_half_storage_keeps_the_printed_distortion():
    """The stored levels are rounded to half precision (a format choice the
    pages leave open).  Against levels kept in float32, the Gaussian
    distortion moves by under 1e-5 relative and still rounds to the README's
    printed "Validated MSE" values."""
    for bits, printed in ((2, 0.1175), (3, 0.0345), (4, 0.0095)):
        dh = cbm.gaussian_distortion(cbm.Codebook(bits, 128, "half").centroids * math.sqrt(128))
        ds = cbm.gaussian_distortion(cbm.Codebook(bits, 128, "single").centroids * math.sqrt(128))
        assert abs(dh - ds) <= 1e-5 * ds, bits
        assert round(dh, 4) == printed and round(ds, 4) == printed, bits


def test_half_storage_quality_matches_single_storage():
    """Same quality either way, at the config-0 shape (T = 1024, keys 3-bit +
    QJL, values 4-bit, dense rotation, 256 queries): reconstruction MSE of
    keys and values, logit RMSE and mean output error against exact FP
    attention agree within 0.5% between half- and float32-stored levels.
    (Exact outputs do differ beyond 1e-3: a level moved by its half-precision
    rounding changes a few codes and, through the residual, the QJL signs,
    and each sign flip moves the Gaussian-S correction by a large amount.)"""
    d, T = 128, 1024
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    S = rot.qjl_matrix(tq_inputs.qjl_draws(0, d), d, "gaussian")
    k = tq_inputs.fp16(tq_inputs.keys(0, d, np.arange(T))).astype(np.float64)
    v = tq_inputs.fp16(tq_inputs.values(0, d, T)).astype(np.float64)
    q = tq_inputs.queries(0, (256, d))

    def attn(K, V):
        l = (K @ q.T).T / math.sqrt(d)
        w = np.exp(l - l.max(1, keepdims=True))
        return l, (w @ V) / w.sum(1, keepdims=True)

    le, oe = attn(k, v)
    res = {}
    for st in ("half", "single"):
        kc, vc = cbm.Codebook(3, d, st), cbm.Codebook(4, d, st)
        ek, ev = codec.encode(k, R, kc, S), codec.encode(v, R, vc)
        K = codec.dequantize(ek.codes, ek.norms, R, kc, ek.signs, ek.rnorms, S, codec.qjl_scale(d))
        V = codec.dequantize(ev.codes, ev.norms, R, vc)
        l, o = attn(K, V)
        res[st] = np.array([np.mean(np.sum((K - k) ** 2, 1) / np.sum(k ** 2, 1)),
                            np.mean(np.sum((V - v) ** 2, 1) / np.sum(v ** 2, 1)),
                            np.sqrt(np.mean((l - le) ** 2)),
                            np.mean(np.linalg.norm(o - oe, axis=1) / np.linalg.norm(oe, axis=1))])
    assert np.all(np.abs(res["half"] - res["single"]) <= 5e-3 * res["single"]), res
