"""Pins for head sizes that are not a power of two (d = 96, 80, 72 with the
transform size D = 128).

"TurboQuant Family Design Study", section "Dense and structured transform
comparison", handles such heads by zero-padding to the next power of two
during append and the query transform.  The oracle's reading (stated in
``oracle.rotation``): records hold all D transform coordinates, FP16 vectors,
queries and outputs keep d.  The pins check what that reading fixes by
mathematics alone: the padded transform is an isometry of R^d into R^D and
its inverse recovers x exactly, inner products survive it (the identity
q.k = (Tq).(Tk) the compressed-domain scores rest on), the rotated
coordinates of a unit vector are close to N(0, 1/D) so the D-level codebook
keeps the printed unit-vector MSE, the error splits exactly between the d
kept and the D - d dropped coordinates, both decode routes agree, and the
record sizes follow D bits per coordinate.
"""

import numpy as np
import pytest

from oracle import attention
from oracle import codebook as cbm
from oracle import codec
from oracle import pages
from oracle import rotation as rot
import tq_inputs
from oracle_cache import Setup, fill

DIMS = [96, 80, 72]


def _rotation(kind, d, seed=0):
    D = rot.transform_dim(d)
    draws = tq_inputs.rotation_draws(seed, D) if kind == "dense" else tq_inputs.hadamard_draws(seed, D)
    return rot.Rotation(kind, draws, d)


def test_transform_dim():
    assert [rot.transform_dim(d) for d in (1, 2, 3, 64, 65, 72, 96, 128, 129)] == [1, 2, 4, 64, 128, 128, 128, 128, 256]


@pytest.mark.parametrize("kind", ["dense", "hadamard"])
@pytest.mark.parametrize("d", DIMS)
def test_padded_transform_is_an_isometry_and_inverts(kind, d):
    R = _rotation(kind, d)
    x = np.random.default_rng(d).standard_normal((64, d))
    y = R.forward(x)
    assert y.shape == (64, 128)
    # the dense matrix holds float32 values, orthogonal to ~1e-7
    tol = 1e-6 if kind == "dense" else 1e-13
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=tol)
    np.testing.assert_allclose(R.inverse(y), x, atol=10 * tol)
    # padding is what the forward map does to a d-vector: a D-vector with a
    # zero tail maps to the same coordinates
    xz = np.concatenate([x, np.zeros((64, 128 - d))], axis=1)
    np.testing.assert_array_equal(R.forward(xz), y)


@pytest.mark.parametrize("kind", ["dense", "hadamard"])
def test_inner_products_survive_the_padded_transform(kind):
    d = 96
    R = _rotation(kind, d, seed=3)
    r = np.random.default_rng(5)
    q, k = r.standard_normal((32, d)), r.standard_normal((32, d))
    want = np.sum(q * k, axis=1)
    got = np.sum(R.forward(q) * R.forward(k), axis=1)
    np.testing.assert_allclose(got, want, atol=1e-5 if kind == "dense" else 1e-12)


def test_hadamard_basis_vectors_spread_evenly():
    """Each basis vector e_j (j < d) maps to D coordinates of magnitude
    exactly 1/sqrt(D): a sign-flipped column of the Sylvester matrix."""
    R = _rotation("hadamard", 96, seed=7)
    y = R.forward(np.eye(96))
    np.testing.assert_allclose(np.abs(y), 1 / np.sqrt(128), rtol=0, atol=1e-15)


@pytest.mark.parametrize("kind", ["dense", "hadamard"])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unit_vector_mse_at_d96(golden, kind, bits):
    """20K unit vectors of R^96: the D = 128 rotated coordinates are close
    to N(0, 1/D), so the D-level codebook's error over all D coordinates
    matches the printed unit-vector MSE (README "Validated MSE") within 3%;
    that error splits exactly into the part on the d kept coordinates and
    the part the inverse drops, and the kept part is what the cache returns."""
    d, D = 96, 128
    g = golden["validated_mse"]
    printed = g["mse"][g["bits"].index(bits)]
    x = np.random.default_rng(3).standard_normal((20_000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    R = _rotation(kind, d)
    cb = cbm.Codebook(bits, D)
    enc = codec.encode(u, R, cb)
    y_hat = enc.norms[:, None].astype(np.float64) * cb.values(cb.unpack(enc.codes, D))
    full = np.sum((R.forward(u) - y_hat) ** 2, axis=1)
    u_hat = codec.dequantize(enc.codes, enc.norms, R, cb)
    kept = np.sum((u - u_hat) ** 2, axis=1)
    if kind == "dense":
        back = y_hat @ R.matrix
    else:
        back = rot.fwht(y_hat) * R.eps / np.sqrt(D)
    dropped = np.sum(back[:, d:] ** 2, axis=1)
    assert abs(np.mean(full) - printed) / printed < 0.03
    np.testing.assert_allclose(kept + dropped, full, rtol=1e-5 if kind == "dense" else 1e-10)
    assert np.all(dropped >= 0) and np.mean(kept) < np.mean(full)


def test_record_sizes_follow_the_transform_size():
    """A d = 96 head stores D = 128 coordinates: b*D/8 key code bytes, D/8
    sign bytes, bV*D/8 value code bytes per token; the header keeps d."""
    lay = pages.Layout(96, 3, 1, 4, num_kv_heads=2, page_tokens=64)
    assert (lay.d, lay.D) == (96, 128)
    assert lay.k_rec == 3 * 128 // 8 and lay.v_rec == 4 * 128 // 8
    per_token = 4 + 4 + 3 * 128 // 8 + 128 // 8 + 4 + 4 * 128 // 8
    assert lay.head_bytes == 64 * per_token
    page = np.zeros(lay.page_bytes, np.uint8)
    pages.write_header(page, lay, 0, 1, 5, 0)
    assert int(page[6:8].view(np.uint16)[0]) == 96


@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("key_mixed", [False, True])
def test_decode_routes_agree_at_d96(rotation, key_mixed):
    """Plain attention over dequantised keys and values (d coordinates)
    against the compressed-domain route (D coordinates): equal in exact
    arithmetic, so to rounding here."""
    s = Setup(d=96, rotation=rotation, Hq=4, Hkv=2, P=32, W=16, key_mixed=key_mixed, key_bits=2 if key_mixed else 3)
    lens = [100, 17, 0]
    c = s.cache(3, 100)
    fill(s, c, lens)
    q = np.random.default_rng(9).standard_normal((3, 4, 96))
    sm = 1 / np.sqrt(96)
    o1, l1 = attention.attention_plain(c, q, sm)
    o2, l2 = attention.attention_compressed(c, q, sm)
    assert o1.shape == (3, 4, 96)
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    for b in range(3):
        for g in range(4):
            np.testing.assert_allclose(l2[b][g], l1[b][g], atol=1e-12)


def test_page_round_trip_at_d96():
    """Records written into pages read back exactly as encoded."""
    s = Setup(d=96, Hq=2, Hkv=2, P=32, W=0)
    c = s.cache(1, 40)
    fill(s, c, [40])
    k, v = tq_inputs.kv_block(s.seed, 96, 40, 0, 1, 0)
    k = np.asarray(k, np.float16).astype(np.float64)
    v = np.asarray(v, np.float16).astype(np.float64)
    krec, vn, vidx = c.compressed(0, 1)
    ke = codec.encode(k, s.R, s.kcb, s.S)
    ve = codec.encode(v, s.R, s.vcb)
    np.testing.assert_array_equal(krec.codes, ke.codes)
    np.testing.assert_array_equal(krec.signs, ke.signs)
    np.testing.assert_array_equal(krec.norms, ke.norms)
    np.testing.assert_array_equal(vidx, s.vcb.unpack(ve.codes, 128))
