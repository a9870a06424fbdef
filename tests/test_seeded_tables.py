"""The library's seed-only and tables-as-data initialisation, on the CPU.

A caller may give the library only a seed ("aither-kvcache" README, "API
Reference": the quantiser is built from head_dim, bits and a seed).  The
random matrices then come from the library's counter-based generator
(Philox4x32-10 with Box-Muller, stated in include/tq.h).  The test side has
its own implementation of that published generator (oracle/philox.py), pinned
to the generator's published known-answer vectors; the library's draws and
the tables built from them are checked against it.  Tables given as data are
validated on the host before any device work."""

import ctypes
import json
import os

import numpy as np
import pytest

import kv_cache_vector_tq_amd as tqa
from oracle import philox
from oracle import rotation as rot

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tqa.LIB_PATH):
        from kv_cache_vector_tq_amd import build
        build.build()
    return tqa.lib()


def test_philox_known_answers():
    kat = json.load(open(os.path.join(ROOT, "tests", "golden", "philox_kat.json")))
    for v in kat["vectors"]:
        ctr = np.array([[int(x, 16) for x in v["ctr"]]], dtype=np.uint64)
        key = tuple(int(x, 16) for x in v["key"])
        out = philox.philox4x32_10(ctr, key)[0]
        assert ["%08x" % int(x) for x in out] == v["out"]


def test_oracle_draws_are_standard_normal():
    z = philox.normals(0, philox.STREAM_QJL, 100_001)
    assert z.shape == (100_001,)
    assert abs(z.mean()) < 4 / np.sqrt(len(z))
    assert abs(z.var() - 1.0) < 4 * np.sqrt(2 / len(z))
    assert abs(np.mean(z ** 4) - 3.0) < 0.1
    # streams and seeds are different sequences
    assert not np.array_equal(z[:100], philox.normals(0, philox.STREAM_ROTATION, 100))
    assert not np.array_equal(z[:100], philox.normals(1, philox.STREAM_QJL, 100))


@pytest.mark.parametrize("seed", [0, 1, 2 ** 40 + 3])
@pytest.mark.parametrize("stream", [tqa.TQ_DRAWS_ROTATION, tqa.TQ_DRAWS_QJL, tqa.TQ_DRAWS_HADAMARD])
def test_library_draws_equal_oracle(L, seed, stream):
    n = 4097
    lib = tqa.tq_seed_draws(seed, stream, n)
    ref = philox.normals(seed, stream, n)
    assert np.array_equal(lib, ref)


def test_library_draws_reject_bad_arguments(L):
    out = np.zeros(4)
    assert L.tq_seed_draws(0, 0, 4, out.ctypes.data) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_seed_draws(0, 4, 4, out.ctypes.data) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_seed_draws(0, 1, -1, out.ctypes.data) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_seed_draws(0, 1, 4, None) == tqa.TQ_ERR_INVALID_ARG


@pytest.mark.parametrize("seed", [0, 9])
@pytest.mark.parametrize("rotation", [tqa.TQ_ROT_DENSE, tqa.TQ_ROT_HADAMARD])
@pytest.mark.parametrize("qjl_kind", [tqa.TQ_QJL_GAUSSIAN, tqa.TQ_QJL_ORTHOGONAL])
def test_seeded_tables_equal_tables_from_the_draws(L, seed, rotation, qjl_kind):
    """Seed only = the same tables as the oracle's generator's draws passed in."""
    p = tqa.make_params(seed=seed, rotation=rotation, qjl_kind=qjl_kind)
    rd = philox.rotation_draws(seed, 128) if rotation == tqa.TQ_ROT_DENSE else philox.hadamard_draws(seed, 128)
    a = tqa.tq_host_tables(p)
    b = tqa.tq_host_tables(p, rd, philox.qjl_draws(seed, 128))
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_seeded_rotation_matches_the_oracle(L):
    """The seed-built dense rotation equals the oracle's QR of its own
    generator's draws (to float32 rounding) and is orthogonal; the seed-built
    Gaussian S is those draws rounded to float32."""
    p = tqa.make_params(seed=4)
    t = tqa.tq_host_tables(p)
    P = rot.dense_rotation(philox.rotation_draws(4, 128))
    assert np.max(np.abs(t["rotation"].astype(np.float64) - P)) <= 2.0 ** -30
    R = t["rotation"].astype(np.float64)
    assert np.max(np.abs(R @ R.T - np.eye(128))) < 1e-5
    assert np.array_equal(t["qjl"], philox.qjl_draws(4, 128).astype(np.float32))


def _init_tables(L, p, **arrays):
    keep = {k: np.ascontiguousarray(v, np.float32) for k, v in arrays.items()}
    t = tqa.tq_tables(*[keep[k].ctypes.data if k in keep else None
                        for k in ("rotation", "qjl", "key_centroids", "value_centroids")])
    out = ctypes.c_void_p()
    return L.tq_codebook_init_tables(ctypes.byref(out), ctypes.byref(p), ctypes.byref(t), None)


def test_tables_as_data_are_validated_on_the_host(L):
    """Bad tables are rejected before any device work (this runs without a GPU)."""
    p = tqa.make_params()
    bad_rot = np.eye(128)
    bad_rot[3, 4] = np.nan
    assert _init_tables(L, p, rotation=bad_rot) == tqa.TQ_ERR_INVALID_ARG
    s = np.zeros((128, 128))
    s[0, 0] = np.inf
    assert _init_tables(L, p, qjl=s) == tqa.TQ_ERR_INVALID_ARG
    cen = np.linspace(-0.2, 0.2, 8)
    cen[4] = cen[3]
    assert _init_tables(L, p, key_centroids=cen) == tqa.TQ_ERR_INVALID_ARG
    # levels that collapse once rounded to half precision
    assert _init_tables(L, p, value_centroids=np.linspace(0.1, 0.1 + 15e-6, 16)) == tqa.TQ_ERR_INVALID_ARG
    ph = tqa.make_params(rotation=tqa.TQ_ROT_HADAMARD)
    signs = np.ones(128)
    signs[7] = 0.5
    assert _init_tables(L, ph, rotation=signs) == tqa.TQ_ERR_INVALID_ARG
    bad_p = tqa.make_params(key_bits=9)
    assert _init_tables(L, bad_p) == tqa.TQ_ERR_INVALID_ARG
    unsup = tqa.make_params(key_norm_u8=1, flags=tqa.TQ_FLAG_VALU_SCAN)
    assert _init_tables(L, unsup) == tqa.TQ_ERR_UNSUPPORTED
