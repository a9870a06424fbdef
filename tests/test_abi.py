"""CPU-side tests of the C-ABI library: it loads, exports every symbol its
header declares, sizes pages like the stated format, rejects bad arguments,
and its host-built tables (an independent Lloyd-Max and Householder QR in
C++) agree with the oracle's."""

import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_vector_tq_amd as tqa
from oracle import codebook as cbm
from oracle import pages
from oracle import rotation as rot
import tq_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tqa.LIB_PATH):
        from kv_cache_vector_tq_amd import build
        build.build()
    return tqa.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    return re.findall(r"TQ_API\s+[\w\s\*]+?\b(tq_\w+)\s*\(", src)


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 10
    assert sorted(names) == sorted(tqa.EXPORTED)
    for n in names:
        assert hasattr(L, n), n


@pytest.mark.parametrize("bK,qjl,bV,H,P", [(3, 1, 4, 8, 256), (2, 1, 2, 8, 256), (4, 0, 3, 2, 64), (3, 1, 4, 1, 32)])
def test_page_bytes_matches_layout(L, bK, qjl, bV, H, P):
    p = tqa.make_params(key_bits=bK, key_qjl=qjl, value_bits=bV, num_q_heads=H, num_kv_heads=H, page_tokens=P)
    assert tqa.tq_page_bytes(p) == pages.Layout(128, bK, qjl, bV, H, P).page_bytes


def test_target_page_size(L):
    p = tqa.make_params(key_bits=3, key_qjl=1, value_bits=4, num_q_heads=32, num_kv_heads=8, page_tokens=256)
    # 8 heads x 256 tokens x (72 + 68) bytes + 256-byte header block
    assert tqa.tq_page_bytes(p) == 256 + 8 * 256 * 140


@pytest.mark.parametrize("field,value", [
    ("key_bits", 1), ("key_bits", 5), ("value_bits", 0), ("key_qjl", 2), ("rotation", 7),
    ("num_q_heads", 6), ("num_kv_heads", 0), ("page_tokens", 48), ("page_tokens", 2048), ("window", -1),
    ("head_dim", 0), ("qjl_kind", 2), ("qjl_shrink", 0.0), ("qjl_shrink", 5.0), ("qjl_shrink", float("nan")),
    ("key_mixed", 2), ("value_mixed", -1), ("key_norm_u8", 2), ("key_norm_u8", -1),
])
def test_bad_params_rejected(L, field, value):
    p = tqa.make_params(num_q_heads=8, num_kv_heads=4)
    setattr(p, field, value)
    assert L.tq_page_bytes(ctypes.byref(p)) == tqa.TQ_ERR_INVALID_ARG
    out = ctypes.c_void_p()
    d = np.zeros(128 * 128)
    assert L.tq_codebook_init(ctypes.byref(out), ctypes.byref(p), d.ctypes.data, d.ctypes.data, None) == \
        tqa.TQ_ERR_INVALID_ARG


def test_null_context_and_pointers(L):
    assert L.tq_encode(None, 0, None, 0, 1, 128, None, None, None, None, None) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_decode_attn(None, None, 0, None, 0, None, 0, 1, None, None, None, 0.1, None, None, 0, 0, None, 0,
                            None) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_append_page(None, None, 0, None, 0, 1, None, None, None, 1, None, None, None, None) == \
        tqa.TQ_ERR_INVALID_ARG
    assert L.tq_destroy(None) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_decode_workspace_bytes(None, 1, 1, 0) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_host_tables(None, None, None, None, None, None, None, None, None) == tqa.TQ_ERR_INVALID_ARG
    assert L.tq_decode_attn_noalloc(None, None, 0, None, 0, None, 0, 1, None, None, None, 0.1, None, 0, None) == \
        tqa.TQ_ERR_INVALID_ARG
    assert L.tq_strerror(tqa.TQ_ERR_WORKSPACE) == b"workspace too small"


def test_read_probe_rejects_bad_arguments(L):
    """tq_read_probe validates on the host before any HIP call (buffer,
    sink and result pointers, size a positive multiple of 16, 16-byte
    alignment, 1..1000 repetitions)."""
    ms = ctypes.c_double(0.0)
    good, sink = 1 << 20, 1 << 21  # aligned stand-in addresses; never dereferenced here
    cases = [(None, 4096, sink, 1), (good, 4096, None, 1), (good, 0, sink, 1), (good, -16, sink, 1),
             (good, 4100, sink, 1), (good + 8, 4096, sink, 1), (good, 4096, sink, 0), (good, 4096, sink, 1001)]
    for buf, nbytes, snk, reps in cases:
        assert L.tq_read_probe(buf, nbytes, snk, reps, ctypes.byref(ms), None) == tqa.TQ_ERR_INVALID_ARG, \
            (buf, nbytes, snk, reps)
    assert L.tq_read_probe(good, 4096, sink, 1, None, None) == tqa.TQ_ERR_INVALID_ARG


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_library_codebook_equals_oracle(L, bits):
    p = tqa.make_params(key_bits=bits, value_bits=bits)
    t = tqa.tq_host_tables(p, tq_inputs.rotation_draws(0, 128), tq_inputs.qjl_draws(0, 128))
    cb = cbm.Codebook(bits, 128)
    assert np.array_equal(t["key_centroids"].astype(np.float64), cb.centroids)
    assert np.array_equal(t["key_boundaries"].astype(np.float64), cb.boundaries)
    assert np.array_equal(t["value_centroids"], t["key_centroids"])


@pytest.mark.parametrize("seed", [0, 1, 7])
def test_library_rotation_equals_oracle(L, seed):
    p = tqa.make_params(seed=seed)
    draws = tq_inputs.rotation_draws(seed, 128)
    t = tqa.tq_host_tables(p, draws, tq_inputs.qjl_draws(seed, 128))
    P = rot.dense_rotation(draws)
    diff = np.abs(t["rotation"].astype(np.float64) - P)
    # independent double-precision QR in both; float32 rounding may differ by one ulp
    assert np.max(diff) <= 2.0 ** -30
    assert np.mean(diff == 0) > 0.999
    S = rot.qjl_matrix(tq_inputs.qjl_draws(seed, 128), 128)
    assert np.array_equal(t["qjl"].astype(np.float64), S)


@pytest.mark.parametrize("seed", [0, 5])
def test_library_orthogonal_qjl_equals_oracle(L, seed):
    p = tqa.make_params(seed=seed, qjl_kind=tqa.TQ_QJL_ORTHOGONAL)
    t = tqa.tq_host_tables(p, tq_inputs.rotation_draws(seed, 128), tq_inputs.qjl_draws(seed, 128))
    S = rot.qjl_matrix(tq_inputs.qjl_draws(seed, 128), 128, "orthogonal")
    diff = np.abs(t["qjl"].astype(np.float64) - S)
    assert np.max(diff) <= 2.0 ** -30
    assert np.mean(diff == 0) > 0.999


def test_library_hadamard_signs(L):
    p = tqa.make_params(rotation=tqa.TQ_ROT_HADAMARD)
    draws = tq_inputs.hadamard_draws(3, 128)
    t = tqa.tq_host_tables(p, draws, tq_inputs.qjl_draws(3, 128))
    assert np.array_equal(t["rotation"], rot.rademacher_signs(draws).astype(np.float32))


@pytest.mark.parametrize("kb,kmix,vb,vmix", [(4, 1, 3, 0), (3, 0, 4, 1)])
def test_mixed_needs_two_or_three_bits(L, kb, kmix, vb, vmix):
    """Mixed-channel rates exist for 2.5 and 3.5 bits only."""
    p = tqa.make_params(key_bits=kb, key_mixed=kmix, value_bits=vb, value_mixed=vmix)
    assert L.tq_page_bytes(ctypes.byref(p)) == tqa.TQ_ERR_INVALID_ARG


def test_mixed_unsupported_on_valu_scan(L):
    """The vector-ALU scan covers integer rates only: rejected at init, before any HIP call."""
    p = tqa.make_params(key_bits=3, key_mixed=1, flags=tqa.TQ_FLAG_VALU_SCAN)
    out = ctypes.c_void_p()
    d = np.zeros(128 * 128)
    assert L.tq_codebook_init(ctypes.byref(out), ctypes.byref(p), d.ctypes.data, d.ctypes.data, None) == \
        tqa.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("kb,kmix,vb,vmix,H,P", [(3, 1, 3, 0, 8, 256), (2, 1, 2, 1, 2, 64), (4, 0, 3, 1, 1, 32)])
def test_mixed_page_bytes_match_layout(L, kb, kmix, vb, vmix, H, P):
    p = tqa.make_params(key_bits=kb, key_mixed=kmix, value_bits=vb, value_mixed=vmix, num_q_heads=H,
                        num_kv_heads=H, page_tokens=P)
    assert tqa.tq_page_bytes(p) == pages.Layout(128, kb, 1, vb, H, P, kmix, vmix).page_bytes


def test_u8_norm_unsupported_on_valu_scan(L):
    """The vector-ALU scan reads float32 key norms only: rejected at init."""
    p = tqa.make_params(key_norm_u8=1, flags=tqa.TQ_FLAG_VALU_SCAN)
    out = ctypes.c_void_p()
    d = np.zeros(128 * 128)
    assert L.tq_codebook_init(ctypes.byref(out), ctypes.byref(p), d.ctypes.data, d.ctypes.data, None) == \
        tqa.TQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("kb,kmix,vb,H,P", [(3, 0, 4, 8, 256), (3, 1, 3, 8, 256), (2, 1, 2, 2, 32)])
def test_u8_norm_page_bytes_match_layout(L, kb, kmix, vb, H, P):
    """u8 log-norm key norms: P bytes per head instead of 4P."""
    p = tqa.make_params(key_bits=kb, key_mixed=kmix, value_bits=vb, num_q_heads=H, num_kv_heads=H, page_tokens=P,
                        key_norm_u8=1)
    lay = pages.Layout(128, kb, 1, vb, H, P, kmix, False, key_norm_u8=True)
    assert tqa.tq_page_bytes(p) == lay.page_bytes
    p0 = tqa.make_params(key_bits=kb, key_mixed=kmix, value_bits=vb, num_q_heads=H, num_kv_heads=H, page_tokens=P)
    assert pages.Layout(128, kb, 1, vb, H, P, kmix, False).head_bytes - lay.head_bytes == 3 * P
    assert tqa.tq_page_bytes(p0) >= tqa.tq_page_bytes(p)


@pytest.mark.parametrize("bits", [2, 3])
def test_library_mixed_codebooks_equal_oracle(L, bits):
    """The b-bit and (b+1)-bit codebooks of a mixed rate, in that order."""
    from oracle import mixed
    p = tqa.make_params(key_bits=bits, key_mixed=1, value_bits=bits, value_mixed=1)
    t = tqa.tq_host_tables(p, tq_inputs.rotation_draws(0, 128), tq_inputs.qjl_draws(0, 128))
    for kind in ("key", "value"):
        cb = mixed.MixedCodebook(bits, 128, kind)
        assert np.array_equal(t[kind + "_centroids"].astype(np.float64), np.concatenate([cb.lo.centroids, cb.hi.centroids]))
        assert np.array_equal(t[kind + "_boundaries"].astype(np.float64),
                              np.concatenate([cb.lo.boundaries, cb.hi.boundaries]))


@pytest.mark.parametrize("d", [96, 72, 120])
@pytest.mark.parametrize("rotation", [tqa.TQ_ROT_DENSE, tqa.TQ_ROT_HADAMARD])
def test_head_sizes_below_the_transform_size(L, d, rotation):
    """Head sizes 72..128 that are not a power of two take the transform size
    D = 128: page bytes as the oracle's layout, tables of D (the rotation and
    S from D x D draws, codebooks at scale 1/sqrt(D))."""
    p = tqa.make_params(head_dim=d, rotation=rotation, num_q_heads=4, num_kv_heads=2, page_tokens=64)
    assert tqa.tq_page_bytes(p) == pages.Layout(d, 3, 1, 4, 2, 64).page_bytes
    assert tqa.tq_page_bytes(p) == tqa.tq_page_bytes(tqa.make_params(head_dim=128, num_q_heads=4, num_kv_heads=2,
                                                                       page_tokens=64))
    seed = 4
    draws = tq_inputs.rotation_draws(seed, 128) if rotation == tqa.TQ_ROT_DENSE else tq_inputs.hadamard_draws(seed, 128)
    t = tqa.tq_host_tables(p, draws, tq_inputs.qjl_draws(seed, 128))
    R = rot.Rotation("dense" if rotation == tqa.TQ_ROT_DENSE else "hadamard", draws, d)
    if rotation == tqa.TQ_ROT_DENSE:
        assert t["rotation"].shape == (128, 128)
        assert np.max(np.abs(t["rotation"].astype(np.float64) - R.matrix)) <= 2.0 ** -30
    else:
        assert np.array_equal(t["rotation"].astype(np.float64), R.eps)
    assert np.array_equal(t["qjl"].astype(np.float64), rot.qjl_matrix(tq_inputs.qjl_draws(seed, 128), 128))
    assert np.array_equal(t["key_centroids"].astype(np.float64), cbm.Codebook(3, 128).centroids)


@pytest.mark.parametrize("d,want", [(64, tqa.TQ_ERR_UNSUPPORTED), (136, tqa.TQ_ERR_UNSUPPORTED),
                                    (256, tqa.TQ_ERR_UNSUPPORTED), (100, tqa.TQ_ERR_INVALID_ARG),
                                    (0, tqa.TQ_ERR_INVALID_ARG)])
def test_head_sizes_without_kernels(L, d, want):
    """Kernels exist for D = 128 (head sizes 72..128 in steps of 8); other
    multiples of 8 are valid parameters (page bytes) but have no kernels, and
    are refused at init before any HIP call."""
    p = tqa.make_params(head_dim=d)
    if want == tqa.TQ_ERR_UNSUPPORTED:
        assert L.tq_page_bytes(ctypes.byref(p)) > 0
    out = ctypes.c_void_p()
    assert L.tq_codebook_init(ctypes.byref(out), ctypes.byref(p), None, None, None) == want
