"""Pins for the mixed-channel fractional rates of the oracle ("TurboQuant
Family Design Study", section "Packed format and complete bit accounting":
2.5 bits per channel = 64 channels at 2 bits + 64 at 3; 3.5 = 64 at 3 + 64 at
4, for d = 128; recommended first mode keys 3.5, values 3.0, section "Final
recommendation and expected gains": R_mem = 4 / ((bK + bV)/8) = 4.92)."""

import math

import numpy as np
import pytest

from oracle import accounting
from oracle import codebook as cbm
from oracle import codec
from oracle import mixed
from oracle import pages
from oracle import rotation as rot
from oracle.attention import attention_compressed, attention_plain
from oracle_cache import Setup, fill
import tq_inputs


@pytest.mark.parametrize("rate", ["2.5", "3.5"])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_channel_split_and_record_bytes(golden, rate, kind):
    """64 coordinates at each of the two printed widths; the record holds
    exactly their bits (40 bytes at 2.5, 56 at 3.5)."""
    g = golden["design_study_mixed_channel"]
    d = g["head_dim"]
    (n_lo, b_lo), (n_hi, b_hi) = g["rates"][rate]
    cb = mixed.MixedCodebook(b_lo, d, kind)
    w = cb.width()
    assert np.sum(w == b_lo) == n_lo and np.sum(w == b_hi) == n_hi and b_hi == b_lo + 1
    assert cb.record_bytes(d) * 8 == n_lo * b_lo + n_hi * b_hi
    assert cb.record_bytes(d) == {"2.5": 40, "3.5": 56}[rate]
    assert cb.record_bytes(d) * 8 / d == float(rate)


def test_high_rate_sets():
    """Keys: coordinates 16..31 of every 32; values: 4..7 of every 8."""
    k = mixed.hi_mask(128, "key")
    v = mixed.hi_mask(128, "value")
    assert np.array_equal(k.reshape(4, 32), np.tile(np.arange(32) >= 16, (4, 1)))
    assert np.array_equal(v.reshape(16, 8), np.tile(np.arange(8) >= 4, (16, 1)))


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_quantize_is_per_half_nearest(bits, kind):
    """Each coordinate takes the nearest level of its own half's codebook."""
    cb = mixed.MixedCodebook(bits, 128, kind)
    y = np.random.default_rng(1).standard_normal((200, 128)) / math.sqrt(128) * 1.5
    y32 = y.astype(np.float32).astype(np.float64)
    idx = cb.quantize(y32)
    lo, hi = cbm.Codebook(bits, 128), cbm.Codebook(bits + 1, 128)
    m = cb.hi_mask
    assert np.array_equal(idx[:, m], hi.nearest(y32[:, m]))
    assert np.array_equal(idx[:, ~m], lo.nearest(y32[:, ~m]))
    assert idx[:, ~m].max() < (1 << bits) and idx[:, m].max() < (1 << (bits + 1))


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_pack_layout_literal(bits, kind):
    """Low-rate codes first (ascending coordinate, LSB-first at b bits), then
    the high-rate codes at b + 1 bits; unpack inverts pack."""
    d = 128
    cb = mixed.MixedCodebook(bits, d, kind)
    r = np.random.default_rng(2)
    idx = np.where(cb.hi_mask, r.integers(0, 1 << (bits + 1), (5, d)), r.integers(0, 1 << bits, (5, d)))
    packed = cb.pack(idx)
    assert packed.shape == (5, cb.record_bytes(d))
    stream = np.unpackbits(packed, axis=-1, bitorder="little").astype(np.int64)
    lo_j = [j for j in range(d) if not cb.hi_mask[j]]
    hi_j = [j for j in range(d) if cb.hi_mask[j]]
    for rank, j in enumerate(lo_j):
        got = sum(int(stream[3, rank * bits + k]) << k for k in range(bits))
        assert got == idx[3, j]
    base = (d // 2) * bits
    for rank, j in enumerate(hi_j):
        got = sum(int(stream[3, base + rank * (bits + 1) + k]) << k for k in range(bits + 1))
        assert got == idx[3, j]
    assert np.array_equal(cb.unpack(packed, d), idx)


@pytest.mark.parametrize("bits", [2, 3])
def test_mse_is_mean_of_the_two_widths(golden, bits):
    """Random unit vectors at d=128, rotated and quantised at b + 1/2: the
    relative error is the mean of the two halves' Gaussian distortions (closed
    form of the stored levels), within Monte Carlo error and the finite-d gap
    of the integer widths; it lies between the printed b and b+1 MSEs."""
    d = 128
    r = np.random.default_rng(12)
    x = r.standard_normal((20_000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    cb = mixed.MixedCodebook(bits, d, "value")
    enc = codec.encode(u, R, cb)
    uh = codec.dequantize(enc.codes, enc.norms, R, cb)
    err = np.sum((u - uh) ** 2, axis=1)
    mse, se = err.mean(), err.std(ddof=1) / math.sqrt(len(err))
    dist = lambda cbk: cbm.gaussian_distortion(cbk.centroids * math.sqrt(d))
    want = 0.5 * (dist(cb.lo) + dist(cb.hi))
    # the integer widths themselves sit within 3% of the closed form at d=128
    assert abs(mse - want) < 4 * se + 0.03 * want
    g = golden["validated_mse"]
    lo_printed, hi_printed = g["mse"][g["bits"].index(bits)], g["mse"][g["bits"].index(bits + 1)]
    assert hi_printed < mse < lo_printed
    # per half: each half's own error equals its integer width's
    for half, cbk in ((~cb.hi_mask, cb.lo), (cb.hi_mask, cb.hi)):
        e_half = np.sum(((u - 0) @ R.matrix.T - (uh @ R.matrix.T))[:, half] ** 2, axis=1).mean() * 2
        assert abs(e_half - dist(cbk)) < 0.05 * dist(cbk)


def test_memory_compression_of_the_recommended_mode(golden):
    """Keys 3.5 + values 3.0 bits: code bytes per token-head 56 + 48, against
    2 x 2 x 128 FP16 bytes: 4.92 (printed)."""
    g = golden["design_study_compression"]
    d = 128
    k = mixed.MixedCodebook(3, d, "key").record_bytes(d)
    v = cbm.Codebook(3, d).record_bytes(d)
    assert (k, v) == (56, 48)
    assert accounting.memory_compression(g["key_bits"], g["value_bits"]) == pytest.approx(2 * 2 * d / (k + v), rel=1e-12)
    assert round(2 * 2 * d / (k + v), 2) == g["r_mem_about"]


def test_page_layout_and_header():
    """Key codes take 56 bytes per token, value groups hold a b-bit block of
    64 coordinates then a (b+1)-bit block; the header bits bytes carry +16."""
    s = Setup(key_bits=3, value_bits=3, key_mixed=True, value_mixed=True, Hkv=2, P=64, W=0)
    lay = s.lay
    assert lay.k_rec == 56 and lay.v_rec == 56
    assert lay.head_bytes == 4 * 64 + 4 * 64 + 56 * 64 + 16 * 64 + 4 * 64 + 56 * 64
    assert lay.v_group_words == 3 * 64 + 4 * 64
    page = np.zeros(lay.page_bytes, np.uint8)
    pages.write_header(page, lay, 0, 7, 10, 0)
    assert (page[8], page[10]) == (3 + 16, 3 + 16)
    # value group literal: coordinate j = 13 (high-rate, rank 5), coordinate 2 (low-rate, rank 2)
    idx = np.where(s.vcb.hi_mask, np.random.default_rng(3).integers(0, 16, (32, 128)),
                   np.random.default_rng(4).integers(0, 8, (32, 128)))
    rec = codec.Encoded(s.vcb.pack(idx), np.ones(32, np.float32))
    pages.write_value_records(page, lay, 1, np.arange(32), s.vcb, rec)
    words = page[lay.head_base(1) + lay.v_codes:][:32 * 56].view(np.uint32)
    big_hi = sum(int(words[3 * 64 + w * 64 + 5]) << (32 * w) for w in range(4))
    big_lo = sum(int(words[w * 64 + 2]) << (32 * w) for w in range(3))
    for i in range(32):
        assert (big_hi >> (4 * i)) & 15 == idx[i, 13]
        assert (big_lo >> (3 * i)) & 7 == idx[i, 2]
    n, back = pages.read_value_idx(page, lay, 1, 32)
    assert np.array_equal(back, idx)


@pytest.mark.parametrize("kmix,vmix,kb,vb", [(True, False, 3, 3), (True, True, 2, 3), (False, True, 4, 3)])
def test_attention_routes_agree(kmix, vmix, kb, vb):
    """Dequantise-then-softmax and the compressed-domain formula agree in
    float64 for mixed rates too (the algebra does not depend on the widths)."""
    s = Setup(key_bits=kb, value_bits=vb, key_mixed=kmix, value_mixed=vmix, Hq=4, Hkv=2, P=64, W=16)
    cache = s.cache(2, 300)
    fill(s, cache, [300, 157])
    q = tq_inputs.queries(5, (2, 4, 128))
    o1, l1 = attention_plain(cache, q, 1 / math.sqrt(128))
    o2, l2 = attention_compressed(cache, q, 1 / math.sqrt(128))
    assert np.max(np.abs(o1 - o2)) <= 1e-12 * np.max(np.abs(o1))
    for b in range(2):
        for g in range(4):
            assert np.max(np.abs(l1[b][g] - l2[b][g])) <= 1e-12 * np.max(np.abs(l1[b][g]))


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_channel_choice_does_not_change_the_error(bits, kind):
    """The page fixes only the counts (d/2 channels at each width).  Which
    half takes the extra bit is this library's choice (the sets the
    matrix-core scan reads as whole operand slices); after the rotation every
    coordinate has the same distribution, so any fixed half gives the same
    expected error.  Pinned: the library's set and the plain contiguous split
    (coordinates d/2 .. d-1 high-rate) reach the same relative MSE within
    Monte Carlo error on the same 20K rotated unit vectors."""
    d = 128
    x = np.random.default_rng(21).standard_normal((20_000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    R = rot.Rotation("dense", tq_inputs.rotation_draws(0, d), d)
    errs = []
    for contiguous in (False, True):
        cb = mixed.MixedCodebook(bits, d, kind)
        if contiguous:
            cb.hi_mask = np.arange(d) >= d // 2
            cb.lo_idx, cb.hi_idx = np.nonzero(~cb.hi_mask)[0], np.nonzero(cb.hi_mask)[0]
        enc = codec.encode(u, R, cb)
        uh = codec.dequantize(enc.codes, enc.norms, R, cb)
        errs.append(np.sum((u - uh) ** 2, axis=1))
    diff = errs[0] - errs[1]
    assert abs(diff.mean()) < 4 * diff.std(ddof=1) / math.sqrt(len(diff)) + 1e-3 * errs[1].mean()
