"""Pins for the oracle's page model and decode attention.

* Two independent routes (dequantise-then-softmax vs compressed-domain) agree
  to 1e-12, the algebra q.k = (Tq).(Tk) of "TurboQuant Family Design Study",
  section "Placement relative to RoPE and attention".
* T <= W reduces to plain FP16 attention, checked against torch's scaled
  dot-product attention in float64 on the CPU.
* Special cases: one token -> o = v_hat; identical keys -> mean of values;
  Hq = Hkv; identical queries in a GQA group give identical outputs.
* Pages: records round-trip through the byte layout, bulk prefill equals
  token-by-token append byte for byte, headers hold the stated fields.
"""

import numpy as np
import pytest
import torch

from oracle import attention as att
from oracle import codec, pages
import tq_inputs
from oracle_cache import Setup, fill


def _q(setup, B, seed=1):
    return tq_inputs.queries(seed, (B, setup.Hq, setup.d))


@pytest.mark.parametrize("rotation,bK,qjl,bV,qk,shrink", [
    ("dense", 3, 1, 4, "gaussian", 1.0), ("hadamard", 2, 1, 2, "gaussian", 1.0), ("dense", 4, 0, 3, "gaussian", 1.0),
    ("dense", 3, 1, 4, "orthogonal", 2 / np.pi), ("hadamard", 3, 1, 4, "orthogonal", 0.7)])
def test_two_routes_agree(rotation, bK, qjl, bV, qk, shrink):
    s = Setup(key_bits=bK, key_qjl=qjl, value_bits=bV, rotation=rotation, Hq=4, Hkv=2, P=64, W=32,
              qjl_kind=qk, qjl_shrink=shrink)
    lens = [300, 45, 32, 1]
    c = s.cache(len(lens), max(lens))
    fill(s, c, lens)
    q = _q(s, len(lens))
    o1, l1 = att.attention_plain(c, q, 1 / np.sqrt(s.d))
    o2, l2 = att.attention_compressed(c, q, 1 / np.sqrt(s.d))
    assert np.max(np.abs(o1 - o2)) <= 1e-12 * np.max(np.abs(o1))
    for b in range(len(lens)):
        for g in range(s.Hq):
            assert len(l1[b][g]) == lens[b]
            assert np.max(np.abs(l1[b][g] - l2[b][g])) <= 1e-11 * max(1.0, np.max(np.abs(l1[b][g])))


def test_window_only_is_sdpa():
    s = Setup(Hq=4, Hkv=2, P=64, W=128)
    lens = [100, 128, 7]
    c = s.cache(len(lens), max(lens))
    k, v = fill(s, c, lens)
    q = _q(s, len(lens))
    o, _ = att.attention_plain(c, q, 1 / np.sqrt(s.d))
    for b, T in enumerate(lens):
        Q = torch.tensor(q[b], dtype=torch.float64)[:, None, :]                     # [Hq, 1, d]
        K = torch.tensor(k[b, :, :T].astype(np.float64)).repeat_interleave(2, 0)    # [Hq, T, d]
        V = torch.tensor(v[b, :, :T].astype(np.float64)).repeat_interleave(2, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V)[:, 0].numpy()
        assert np.allclose(o[b], ref, rtol=1e-12, atol=1e-12)


def test_single_compressed_token_and_identical_keys():
    s = Setup(P=64, W=0)
    c = s.cache(1, 64)
    x = tq_inputs.fp16(tq_inputs.keys(0, s.d, np.arange(1))).astype(np.float64)
    v = tq_inputs.fp16(np.random.default_rng(0).standard_normal((1, s.d))).astype(np.float64)
    c.append(x[None, None], v[None, None])
    q = _q(s, 1)
    o, l = att.attention_plain(c, q, 1 / np.sqrt(s.d))
    krec, vn, vidx = c.compressed(0, 0)
    vhat = s.R.inverse(vn.astype(np.float64)[:, None] * s.vcb.centroids[vidx])[0]
    assert np.allclose(o[0, 0], vhat, atol=1e-12)
    # 40 identical keys with different values -> uniform weights -> mean of v_hat
    c2 = s.cache(1, 64)
    vs = np.random.default_rng(2).standard_normal((40, s.d))
    c2.append(np.repeat(x, 40, 0)[None, None], vs[None, None])
    o2, l2 = att.attention_plain(c2, q, 1 / np.sqrt(s.d))
    assert np.ptp(l2[0][0]) == 0.0
    _, vn2, vidx2 = c2.compressed(0, 0)
    vh2 = s.R.inverse(vn2.astype(np.float64)[:, None] * s.vcb.centroids[vidx2])
    assert np.allclose(o2[0, 0], vh2.mean(axis=0), atol=1e-12)


def test_gqa_identical_queries_and_mha():
    s = Setup(Hq=4, Hkv=2, P=64, W=16)
    lens = [150]
    c = s.cache(1, 150)
    fill(s, c, lens)
    q = _q(s, 1)
    q[0, 1] = q[0, 0]
    o, _ = att.attention_plain(c, q, 1 / np.sqrt(s.d))
    assert np.array_equal(o[0, 0], o[0, 1])
    assert not np.allclose(o[0, 0], o[0, 2])
    # MHA: heads 0 and 2 of the GQA run read kv heads 0 and 1
    m = Setup(Hq=2, Hkv=2, P=64, W=16)
    cm = m.cache(1, 150)
    fill(m, cm, lens)
    om, _ = att.attention_plain(cm, q[:, [0, 2]], 1 / np.sqrt(s.d))
    assert np.allclose(om[0, 0], o[0, 0], atol=1e-14) and np.allclose(om[0, 1], o[0, 2], atol=1e-14)


def test_bulk_equals_streaming_append():
    s = Setup(key_bits=3, value_bits=3, Hq=2, Hkv=2, P=32, W=20)
    lens = [97, 20, 5]
    c1 = s.cache(3, 97)
    c2 = s.cache(3, 97)
    fill(s, c1, lens)
    fill(s, c2, lens, chunked=True)
    assert np.array_equal(c1.pool, c2.pool)
    assert np.array_equal(c1.k_win, c2.k_win) and np.array_equal(c1.v_win, c2.v_win)
    assert np.array_equal(c1.seq_lens, lens)


def test_page_records_round_trip_and_header():
    s = Setup(key_bits=3, value_bits=3, Hq=2, Hkv=2, P=64, W=8)
    c = s.cache(1, 200)
    k, v = fill(s, c, [200])
    krec, vn, vidx = c.compressed(0, 1)
    x = k[0, 1, :192].astype(np.float64)
    ek = codec.encode(x, s.R, s.kcb, s.S)
    ev = codec.encode(v[0, 1, :192].astype(np.float64), s.R, s.vcb)
    assert np.array_equal(krec.codes, ek.codes) and np.array_equal(krec.signs, ek.signs)
    assert np.array_equal(krec.norms, ek.norms) and np.array_equal(krec.rnorms, ek.rnorms)
    assert np.array_equal(vidx, ev.idx) and np.array_equal(vn, ev.norms)
    page = c.pool[c.block_table[0, 2]]
    hdr = page[:64]
    assert hdr[:4].view(np.uint32)[0] == pages.MAGIC
    assert hdr[16:20].view(np.uint32)[0] == 192 - 128
    assert hdr[32:36].view(np.uint32)[0] == 2
    assert (hdr[8], hdr[9], hdr[10]) == (3, 1, 3)
    assert s.lay.page_bytes % 256 == 0
    assert s.lay.head_bytes == 64 * (4 + 4 + 48 + 16 + 4 + 48)


def test_value_group_layout_literal():
    """Value codes: word w of coordinate j in a 32-token group holds token i's
    code at bits [i*bV, (i+1)*bV) of the concatenated words (w=0 lowest)."""
    s = Setup(key_bits=2, key_qjl=0, value_bits=3, Hkv=1, P=32, W=0)
    lay = s.lay
    page = np.zeros(lay.page_bytes, np.uint8)
    idx = np.random.default_rng(0).integers(0, 8, (32, s.d))
    rec = codec.Encoded(codec.pack_bits(idx, 3), np.ones(32, np.float32))
    pages.write_value_records(page, lay, 0, np.arange(32), s.vcb, rec)
    words = page[lay.head_base(0) + lay.v_codes:][:32 * s.d * 3 // 8].view(np.uint32).reshape(1, 3, s.d)
    j = 5
    big = int(words[0, 0, j]) | (int(words[0, 1, j]) << 32) | (int(words[0, 2, j]) << 64)
    for i in range(32):
        assert (big >> (3 * i)) & 7 == idx[i, j]
    n, back = pages.read_value_idx(page, lay, 0, 32)
    assert np.array_equal(back, idx)
