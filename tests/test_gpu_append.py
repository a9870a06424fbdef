"""GPU parity of tq_append_page: the pages and rings the GPU writes, read
back through the oracle's page reader, hold the oracle's records (codes and
signs under the guard-band rule), the rings and lengths match exactly, bulk
prefill and token-by-token appends agree, and decode over GPU-built pages
matches the oracle's attention over the same pages."""

import numpy as np
import pytest
import torch

import kv_cache_vector_tq_amd as tqa
from oracle import attention as att
from oracle import codec, pages
import tq_inputs
from gpu_helpers import check_codes, check_signs, context_for, assert_out_close, run_decode, upload_cache
from oracle_cache import Setup, fill

pytestmark = pytest.mark.gpu


def _gpu_append(ctx, dev, k, v, counts=None):
    tqa.tq_append_page(ctx, dev["pool"], dev["block_table"], dev["seq_lens"],
                       torch.from_numpy(k.view(np.uint16)).cuda().view(torch.float16),
                       torch.from_numpy(v.view(np.uint16)).cuda().view(torch.float16),
                       dev["k_win"], dev["v_win"],
                       None if counts is None else torch.from_numpy(np.asarray(counts, np.int32)).cuda(),
                       num_pages=dev["num_pages"])


def _compare_caches(s, ref, pool_gpu, kwin, vwin, lens_gpu):
    assert np.array_equal(lens_gpu, ref.seq_lens)
    assert np.array_equal(kwin, ref.k_win.view(np.uint16)) and np.array_equal(vwin, ref.v_win.view(np.uint16))
    gcache = s.cache(len(lens_gpu), 1)
    gcache.pool = pool_gpu.reshape(ref.pool.shape)
    gcache.block_table = ref.block_table
    gcache.seq_lens = ref.seq_lens
    gcache.k_win = kwin.view(np.float16).reshape(ref.k_win.shape)
    gcache.v_win = vwin.view(np.float16).reshape(ref.v_win.shape)
    for b in range(len(lens_gpu)):
        C = max(int(ref.seq_lens[b]) - s.W, 0)
        for pg in range(-(-C // s.P)):
            pid = int(ref.block_table[b, pg])
            # header identical
            assert np.array_equal(gcache.pool[pid, :64], ref.pool[pid, :64]), (b, pg)
        for h in range(s.Hkv):
            comp_g = gcache.compressed(b, h)
            if comp_g is None:
                continue
            kg, vng, vig = comp_g
            kr, vnr, vir = ref.compressed(b, h)
            # the FP16 inputs of these compressed tokens: reconstruct from the oracle's encode inputs
            x = ref._src_k[(b, h)][:C]
            xv = ref._src_v[(b, h)][:C]
            assert np.array_equal(kg.norms, kr.norms) and np.array_equal(vng, vnr)
            gidx = s.kcb.unpack(kg.codes, s.D)
            check_codes(x, gidx, s.kcb.unpack(kr.codes, s.D), s.R, s.kcb)
            check_codes(xv, vig, vir, s.R, s.vcb)
            if s.qjl:
                check_signs(x, gidx, kg.norms, kg.signs, s.R, s.kcb, s.S)
                assert np.allclose(kg.rnorms, kr.rnorms, rtol=2e-5, atol=1e-30)
    return gcache


def _records_match(s, caches, k, v, lens):
    """Two GPU-built caches of the same tokens hold the same records: norms
    exactly, codes exactly outside the guard band (either neighbour inside
    it), each cache's sign bits those of the oracle for its own codes, the
    residual norms to 2e-5.  (Bulk appends run on the matrix cores, appends
    of a few tokens on the vector ALU: their sums differ in rounding.)"""
    a, b2 = caches
    for b in range(len(lens)):
        for h in range(s.Hkv):
            ca, cb = a.compressed(b, h), b2.compressed(b, h)
            if ca is None:
                assert cb is None
                continue
            (ka, vna, via), (kb, vnb, vib) = ca, cb
            C = ka.norms.shape[0]
            x = k[b, h, :C].astype(np.float64)
            xv = v[b, h, :C].astype(np.float64)
            assert np.array_equal(ka.norms, kb.norms) and np.array_equal(vna, vnb), (b, h)
            ia, ib = s.kcb.unpack(ka.codes, s.D), s.kcb.unpack(kb.codes, s.D)
            check_codes(x, ia, ib, s.R, s.kcb)
            check_codes(xv, via, vib, s.R, s.vcb)
            if s.qjl:
                check_signs(x, ia, ka.norms, ka.signs, s.R, s.kcb, s.S)
                check_signs(x, ib, kb.norms, kb.signs, s.R, s.kcb, s.S)
                assert np.allclose(ka.rnorms, kb.rnorms, rtol=2e-5, atol=1e-30)


def _host_cache(s, dv, B, T):
    g = s.cache(B, T)
    g.pool = dv["pool"].cpu().numpy().reshape(g.pool.shape)
    g.seq_lens = dv["seq_lens"].cpu().numpy()
    g.block_table = dv["block_table"].cpu().numpy()
    g.k_win = dv["k_win"].cpu().numpy()
    g.v_win = dv["v_win"].cpu().numpy()
    return g


def _track_sources(s, cache, k, v, lens):
    cache._src_k, cache._src_v = {}, {}
    for b in range(len(lens)):
        for h in range(s.Hkv):
            cache._src_k[(b, h)] = k[b, h, :lens[b]].astype(np.float64)
            cache._src_v[(b, h)] = v[b, h, :lens[b]].astype(np.float64)


CASES = [
    ("cfg0_W128", dict(Hq=1, Hkv=1, W=128), [1024]),
    ("gqa_ragged_P64", dict(Hq=8, Hkv=2, W=40, P=64), [300, 41, 40, 7, 0, 129]),
    ("hadamard_k2v2_W0", dict(Hq=8, Hkv=1, key_bits=2, value_bits=2, rotation="hadamard", W=0, P=32), [100, 33]),
    ("k4_noqjl_v3", dict(Hq=2, Hkv=2, key_bits=4, key_qjl=0, value_bits=3, W=16, P=32), [77, 16, 15]),
    ("orthoS_shrink", dict(Hq=4, Hkv=2, W=32, P=64, qjl_kind="orthogonal", qjl_shrink=2 / np.pi), [200, 33]),
    # mixed-channel rates (keys / values at 2.5 or 3.5 bits)
    ("mixed_k35_v35", dict(Hq=4, Hkv=2, W=32, P=64, key_bits=3, value_bits=3, key_mixed=True, value_mixed=True),
     [200, 33]),
    ("mixed_k25_v4_hadamard", dict(Hq=8, Hkv=2, W=16, P=32, key_bits=2, key_mixed=True, value_bits=4,
                                   rotation="hadamard"), [100, 47]),
    ("mixed_k3_v25_noqjl", dict(Hq=2, Hkv=2, key_bits=3, key_qjl=0, value_bits=2, value_mixed=True, W=0, P=32),
     [77, 16]),
    # u8 log-norm key norms
    ("u8norm_k35_v3", dict(Hq=4, Hkv=2, W=32, P=64, key_bits=3, key_mixed=True, value_bits=3, key_norm_u8=True),
     [200, 33]),
    ("u8norm_k3_v4_hadamard", dict(Hq=8, Hkv=2, W=16, P=32, rotation="hadamard", key_norm_u8=True), [100, 47]),
    # head sizes below the transform size (zero-padded to D = 128)
    ("d96_k3qjl_v4", dict(d=96, Hq=8, Hkv=2, W=40, P=64), [300, 41, 40, 7, 0, 129]),
    ("d96_k2qjl_v2_hadamard", dict(d=96, Hq=4, Hkv=2, key_bits=2, value_bits=2, rotation="hadamard", W=16, P=32),
     [100, 33]),
    ("d72_k35_v3_u8norm", dict(d=72, Hq=4, Hkv=2, W=32, P=64, key_bits=3, key_mixed=True, value_bits=3,
                               key_norm_u8=True), [200, 33]),
    ("d120_k4_noqjl_v3", dict(d=120, Hq=2, Hkv=2, key_bits=4, key_qjl=0, value_bits=3, W=16, P=32), [77, 16, 15]),
]


@pytest.mark.parametrize("name,kw,lens", CASES, ids=[c[0] for c in CASES])
def test_bulk_prefill_parity(name, kw, lens):
    print(f"case {name}", flush=True)
    s = Setup(**kw)
    ref = s.cache(len(lens), max(lens))
    k, v = fill(s, ref, lens)
    _track_sources(s, ref, k, v, lens)
    ctx = context_for(s)
    empty = s.cache(len(lens), max(lens))
    dev = upload_cache(empty)
    _gpu_append(ctx, dev, k, v, counts=lens)
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) == 0
    g = _compare_caches(s, ref, dev["pool"].cpu().numpy(), dev["k_win"].cpu().view(torch.int16).numpy().view(np.uint16),
                        dev["v_win"].cpu().view(torch.int16).numpy().view(np.uint16), dev["seq_lens"].cpu().numpy())
    # decode over the GPU-built cache against the oracle's attention over the same bytes
    q = tq_inputs.queries(8, (len(lens), s.Hq, s.d))
    out, dbg = run_decode(ctx, torch.from_numpy(q.astype(np.float32)).cuda(), dev, 1 / np.sqrt(s.d),
                          logits_len=max(lens) + 1)
    ref_o, _ = att.attention_plain(g, q.astype(np.float32).astype(np.float64), 1 / np.sqrt(s.d))
    for b in range(len(lens)):
        for hq in range(s.Hq):
            if lens[b]:
                assert_out_close(out[b, hq], ref_o[b, hq], 1e-3, (b, hq))


@pytest.mark.parametrize("d", [128, 96])
@pytest.mark.parametrize("kn8", [False, True])
@pytest.mark.parametrize("late_step", [5, 20, 30])
def test_streaming_appends_match_bulk(late_step, kn8, d):
    """Chunked appends (1 token, then late_step tokens: up to and beyond the
    window, evictions spanning two 32-token groups) equal one bulk append."""
    print(f"case streaming late_step={late_step} u8 key norms={kn8} d={d}", flush=True)
    s = Setup(d=d, Hq=4, Hkv=2, W=24, P=32, key_norm_u8=kn8)
    lens = [90, 30]
    ref = s.cache(2, 90)
    k, v = fill(s, ref, lens)
    ctx = context_for(s)
    # bulk on one cache, 1-token and 5-token chunks on another
    d1 = upload_cache(s.cache(2, 90))
    _gpu_append(ctx, d1, k, v, counts=lens)
    d2 = upload_cache(s.cache(2, 90))
    t = 0
    while t < max(lens):
        step = 1 if t < 40 else late_step
        cnt = np.clip(np.asarray(lens) - t, 0, step)
        kk = np.ascontiguousarray(k[:, :, t:t + step])
        vv = np.ascontiguousarray(v[:, :, t:t + step])
        if kk.shape[2] < step:
            pad = step - kk.shape[2]
            kk = np.concatenate([kk, np.zeros(kk.shape[:2] + (pad, s.d), np.float16)], 2)
            vv = np.concatenate([vv, np.zeros(vv.shape[:2] + (pad, s.d), np.float16)], 2)
        _gpu_append(ctx, d2, kk, vv, counts=cnt)
        t += step
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) == 0
    for key in ("k_win", "v_win", "seq_lens"):
        assert torch.equal(d1[key].cpu(), d2[key].cpu()), key
    g1, g2 = _host_cache(s, d1, 2, 90), _host_cache(s, d2, 2, 90)
    for b in range(2):
        for pg in range(-(-max(lens[b] - s.W, 0) // s.P)):
            pid = int(g1.block_table[b, pg])
            assert np.array_equal(g1.pool[pid, :64], g2.pool[pid, :64]), (b, pg)  # headers
    _records_match(s, (g1, g2), k, v, lens)


def test_invalid_page_leaves_sequence_unchanged():
    s = Setup(Hq=2, Hkv=1, W=8, P=32)
    lens = [50, 50]
    c = s.cache(2, 50)
    k, v = fill(s, s.cache(2, 50), lens)
    dev = upload_cache(c)
    dev["block_table"][1, 1] = -1
    ctx = context_for(s)
    before = dev["pool"].clone()
    _gpu_append(ctx, dev, k, v, counts=lens)
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) & tqa.TQ_STATUS_BAD_PAGE
    lens_after = dev["seq_lens"].cpu().numpy()
    assert lens_after[0] == 50 and lens_after[1] == 0
    # sequence 1's pages untouched
    pb = tqa.tq_page_bytes(ctx.params)
    pid0 = int(c.block_table[1, 0])
    assert torch.equal(dev["pool"][pid0 * pb:(pid0 + 1) * pb].cpu(), before[pid0 * pb:(pid0 + 1) * pb].cpu())
    assert not dev["k_win"][1].any()


@pytest.mark.parametrize("mixed", [False, True])
def test_one_token_append_over_stale_slots(mixed):
    """A sequence shortened by the caller (or a recycled page) leaves stale
    codes in the slots past its length.  One-token appends into those slots
    must replace every bit of their own codes: the records read back equal
    those of a cache built in one bulk append from the same tokens."""
    print(f"case stale-slot one-token append mixed={mixed}", flush=True)
    kw = dict(Hq=2, Hkv=2, W=8, P=32)
    if mixed:
        kw.update(key_bits=3, value_bits=3, key_mixed=True, value_mixed=True)
    s = Setup(**kw)
    T, T_cut = 60, 50
    a_k, a_v = fill(s, s.cache(1, T), [T])
    b_k, b_v = fill(s, s.cache(1, T), [T], layer=1)
    # the mixed stream: tokens from T_cut - W on come from a second draw
    mix_k = a_k.copy(); mix_v = a_v.copy()
    mix_k[:, :, T_cut - s.W:] = b_k[:, :, T_cut - s.W:]
    mix_v[:, :, T_cut - s.W:] = b_v[:, :, T_cut - s.W:]
    ctx = context_for(s)
    # stale cache: all T tokens of stream a, then cut back to T_cut with the
    # ring restored to the mixed stream's last W tokens before T_cut
    d1 = upload_cache(s.cache(1, T))
    _gpu_append(ctx, d1, a_k, a_v, counts=[T])
    torch.cuda.synchronize()
    d1["seq_lens"].fill_(T_cut)
    for t in range(T_cut - s.W, T_cut):
        d1["k_win"][0, :, t % s.W] = torch.from_numpy(mix_k[0, :, t].view(np.uint16)).cuda().view(torch.float16)
        d1["v_win"][0, :, t % s.W] = torch.from_numpy(mix_v[0, :, t].view(np.uint16)).cuda().view(torch.float16)
    for t in range(T_cut, T):
        _gpu_append(ctx, d1, np.ascontiguousarray(mix_k[:, :, t:t + 1]), np.ascontiguousarray(mix_v[:, :, t:t + 1]),
                    counts=[1])
    # reference: one bulk append of the mixed stream
    d2 = upload_cache(s.cache(1, T))
    _gpu_append(ctx, d2, mix_k, mix_v, counts=[T])
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) == 0
    caches = [_host_cache(s, dv, 1, T) for dv in (d1, d2)]
    assert caches[0].seq_lens[0] == T and caches[1].seq_lens[0] == T
    _records_match(s, caches, mix_k, mix_v, [T])
    assert torch.equal(d1["k_win"].cpu(), d2["k_win"].cpu()) and torch.equal(d1["v_win"].cpu(), d2["v_win"].cpu())


MMA_CASES = [
    # name, setup kwargs, prefill lengths, second append (tokens per sequence)
    ("k3qjl_v4_dense", dict(Hq=8, Hkv=2, W=40, P=64), [300, 41, 40, 7, 0, 129], 37),
    ("k2qjl_v2_hadamard", dict(Hq=8, Hkv=2, key_bits=2, value_bits=2, rotation="hadamard", W=16, P=32), [200, 77], 50),
    ("k4_noqjl_v3", dict(Hq=4, Hkv=2, key_bits=4, key_qjl=0, value_bits=3, W=8, P=64), [333, 64, 17], 9),
    ("k3qjl_u8norm_v4", dict(Hq=4, Hkv=1, W=0, P=32, key_norm_u8=True), [150, 31], 20),
    ("orthoS_k3_v2", dict(Hq=4, Hkv=2, value_bits=2, W=24, P=64, qjl_kind="orthogonal", qjl_shrink=0.7), [90, 260], 33),
    ("d96_k3qjl_v4", dict(d=96, Hq=8, Hkv=2, W=40, P=64), [300, 41, 40, 7, 0, 129], 37),
    ("d80_k2qjl_v3_hadamard", dict(d=80, Hq=4, Hkv=2, key_bits=2, value_bits=3, rotation="hadamard", W=16, P=32),
     [200, 77], 50),
    # mixed-channel rates (keys and values at 2.5 or 3.5 bits)
    ("mixed_k35qjl_v35", dict(Hq=8, Hkv=2, W=40, P=64, key_bits=3, key_mixed=True, value_bits=3, value_mixed=True),
     [300, 41, 40, 7, 0, 129], 37),
    ("mixed_k25qjl_v25_hadamard", dict(Hq=8, Hkv=2, W=16, P=32, key_bits=2, key_mixed=True, value_bits=2,
                                       value_mixed=True, rotation="hadamard"), [200, 77], 50),
    ("mixed_k35qjl_u8norm_v3", dict(Hq=4, Hkv=2, W=24, P=64, key_bits=3, key_mixed=True, value_bits=3,
                                    key_norm_u8=True), [150, 31, 64], 20),
    ("mixed_k3_noqjl_v25", dict(Hq=4, Hkv=2, key_bits=3, key_qjl=0, value_bits=2, value_mixed=True, W=8, P=32),
     [333, 64, 17], 9),
    ("mixed_d96_k35qjl_v35", dict(d=96, Hq=4, Hkv=2, W=40, P=64, key_bits=3, key_mixed=True, value_bits=3,
                                  value_mixed=True), [300, 41], 37),
]


@pytest.mark.parametrize("name,kw,lens,extra", MMA_CASES, ids=[c[0] for c in MMA_CASES])
def test_matrix_core_append_matches_vector_alu_append(name, kw, lens, extra):
    """The bulk append on the matrix cores writes the records of the
    vector-ALU append (flag TQ_FLAG_VALU_APPEND) for the same tokens, under
    the guard-band rule, including a second append that starts inside a
    value group (earlier tokens' bits kept) and takes tokens from the ring;
    both equal the oracle's records."""
    print(f"case mma append {name}", flush=True)
    s = Setup(**kw)
    B = len(lens)
    total = [n + extra for n in lens]
    ref = s.cache(B, max(total))
    k, v = fill(s, ref, total)
    _track_sources(s, ref, k, v, total)
    devs = []
    for flags in (0, tqa.TQ_FLAG_VALU_APPEND):
        ctx = context_for(s, flags)
        dv = upload_cache(s.cache(B, max(total)))
        _gpu_append(ctx, dv, np.ascontiguousarray(k[:, :, :max(lens)]), np.ascontiguousarray(v[:, :, :max(lens)]),
                    counts=lens)
        # the next `extra` tokens of every sequence, as one more bulk append
        kk = np.zeros((B, s.Hkv, extra, s.d), np.float16)
        vv = np.zeros_like(kk)
        for b in range(B):
            kk[b] = k[b, :, lens[b]:lens[b] + extra]
            vv[b] = v[b, :, lens[b]:lens[b] + extra]
        _gpu_append(ctx, dv, kk, vv)
        torch.cuda.synchronize()
        assert tqa.tq_get_status(ctx) == 0
        devs.append(dv)
    g = [_host_cache(s, dv, B, max(total)) for dv in devs]
    for key in ("k_win", "v_win", "seq_lens"):
        assert torch.equal(devs[0][key].cpu(), devs[1][key].cpu()), key
    assert np.array_equal(g[0].seq_lens, np.asarray(total))
    _records_match(s, g, k, v, total)
    _compare_caches(s, ref, devs[0]["pool"].cpu().numpy(), devs[0]["k_win"].cpu().view(torch.int16).numpy().view(np.uint16),
                    devs[0]["v_win"].cpu().view(torch.int16).numpy().view(np.uint16), devs[0]["seq_lens"].cpu().numpy())


@pytest.mark.parametrize("W", [0, 8])
def test_one_token_appends_commit_themselves(W):
    """Decode-step appends commit themselves (the last work-group of each
    sequence advances its length and rewrites its page headers), over more
    calls than there are sets of arrival counts, and equal one bulk append
    of the same tokens.  A sequence whose next page is invalid stops there
    with a status bit while the others go on; a count of 0 leaves a
    sequence as it was."""
    print(f"case self-committing one-token appends W={W}", flush=True)
    s = Setup(Hq=2, Hkv=2, W=W, P=32)
    B, T = 3, 60
    k, v = fill(s, s.cache(B, T), [T] * B)
    ctx = context_for(s)
    dev = upload_cache(s.cache(B, T))
    dev["block_table"][1, 1] = -1  # sequence 1 cannot store past its first page
    stop1 = s.P + W  # its length once the next token would leave the window into page 1
    taken = [0] * B
    for t in range(T):
        cnt = [1, 1, 0 if t % 3 == 2 else 1]
        kk = np.zeros((B, s.Hkv, 1, s.d), np.float16)
        vv = np.zeros((B, s.Hkv, 1, s.d), np.float16)
        for b in range(B):
            kk[b, :, 0] = k[b, :, min(taken[b], T - 1)]
            vv[b, :, 0] = v[b, :, min(taken[b], T - 1)]
        _gpu_append(ctx, dev, kk, vv, counts=cnt)
        for b in range(B):
            if cnt[b] and not (b == 1 and taken[1] >= stop1):
                taken[b] += 1
    torch.cuda.synchronize()
    lens = [int(x) for x in dev["seq_lens"].cpu().numpy()]
    assert lens == [T, stop1, taken[2]] and taken[2] < T
    assert tqa.tq_get_status(ctx) == tqa.TQ_STATUS_BAD_PAGE
    # the same tokens in one bulk append (its own commit kernel)
    ref = upload_cache(s.cache(B, T))
    _gpu_append(ctx, ref, k, v, counts=lens)
    torch.cuda.synchronize()
    for key in ("k_win", "v_win", "seq_lens"):
        assert torch.equal(dev[key].cpu(), ref[key].cpu()), key
    g1, g2 = _host_cache(s, dev, B, T), _host_cache(s, ref, B, T)
    for b in range(B):
        for pg in range(-(-max(lens[b] - W, 0) // s.P)):
            pid = int(g2.block_table[b, pg])
            assert np.array_equal(g1.pool[pid, :64], g2.pool[pid, :64]), (b, pg)  # headers
    _records_match(s, (g1, g2), k, v, lens)
