"""Parity at the full workload sizes, on sampled outputs.

Each test builds a cache of the real shape on the GPU with tq_append_page
(bulk prefill, then single-token decode appends), decodes with the automatic
split choice (the launch configuration the benchmark times) and checks a
sample against the oracle, which evaluates it one (sequence, KV head) at a
time from the GPU's own pages:
  * encode: codes and sign bits of sampled tokens under the guard-band rule,
    norms exactly, residual norms to 2e-5; the FP16 ring slots exactly;
  * decode: logits of the sampled heads within 1e-3 of max|logit| and their
    outputs within 1e-3 (L2) of the oracle's dequantise-then-softmax
    attention; the output without logit capture is the same up to the
    grouping of the sums (within 1e-5 of max|o|; bit-identical under the
    deterministic schedule, checked at the B=16 shape).
Shapes: B=16 Hq=32 Hkv=8 T=32K (3-bit+QJL keys, 4-bit values, dense);
B=1 Hq=64 Hkv=8 T=128K (2-bit+QJL, 2-bit, Hadamard, 4 decode steps);
one layer of 64 ragged sequences, lengths U[1K, 16K], Hq=16 Hkv=2;
and tq_encode of 4M vectors at 2/3/4 bits, dense and Hadamard."""

import numpy as np
import pytest
import torch

import kv_cache_vector_tq_amd as tqa
from oracle import attention as att
from oracle import codec, pages
import tq_inputs
from gpu_helpers import ErrStats, assert_out_close, check_codes, check_signs, context_for
from oracle_cache import Setup

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _same_sums(a, b):
    """Two decodes of the same inputs under the default schedule: equal up to
    the grouping of the floating-point sums."""
    a, b = a.cpu().numpy(), b.cpu().numpy()
    assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(b))


class GpuCache:
    """A cache of B sequences on the GPU, pages scattered over the pool."""

    def __init__(self, s, B, max_tokens, seed=1):
        self.s, self.B = s, B
        self.ctx = context_for(s)
        self.pb = tqa.tq_page_bytes(self.ctx.params)
        self.max_pages = max(1, -(-(max_tokens - s.W) // s.P))
        self.npages = B * self.max_pages
        self.pool = torch.zeros(self.npages * self.pb, dtype=torch.uint8, device="cuda")
        perm = np.random.default_rng(seed).permutation(self.npages).astype(np.int32)
        self.bt = torch.from_numpy(perm.reshape(B, self.max_pages)).cuda()
        self.sl = torch.zeros(B, dtype=torch.int32, device="cuda")
        self.kw = torch.zeros((B, s.Hkv, max(s.W, 1), s.d), dtype=torch.float16, device="cuda")
        self.vw = torch.zeros_like(self.kw)

    def append(self, k, v, counts=None):
        c = None if counts is None else torch.as_tensor(np.asarray(counts, np.int32)).cuda()
        tqa.tq_append_page(self.ctx, self.pool, self.bt, self.sl, k.contiguous(), v.contiguous(), self.kw, self.vw,
                           c, num_pages=self.npages)

    def decode(self, q, dbg_len=None, ctx=None):
        ws = torch.empty(tqa.tq_decode_workspace_bytes(self.ctx, self.B, self.max_pages, 0), dtype=torch.uint8,
                         device="cuda")
        out = torch.full((self.B, q.shape[1], self.s.d), float("nan"), dtype=torch.float32, device="cuda")
        dbg = None
        if dbg_len is not None:
            dbg = torch.full((self.B, q.shape[1], dbg_len), float("nan"), dtype=torch.float32, device="cuda")
        tqa.tq_decode_attn(ctx or self.ctx, q, self.pool, self.bt, self.sl, self.kw, self.vw, out, ws,
                           1 / np.sqrt(self.s.d), dbg_logits=dbg, num_pages=self.npages)
        torch.cuda.synchronize()
        return out, dbg

    def host(self):
        s = self.s
        c = pages.PagedCache(s.lay, s.R, s.kcb, s.vcb, s.S, s.W, num_pages=1, batch=1, max_pages=1,
                             rotation_kind=0 if s.rotation == "dense" else 1, seed=s.seed, qjl_coef=s.qjl_coef)
        c.pool = self.pool.cpu().numpy().reshape(self.npages, self.pb)
        c.block_table = self.bt.cpu().numpy()
        c.seq_lens = self.sl.cpu().numpy()
        c.k_win = self.kw.cpu().numpy()
        c.v_win = self.vw.cpu().numpy()
        return c


def check_records(s, cache, k, v, pairs, rng, nsamp=384, extra=()):
    """Sampled compressed tokens of each (b, h) in `pairs` hold the oracle's
    records for the FP16 source vectors k[b, h, pos], v[b, h, pos]."""
    for b, h in pairs:
        C = max(int(cache.seq_lens[b]) - s.W, 0)
        if C == 0:
            continue
        kr, vn, vidx = cache.compressed(b, h)
        pos = np.unique(np.concatenate([rng.integers(0, C, nsamp), [0, C - 1],
                                        [p for p in extra if 0 <= p < C]]).astype(np.int64))
        pt = torch.from_numpy(pos).cuda()
        x = k[b, h].index_select(0, pt).float().cpu().numpy().astype(np.float64)
        xv = v[b, h].index_select(0, pt).float().cpu().numpy().astype(np.float64)
        ref = codec.encode(x, s.R, s.kcb, s.S if s.qjl else None)
        assert np.array_equal(kr.norms[pos], ref.norms), (b, h)
        gidx = codec.unpack_bits(kr.codes[pos], s.bK, s.d)
        check_codes(x, gidx, ref.idx, s.R, s.kcb)
        if s.qjl:
            check_signs(x, gidx, kr.norms[pos], kr.signs[pos], s.R, s.kcb, s.S)
            r = codec.residual_from_codes(x, s.R, s.kcb, kr.norms[pos].astype(np.float64), gidx)
            assert np.allclose(kr.rnorms[pos], np.linalg.norm(r, axis=1), rtol=2e-5, atol=1e-30)
        vref = codec.encode(xv, s.R, s.vcb)
        assert np.array_equal(vn[pos], vref.norms), (b, h)
        check_codes(xv, vidx[pos], vref.idx, s.R, s.vcb)


def check_window(s, cache, k, v, pairs):
    for b, h in pairs:
        T = int(cache.seq_lens[b])
        p = np.arange(max(T - s.W, 0), T)
        pt = torch.from_numpy(p).cuda()
        assert np.array_equal(cache.k_win[b, h, p % s.W].view(np.uint16),
                              k[b, h].index_select(0, pt).cpu().numpy().view(np.uint16))
        assert np.array_equal(cache.v_win[b, h, p % s.W].view(np.uint16),
                              v[b, h].index_select(0, pt).cpu().numpy().view(np.uint16))


def check_decode(s, cache, q, out, dbg, pairs, name="decode"):
    """Every query head of the sampled (b, kv head) pairs: logits within 1e-3
    of max|logit| (when captured), outputs within 1e-3 (L2 and per coordinate)."""
    qh = q.float().cpu().numpy().astype(np.float64)
    ref_o, ref_l = att.attention_plain(cache, qh, 1 / np.sqrt(s.d), pairs=pairs)
    out = out.cpu().numpy()
    dbg = None if dbg is None else dbg.cpu().numpy()
    G = s.Hq // s.Hkv
    st = ErrStats(name)
    for b, h in pairs:
        T = int(cache.seq_lens[b])
        for g in range(h * G, (h + 1) * G):
            if dbg is not None:
                l = ref_l[b][g]
                le = np.max(np.abs(dbg[b, g, :T] - l)) / np.max(np.abs(l))
                assert le <= 1e-3, (b, g, le)
                st.add(logit=le)
            st.add(out=assert_out_close(out[b, g], ref_o[b, g], 1e-3, (b, g)))
    st.report()


def test_decode_step_B16_Hq32_Hkv8_T32K():
    print("case B16 Hq32 Hkv8 T32K", flush=True)
    B, Hq, Hkv, T = 16, 32, 8, 32768
    s = Setup(Hq=Hq, Hkv=Hkv, key_bits=3, key_qjl=1, value_bits=4, P=256, W=128)
    gc = GpuCache(s, B, T)
    k, v = tq_inputs.torch_kv(0, B, Hkv, T, s.d, "cuda")
    gc.append(k[:, :, :T - 2], v[:, :, :T - 2])          # bulk prefill
    for t in (T - 2, T - 1):                             # two decode-step appends
        gc.append(k[:, :, t:t + 1], v[:, :, t:t + 1])
    q = tq_inputs.torch_queries(0, (B, Hq, s.d), "cuda", torch.bfloat16)
    out, _ = gc.decode(q)
    out2, dbg = gc.decode(q, dbg_len=T)
    _same_sums(out, out2)
    ctx_d = context_for(s, tqa.TQ_FLAG_DETERMINISTIC)
    od = [gc.decode(q, ctx=ctx_d)[0] for _ in range(2)]
    assert torch.equal(od[0], od[1])
    _same_sums(od[0], out)
    assert tqa.tq_get_status(gc.ctx) == 0
    cache = gc.host()
    assert np.all(cache.seq_lens == T)
    # 16 (sequence, KV head) pairs: every sequence once, every KV head twice
    pairs = [(b, (3 * b) % Hkv) for b in range(B)]
    assert len(set(h for _, h in pairs)) == Hkv
    rng = np.random.default_rng(5)
    check_records(s, cache, k, v, pairs[::4], rng, extra=(T - s.W - 2, T - s.W - 1))
    check_window(s, cache, k, v, pairs)
    check_decode(s, cache, q, out, dbg, pairs, "B16 T32K")


def test_long_context_B1_Hq64_T128K_hadamard_2bit():
    print("case B1 Hq64 Hkv8 T128K", flush=True)
    B, Hq, Hkv, T, steps = 1, 64, 8, 131072, 4
    s = Setup(Hq=Hq, Hkv=Hkv, key_bits=2, key_qjl=1, value_bits=2, rotation="hadamard", P=256, W=128)
    gc = GpuCache(s, B, T)
    k, v = tq_inputs.torch_kv(3, B, Hkv, T, s.d, "cuda")
    T0 = T - steps
    gc.append(k[:, :, :T0], v[:, :, :T0])
    for i in range(steps):
        t = T0 + i
        gc.append(k[:, :, t:t + 1], v[:, :, t:t + 1])
        q = tq_inputs.torch_queries(3, (B, Hq, s.d), "cuda", torch.bfloat16, step=i)
        out, _ = gc.decode(q)
    out2, dbg = gc.decode(q, dbg_len=T)
    _same_sums(out, out2)
    assert tqa.tq_get_status(gc.ctx) == 0
    cache = gc.host()
    pairs = [(0, h) for h in range(Hkv)]
    check_records(s, cache, k, v, pairs[::3], np.random.default_rng(6), extra=range(T0 - s.W, T - s.W))
    check_window(s, cache, k, v, pairs)
    check_decode(s, cache, q, out, dbg, pairs, "B1 T128K")


def test_ragged_layer_B64_Hq16_Hkv2():
    print("case ragged B64 Hq16 Hkv2", flush=True)
    B, Hq, Hkv = 64, 16, 2
    lens = tq_inputs.ragged_lengths(0, B, 1024, 16384).astype(np.int64)
    Tm = int(lens.max())
    s = Setup(Hq=Hq, Hkv=Hkv, key_bits=3, key_qjl=1, value_bits=4, P=256, W=128)
    gc = GpuCache(s, B, Tm)
    k, v = tq_inputs.torch_kv(4, B, Hkv, Tm, s.d, "cuda")
    gc.append(k[:, :, :Tm - 1], v[:, :, :Tm - 1], counts=lens - 1)   # ragged prefill
    # one decode-step append: token lens[b] - 1 of each sequence
    idx = torch.from_numpy(lens - 1).cuda().view(B, 1, 1, 1).expand(B, Hkv, 1, s.d)
    gc.append(torch.gather(k, 2, idx), torch.gather(v, 2, idx))
    q = tq_inputs.torch_queries(4, (B, Hq, s.d), "cuda", torch.bfloat16)
    out, _ = gc.decode(q)
    out2, dbg = gc.decode(q, dbg_len=Tm)
    _same_sums(out, out2)
    assert tqa.tq_get_status(gc.ctx) == 0
    cache = gc.host()
    assert np.array_equal(cache.seq_lens, lens)
    # 16 pairs spread over the length distribution, both KV heads
    order = np.argsort(lens)
    pairs = [(int(order[i]), i % Hkv) for i in np.linspace(0, B - 1, 16).astype(int)]
    check_records(s, cache, k, v, pairs[::4], np.random.default_rng(7))
    check_window(s, cache, k, v, pairs)
    check_decode(s, cache, q, out, dbg, pairs, "ragged B64")


@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
def test_encode_4M_vectors(rotation):
    print(f"case encode 4M {rotation}", flush=True)
    n = 4 * 1024 * 1024
    k, v = tq_inputs.torch_kv(5, 4096, 1, 1024, 128, "cuda")
    k = k.view(n, 128)
    v = v.view(n, 128)
    rng = np.random.default_rng(8)
    sel = np.unique(np.concatenate([rng.integers(0, n, 2048), [0, n - 1]]))
    st = torch.from_numpy(sel).cuda()
    x = k.index_select(0, st).float().cpu().numpy().astype(np.float64)
    xv = v.index_select(0, st).float().cpu().numpy().astype(np.float64)
    for bits in (2, 3, 4):
        s = Setup(key_bits=bits, value_bits=bits, rotation=rotation)
        ctx = context_for(s)
        codes = torch.empty((n, 16 * bits), dtype=torch.uint8, device="cuda")
        norms = torch.empty(n, dtype=torch.float32, device="cuda")
        signs = torch.empty((n, 16), dtype=torch.uint8, device="cuda")
        rnorms = torch.empty(n, dtype=torch.float32, device="cuda")
        tqa.tq_encode(ctx, tqa.TQ_KIND_KEY, k, codes, norms, signs, rnorms)
        g = lambda t: t.index_select(0, st).cpu().numpy()
        gc, gn, gs, gr = g(codes), g(norms), g(signs), g(rnorms)
        ref = codec.encode(x, s.R, s.kcb, s.S)
        assert np.array_equal(gn, ref.norms)
        gidx = codec.unpack_bits(gc, bits, 128)
        assert check_codes(x, gidx, ref.idx, s.R, s.kcb) <= 0.002 * x.size
        check_signs(x, gidx, gn, gs, s.R, s.kcb, s.S)
        r = codec.residual_from_codes(x, s.R, s.kcb, gn.astype(np.float64), gidx)
        assert np.allclose(gr, np.linalg.norm(r, axis=1), rtol=2e-5, atol=1e-30)
        tqa.tq_encode(ctx, tqa.TQ_KIND_VALUE, v, codes, norms)
        vref = codec.encode(xv, s.R, s.vcb)
        assert np.array_equal(g(norms), vref.norms)
        check_codes(xv, codec.unpack_bits(g(codes), bits, 128), vref.idx, s.R, s.vcb)
    torch.cuda.synchronize()


def test_streaming_layers_B64_Hq16_Hkv2():
    """Full-model streaming at the 36-layer workload's shape, cut to 3 layers
    and 16 steps: every layer (its own cache and K/V draws) is prefilled with
    a ragged batch (64 sequences, lengths U[1K, 16K]), then each step appends
    one token per sequence to every layer and decodes every layer.  Checked
    at the end: lengths and rings exactly, the records of the tokens the steps
    evicted into pages (and a sample of the prefill's) under the guard-band
    rule, and the decode outputs of steps 0, 7 and 15 for 4 (sequence, KV
    head) pairs per layer against the oracle over the cache as it stood at
    that step (the pages are append-only; the ring of step i is refilled from
    the FP16 sources)."""
    print("case streaming 3 layers x 16 steps, B64 Hq16 Hkv2", flush=True)
    B, Hq, Hkv, nl, steps = 64, 16, 2, 3, 16
    lens = tq_inputs.ragged_lengths(0, B, 1024, 16384).astype(np.int64)
    Tm = int(lens.max())
    s = Setup(Hq=Hq, Hkv=Hkv, key_bits=3, key_qjl=1, value_bits=4, P=256, W=128)
    order = np.argsort(lens)
    pairs = [(int(order[i]), i % Hkv) for i in (0, B // 3, 2 * B // 3, B - 1)]
    checked_steps = (0, 7, steps - 1)
    layers = []
    for li in range(nl):
        gc = GpuCache(s, B, Tm + steps, seed=10 + li)
        k, v = tq_inputs.torch_kv(20 + li, B, Hkv, Tm + steps, s.d, "cuda", layer=li)
        gc.append(k[:, :, :Tm], v[:, :, :Tm], counts=lens)
        layers.append(dict(gc=gc, k=k, v=v, outs={}))
    torch.cuda.synchronize()
    for i in range(steps):
        idx = torch.from_numpy(lens + i).cuda().view(B, 1, 1, 1).expand(B, Hkv, 1, s.d)
        for li, L in enumerate(layers):
            L["gc"].append(torch.gather(L["k"], 2, idx), torch.gather(L["v"], 2, idx))
            q = tq_inputs.torch_queries(30 + li, (B, Hq, s.d), "cuda", torch.bfloat16, step=i)
            out, _ = L["gc"].decode(q)
            if i in checked_steps:
                L["outs"][i] = (q, out)
    for li, L in enumerate(layers):
        gc = L["gc"]
        assert tqa.tq_get_status(gc.ctx) == 0
        cache = gc.host()
        assert np.array_equal(cache.seq_lens, lens + steps), li
        k, v = L["k"], L["v"]
        check_window(s, cache, k, v, pairs)
        # the tokens evicted during the steps, and a sample of the prefill
        for b, h in pairs:
            ev = range(int(lens[b]) - s.W, int(lens[b]) + steps - s.W)
            check_records(s, cache, k, v, [(b, h)], np.random.default_rng(40 + li), nsamp=64, extra=ev)
        for i in checked_steps:
            q, out = L["outs"][i]
            c = gc.host()
            c.seq_lens = lens + i + 1
            for b, h in pairs:  # the ring as it stood after step i
                p = np.arange(int(c.seq_lens[b]) - s.W, int(c.seq_lens[b]))
                pt = torch.from_numpy(p).cuda()
                c.k_win[b, h, p % s.W] = k[b, h].index_select(0, pt).cpu().numpy()
                c.v_win[b, h, p % s.W] = v[b, h].index_select(0, pt).cpu().numpy()
            check_decode(s, c, q, out, None, pairs, f"layer {li} step {i}")
