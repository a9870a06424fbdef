"""GPU parity of tq_decode_attn on oracle-built pages (isolates the decode
arithmetic): logits per (b, q-head) within 1e-3 of max|logit|, and outputs
per (b, q-head) within 1e-3 relative (L2) and coordinate by coordinate within
1e-3 of max|o_j| of the oracle's plain dequantise-then-softmax attention.
Also: split-K partition invariance, repeat bit-identity under the
deterministic schedule (the default one within 1e-5), ragged and
degenerate lengths, GQA groupings, bf16/f16/f32 queries, bad pages, and the
launch shapes of the prep and merge kernels (one, two or four query heads
per work-group; split counts past each merge batch)."""

import numpy as np
import pytest
import torch

import kv_cache_vector_tq_amd as tqa
from oracle import attention as att
import tq_inputs
from gpu_helpers import ErrStats, assert_out_close, context_for, run_decode, upload_cache
from oracle_cache import Setup, fill

pytestmark = pytest.mark.gpu


def _check(cache, q, out, dbg, tol=1e-3, name="decode"):
    ref_o, ref_l = att.attention_plain(cache, q, 1 / np.sqrt(q.shape[-1]))
    B, Hq, _ = q.shape
    st = ErrStats(name)
    for b in range(B):
        T = int(cache.seq_lens[b])
        for g in range(Hq):
            if T == 0:
                assert np.all(out[b, g] == 0)
                continue
            if dbg is not None:
                l = ref_l[b][g]
                le = np.max(np.abs(dbg[b, g, :T] - l)) / np.max(np.abs(l))
                assert le <= tol, (b, g, le)
                st.add(logit=le)
            st.add(out=assert_out_close(out[b, g], ref_o[b, g], tol, (b, g)))
    st.report()
    return ref_o


CASES = [
    # name, setup kwargs, lens
    ("cfg0_T1024_W0", dict(Hq=1, Hkv=1, W=0), [1024]),
    ("cfg0_T1024_W128", dict(Hq=1, Hkv=1, W=128), [1024]),
    ("gqa4_ragged", dict(Hq=8, Hkv=2, W=128), [700, 129, 128, 40, 1, 0, 1000]),
    ("gqa8_2bit_hadamard", dict(Hq=8, Hkv=1, key_bits=2, value_bits=2, rotation="hadamard", W=128), [900, 300]),
    ("k4_noqjl_v3_P64", dict(Hq=2, Hkv=2, key_bits=4, key_qjl=0, value_bits=3, P=64, W=16), [333, 64, 17]),
    ("mha_k2_v4_W0_P32", dict(Hq=4, Hkv=4, key_bits=2, value_bits=4, P=32, W=0), [95, 32, 31]),
    ("gqa4_orthoS_shrink", dict(Hq=8, Hkv=2, W=64, qjl_kind="orthogonal", qjl_shrink=2 / np.pi), [600, 70, 1]),
    ("gqa8_orthoS_hadamard", dict(Hq=16, Hkv=2, key_bits=2, value_bits=2, rotation="hadamard", W=32,
                                  qjl_kind="orthogonal", qjl_shrink=0.7), [500, 33]),
    # head sizes below the transform size (zero-padded to D = 128); windows
    # past 128 slots take the merge kernel's second batch of window loads
    ("d96_gqa4_ragged", dict(d=96, Hq=8, Hkv=2, W=200), [700, 129, 201, 40, 1, 0, 1000]),
    ("d96_gqa1_hadamard_k2v2", dict(d=96, Hq=2, Hkv=2, key_bits=2, value_bits=2, rotation="hadamard", W=16,
                                    P=64), [333, 64, 17]),
    ("d72_gqa8_k4_noqjl_v3", dict(d=72, Hq=16, Hkv=2, key_bits=4, key_qjl=0, value_bits=3, W=64), [600, 70]),
    ("d112_gqa2_orthoS", dict(d=112, Hq=4, Hkv=2, W=32, P=32, qjl_kind="orthogonal", qjl_shrink=2 / np.pi),
     [300, 33]),
]

# mixed-channel rates (keys / values at 2.5 or 3.5 bits); matrix-core scan only
MIXED = [
    ("mixed_k35_v3_gqa4", dict(Hq=8, Hkv=2, key_bits=3, key_mixed=True, value_bits=3, W=64), [700, 129, 1]),
    ("mixed_k35_v4_wide", dict(Hq=8, Hkv=2, key_bits=3, key_mixed=True, value_bits=4, W=32), [600, 65]),
    ("mixed_k35_v35", dict(Hq=4, Hkv=4, key_bits=3, key_mixed=True, value_bits=3, value_mixed=True, W=16,
                           P=64), [333, 64, 17]),
    ("mixed_k25_v25_hadamard", dict(Hq=8, Hkv=1, key_bits=2, key_mixed=True, value_bits=2, value_mixed=True,
                                    rotation="hadamard", W=128), [900, 300]),
    ("mixed_k4_v35_noqjl", dict(Hq=2, Hkv=2, key_bits=4, key_qjl=0, value_bits=3, value_mixed=True, P=32, W=0),
     [95, 32, 31]),
    ("mixed_k3_v25_gqa8_orthoS", dict(Hq=16, Hkv=2, key_bits=3, value_bits=2, value_mixed=True, W=32,
                                      qjl_kind="orthogonal", qjl_shrink=2 / np.pi), [500, 33]),
    # u8 log-norm key norms (the design study's recommended first mode: keys 3.5 + u8 log-norm, values 3)
    ("u8norm_k35_v3_gqa4", dict(Hq=8, Hkv=2, key_bits=3, key_mixed=True, value_bits=3, W=64, key_norm_u8=True),
     [700, 129, 1]),
    ("u8norm_k3_v4_noqjl_gqa1", dict(Hq=2, Hkv=2, key_bits=3, key_qjl=0, value_bits=4, W=16, P=64,
                                     key_norm_u8=True), [300, 64]),
    ("u8norm_k2_v2_hadamard_gqa8", dict(Hq=16, Hkv=2, key_bits=2, value_bits=2, rotation="hadamard", W=32,
                                        key_norm_u8=True), [400, 33]),
    ("d96_u8norm_k35_v35", dict(d=96, Hq=8, Hkv=2, key_bits=3, key_mixed=True, value_bits=3, value_mixed=True,
                                W=64, key_norm_u8=True), [700, 129, 1]),
]


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
@pytest.mark.parametrize("name,kw,lens", CASES, ids=[c[0] for c in CASES])
def test_decode_parity_oracle_pages(name, kw, lens, kernel):
    _decode_parity(name, kw, lens, kernel)


@pytest.mark.parametrize("name,kw,lens", MIXED, ids=[c[0] for c in MIXED])
def test_decode_parity_mixed_rates(name, kw, lens):
    _decode_parity(name, kw, lens, "mfma")


def _decode_parity(name, kw, lens, kernel):
    print(f"case {name} {kernel}", flush=True)
    s = Setup(**kw)
    cache = s.cache(len(lens), max(lens))
    fill(s, cache, lens)
    ctx = context_for(s, tqa.TQ_FLAG_VALU_SCAN if kernel == "valu" else 0)
    dev = upload_cache(cache)
    q = tq_inputs.queries(5, (len(lens), s.Hq, s.d))
    qt = torch.from_numpy(q.astype(np.float32)).cuda()
    out, dbg = run_decode(ctx, qt, dev, 1 / np.sqrt(s.d), logits_len=max(lens) + 1)
    _check(cache, q.astype(np.float32).astype(np.float64), out, dbg, name=f"{name} {kernel}")
    assert tqa.tq_get_status(ctx) == 0


@pytest.mark.parametrize("d", [128, 96])
@pytest.mark.parametrize("qdtype", [torch.bfloat16, torch.float16])
def test_decode_query_dtypes(qdtype, d):
    s = Setup(d=d, Hq=4, Hkv=1, W=128)
    lens = [800]
    cache = s.cache(1, 800)
    fill(s, cache, lens)
    ctx = context_for(s)
    dev = upload_cache(cache)
    qt = torch.from_numpy(tq_inputs.queries(6, (1, 4, d)).astype(np.float32)).to(qdtype).cuda()
    out, dbg = run_decode(ctx, qt, dev, 1 / np.sqrt(d), logits_len=801)
    _check(cache, qt.float().cpu().numpy().astype(np.float64), out, dbg)


def _repeat_close(a, b, what=""):
    """Repeated calls of the default (balanced) schedule: the same result up
    to the grouping of the floating-point sums."""
    assert np.max(np.abs(a - b)) <= 1e-5 * np.max(np.abs(b)), what


@pytest.mark.parametrize("flags", [0, tqa.TQ_FLAG_DETERMINISTIC], ids=["balanced", "deterministic"])
def test_split_invariance_and_repeatability(flags):
    s = Setup(Hq=8, Hkv=2, W=128, P=64)
    lens = [2000, 1500]
    cache = s.cache(2, 2000)
    fill(s, cache, lens)
    ctx = context_for(s, flags)
    dev = upload_cache(cache)
    qt = torch.from_numpy(tq_inputs.queries(7, (2, 8, 128)).astype(np.float32)).cuda()
    outs = [run_decode(ctx, qt, dev, 1 / np.sqrt(128), pages_per_split=pps)[0] for pps in (0, 1, 3, 100)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-5 * np.max(np.abs(outs[0]))
    for _ in range(3):
        again = run_decode(ctx, qt, dev, 1 / np.sqrt(128), pages_per_split=3)[0]
        if flags & tqa.TQ_FLAG_DETERMINISTIC:
            assert np.array_equal(again, outs[2])
        else:
            _repeat_close(again, outs[2])


def test_ragged_batch_split_invariance():
    """One long sequence among short and empty ones (most work-groups of the
    long sequence's splits, the short ones' splits mostly empty): parity with
    the oracle at the automatic split, and with splits of 1 and 7 pages
    within 1e-5."""
    print("case ragged split invariance", flush=True)
    s = Setup(Hq=8, Hkv=2, W=16, P=32)
    lens = [4000] + [40] * 12 + [0, 17, 1]
    cache = s.cache(len(lens), max(lens))
    fill(s, cache, lens)
    ctx = context_for(s)
    dev = upload_cache(cache)
    q = tq_inputs.queries(8, (len(lens), s.Hq, 128))
    qt = torch.from_numpy(q.astype(np.float32)).cuda()
    out, dbg = run_decode(ctx, qt, dev, 1 / np.sqrt(128), logits_len=max(lens) + 1)
    _check(cache, q.astype(np.float32).astype(np.float64), out, dbg)
    for pps in (1, 7):
        o = run_decode(ctx, qt, dev, 1 / np.sqrt(128), pages_per_split=pps)[0]
        assert np.max(np.abs(o - out)) <= 1e-5 * np.max(np.abs(out)), pps
    again = run_decode(ctx, qt, dev, 1 / np.sqrt(128))[0]
    _repeat_close(again, out)
    ctx_d = context_for(s, tqa.TQ_FLAG_DETERMINISTIC)
    od = [run_decode(ctx_d, qt, dev, 1 / np.sqrt(128))[0] for _ in range(2)]
    assert np.array_equal(od[0], od[1])
    _repeat_close(od[0], out)
    assert tqa.tq_get_status(ctx) == 0


@pytest.mark.parametrize("Hq", [8, 16], ids=["G4_fused", "G8_finalize_kernel"])
def test_balanced_splits_many_sequences(Hq):
    """More sequences than one round of the split planner (270), ragged
    lengths from empty to a few pages, some inside the window only: parity
    with the oracle at the automatic (length-balanced) split, and with a
    fixed split of 2 pages within 1e-5."""
    print(f"case balanced splits many sequences Hq={Hq}", flush=True)
    s = Setup(Hq=Hq, Hkv=2, W=16, P=32)
    lens = [int(x) for x in np.random.default_rng(11).integers(0, 300, 270)]
    lens[5], lens[6] = 0, 16
    cache = s.cache(len(lens), max(lens))
    fill(s, cache, lens)
    ctx = context_for(s)
    dev = upload_cache(cache)
    q = tq_inputs.queries(9, (len(lens), s.Hq, 128))
    qt = torch.from_numpy(q.astype(np.float32)).cuda()
    out, dbg = run_decode(ctx, qt, dev, 1 / np.sqrt(128), logits_len=max(lens) + 1)
    _check(cache, q.astype(np.float32).astype(np.float64), out, dbg)
    o = run_decode(ctx, qt, dev, 1 / np.sqrt(128), pages_per_split=2)[0]
    assert np.max(np.abs(o - out)) <= 1e-5 * np.max(np.abs(out))
    assert tqa.tq_get_status(ctx) == 0


def test_bad_page_sets_status():
    s = Setup(Hq=2, Hkv=1, W=16, P=32)
    cache = s.cache(1, 200)
    fill(s, cache, [200])
    ctx = context_for(s)
    dev = upload_cache(cache)
    dev["block_table"][0, 1] = -1
    qt = torch.zeros((1, 2, 128), dtype=torch.float32, device="cuda")
    out, _ = run_decode(ctx, qt, dev, 1 / np.sqrt(128))
    assert np.all(np.isfinite(out))
    assert tqa.tq_get_status(ctx) & tqa.TQ_STATUS_BAD_PAGE
    assert tqa.tq_get_status(ctx) == 0


def test_workspace_too_small():
    s = Setup(Hq=2, Hkv=1)
    ctx = context_for(s)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    z = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(tqa.TQError) as e:
        tqa.tq_decode_attn(ctx, torch.zeros((1, 2, 128), device="cuda"), z, torch.zeros((1, 4), dtype=torch.int32,
                           device="cuda"), torch.zeros(1, dtype=torch.int32, device="cuda"),
                           torch.zeros((1, 1, 128, 128), dtype=torch.float16, device="cuda"),
                           torch.zeros((1, 1, 128, 128), dtype=torch.float16, device="cuda"),
                           torch.zeros((1, 2, 128), device="cuda"), ws, 0.1, num_pages=0)
    assert e.value.code == tqa.TQ_ERR_WORKSPACE


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_garbage_beyond_live_tokens(kernel):
    """Slots of a page past its live tokens hold NaN norms and all-ones key
    codes/signs: the result must still equal the oracle's (dead tokens are
    masked, never multiplied by zero)."""
    print(f"case garbage {kernel}", flush=True)
    s = Setup(Hq=8, Hkv=2, W=16, P=64)
    lens = [16 + 64 * 3 + 5, 16 + 31, 16 + 64]
    cache = s.cache(len(lens), max(lens))
    fill(s, cache, lens)
    pool = cache.pool.copy()
    lay = s.lay
    nan4 = np.frombuffer(np.float32(np.nan).tobytes(), np.uint8)
    for b, T in enumerate(lens):
        C = max(0, T - s.W)
        for j in range(-(-C // s.P)):
            live = min(s.P, C - j * s.P)
            page = pool[int(cache.block_table[b, j])]
            for h in range(s.Hkv):
                base = lay.head_base(h)
                for slot in range(live, s.P):
                    for off in (lay.k_norm, lay.k_rnorm, lay.v_norm):
                        page[base + off + 4 * slot: base + off + 4 * slot + 4] = nan4
                    kc = base + lay.k_codes + slot * (lay.d * lay.bK // 8)
                    page[kc: kc + lay.d * lay.bK // 8] = 0xFF
                    sg = base + lay.k_signs + slot * (lay.d // 8)
                    page[sg: sg + lay.d // 8] = 0xFF
    ctx = context_for(s, tqa.TQ_FLAG_VALU_SCAN if kernel == "valu" else 0)
    dev = upload_cache(cache)
    dev["pool"].copy_(torch.from_numpy(pool.reshape(-1)).cuda())
    q = tq_inputs.queries(9, (len(lens), s.Hq, 128))
    qt = torch.from_numpy(q.astype(np.float32)).cuda()
    out, dbg = run_decode(ctx, qt, dev, 1 / np.sqrt(128), logits_len=max(lens) + 1)
    _check(cache, q.astype(np.float32).astype(np.float64), out, dbg)
    assert tqa.tq_get_status(ctx) == 0


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_largest_page_and_window(kernel):
    """The largest page (P = 1024 tokens) and FP16 window (W = 1024) the
    library takes, with contexts shorter than, equal to and longer than the
    window and spanning two pages."""
    _decode_parity("P1024_W1024", dict(Hq=8, Hkv=2, P=1024, W=1024), [3100, 1024, 1025, 700], kernel)


def test_zero_size_calls_are_no_ops():
    """Empty batches, zero vectors and zero new tokens return OK and write nothing."""
    s = Setup(Hq=4, Hkv=2, W=16, P=32)
    ctx = context_for(s)
    cache = s.cache(2, 100)
    fill(s, cache, [100, 50])
    dev = upload_cache(cache)
    before = {k: v.clone() for k, v in dev.items() if isinstance(v, torch.Tensor)}
    empty16 = torch.zeros((0, 128), dtype=torch.float16, device="cuda")
    codes = torch.zeros((0, 48), dtype=torch.uint8, device="cuda")
    norms = torch.zeros(0, dtype=torch.float32, device="cuda")
    signs = torch.zeros((0, 16), dtype=torch.uint8, device="cuda")
    tqa.tq_encode(ctx, tqa.TQ_KIND_KEY, empty16, codes, norms, signs, norms)
    tqa.tq_decode(ctx, tqa.TQ_KIND_KEY, codes, norms, torch.zeros((0, 128), device="cuda"), signs, norms)
    kn = torch.zeros((2, 2, 0, 128), dtype=torch.float16, device="cuda")
    tqa.tq_append_page(ctx, dev["pool"], dev["block_table"], dev["seq_lens"], kn, kn.clone(), dev["k_win"],
                       dev["v_win"], num_pages=dev["num_pages"])
    kb0 = torch.zeros((0, 2, 1, 128), dtype=torch.float16, device="cuda")
    tqa.tq_append_page(ctx, dev["pool"], dev["block_table"][:0], dev["seq_lens"][:0], kb0, kb0.clone(),
                       dev["k_win"][:0], dev["v_win"][:0], num_pages=dev["num_pages"])
    q0 = torch.zeros((0, 4, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(tqa.tq_decode_workspace_bytes(ctx, 0, dev["block_table"].shape[1]), 1), dtype=torch.uint8,
                     device="cuda")
    tqa.tq_decode_attn(ctx, q0, dev["pool"], dev["block_table"][:0], dev["seq_lens"][:0], dev["k_win"][:0],
                       dev["v_win"][:0], torch.zeros((0, 4, 128), device="cuda"), ws, 1 / np.sqrt(128),
                       num_pages=dev["num_pages"])
    torch.cuda.synchronize()
    assert tqa.tq_get_status(ctx) == 0
    for k, v in before.items():
        assert torch.equal(dev[k], v), k


# Launch shapes of the prep and merge kernels: GW query heads per work-group
# (four, two or one; the library halves GW while B * H_kv * G / GW < 128) and
# split counts past the merge's first batch of partials (8 * 8 / GW splits
# for GW = 2 and 4, 16 * 8 for GW = 1) and past its second.
SHAPES = [
    # name, setup kwargs, lens, pages_per_split values (0 = automatic)
    ("GW2_B8_Hq32_Hkv8", dict(Hq=32, Hkv=8, W=16, P=32), [1300, 1100, 700, 1299, 40, 17, 1, 1000], (0, 1)),
    ("GW4_B64_Hq8_Hkv2", dict(Hq=8, Hkv=2, W=16, P=32), None, (0, 1)),
    ("GW1_B1_Hq2_Hkv1_5000", dict(Hq=2, Hkv=1, W=16, P=32), [5000], (0, 1, 2)),
    ("GW1_B1_Hq2_Hkv1_9000", dict(Hq=2, Hkv=1, W=16, P=32), [9000], (1,)),
]


@pytest.mark.parametrize("name,kw,lens,ppss", SHAPES, ids=[c[0] for c in SHAPES])
def test_prep_merge_launch_shapes(name, kw, lens, ppss):
    """Parity with the oracle at each split size, split invariance within
    1e-5 of max|o| and repeat bit-identity (deterministic schedule; the
    default one within 1e-5)."""
    print(f"case {name}", flush=True)
    s = Setup(**kw)
    if lens is None:
        lens = list(tq_inputs.ragged_lengths(11, 64, 1, 720))
    cache = s.cache(len(lens), max(lens))
    fill(s, cache, lens)
    ctx = context_for(s)
    ctx_d = context_for(s, tqa.TQ_FLAG_DETERMINISTIC)
    dev = upload_cache(cache)
    q = tq_inputs.queries(12, (len(lens), s.Hq, 128))
    qt = torch.from_numpy(q.astype(np.float32)).cuda()
    qh = q.astype(np.float32).astype(np.float64)
    outs = []
    for pps in ppss:
        out, dbg = run_decode(ctx, qt, dev, 1 / np.sqrt(128), pages_per_split=pps, logits_len=max(lens) + 1)
        _check(cache, qh, out, dbg, name=f"{name} pages_per_split={pps}")
        outs.append(out)
        again = run_decode(ctx, qt, dev, 1 / np.sqrt(128), pages_per_split=pps)[0]
        _repeat_close(again, out, pps)
        od = [run_decode(ctx_d, qt, dev, 1 / np.sqrt(128), pages_per_split=pps)[0] for _ in range(2)]
        assert np.array_equal(od[0], od[1]), pps
        _repeat_close(od[0], out, pps)
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-5 * np.max(np.abs(outs[0]))
    assert tqa.tq_get_status(ctx) == 0
