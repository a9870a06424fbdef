"""GPU parity of tq_decode (dequantise flat records) against the oracle's
dequantiser applied to the same records, and a quality report of the
compressed cache against exact attention over the FP16 inputs.

Dequantise: out = Pi^T(n c[idx] + a ||r|| S^T(2 sigma - 1)) in float32 vs the
oracle in float64: within 2e-6 of each vector's norm (128-term fp32 sums).

Quality (reported, not gated beyond sanity): the pages print no value for
synthetic inputs, so these numbers are "parity unpinned"; they show what the
QJL variants do to attention at the config-0 shape (T=1024, keys 3-bit+QJL,
values 4-bit, dense rotation)."""

import math

import numpy as np
import pytest
import torch

import kv_cache_vector_tq_amd as tqa
from oracle import codec
import tq_inputs
from gpu_helpers import context_for, run_decode, upload_cache
from oracle_cache import Setup, fill

pytestmark = pytest.mark.gpu


def _records(ctx, kind, x16, qjl, bits, mixed=False):
    n = x16.shape[0]
    xt = torch.from_numpy(x16.astype(np.float32)).to(torch.float16).cuda()
    codes = torch.zeros((n, 16 * bits + (8 if mixed else 0)), dtype=torch.uint8, device="cuda")
    norms = torch.zeros(n, dtype=torch.float32, device="cuda")
    signs = torch.zeros((n, 16), dtype=torch.uint8, device="cuda") if qjl else None
    rnorms = torch.zeros(n, dtype=torch.float32, device="cuda") if qjl else None
    tqa.tq_encode(ctx, kind, xt, codes, norms, signs, rnorms)
    return codes, norms, signs, rnorms


@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("qjl_kind,shrink", [("gaussian", 1.0), ("orthogonal", 2 / math.pi)])
@pytest.mark.parametrize("n", [77, 1000])
def test_dequant_parity(rotation, qjl_kind, shrink, n):
    print(f"case dequant {rotation} {qjl_kind} n={n}", flush=True)
    s = Setup(key_bits=3, value_bits=4, rotation=rotation, qjl_kind=qjl_kind, qjl_shrink=shrink)
    ctx = context_for(s)
    x = tq_inputs.keys(2, 128, np.arange(n)).astype(np.float64)
    x[5] = 0.0
    x16 = tq_inputs.fp16(x)
    for kind, bits, cb, qjl in ((tqa.TQ_KIND_KEY, 3, s.kcb, True), (tqa.TQ_KIND_VALUE, 4, s.vcb, False)):
        codes, norms, signs, rnorms = _records(ctx, kind, x16, qjl, bits)
        out = torch.full((n, 128), float("nan"), dtype=torch.float32, device="cuda")
        tqa.tq_decode(ctx, kind, codes, norms, out, signs, rnorms)
        torch.cuda.synchronize()
        cpu = lambda t: None if t is None else t.cpu().numpy()
        ref = codec.dequantize(cpu(codes), cpu(norms), s.R, cb, cpu(signs), cpu(rnorms),
                               s.S if qjl else None, s.qjl_coef)
        got = cpu(out)
        scale = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
        assert np.all(np.max(np.abs(got - ref), axis=1) <= 2e-6 * scale + 1e-30)
        assert np.all(got[5] == 0.0)


def _quality(qjl_kind, shrink):
    """Compressed decode (tq_decode_attn) vs exact softmax attention over the
    FP16 keys and values, and key reconstruction error from tq_decode, at
    T=1024 (no window)."""
    s = Setup(Hq=4, Hkv=1, W=0, qjl_kind=qjl_kind, qjl_shrink=shrink)
    T = 1024
    cache = s.cache(1, T)
    k16, v16 = fill(s, cache, [T])
    ctx = context_for(s)
    dev = upload_cache(cache)
    q = tq_inputs.queries(7, (1, 4, 128))
    qt = torch.from_numpy(q.astype(np.float32)).cuda()
    out, logits = run_decode(ctx, qt, dev, 1 / math.sqrt(128), logits_len=T)
    K = k16[0, 0].astype(np.float64)
    V = v16[0, 0].astype(np.float64)
    ex_l = (q[0] @ K.T) / math.sqrt(128)
    w = np.exp(ex_l - ex_l.max(axis=1, keepdims=True))
    ex_o = (w / w.sum(axis=1, keepdims=True)) @ V
    lg = logits[0, :, :T]
    codes, norms, signs, rnorms = _records(ctx, tqa.TQ_KIND_KEY, k16[0, 0], True, 3)
    kh = torch.empty((T, 128), dtype=torch.float32, device="cuda")
    tqa.tq_decode(ctx, tqa.TQ_KIND_KEY, codes, norms, kh, signs, rnorms)
    kh = kh.cpu().numpy()
    return {
        "logit_rmse": float(np.sqrt(np.mean((lg - ex_l) ** 2))), "logit_std": float(ex_l.std()),
        "top1": float(np.mean(np.argmax(lg, axis=1) == np.argmax(ex_l, axis=1))),
        "top8": float(np.mean([len(set(np.argsort(-lg[g])[:8]) & set(np.argsort(-ex_l[g])[:8])) / 8
                               for g in range(4)])),
        "cosine": float(np.mean(np.sum(out[0] * ex_o, axis=1) /
                                (np.linalg.norm(out[0], axis=1) * np.linalg.norm(ex_o, axis=1)))),
        "key_rel_mse": float(np.mean(np.sum((kh - K) ** 2, axis=1) / np.sum(K ** 2, axis=1))),
    }


def test_quality_report():
    """Reported for the paper's Gaussian QJL, the orthogonal variant and the
    orthogonal variant with 2/pi shrinkage.  The only gate is the pages'
    qualitative claim ("The QJL detective story": same expectation, far lower
    variance): the orthogonal variants score keys with a smaller logit error
    than the Gaussian one."""
    res = {}
    for kind, shrink in (("gaussian", 1.0), ("orthogonal", 1.0), ("orthogonal", 2 / math.pi)):
        r = _quality(kind, shrink)
        res[(kind, shrink)] = r
        print(f"quality qjl={kind} shrink={shrink:.4f}: logit rmse {r['logit_rmse']:.4f} "
              f"(logit std {r['logit_std']:.3f}), top-1 {r['top1']:.2f}, top-8 overlap {r['top8']:.2f}, "
              f"output cosine {r['cosine']:.4f}, key rel. MSE {r['key_rel_mse']:.5f}", flush=True)
        assert all(np.isfinite(v) for v in r.values())
    g = res[("gaussian", 1.0)]["logit_rmse"]
    assert res[("orthogonal", 1.0)]["logit_rmse"] < g
    assert res[("orthogonal", 2 / math.pi)]["logit_rmse"] < g


@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("bits", [2, 3])
def test_dequant_parity_mixed(rotation, bits):
    """Mixed-channel records (bits + 1/2) dequantise like the oracle's."""
    print(f"case dequant mixed {rotation} bits={bits}+", flush=True)
    s = Setup(key_bits=bits, value_bits=bits, rotation=rotation, key_mixed=True, value_mixed=True)
    ctx = context_for(s)
    n = 300
    x = tq_inputs.keys(3, 128, np.arange(n)).astype(np.float64)
    x[5] = 0.0
    x16 = tq_inputs.fp16(x)
    for kind, cb, qjl in ((tqa.TQ_KIND_KEY, s.kcb, True), (tqa.TQ_KIND_VALUE, s.vcb, False)):
        codes, norms, signs, rnorms = _records(ctx, kind, x16, qjl, bits, mixed=True)
        out = torch.full((n, 128), float("nan"), dtype=torch.float32, device="cuda")
        tqa.tq_decode(ctx, kind, codes, norms, out, signs, rnorms)
        torch.cuda.synchronize()
        cpu = lambda t: None if t is None else t.cpu().numpy()
        ref = codec.dequantize(cpu(codes), cpu(norms), s.R, cb, cpu(signs), cpu(rnorms), s.S if qjl else None,
                               s.qjl_coef)
        got = cpu(out)
        scale = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
        assert np.all(np.max(np.abs(got - ref), axis=1) <= 2e-6 * scale + 1e-30)
        assert np.all(got[5] == 0.0)


@pytest.mark.parametrize("d", [96, 72])
@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
def test_dequant_parity_head_sizes(d, rotation):
    """Head sizes below the transform size: the records hold D = 128
    coordinates and the output rows the first d of Pi^T(...)."""
    print(f"case dequant d={d} {rotation}", flush=True)
    s = Setup(d=d, key_bits=3, value_bits=4, rotation=rotation)
    ctx = context_for(s)
    n = 200
    x = tq_inputs.keys(4, d, np.arange(n)).astype(np.float64)
    x[5] = 0.0
    x16 = tq_inputs.fp16(x)
    for kind, bits, cb, qjl in ((tqa.TQ_KIND_KEY, 3, s.kcb, True), (tqa.TQ_KIND_VALUE, 4, s.vcb, False)):
        codes, norms, signs, rnorms = _records(ctx, kind, x16, qjl, bits)
        out = torch.full((n, d + 1), float("nan"), dtype=torch.float32, device="cuda")
        tqa.tq_decode(ctx, kind, codes, norms, out, signs, rnorms)
        torch.cuda.synchronize()
        cpu = lambda t: None if t is None else t.cpu().numpy()
        ref = codec.dequantize(cpu(codes), cpu(norms), s.R, cb, cpu(signs), cpu(rnorms),
                               s.S if qjl else None, s.qjl_coef)
        assert ref.shape == (n, d)
        # n rows of d: the output ends at n * d floats (the rest stays untouched)
        flat = cpu(out).reshape(-1)
        got = flat[:n * d].reshape(n, d)
        assert np.all(np.isnan(flat[n * d:]))
        scale = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
        assert np.all(np.max(np.abs(got - ref), axis=1) <= 2e-6 * scale + 1e-30)
        assert np.all(got[5] == 0.0)
