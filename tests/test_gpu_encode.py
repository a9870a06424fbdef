"""GPU parity of tq_encode against the oracle (codes and sign bits under the
guard-band rule in gpu_helpers, norms to float32, residual norms to 1e-5)."""

import numpy as np
import pytest
import torch

import kv_cache_vector_tq_amd as tqa
from oracle import codec
import tq_inputs
from gpu_helpers import check_codes, check_signs, context_for
from oracle_cache import Setup

pytestmark = pytest.mark.gpu


def _inputs(n, seed=0):
    x = tq_inputs.keys(seed, 128, np.arange(n)).astype(np.float64)
    x[3] = 0.0                      # zero vector
    x[5] = 1e-3 * x[5]              # tiny
    x[7, :] = 0.0
    x[7, 11] = -2.5                 # one-hot
    return tq_inputs.fp16(x)


def _gpu_encode(ctx, kind, x16, qjl, dtype=torch.float16):
    n = x16.shape[0]
    key = kind == tqa.TQ_KIND_KEY
    bits = ctx.params.key_bits if key else ctx.params.value_bits
    mixed = ctx.params.key_mixed if key else ctx.params.value_mixed
    xt = torch.from_numpy(x16.astype(np.float32)).to(dtype).cuda()
    codes = torch.zeros((n, 16 * bits + (8 if mixed else 0)), dtype=torch.uint8, device="cuda")
    norms = torch.zeros(n, dtype=torch.float32, device="cuda")
    signs = torch.zeros((n, 16), dtype=torch.uint8, device="cuda") if qjl else None
    rnorms = torch.zeros(n, dtype=torch.float32, device="cuda") if qjl else None
    tqa.tq_encode(ctx, kind, xt, codes, norms, signs, rnorms)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    return cpu(codes), cpu(norms), cpu(signs), cpu(rnorms)


@pytest.mark.parametrize("qjl_kind", ["gaussian", "orthogonal"])
@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("bK,bV", [(3, 4), (2, 2), (4, 3)])
@pytest.mark.parametrize("n", [1024, 77])
def test_encode_parity(rotation, bK, bV, n, qjl_kind):
    s = Setup(key_bits=bK, value_bits=bV, rotation=rotation, qjl_kind=qjl_kind)
    ctx = context_for(s)
    x16 = _inputs(n)
    x = x16.astype(np.float64)
    print(f"case rotation={rotation} bK={bK} bV={bV} n={n} qjl={qjl_kind}", flush=True)
    # keys with QJL
    codes, norms, signs, rnorms = _gpu_encode(ctx, tqa.TQ_KIND_KEY, x16, True)
    ref = codec.encode(x, s.R, s.kcb, s.S)
    assert np.array_equal(norms, ref.norms)
    gidx = codec.unpack_bits(codes, bK, 128)
    nband = check_codes(x, gidx, ref.idx, s.R, s.kcb)
    check_signs(x, gidx, norms, signs, s.R, s.kcb, s.S)
    r = codec.residual_from_codes(x, s.R, s.kcb, norms, gidx)
    assert np.allclose(rnorms, np.linalg.norm(r, axis=1), rtol=1e-5, atol=1e-30)
    assert nband <= 0.002 * x.size
    # zero vector
    assert norms[3] == 0 and rnorms[3] == 0 and not codes[3].any() and not signs[3].any()
    # values
    vcodes, vnorms, _, _ = _gpu_encode(ctx, tqa.TQ_KIND_VALUE, x16, False)
    vref = codec.encode(x, s.R, s.vcb)
    assert np.array_equal(vnorms, vref.norms)
    check_codes(x, codec.unpack_bits(vcodes, bV, 128), vref.idx, s.R, s.vcb)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_encode_other_dtypes(dtype):
    s = Setup()
    ctx = context_for(s)
    x16 = _inputs(300, seed=4)
    xin = torch.from_numpy(x16.astype(np.float32)).to(dtype)
    x = xin.float().numpy().astype(np.float64)  # exactly what the library reads
    codes, norms, signs, rnorms = _gpu_encode(ctx, tqa.TQ_KIND_KEY, x.astype(np.float32), True, dtype)
    ref = codec.encode(x, s.R, s.kcb, s.S)
    assert np.array_equal(norms, ref.norms)
    gidx = codec.unpack_bits(codes, 3, 128)
    check_codes(x, gidx, ref.idx, s.R, s.kcb)
    check_signs(x, gidx, norms, signs, s.R, s.kcb, s.S)


def test_encode_repeatable():
    s = Setup()
    ctx = context_for(s)
    x16 = _inputs(500, seed=9)
    a = _gpu_encode(ctx, tqa.TQ_KIND_KEY, x16, True)
    b = _gpu_encode(ctx, tqa.TQ_KIND_KEY, x16, True)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("bK,kmix,bV,vmix", [(3, 1, 3, 1), (2, 1, 2, 1), (3, 1, 4, 0), (4, 0, 2, 1)])
@pytest.mark.parametrize("n", [1024, 77])
def test_encode_parity_mixed(rotation, bK, kmix, bV, vmix, n):
    """Mixed-channel rates (2.5 / 3.5 bits): records as the oracle packs them
    (low-rate half first), codes and signs under the guard-band rule."""
    s = Setup(key_bits=bK, value_bits=bV, rotation=rotation, key_mixed=kmix, value_mixed=vmix)
    ctx = context_for(s)
    x16 = _inputs(n, seed=2)
    x = x16.astype(np.float64)
    print(f"case mixed rotation={rotation} bK={bK}{'+' if kmix else ''} bV={bV}{'+' if vmix else ''} n={n}", flush=True)
    codes, norms, signs, rnorms = _gpu_encode(ctx, tqa.TQ_KIND_KEY, x16, True)
    ref = codec.encode(x, s.R, s.kcb, s.S)
    assert codes.shape[1] == s.kcb.record_bytes(128)
    assert np.array_equal(norms, ref.norms)
    gidx = s.kcb.unpack(codes, 128)
    nband = check_codes(x, gidx, ref.idx, s.R, s.kcb)
    check_signs(x, gidx, norms, signs, s.R, s.kcb, s.S)
    r = codec.residual_from_codes(x, s.R, s.kcb, norms, gidx)
    assert np.allclose(rnorms, np.linalg.norm(r, axis=1), rtol=1e-5, atol=1e-30)
    assert nband <= 0.002 * x.size
    assert np.array_equal(codes[~np.any(gidx != ref.idx, axis=1)], ref.codes[~np.any(gidx != ref.idx, axis=1)])
    vcodes, vnorms, _, _ = _gpu_encode(ctx, tqa.TQ_KIND_VALUE, x16, False)
    vref = codec.encode(x, s.R, s.vcb)
    assert vcodes.shape[1] == s.vcb.record_bytes(128)
    assert np.array_equal(vnorms, vref.norms)
    check_codes(x, s.vcb.unpack(vcodes, 128), vref.idx, s.R, s.vcb)


@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("bK,kmix,qjl", [(3, 0, True), (3, 1, True), (4, 0, False)])
@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_encode_parity_u8_key_norm(rotation, bK, kmix, qjl, dtype):
    """u8 log-norm key norms: the record's norm is the level of the oracle's
    code (exactly, as float32), codes and signs under the guard-band rule with
    the residual against that level; values keep float32 norms."""
    print(f"case u8 key norm rotation={rotation} bK={bK}{'+' if kmix else ''} qjl={qjl} {dtype}", flush=True)
    s = Setup(key_bits=bK, key_qjl=int(qjl), value_bits=3, rotation=rotation, key_mixed=bool(kmix),
              key_norm_u8=True)
    ctx = context_for(s)
    x16 = _inputs(700, seed=4)
    x16[11] = 0
    x = x16.astype(np.float64)
    codes, norms, signs, rnorms = _gpu_encode(ctx, tqa.TQ_KIND_KEY, x16, qjl, dtype)
    ref = codec.encode(x, s.R, s.kcb, s.S if qjl else None, norm_u8=True)
    assert np.array_equal(norms, ref.norms)
    assert norms[11] == 0
    gidx = s.kcb.unpack(codes, 128)
    nband = check_codes(x, gidx, ref.idx, s.R, s.kcb)
    assert nband <= 0.002 * x.size
    if qjl:
        check_signs(x, gidx, norms, signs, s.R, s.kcb, s.S)
        r = codec.residual_from_codes(x, s.R, s.kcb, norms, gidx)
        assert np.allclose(rnorms, np.linalg.norm(r, axis=1), rtol=1e-5, atol=1e-30)
    vcodes, vnorms, _, _ = _gpu_encode(ctx, tqa.TQ_KIND_VALUE, x16, False, dtype)
    vref = codec.encode(x, s.R, s.vcb)
    assert np.array_equal(vnorms, vref.norms)


@pytest.mark.parametrize("d", [96, 72, 120])
@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("dtype", [torch.float16, torch.float32])
def test_encode_parity_head_sizes(d, rotation, dtype):
    """Head sizes below the transform size D = 128: rows of d coordinates
    (here inside wider rows, row_stride = d + 8) are zero-padded to D; the
    records hold D codes and D sign bits.  fp16 rows take the matrix-core
    encoder, f32 rows the vector-ALU one."""
    print(f"case head size d={d} rotation={rotation} dtype={dtype}", flush=True)
    s = Setup(d=d, rotation=rotation)
    ctx = context_for(s)
    n = 300
    x = tq_inputs.keys(6, d, np.arange(n)).astype(np.float64)
    x[3] = 0.0
    x[7, :] = 0.0
    x[7, d - 1] = 1.5
    x16 = tq_inputs.fp16(x)
    wide = np.zeros((n, d + 8), np.float32)
    wide[:, :d] = x16.astype(np.float32)
    wide[:, d:] = 1e4  # past the row: must not be read
    xt = torch.from_numpy(wide).to(dtype).cuda()[:, :d]
    x = x16.astype(np.float64)
    for kind, cb, qjl in ((tqa.TQ_KIND_KEY, s.kcb, True), (tqa.TQ_KIND_VALUE, s.vcb, False)):
        codes = torch.zeros((n, cb.record_bytes(128)), dtype=torch.uint8, device="cuda")
        norms = torch.zeros(n, dtype=torch.float32, device="cuda")
        signs = torch.zeros((n, 16), dtype=torch.uint8, device="cuda") if qjl else None
        rnorms = torch.zeros(n, dtype=torch.float32, device="cuda") if qjl else None
        tqa.tq_encode(ctx, kind, xt, codes, norms, signs, rnorms)
        torch.cuda.synchronize()
        codes, norms = codes.cpu().numpy(), norms.cpu().numpy()
        ref = codec.encode(x, s.R, cb, s.S if qjl else None)
        assert np.array_equal(norms, ref.norms)
        gidx = cb.unpack(codes, 128)
        assert check_codes(x, gidx, ref.idx, s.R, cb) <= 0.002 * n * 128
        if qjl:
            signs, rnorms = signs.cpu().numpy(), rnorms.cpu().numpy()
            check_signs(x, gidx, norms, signs, s.R, cb, s.S)
            r = codec.residual_from_codes(x, s.R, cb, norms, gidx)
            assert np.allclose(rnorms, np.linalg.norm(r, axis=1), rtol=1e-5, atol=1e-30)
            assert rnorms[3] == 0 and not signs[3].any()
        assert norms[3] == 0 and not codes[3].any()
