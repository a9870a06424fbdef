"""GPU checks of the seed-only and tables-as-data contexts: records encoded
through them hold the oracle's codes (guard-band rule) for the oracle's
tables built from the test side's own Philox draws (seed only) or passed in
as data, and decode over their pages matches the oracle."""

import numpy as np
import pytest
import torch

import kv_cache_vector_tq_amd as tqa
from oracle import codebook as cbm
from oracle import codec, philox
from oracle import rotation as rot
import tq_inputs
from gpu_helpers import check_codes, check_signs, params_for, to_dev

pytestmark = pytest.mark.gpu


def _encode(ctx, x16, bits, qjl, kind):
    n = x16.shape[0]
    xt = to_dev(x16.view(np.uint16)).view(torch.float16)
    codes = torch.zeros((n, 16 * bits), dtype=torch.uint8, device="cuda")
    norms = torch.zeros(n, dtype=torch.float32, device="cuda")
    signs = torch.zeros((n, 16), dtype=torch.uint8, device="cuda") if qjl else None
    rnorms = torch.zeros(n, dtype=torch.float32, device="cuda") if qjl else None
    tqa.tq_encode(ctx, kind, xt, codes, norms, signs, rnorms)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.cpu().numpy()
    return cpu(codes), cpu(norms), cpu(signs), cpu(rnorms)


@pytest.mark.parametrize("rotation", ["dense", "hadamard"])
@pytest.mark.parametrize("how", ["seed", "tables"])
def test_seed_and_table_contexts_encode_like_the_oracle(rotation, how):
    print(f"case init {how} {rotation}", flush=True)
    seed, d, n = 11, 128, 3000
    rk = tqa.TQ_ROT_DENSE if rotation == "dense" else tqa.TQ_ROT_HADAMARD
    p = tqa.make_params(key_bits=3, key_qjl=1, value_bits=4, rotation=rk, seed=seed)
    rd = philox.rotation_draws(seed, d) if rotation == "dense" else philox.hadamard_draws(seed, d)
    R = rot.Rotation(rotation, rd, d)
    S = rot.qjl_matrix(philox.qjl_draws(seed, d), d)
    kcb, vcb = cbm.Codebook(3, d), cbm.Codebook(4, d)
    if how == "seed":
        ctx = tqa.Context(p)
    else:
        Rt = R.matrix if rotation == "dense" else rot.rademacher_signs(rd)
        ctx = tqa.Context(p, tables={"rotation": Rt, "qjl": S, "key_centroids": kcb.centroids,
                                     "value_centroids": vcb.centroids})
    x = tq_inputs.fp16(tq_inputs.keys(3, d, np.arange(n)))
    xv = tq_inputs.fp16(tq_inputs.values(3, d, n))
    x64, xv64 = x.astype(np.float64), xv.astype(np.float64)
    codes, norms, signs, rnorms = _encode(ctx, x, 3, True, tqa.TQ_KIND_KEY)
    ref = codec.encode(x64, R, kcb, S)
    assert np.array_equal(norms, ref.norms)
    gidx = codec.unpack_bits(codes, 3, d)
    check_codes(x64, gidx, ref.idx, R, kcb)
    check_signs(x64, gidx, norms, signs, R, kcb, S)
    vcodes, vnorms, _, _ = _encode(ctx, xv, 4, False, tqa.TQ_KIND_VALUE)
    vref = codec.encode(xv64, R, vcb)
    assert np.array_equal(vnorms, vref.norms)
    check_codes(xv64, codec.unpack_bits(vcodes, 4, d), vref.idx, R, vcb)


def test_tables_context_equals_draws_context():
    """A context built from the library's own host tables passed back as
    data encodes byte for byte like the context built from the draws."""
    print("case tables round trip", flush=True)
    seed, d, n = 2, 128, 2000
    p = tqa.make_params(key_bits=2, key_qjl=1, value_bits=3, seed=seed, qjl_kind=tqa.TQ_QJL_ORTHOGONAL)
    rd, qd = tq_inputs.rotation_draws(seed, d), tq_inputs.qjl_draws(seed, d)
    t = tqa.tq_host_tables(p, rd, qd)
    a = tqa.Context(p, rd, qd)
    b = tqa.Context(p, tables={"rotation": t["rotation"], "qjl": t["qjl"], "key_centroids": t["key_centroids"],
                               "value_centroids": t["value_centroids"]})
    x = tq_inputs.fp16(tq_inputs.keys(4, d, np.arange(n)))
    for kind, bits, qjl in ((tqa.TQ_KIND_KEY, 2, True), (tqa.TQ_KIND_VALUE, 3, False)):
        ra, rb = _encode(a, x, bits, qjl, kind), _encode(b, x, bits, qjl, kind)
        for u, v in zip(ra, rb):
            assert (u is None and v is None) or np.array_equal(u, v)
