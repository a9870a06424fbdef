"""Helpers for the GPU parity tests: library contexts built from the same
seeded draws as the oracle, and the comparison rules.

Bit-exact rule for codes and sign bits.  The oracle decides each code from
float64 y = Pi x / n rounded to float32; the GPU computes y in float32.  The
two can straddle a decision boundary only when y is within the float32
arithmetic error of it: the dot product of a float32 row of Pi with x/n is
off by at most gamma_128 * sum|Pi_ij x_j|/n <= 128 * 2^-24 * 1 ~ 2^-17.  So a
code must match exactly wherever y lies more than 2^-16 from every boundary
(unit-vector units), and may differ by one level inside that band.  Sign bits
are checked against the oracle recomputed from the GPU's own codes and norms,
exactly wherever |(S r)_j| > 2^-16 * sqrt(D) * ||r|| (D = 128 transform
coordinates, also for head sizes below 128, which are zero-padded to D).
"""

import numpy as np
import torch

import kv_cache_vector_tq_amd as tqa
from oracle import codec

BAND = 2.0 ** -16


def params_for(setup, flags=0):
    return tqa.make_params(flags=flags,
        head_dim=setup.d, key_bits=setup.bK, key_qjl=setup.qjl, value_bits=setup.bV,
        rotation=tqa.TQ_ROT_DENSE if setup.rotation == "dense" else tqa.TQ_ROT_HADAMARD,
        num_q_heads=setup.Hq, num_kv_heads=setup.Hkv, page_tokens=setup.P, window=setup.W, seed=setup.seed,
        qjl_kind=tqa.TQ_QJL_ORTHOGONAL if setup.qjl_kind == "orthogonal" else tqa.TQ_QJL_GAUSSIAN,
        qjl_shrink=setup.qjl_shrink, key_mixed=int(setup.kmix), value_mixed=int(setup.vmix),
        key_norm_u8=int(getattr(setup, "kn8", False)))


def context_for(setup, flags=0):
    return tqa.Context(params_for(setup, flags), setup.rot_draws, setup.qjl_draws if setup.qjl else None)


def code_band(x, R, cb):
    """Boolean [n, d]: oracle's float32 y within BAND of a decision boundary."""
    x = np.asarray(x, dtype=np.float64)
    n = np.linalg.norm(x, axis=1)
    y = R.forward(x / np.where(n > 0, n, 1.0)[:, None]).astype(np.float32).astype(np.float64)
    near = lambda bnd: np.min(np.abs(y[..., None] - bnd[None, None, :]), axis=-1)
    if getattr(cb, "mixed", False):  # each half against its own codebook
        dist = np.where(cb.hi_mask, near(cb.hi.boundaries), near(cb.lo.boundaries))
    else:
        dist = near(cb.boundaries)
    return (dist < BAND) & (n[:, None] > 0)


def check_codes(x, gpu_idx, ref_idx, R, cb):
    """Returns number of in-band coordinates; asserts the rule."""
    band = code_band(x, R, cb)
    diff = gpu_idx != ref_idx
    assert not np.any(diff & ~band), f"{int(np.sum(diff & ~band))} code mismatches outside the guard band"
    assert np.all(np.abs(gpu_idx - ref_idx)[band] <= 1)
    return int(band.sum())


def check_signs(x, gpu_idx, gpu_norms, gpu_signs, R, cb, S):
    d = gpu_idx.shape[1]  # the transform size D (the input rows may hold fewer)
    r = codec.residual_from_codes(x, R, cb, gpu_norms.astype(np.float64), gpu_idx)
    z = r @ S.T
    rn = np.linalg.norm(r, axis=1)
    want = (z >= 0).astype(np.int64)
    want[np.asarray(gpu_norms) == 0] = 0
    got = codec.unpack_bits(gpu_signs, 1, d)
    firm = np.abs(z) > BAND * np.sqrt(d) * rn[:, None]
    assert not np.any((got != want) & firm), f"{int(np.sum((got != want) & firm))} sign mismatches"
    return int((~firm).sum())


def rel_close(got, want, tol=1e-3):
    """||got - want|| <= tol * ||want|| (vectors), used per (b, q-head)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    return np.linalg.norm(got - want) <= tol * max(np.linalg.norm(want), 1e-30)


def out_errors(got, want):
    """(L2 relative error, largest coordinate error / largest |coordinate|) of
    one output vector."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    d = np.abs(got - want)
    return (float(np.linalg.norm(d) / max(np.linalg.norm(want), 1e-30)),
            float(np.max(d) / max(np.max(np.abs(want)), 1e-30)))


def assert_out_close(got, want, tol=1e-3, what=""):
    """The output bar, per (b, q-head): ||got - want||_2 <= tol ||want||_2 and,
    coordinate by coordinate, |got_j - want_j| <= tol max_j |want_j|.
    Returns the two errors."""
    l2, co = out_errors(got, want)
    assert np.all(np.isfinite(got)), f"non-finite output {what}"
    assert l2 <= tol, f"L2 error {l2:.3g} > {tol} {what}"
    assert co <= tol, f"coordinate error {co:.3g} (of max |o|) > {tol} {what}"
    return l2, co


class ErrStats:
    """Largest logit / output errors seen by a test (printed at the end, so a
    run shows how far inside the bar the results are)."""

    def __init__(self, name):
        self.name, self.logit, self.l2, self.co, self.n = name, None, 0.0, 0.0, 0

    def add(self, logit=None, out=None):
        if logit is not None:
            self.logit = logit if self.logit is None else max(self.logit, logit)
        if out is not None:
            self.l2, self.co = max(self.l2, out[0]), max(self.co, out[1])
            self.n += 1

    def report(self):
        lg = "not captured" if self.logit is None else f"{self.logit:.3g}"
        print(f"{self.name}: {self.n} outputs checked; max logit err {lg}, max L2 err {self.l2:.3g}, "
              f"max coordinate err {self.co:.3g} (bar 1e-3)", flush=True)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def upload_cache(cache):
    """Device copies of an oracle cache: pool (uint8), block table, lengths, rings."""
    return dict(
        pool=to_dev(cache.pool.reshape(-1)),
        block_table=to_dev(cache.block_table.astype(np.int32)),
        seq_lens=to_dev(cache.seq_lens.astype(np.int32)),
        k_win=to_dev(cache.k_win.view(np.uint16)).view(torch.float16),
        v_win=to_dev(cache.v_win.view(np.uint16)).view(torch.float16),
        num_pages=cache.pool.shape[0],
    )


def run_decode(ctx, q, dev, sm_scale, pages_per_split=0, logits_len=None):
    B, Hq, d = q.shape
    bt = dev["block_table"]
    ws = torch.empty(tqa.tq_decode_workspace_bytes(ctx, B, bt.shape[1], pages_per_split), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
    dbg = None
    if logits_len is not None:
        dbg = torch.full((B, Hq, logits_len), float("nan"), dtype=torch.float32, device="cuda")
    tqa.tq_decode_attn(ctx, q, dev["pool"], bt, dev["seq_lens"], dev["k_win"], dev["v_win"], out, ws, sm_scale,
                       pages_per_split=pages_per_split, dbg_logits=dbg, num_pages=dev["num_pages"])
    torch.cuda.synchronize()
    return out.cpu().numpy(), (None if dbg is None else dbg.cpu().numpy())
